// Internal helpers shared by the library's translation units: error
// reporting, argument validation and the launch check.  Not part of the ABI.
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/tb.h"

namespace tb {

// thread-local message for tb_last_error()
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kGroup = 128;        // weights per fp16 scale/bias
constexpr int kCodesPerWord = 16;  // 2-bit codes per uint32

inline bool block_known(int block) {
  return block == 0 || block == 512 || block == 1024 || block == 2048 || block == 4096;
}

// Shared validation of the (K, block, signs) triple of a rotated input.
// Returns TB_OK or an error (message set).
int check_rotation(int64_t K, int block, const int8_t* signs, const char* who);

// Shared validation of a (codes, scales, biases) container of N rows, width K:
// non-NULL, codes 16-byte aligned, scales and biases aligned to sb_align bytes
// (2 = their element size; the decode-matmul kernels load them as dwords and
// larger vectors and ask for 4).
int check_container(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                    const char* who, int sb_align = 2);

int check_dtype(int x_dtype, const void* x, const char* who);

}  // namespace tb

#define TB_TRY(expr)            \
  do {                          \
    int _st = (expr);           \
    if (_st != TB_OK) return _st; \
  } while (0)
