// Host side of the C ABI: status strings, the thread-local error message,
// shared argument checks, and the host container functions tb_pack /
// tb_unpack / tb_signs_validate.
//
// Container [kwkr.cn/news/564617, "packing-format engineering"]: one fp16
// scale and one fp16 bias (= -scale) per 128 weights, 2-bit codes {0,1,2}
// for -1/0/+1 ([trdm.cn/news/822023 section 3.2] gives the same mapping),
// 16 codes per uint32 word ([lpnh.cn/news/2438023, "text model loading"]),
// code k of a word at bits 2k (little end first).
#include <cstring>

#include "tb_common.h"

namespace tb {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

int check_rotation(int64_t K, int block, const int8_t* signs, const char* who) {
  if (K <= 0) {
    set_error("%s: K must be positive (got %lld)", who, (long long)K);
    return TB_ERR_ARG;
  }
  if (K % kGroup) {
    set_error("%s: K=%lld is not a multiple of the group size %d", who, (long long)K, kGroup);
    return TB_ERR_SHAPE;
  }
  if (!block_known(block)) {
    set_error("%s: block %d is not one of 0, 512, 1024, 2048, 4096", who, block);
    return TB_ERR_BLOCK;
  }
  if (block == 0 && signs != nullptr) {
    set_error("%s: block 0 (no rotation) takes no sign vector", who);
    return TB_ERR_ARG;
  }
  if (block > 0) {
    if (signs == nullptr) {
      set_error("%s: block %d needs a sign vector", who, block);
      return TB_ERR_ARG;
    }
    if (K % block) {
      set_error("%s: K=%lld is not a multiple of block %d", who, (long long)K, block);
      return TB_ERR_SHAPE;
    }
  }
  return TB_OK;
}

int check_container(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                    const char* who, int sb_align) {
  if (!codes || !scales || !biases) {
    set_error("%s: codes, scales and biases must be non-NULL", who);
    return TB_ERR_ARG;
  }
  if (!aligned(codes, 16)) {
    set_error("%s: codes must be 16-byte aligned", who);
    return TB_ERR_ALIGN;
  }
  if (!aligned(scales, sb_align) || !aligned(biases, sb_align)) {
    set_error("%s: scales and biases must be %d-byte aligned", who, sb_align);
    return TB_ERR_ALIGN;
  }
  return TB_OK;
}

int check_dtype(int x_dtype, const void* x, const char* who) {
  if (x_dtype != TB_F32 && x_dtype != TB_BF16) {
    set_error("%s: activation dtype %d is neither TB_F32 nor TB_BF16", who, x_dtype);
    return TB_ERR_DTYPE;
  }
  if (!x) {
    set_error("%s: x is NULL", who);
    return TB_ERR_ARG;
  }
  if (!aligned(x, x_dtype == TB_F32 ? 4 : 2)) {
    set_error("%s: x is not aligned to its element size", who);
    return TB_ERR_ALIGN;
  }
  return TB_OK;
}

}  // namespace tb

using namespace tb;

extern "C" int tb_abi_version(void) { return TB_ABI_VERSION; }

extern "C" const char* tb_last_error(void) { return g_last_error.c_str(); }

extern "C" const char* tb_status_str(int status) {
  switch (status) {
    case TB_OK: return "TB_OK";
    case TB_ERR_ARG: return "TB_ERR_ARG";
    case TB_ERR_SHAPE: return "TB_ERR_SHAPE";
    case TB_ERR_BLOCK: return "TB_ERR_BLOCK";
    case TB_ERR_UNSUPPORTED: return "TB_ERR_UNSUPPORTED";
    case TB_ERR_SIGN: return "TB_ERR_SIGN";
    case TB_ERR_CODE: return "TB_ERR_CODE";
    case TB_ERR_DTYPE: return "TB_ERR_DTYPE";
    case TB_ERR_ALIGN: return "TB_ERR_ALIGN";
    case TB_ERR_HIP: return "TB_ERR_HIP";
    case TB_ERR_WORKSPACE: return "TB_ERR_WORKSPACE";
    default: return "TB_ERR_UNKNOWN";
  }
}

static int check_pack_shape(int64_t N, int64_t K, const char* who) {
  if (N < 0 || K <= 0) {
    set_error("%s: need N >= 0 and K > 0 (got N=%lld, K=%lld)", who, (long long)N, (long long)K);
    return TB_ERR_ARG;
  }
  if (K % kGroup) {
    set_error("%s: K=%lld is not a multiple of %d", who, (long long)K, kGroup);
    return TB_ERR_SHAPE;
  }
  return TB_OK;
}

extern "C" int tb_pack(const int8_t* t, const uint16_t* scales, int64_t N, int64_t K,
                       uint32_t* codes, uint16_t* scales_out, uint16_t* biases_out) {
  TB_TRY(check_pack_shape(N, K, "tb_pack"));
  if (N == 0) return TB_OK;
  if (!t || !scales || !codes || !scales_out || !biases_out) {
    set_error("tb_pack: NULL pointer");
    return TB_ERR_ARG;
  }
  const int64_t W = K / kCodesPerWord, G = K / kGroup;
  int64_t bad = 0;
  for (int64_t n = 0; n < N; ++n) {
    const int8_t* tr = t + n * K;
    uint32_t* cr = codes + n * W;
    for (int64_t w = 0; w < W; ++w) {
      uint32_t word = 0;
      for (int j = 0; j < kCodesPerWord; ++j) {
        const int v = tr[w * kCodesPerWord + j];
        bad += (v < -1) | (v > 1);
        word |= (uint32_t)((v + 1) & 3) << (2 * j);
      }
      cr[w] = word;
    }
  }
  if (bad) {
    set_error("tb_pack: %lld ternary values outside {-1,0,1}", (long long)bad);
    return TB_ERR_CODE;
  }
  for (int64_t i = 0; i < N * G; ++i) {
    scales_out[i] = scales[i];
    biases_out[i] = (uint16_t)(scales[i] ^ 0x8000u);  // fp16 negation
  }
  return TB_OK;
}

extern "C" int tb_unpack(const uint32_t* codes, int64_t N, int64_t K, int8_t* t_out) {
  TB_TRY(check_pack_shape(N, K, "tb_unpack"));
  if (N == 0) return TB_OK;
  if (!codes || !t_out) {
    set_error("tb_unpack: NULL pointer");
    return TB_ERR_ARG;
  }
  const int64_t W = K / kCodesPerWord;
  int64_t threes = 0;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t w = 0; w < W; ++w) {
      const uint32_t word = codes[n * W + w];
      for (int j = 0; j < kCodesPerWord; ++j) {
        const int c = (word >> (2 * j)) & 3;
        threes += (c == 3);
        t_out[n * K + w * kCodesPerWord + j] = (int8_t)(c - 1);
      }
    }
  }
  if (threes) {
    set_error("tb_unpack: %lld codes equal 3 (not a ternary container)", (long long)threes);
    return TB_ERR_CODE;
  }
  return TB_OK;
}

extern "C" int tb_signs_validate(const int8_t* signs, int64_t K) {
  if (K <= 0 || !signs) {
    set_error("tb_signs_validate: need K > 0 and a non-NULL sign vector");
    return TB_ERR_ARG;
  }
  for (int64_t k = 0; k < K; ++k) {
    if (signs[k] != 1 && signs[k] != -1) {
      set_error("tb_signs_validate: signs[%lld] = %d is not +-1", (long long)k, (int)signs[k]);
      return TB_ERR_SIGN;
    }
  }
  return TB_OK;
}
