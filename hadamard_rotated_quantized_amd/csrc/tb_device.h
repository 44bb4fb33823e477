// Device helpers shared by the gfx950 kernels: element loads, fp16 decode,
// and the workgroup-level block Walsh-Hadamard transform in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "tb_common.h"

namespace tb {

constexpr int kThreads = 256;  // workgroup size of the transform kernels

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return static_cast<float>(v);
}

// Element i of an activation row stored as fp32 (dtype TB_F32) or bf16 bits.
template <int DT>
__device__ __forceinline__ float load_x(const void* x, int64_t i) {
  if constexpr (DT == TB_F32) {
    return static_cast<const float*>(x)[i];
  } else {
    return bf16_bits_to_float(static_cast<const uint16_t*>(x)[i]);
  }
}

// Round-to-nearest-even fp32 -> bf16 bit pattern (finite inputs).
__device__ __forceinline__ uint16_t float_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// In-place unnormalized Sylvester transform of L values in LDS by a 256-thread
// workgroup: H[i][j] = (-1)^popcount(i & j) (natural order), built from the
// recurrence H_2n = [[H_n, H_n], [H_n, -H_n]] [trdm.cn/news/822023 section
// 2.2]; two butterfly stages (radix 4) per pass, one LDS pass per pair of
// index bits.  Caller has written buf and must __syncthreads() before the
// call; the function ends with a barrier.
template <int L>
__device__ __forceinline__ void fwht_lds(float* buf) {
  static_assert(L >= 4 && (L & (L - 1)) == 0, "power of two");
  const int tid = threadIdx.x;
  int h = 1;
#pragma unroll
  for (; h * 4 <= L; h *= 4) {
    for (int q = tid; q < L / 4; q += kThreads) {
      const int lo = q % h, hi = q / h;
      const int base = hi * 4 * h + lo;
      const float a = buf[base], b = buf[base + h], c = buf[base + 2 * h], d = buf[base + 3 * h];
      const float ab0 = a + b, ab1 = a - b, cd0 = c + d, cd1 = c - d;
      buf[base] = ab0 + cd0;
      buf[base + h] = ab1 + cd1;
      buf[base + 2 * h] = ab0 - cd0;
      buf[base + 3 * h] = ab1 - cd1;
    }
    __syncthreads();
  }
  if (h < L) {  // odd number of index bits: one radix-2 stage left
    for (int q = tid; q < L / 2; q += kThreads) {
      const int lo = q % h, hi = q / h;
      const int base = hi * 2 * h + lo;
      const float a = buf[base], b = buf[base + h];
      buf[base] = a + b;
      buf[base + h] = a - b;
    }
    __syncthreads();
  }
}

// 1/sqrt(L) as a float: exact for 1024 (2^-5) and 4096 (2^-6), rounded
// to nearest for 512 and 2048.
template <int L>
__device__ __forceinline__ float inv_sqrt_block() {
  if constexpr (L == 1024) return 0.03125f;
  else if constexpr (L == 4096) return 0.015625f;
  else if constexpr (L == 512) return 0.04419417382415922f;
  else return 0.02209708691207961f;  // 2048
}


// ---------------------------------------------------------------------------
// host helpers shared by the launchers
// ---------------------------------------------------------------------------
// Compute units of the current device, queried once per device and cached
// (256, the MI355X count, when the runtime cannot say).  Thread-safe.
inline int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  std::atomic<int>& c = cache[dev & 63];
  int v = c.load(std::memory_order_relaxed);
  if (v <= 0) {
    v = 256;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    c.store(v, std::memory_order_relaxed);
  }
  return v;
}

// Raise a kernel's dynamic LDS limit to `bytes` once per device.  `done`
// is the kernel's own bit mask of devices already set; two threads racing
// both make the same idempotent call.
inline void lds_limit_once(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  const uint64_t bit = uint64_t(1) << (dev & 63);
  if (done.load(std::memory_order_acquire) & bit) return;
  (void)hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  done.fetch_or(bit, std::memory_order_release);
}

}  // namespace tb

// Report a failed launch through the error string.
#define TB_LAUNCH_CHECK(who)                                                    \
  do {                                                                          \
    hipError_t _e = hipGetLastError();                                          \
    if (_e != hipSuccess) {                                                     \
      tb::set_error("%s: kernel launch failed: %s", who, hipGetErrorString(_e)); \
      return TB_ERR_HIP;                                                        \
    }                                                                           \
  } while (0)
