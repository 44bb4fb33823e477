// tb_fwht_signed and tb_embed_inverse.
//
// Forward transform [lpnh.cn/news/2438023, "text model loading"]: multiply by
// the explicit sign vector, then the normalized Sylvester-Walsh-Hadamard
// transform of each block of the input (last) axis.  Inverse
// [kwkr.cn/news/564617, "ternary weights + folded Hadamard rotation"]: the
// normalized transform, then the signs again.  Embedding [lpnh.cn,
// "text model loading"]: dequantize the looked-up row, then the inverse.
//
// One 256-thread workgroup per (row, block): the block is staged in LDS as
// fp32 (at most 4096 values = 16 KB), transformed in place by radix-4 LDS
// passes, scaled once by 1/sqrt(L), and written back.
#include <algorithm>

#include "tb_device.h"

namespace tb {

template <int L, int DT>
__global__ __launch_bounds__(kThreads) void fwht_signed_kernel(const void* __restrict__ x,
                                                               float* y,
                                                               const int8_t* __restrict__ signs,
                                                               int64_t K, int inverse) {
  __shared__ float buf[L];
  const int64_t blk = blockIdx.x;
  const int64_t row = blockIdx.y;
  const int64_t base = row * K + blk * L;
  const int8_t* sg = signs + blk * L;
  for (int i = threadIdx.x; i < L; i += kThreads) {
    float v = load_x<DT>(x, base + i);
    if (!inverse) v *= static_cast<float>(sg[i]);
    buf[i] = v;
  }
  __syncthreads();
  fwht_lds<L>(buf);
  const float sc = inv_sqrt_block<L>();
  for (int i = threadIdx.x; i < L; i += kThreads) {
    float v = buf[i] * sc;
    if (inverse) v *= static_cast<float>(sg[i]);
    y[base + i] = v;
  }
}

// Dequantize element k of table row r: s * code + b in fp32 (one rounding).
__device__ __forceinline__ float decode_weight(const uint32_t* __restrict__ codes,
                                               const uint16_t* __restrict__ scales,
                                               const uint16_t* __restrict__ biases,
                                               int64_t r, int64_t K, int64_t k) {
  const uint32_t w = codes[r * (K / kCodesPerWord) + k / kCodesPerWord];
  const int c = (w >> (2 * (k % kCodesPerWord))) & 3;
  const int64_t gi = r * (K / kGroup) + k / kGroup;
  return fmaf(half_bits_to_float(scales[gi]), static_cast<float>(c), half_bits_to_float(biases[gi]));
}

template <int L>
__global__ __launch_bounds__(kThreads) void embed_inverse_kernel(
    const int32_t* __restrict__ ids, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases, int64_t V, int64_t K,
    const int8_t* __restrict__ signs, float* __restrict__ out) {
  __shared__ float buf[L];
  const int64_t blk = blockIdx.x;
  const int64_t t = blockIdx.y;
  const int64_t r = ids[t];
  float* o = out + t * K + blk * L;
  if (r < 0 || r >= V) {
    for (int i = threadIdx.x; i < L; i += kThreads) o[i] = __builtin_nanf("");
    return;
  }
  for (int i = threadIdx.x; i < L; i += kThreads)
    buf[i] = decode_weight(codes, scales, biases, r, K, blk * L + i);
  __syncthreads();
  fwht_lds<L>(buf);
  const float sc = inv_sqrt_block<L>();
  const int8_t* sg = signs + blk * L;
  for (int i = threadIdx.x; i < L; i += kThreads) o[i] = buf[i] * sc * static_cast<float>(sg[i]);
}

// block = 0: the dequantized row itself, 1024 elements per workgroup.
__global__ __launch_bounds__(kThreads) void embed_plain_kernel(
    const int32_t* __restrict__ ids, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases, int64_t V, int64_t K,
    float* __restrict__ out) {
  const int64_t t = blockIdx.y;
  const int64_t r = ids[t];
  float* o = out + t * K;
  for (int64_t k = blockIdx.x * 1024 + threadIdx.x; k < K && k < (blockIdx.x + 1) * 1024; k += kThreads)
    o[k] = (r < 0 || r >= V) ? __builtin_nanf("") : decode_weight(codes, scales, biases, r, K, k);
}

// Rows (and embedding ids) go in grid.y, which takes at most 65535: larger
// calls are launched in row chunks with offset pointers.
constexpr int64_t kRowChunk = 65535;

template <int L>
static void launch_fwht(const void* x, int dt, float* y, const int8_t* s, int64_t rows, int64_t K,
                        int inverse, hipStream_t st) {
  const int64_t esz = dt == TB_F32 ? 4 : 2;
  for (int64_t r0 = 0; r0 < rows; r0 += kRowChunk) {
    const dim3 grid(static_cast<unsigned>(K / L), static_cast<unsigned>(std::min(kRowChunk, rows - r0)));
    const void* xr = static_cast<const char*>(x) + r0 * K * esz;
    float* yr = y + r0 * K;
    if (dt == TB_F32)
      hipLaunchKernelGGL((fwht_signed_kernel<L, TB_F32>), grid, dim3(kThreads), 0, st, xr, yr, s, K, inverse);
    else
      hipLaunchKernelGGL((fwht_signed_kernel<L, TB_BF16>), grid, dim3(kThreads), 0, st, xr, yr, s, K, inverse);
  }
}

template <int L>
static void launch_embed(const int32_t* ids, int64_t T, const uint32_t* codes, const uint16_t* scales,
                         const uint16_t* biases, int64_t V, int64_t K, const int8_t* signs, float* out,
                         hipStream_t st) {
  for (int64_t t0 = 0; t0 < T; t0 += kRowChunk) {
    const unsigned nt = static_cast<unsigned>(std::min(kRowChunk, T - t0));
    if constexpr (L == 0)
      hipLaunchKernelGGL(embed_plain_kernel, dim3(static_cast<unsigned>((K + 1023) / 1024), nt), dim3(kThreads), 0,
                         st, ids + t0, codes, scales, biases, V, K, out + t0 * K);
    else
      hipLaunchKernelGGL(embed_inverse_kernel<L>, dim3(static_cast<unsigned>(K / L), nt), dim3(kThreads), 0, st,
                         ids + t0, codes, scales, biases, V, K, signs, out + t0 * K);
  }
}

}  // namespace tb

using namespace tb;

extern "C" int tb_fwht_signed(const void* x, int x_dtype, float* y, const int8_t* signs,
                              int64_t rows, int64_t K, int block, int inverse, void* stream) {
  const char* who = "tb_fwht_signed";
  if (rows < 0) {
    set_error("%s: rows must be >= 0", who);
    return TB_ERR_ARG;
  }
  if (block == 0) {
    set_error("%s: block must be one of 512, 1024, 2048, 4096", who);
    return TB_ERR_BLOCK;
  }
  TB_TRY(check_rotation(K, block, signs, who));
  if (inverse != 0 && inverse != 1) {
    set_error("%s: inverse must be 0 or 1", who);
    return TB_ERR_ARG;
  }
  if (rows == 0) return TB_OK;
  TB_TRY(check_dtype(x_dtype, x, who));
  if (!y) {
    set_error("%s: y is NULL", who);
    return TB_ERR_ARG;
  }
  if (!aligned(y, 4)) {
    set_error("%s: y must be 4-byte aligned", who);
    return TB_ERR_ALIGN;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (block) {
    case 512: launch_fwht<512>(x, x_dtype, y, signs, rows, K, inverse, st); break;
    case 1024: launch_fwht<1024>(x, x_dtype, y, signs, rows, K, inverse, st); break;
    case 2048: launch_fwht<2048>(x, x_dtype, y, signs, rows, K, inverse, st); break;
    default: launch_fwht<4096>(x, x_dtype, y, signs, rows, K, inverse, st); break;
  }
  TB_LAUNCH_CHECK(who);
  return TB_OK;
}

extern "C" int tb_embed_inverse(const int32_t* ids, int64_t T, const uint32_t* codes,
                                const uint16_t* scales, const uint16_t* biases, int64_t V,
                                int64_t K, const int8_t* signs, int block, float* out,
                                void* stream) {
  const char* who = "tb_embed_inverse";
  if (T < 0 || V < 0) {
    set_error("%s: T and V must be >= 0", who);
    return TB_ERR_ARG;
  }
  TB_TRY(check_rotation(K, block, signs, who));
  if (T == 0) return TB_OK;
  if (!ids || !out) {
    set_error("%s: ids and out must be non-NULL", who);
    return TB_ERR_ARG;
  }
  if (V > 0) TB_TRY(check_container(codes, scales, biases, who));
  if (!aligned(ids, 4) || !aligned(out, 4)) {
    set_error("%s: ids and out must be 4-byte aligned", who);
    return TB_ERR_ALIGN;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (block) {
    case 0: launch_embed<0>(ids, T, codes, scales, biases, V, K, signs, out, st); break;
    case 512: launch_embed<512>(ids, T, codes, scales, biases, V, K, signs, out, st); break;
    case 1024: launch_embed<1024>(ids, T, codes, scales, biases, V, K, signs, out, st); break;
    case 2048: launch_embed<2048>(ids, T, codes, scales, biases, V, K, signs, out, st); break;
    default: launch_embed<4096>(ids, T, codes, scales, biases, V, K, signs, out, st); break;
  }
  TB_LAUNCH_CHECK(who);
  return TB_OK;
}
