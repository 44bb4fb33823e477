// tb_pack_device: the container packer of tb_pack, run on the device for
// containers too large to stage on the host.  [kwkr.cn/news/564617,
// "packing-format engineering"]: code = t + 1 (so -1/0/1 -> 0/1/2, as in
// trdm.cn/news/822023 section 3.2), 16 codes per uint32 word with code k at
// bits 2k, bias = -scale (fp16 sign flip).
#include "tb_device.h"

namespace tb {

// One thread per output word: reads 16 int8 values (one 128-bit load).
__global__ __launch_bounds__(kThreads) void pack_words_kernel(const int8_t* __restrict__ t,
                                                              uint32_t* __restrict__ codes,
                                                              int64_t nwords,
                                                              int32_t* __restrict__ bad) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= nwords) return;
  const uint4 v = reinterpret_cast<const uint4*>(t)[i];
  const uint32_t parts[4] = {v.x, v.y, v.z, v.w};
  uint32_t word = 0;
  int nbad = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int val = static_cast<int8_t>((parts[p] >> (8 * j)) & 0xFFu);
      const bool ok = val >= -1 && val <= 1;
      nbad += !ok;
      const uint32_t code = ok ? static_cast<uint32_t>(val + 1) : 3u;
      word |= code << (2 * (4 * p + j));
    }
  }
  codes[i] = word;
  if (nbad) atomicAdd(bad, nbad);
}

__global__ __launch_bounds__(kThreads) void pack_scales_kernel(const uint16_t* __restrict__ s,
                                                               uint16_t* __restrict__ so,
                                                               uint16_t* __restrict__ bo,
                                                               int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= n) return;
  const uint16_t v = s[i];
  so[i] = v;
  bo[i] = static_cast<uint16_t>(v ^ 0x8000u);
}

}  // namespace tb

using namespace tb;

extern "C" int tb_pack_device(const int8_t* t, const uint16_t* scales, int64_t N, int64_t K,
                              uint32_t* codes, uint16_t* scales_out, uint16_t* biases_out,
                              int32_t* bad_count, void* stream) {
  const char* who = "tb_pack_device";
  if (N < 0 || K <= 0) {
    set_error("%s: need N >= 0 and K > 0", who);
    return TB_ERR_ARG;
  }
  if (K % kGroup) {
    set_error("%s: K=%lld is not a multiple of %d", who, (long long)K, kGroup);
    return TB_ERR_SHAPE;
  }
  if (N == 0) return TB_OK;
  if (!t || !scales || !codes || !scales_out || !biases_out || !bad_count) {
    set_error("%s: NULL pointer", who);
    return TB_ERR_ARG;
  }
  if (!aligned(t, 16) || !aligned(codes, 16) || !aligned(bad_count, 4) || !aligned(scales, 2) ||
      !aligned(scales_out, 2) || !aligned(biases_out, 2)) {
    set_error("%s: t and codes must be 16-byte aligned, bad_count 4-byte", who);
    return TB_ERR_ALIGN;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t nwords = N * (K / kCodesPerWord);
  const int64_t ngroups = N * (K / kGroup);
  const int64_t bw = (nwords + kThreads - 1) / kThreads, bs = (ngroups + kThreads - 1) / kThreads;
  if (bw > 0x7FFFFFFF) {
    set_error("%s: container too large for one launch", who);
    return TB_ERR_SHAPE;
  }
  hipLaunchKernelGGL(pack_words_kernel, dim3((unsigned)bw), dim3(kThreads), 0, st, t, codes, nwords,
                     bad_count);
  TB_LAUNCH_CHECK(who);
  hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)bs), dim3(kThreads), 0, st, scales, scales_out,
                     biases_out, ngroups);
  TB_LAUNCH_CHECK(who);
  return TB_OK;
}
