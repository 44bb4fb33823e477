// Batch-1 Packed linear on the two block containers [kwkr.cn/news/564617,
// "packing-format engineering": GGUF blocks of 128 ternary weights, PQ2_0
// (one 2-bit slot per trit and an fp16 scale, 34 bytes, 2.125 bits/weight)
// and PTQ1_0 (dense trits, 28 bytes, 1.75 bits/weight)], consumed as stored.
// Block layouts (a reading; the pages print neither): the fp16 scale d
// first, then the codes; code c (t = c - 1) decodes to (c - 1) d.  PQ2_0:
// code k at bits 2 (k % 4) of code byte k / 4 (the MLX group's code words,
// byte for byte).  PTQ1_0: 26 trit bytes, five codes each in base 3 with the
// first code as the lowest digit (the last byte holds three).
//
//   y[n] = sum_g d[n][g] (sum_{k in g} (c[n][k] - 1) xr[k])
//        = sum_g d[n][g] (f_g sum_k c q_k - X_g),   xr ~= f_g q (exact limbs)
//
// 1. blocks_prep_kernel: one wave per 1024-input chunk: the signed block
//    transform on the matrix cores and its exact four-limb split
//    (tb_xform.h), written to the workspace as the operand image and the
//    group terms (X_g, f_g).
// 2. blocks_stream_kernel: 8 waves per workgroup, each streaming whole
//    16-row tiles.  The workgroup copies the operand image to LDS once.  A
//    span is 4 groups of the tile's 16 rows: lane (lane group lg, row c)
//    loads the whole block (row c, group 4 s + lg) with dword-aligned loads,
//    rebuilds its eight 16-code words in registers (PQ2_0: byte-align the
//    code bytes that follow the 2-byte scale; PTQ1_0: a 256-entry LDS table
//    maps a trit byte to its five 2-bit codes), and the span is 8
//    v_mfma_i32_16x16x64_i8 against a block-diagonal activation operand (A row
//    (group a, limb l) non-zero only in k-block a, so one instruction keeps
//    the 4 groups apart).  A ring of P spans of loads is in flight per wave.
#include <algorithm>

#include "tb_xform.h"

namespace tb {

constexpr int kBlkWaves = 8;
constexpr int kBlkThreads = 64 * kBlkWaves;
constexpr int kBlkArow = 144;                        // LDS bytes per (group, limb) operand row
constexpr int kBlkImgChunk = 8 * kXfLimbs * 128;     // workspace bytes of one chunk's operand image
constexpr int kBlkYbuf = 16;                         // finished tiles a wave parks in LDS
constexpr int kBlkRing = 4;                          // spans of loads in flight per wave
constexpr int64_t kBlkLdsMax = 150 * 1024;

enum BlockFormat { kPq2 = 0, kPtq1 = 1 };
template <int FMT>
struct BlkFmt;
template <>
struct BlkFmt<kPq2> {
  static constexpr int BYTES = 34, DW = 9;  // 36-byte aligned window around a block
};
template <>
struct BlkFmt<kPtq1> {
  static constexpr int BYTES = 28, DW = 7;
};

__host__ __device__ inline int blk_nch(int K) { return (K + 1023) >> 10; }
__host__ __device__ inline int64_t blk_ws_bytes(int K) {
  return static_cast<int64_t>(blk_nch(K)) * (kBlkImgChunk + 8 * 8);
}
// LDS: operand image, group terms, trit table, per-wave finished rows
__host__ __device__ inline int64_t blk_lds_xf(int nch) { return static_cast<int64_t>(nch) * 8 * kXfLimbs * kBlkArow; }
__host__ __device__ inline int64_t blk_lds_lut(int nch) { return blk_lds_xf(nch) + nch * 8 * 8; }
__host__ __device__ inline int64_t blk_lds_ybuf(int nch) { return blk_lds_lut(nch) + 256 * 4; }
__host__ __device__ inline int64_t blk_lds_total(int nch) { return blk_lds_ybuf(nch) + kBlkWaves * kBlkYbuf * 16 * 4; }

// ---------------------------------------------------------------------------
// 1. the activation's operand image
// ---------------------------------------------------------------------------
template <int L, int DT>
__global__ __launch_bounds__(256) void blocks_prep_kernel(const void* __restrict__ x, const int8_t* __restrict__ signs,
                                                          int K, char* __restrict__ ws) {
  const int lane = threadIdx.x & 63;
  const int c = static_cast<int>(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nch = blk_nch(K);
  if (c >= nch) return;  // whole wave; no barrier in this kernel
  constexpr int ESZ = DT == TB_F32 ? 4 : 2;
  const auto rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(x), 0, K * ESZ, kRsrcWord3);
  const auto rsg = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(signs), 0, L > 0 ? K : 0, kRsrcWord3);
  XformIn<DT> in;
  xform_issue<L, DT>(rx, rsg, static_cast<int64_t>(c) * 1024, c * 1024, lane, in);
  const v4u* cst = reinterpret_cast<const v4u*>(&kXformConst.w[xf_mode<L>()][0][lane][0]);
  const v4u* cst2 = reinterpret_cast<const v4u*>(&kXformConst.w[xf_mode<L>()][1][lane][0]);
  const v4u cf[2] = {cst[0], cst[1]};
  const v4u cs[2] = {cst2[0], cst2[1]};
  float2* xf = reinterpret_cast<float2*>(ws + static_cast<int64_t>(nch) * kBlkImgChunk);
  xform_chunk<L, DT>(in, 8 * c, lane, cf, cs, ws, xf, 128);
}

// ---------------------------------------------------------------------------
// 2. stream the blocks
// ---------------------------------------------------------------------------
template <int FMT>
struct BlkSlot {
  uint32_t d[BlkFmt<FMT>::DW];
};

// Trit byte b -> its five 2-bit codes at bits 0, 2, .., 8 (lowest base-3
// digit first); bytes above 242 hold no valid trits and decode to whatever
// digits the division gives (the host-side unpack rejects them).
__device__ __forceinline__ uint32_t trit_byte_codes(uint32_t b) {
  uint32_t v = 0;
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    v |= (b % 3u) << (2 * m);
    b /= 3u;
  }
  return v;
}

// The block's eight 16-code words and its scale bits.
template <int FMT>
__device__ __forceinline__ void blk_words(const BlkSlot<FMT>& sl, int sh, const uint32_t* lut, uint32_t w[8],
                                          uint32_t& scale) {
  if constexpr (FMT == kPq2) {
    // window of 36 bytes from the dword holding the block's first byte; the
    // block starts at byte sh (0 or 2) of it, its codes at byte sh + 2
    uint32_t e[9];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = sh ? sl.d[i + 1] : sl.d[i];
    e[8] = sl.d[8];
    const uint32_t bs = sh ? 0u : 2u;
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = __builtin_amdgcn_alignbyte(e[i + 1], e[i], bs);
    scale = sh ? (sl.d[0] >> 16) : (sl.d[0] & 0xFFFFu);
  } else {
    // trit byte i sits at byte 2 + i of the 28-byte block; its five codes go
    // to bits 10 i .. 10 i + 9 of the 256 code bits
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = 0u;
#pragma unroll
    for (int i = 0; i < 26; ++i) {
      const int byte = 2 + i;
      const uint32_t b = (sl.d[byte >> 2] >> (8 * (byte & 3))) & 0xFFu;
      const uint32_t v = lut[b];
      const int pos = 10 * i, wi = pos >> 5, o = pos & 31;
      w[wi] |= v << o;
      if (o > 22 && wi + 1 < 8) w[wi + 1] |= v >> (32 - o);
    }
    scale = sl.d[0] & 0xFFFFu;
  }
}

template <int FMT, int P>
__global__ __launch_bounds__(kBlkThreads, 1) void blocks_stream_kernel(const char* __restrict__ ws,
                                                                        const uint8_t* __restrict__ blocks, int N,
                                                                        int K, int tpw, float* __restrict__ y) {
  constexpr int NW = kBlkWaves, M = 16, GPS = 4, BB = BlkFmt<FMT>::BYTES, DW = BlkFmt<FMT>::DW;
  extern __shared__ uint4 blk_lds_dyn[];
  char* const lds = reinterpret_cast<char*>(blk_lds_dyn);
  const int G = K / kGroup, S = (G + GPS - 1) / GPS, nch = blk_nch(K);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lg = lane >> 4, c = lane & 15;
  const int ar = c & 3, alg = (c >> 2) & 3;
  const bool a_lane = alg == lg;
  char* const lds_a = lds;
  float2* const lds_xf = reinterpret_cast<float2*>(lds + blk_lds_xf(nch));
  uint32_t* const lut = reinterpret_cast<uint32_t*>(lds + blk_lds_lut(nch));
  float* const ybuf = reinterpret_cast<float*>(lds + blk_lds_ybuf(nch)) + wave * (kBlkYbuf * 16);

  // this wave's tiles: t0 + wave + NW j, j < ntw; steps k = j S + s
  const int T = (N + M - 1) / M;
  const int t0 = static_cast<int>(blockIdx.x) * NW * tpw;
  const int t1 = min(T, t0 + NW * tpw);
  const int ntw = t0 + wave < t1 ? (t1 - t0 - wave + NW - 1) / NW : 0;
  const int nsteps = ntw * S;
  const auto rbl = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blocks), 0, N * G * BB, kRsrcWord3);
  const auto ry = __builtin_amdgcn_make_buffer_rsrc(y, 0, N * 4, kRsrcWord3);
  // G is even (K % 256 == 0), so block (row, 4 s + lg) starts at byte
  // 2 (lg & 1) of a dword for PQ2_0; PTQ1_0 blocks are dword aligned
  const int sh = FMT == kPq2 ? 2 * (lg & 1) : 0;
  int ks = 0, kt = 0;  // span and tile of the next step to load
  const int lane_b = ((t0 + wave) * M + c) * G * BB + lg * BB - sh;
  auto load = [&](int k, BlkSlot<FMT>& st) {
    const int off = k < nsteps ? lane_b + kt * (NW * M * G * BB) + ks * (GPS * BB) : kOob;
    const v4u u0 = __builtin_amdgcn_raw_buffer_load_b128(rbl, off, 0, 0);
    st.d[0] = u0.x;
    st.d[1] = u0.y;
    st.d[2] = u0.z;
    st.d[3] = u0.w;
    if constexpr (FMT == kPq2) {
      const v4u u1 = __builtin_amdgcn_raw_buffer_load_b128(rbl, off + 16, 0, 0);
      st.d[4] = u1.x;
      st.d[5] = u1.y;
      st.d[6] = u1.z;
      st.d[7] = u1.w;
      st.d[8] = __builtin_amdgcn_raw_buffer_load_b32(rbl, off + 32, 0, 0);
    } else {
      const v3u u1 = __builtin_amdgcn_raw_buffer_load_b96(rbl, off + 16, 0, 0);
      st.d[4] = u1.x;
      st.d[5] = u1.y;
      st.d[6] = u1.z;
    }
    if (++ks == S) {
      ks = 0;
      ++kt;
    }
  };
  BlkSlot<FMT> ring[P];
#pragma unroll
  for (int k = 0; k < P; ++k) load(k, ring[k]);

  // the operand image and group terms into LDS (the ring's loads are in
  // flight meanwhile); the trit table
  {
    const int rows = nch * 8 * kXfLimbs;
    for (int i = tid; i < rows * 8; i += kBlkThreads) {
      const int r = i >> 3, q = i & 7;
      *reinterpret_cast<uint4*>(lds_a + r * kBlkArow + q * 16) = *reinterpret_cast<const uint4*>(ws + r * 128 + q * 16);
    }
    const float2* xfg = reinterpret_cast<const float2*>(ws + static_cast<int64_t>(nch) * kBlkImgChunk);
    for (int i = tid; i < nch * 8; i += kBlkThreads) lds_xf[i] = xfg[i];
    if constexpr (FMT == kPtq1)
      for (int i = tid; i < 256; i += kBlkThreads) lut[i] = trit_byte_codes(static_cast<uint32_t>(i));
  }
  __syncthreads();
  if (nsteps == 0) return;  // no barrier follows

  uint4 av[kWordsPerGroup];
#pragma unroll
  for (int w = 0; w < kWordsPerGroup; ++w) av[w] = make_uint4(0, 0, 0, 0);
  float yacc = 0.f;
  int s = 0, j = 0, j0 = 0;  // span and tile of the step being consumed; first parked tile
  auto flush = [&](int upto) {  // write parked tiles j0 .. upto - 1 of this wave
    for (int i = lane; i < (upto - j0) * 16; i += 64) {
      const int row = (t0 + wave + NW * (j0 + (i >> 4))) * M + (i & 15);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ybuf[i]), ry, row * 4, 0, 0);  // rows past N: dropped
    }
    j0 = upto;
  };
  for (int base = 0; base < nsteps; base += P) {
#pragma unroll
    for (int q = 0; q < P; ++q) {
      const BlkSlot<FMT> cur = ring[q];
      load(base + q + P, ring[q]);  // refill the slot before computing on its data
      if (base + q < nsteps) {
        uint32_t w[8], sbits;
        blk_words<FMT>(cur, sh, lut, w, sbits);
        if (a_lane) {
          const uint4* ap = reinterpret_cast<const uint4*>(lds_a + ((s * GPS + alg) * kXfLimbs + ar) * kBlkArow);
#pragma unroll
          for (int i = 0; i < kWordsPerGroup; ++i) av[i] = ap[i];
        }
        v4i acc0 = {}, acc1 = {};
#pragma unroll
        for (int i = 0; i < kWordsPerGroup; i += 2) {
          acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(v4i{(int)av[i].x, (int)av[i].y, (int)av[i].z, (int)av[i].w},
                                                       decode_word(w[i]), acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
              v4i{(int)av[i + 1].x, (int)av[i + 1].y, (int)av[i + 1].z, (int)av[i + 1].w}, decode_word(w[i + 1]), acc1,
              0, 0, 0);
        }
        const v4i acc = acc0 + acc1;
        const float2 xf = lds_xf[s * GPS + lg];
        const float v = static_cast<float>(acc[3]) * 16777216.f + static_cast<float>(acc[2]) * 65536.f +
                        static_cast<float>(acc[1]) * 256.f + static_cast<float>(acc[0]);
        const float d = half_bits_to_float(static_cast<uint16_t>(sbits));
        // groups past K (the last span's padding) contribute nothing
        yacc += s * GPS + lg < G ? d * (v * xf.y - xf.x) : 0.f;
        if (++s == S) {
          float t = yacc + xor_lane(yacc, 4, lane);
          t += xor_lane(t, 5, lane);
          if (lg == 0) ybuf[(j - j0) * 16 + c] = t;
          yacc = 0.f;
          s = 0;
          if (++j - j0 == kBlkYbuf) flush(j);
        }
      }
    }
  }
  flush(j);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <int L>
static void blocks_prep_launch(const void* x, int dt, const int8_t* signs, int K, void* ws, hipStream_t st) {
  const dim3 grid((blk_nch(K) + 3) / 4);
  if (dt == TB_F32)
    hipLaunchKernelGGL((blocks_prep_kernel<L, TB_F32>), grid, dim3(256), 0, st, x, signs, K, static_cast<char*>(ws));
  else
    hipLaunchKernelGGL((blocks_prep_kernel<L, TB_BF16>), grid, dim3(256), 0, st, x, signs, K, static_cast<char*>(ws));
}

template <int FMT>
static void blocks_stream_launch(const void* ws, const uint8_t* blocks, int N, int K, float* y, hipStream_t st) {
  // one 16-row tile per wave per round, several rounds per workgroup for
  // wide layers: about two workgroups' worth of tiles per CU
  const int T = (N + 15) / 16;
  const int tpw = std::max(1, (T + 2 * kBlkWaves * device_cus() - 1) / (2 * kBlkWaves * device_cus()));
  const int grid = (T + kBlkWaves * tpw - 1) / (kBlkWaves * tpw);
  const size_t lds = static_cast<size_t>(blk_lds_total(blk_nch(K)));
  static std::atomic<uint64_t> lds_set{0};
  lds_limit_once(reinterpret_cast<const void*>(blocks_stream_kernel<FMT, kBlkRing>), static_cast<int>(kBlkLdsMax),
                 lds_set);
  hipLaunchKernelGGL((blocks_stream_kernel<FMT, kBlkRing>), dim3(grid), dim3(kBlkThreads), lds, st,
                     static_cast<const char*>(ws), blocks, N, K, tpw, y);
}

template <int FMT>
static int blocks_gemv(const void* x, int x_dtype, int64_t B, int64_t K, const int8_t* signs, int block,
                       const uint8_t* blocks, int64_t N, float* y, void* workspace, size_t ws_bytes, void* stream,
                       const char* who) {
  if (B < 0 || N < 0) {
    set_error("%s: B and N must be >= 0", who);
    return TB_ERR_ARG;
  }
  TB_TRY(check_rotation(K, block, signs, who));
  if (B > 1) {
    set_error("%s: batch %lld: the block containers are consumed at batch 1", who, (long long)B);
    return TB_ERR_UNSUPPORTED;
  }
  if (K % 256) {
    set_error("%s: K=%lld must be a multiple of 256", who, (long long)K);
    return TB_ERR_SHAPE;
  }
  if (!(block == 0 || block == 512 || block == 1024)) {
    set_error("%s: block %d: this path takes 0, 512 or 1024", who, block);
    return TB_ERR_UNSUPPORTED;
  }
  if (B == 0 || N == 0) return TB_OK;
  TB_TRY(check_dtype(x_dtype, x, who));
  if (!blocks || !y) {
    set_error("%s: blocks and y must be non-NULL", who);
    return TB_ERR_ARG;
  }
  if (!aligned(x, 16) || (signs && !aligned(signs, 16)) || !aligned(blocks, 4) || !aligned(y, 4)) {
    set_error("%s: x and signs need 16-byte, blocks and y 4-byte alignment", who);
    return TB_ERR_ALIGN;
  }
  const int64_t G = K / kGroup;
  if (N > (int64_t(1) << 30) || (N + 16) * G * BlkFmt<FMT>::BYTES + 64 > INT32_MAX) {
    set_error("%s: N=%lld x K=%lld is too large for one call (blocks under 2 GiB)", who, (long long)N,
              (long long)K);
    return TB_ERR_SHAPE;
  }
  if (blk_lds_total(blk_nch(static_cast<int>(K))) > kBlkLdsMax) {
    set_error("%s: K=%lld takes more LDS than the stream kernel has", who, (long long)K);
    return TB_ERR_UNSUPPORTED;
  }
  if (!workspace || ws_bytes < static_cast<size_t>(blk_ws_bytes(static_cast<int>(K))) || !aligned(workspace, 16)) {
    set_error("%s: workspace of %zu bytes at %p; %lld bytes, 16-byte aligned, needed", who, ws_bytes, workspace,
              (long long)blk_ws_bytes(static_cast<int>(K)));
    return TB_ERR_WORKSPACE;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int k = static_cast<int>(K);
  if (block == 0) blocks_prep_launch<0>(x, x_dtype, signs, k, workspace, st);
  else if (block == 512) blocks_prep_launch<512>(x, x_dtype, signs, k, workspace, st);
  else blocks_prep_launch<1024>(x, x_dtype, signs, k, workspace, st);
  TB_LAUNCH_CHECK(who);
  blocks_stream_launch<FMT>(workspace, blocks, static_cast<int>(N), k, y, st);
  TB_LAUNCH_CHECK(who);
  return TB_OK;
}

}  // namespace tb

using namespace tb;

extern "C" size_t tb_blocks_gemv_workspace_size(int64_t K) {
  if (K <= 0 || K % 256 || K > (int64_t(1) << 24)) return 0;
  return static_cast<size_t>(blk_ws_bytes(static_cast<int>(K)));
}

extern "C" int tb_pq2_gemv(const void* x, int x_dtype, int64_t B, int64_t K, const int8_t* signs, int block,
                           const uint8_t* blocks, int64_t N, float* y, void* workspace, size_t ws_bytes,
                           void* stream) {
  return blocks_gemv<kPq2>(x, x_dtype, B, K, signs, block, blocks, N, y, workspace, ws_bytes, stream, "tb_pq2_gemv");
}

extern "C" int tb_ptq1_gemv(const void* x, int x_dtype, int64_t B, int64_t K, const int8_t* signs, int block,
                            const uint8_t* blocks, int64_t N, float* y, void* workspace, size_t ws_bytes,
                            void* stream) {
  return blocks_gemv<kPtq1>(x, x_dtype, B, K, signs, block, blocks, N, y, workspace, ws_bytes, stream,
                            "tb_ptq1_gemv");
}
