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
// Two kernels, one launch each, one workgroup per band of ceil(N / CUs)
// rows (tiles of 16 rows, the last one possibly partial):
// blocks_band_kernel (further below) copies a band's blocks into LDS whole
// where they fit; blocks_gemv_kernel, the general path, streams them through
// registers.  In blocks_gemv_kernel each wave first issues the activation
// loads of its chunk transforms, then the block loads of its first items,
// and rotates the activation itself while the blocks are in flight: the
// waves transform the 1024-input chunks on the matrix cores and split them
// exactly into four limbs, writing the operand image and the group terms
// (X_g, f_g) straight to LDS (tb_xform.h).  The band's work is (tile, span)
// items, a span being 4 groups of the tile's 16 rows; each wave takes a
// contiguous range of items.
// Lane (lane group lg, row c) loads the whole block (row c, group 4 s + lg)
// with dword-aligned loads, rebuilds its eight 16-code words in registers
// (PQ2_0: byte-align the code bytes that follow the 2-byte scale; PTQ1_0: a
// 256-entry LDS table maps a trit byte to its five codes as bytes, the
// operand in natural element order against limb rows written in that order
// too, tb_ptq1_nat.h), and the
// span is 8 v_mfma_i32_16x16x64_i8 against a block-diagonal activation
// operand (A row (group a, limb l) non-zero only in k-block a, so one
// instruction keeps the 4 groups apart).  A ring of P items of loads is in
// flight per wave.  Each wave leaves one partial row sum per tile it touched
// in LDS; the band's rows are the sums over the waves in wave order.
#include <algorithm>

#include "tb_ptq1_nat.h"

namespace tb {

constexpr int kBlkWaves = 8;
constexpr int kBlkThreads = 64 * kBlkWaves;
constexpr int kBlkArow = 144;                        // LDS bytes per (group, limb) operand row
constexpr int kBlkRing = 4;                          // items of loads in flight per wave
constexpr int kBlkMaxTiles = 48;                     // tiles of a band (LDS of the partial sums)
constexpr int kBlkMaxTasks = 3;                      // chunk transforms per wave loaded up front
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
// LDS: operand image, group terms, trit table, partial row sums
__host__ __device__ inline int64_t blk_lds_xf(int nch) { return static_cast<int64_t>(nch) * 8 * kXfLimbs * kBlkArow; }
__host__ __device__ inline int64_t blk_lds_lut(int nch) { return blk_lds_xf(nch) + nch * 8 * 8; }
// (the trit table: 256 entries of 8 bytes, used by PTQ1_0)
__host__ __device__ inline int64_t blk_lds_red(int nch) { return blk_lds_lut(nch) + 256 * 8; }
__host__ __device__ inline int64_t blk_lds_total(int nch, int tiles) {
  return blk_lds_red(nch) + static_cast<int64_t>(tiles) * kBlkWaves * 16 * 4;
}

template <int FMT>
struct BlkSlot {
  uint32_t d[BlkFmt<FMT>::DW];
};

// PQ2_0: the block's eight 16-code words and its scale bits, from the window
// of 36 bytes from the dword holding the block's first byte (the block
// starts at byte sh, 0 or 2, of it; its codes at byte sh + 2).  PTQ1_0 blocks
// decode through the trit table (tb_ptq1_nat.h).
__device__ __forceinline__ void pq2_words(const BlkSlot<kPq2>& sl, int sh, uint32_t w[8], uint32_t& scale) {
  uint32_t e[9];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = sh ? sl.d[i + 1] : sl.d[i];
  e[8] = sl.d[8];
  const uint32_t bs = sh ? 0u : 2u;
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = __builtin_amdgcn_alignbyte(e[i + 1], e[i], bs);
  scale = sh ? (sl.d[0] >> 16) : (sl.d[0] & 0xFFFFu);
}

template <int L, int DT, int FMT, int P>
__global__ __launch_bounds__(kBlkThreads, 1) void blocks_gemv_kernel(const void* __restrict__ x,
                                                                      const int8_t* __restrict__ signs,
                                                                      const uint8_t* __restrict__ blocks, int N, int K,
                                                                      int R, float* __restrict__ y) {
  constexpr int NW = kBlkWaves, M = 16, GPS = 4, BB = BlkFmt<FMT>::BYTES;
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
  uint2* const lut8 = reinterpret_cast<uint2*>(lds + blk_lds_lut(nch));  // PTQ1_0 trit table
  float* const red = reinterpret_cast<float*>(lds + blk_lds_red(nch));

  // the band: rows band0 .. band0 + nrow - 1 in tiles of 16 (the last may be
  // partial); items i = t S + s; this wave's items i0 .. i1 - 1
  const int band0 = static_cast<int>(blockIdx.x) * R;
  const int nrow = min(R, N - band0);
  const int tsub = (nrow + M - 1) / M;
  const int items = tsub * S;
  const int i0 = items * wave / NW, i1 = items * (wave + 1) / NW;
  const int nit = i1 - i0;

  // 1. the activation loads of this wave's chunk transforms, first: the
  //    transforms then wait for these alone (loads complete in order)
  constexpr int ESZ = DT == TB_F32 ? 4 : 2;
  const auto rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(x), 0, K * ESZ, kRsrcWord3);
  const auto rsg = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(signs), 0, L > 0 ? K : 0, kRsrcWord3);
  XformIn<DT> xin[kBlkMaxTasks];
#pragma unroll
  for (int r = 0; r < kBlkMaxTasks; ++r) {
    const int ch = wave + NW * r;
    if (ch < nch) xform_issue<L, DT>(rx, rsg, static_cast<int64_t>(ch) * 1024, ch * 1024, lane, xin[r]);
  }

  // 2. the first P items' loads.  Lane (lg, c) loads block (row c of the
  //    item's tile, group 4 s + lg); rows past the band and items past the
  //    wave's range read from an offset past every buffer (zeros, no traffic)
  const auto rbl = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blocks), 0, N * G * BB, kRsrcWord3);
  // G is even (K % 256 == 0), so block (row, 4 s + lg) starts at byte
  // 2 (lg & 1) of a dword for PQ2_0; PTQ1_0 blocks are dword aligned
  const int sh = FMT == kPq2 ? 2 * (lg & 1) : 0;
  int lt = i0 / S, ls = i0 - (i0 / S) * S;  // tile (in the band) and span of the next item to load
  int nload = 0;
  auto load = [&](BlkSlot<FMT>& st) {
    const int rib = lt * M + c;  // row in the band
    const bool live = nload < nit && rib < nrow;
    const int blk = (band0 + rib) * G + ls * GPS + lg;
    const int off = live ? blk * BB - sh : kOob;
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
    ++nload;
    if (++ls == S) {
      ls = 0;
      ++lt;
    }
  };
  BlkSlot<FMT> ring[P];
#pragma unroll
  for (int k = 0; k < P; ++k) load(ring[k]);

  // 3. the band's rotation while the blocks are in flight: wave w transforms
  //    chunks w, w + 8, ... into the LDS operand image (chunks beyond the
  //    up-front tasks load and transform in turn)
  {
    const v4u* cst = reinterpret_cast<const v4u*>(&kXformConst.w[xf_mode<L>()][0][lane][0]);
    const v4u* cst2 = reinterpret_cast<const v4u*>(&kXformConst.w[xf_mode<L>()][1][lane][0]);
    const v4u cf[2] = {cst[0], cst[1]};
    const v4u cs[2] = {cst2[0], cst2[1]};
    // PTQ1_0: limb rows in natural element order, to match its code bytes
    auto xform = [&](const XformIn<DT>& in, int ch) {
      if constexpr (FMT == kPtq1) xform_chunk_natural<L, DT>(in, 8 * ch, lane, cf, cs, lds_a, lds_xf, kBlkArow);
      else xform_chunk<L, DT>(in, 8 * ch, lane, cf, cs, lds_a, lds_xf, kBlkArow);
    };
#pragma unroll
    for (int r = 0; r < kBlkMaxTasks; ++r) {
      const int ch = wave + NW * r;
      if (ch < nch) xform(xin[r], ch);
    }
    for (int ch = wave + NW * kBlkMaxTasks; ch < nch; ch += NW) {
      XformIn<DT> in;
      xform_issue<L, DT>(rx, rsg, static_cast<int64_t>(ch) * 1024, ch * 1024, lane, in);
      xform(in, ch);
    }
    if constexpr (FMT == kPtq1)
      for (int i = tid; i < 256; i += kBlkThreads) lut8[i] = trit_entry(static_cast<uint32_t>(i));
    for (int i = tid; i < tsub * NW * 16; i += kBlkThreads) red[i] = 0.f;
  }
  __syncthreads();

  // 4. the items
  uint4 av[kWordsPerGroup];
#pragma unroll
  for (int w = 0; w < kWordsPerGroup; ++w) av[w] = make_uint4(0, 0, 0, 0);
  float yacc = 0.f;
  int ct = i0 / S, cs = i0 - (i0 / S) * S;  // tile and span of the item being consumed
  for (int base = 0; base < nit; base += P) {
#pragma unroll
    for (int q = 0; q < P; ++q) {
      const BlkSlot<FMT> cur = ring[q];
      load(ring[q]);  // refill the slot before computing on its data
      if (base + q < nit) {
        // MFMA operands of the block's codes: PQ2_0 the 2-bit words decoded;
        // PTQ1_0 the codes as bytes in natural order (trit table)
        v4i bq[kWordsPerGroup];
        uint32_t sbits;
        if constexpr (FMT == kPq2) {
          uint32_t w[8];
          pq2_words(cur, sh, w, sbits);
#pragma unroll
          for (int i = 0; i < 8; ++i) bq[i] = decode_word(w[i]);
        } else {
          uint32_t cb[32];
          ptq1_code_bytes([&](int i) { return (cur.d[(2 + i) >> 2] >> (8 * ((2 + i) & 3))) & 0xFFu; }, lut8, cb);
#pragma unroll
          for (int i = 0; i < 8; ++i) bq[i] = v4i{(int)cb[4 * i], (int)cb[4 * i + 1], (int)cb[4 * i + 2], (int)cb[4 * i + 3]};
          sbits = cur.d[0] & 0xFFFFu;
        }
        if (a_lane) {
          const uint4* ap = reinterpret_cast<const uint4*>(lds_a + ((cs * GPS + alg) * kXfLimbs + ar) * kBlkArow);
#pragma unroll
          for (int i = 0; i < kWordsPerGroup; ++i) av[i] = ap[i];
        }
        v4i acc0 = {}, acc1 = {};
#pragma unroll
        for (int i = 0; i < kWordsPerGroup; i += 2) {
          acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(v4i{(int)av[i].x, (int)av[i].y, (int)av[i].z, (int)av[i].w},
                                                       bq[i], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
              v4i{(int)av[i + 1].x, (int)av[i + 1].y, (int)av[i + 1].z, (int)av[i + 1].w}, bq[i + 1], acc1, 0, 0, 0);
        }
        const v4i acc = acc0 + acc1;
        const float2 xf = lds_xf[cs * GPS + lg];
        const float v = static_cast<float>(acc[3]) * 16777216.f + static_cast<float>(acc[2]) * 65536.f +
                        static_cast<float>(acc[1]) * 256.f + static_cast<float>(acc[0]);
        const float d = half_bits_to_float(static_cast<uint16_t>(sbits));
        // groups past K (the last span's padding) contribute nothing
        yacc += cs * GPS + lg < G ? d * (v * xf.y - xf.x) : 0.f;
        // the wave's partial for this tile, at the tile's last span or the
        // wave's last item
        if (++cs == S || base + q + 1 == nit) {
          float t = yacc + xor_lane(yacc, 4, lane);
          t += xor_lane(t, 5, lane);
          if (lg == 0) red[(ct * NW + wave) * 16 + c] = t;
          yacc = 0.f;
          if (cs == S) {
            cs = 0;
            ++ct;
          }
        }
      }
    }
  }
  __syncthreads();
  // 5. the band's rows: partial sums added in wave order
  for (int i = tid; i < tsub * 16; i += kBlkThreads) {
    const int t = i >> 4, r = i & 15, rib = t * M + r;
    if (rib < nrow) {
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) a += red[(t * NW + w) * 16 + r];
      y[band0 + rib] = a;
    }
  }
}

// ---------------------------------------------------------------------------
// staged band: the band's blocks copied into LDS whole
// ---------------------------------------------------------------------------
// When a band's blocks fit the LDS next to the operand image, the band is
// moved in by direct-to-LDS loads of 1 KB per wave instruction (contiguous
// memory: the band's rows are consecutive) while the transform waves rotate
// the activation, and every wave then reads its items' blocks from LDS.
// Roles as in the MLX band kernel: waves below min(chunks, 8) transform, the
// others copy (all 8 copy when every wave transforms).  Items (16-row tile
// t, span s) are dealt round robin, item i = t S + s to wave i % 8; MI is the
// most items a wave gets, so a wave's items carry no branches but the last.
//
// LDS: operand image, group terms, trit table, partial row sums, then the
// staged bytes: the band's blocks from the 16-byte boundary at or below its
// first byte, with room for the 9-dword windows of the tiles' padding rows.
struct BlkStage {
  int64_t stage, total;
};
__host__ __device__ inline BlkStage blk_stage_layout(int nch, int tsub, int G, int BB) {
  BlkStage l;
  l.stage = (blk_lds_total(nch, tsub) + 15) & ~int64_t(15);
  // a window reaches at most 7 blocks and 40 bytes past the tiles' rows
  l.total = l.stage + (16 + static_cast<int64_t>(tsub) * 16 * G * BB + 8 * BB + 64 + 1023) / 1024 * 1024;
  return l;
}

// Spans of a row in the staged kernel and the group lane group q takes in
// span s.  PTQ1_0: groups 4 s .. 4 s + 3.  PQ2_0: span pairs cover 8 groups,
// span 2 h + p taking groups 8 h + 2 q + p, so that the 4 lane groups' blocks
// (68 bytes apart) start in distinct LDS bank quarters and every block of a
// span starts at the same byte of a dword (p = 0: byte 0, p = 1: byte 2).
template <int FMT>
__host__ __device__ inline int blk_spans(int G) {
  return FMT == kPq2 ? 2 * ((G + 7) / 8) : (G + 3) / 4;
}
template <int FMT>
__device__ __forceinline__ int blk_group(int s, int q) {
  return FMT == kPq2 ? 8 * (s >> 1) + 2 * q + (s & 1) : 4 * s + q;
}

template <int L, int DT, int FMT, int MI>
__global__ __launch_bounds__(kBlkThreads, 1) void blocks_band_kernel(const void* __restrict__ x,
                                                                      const int8_t* __restrict__ signs,
                                                                      const uint8_t* __restrict__ blocks, int N, int K,
                                                                      int R, float* __restrict__ y) {
  constexpr int NW = kBlkWaves, M = 16, BB = BlkFmt<FMT>::BYTES, DW = BlkFmt<FMT>::DW;
  typedef __attribute__((address_space(3))) void lds_void;
  extern __shared__ uint4 blk_lds_dyn[];
  char* const lds = reinterpret_cast<char*>(blk_lds_dyn);
  const int G = K / kGroup, S = blk_spans<FMT>(G), nch = blk_nch(K);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lg = lane >> 4, c = lane & 15;
  const int ar = c & 3, alg = (c >> 2) & 3;
  const bool a_lane = alg == lg;
  const int band0 = static_cast<int>(blockIdx.x) * R;
  const int nrow = min(R, N - band0);
  const int tsub = (R + M - 1) / M;  // the layout is sized for a full band
  const BlkStage lay = blk_stage_layout(nch, tsub, G, BB);
  char* const lds_a = lds;
  float2* const lds_xf = reinterpret_cast<float2*>(lds + blk_lds_xf(nch));
  uint2* const lut8 = reinterpret_cast<uint2*>(lds + blk_lds_lut(nch));  // PTQ1_0 trit table
  float* const red = reinterpret_cast<float*>(lds + blk_lds_red(nch));
  char* const stage = lds + lay.stage;

  // 1. transform waves: their chunks' activation loads; copy waves: the band
  const int ntask_waves = nch < NW ? nch : NW;
  const bool xwave = wave < ntask_waves;
  constexpr int ESZ = DT == TB_F32 ? 4 : 2;
  const auto rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(x), 0, K * ESZ, kRsrcWord3);
  const auto rsg = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(signs), 0, L > 0 ? K : 0, kRsrcWord3);
  XformIn<DT> xin[kBlkMaxTasks];
  if (xwave) {
#pragma unroll
    for (int r = 0; r < kBlkMaxTasks; ++r) {
      const int ch = wave + NW * r;
      if (ch < nch) xform_issue<L, DT>(rx, rsg, static_cast<int64_t>(ch) * 1024, ch * 1024, lane, xin[r]);
    }
  }
  // the band's bytes [e0, e1) of the block array, staged from e0 rounded
  // down to 16 bytes (delta bytes earlier); the range ends at e1
  const int64_t e0 = static_cast<int64_t>(band0) * G * BB, e1 = e0 + static_cast<int64_t>(nrow) * G * BB;
  const int64_t a0 = e0 & ~int64_t(15);
  const int delta = static_cast<int>(e0 - a0);
  const int nbytes = static_cast<int>(e1 - a0);
  {
    const int first = ntask_waves < NW ? ntask_waves : 0;
    const int nload = NW - first;
    if (wave >= first) {
      const auto rbl = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blocks) + a0, 0, nbytes, kRsrcWord3);
      const int slots = (nbytes + 1023) >> 10;
      for (int q = wave - first; q < slots; q += nload)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rbl, (lds_void*)(stage + q * 1024), 16, q * 1024 + lane * 16, 0, 0, 0);
    }
  }

  // 2. the operand image, the trit table, zeroed partial sums
  for (int i = tid; i < tsub * NW * 16; i += kBlkThreads) red[i] = 0.f;
  if constexpr (FMT == kPtq1)
    for (int i = tid; i < 256; i += kBlkThreads) lut8[i] = trit_entry(static_cast<uint32_t>(i));
  if (xwave) {
    const v4u* cst = reinterpret_cast<const v4u*>(&kXformConst.w[xf_mode<L>()][0][lane][0]);
    const v4u* cst2 = reinterpret_cast<const v4u*>(&kXformConst.w[xf_mode<L>()][1][lane][0]);
    const v4u cf[2] = {cst[0], cst[1]};
    const v4u cs[2] = {cst2[0], cst2[1]};
#pragma unroll
    for (int r = 0; r < kBlkMaxTasks; ++r) {
      const int ch = wave + NW * r;
      if (ch < nch) {
        // PTQ1_0: limb rows in natural element order, to match its code bytes
        if constexpr (FMT == kPtq1) xform_chunk_natural<L, DT>(xin[r], 8 * ch, lane, cf, cs, lds_a, lds_xf, kBlkArow);
        else xform_chunk<L, DT>(xin[r], 8 * ch, lane, cf, cs, lds_a, lds_xf, kBlkArow);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // vmcnt(0): this wave's staging landed
  __syncthreads();

  // 3. the items.  Lane (lg, c) takes block (row t 16 + c, group
  //    blk_group(s, lg)): PTQ1_0 its 7 dwords; PQ2_0 the 9 dwords from the
  //    one holding its first code byte, and its scale (rows past the band
  //    read what the stage holds there; their sums are never written)
  const int items = tsub * S;
  int tt[MI], ss[MI];
  bool iv[MI];
#pragma unroll
  for (int j = 0; j < MI; ++j) {
    const int i = wave + NW * j;
    iv[j] = i < items;
    const int ic = iv[j] ? i : 0;
    tt[j] = ic / S;
    ss[j] = ic - tt[j] * S;
  }
  BlkSlot<FMT> bl[MI];
  uint16_t sb16[MI];  // PQ2_0: the block's scale bits
  uint4 av[MI][kWordsPerGroup];
  float2 xfv[MI];
#pragma unroll
  for (int j = 0; j < MI; ++j) {
#pragma unroll
    for (int d = 0; d < DW; ++d) bl[j].d[d] = 0u;
    sb16[j] = 0;
    xfv[j] = make_float2(0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kWordsPerGroup; ++w) av[j][w] = make_uint4(0, 0, 0, 0);
    if (j < MI - 1 || iv[j]) {
      const int t = tt[j], s = ss[j];
      const int g = blk_group<FMT>(s, lg);
      const int b0 = delta + ((t * M + c) * G + g) * BB;  // the block's first byte
      if constexpr (FMT == kPq2) {
        sb16[j] = *reinterpret_cast<const uint16_t*>(stage + b0);
        const uint32_t* src = reinterpret_cast<const uint32_t*>(stage + ((b0 + 2) & ~3));
#pragma unroll
        for (int d = 0; d < DW; ++d) bl[j].d[d] = src[d];
      } else {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(stage + b0);  // dword aligned
#pragma unroll
        for (int d = 0; d < DW; ++d) bl[j].d[d] = src[d];
      }
      xfv[j] = lds_xf[g];
      if (a_lane) {
        const uint4* ap =
            reinterpret_cast<const uint4*>(lds_a + (blk_group<FMT>(s, alg) * kXfLimbs + ar) * kBlkArow);
#pragma unroll
        for (int w = 0; w < kWordsPerGroup; ++w) av[j][w] = ap[w];
      }
    }
  }
  float part[MI];
#pragma unroll
  for (int j = 0; j < MI; ++j) {
    part[j] = 0.f;
    if (j < MI - 1 || iv[j]) {
      // the MFMA operands of the block's 8 code words: PQ2_0 the 2-bit words
      // decoded; PTQ1_0 the codes as bytes in natural order (trit table)
      v4i bq[kWordsPerGroup];
      uint32_t sbits;
      if constexpr (FMT == kPq2) {
        // codes from byte 2 (even spans) or 0 (odd spans) of the first dword
        const int o = (ss[j] & 1) ? 0 : 2;
#pragma unroll
        for (int i = 0; i < 8; ++i) bq[i] = decode_word(__builtin_amdgcn_alignbyte(bl[j].d[i + 1], bl[j].d[i], o));
        sbits = sb16[j];
      } else {
        uint32_t cb[32];
        ptq1_code_bytes([&](int i) { return (bl[j].d[(2 + i) >> 2] >> (8 * ((2 + i) & 3))) & 0xFFu; }, lut8, cb);
#pragma unroll
        for (int i = 0; i < 8; ++i) bq[i] = v4i{(int)cb[4 * i], (int)cb[4 * i + 1], (int)cb[4 * i + 2], (int)cb[4 * i + 3]};
        sbits = bl[j].d[0] & 0xFFFFu;
      }
      v4i acc0 = {}, acc1 = {};
#pragma unroll
      for (int i = 0; i < kWordsPerGroup; i += 2) {
        const uint4 u0 = av[j][i], u1 = av[j][i + 1];
        acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(v4i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w}, bq[i], acc0, 0, 0,
                                                     0);
        acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(v4i{(int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w}, bq[i + 1], acc1,
                                                     0, 0, 0);
      }
      const v4i acc = acc0 + acc1;
      const float v = static_cast<float>(acc[3]) * 16777216.f + static_cast<float>(acc[2]) * 65536.f +
                      static_cast<float>(acc[1]) * 256.f + static_cast<float>(acc[0]);
      const float d = half_bits_to_float(static_cast<uint16_t>(sbits));
      // groups past K (the last span's padding) contribute nothing
      part[j] = iv[j] && blk_group<FMT>(ss[j], lg) < G ? d * (v * xfv[j].y - xfv[j].x) : 0.f;
    }
  }
  // per tile: this wave's items in registers, then over the 4 lane groups,
  // parked in red[t][wave]
  int tend = tt[0];
#pragma unroll
  for (int j = 1; j < MI; ++j) tend = iv[j] ? tt[j] : tend;
  for (int t = tt[0]; t < tsub && t <= tend; ++t) {
    float v = 0.f;
    bool any = false;
#pragma unroll
    for (int j = 0; j < MI; ++j) {
      const bool mine = tt[j] == t && iv[j];
      v += mine ? part[j] : 0.f;
      any |= mine;
    }
    if (any) {
      v += xor_lane(v, 4, lane);
      v += xor_lane(v, 5, lane);
      if (lg == 0) red[(t * NW + wave) * 16 + c] = v;
    }
  }
  __syncthreads();
  // 4. the band's rows: partial sums added in wave order
  for (int i = tid; i < tsub * 16; i += kBlkThreads) {
    const int t = i >> 4, r = i & 15, rib = t * M + r;
    if (rib < nrow) {
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) a += red[(t * NW + w) * 16 + r];
      y[band0 + rib] = a;
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct BlkPlan {
  int grid, rows;
  int64_t lds;
};

// One workgroup per CU, each with a band of ceil(N / CUs) rows (at least one
// tile), while the bands' partial sums fit LDS; more (and narrower) bands
// beyond that.
static BlkPlan blk_plan(int64_t N, int64_t K) {
  BlkPlan p{};
  const int64_t cus = device_cus();
  int64_t rows = std::max<int64_t>(16, (N + cus - 1) / cus);
  rows = std::min<int64_t>(rows, int64_t(kBlkMaxTiles) * 16);
  p.rows = static_cast<int>(rows);
  p.grid = static_cast<int>((N + rows - 1) / rows);
  p.lds = blk_lds_total(blk_nch(static_cast<int>(K)), static_cast<int>((rows + 15) / 16));
  return p;
}

// The staged band kernel applies when the block array is 16-byte aligned
// (the staging loads start at 16-byte boundaries), the band's blocks fit the
// LDS with the operand image, and every wave takes at most kBlkStageItems
// items and at most kBlkMaxTasks chunk transforms.
constexpr int kBlkStageItems = 4;
template <int FMT>
static int blk_stage_items(const BlkPlan& p, int64_t K, const uint8_t* blocks) {
  if (!aligned(blocks, 16)) return 0;
  const int nch = blk_nch(static_cast<int>(K));
  const int G = static_cast<int>(K / kGroup), S = blk_spans<FMT>(G), tsub = (p.rows + 15) / 16;
  const int mi = (tsub * S + kBlkWaves - 1) / kBlkWaves;
  if (nch > kBlkWaves * kBlkMaxTasks || mi > kBlkStageItems) return 0;
  if (blk_stage_layout(nch, tsub, G, BlkFmt<FMT>::BYTES).total > kBlkLdsMax) return 0;
  return mi;
}

template <int FMT, int L, int DT, int MI>
static void blocks_band_launch(const void* x, const int8_t* signs, const uint8_t* blocks, int N, int K, float* y,
                               const BlkPlan& p, hipStream_t st) {
  auto kern = blocks_band_kernel<L, DT, FMT, MI>;
  static std::atomic<uint64_t> lds_set{0};
  lds_limit_once(reinterpret_cast<const void*>(kern), static_cast<int>(kBlkLdsMax), lds_set);
  const int64_t lds = blk_stage_layout(blk_nch(K), (p.rows + 15) / 16, K / kGroup, BlkFmt<FMT>::BYTES).total;
  hipLaunchKernelGGL(kern, dim3(p.grid), dim3(kBlkThreads), static_cast<size_t>(lds), st, x, signs, blocks, N, K,
                     p.rows, y);
}

template <int FMT, int L, int DT>
static void blocks_launch_t(const void* x, const int8_t* signs, const uint8_t* blocks, int N, int K, float* y,
                            const BlkPlan& p, hipStream_t st) {
  switch (blk_stage_items<FMT>(p, K, blocks)) {
    case 1: return blocks_band_launch<FMT, L, DT, 1>(x, signs, blocks, N, K, y, p, st);
    case 2: return blocks_band_launch<FMT, L, DT, 2>(x, signs, blocks, N, K, y, p, st);
    case 3: return blocks_band_launch<FMT, L, DT, 3>(x, signs, blocks, N, K, y, p, st);
    case 4: return blocks_band_launch<FMT, L, DT, 4>(x, signs, blocks, N, K, y, p, st);
    default: break;
  }
  auto kern = blocks_gemv_kernel<L, DT, FMT, kBlkRing>;
  static std::atomic<uint64_t> lds_set{0};
  lds_limit_once(reinterpret_cast<const void*>(kern), static_cast<int>(kBlkLdsMax), lds_set);
  hipLaunchKernelGGL(kern, dim3(p.grid), dim3(kBlkThreads), static_cast<size_t>(p.lds), st, x, signs, blocks, N, K,
                     p.rows, y);
}

template <int FMT, int L>
static void blocks_launch_l(int dt, const void* x, const int8_t* signs, const uint8_t* blocks, int N, int K, float* y,
                            const BlkPlan& p, hipStream_t st) {
  if (dt == TB_F32) blocks_launch_t<FMT, L, TB_F32>(x, signs, blocks, N, K, y, p, st);
  else blocks_launch_t<FMT, L, TB_BF16>(x, signs, blocks, N, K, y, p, st);
}

template <int FMT>
static int blocks_gemv(const void* x, int x_dtype, int64_t B, int64_t K, const int8_t* signs, int block,
                       const uint8_t* blocks, int64_t N, float* y, void* stream, const char* who) {
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
  const BlkPlan p = blk_plan(N, K);
  if (p.lds > kBlkLdsMax) {
    set_error("%s: K=%lld takes more LDS than the kernel has", who, (long long)K);
    return TB_ERR_UNSUPPORTED;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int n = static_cast<int>(N), k = static_cast<int>(K);
  if (block == 0) blocks_launch_l<FMT, 0>(x_dtype, x, signs, blocks, n, k, y, p, st);
  else if (block == 512) blocks_launch_l<FMT, 512>(x_dtype, x, signs, blocks, n, k, y, p, st);
  else blocks_launch_l<FMT, 1024>(x_dtype, x, signs, blocks, n, k, y, p, st);
  TB_LAUNCH_CHECK(who);
  return TB_OK;
}

}  // namespace tb

using namespace tb;

extern "C" int tb_pq2_gemv(const void* x, int x_dtype, int64_t B, int64_t K, const int8_t* signs, int block,
                           const uint8_t* blocks, int64_t N, float* y, void* stream) {
  return blocks_gemv<kPq2>(x, x_dtype, B, K, signs, block, blocks, N, y, stream, "tb_pq2_gemv");
}

extern "C" int tb_ptq1_gemv(const void* x, int x_dtype, int64_t B, int64_t K, const int8_t* signs, int block,
                            const uint8_t* blocks, int64_t N, float* y, void* stream) {
  return blocks_gemv<kPtq1>(x, x_dtype, B, K, signs, block, blocks, N, y, stream, "tb_ptq1_gemv");
}
