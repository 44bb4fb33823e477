// Multi-module decode: many Packed linears of one decode step (batch 1) in
// two launches [lpnh.cn/news/2438023, "text model loading" (every packed
// module applies fwht(x, block, signs) and then the quantized matmul);
// kwkr.cn/news/564617, "ternary weights + folded Hadamard rotation" and
// "packing-format engineering"].
//
// A decode step runs hundreds of linears of 1.5 to 360 MB each; launched one
// by one, each pays a kernel launch and its own ramp.  Here:
//
// 1. multi_prep_kernel: one wave per 1024-input chunk of every distinct
//    input, the in-register MFMA transform (tb_xform.h), writing its exact
//    four-limb operand image and group sums to the workspace.  Modules that
//    read the same x with the same signs (q/k/v_proj, gate/up_proj and
//    in_proj_qkv/z of a layer: one sign vector per input width, kwkr.cn
//    "ternary weights + folded Hadamard rotation") share one image.
//
// 2. multi_stream_kernel: one persistent workgroup per CU.  The host cuts
//    the concatenated list of 16-row tiles (all modules, in order) into
//    pieces of one module each, large first and smaller toward the end of the
//    list (each about 1 / workgroups of the weight bytes still left, down to
//    a floor), and the workgroups take pieces in list order from a
//    counter in the workspace (the transform kernel zeroes it), so a
//    workgroup that streams slower than the others simply takes fewer pieces.
//    For a piece of a module other than its last one a workgroup copies the
//    module's operand image into LDS; its 8 waves then take the piece's tiles
//    round robin.  A wave
//    streams its tiles span by span (16 rows x 4 groups: 2 KB of codes, 128 B
//    of scales, 128 B of biases) through a ring of P register slots: lane
//    (lane group lg, row c) loads the 32 code bytes it multiplies straight
//    into its B-operand registers, plus its group's scale and bias, so P spans
//    per wave are in flight while one is multiplied, and a wave waits only
//    for its own loads (no barrier inside a module).  A span is 8
//    v_mfma_i32_16x16x64_i8 against the exact integer activation (4 balanced
//    base-256 limbs, one A row each, read from LDS), with the fp16 scale and
//    bias applied in fp32; a tile's rows are written once, after its last
//    span.
//
// The same plan and kernels take the weights as PQ2_0 or PTQ1_0 blocks
// (kwkr.cn/news/564617, "packing-format engineering"; a plan holds one
// container for all its modules).  There a lane's span pair is two adjacent
// blocks of its row (groups 8 p + 2 lg and 8 p + 2 lg + 1, with the A rows
// in the same group order), one contiguous run of 68 or 56 bytes that
// carries the codes and both scales; PTQ1_0's trit bytes go through a
// 256-entry table in LDS to the 2-bit codes the other paths decode.
#include <algorithm>
#include <array>
#include <map>
#include <tuple>
#include <type_traits>
#include <vector>

#include "tb_ptq1_nat.h"

namespace tb {

// ---------------------------------------------------------------------------
// the device plan (built on the host, copied to device memory by the caller)
// ---------------------------------------------------------------------------
constexpr int32_t kPlanMagic = 0x4D504254;  // "TBPM"
constexpr int kMultiWaves = 8;                      // waves per streaming workgroup
constexpr int kMultiArow = 144;          // LDS bytes per (group, limb) operand row
constexpr int kMultiImgChunk = 8 * kXfLimbs * 128;  // workspace bytes of one chunk's operand image
constexpr int kMultiRing = 4;                       // span pairs in flight per wave
constexpr int kMultiYbuf = 32;                      // finished tiles a wave holds in LDS before writing them
constexpr int64_t kMultiLdsMax = 150 * 1024;
constexpr int kMultiWsHead = 256;                   // workspace bytes before the first image: the piece counter
constexpr int kMultiPieceFloor = 64;                // smallest piece: 1 / 64 of a workgroup's mean share

// weight containers of a plan: the MLX affine container (codes, scales,
// biases), or PQ2_0 / PTQ1_0 blocks (the module's codes pointer holds the
// blocks)
constexpr int kMultiMlx = 0, kMultiPq2 = 1, kMultiPtq1 = 2;
constexpr int kPq2Bytes = 34;   // PQ2_0 block: fp16 scale, then 32 code bytes
constexpr int kPtq1Bytes = 28;  // PTQ1_0 block: fp16 scale, then 26 trit bytes (5 codes each, base 3)
__host__ __device__ inline int multi_block_bytes(int fmt) { return fmt == kMultiPq2 ? kPq2Bytes : kPtq1Bytes; }

struct MultiHeader {  // 64 bytes
  int32_t magic, count, tasks, grid;
  int32_t block, x_dtype, max_nch, pieces;
  int64_t modules_off, tasks_off, pieces_off;
  int32_t total_bytes, format;
};
struct MultiModule {  // 64 bytes
  const void* x;
  const int8_t* signs;
  const uint32_t* codes;
  const uint16_t* scales;
  const uint16_t* biases;
  float* y;
  int32_t N, K;
  int32_t tile0;  // index of the module's first 16-row tile in the concatenated list
  int32_t ws_off; // workspace byte offset of the module's operand image (group sums follow)
};
static_assert(sizeof(MultiHeader) == 64 && sizeof(MultiModule) == 64, "plan layout");

__host__ __device__ inline int multi_nch(int K) { return (K + 1023) >> 10; }

// LDS layout of the stream kernel: the operand image, the group sums, then
// each wave's buffer of finished output rows
__host__ __device__ inline int64_t multi_lds_xf(int max_nch) {
  return static_cast<int64_t>(max_nch) * 8 * kXfLimbs * kMultiArow;
}
__host__ __device__ inline int64_t multi_lds_ybuf(int max_nch) { return multi_lds_xf(max_nch) + max_nch * 8 * 8; }
__host__ __device__ inline int64_t multi_lds_lut(int max_nch) {
  return multi_lds_ybuf(max_nch) + kMultiWaves * kMultiYbuf * 16 * 4;
}
// (the trit table, 256 entries of 8 bytes, is used by PTQ1_0 plans only)
__host__ __device__ inline int64_t multi_lds_total(int max_nch) { return multi_lds_lut(max_nch) + 256 * 8; }

// ---------------------------------------------------------------------------
// 1. transform every chunk of every module's input
// ---------------------------------------------------------------------------
template <int L, int DT, bool NAT>
__global__ __launch_bounds__(256) void multi_prep_kernel(const char* __restrict__ plan, char* __restrict__ ws) {
  const MultiHeader* hd = reinterpret_cast<const MultiHeader*>(plan);
  const int lane = threadIdx.x & 63;
  const int task = static_cast<int>(blockIdx.x) * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the stream kernel's piece counter starts at zero (this kernel runs first
  // on the stream)
  if (blockIdx.x == 0 && threadIdx.x == 0) *reinterpret_cast<int*>(ws) = 0;
  if (task >= hd->tasks) return;  // whole wave; the kernel has no barrier
  const int2 tk = reinterpret_cast<const int2*>(plan + hd->tasks_off)[task];
  const MultiModule md = reinterpret_cast<const MultiModule*>(plan + hd->modules_off)[tk.x];
  const int c = tk.y;
  constexpr int ESZ = DT == TB_F32 ? 4 : 2;
  const auto rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(md.x), 0, md.K * ESZ, kRsrcWord3);
  const auto rsg = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(md.signs), 0, L > 0 ? md.K : 0, kRsrcWord3);
  XformIn<DT> in;
  xform_issue<L, DT>(rx, rsg, static_cast<int64_t>(c) * 1024, c * 1024, lane, in);
  const v4u* cst = reinterpret_cast<const v4u*>(&kXformConst.w[xf_mode<L>()][0][lane][0]);
  const v4u* cst2 = reinterpret_cast<const v4u*>(&kXformConst.w[xf_mode<L>()][1][lane][0]);
  const v4u cf[2] = {cst[0], cst[1]};
  const v4u cs[2] = {cst2[0], cst2[1]};
  char* img = ws + md.ws_off;
  float2* xf = reinterpret_cast<float2*>(img + static_cast<int64_t>(multi_nch(md.K)) * kMultiImgChunk);
  if constexpr (NAT) xform_chunk_natural<L, DT>(in, 8 * c, lane, cf, cs, img, xf, 128);
  else xform_chunk<L, DT>(in, 8 * c, lane, cf, cs, img, xf, 128);
}

// ---------------------------------------------------------------------------
// 2. stream every module's weights
// ---------------------------------------------------------------------------
struct MultiPair {
  uint4 w[4];  // 8 code words of (row, group) in each of the pair's two spans
  uint4 s, b;  // 8 fp16 scales / biases of the row's 8 groups of the pair
};

// PQ2_0: a lane's span pair is two adjacent blocks, groups 8 p + 2 lg and
// 8 p + 2 lg + 1 of its row: 68 bytes from a dword boundary (G is even)
struct MultiPairPq2 {
  uint32_t d[17];
};
// PTQ1_0: likewise two adjacent blocks, 56 bytes from an 8-byte boundary
struct MultiPairPtq1 {
  uint32_t d[14];
};

template <int NW, int P, int FMT>
__global__ __launch_bounds__(64 * NW, 1) void multi_stream_kernel(const char* __restrict__ plan,
                                                                  char* __restrict__ ws) {
  using Pair = typename std::conditional<
      FMT == kMultiPq2, MultiPairPq2, typename std::conditional<FMT == kMultiPtq1, MultiPairPtq1, MultiPair>::type>::type;
  constexpr int kMultiThreads = 64 * NW;
  constexpr int M = 16, GPS = 4;
  extern __shared__ uint4 lds_dyn[];
  char* const lds = reinterpret_cast<char*>(lds_dyn);
  const MultiHeader* hd = reinterpret_cast<const MultiHeader*>(plan);
  const MultiModule* mods = reinterpret_cast<const MultiModule*>(plan + hd->modules_off);
  const int4* const pieces = reinterpret_cast<const int4*>(plan + hd->pieces_off);
  const int npieces = hd->pieces;
  int* const counter = reinterpret_cast<int*>(ws);
  __shared__ int piece_next;
  const int max_nch = hd->max_nch;
  char* const lds_a = lds;
  const float2* const lds_xf = reinterpret_cast<const float2*>(lds + multi_lds_xf(max_nch));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lg = lane >> 4, c = lane & 15;
  const int ar = c & 3, alg = (c >> 2) & 3;
  const bool a_lane = alg == lg;
  float* const ybuf = reinterpret_cast<float*>(lds + multi_lds_ybuf(max_nch)) + wave * (kMultiYbuf * 16);
  // PTQ1_0: trit byte -> its five codes (lowest base-3 digit first) as
  // bytes 0-4 of an 8-byte entry, written before the first piece's barrier
  uint2* const lut = reinterpret_cast<uint2*>(lds + multi_lds_lut(max_nch));
  if constexpr (FMT == kMultiPtq1)
    for (int i = tid; i < 256; i += kMultiThreads) lut[i] = trit_entry(static_cast<uint32_t>(i));

  int img_off = -1;  // workspace offset of the operand image in LDS
  for (;;) {
    // the next piece, taken by one lane (a vector atomic) and shared in LDS
    if (tid == 0) piece_next = atomicAdd(counter, 1);
    __syncthreads();
    const int pc = __builtin_amdgcn_readfirstlane(piece_next);
    if (pc >= npieces) break;  // uniform: every wave leaves
    const int4 pz = pieces[pc];
    const int m = __builtin_amdgcn_readfirstlane(pz.x);
    const int ta = __builtin_amdgcn_readfirstlane(pz.y), tb = __builtin_amdgcn_readfirstlane(pz.z);
    const MultiModule md = mods[m];
    const int K = md.K, G = K / kGroup, RB = K / 4;
    const int S = (G + GPS - 1) / GPS;
    const int nch = multi_nch(K);
    // the module's operand image and group sums into LDS, unless the
    // previous piece left the same image there (the same module, or another
    // module reading the same input)
    if (md.ws_off != img_off) {
      img_off = md.ws_off;
      const char* img = ws + md.ws_off;
      const int rows = nch * 8 * kXfLimbs;
      for (int i = tid; i < rows * 8; i += kMultiThreads) {
        const int r = i >> 3, q = i & 7;
        *reinterpret_cast<uint4*>(lds_a + r * kMultiArow + q * 16) =
            *reinterpret_cast<const uint4*>(img + r * 128 + q * 16);
      }
      const float2* xfg = reinterpret_cast<const float2*>(img + static_cast<int64_t>(nch) * kMultiImgChunk);
      for (int i = tid; i < nch * 8; i += kMultiThreads) const_cast<float2*>(lds_xf)[i] = xfg[i];
      __syncthreads();
    }

    // this wave's tiles: ta + wave + NW j, j < ntw.  The unit of the ring is
    // a pair of spans (2 p, 2 p + 1) of one tile: P2 = ceil(S / 2) pairs per
    // tile, pair steps k = j * P2 + p.
    // PQ2_0: span 2 p + h takes groups 8 p + 2 lg + h, so a pair covers 8
    // groups whatever S is
    const int P2 = FMT != kMultiMlx ? (G + 7) >> 3 : (S + 1) >> 1;
    const int ntw = ta + wave < tb ? (tb - ta - wave + NW - 1) / NW : 0;
    const int nsteps = ntw * P2;
    const auto rc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(md.codes), 0, FMT == kMultiMlx ? md.N * RB : md.N * G * multi_block_bytes(FMT),
        kRsrcWord3);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(md.scales), 0, md.N * G * 2, kRsrcWord3);
    const auto rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(md.biases), 0, md.N * G * 2, kRsrcWord3);
    const auto ry = __builtin_amdgcn_make_buffer_rsrc(md.y, 0, md.N * 4, kRsrcWord3);
    // Finished rows wait in the wave's LDS buffer and are written in bursts:
    // a store in the stream would make the compiler drain every load before
    // the next use of one.  Tile j0 + i of the wave sits at ybuf[16 i + c].
    int j0 = 0;
    auto flush = [&](int upto) {  // write tiles j0 .. upto - 1 of this wave
      for (int i = lane; i < (upto - j0) * 16; i += 64) {
        const int row = (ta - md.tile0 + wave + NW * (j0 + (i >> 4))) * M + (i & 15);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ybuf[i]), ry, row * 4, 0, 0);  // rows past N: dropped
      }
      j0 = upto;
    };
    // Lane (lg, c) loads, for pair (tile, p), the 8 code words of row
    // tile*16 + c in groups 8 p + lg and 8 p + 4 + lg (2 x 32 bytes), and the
    // 8 consecutive fp16 scales (and biases) of groups 8 p .. 8 p + 7 of that
    // row -- one 16-byte load each, shared by the row's 4 lane groups.  A pair
    // past the end loads nothing useful: its offsets lie beyond every buffer
    // and read as zero, so every ring slot is refilled unconditionally and the
    // loads stay in one static order.
    int ip = 0, it = 0;  // pair and tile of the next step to load
    const int lane_c = (ta - md.tile0 + wave) * M * RB + c * RB + lg * 32;
    const int lane_s = ((ta - md.tile0 + wave) * M + c) * G * 2;
    // The scales and biases of a round of P = 4 consecutive steps travel with
    // the round's first slot: lane group lg loads the 16 bytes of step
    // k + lg for its row (the 8 fp16 of the step's 8 groups), so the row's 4
    // lanes read one contiguous run when the steps share a tile.  The lanes
    // exchange them when the round is consumed.
    auto load = [&](int k, Pair& st, bool round_head) {
      const bool live = k < nsteps;
      if constexpr (FMT == kMultiPq2) {
        // blocks (row, 8 p + 2 lg) and (row, 8 p + 2 lg + 1): 68 contiguous
        // bytes, the 4 lane groups of a row one run of 272 (offsets past the
        // buffer read zeros; the constant parts go in soffset)
        const int row = (ta - md.tile0 + wave + it * NW) * M + c;
        const int b0 = live ? (row * G + 8 * ip + 2 * lg) * kPq2Bytes : kOob;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v4u u = __builtin_amdgcn_raw_buffer_load_b128(rc, b0, 16 * q, 0);
          st.d[4 * q] = u.x; st.d[4 * q + 1] = u.y; st.d[4 * q + 2] = u.z; st.d[4 * q + 3] = u.w;
        }
        st.d[16] = __builtin_amdgcn_raw_buffer_load_b32(rc, b0, 64, 0);
        if (++ip == P2) {
          ip = 0;
          ++it;
        }
        return;
      } else if constexpr (FMT == kMultiPtq1) {
        // blocks (row, 8 p + 2 lg) and (row, 8 p + 2 lg + 1): 56 contiguous bytes
        const int row = (ta - md.tile0 + wave + it * NW) * M + c;
        const int b0 = live ? (row * G + 8 * ip + 2 * lg) * kPtq1Bytes : kOob;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          const v4u u = __builtin_amdgcn_raw_buffer_load_b128(rc, b0, 16 * q, 0);
          st.d[4 * q] = u.x; st.d[4 * q + 1] = u.y; st.d[4 * q + 2] = u.z; st.d[4 * q + 3] = u.w;
        }
        const v2u u = __builtin_amdgcn_raw_buffer_load_b64(rc, b0, 48, 0);
        st.d[12] = u.x;
        st.d[13] = u.y;
        if (++ip == P2) {
          ip = 0;
          ++it;
        }
        return;
      } else {
      const int oc = live ? lane_c + it * (NW * M * RB) + ip * 256 : kOob;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const v4u u = __builtin_amdgcn_raw_buffer_load_b128(rc, oc + (h >> 1) * 128 + (h & 1) * 16, 0, 0);
        st.w[h] = make_uint4(u.x, u.y, u.z, u.w);
      }
      if (round_head) {
        int jp = ip + lg, jt = it;
        while (jp >= P2) {
          jp -= P2;
          ++jt;
        }
        const int os = k + lg < nsteps ? lane_s + jt * (NW * M * G * 2) + jp * 16 : kOob;
        const v4u us = __builtin_amdgcn_raw_buffer_load_b128(rs, os, 0, 0);
        const v4u ub = __builtin_amdgcn_raw_buffer_load_b128(rb, os, 0, 0);
        st.s = make_uint4(us.x, us.y, us.z, us.w);
        st.b = make_uint4(ub.x, ub.y, ub.z, ub.w);
      }
      if (++ip == P2) {
        ip = 0;
        ++it;
      }
      }
    };
    static_assert(P % 4 == 0, "a round of scale loads covers 4 ring slots");
    Pair ring[P];
#pragma unroll
    for (int k = 0; k < P; ++k) load(k, ring[k], k % 4 == 0);

    uint4 av[kWordsPerGroup];
#pragma unroll
    for (int w = 0; w < kWordsPerGroup; ++w) av[w] = make_uint4(0, 0, 0, 0);
    float yacc = 0.f;
    int p = 0, j = 0;  // pair and tile of the step being consumed
    // one span: 8 MFMAs of the lane's (row, group) words against the A rows
    // of groups 4 s .. 4 s + 3, then the fp16 scale and bias in fp32
    auto span = [&](int s, const uint4& w0, const uint4& w1, uint32_t sdw, uint32_t bdw) {
      const float2 xf = lds_xf[s * GPS + lg];
      if (a_lane) {
        const uint4* ap = reinterpret_cast<const uint4*>(lds_a + ((s * GPS + alg) * kXfLimbs + ar) * kMultiArow);
#pragma unroll
        for (int w = 0; w < kWordsPerGroup; ++w) av[w] = ap[w];
      }
      v4i bop[kWordsPerGroup];
      bop[0] = decode_word(w0.x);
      bop[1] = decode_word(w0.y);
      bop[2] = decode_word(w0.z);
      bop[3] = decode_word(w0.w);
      bop[4] = decode_word(w1.x);
      bop[5] = decode_word(w1.y);
      bop[6] = decode_word(w1.z);
      bop[7] = decode_word(w1.w);
      v4i acc0 = {}, acc1 = {};
#pragma unroll
      for (int w = 0; w < kWordsPerGroup; w += 2) {
        acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(v4i{(int)av[w].x, (int)av[w].y, (int)av[w].z, (int)av[w].w},
                                                     bop[w], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
            v4i{(int)av[w + 1].x, (int)av[w + 1].y, (int)av[w + 1].z, (int)av[w + 1].w}, bop[w + 1], acc1, 0, 0, 0);
      }
      const v4i acc = acc0 + acc1;
      // the lane's fp16 scale / bias: half (lg & 1) of the dword it was given
      const float sc = half_bits_to_float(static_cast<uint16_t>(sdw >> (16 * (lg & 1))));
      const float bi = half_bits_to_float(static_cast<uint16_t>(bdw >> (16 * (lg & 1))));
      const float v = static_cast<float>(acc[3]) * 16777216.f + static_cast<float>(acc[2]) * 65536.f +
                      static_cast<float>(acc[1]) * 256.f + static_cast<float>(acc[0]);
      // groups past K (padding of the last span) contribute nothing
      yacc += s * GPS + lg < G ? sc * (v * xf.y) + bi * xf.x : 0.f;
    };
    // PQ2_0 span h of pair p: group 8 p + 2 lg + h of the lane's row (A rows
    // of group 8 p + 2 alg + h); block 0 of the pair: scale in bytes 0-1,
    // codes from byte 2 (byte-aligned); block 1: scale in bytes 34-35, codes
    // in dwords 9-16.  bias = -scale.
    auto span_pq2 = [&](int pp, int h, const uint32_t* d) {
      const int g = 8 * pp + 2 * lg + h;
      const float2 xf = lds_xf[g];
      if (a_lane) {
        const uint4* ap =
            reinterpret_cast<const uint4*>(lds_a + ((8 * pp + 2 * alg + h) * kXfLimbs + ar) * kMultiArow);
#pragma unroll
        for (int w = 0; w < kWordsPerGroup; ++w) av[w] = ap[w];
      }
      const uint32_t sbits = h ? d[8] >> 16 : d[0];
      v4i acc0 = {}, acc1 = {};
#pragma unroll
      for (int w = 0; w < kWordsPerGroup; w += 2) {
        const uint32_t c0 = h ? d[9 + w] : __builtin_amdgcn_alignbyte(d[w + 1], d[w], 2);
        const uint32_t c1 = h ? d[10 + w] : __builtin_amdgcn_alignbyte(d[w + 2], d[w + 1], 2);
        acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(v4i{(int)av[w].x, (int)av[w].y, (int)av[w].z, (int)av[w].w},
                                                     decode_word(c0), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
            v4i{(int)av[w + 1].x, (int)av[w + 1].y, (int)av[w + 1].z, (int)av[w + 1].w}, decode_word(c1), acc1, 0, 0, 0);
      }
      const v4i acc = acc0 + acc1;
      const float sc = half_bits_to_float(static_cast<uint16_t>(sbits));
      const float v = static_cast<float>(acc[3]) * 16777216.f + static_cast<float>(acc[2]) * 65536.f +
                      static_cast<float>(acc[1]) * 256.f + static_cast<float>(acc[0]);
      yacc += g < G ? sc * (v * xf.y - xf.x) : 0.f;
    };
    // PTQ1_0 span h of pair p: group 8 p + 2 lg + h; block h at byte 28 h of
    // the pair (scale first, then 26 trit bytes); the table turns each trit
    // byte into its five codes at bits 10 i .. 10 i + 9 of the 256 code bits
    auto span_ptq1 = [&](int pp, int h, const uint32_t* d) {
      const int g = 8 * pp + 2 * lg + h;
      const float2 xf = lds_xf[g];
      if (a_lane) {
        const uint4* ap =
            reinterpret_cast<const uint4*>(lds_a + ((8 * pp + 2 * alg + h) * kXfLimbs + ar) * kMultiArow);
#pragma unroll
        for (int w = 0; w < kWordsPerGroup; ++w) av[w] = ap[w];
      }
      // the group's 128 codes as bytes in natural order (the operand image of
      // PTQ1_0 plans is in natural order too)
      uint32_t cb[32];
      ptq1_code_bytes([&](int i) {
        const int byte = kPtq1Bytes * h + 2 + i;
        return (d[byte >> 2] >> (8 * (byte & 3))) & 0xFFu;
      }, lut, cb);
      const uint32_t sbits = d[7 * h] & 0xFFFFu;
      v4i acc0 = {}, acc1 = {};
#pragma unroll
      for (int w = 0; w < kWordsPerGroup; w += 2) {
        acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
            v4i{(int)av[w].x, (int)av[w].y, (int)av[w].z, (int)av[w].w},
            v4i{(int)cb[4 * w], (int)cb[4 * w + 1], (int)cb[4 * w + 2], (int)cb[4 * w + 3]}, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
            v4i{(int)av[w + 1].x, (int)av[w + 1].y, (int)av[w + 1].z, (int)av[w + 1].w},
            v4i{(int)cb[4 * w + 4], (int)cb[4 * w + 5], (int)cb[4 * w + 6], (int)cb[4 * w + 7]}, acc1, 0, 0, 0);
      }
      const v4i acc = acc0 + acc1;
      const float sc = half_bits_to_float(static_cast<uint16_t>(sbits));
      const float v = static_cast<float>(acc[3]) * 16777216.f + static_cast<float>(acc[2]) * 65536.f +
                      static_cast<float>(acc[1]) * 256.f + static_cast<float>(acc[0]);
      yacc += g < G ? sc * (v * xf.y - xf.x) : 0.f;
    };
    // Step sl of a round needs, from lane group sl of its row, dword
    // (lg >> 1) of the step's 8 halves for the pair's first span and dword
    // 2 + (lg >> 1) for its second (the lane's group is 8 p + lg / 8 p + 4 + lg).
    // Lanes pass that pair of dwords on with the lane-group swaps: a swap of
    // 16 lanes links lane groups of the same class (lg >> 1), a swap of 32
    // lanes the other class, so each lane sends the class's pair it will be
    // read for.  sN / bN: the scale / bias dwords from lane group lg ^ N.
    const bool k1 = lg >= 2;
    uint32_t s0x = 0, s0y = 0, s1x = 0, s1y = 0, s2x = 0, s2y = 0, s3x = 0, s3y = 0;
    uint32_t b0x = 0, b0y = 0, b1x = 0, b1y = 0, b2x = 0, b2y = 0, b3x = 0, b3y = 0;
    auto xl = [&](uint32_t v, int j) { return static_cast<uint32_t>(xor_lane_i(static_cast<int>(v), j, lane)); };
    if constexpr (FMT != kMultiMlx) {
      for (int base = 0; base < nsteps; base += P) {
#pragma unroll
        for (int sl = 0; sl < P; ++sl) {
          const Pair cur = ring[sl];
          load(base + sl + P, ring[sl], false);  // refill the slot before computing on its data
          if (base + sl < nsteps) {
            if constexpr (FMT == kMultiPq2) {
              span_pq2(p, 0, cur.d);
              span_pq2(p, 1, cur.d);
            } else {
              span_ptq1(p, 0, cur.d);
              span_ptq1(p, 1, cur.d);
            }
            if (++p == P2) {
              float t = yacc + xor_lane(yacc, 4, lane);
              t += xor_lane(t, 5, lane);
              if (lg == 0) ybuf[(j - j0) * 16 + c] = t;
              yacc = 0.f;
              p = 0;
              if (++j - j0 == kMultiYbuf) flush(j);
            }
          }
        }
      }
    } else {
    for (int base = 0; base < nsteps; base += P) {
#pragma unroll
      for (int sl = 0; sl < P; ++sl) {
        const Pair cur = ring[sl];
        if (sl % 4 == 0) {
          const uint32_t osx = k1 ? cur.s.y : cur.s.x, osy = k1 ? cur.s.w : cur.s.z;  // own class
          const uint32_t tsx = k1 ? cur.s.x : cur.s.y, tsy = k1 ? cur.s.z : cur.s.w;  // other class
          const uint32_t obx = k1 ? cur.b.y : cur.b.x, oby = k1 ? cur.b.w : cur.b.z;
          const uint32_t tbx = k1 ? cur.b.x : cur.b.y, tby = k1 ? cur.b.z : cur.b.w;
          s0x = osx;
          s0y = osy;
          s1x = xl(osx, 4);
          s1y = xl(osy, 4);
          s2x = xl(tsx, 5);
          s2y = xl(tsy, 5);
          s3x = xl(xl(tsx, 4), 5);
          s3y = xl(xl(tsy, 4), 5);
          b0x = obx;
          b0y = oby;
          b1x = xl(obx, 4);
          b1y = xl(oby, 4);
          b2x = xl(tbx, 5);
          b2y = xl(tby, 5);
          b3x = xl(xl(tbx, 4), 5);
          b3y = xl(xl(tby, 4), 5);
        }
        load(base + sl + P, ring[sl], sl % 4 == 0);  // refill the slot before computing on its data
        if (base + sl < nsteps) {
          const int m = lg ^ (sl & 3);  // this step's halves came from lane group sl % 4
          const bool m0 = m & 1, m1 = m & 2;
          const uint32_t sdx = m1 ? (m0 ? s3x : s2x) : (m0 ? s1x : s0x);
          const uint32_t sdy = m1 ? (m0 ? s3y : s2y) : (m0 ? s1y : s0y);
          const uint32_t bdx = m1 ? (m0 ? b3x : b2x) : (m0 ? b1x : b0x);
          const uint32_t bdy = m1 ? (m0 ? b3y : b2y) : (m0 ? b1y : b0y);
          span(2 * p, cur.w[0], cur.w[1], sdx, bdx);
          if (2 * p + 1 < S) span(2 * p + 1, cur.w[2], cur.w[3], sdy, bdy);
          if (++p == P2) {
            // tile done: add the 4 lane groups and park its rows
            float t = yacc + xor_lane(yacc, 4, lane);
            t += xor_lane(t, 5, lane);
            if (lg == 0) ybuf[(j - j0) * 16 + c] = t;
            yacc = 0.f;
            p = 0;
            if (++j - j0 == kMultiYbuf) flush(j);
          }
        }
      }
    }
    }
    flush(j);
    __syncthreads();  // the next piece's number and image replace this one's
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static inline int64_t align64(int64_t v) { return (v + 63) & ~int64_t(63); }

// byte offsets of the plan's sections (each 64-byte aligned: the kernels read
// them with vector and scalar loads of up to 16 bytes)
struct PlanOffsets {
  int64_t modules, tasks, pieces, total;
};
static PlanOffsets plan_offsets(int64_t count, int64_t ntasks, int64_t npieces) {
  PlanOffsets o;
  o.modules = sizeof(MultiHeader);
  o.tasks = align64(o.modules + count * static_cast<int64_t>(sizeof(MultiModule)));
  o.pieces = align64(o.tasks + ntasks * 8);
  o.total = align64(o.pieces + npieces * 16);
  return o;
}

// The pieces of the concatenated tile list, as (module, first tile, end tile)
// with global tile indices.  A tile costs its weight groups plus 2 (its
// scale / bias rows and fixed work); a piece takes tiles of one module until
// its cost reaches max(floor, left / grid), where left is the cost not yet
// cut, rounded up to a multiple of the workgroup's waves (or the module's
// last tiles), so pieces shrink toward the end and the last ones even out
// the workgroups' finishing times.
static std::vector<std::array<int32_t, 3>> multi_pieces(const tb_gemv_module* mods, int64_t count, int grid) {
  int64_t total = 0;
  for (int64_t i = 0; i < count; ++i)
    if (mods[i].N > 0) total += (mods[i].N + 15) / 16 * (mods[i].K / 128 + 2);
  const int64_t floor_cost = std::max<int64_t>(1, total / (static_cast<int64_t>(grid) * kMultiPieceFloor));
  std::vector<std::array<int32_t, 3>> out;
  int64_t left = total, tile = 0;
  for (int64_t i = 0; i < count; ++i) {
    const tb_gemv_module& m = mods[i];
    if (m.N <= 0) continue;
    const int64_t ntm = (m.N + 15) / 16, tc = m.K / 128 + 2;
    int64_t t = 0;
    while (t < ntm) {
      const int64_t want = std::max(floor_cost, left / static_cast<int64_t>(grid));
      // whole rounds of the workgroup's waves: a piece's tiles are dealt
      // round robin and its waves meet at a barrier when it ends
      const int64_t tiles = std::max<int64_t>(1, (want + tc - 1) / tc);
      const int64_t take = std::min(ntm - t, (tiles + kMultiWaves - 1) / kMultiWaves * kMultiWaves);
      out.push_back({static_cast<int32_t>(i), static_cast<int32_t>(tile + t), static_cast<int32_t>(tile + t + take)});
      t += take;
      left -= take * tc;
    }
    tile += ntm;
  }
  return out;
}

// Modules that read the same input -- the same x and sign vector at the same
// width, as q/k/v_proj, gate/up_proj and in_proj_qkv/z of one layer do --
// share one operand image and its transform tasks.  Per module: the first
// module of the list with the same input (the image's owner; itself for
// modules that are skipped or own their image).
static std::vector<int64_t> multi_image_owner(const tb_gemv_module* mods, int64_t count) {
  std::vector<int64_t> owner(static_cast<size_t>(count));
  std::map<std::tuple<const void*, const int8_t*, int64_t>, int64_t> first;
  for (int64_t i = 0; i < count; ++i) {
    owner[i] = i;
    if (mods[i].N <= 0) continue;
    owner[i] = first.emplace(std::make_tuple(mods[i].x, mods[i].signs, mods[i].K), i).first->second;
  }
  return owner;
}

static int64_t multi_total_tasks(const tb_gemv_module* mods, int64_t count) {
  const std::vector<int64_t> owner = multi_image_owner(mods, count);
  int64_t t = 0;
  for (int64_t i = 0; i < count; ++i)
    if (mods[i].N > 0 && owner[i] == i) t += multi_nch(static_cast<int>(mods[i].K));
  return t;
}

}  // namespace tb

using namespace tb;

extern "C" size_t tb_gemv_multi_plan_size(const tb_gemv_module* mods, int64_t count) {
  if (!mods || count <= 0) return 0;
  for (int64_t i = 0; i < count; ++i)
    if (mods[i].N < 0 || mods[i].K <= 0) return 0;  // the plan call reports the error
  const int64_t np = static_cast<int64_t>(multi_pieces(mods, count, device_cus()).size());
  return static_cast<size_t>(plan_offsets(count, multi_total_tasks(mods, count), np).total);
}

static int multi_plan(const tb_gemv_module* mods, int64_t count, int x_dtype, int block, int fmt, void* plan,
                      size_t plan_bytes, size_t* workspace_bytes, const char* who) {
  if (!mods || count <= 0 || !plan || !workspace_bytes) {
    set_error("%s: null argument or empty module list", who);
    return TB_ERR_ARG;
  }
  if (!(block == 0 || block == 512 || block == 1024)) {
    set_error("%s: block %d: the multi-module path takes 0, 512 or 1024", who, block);
    return block_known(block) ? TB_ERR_UNSUPPORTED : TB_ERR_BLOCK;
  }
  if (x_dtype != TB_F32 && x_dtype != TB_BF16) {
    set_error("%s: x_dtype %d is not TB_F32 or TB_BF16", who, x_dtype);
    return TB_ERR_DTYPE;
  }
  if (count > (1 << 20)) {
    set_error("%s: %lld modules is more than the plan format takes", who, (long long)count);
    return TB_ERR_ARG;
  }
  int max_nch = 1;
  int64_t tiles = 0, ws = 0;
  for (int64_t i = 0; i < count; ++i) {
    const tb_gemv_module& m = mods[i];
    if (m.N < 0 || m.K <= 0) {
      set_error("%s: module %lld: N=%lld K=%lld", who, (long long)i, (long long)m.N, (long long)m.K);
      return TB_ERR_ARG;
    }
    if (m.K % 256 != 0 || (block > 0 && m.K % block != 0)) {
      set_error("%s: module %lld: K=%lld must be a multiple of 256 and of the block", who, (long long)i,
                (long long)m.K);
      return TB_ERR_SHAPE;
    }
    if (m.N == 0) continue;
    if (fmt != kMultiMlx) {
      if (!m.x || !m.codes || m.scales || m.biases || !m.y || (block > 0) != (m.signs != nullptr)) {
        set_error("%s: module %lld: null pointer, or scales / biases given (the blocks carry the scales; signs "
                  "must be given exactly when block > 0)", who, (long long)i);
        return TB_ERR_ARG;
      }
      if (!aligned(m.x, 16) || !aligned(m.codes, 4) || !aligned(m.y, 4) || (m.signs && !aligned(m.signs, 4))) {
        set_error("%s: module %lld: x needs 16-byte, blocks, y and signs 4-byte alignment", who, (long long)i);
        return TB_ERR_ALIGN;
      }
    } else {
      if (!m.x || !m.codes || !m.scales || !m.biases || !m.y || (block > 0) != (m.signs != nullptr)) {
        set_error("%s: module %lld: null pointer (signs must be given exactly when block > 0)", who, (long long)i);
        return TB_ERR_ARG;
      }
      if (!aligned(m.x, 16) || !aligned(m.codes, 16) || !aligned(m.scales, 4) || !aligned(m.biases, 4) ||
          !aligned(m.y, 4) || (m.signs && !aligned(m.signs, 4))) {
        set_error("%s: module %lld: x and codes need 16-byte, scales, biases, y and signs 4-byte alignment", who,
                  (long long)i);
        return TB_ERR_ALIGN;
      }
    }
    if (m.N > (1 << 26) || m.K > (1 << 20) || m.N * (m.K / 4) > INT32_MAX ||
        (m.N + 16) * (m.K / kGroup) * kPq2Bytes + 512 > INT32_MAX) {
      set_error("%s: module %lld: N=%lld K=%lld is too large for one module", who, (long long)i, (long long)m.N,
                (long long)m.K);
      return TB_ERR_SHAPE;
    }
    const int nch = multi_nch(static_cast<int>(m.K));
    max_nch = std::max(max_nch, nch);
    tiles += (m.N + 15) / 16;
  }
  const std::vector<int64_t> owner = multi_image_owner(mods, count);
  for (int64_t i = 0; i < count; ++i)
    if (mods[i].N > 0 && owner[i] == i) ws += static_cast<int64_t>(multi_nch(static_cast<int>(mods[i].K))) * (kMultiImgChunk + 64);
  if (multi_lds_total(max_nch) > kMultiLdsMax) {
    set_error("%s: K up to %d takes too much LDS for the stream kernel", who, max_nch * 1024);
    return TB_ERR_UNSUPPORTED;
  }
  if (tiles >= INT32_MAX || ws >= INT32_MAX) {
    set_error("%s: the module list is too large for one plan", who);
    return TB_ERR_SHAPE;
  }
  const int grid = device_cus();
  const int64_t ntasks = multi_total_tasks(mods, count);
  const std::vector<std::array<int32_t, 3>> pcs = multi_pieces(mods, count, grid);
  if (pcs.size() >= (size_t(1) << 30) ||
      plan_offsets(count, ntasks, static_cast<int64_t>(pcs.size())).total >= INT32_MAX) {
    set_error("%s: the module list is too large for one plan", who);
    return TB_ERR_SHAPE;
  }
  const PlanOffsets po = plan_offsets(count, ntasks, static_cast<int64_t>(pcs.size()));
  const size_t need = static_cast<size_t>(po.total);
  if (plan_bytes < need) {
    set_error("%s: plan buffer of %zu bytes, %zu needed", who, plan_bytes, need);
    return TB_ERR_WORKSPACE;
  }
  char* p = static_cast<char*>(plan);
  std::memset(p, 0, need);
  MultiHeader hd{};
  hd.magic = kPlanMagic;
  hd.count = static_cast<int32_t>(count);
  hd.tasks = static_cast<int32_t>(ntasks);
  hd.grid = grid;
  hd.block = block;
  hd.x_dtype = x_dtype;
  hd.max_nch = max_nch;
  hd.pieces = static_cast<int32_t>(pcs.size());
  hd.modules_off = po.modules;
  hd.tasks_off = po.tasks;
  hd.pieces_off = po.pieces;
  hd.total_bytes = static_cast<int32_t>(need);
  hd.format = fmt;
  std::memcpy(p, &hd, sizeof hd);
  MultiModule* md = reinterpret_cast<MultiModule*>(p + hd.modules_off);
  int32_t* tk = reinterpret_cast<int32_t*>(p + hd.tasks_off);
  std::vector<int64_t> img_off(static_cast<size_t>(count), 0);  // per image owner: its workspace offset
  int64_t t0 = 0, off = kMultiWsHead, nt = 0;
  for (int64_t i = 0; i < count; ++i) {
    const tb_gemv_module& m = mods[i];
    MultiModule d{};
    d.x = m.x;
    d.signs = m.signs;
    d.codes = m.codes;
    d.scales = m.scales;
    d.biases = m.biases;
    d.y = m.y;
    d.N = static_cast<int32_t>(m.N);
    d.K = static_cast<int32_t>(m.K);
    d.tile0 = static_cast<int32_t>(t0);
    const bool owns = owner[i] == i;
    if (m.N > 0 && owns) img_off[i] = off;
    d.ws_off = static_cast<int32_t>(m.N > 0 ? img_off[owner[i]] : off);
    std::memcpy(md + i, &d, sizeof d);
    if (m.N == 0) continue;
    t0 += (m.N + 15) / 16;
    if (!owns) continue;  // the owner's tasks write the shared image
    const int nch = multi_nch(static_cast<int>(m.K));
    for (int c = 0; c < nch; ++c) {
      tk[2 * nt] = static_cast<int32_t>(i);
      tk[2 * nt + 1] = c;
      ++nt;
    }
    off += static_cast<int64_t>(nch) * (kMultiImgChunk + 64);
  }
  int32_t* pq = reinterpret_cast<int32_t*>(p + hd.pieces_off);
  for (size_t k = 0; k < pcs.size(); ++k) {
    pq[4 * k] = pcs[k][0];
    pq[4 * k + 1] = pcs[k][1];
    pq[4 * k + 2] = pcs[k][2];
    pq[4 * k + 3] = 0;
  }
  *workspace_bytes = static_cast<size_t>(kMultiWsHead + ws);
  return TB_OK;
}

extern "C" int tb_gemv_multi_plan(const tb_gemv_module* mods, int64_t count, int x_dtype, int block, void* plan,
                                  size_t plan_bytes, size_t* workspace_bytes) {
  return multi_plan(mods, count, x_dtype, block, kMultiMlx, plan, plan_bytes, workspace_bytes, "tb_gemv_multi_plan");
}

extern "C" int tb_pq2_gemv_multi_plan(const tb_gemv_module* mods, int64_t count, int x_dtype, int block, void* plan,
                                      size_t plan_bytes, size_t* workspace_bytes) {
  return multi_plan(mods, count, x_dtype, block, kMultiPq2, plan, plan_bytes, workspace_bytes,
                    "tb_pq2_gemv_multi_plan");
}

extern "C" int tb_ptq1_gemv_multi_plan(const tb_gemv_module* mods, int64_t count, int x_dtype, int block,
                                       void* plan, size_t plan_bytes, size_t* workspace_bytes) {
  return multi_plan(mods, count, x_dtype, block, kMultiPtq1, plan, plan_bytes, workspace_bytes,
                    "tb_ptq1_gemv_multi_plan");
}

template <int L, int DT>
static void multi_prep_launch(const void* plan, void* ws, int tasks, bool natural, hipStream_t st) {
  if (natural)
    hipLaunchKernelGGL((multi_prep_kernel<L, DT, true>), dim3((tasks + 3) / 4), dim3(256), 0, st,
                       static_cast<const char*>(plan), static_cast<char*>(ws));
  else
    hipLaunchKernelGGL((multi_prep_kernel<L, DT, false>), dim3((tasks + 3) / 4), dim3(256), 0, st,
                       static_cast<const char*>(plan), static_cast<char*>(ws));
}

template <int NW, int P, int FMT>
static void multi_stream_launch(const void* plan, void* ws, int grid, size_t lds, hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};
  lds_limit_once(reinterpret_cast<const void*>(multi_stream_kernel<NW, P, FMT>), static_cast<int>(kMultiLdsMax),
                 lds_set);
  hipLaunchKernelGGL((multi_stream_kernel<NW, P, FMT>), dim3(grid), dim3(64 * NW), lds, st,
                     static_cast<const char*>(plan), static_cast<char*>(ws));
}

extern "C" int tb_ternary_gemv_multi(const void* plan_host, const void* plan_device, void* workspace,
                                     size_t ws_bytes, void* stream) {
  const char* who = "tb_ternary_gemv_multi";
  if (!plan_host || !plan_device || !workspace) {
    set_error("%s: null plan or workspace", who);
    return TB_ERR_ARG;
  }
  MultiHeader hd;
  std::memcpy(&hd, plan_host, sizeof hd);
  if (hd.magic != kPlanMagic || hd.count <= 0 || hd.grid <= 0 || hd.pieces < 0 ||
      (hd.format != kMultiMlx && hd.format != kMultiPq2 && hd.format != kMultiPtq1)) {
    set_error("%s: the host plan was not built by tb_gemv_multi_plan", who);
    return TB_ERR_ARG;
  }
  if (!aligned(plan_device, 16) || !aligned(workspace, 16)) {
    set_error("%s: plan and workspace need 16-byte alignment", who);
    return TB_ERR_ALIGN;
  }
  // the workspace size the plan needs: the last module's image end
  const MultiModule* md = reinterpret_cast<const MultiModule*>(static_cast<const char*>(plan_host) + hd.modules_off);
  int64_t need = kMultiWsHead;
  for (int i = 0; i < hd.count; ++i)
    if (md[i].N > 0) need = std::max<int64_t>(need, md[i].ws_off + static_cast<int64_t>(multi_nch(md[i].K)) * (kMultiImgChunk + 64));
  if (ws_bytes < static_cast<size_t>(need)) {
    set_error("%s: workspace of %zu bytes, %lld needed", who, ws_bytes, (long long)need);
    return TB_ERR_WORKSPACE;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hd.tasks > 0) {
    const int L = hd.block;
    const bool nat = hd.format == kMultiPtq1;  // PTQ1_0: the operand image in natural element order
    if (hd.x_dtype == TB_F32) {
      if (L == 0) multi_prep_launch<0, TB_F32>(plan_device, workspace, hd.tasks, nat, st);
      else if (L == 512) multi_prep_launch<512, TB_F32>(plan_device, workspace, hd.tasks, nat, st);
      else multi_prep_launch<1024, TB_F32>(plan_device, workspace, hd.tasks, nat, st);
    } else {
      if (L == 0) multi_prep_launch<0, TB_BF16>(plan_device, workspace, hd.tasks, nat, st);
      else if (L == 512) multi_prep_launch<512, TB_BF16>(plan_device, workspace, hd.tasks, nat, st);
      else multi_prep_launch<1024, TB_BF16>(plan_device, workspace, hd.tasks, nat, st);
    }
    TB_LAUNCH_CHECK(who);
    const size_t lds = static_cast<size_t>(multi_lds_total(hd.max_nch));
    if (hd.format == kMultiPq2) multi_stream_launch<kMultiWaves, kMultiRing, kMultiPq2>(plan_device, workspace, hd.grid, lds, st);
    else if (hd.format == kMultiPtq1) multi_stream_launch<kMultiWaves, kMultiRing, kMultiPtq1>(plan_device, workspace, hd.grid, lds, st);
    else multi_stream_launch<kMultiWaves, kMultiRing, kMultiMlx>(plan_device, workspace, hd.grid, lds, st);
    TB_LAUNCH_CHECK(who);
  }
  return TB_OK;
}
