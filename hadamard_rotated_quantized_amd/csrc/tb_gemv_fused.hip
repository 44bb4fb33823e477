// Single-launch Packed linear for decode batches: the signed block transform,
// the exact integer split and the weight-streaming 2-bit matmul in one kernel
// [lpnh.cn/news/2438023, "text model loading"; kwkr.cn/news/564617,
// "ternary weights + folded Hadamard rotation"].
//
// A decode call is short (q_proj: 8.8 MB of weights, about a microsecond of
// HBM time), so its cost is a chain of latencies, and the work every
// workgroup repeats (the transform of the input) competes with the stream
// for the VALUs.  The kernel is built around that:
//
// * every argument the loads need arrives in SGPRs preloaded by the
//   dispatcher (the library is built with kernarg preloading), so a wave
//   issues its first loads without waiting for a kernel-argument fetch;
// * every wave first issues the loads of its activation chunks, then the
//   weight loads of its first items (a ring of 4 kept in flight), and only
//   then waits -- for the activations alone, since loads complete in order;
// * each workgroup transforms the whole input row(s) itself, one 1024-input
//   chunk per wave, into LDS, while its weights are in flight.  Index bits
//   0-3 of a chunk are in-lane, bits 4-5 are exchanged with DPP quad
//   permutations, and bits 6-9 are brought in-lane by an LDS transpose, so
//   the butterflies cost about a third of an all-lane-exchange version;
// * small layers ("split" mode) get one workgroup per CU, each owning a
//   band of about N / CUs rows cut into subtiles of M rows; the 8 waves deal
//   the (subtile, span) items round robin, park their partial sums in LDS
//   and add them up once at the end.  Wide layers ("persistent" mode) give
//   every wave whole tiles and loop the workgroups over tile groups.
//
// Used when one workgroup can afford the transform: block 0, 512 or 1024,
// at most 3 chunk transforms per wave (batch x K/1024 <= 24) and an LDS
// footprint within the limit; tb_ternary_gemv takes the two-kernel path
// otherwise.
#include <algorithm>

#include "tb_gemv.h"

namespace tb {

constexpr int kFusedWaves = 8;
constexpr int kFusedThreads = 64 * kFusedWaves;
constexpr int kFusedChunksPerWave = 3;
constexpr int kFusedRing = 4;
constexpr int kFusedMaxSub = 7;        // subtiles per workgroup in split mode (3 bits of cfg)
constexpr int kScratchFloats = 64 * 17;  // per-wave transpose area (64 rows of 16 + 1 pad)
constexpr int64_t kFusedLdsMax = 150 * 1024;
constexpr int kPersistent = 0, kSplitRing = 1, kSplitStaged = 2;  // kernel modes
constexpr int kStageSlot = 1024 + 16;  // LDS bytes per staged 1 KB of band
constexpr int kStageLoads = 6;         // direct-to-LDS loads per wave: at most 48 KB of band codes
constexpr int kStagedItems = 4;        // items per wave in the staged mode
// s_waitcnt immediate with vmcnt(0) and the other counters left alone
constexpr int kWaitVmcnt0 = (0x7 << 4) | (0xF << 8);

// LDS layout (bytes): 8 zero uint4; limbs [B][Gp][3] rows of kLdsRow uint4;
// (f * sum q, f) float2 [B][Gp]; per-wave transpose scratch; split mode:
// partial sums float [tsub][8 waves][NB][M].
struct FusedLds {
  int64_t limbs, xf, scratch, red, total;
};
__host__ __device__ inline FusedLds fused_lds_layout(int64_t B, int64_t Gp, int64_t red_floats) {
  FusedLds l;
  l.limbs = 16 * kWordsPerGroup;
  l.xf = l.limbs + B * Gp * kLimbs * kLdsRow * 16;
  l.scratch = l.xf + B * Gp * 8;
  l.red = l.scratch + (int64_t)kFusedWaves * kScratchFloats * 4;
  l.total = l.red + red_floats * 4;
  return l;
}

struct FusedSpan {
  uint4 w0, w1;       // 8 code words of (row, group)
  uint16_t s, bias;   // fp16 bits, converted at use so the load does not wait
};

// Signed transform of one 1024-input chunk held 16 per lane (lane l: inputs
// 16 l + r), natural-order Sylvester butterflies [trdm.cn/news/822023
// section 2.2], scaled by 1/sqrt(L).  For L = 512 the two halves of the chunk
// are separate blocks (index bit 9 is not combined).  scratch: this wave's
// kScratchFloats of LDS.
template <int L>
__device__ __forceinline__ void transform_chunk(float v[16], int lane, float* scratch) {
  // bits 0-3 in-lane
#pragma unroll
  for (int hb = 1; hb < 16; hb <<= 1)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (!(r & hb)) {
        const float a0 = v[r], a1 = v[r + hb];
        v[r] = a0 + a1;
        v[r + hb] = a0 - a1;
      }
  // bits 4, 5 = lane bits 0, 1: lower lane v + p, upper lane p - v
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = xor_lane(v[r], j, lane);
    const float sgn = ((lane >> j) & 1) ? -1.f : 1.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = fmaf(sgn, v[r], p[r]);
  }
  // transpose: input k = 16 lane + r goes to row k & 63, column k >> 6 of a
  // 64 x 17 array; lane l' then reads row l', i.e. inputs l' + 64 r'
#pragma unroll
  for (int r = 0; r < 16; ++r) scratch[(16 * (lane & 3) + r) * 17 + (lane >> 2)] = v[r];
  float w[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) w[r] = scratch[lane * 17 + r];
  // bits 6-9 (6-8 for 512-blocks) in-lane
  constexpr int TOP = L == 512 ? 8 : 16;
#pragma unroll
  for (int hb = 1; hb < TOP; hb <<= 1)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (!(r & hb)) {
        const float a0 = w[r], a1 = w[r + hb];
        w[r] = a0 + a1;
        w[r + hb] = a0 - a1;
      }
  // back to 16 consecutive inputs per lane (plain layout k)
#pragma unroll
  for (int r = 0; r < 16; ++r) scratch[lane + 64 * r] = w[r];
  const float sc = inv_sqrt_block<L>();
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float4 f = *reinterpret_cast<const float4*>(scratch + 16 * lane + 4 * e);
    v[4 * e] = f.x * sc;
    v[4 * e + 1] = f.y * sc;
    v[4 * e + 2] = f.z * sc;
    v[4 * e + 3] = f.w * sc;
  }
}

// cfg: batch rows B (bits 0-3), remainder flag (bit 4), subtiles per
// workgroup (bits 5-7, split modes), grid size (bits 8-31).  aux: split modes, rows per workgroup;
// persistent mode, tile groups (8 tiles of M rows).  The 14 argument SGPRs
// the dispatcher can preload (16 user SGPRs minus the kernel-argument
// pointer) hold everything but y, which is needed last.
//
// MODE kPersistent / kSplitRing stream each wave's items through a ring of
// registers; kSplitStaged first copies the codes of the workgroup's whole
// band (contiguous in memory) into LDS with direct-to-LDS buffer loads of
// 1 KB per wave instruction -- fully coalesced, where the per-item loads of
// a tile touch 16 rows per instruction -- and fetches the scale and bias of
// each of its (at most kStagedItems) items with 2-byte loads up front.
//
// Remainder flag (one batch row, kSplitRing): the band's last subtile holds
// at most 4 rows, and a 16-row MFMA item would spend three quarters of its
// decode and matmul on padding.  Those rows go through 4x4x4 MFMA blocks
// instead: a unit is 8 groups, block b = (group, half of its 8 words);
// block b's A is the 4 limb rows (limb 3 zero) of its 64 activations, its B
// the same 64 codes of the 4 rows, so D[b][limb][row] is one half-group's
// limb sums, row r's in lane 4 b + r.  Wave w takes units 7 - w, 15 - w, ...
// (the waves with fewer 16-row items first).
template <int NB, int M, int L, int DT, int MODE>
__global__ __launch_bounds__(kFusedThreads, NB == 8 ? 2 : 4) void gemv_fused_kernel(
    const void* __restrict__ x, const int8_t* __restrict__ signs, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases, int N, int K, int cfg, int aux,
    float* __restrict__ y) {
  using MF = Mfma<M>;
  constexpr bool SPLIT = MODE != kPersistent;
  constexpr bool STAGED = MODE == kSplitStaged;
  constexpr int GPS = MF::GPS, BPI = MF::BPI;
  constexpr int NBC = (NB + BPI - 1) / BPI;  // MFMA chains per item
  constexpr int P = kFusedRing;
  constexpr int ESZ = DT == TB_F32 ? 4 : 2;
  constexpr int XW = 8 * ESZ / 2;            // dwords of 16 activations
  extern __shared__ uint4 lds_dyn[];

  const int B = NB == 1 ? 1 : (cfg & 15);
  const int tsub = (cfg >> 5) & 7;
  const int grid = cfg >> 8;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bid = static_cast<int>(blockIdx.x);
  const int lg = lane / M, c = lane % M;
  // A-operand role of this lane: A row c = (batch jb, group alg, limb ar) is
  // non-zero only in lane group alg == lg, for limbs 0..2.
  const int ar = c & 3;
  const int alg = (c >> 2) & (GPS - 1);
  const int ajb = c / (4 * GPS);
  const bool a_lane = (alg == lg) && (ar < kLimbs);

  const int G = K / kGroup;
  const int W = K / kCodesPerWord;
  const int Gp = (G + kGroupPad - 1) / kGroupPad * kGroupPad;
  const int S = Gp / GPS;  // spans per row band
  const int nch = (K + 1023) >> 10;

  const FusedLds lay = fused_lds_layout(B, Gp, SPLIT ? tsub * kFusedWaves * NB * M : 0);
  char* const lds_base = reinterpret_cast<char*>(lds_dyn);
  uint4* const lds_zero = lds_dyn;
  uint4* const lds_a = reinterpret_cast<uint4*>(lds_base + lay.limbs);
  float2* const lds_xf = reinterpret_cast<float2*>(lds_base + lay.xf);
  float* const scratch = reinterpret_cast<float*>(lds_base + lay.scratch) + wave * kScratchFloats;
  float* const red = reinterpret_cast<float*>(lds_base + lay.red);
  char* const stage = lds_base + lay.total;  // staged band (kSplitStaged)

  // 1. activation chunks of this wave (lane l: inputs 16 l .. 16 l + 15 of
  //    the chunk); inputs past K read as zero
  const auto rxa = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(x), 0, B * K * ESZ, kRsrcWord3);
  const auto rsg = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(signs), 0, L > 0 ? K : 0, kRsrcWord3);
  const int nitems = B * nch;
  auto item_chunk = [&](int it, int& b, int& ch) {
    b = 0;
    ch = it;
    if constexpr (NB > 1) {
      while (ch >= nch) {
        ch -= nch;
        ++b;
      }
    }
  };
  uint32_t xr[kFusedChunksPerWave][XW];
  uint32_t sr[kFusedChunksPerWave][4];
#pragma unroll
  for (int r = 0; r < kFusedChunksPerWave; ++r) {
    const int it = wave + kFusedWaves * r;
    if (it < nitems) {
      int b, ch;
      item_chunk(it, b, ch);
      const int k = ch * 1024 + 16 * lane;
      const int xo = k < K ? (b * K + k) * ESZ : kOob;
#pragma unroll
      for (int e = 0; e < XW / 4; ++e) {
        const v4u u = __builtin_amdgcn_raw_buffer_load_b128(rxa, xo + 16 * e, 0, 0);
        xr[r][4 * e] = u.x; xr[r][4 * e + 1] = u.y; xr[r][4 * e + 2] = u.z; xr[r][4 * e + 3] = u.w;
      }
      if constexpr (L > 0) {
        const v4u u = __builtin_amdgcn_raw_buffer_load_b128(rsg, k < K ? k : kOob, 0, 0);
        sr[r][0] = u.x; sr[r][1] = u.y; sr[r][2] = u.z; sr[r][3] = u.w;
      }
    }
  }

  // 2. weight stream.  An item is span s (GPS groups) of the M rows of a
  //    tile.  Split modes: the workgroup owns a band of rows, tsub subtiles
  //    of M rows; item i = t * S + s, and wave w takes items w, w + 8, ...
  //    Persistent mode: wave w owns tile 8 t + w of each tile group t =
  //    blockIdx.x, + grid, ..., all S spans of it.  The buffer resources
  //    cover exactly the band (split) or the matrix (persistent), so rows
  //    past the end read as zero; an item past the end of the wave's stream
  //    reads from an offset past any buffer.  Only the row of the tile and
  //    the lane group vary per lane, so an item's offsets are one add.
  int band0 = 0, nrows = N, total;
  if constexpr (SPLIT) {
    band0 = bid * aux;
    nrows = min(aux, N - band0);
    const int items = (tsub - ((cfg >> 4) & 1)) * S;
    total = items > wave ? (items - wave + kFusedWaves - 1) / kFusedWaves : 0;
  } else {
    total = ((aux - 1 - bid) / grid + 1) * S;
  }
  const auto rc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(codes + (int64_t)band0 * W), 0,
                                                    nrows * W * 4, kRsrcWord3);
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales + (int64_t)band0 * G), 0,
                                                    nrows * G * 2, kRsrcWord3);
  const auto rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(biases + (int64_t)band0 * G), 0,
                                                    nrows * G * 2, kRsrcWord3);
  const uint32_t lane_c = static_cast<uint32_t>(c * (W * 4) + lg * 32);
  const uint32_t lane_s = static_cast<uint32_t>(c * (G * 2) + lg * 2);
  struct Cursor {
    int j, s, t;
  };
  // first row of the cursor's tile, relative to the buffer resources
  auto tile_row = [&](const Cursor& cu) { return SPLIT ? cu.t * M : (cu.t * kFusedWaves + wave) * M; };
  auto step = [&](Cursor& cu) {
    ++cu.j;
    if constexpr (SPLIT) {
      cu.s += kFusedWaves;
      while (cu.s >= S) {
        cu.s -= S;
        ++cu.t;
      }
    } else if (++cu.s == S) {
      cu.s = 0;
      cu.t += grid;
    }
  };
  Cursor first{0, SPLIT ? wave : 0, SPLIT ? 0 : bid};
  while (first.s >= S) {
    first.s -= S;
    ++first.t;
  }
  auto load_item = [&](const Cursor& cu, FusedSpan& sp) {
    const bool live = cu.j < total;
    const uint32_t row = static_cast<uint32_t>(tile_row(cu));
    const uint32_t uc = live ? row * static_cast<uint32_t>(W * 4) + cu.s * (GPS * 32) : kOob;
    const uint32_t us = live ? row * static_cast<uint32_t>(G * 2) + cu.s * (GPS * 2) : kOob;
    const int cw = static_cast<int>(lane_c + uc);
    const v4u w0 = __builtin_amdgcn_raw_buffer_load_b128(rc, cw, 0, 0);
    const v4u w1 = __builtin_amdgcn_raw_buffer_load_b128(rc, cw + 16, 0, 0);
    sp.w0 = make_uint4(w0.x, w0.y, w0.z, w0.w);
    sp.w1 = make_uint4(w1.x, w1.y, w1.z, w1.w);
    const int so = static_cast<int>(lane_s + us);
    sp.s = __builtin_amdgcn_raw_buffer_load_b16(rs, so, 0, 0);
    sp.bias = __builtin_amdgcn_raw_buffer_load_b16(rb, so, 0, 0);
  };

  // staged codes: 1 KB slots of kStageSlot bytes (16 B of padding keeps the
  // 16 rows of an item on distinct LDS banks) in [0, ncc), then one dump
  // slot that the surplus loads (past the band) fill with zeros.  Every row
  // is a whole number of 32-byte groups, so no load straddles the band end.
  const int ncc = STAGED ? (nrows * W * 4 + 1023) >> 10 : 0;
  auto stage_at = [&](uint32_t off) {  // LDS offset of byte `off` of the staged codes
    return off + (off >> 10) * (kStageSlot - 1024);
  };

  Cursor rcur = first;
  FusedSpan ring[STAGED ? 1 : P];
  uint16_t st_s[STAGED ? kStagedItems : 1], st_b[STAGED ? kStagedItems : 1];
  if constexpr (STAGED) {
#pragma unroll
    for (int i = 0; i < kStageLoads; ++i) {
      const int q = wave + kFusedWaves * i;  // slot
      const bool real = q < ncc;
      char* dst = stage + (real ? q : ncc) * kStageSlot;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (__attribute__((address_space(3))) void*)dst, 16,
                                               real ? q * 1024 + lane * 16 : kOob, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kStagedItems; ++j) {
      const uint32_t us = rcur.j < total
                              ? static_cast<uint32_t>(tile_row(rcur)) * static_cast<uint32_t>(G * 2) +
                                    rcur.s * (GPS * 2)
                              : kOob;
      st_s[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, static_cast<int>(lane_s + us), 0, 0);
      st_b[j] = __builtin_amdgcn_raw_buffer_load_b16(rb, static_cast<int>(lane_s + us), 0, 0);
      step(rcur);
    }
  } else {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      load_item(rcur, ring[i]);
      step(rcur);
    }
  }

  // 3. transform the chunks into LDS while the weights are in flight
#pragma unroll
  for (int r = 0; r < kFusedChunksPerWave; ++r) {
    const int it = wave + kFusedWaves * r;
    if (it < nitems) {
      int b, ch;
      item_chunk(it, b, ch);
      float v[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if constexpr (DT == TB_F32) v[e] = __uint_as_float(xr[r][e]);
        else v[e] = __uint_as_float((e & 1) ? (xr[r][e >> 1] & 0xFFFF0000u) : (xr[r][e >> 1] << 16));
      }
      if constexpr (L > 0) {
        // sign flip: bit 7 of the int8 sign (+1 or -1) onto the fp32 sign bit
#pragma unroll
        for (int e = 0; e < 16; ++e)
          v[e] = __uint_as_float(__float_as_uint(v[e]) ^ ((sr[r][e >> 2] << (24 - 8 * (e & 3))) & 0x80000000u));
        transform_chunk<L>(v, lane, scratch);
      }
      uint4 limb[kLimbs];
      float2 xf;
      split_limbs(v, lane, limb, xf);
      const int g = ch * 8 + (lane >> 3), t = lane & 7;
      if (g < G) {
#pragma unroll
        for (int l = 0; l < kLimbs; ++l) lds_a[((b * Gp + g) * kLimbs + l) * kLdsRow + t] = limb[l];
        if (t == 0) lds_xf[b * Gp + g] = xf;
      }
    }
  }
  if (tid < kWordsPerGroup) lds_zero[tid] = make_uint4(0, 0, 0, 0);
  {
    // groups G .. Gp-1 pad the last span: zero limbs and (f sum q, f) make
    // whatever their code loads return contribute nothing
    const int npad = Gp - G;
    for (int i = tid; i < B * npad * kLimbs * kLdsRow; i += kFusedThreads) {
      const int b = i / (npad * kLimbs * kLdsRow), rem = i - b * (npad * kLimbs * kLdsRow);
      lds_a[(b * Gp + G) * kLimbs * kLdsRow + rem] = make_uint4(0, 0, 0, 0);
    }
    if (tid < B * npad) {
      const int b = tid / npad;
      lds_xf[b * Gp + G + (tid - b * npad)] = make_float2(0.f, 0.f);
    }
  }
  if constexpr (SPLIT) {
    for (int i = tid; i < tsub * kFusedWaves * NB * M; i += kFusedThreads) red[i] = 0.f;
  }
  // remainder units (see above): this lane is block rbk, limb and row rri
  constexpr bool REMK = NB == 1 && M == 16 && MODE == kSplitRing;
  constexpr int RR = REMK ? 3 : 1;  // units in flight per wave
  const bool remp = REMK && ((cfg >> 4) & 1);
  const int rbk = lane >> 2, rri = lane & 3;
  const int rfirst = kFusedWaves - 1 - wave;
  const int nru = (G + 7) >> 3;
  const int rtotal = remp && nru > rfirst ? (nru - rfirst + kFusedWaves - 1) / kFusedWaves : 0;
  const int rrow = (tsub - 1) * M + rri;  // band row of this lane's codes
  struct RemUnit {
    uint4 w;
    uint16_t s, bias;
  };
  auto rem_group = [&](int k) { return (rfirst + kFusedWaves * k) * 8 + (rbk >> 1); };
  auto load_rem = [&](int k, RemUnit& u) {
    const int g = rem_group(k);
    const bool live = k < rtotal && g < G;
    const int co = live ? rrow * (W * 4) + g * 32 + (rbk & 1) * 16 : kOob;
    const int so = live ? rrow * (G * 2) + g * 2 : kOob;
    const v4u w = __builtin_amdgcn_raw_buffer_load_b128(rc, co, 0, 0);
    u.w = make_uint4(w.x, w.y, w.z, w.w);
    u.s = __builtin_amdgcn_raw_buffer_load_b16(rs, so, 0, 0);
    u.bias = __builtin_amdgcn_raw_buffer_load_b16(rb, so, 0, 0);
  };
  RemUnit ru[RR];
  if (rtotal > 0) {
#pragma unroll
    for (int k = 0; k < RR; ++k) load_rem(k, ru[k]);
  }

  if constexpr (STAGED) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's band slots have landed
  __syncthreads();

  // 4. the matmul.  Ring modes: the loop is unrolled over the ring slots,
  //    and every slot is refilled unconditionally (with a zero-reading load
  //    past the end), so the loads are issued in the same static order in
  //    every iteration and each wait covers exactly the slot being consumed.
  float yacc[NB];
#pragma unroll
  for (int bq = 0; bq < NB; ++bq) yacc[bq] = 0.f;
  // LDS address of this lane's A operand for span 0, and its step per span
  // (lanes whose A rows are zero read the zero row at every span)
  const uint4* a_base[NBC];
  int a_step[NBC];
#pragma unroll
  for (int bc = 0; bc < NBC; ++bc) {
    const int bq_a = bc * BPI + ajb;
    const bool on = a_lane && bq_a < B;
    a_base[bc] = on ? lds_a + ((bq_a * Gp + alg) * kLimbs + ar) * kLdsRow : lds_zero;
    a_step[bc] = on ? GPS * kLimbs * kLdsRow : 0;
  }
  auto consume = [&](const FusedSpan& cur, int s) {
    v4i bop[kWordsPerGroup];
    bop[0] = decode_word(cur.w0.x);
    bop[1] = decode_word(cur.w0.y);
    bop[2] = decode_word(cur.w0.z);
    bop[3] = decode_word(cur.w0.w);
    bop[4] = decode_word(cur.w1.x);
    bop[5] = decode_word(cur.w1.y);
    bop[6] = decode_word(cur.w1.z);
    bop[7] = decode_word(cur.w1.w);
    // groups past K (padding of the last span) contribute nothing, whatever
    // their scale and bias loads returned
    const bool gin = s * GPS + lg < G;
    const float sc = gin ? half_bits_to_float(cur.s) : 0.f, bi = gin ? half_bits_to_float(cur.bias) : 0.f;
    const float2* xfp = lds_xf + s * GPS + lg;  // (f sum q, f) of this lane's group, batch row 0
#pragma unroll
    for (int bc = 0; bc < NBC; ++bc) {
      const uint4* ap = a_base[bc] + s * a_step[bc];
      v4i av[kWordsPerGroup];
#pragma unroll
      for (int t = 0; t < kWordsPerGroup; ++t) {
        const uint4 u = ap[t];
        av[t] = v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
      }
      // two independent accumulation chains (even and odd words)
      typename MF::acc_t acc0 = {}, acc1 = {};
#pragma unroll
      for (int t = 0; t < kWordsPerGroup; t += 2) {
        acc0 = MF::mac(av[t], bop[t], acc0);
        acc1 = MF::mac(av[t + 1], bop[t + 1], acc1);
      }
      const typename MF::acc_t acc = acc0 + acc1;
      // lane (lg, c) holds D[(4 GPS) j + 4 lg + r][c]: the limb-r sums of
      // row c, group s GPS + lg, batch row BPI bc + j  (register 4 j + r)
#pragma unroll
      for (int jj = 0; jj < BPI; ++jj) {
        const int bq = bc * BPI + jj;
        if (bq < NB && bq < B) {
          // limb 0 = low digit l, limb 1 = m, limb 2 = high digit h
          const float v = static_cast<float>(acc[4 * jj + 2]) * 65536.f +
                          static_cast<float>(acc[4 * jj + 1]) * 256.f + static_cast<float>(acc[4 * jj]);
          const float2 xf = xfp[bq * Gp];
          yacc[bq] += sc * (v * xf.y) + bi * xf.x;
        }
      }
    }
  };
  // sum over the lane groups of the MFMA (lanes c, c + M, ...)
  auto lane_group_sum = [&](float v) {
    if constexpr (M == 16) v += xor_lane(v, 4, lane);
    return v + xor_lane(v, 5, lane);
  };
  // after consuming the item at ccur: park or store the tile when it ends
  auto tile_end = [&](const Cursor& ccur, const Cursor& nxt) {
    if (nxt.j >= total || nxt.t != ccur.t) {
      // this wave is done with the tile: split modes park its partial sums,
      // persistent mode stores the rows it owns
      const int row0 = tile_row(ccur);
#pragma unroll
      for (int bq = 0; bq < NB; ++bq) {
        const float v = lane_group_sum(yacc[bq]);
        if (lg == 0 && bq < B) {
          if constexpr (SPLIT) red[((ccur.t * kFusedWaves + wave) * NB + bq) * M + c] = v;
          else if (row0 + c < N) y[(int64_t)bq * N + row0 + c] = v;
        }
        yacc[bq] = 0.f;
      }
    }
  };

  Cursor ccur = first;
  if constexpr (STAGED) {
#pragma unroll
    for (int j = 0; j < kStagedItems; ++j) {
      if (j < total) {
        const uint32_t oc =
            lane_c + static_cast<uint32_t>(tile_row(ccur)) * static_cast<uint32_t>(W * 4) + ccur.s * (GPS * 32);
        FusedSpan cur;
        cur.w0 = *reinterpret_cast<const uint4*>(stage + stage_at(oc));
        cur.w1 = *reinterpret_cast<const uint4*>(stage + stage_at(oc) + 16);
        cur.s = st_s[j];
        cur.bias = st_b[j];
        consume(cur, ccur.s);
        Cursor nxt = ccur;
        step(nxt);
        tile_end(ccur, nxt);
        ccur = nxt;
      }
    }
  } else {
    for (int base = 0; base < total; base += P) {
#pragma unroll
      for (int sl = 0; sl < P; ++sl) {
        if (base + sl < total) {
          consume(ring[sl], ccur.s);
          Cursor nxt = ccur;
          step(nxt);
          tile_end(ccur, nxt);
          ccur = nxt;
        }
        load_item(rcur, ring[sl]);
        step(rcur);
      }
    }
  }
  if constexpr (REMK) {
    if (rtotal > 0) {
      float yr = 0.f;
      auto consume_rem = [&](const RemUnit& u, int k) {
        const int g = rem_group(k);
        const int h = rbk & 1;
        const bool gin = g < G;
        const uint4* ap = (gin && rri < kLimbs) ? lds_a + (g * kLimbs + rri) * kLdsRow + 4 * h : lds_zero;
        const uint32_t wv[4] = {u.w.x, u.w.y, u.w.z, u.w.w};
        v4i acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint4 a = ap[t];
          const uint32_t w = wv[t];
          acc0 = __builtin_amdgcn_mfma_i32_4x4x4i8(static_cast<int>(a.x), static_cast<int>(w & 0x03030303u), acc0,
                                                   0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_i32_4x4x4i8(static_cast<int>(a.y),
                                                   static_cast<int>((w >> 2) & 0x03030303u), acc1, 0, 0, 0);
          acc0 = __builtin_amdgcn_mfma_i32_4x4x4i8(static_cast<int>(a.z),
                                                   static_cast<int>((w >> 4) & 0x03030303u), acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_i32_4x4x4i8(static_cast<int>(a.w),
                                                   static_cast<int>((w >> 6) & 0x03030303u), acc1, 0, 0, 0);
        }
        const v4i acc = acc0 + acc1;
        const float v = static_cast<float>(acc[2]) * 65536.f + static_cast<float>(acc[1]) * 256.f +
                        static_cast<float>(acc[0]);
        // the bias term once per group (in its first half)
        const float2 xf = gin ? lds_xf[g] : make_float2(0.f, 0.f);
        const float sc = gin ? half_bits_to_float(u.s) : 0.f;
        const float bi = (gin && h == 0) ? half_bits_to_float(u.bias) : 0.f;
        yr += sc * (v * xf.y) + bi * xf.x;
      };
      for (int base = 0; base < rtotal; base += RR) {
#pragma unroll
        for (int sl = 0; sl < RR; ++sl) {
          if (base + sl < rtotal) {
            consume_rem(ru[sl], base + sl);
            if (base + sl + RR < rtotal) load_rem(base + sl + RR, ru[sl]);
          }
        }
      }
      // add up the 16 blocks of each row (lanes r, r + 4, ..., r + 60)
#pragma unroll
      for (int j = 2; j < 6; ++j) yr += xor_lane(yr, j, lane);
      if (lane < 4) red[((tsub - 1) * kFusedWaves + wave) * M + lane] = yr;
    }
  }
  if constexpr (SPLIT) {
    // add up the waves' partial sums of every row of the band
    __syncthreads();
    for (int i = tid; i < tsub * NB * M; i += kFusedThreads) {
      const int t = i / (NB * M), bq = (i / M) % NB, cc = i % M;
      if (bq < B && t * M + cc < nrows) {
        float a = 0.f;
#pragma unroll
        for (int w = 0; w < kFusedWaves; ++w) a += red[((t * kFusedWaves + w) * NB + bq) * M + cc];
        y[(int64_t)bq * N + band0 + t * M + cc] = a;
      }
    }
  }
}

// Launch shape of one call.
struct FusedPlan {
  int mode;
  int rem;  // 4-row remainder blocks (split ring mode, one batch row)
  int tsub, aux, grid;
  int64_t lds;
};

static FusedPlan fused_plan(int64_t B, int64_t K, int64_t N, int cus) {
  const int M = B == 1 ? 16 : 32;
  const int NB = B == 1 ? 1 : (B <= 4 ? 4 : 8);
  const int64_t Gp = padded_groups(K);
  const int64_t rb = K / kCodesPerWord * 4;  // code bytes per row
  FusedPlan p;
  p.rem = 0;
  // split modes: one band of about N / CUs rows (at least 16) per workgroup
  const int64_t rows = std::max<int64_t>((N + cus - 1) / cus, 16);
  const int64_t tsub = (rows + M - 1) / M;
  if (tsub <= kFusedMaxSub) {
    p.tsub = static_cast<int>(tsub);
    p.aux = static_cast<int>(rows);
    p.grid = static_cast<int>((N + rows - 1) / rows);
    const int64_t base = fused_lds_layout(B, Gp, tsub * kFusedWaves * NB * M).total;
    // staged codes: the slots the loads fill, every slot an item of the last
    // subtile can address (an item may run up to 3 padding groups past the
    // last row), and the dump slot
    const int64_t nst = (rows * rb + 1023) / 1024;
    const int64_t slots = (tsub * M * rb + 96 + 1023) / 1024 + 1;
    const int64_t staged = base + slots * kStageSlot;
    const int64_t items = tsub * (Gp / (64 / M));
    if (nst <= (int64_t)kFusedWaves * kStageLoads && items <= (int64_t)kFusedWaves * kStagedItems &&
        staged <= kFusedLdsMax) {
      p.mode = kSplitStaged;
      p.lds = staged;
    } else {
      p.mode = kSplitRing;
      p.lds = base;
      // remainder blocks where measured faster: bands of 2 to 4 subtiles
      // (down_proj, 20 rows: -6%); at 5 (gate_proj, 68 rows) they were 3%
      // slower than the 16-row subtile
      const int64_t rr = rows % M;
      p.rem = (B == 1 && rr >= 1 && rr <= 4 && tsub <= 4) ? 1 : 0;
    }
  } else {
    // persistent mode: tile groups of 8 tiles, at most 2 workgroups per CU
    const int64_t tiles = (N + M - 1) / M;
    const int64_t ntg = (tiles + kFusedWaves - 1) / kFusedWaves;
    p.mode = kPersistent;
    p.tsub = 0;
    p.aux = static_cast<int>(ntg);
    p.lds = fused_lds_layout(B, Gp, 0).total;
    // two per CU when LDS allows and the registers do (8 batch rows need 2x)
    const int per_cu = (p.lds <= 75 * 1024 && NB < 8) ? 2 : 1;
    p.grid = static_cast<int>(std::min<int64_t>(ntg, (int64_t)cus * per_cu));
  }
  return p;
}

bool gemv_fused_eligible(int64_t B, int64_t K, int64_t N, int block) {
  if (!(block == 0 || block == 512 || block == 1024)) return false;
  const int64_t nch = (K + 1023) / 1024;
  if (B * nch > (int64_t)kFusedWaves * kFusedChunksPerWave) return false;
  return fused_plan(B, K, N, device_cus()).lds <= kFusedLdsMax;
}

template <int NB, int L, int DT, int MODE>
static void fused_launch_m(const void* x, const int8_t* signs, const uint32_t* codes, const uint16_t* scales,
                           const uint16_t* biases, float* y, int N, int K, int cfg, int aux, int grid,
                           size_t lds, hipStream_t st) {
  constexpr int M = NB == 1 ? 16 : 32;
  auto kern = gemv_fused_kernel<NB, M, L, DT, MODE>;
  static std::atomic<uint64_t> lds_set{0};
  lds_limit_once(reinterpret_cast<const void*>(kern), static_cast<int>(kFusedLdsMax), lds_set);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kFusedThreads), lds, st, x, signs, codes, scales, biases, N, K, cfg,
                     aux, y);
}

template <int NB, int L, int DT>
static void fused_launch_t(int mode, const void* x, const int8_t* signs, const uint32_t* codes,
                           const uint16_t* scales, const uint16_t* biases, float* y, int N, int K, int cfg,
                           int aux, int grid, size_t lds, hipStream_t st) {
  if (mode == kSplitStaged)
    fused_launch_m<NB, L, DT, kSplitStaged>(x, signs, codes, scales, biases, y, N, K, cfg, aux, grid, lds, st);
  else if (mode == kSplitRing)
    fused_launch_m<NB, L, DT, kSplitRing>(x, signs, codes, scales, biases, y, N, K, cfg, aux, grid, lds, st);
  else
    fused_launch_m<NB, L, DT, kPersistent>(x, signs, codes, scales, biases, y, N, K, cfg, aux, grid, lds, st);
}

template <int NB, int L>
static void fused_launch_dt(int mode, int dt, const void* x, const int8_t* signs, const uint32_t* codes,
                            const uint16_t* scales, const uint16_t* biases, float* y, int N, int K, int cfg,
                            int aux, int grid, size_t lds, hipStream_t st) {
  if (dt == TB_F32)
    fused_launch_t<NB, L, TB_F32>(mode, x, signs, codes, scales, biases, y, N, K, cfg, aux, grid, lds, st);
  else
    fused_launch_t<NB, L, TB_BF16>(mode, x, signs, codes, scales, biases, y, N, K, cfg, aux, grid, lds, st);
}

template <int NB>
static void fused_launch_l(int mode, int block, int dt, const void* x, const int8_t* signs,
                           const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, float* y,
                           int N, int K, int cfg, int aux, int grid, size_t lds, hipStream_t st) {
  switch (block) {
    case 0:
      fused_launch_dt<NB, 0>(mode, dt, x, signs, codes, scales, biases, y, N, K, cfg, aux, grid, lds, st);
      break;
    case 512:
      fused_launch_dt<NB, 512>(mode, dt, x, signs, codes, scales, biases, y, N, K, cfg, aux, grid, lds, st);
      break;
    default:
      fused_launch_dt<NB, 1024>(mode, dt, x, signs, codes, scales, biases, y, N, K, cfg, aux, grid, lds, st);
      break;
  }
}

void gemv_fused_launch(const void* x, int x_dtype, int64_t B, int64_t K, const int8_t* signs, int block,
                       const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t N,
                       float* y, hipStream_t st) {
  const FusedPlan p = fused_plan(B, K, N, device_cus());
  const int cfg = static_cast<int>(B) | (p.rem << 4) | (p.tsub << 5) | (p.grid << 8);
  const int n = static_cast<int>(N), k = static_cast<int>(K);
  const size_t lds = static_cast<size_t>(p.lds);
  if (B == 1)
    fused_launch_l<1>(p.mode, block, x_dtype, x, signs, codes, scales, biases, y, n, k, cfg, p.aux, p.grid, lds, st);
  else if (B <= 4)
    fused_launch_l<4>(p.mode, block, x_dtype, x, signs, codes, scales, biases, y, n, k, cfg, p.aux, p.grid, lds, st);
  else
    fused_launch_l<8>(p.mode, block, x_dtype, x, signs, codes, scales, biases, y, n, k, cfg, p.aux, p.grid, lds, st);
}

}  // namespace tb
