// Single-launch Packed linear for one activation row (decode batch 1): the
// signed block transform, its exact integer split and the weight-streaming
// 2-bit matmul in one kernel, one workgroup per band of output rows
// [lpnh.cn/news/2438023, "text model loading"; kwkr.cn/news/564617,
// "ternary weights + folded Hadamard rotation" and "packing-format
// engineering"].
//
// A decode call is short: q_proj streams 8.8 MB, about a microsecond of
// HBM time, so its cost is a chain of latencies.  The kernel keeps that
// chain short:
//
// * Roles.  Each 1024-input chunk of x is transformed by one wave ("transform
//   waves"); the other waves ("loader waves") copy the workgroup's whole band
//   of packed weights -- codes, fp16 scales and fp16 biases, each a
//   contiguous run of memory -- into LDS with direct-to-LDS buffer loads of
//   1 KB per wave instruction.  Contiguous 1 KB loads are the cheapest way to
//   move the band, and a wave stalled on a full memory pipeline is never one
//   that has transform work to do.
//
// * The transform on the matrix cores.  H_1024 factors over any split of the
//   ten index bits into two sets of five: H_1024 = H_32 (x) H_32.  With the
//   chunk viewed as a 32 x 32 matrix X whose row index holds element bits
//   {2,3,7,8,9} and whose column index holds bits {0,1,4,5,6}, the
//   transform is U = H_32 X H_32: two bf16 MFMA products
//   (v_mfma_f32_32x32x16_bf16) against constant +-1 operands.  X enters
//   exactly (bf16 activations are bf16; fp32 ones as an exact sum of three
//   bf16 pieces), and so does the intermediate P = X H, re-entered as three
//   bf16 pieces; only the fp32 accumulation inside the MFMAs rounds.  The bit split is chosen so that the
//   accumulator layout of the second product is already the byte order of
//   the matmul operand: every lane ends up holding, for 4 groups of 128
//   inputs, the 4 values that form one dword of that group's operand row.
//   The natural-order Sylvester matrix H[i][j] = (-1)^popcount(i & j)
//   [trdm.cn/news/822023 section 2.2] is the Kronecker product over bits, so
//   the constant operands are +-1 patterns of lane and slot.
//
// * Exact integer activations.  The transformed chunk is scaled by one power
//   of two so that its largest magnitude is just below 2^30 and converted to
//   integers q (error below 2^-29 of the chunk's largest |u|, far below the
//   fp32 rounding of the transform itself).  q splits into four balanced
//   base-256 digits ("limbs"), which fill the four A-operand rows a group
//   owns in v_mfma_i32_16x16x64_i8 against the 2-bit codes.  Integer
//   MFMA sums are exact; the fp16 scale and bias are applied per (row,
//   group) in fp32.  The bias term needs sum_{k in g} u_k, which for a
//   normalized Sylvester transform is 128 / sqrt(L) times an 8-point
//   transform of the inputs at positions 128 c (all other inputs cancel), so
//   the group sums cost three lane-exchange stages.
//
// * One barrier.  Once the transform waves have written the operand image
//   and every wave's staging loads have landed, all 8 waves run the matmul
//   from LDS: items of (16-row subtile, span of 4 groups), dealt round robin,
//   with all of a wave's LDS reads issued before its MFMAs.  Partial sums
//   meet in LDS and every row of y is written once.
//
// Used for batch 1, blocks 0 / 512 / 1024, at most 3 chunk transforms per
// wave, bands of at most 7 subtiles and an LDS footprint within the limit;
// tb_ternary_gemv takes other paths otherwise.
#include <algorithm>

#include "tb_gemv.h"

namespace tb {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBandWaves = 8;
constexpr int kBandThreads = 64 * kBandWaves;
constexpr int kBandMaxTasks = 3;      // chunk transforms per wave
constexpr int kBandMaxItems = 4;      // matmul items per wave
constexpr int kBandMaxSub = 7;        // 16-row subtiles per band
constexpr int kBandLimbs = 4;         // base-256 digits of the fixed-point activation
constexpr int kBandArow = 144;        // LDS bytes per (group, limb) operand row: 128 + 16 pad
constexpr int kBandSlot = 1024 + 16;  // LDS bytes per staged 1 KB of codes (16 B pad per KB)
constexpr int kBandMaxLoads = 24;     // staging loads per loader wave
constexpr int64_t kBandLdsMax = 150 * 1024;
constexpr int kBandWaitVm0 = (0x7 << 4) | (0xF << 8);  // s_waitcnt vmcnt(0)

// --------------------------------------------------------------------------
// constant MFMA operands of the transform
// --------------------------------------------------------------------------
// Element e (0..1023) of a chunk has row index a (bits 2,3,7,8,9 of e) and
// column index b (bits 0,1,4,5,6).  First product P = X H_b: X is the A
// operand (lane l: row a = l & 31), H_b the B operand (lane l: column
// j = l & 31); the K slot (step s, lane half h, element t of 8) carries
// b = t + 8 s + 16 h.  Second product U = H_a P: H_a is the A operand (lane
// l: row i = l & 31), P the B operand taken from the first product's
// accumulators, whose register r = 8 s + t of lane half h holds row
// a = 16 s + 8 (t >> 2) + 4 h + (t & 3) -- so that is the a of K slot
// (s, h, t).  Mode 0: no rotation (identity matrices); mode 1: 512-blocks
// (element bit 9 = a bit 4 is not transformed); mode 2: 1024-blocks.
constexpr int xf_parity(unsigned v) {
  v ^= v >> 16;
  v ^= v >> 8;
  v ^= v >> 4;
  v ^= v >> 2;
  v ^= v >> 1;
  return static_cast<int>(v & 1u);
}
constexpr uint32_t kBfPlus = 0x3F80u, kBfMinus = 0xBF80u;  // bf16 +1, -1
constexpr uint32_t xf_first(int mode, int lane, int s, int t) {
  const int j = lane & 31, b = t + 8 * s + 16 * (lane >> 5);
  if (mode == 0) return b == j ? kBfPlus : 0u;
  return xf_parity(static_cast<unsigned>(b & j)) ? kBfMinus : kBfPlus;
}
constexpr uint32_t xf_second(int mode, int lane, int s, int t) {
  const int i = lane & 31, a = 16 * s + 8 * (t >> 2) + 4 * (lane >> 5) + (t & 3);
  if (mode == 0) return a == i ? kBfPlus : 0u;
  if (mode == 1 && (i >> 4) != (a >> 4)) return 0u;
  const int m = mode == 1 ? 15 : 31;
  return xf_parity(static_cast<unsigned>(i & a & m)) ? kBfMinus : kBfPlus;
}
struct XformConst {
  uint32_t w[3][2][64][8];  // [mode][first B / second A][lane][step * 4 + pair]
};
constexpr XformConst make_xform_const() {
  XformConst c{};
  for (int mode = 0; mode < 3; ++mode)
    for (int lane = 0; lane < 64; ++lane)
      for (int d = 0; d < 8; ++d) {
        const int s = d >> 2, t = 2 * (d & 3);
        c.w[mode][0][lane][d] = xf_first(mode, lane, s, t) | (xf_first(mode, lane, s, t + 1) << 16);
        c.w[mode][1][lane][d] = xf_second(mode, lane, s, t) | (xf_second(mode, lane, s, t + 1) << 16);
      }
  return c;
}
__device__ const XformConst kXformConst = make_xform_const();

template <int L>
constexpr int xf_mode() {
  return L == 0 ? 0 : (L == 512 ? 1 : 2);
}

template <int L>
__device__ __forceinline__ float inv_sqrt_block_or_one() {
  if constexpr (L == 0) return 1.f;
  else return inv_sqrt_block<L>();
}

__device__ __forceinline__ v8bf as_v8bf(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(v8bf, v4u{a, b, c, d});
}

// Exact split of two floats into three bf16 pieces each, packed as pairs
// (first float in the low half): hi = the top 8 significant bits, mid = the
// next 8 bits of the remainder, lo = what is left, which has at most 8
// significant bits and is therefore a bf16 value too.  a = hi + mid + lo
// exactly (finite, normal inputs).
__device__ __forceinline__ void split3_bf16x2(float a, float b, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  hi = __builtin_amdgcn_perm(ub, ua, 0x07060302u);
  const float ra = a - __uint_as_float(ua & 0xFFFF0000u), rb = b - __uint_as_float(ub & 0xFFFF0000u);
  const uint32_t va = __float_as_uint(ra), vb = __float_as_uint(rb);
  mid = __builtin_amdgcn_perm(vb, va, 0x07060302u);
  const float qa = ra - __uint_as_float(va & 0xFFFF0000u), qb = rb - __uint_as_float(vb & 0xFFFF0000u);
  lo = __builtin_amdgcn_perm(__float_as_uint(qb), __float_as_uint(qa), 0x07060302u);
}

// Raw activation and sign data of one chunk task, loaded before the lane
// needs it.  Lane l holds the 16 elements of row a = l & 31 whose column
// index b has bit 4 (element bit 6) = l >> 5: four runs of 4 consecutive
// elements at element offsets base + 32 s + 16 u (s, u in {0, 1}).
template <int DT>
struct XformIn {
  uint32_t x[4][DT == TB_F32 ? 4 : 2];  // run (2 s + u): 4 elements
  uint32_t sg[4];                        // run (2 s + u): 4 int8 signs
};

__device__ __forceinline__ int xf_lane_base(int lane) {
  const int a = lane & 31;
  return ((a & 3) << 2) | ((lane >> 5) << 6) | ((a >> 2) << 7);
}

template <int L, int DT>
__device__ __forceinline__ void xform_issue(__amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rsg, int64_t e0,
                                            int k0, int lane, XformIn<DT>& in) {
  // e0: element offset of the chunk in x (batch row included); k0: in signs
  constexpr int ESZ = DT == TB_F32 ? 4 : 2;
  const int base = xf_lane_base(lane);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int off = base + 32 * (q >> 1) + 16 * (q & 1);
    const int xo = static_cast<int>((e0 + off) * ESZ);
    if constexpr (DT == TB_F32) {
      const v4u u = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0);
      in.x[q][0] = u.x; in.x[q][1] = u.y; in.x[q][2] = u.z; in.x[q][3] = u.w;
    } else {
      const v2u u = __builtin_amdgcn_raw_buffer_load_b64(rx, xo, 0, 0);
      in.x[q][0] = u.x; in.x[q][1] = u.y;
    }
    if constexpr (L > 0) in.sg[q] = __builtin_amdgcn_raw_buffer_load_b32(rsg, k0 + off, 0, 0);
  }
}

// Transform one chunk (rows 8 c0 .. 8 c0 + 7 of the operand image) and write
// its limbs and (group sum, f) into LDS.  lds_a: operand rows [group][limb]
// of kBandArow bytes; lds_xf: float2 per group.
template <int L, int DT>
__device__ __forceinline__ void xform_chunk(const XformIn<DT>& in, int g0, int lane, const v4u cfirst[2],
                                            const v4u csecond[2], char* lds_a, float2* lds_xf) {
  // 1. signs onto the activations, as bf16 operand pairs
  uint32_t xop[2][4];        // exact bf16 (bf16 input) or the hi piece of an fp32 input
  uint32_t xmid[2][4] = {};  // fp32 input: the mid and lo pieces
  uint32_t xlo[2][4] = {};
  float v128 = 0.f;         // element 128 c of lanes 4 c (c < 8): for the group sums
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int s = q >> 1, u = q & 1;
    if constexpr (DT == TB_F32) {
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t w = in.x[q][e];
        if constexpr (L > 0) w ^= (in.sg[q] << (24 - 8 * e)) & 0x80000000u;
        f[e] = __uint_as_float(w);
      }
      if (q == 0) v128 = f[0];
#pragma unroll
      for (int p = 0; p < 2; ++p)
        split3_bf16x2(f[2 * p], f[2 * p + 1], xop[s][2 * u + p], xmid[s][2 * u + p], xlo[s][2 * u + p]);
    } else {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        uint32_t w = in.x[q][p];
        if constexpr (L > 0) {
          // sign bytes 2p, 2p+1 (bit 7 set for -1) onto bf16 sign bits 15 and 31
          const uint32_t m = __builtin_amdgcn_perm(0u, in.sg[q], 0x000C000Cu | ((2u * p) << 8) | ((2u * p + 1) << 24));
          w ^= m & 0x80008000u;
        }
        xop[s][2 * u + p] = w;
      }
      if (q == 0) v128 = __uint_as_float(xop[0][0] << 16);
    }
  }
  // 2. P = X H_b
  v16f P = {};
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const v8bf hb = __builtin_bit_cast(v8bf, cfirst[s]);
    P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_v8bf(xop[s][0], xop[s][1], xop[s][2], xop[s][3]), hb, P, 0, 0, 0);
    if constexpr (DT == TB_F32) {
      P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_v8bf(xmid[s][0], xmid[s][1], xmid[s][2], xmid[s][3]), hb, P, 0, 0, 0);
      P = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_v8bf(xlo[s][0], xlo[s][1], xlo[s][2], xlo[s][3]), hb, P, 0, 0, 0);
    }
  }
  // 3. U = H_a P, with P entered as three exact bf16 pieces
  v16f U = {};
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    uint32_t hi[4], mid[4], lo[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) split3_bf16x2(P[8 * s + 2 * p], P[8 * s + 2 * p + 1], hi[p], mid[p], lo[p]);
    const v8bf ha = __builtin_bit_cast(v8bf, csecond[s]);
    U = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ha, as_v8bf(hi[0], hi[1], hi[2], hi[3]), U, 0, 0, 0);
    U = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ha, as_v8bf(mid[0], mid[1], mid[2], mid[3]), U, 0, 0, 0);
    U = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ha, as_v8bf(lo[0], lo[1], lo[2], lo[3]), U, 0, 0, 0);
  }
  // 4. one power-of-two scale for the chunk: |q| < 2^30
  float m = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(U[r]));
#pragma unroll
  for (int j = 0; j < 6; ++j) m = fmaxf(m, xor_lane(m, j, lane));
  const uint32_t mb = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(__float_as_uint(m))));
  int e = static_cast<int>((mb >> 23) & 0xFF) - 127;  // floor(log2 m) for normal m
  e = mb == 0 ? 0 : (e < -90 ? -90 : e);
  const float sigma = __uint_as_float(static_cast<uint32_t>(29 - e + 127) << 23);  // 2^(29 - e)
  const float f = __uint_as_float(static_cast<uint32_t>(e - 29 + 127) << 23) * inv_sqrt_block_or_one<L>();
  // 5. q + 0x808080, then the balanced digits: limbs 0-2 = bytes 0-2 ^ 0x80,
  //    limb 3 = byte 3 (signed): q = sum_l limb_l 256^l
  uint32_t qd[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) qd[r] = static_cast<uint32_t>(static_cast<int>(U[r] * sigma)) + 0x808080u;
  const int h = lane >> 5;
  char* const arow = lds_a + static_cast<int64_t>(g0 + h) * (kBandLimbs * kBandArow) + (lane & 31) * 4;
#pragma unroll
  for (int Q = 0; Q < 4; ++Q) {
    const uint32_t a0 = qd[4 * Q], a1 = qd[4 * Q + 1], a2 = qd[4 * Q + 2], a3 = qd[4 * Q + 3];
    const uint32_t l0 = (__builtin_amdgcn_perm(a1, a0, 0x0C0C0400u) | __builtin_amdgcn_perm(a3, a2, 0x04000C0Cu)) ^ 0x80808080u;
    const uint32_t l1 = (__builtin_amdgcn_perm(a1, a0, 0x0C0C0501u) | __builtin_amdgcn_perm(a3, a2, 0x05010C0Cu)) ^ 0x80808080u;
    const uint32_t l2 = (__builtin_amdgcn_perm(a1, a0, 0x0C0C0602u) | __builtin_amdgcn_perm(a3, a2, 0x06020C0Cu)) ^ 0x80808080u;
    const uint32_t l3 = __builtin_amdgcn_perm(a1, a0, 0x0C0C0703u) | __builtin_amdgcn_perm(a3, a2, 0x07030C0Cu);
    char* row = arow + static_cast<int64_t>(2 * Q) * (kBandLimbs * kBandArow);  // group g0 + h + 2 Q
    *reinterpret_cast<uint32_t*>(row) = l0;
    *reinterpret_cast<uint32_t*>(row + kBandArow) = l1;
    *reinterpret_cast<uint32_t*>(row + 2 * kBandArow) = l2;
    *reinterpret_cast<uint32_t*>(row + 3 * kBandArow) = l3;
  }
  // 6. group sums of the normalized transform
  if constexpr (L > 0) {
    // sum_{k in group m} (H v)_k = 128 sum_c (-1)^popcount(m & c) v[128 c]; v[128 c]
    // is element 0 of lane 4 c.  Butterflies over lane bits 2, 3 (and 4 for 1024-blocks).
    float g = v128;
#pragma unroll
    for (int j = 2; j < (L == 512 ? 4 : 5); ++j) {
      const float sgn = ((lane >> j) & 1) ? -1.f : 1.f;
      g = fmaf(sgn, g, xor_lane(g, j, lane));
    }
    if (lane < 32 && (lane & 3) == 0)
      lds_xf[g0 + (lane >> 2)] = make_float2(g * (128.f * inv_sqrt_block_or_one<L>()), f);
  } else {
    // no rotation: sum the 4 values of each group held by the lane, then over
    // the 32 lanes of the lane half
#pragma unroll
    for (int Q = 0; Q < 4; ++Q) {
      float sm = (U[4 * Q] + U[4 * Q + 1]) + (U[4 * Q + 2] + U[4 * Q + 3]);
#pragma unroll
      for (int j = 0; j < 5; ++j) sm += xor_lane(sm, j, lane);
      if ((lane & 31) == 0) lds_xf[g0 + h + 2 * Q] = make_float2(sm, f);
    }
  }
}

// --------------------------------------------------------------------------
// the kernel
// --------------------------------------------------------------------------
struct BandLds {
  int64_t a, xf, red, codes, sc, bi, total;
};
// sb_slots: 1 KB slots reserved for each of the scale and bias arrays, enough
// for every (row, group) index an item of the band can form
__host__ __device__ inline BandLds band_lds_layout(int64_t nch, int64_t tsub, int64_t code_slots, int64_t sb_slots) {
  BandLds l;
  l.a = 0;
  l.xf = l.a + nch * 8 * kBandLimbs * kBandArow;
  l.red = l.xf + nch * 8 * 8;
  l.codes = l.red + tsub * kBandWaves * 16 * 4;
  l.sc = l.codes + code_slots * kBandSlot;
  l.bi = l.sc + sb_slots * 1024;
  l.total = l.bi + sb_slots * 1024;
  return l;
}

// rows: output rows per band (the last band may be short); tsub: 16-row
// subtiles per band.
template <int L, int DT>
__global__ __launch_bounds__(kBandThreads, 1) void gemv_band_kernel(
    const void* __restrict__ x, const int8_t* __restrict__ signs, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases, int N, int K, int rows,
    int tsub, float* __restrict__ y) {
  constexpr int M = 16, GPS = 4;
  extern __shared__ uint4 lds_dyn[];
  char* const lds = reinterpret_cast<char*>(lds_dyn);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bid = static_cast<int>(blockIdx.x);
  const int G = K / kGroup;
  const int W = K / kCodesPerWord;
  const int RB = W * 4;                     // code bytes per row
  const int Gp = (G + GPS - 1) / GPS * GPS;
  const int S = Gp / GPS;                   // spans per row
  const int nch = (K + 1023) >> 10;         // chunk transforms
  const int band0 = bid * rows;
  const int nrows = min(rows, N - band0);
  const int code_bytes = nrows * RB;
  const int ncs = (code_bytes + 1023) >> 10;           // staged code slots with data
  const int sb_bytes = nrows * G * 2;
  const int nss = (sb_bytes + 1023) >> 10;             // slots per scale / bias array
  const int cslots = (tsub * M * RB + 96 + 1023) / 1024 + 1;
  const int sbslots = (tsub * M * G * 2 + 64 + 1023) / 1024;
  const BandLds lay = band_lds_layout(nch, tsub, cslots, sbslots);
  char* const lds_a = lds + lay.a;
  float2* const lds_xf = reinterpret_cast<float2*>(lds + lay.xf);
  float* const red = reinterpret_cast<float*>(lds + lay.red);
  char* const st_codes = lds + lay.codes;
  const uint16_t* const st_sc = reinterpret_cast<const uint16_t*>(lds + lay.sc);
  const uint16_t* const st_bi = reinterpret_cast<const uint16_t*>(lds + lay.bi);

  // ---- 1. issue: transform waves load their chunks, loader waves the band
  const int ntask_waves = nch < kBandWaves ? nch : kBandWaves;
  const bool xwave = wave < ntask_waves;
  XformIn<DT> xin[kBandMaxTasks];
  const auto rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(x), 0, K * (DT == TB_F32 ? 4 : 2), kRsrcWord3);
  const auto rsg = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(signs), 0, L > 0 ? K : 0, kRsrcWord3);
  if (xwave) {
#pragma unroll
    for (int r = 0; r < kBandMaxTasks; ++r) {
      const int c = wave + kBandWaves * r;
      if (c < nch) xform_issue<L, DT>(rx, rsg, static_cast<int64_t>(c) * 1024, c * 1024, lane, xin[r]);
    }
  }
  // The buffer range check works on whole dwords: when the band's fp16 scale
  // (and bias) array ends in the middle of a dword, the staging load returns
  // zero for its last element, which the owner of that slot then loads on its
  // own and writes into LDS after the staging has landed.
  uint16_t tail_s = 0, tail_b = 0;
  bool own_tail_s = false, own_tail_b = false;
  {
    // loader waves: all waves past the transform waves, or all 8 when every
    // wave transforms
    const int first = ntask_waves < kBandWaves ? ntask_waves : 0;
    const int nload = kBandWaves - first;
    if (wave >= first) {
      const auto rc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(codes + static_cast<int64_t>(band0) * W),
                                                        0, code_bytes, kRsrcWord3);
      const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales + static_cast<int64_t>(band0) * G),
                                                        0, sb_bytes, kRsrcWord3);
      const auto rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(biases + static_cast<int64_t>(band0) * G),
                                                        0, sb_bytes, kRsrcWord3);
      const int total = ncs + 2 * nss;
      for (int q = wave - first; q < total; q += nload) {
        if (q < ncs) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (__attribute__((address_space(3))) void*)(st_codes + q * kBandSlot),
                                                   16, q * 1024 + lane * 16, 0, 0, 0);
        } else if (q < ncs + nss) {
          const int p = q - ncs;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds + lay.sc + p * 1024),
                                                   16, p * 1024 + lane * 16, 0, 0, 0);
        } else {
          const int p = q - ncs - nss;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (__attribute__((address_space(3))) void*)(lds + lay.bi + p * 1024),
                                                   16, p * 1024 + lane * 16, 0, 0, 0);
        }
      }
      if (sb_bytes & 2) {
        own_tail_s = (ncs + nss - 1) % nload == wave - first;
        own_tail_b = (ncs + 2 * nss - 1) % nload == wave - first;
        if (own_tail_s) tail_s = __builtin_amdgcn_raw_buffer_load_b16(rs, sb_bytes - 2, 0, 0);
        if (own_tail_b) tail_b = __builtin_amdgcn_raw_buffer_load_b16(rb, sb_bytes - 2, 0, 0);
      }
    }
  }

  // ---- 2. transform waves: the operand image of their chunks
  for (int i = tid; i < tsub * kBandWaves * 16; i += kBandThreads) red[i] = 0.f;
  if (xwave) {
    const v4u* cst = reinterpret_cast<const v4u*>(&kXformConst.w[xf_mode<L>()][0][lane][0]);
    const v4u* cst2 = reinterpret_cast<const v4u*>(&kXformConst.w[xf_mode<L>()][1][lane][0]);
    const v4u cf[2] = {cst[0], cst[1]};
    const v4u cs[2] = {cst2[0], cst2[1]};
#pragma unroll
    for (int r = 0; r < kBandMaxTasks; ++r) {
      const int c = wave + kBandWaves * r;
      if (c < nch) xform_chunk<L, DT>(xin[r], 8 * c, lane, cf, cs, lds_a, lds_xf);
    }
  }
  __builtin_amdgcn_s_waitcnt(kBandWaitVm0);  // this wave's staging loads have landed
  if (lane == 0) {
    if (own_tail_s) reinterpret_cast<uint16_t*>(lds + lay.sc)[sb_bytes / 2 - 1] = tail_s;
    if (own_tail_b) reinterpret_cast<uint16_t*>(lds + lay.bi)[sb_bytes / 2 - 1] = tail_b;
  }
  __syncthreads();

  // ---- 3. the matmul: items (subtile t, span s), item i = t * S + s,
  //         wave w takes items w, w + 8, ...
  const int lg = lane >> 4, c = lane & 15;
  const int ar = c & 3, alg = (c >> 2) & 3;
  const bool a_lane = alg == lg;
  const int items = tsub * S;
  const uint32_t lane_c = static_cast<uint32_t>(c * RB + lg * 32);
  auto stage_at = [](uint32_t off) { return off + (off >> 10) * (kBandSlot - 1024); };

  // all LDS reads of the wave's items first: codes, scale, bias, the
  // group's (sum, f), and the A operand -- read only by the 16 lanes whose A
  // row is non-zero (the others keep zeros)
  uint4 cw[kBandMaxItems][2];
  uint4 av[kBandMaxItems][kWordsPerGroup];
  float2 xfv[kBandMaxItems];
  uint16_t sraw[kBandMaxItems], braw[kBandMaxItems];
  int tt[kBandMaxItems], ss[kBandMaxItems];
  {
    int t = wave / S, s = wave - (wave / S) * S;  // item wave = t * S + s
#pragma unroll
    for (int j = 0; j < kBandMaxItems; ++j) {
      tt[j] = t;
      ss[j] = s;
      if (wave + kBandWaves * j < items) {
        const uint32_t so = stage_at(lane_c + static_cast<uint32_t>(t * M * RB + s * 128));
        cw[j][0] = *reinterpret_cast<const uint4*>(st_codes + so);
        cw[j][1] = *reinterpret_cast<const uint4*>(st_codes + so + 16);
        const int si = (t * M + c) * G + s * GPS + lg;
        sraw[j] = st_sc[si];
        braw[j] = st_bi[si];
        xfv[j] = lds_xf[s * GPS + lg];
#pragma unroll
        for (int w = 0; w < kWordsPerGroup; ++w) av[j][w] = make_uint4(0, 0, 0, 0);
        if (a_lane) {
          const uint4* ap = reinterpret_cast<const uint4*>(lds_a + ((s * GPS + alg) * kBandLimbs + ar) * kBandArow);
#pragma unroll
          for (int w = 0; w < kWordsPerGroup; ++w) av[j][w] = ap[w];
        }
      }
      // next item of this wave: 8 items further
      s += kBandWaves;
      while (s >= S) {
        s -= S;
        ++t;
      }
    }
  }
  float part[kBandMaxItems];
#pragma unroll
  for (int j = 0; j < kBandMaxItems; ++j) {
    part[j] = 0.f;
    if (wave + kBandWaves * j < items) {
      v4i bop[kWordsPerGroup];
      bop[0] = decode_word(cw[j][0].x);
      bop[1] = decode_word(cw[j][0].y);
      bop[2] = decode_word(cw[j][0].z);
      bop[3] = decode_word(cw[j][0].w);
      bop[4] = decode_word(cw[j][1].x);
      bop[5] = decode_word(cw[j][1].y);
      bop[6] = decode_word(cw[j][1].z);
      bop[7] = decode_word(cw[j][1].w);
      v4i acc0 = {}, acc1 = {};
#pragma unroll
      for (int w = 0; w < kWordsPerGroup; w += 2) {
        const uint4 u0 = av[j][w], u1 = av[j][w + 1];
        acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(v4i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w}, bop[w], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(v4i{(int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w}, bop[w + 1], acc1, 0, 0, 0);
      }
      const v4i acc = acc0 + acc1;
      // lane (lg, c): limb sums of row t*16 + c, group s*4 + lg
      const bool gin = ss[j] * GPS + lg < G;
      const float sc = gin ? half_bits_to_float(sraw[j]) : 0.f;
      const float bi = gin ? half_bits_to_float(braw[j]) : 0.f;
      const float v = static_cast<float>(acc[3]) * 16777216.f + static_cast<float>(acc[2]) * 65536.f +
                      static_cast<float>(acc[1]) * 256.f + static_cast<float>(acc[0]);
      part[j] = sc * (v * xfv[j].y) + bi * xfv[j].x;
    }
  }
  // per subtile: add this wave's items in registers, then over the 4 lane
  // groups, and park the 16 row sums in red[t][wave] (one plain store)
  for (int t = tt[0]; t < tsub && t <= tt[kBandMaxItems - 1]; ++t) {
    float v = 0.f;
    bool any = false;
#pragma unroll
    for (int j = 0; j < kBandMaxItems; ++j) {
      const bool mine = tt[j] == t && wave + kBandWaves * j < items;
      v += mine ? part[j] : 0.f;
      any |= mine;
    }
    if (any) {
      v += xor_lane(v, 4, lane);
      v += xor_lane(v, 5, lane);
      if (lg == 0) red[(t * kBandWaves + wave) * 16 + c] = v;
    }
  }
  __syncthreads();
  for (int i = tid; i < tsub * M; i += kBandThreads) {
    const int t = i >> 4, cc = i & 15;
    if (t * M + cc < nrows) {
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < kBandWaves; ++w) a += red[(t * kBandWaves + w) * 16 + cc];
      y[band0 + t * M + cc] = a;
    }
  }
}

// --------------------------------------------------------------------------
// host side
// --------------------------------------------------------------------------
static int band_device_cus() {
  int dev = 0, cus = 256;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  return cus;
}

struct BandPlan {
  int rows, tsub, grid;
  int64_t lds;
  bool ok;
};

static BandPlan band_plan(int64_t K, int64_t N, int cus) {
  BandPlan p{};
  const int64_t G = K / kGroup, W = K / kCodesPerWord, RB = W * 4;
  const int64_t Gp = (G + 3) / 4 * 4, S = Gp / 4;
  const int64_t nch = (K + 1023) / 1024;
  const int64_t rows = std::max<int64_t>((N + cus - 1) / cus, 16);
  const int64_t tsub = (rows + 15) / 16;
  p.rows = static_cast<int>(rows);
  p.tsub = static_cast<int>(tsub);
  p.grid = static_cast<int>((N + rows - 1) / rows);
  const int64_t cslots = (tsub * 16 * RB + 96 + 1023) / 1024 + 1;
  const int64_t sbslots = (tsub * 16 * G * 2 + 64 + 1023) / 1024;
  const int64_t nss = (rows * G * 2 + 1023) / 1024;
  const int64_t ncs = (rows * RB + 1023) / 1024;
  const int ntw = static_cast<int>(std::min<int64_t>(nch, kBandWaves));
  const int nload = ntw < kBandWaves ? kBandWaves - ntw : kBandWaves;
  p.lds = band_lds_layout(nch, tsub, cslots, sbslots).total;
  p.ok = tsub <= kBandMaxSub && tsub * S <= (int64_t)kBandWaves * kBandMaxItems &&
         nch <= (int64_t)kBandWaves * kBandMaxTasks && p.lds <= kBandLdsMax &&
         (ncs + 2 * nss + nload - 1) / nload <= kBandMaxLoads;
  return p;
}

bool gemv_band_eligible(int64_t B, int64_t K, int64_t N, int block) {
  if (B != 1 || !(block == 0 || block == 512 || block == 1024)) return false;
  return band_plan(K, N, band_device_cus()).ok;
}

template <int L, int DT>
static void band_launch_t(const void* x, const int8_t* signs, const uint32_t* codes, const uint16_t* scales,
                          const uint16_t* biases, float* y, int N, int K, const BandPlan& p, hipStream_t st) {
  auto kern = gemv_band_kernel<L, DT>;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(kBandLdsMax));
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(p.grid), dim3(kBandThreads), static_cast<size_t>(p.lds), st, x, signs, codes, scales,
                     biases, N, K, p.rows, p.tsub, y);
}

template <int L>
static void band_launch_l(int dt, const void* x, const int8_t* signs, const uint32_t* codes, const uint16_t* scales,
                          const uint16_t* biases, float* y, int N, int K, const BandPlan& p, hipStream_t st) {
  if (dt == TB_F32) band_launch_t<L, TB_F32>(x, signs, codes, scales, biases, y, N, K, p, st);
  else band_launch_t<L, TB_BF16>(x, signs, codes, scales, biases, y, N, K, p, st);
}

void gemv_band_launch(const void* x, int x_dtype, int64_t K, const int8_t* signs, int block, const uint32_t* codes,
                      const uint16_t* scales, const uint16_t* biases, int64_t N, float* y, hipStream_t st) {
  const BandPlan p = band_plan(K, N, band_device_cus());
  const int n = static_cast<int>(N), k = static_cast<int>(K);
  if (block == 0) band_launch_l<0>(x_dtype, x, signs, codes, scales, biases, y, n, k, p, st);
  else if (block == 512) band_launch_l<512>(x_dtype, x, signs, codes, scales, biases, y, n, k, p, st);
  else band_launch_l<1024>(x_dtype, x, signs, codes, scales, biases, y, n, k, p, st);
}

}  // namespace tb
