// The signed 1024-input block transform on the matrix cores, and its exact
// split into the int8 operand rows of the decode matmul.  Shared by the
// batch-1 band kernel (operand image in LDS) and the multi-module prepare
// kernel (operand image in the workspace).
//
// H_1024 factors over any split of the ten index bits into two sets of five:
// H_1024 = H_32 (x) H_32 [natural-order Sylvester matrix, trdm.cn/news/822023
// section 2.2: H[i][j] = (-1)^popcount(i & j), the Kronecker product over
// bits].  With a chunk viewed as a 32 x 32 matrix X whose row index holds
// element bits {2,3,7,8,9} and whose column index holds bits {0,1,4,5,6},
// the transform is U = H_32 X H_32: two bf16 MFMA products
// (v_mfma_f32_32x32x16_bf16) against constant +-1 operands.  X enters exactly
// (bf16 activations are bf16; fp32 ones as an exact sum of three bf16
// pieces), and so does the intermediate P = X H, re-entered as three bf16
// pieces; only the fp32 accumulation inside the MFMAs rounds.  The bit split
// is chosen so that the accumulator layout of the second product is already
// the byte order of the matmul operand: each lane ends up holding, for 4
// groups of 128 inputs, the 4 values that form one dword of that group's
// operand row.  The chunk is then scaled by one power of two so that its
// largest magnitude is just below 2^30, converted to integers q (error below
// 2^-29 of the chunk's largest |u|), and q is split into four balanced
// base-256 digits ("limbs").  The bias term of the matmul needs the group
// sums of u, which for a normalized Sylvester transform are 128 / sqrt(L)
// times an 8-point transform of the inputs at positions 128 c (all other
// inputs cancel) [kwkr.cn/news/564617, "ternary weights + folded Hadamard
// rotation": normalized transform, scale 1/sqrt(block)].
#pragma once

#include "tb_gemv.h"

namespace tb {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kXfLimbs = 4;  // base-256 digits of the fixed-point activation

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
__device__ inline const XformConst kXformConst = make_xform_const();

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

// The rotated chunk U = H (signs .* x) (unnormalized) in the accumulator
// layout of the second product: lane l, register 4 Q + t holds element
//   e = (l & 3) | t << 2 | ((l >> 2) & 7) << 4 | (l >> 5) << 7 | Q << 8,
// so group (128 inputs) h + 2 Q of the chunk with h = l >> 5.  v128: element
// 128 c in lanes 4 c (c < 8), for the group sums.
template <int L, int DT>
__device__ __forceinline__ v16f xform_rotate(const XformIn<DT>& in, int lane, const v4u cfirst[2],
                                             const v4u csecond[2], float& v128) {
  // 1. signs onto the activations, as bf16 operand pairs
  uint32_t xop[2][4];        // exact bf16 (bf16 input) or the hi piece of an fp32 input
  uint32_t xmid[2][4] = {};  // fp32 input: the mid and lo pieces
  uint32_t xlo[2][4] = {};
  v128 = 0.f;
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
  return U;
}

// Group sums of the normalized transform and the chunk's dequantization
// factor f, as float2 (sum, f) per group of the chunk (groups g0 .. g0 + 7).
template <int L>
__device__ __forceinline__ void xform_group_sums(const v16f& U, float v128, int g0, int lane, float f,
                                                 float2* lds_xf) {
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
    const int h = lane >> 5;
#pragma unroll
    for (int Q = 0; Q < 4; ++Q) {
      float sm = (U[4 * Q] + U[4 * Q + 1]) + (U[4 * Q + 2] + U[4 * Q + 3]);
#pragma unroll
      for (int j = 0; j < 5; ++j) sm += xor_lane(sm, j, lane);
      if ((lane & 31) == 0) lds_xf[g0 + h + 2 * Q] = make_float2(sm, f);
    }
  }
}

// Transform one chunk (groups g0 .. g0 + 7 of the operand image) and write
// its limbs and (group sum, f).  lds_a: operand rows [group][limb] of
// arow_bytes bytes (128 of data; LDS images pad them); lds_xf: float2 per
// group.  Both may be LDS or global memory.
template <int L, int DT>
__device__ __forceinline__ void xform_chunk(const XformIn<DT>& in, int g0, int lane, const v4u cfirst[2],
                                            const v4u csecond[2], char* lds_a, float2* lds_xf, int arow_bytes) {
  float v128;
  const v16f U = xform_rotate<L, DT>(in, lane, cfirst, csecond, v128);
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
  char* const arow = lds_a + static_cast<int64_t>(g0 + h) * (kXfLimbs * arow_bytes) + (lane & 31) * 4;
#pragma unroll
  for (int Q = 0; Q < 4; ++Q) {
    const uint32_t a0 = qd[4 * Q], a1 = qd[4 * Q + 1], a2 = qd[4 * Q + 2], a3 = qd[4 * Q + 3];
    const uint32_t l0 = (__builtin_amdgcn_perm(a1, a0, 0x0C0C0400u) | __builtin_amdgcn_perm(a3, a2, 0x04000C0Cu)) ^ 0x80808080u;
    const uint32_t l1 = (__builtin_amdgcn_perm(a1, a0, 0x0C0C0501u) | __builtin_amdgcn_perm(a3, a2, 0x05010C0Cu)) ^ 0x80808080u;
    const uint32_t l2 = (__builtin_amdgcn_perm(a1, a0, 0x0C0C0602u) | __builtin_amdgcn_perm(a3, a2, 0x06020C0Cu)) ^ 0x80808080u;
    const uint32_t l3 = __builtin_amdgcn_perm(a1, a0, 0x0C0C0703u) | __builtin_amdgcn_perm(a3, a2, 0x07030C0Cu);
    char* row = arow + static_cast<int64_t>(2 * Q) * (kXfLimbs * arow_bytes);  // group g0 + h + 2 Q
    *reinterpret_cast<uint32_t*>(row) = l0;
    *reinterpret_cast<uint32_t*>(row + arow_bytes) = l1;
    *reinterpret_cast<uint32_t*>(row + 2 * arow_bytes) = l2;
    *reinterpret_cast<uint32_t*>(row + 3 * arow_bytes) = l3;
  }
  // 6. group sums of the normalized transform
  xform_group_sums<L>(U, v128, g0, lane, f, lds_xf);
}

}  // namespace tb
