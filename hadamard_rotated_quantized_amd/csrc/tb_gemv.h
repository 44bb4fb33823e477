// Device pieces shared by the two decode-matmul paths (the two-kernel
// prepare/run path in tb_gemv.hip and the single-launch path in
// tb_gemv_fused.hip): operand layouts, lane exchanges, the in-register
// signed transform of a 1024-input chunk, the exact integer split of the
// rotated activations, and the integer MFMA shapes.
#pragma once

#include <type_traits>

#include "tb_device.h"

namespace tb {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef unsigned int v3u __attribute__((ext_vector_type(3)));

constexpr int kLimbs = 3;
constexpr int kWordsPerGroup = kGroup / kCodesPerWord;  // 8
constexpr int kGroupPad = 4;                            // groups padded to a multiple of 4
// bytes of prepared A operand per (batch row, group): 3 limbs x 8 words x 16 B
constexpr int64_t kAopsGroupBytes = (int64_t)kLimbs * kWordsPerGroup * 16;  // 384
constexpr int kRsrcWord3 = 0x00020000;  // buffer resource word 3 for gfx9-family raw buffers
constexpr int kOob = 0x7FFFFFF0;        // a buffer offset past any size: loads return 0
// LDS layout of the limbs: one 144-byte row (8 x 16 B + 16 B pad) per
// (batch row, group, limb), so the 16-byte reads of the active A lanes land
// on distinct banks.
constexpr int kLdsRow = kWordsPerGroup + 1;  // uint4 per (batch, group, limb) row

__host__ __device__ inline int64_t padded_groups(int64_t K) {
  return (K / kGroup + kGroupPad - 1) / kGroupPad * kGroupPad;
}

// Value of lane l ^ 2^j, with VALU lane exchanges only (no LDS round trip):
// DPP quad permutations for j = 0, 1; DPP row shifts with bank masks for
// j = 2, 3 (the banks whose partner is 4 or 8 lanes up read row_shl, the
// others row_shr); gfx950's permlane16/32 swaps for j = 4, 5 (each swap
// hands one half of the lanes its partner's value in each output).
__device__ __forceinline__ int xor_lane_i(int vi, int j, int lane) {
  int p;
  switch (j) {
    case 0: p = __builtin_amdgcn_mov_dpp(vi, 0xB1, 0xF, 0xF, false); break;  // quad_perm [1,0,3,2]
    case 1: p = __builtin_amdgcn_mov_dpp(vi, 0x4E, 0xF, 0xF, false); break;  // quad_perm [2,3,0,1]
    case 2:
      p = __builtin_amdgcn_update_dpp(0, vi, 0x104, 0xF, 0x5, false);        // row_shl:4, banks 0, 2
      p = __builtin_amdgcn_update_dpp(p, vi, 0x114, 0xF, 0xA, false);        // row_shr:4, banks 1, 3
      break;
    case 3:
      p = __builtin_amdgcn_update_dpp(0, vi, 0x108, 0xF, 0x3, false);        // row_shl:8, banks 0, 1
      p = __builtin_amdgcn_update_dpp(p, vi, 0x118, 0xF, 0xC, false);        // row_shr:8, banks 2, 3
      break;
    case 4: {
      const auto r = __builtin_amdgcn_permlane16_swap(vi, vi, false, false);
      p = (lane & 16) ? static_cast<int>(r[0]) : static_cast<int>(r[1]);
      break;
    }
    default: {
      const auto r = __builtin_amdgcn_permlane32_swap(vi, vi, false, false);
      p = (lane & 32) ? static_cast<int>(r[0]) : static_cast<int>(r[1]);
      break;
    }
  }
  return p;
}

__device__ __forceinline__ float xor_lane(float v, int j, int lane) {
  return __int_as_float(xor_lane_i(__float_as_int(v), j, lane));
}

// Unnormalized Sylvester butterflies of one 1024-input chunk held 16 per
// lane (lane l holds inputs 16 l + r, r < 16), natural order
// [trdm.cn/news/822023 section 2.2]: index bits 0-3 are in-lane, bits 4-9
// are lane bits.  XST cross-lane stages: 6 for a 1024-block, 5 for 512-blocks
// (each half of the wave is then one block).
template <int XST>
__device__ __forceinline__ void fwht_lane16(float v[16], int lane) {
#pragma unroll
  for (int hb = 1; hb < 16; hb <<= 1)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (!(r & hb)) {
        const float a0 = v[r], a1 = v[r + hb];
        v[r] = a0 + a1;
        v[r + hb] = a0 - a1;
      }
#pragma unroll
  for (int j = 0; j < XST; ++j) {
    // butterfly with lane l ^ 2^j: lower lane v + p, upper lane p - v
    const float sgn = ((lane >> j) & 1) ? -1.f : 1.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = fmaf(sgn, v[r], xor_lane(v[r], j, lane));
  }
}

// Exact integer split of one 128-input group held by 8 consecutive lanes (16
// values each).  With f = 2^E, E = ilogb(max |v|) - 21, every v ~= f q with
// |q| <= 2^22 (rounding error at most 2^-23 of the group's largest |v|), and
// q = h 2^16 + m 2^8 + l with balanced digits in [-128, 127]:
//   l = byte 0 of q, m = byte 1 of q + 128, h = byte 2 of q + 32896.
// The three digit planes ("limbs") come back in the byte order of the
// matmul's A operand: dword d carries, in byte j, element d + 4 j of the
// lane's 16 -- the order in which (w >> 2 d) & 0x03030303 extracts codes
// from a 16-code weight word.  xf = (f * sum q, f) of the group.
__device__ __forceinline__ void split_limbs(const float v[16], int lane, uint4 limb[kLimbs], float2& xf) {
  float m = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(v[r]));
  m = fmaxf(m, xor_lane(m, 0, lane));
  m = fmaxf(m, xor_lane(m, 1, lane));
  m = fmaxf(m, xor_lane(m, 2, lane));
  const int E = (m > 0.f) ? ilogbf(m) - 21 : 0;
  int q[16];
  int qs = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    q[r] = static_cast<int>(rintf(ldexpf(v[r], -E)));
    qs += q[r];
  }
  qs += xor_lane_i(qs, 0, lane);
  qs += xor_lane_i(qs, 1, lane);
  qs += xor_lane_i(qs, 2, lane);
  const float f = ldexpf(1.f, E);
  xf = make_float2(f * static_cast<float>(qs), f);
  uint32_t d[kLimbs][4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t a0 = q[e], a1 = q[e + 4], a2 = q[e + 8], a3 = q[e + 12];
    // v_perm_b32 picks bytes of {first, second}: selectors 0-3 address the
    // second operand, 4-7 the first, 0x0C gives a zero byte
    d[0][e] = __builtin_amdgcn_perm(a1, a0, 0x0C0C0400u) | __builtin_amdgcn_perm(a3, a2, 0x04000C0Cu);
    d[1][e] = __builtin_amdgcn_perm(a1 + 128u, a0 + 128u, 0x0C0C0501u) |
              __builtin_amdgcn_perm(a3 + 128u, a2 + 128u, 0x05010C0Cu);
    d[2][e] = __builtin_amdgcn_perm(a1 + 32896u, a0 + 32896u, 0x0C0C0602u) |
              __builtin_amdgcn_perm(a3 + 32896u, a2 + 32896u, 0x06020C0Cu);
  }
#pragma unroll
  for (int l = 0; l < kLimbs; ++l) limb[l] = make_uint4(d[l][0], d[l][1], d[l][2], d[l][3]);
}

// Codes of one 16-code word as the int8 B operand of 4 MFMA K-steps:
// (w >> 2 i) & 0x03030303 holds codes {i, i + 4, i + 8, i + 12} as bytes.
__device__ __forceinline__ v4i decode_word(uint32_t w) {
  v4i r;
  r[0] = static_cast<int>(w & 0x03030303u);
  r[1] = static_cast<int>((w >> 2) & 0x03030303u);
  r[2] = static_cast<int>((w >> 4) & 0x03030303u);
  r[3] = static_cast<int>((w >> 6) & 0x03030303u);
  return r;
}

// Shapes of the two integer MFMA variants.
//   M = 16: v_mfma_i32_16x16x64_i8, 4 lane groups of 16 lanes, one batch row
//           per instruction, 4 groups per span, A row i = 4 lg + r.
//   M = 32: v_mfma_i32_32x32x32_i8, 2 lane halves of 32 lanes, 4 batch rows
//           per instruction, 2 groups per span, A row i = 8 j + 4 lg + r.
template <int M>
struct Mfma {
  static constexpr int GPS = 64 / M;         // groups per span = lane groups
  static constexpr int BPI = M / (4 * GPS);  // batch rows per instruction
  using acc_t = typename std::conditional<M == 16, v4i, v16i>::type;
  __device__ static acc_t mac(v4i a, v4i b, acc_t c) {
    if constexpr (M == 16) return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
};

// Host side of the single-launch path (tb_gemv_fused.hip).
// True when one workgroup can transform the whole input itself: block in
// {0, 512, 1024}, at most 3 chunk transforms per wave, and an LDS footprint
// within the limit for this (B, K, N).
// Host side of the batch-1 band path (tb_gemv_band.hip): true when one
// workgroup per band of output rows can hold the band's packed weights and
// the transformed input in LDS.
bool gemv_band_eligible(int64_t B, int64_t K, int64_t N, int block);
// decode batches of 2 to 8 rows: in-workgroup transform + K-split streaming
// (+ slice sum); the workspace holds the slices' partial rows (0 bytes when
// one slice covers K)
bool gemv_batch_eligible(int64_t B, int64_t K, int64_t N, int block);
size_t gemv_batch_workspace(int64_t B, int64_t K, int64_t N);
void gemv_batch_launch(const void* x, int x_dtype, int64_t B, int64_t K, const int8_t* signs, int block,
                       const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t N, float* y,
                       void* workspace, hipStream_t st);
void gemv_band_launch(const void* x, int x_dtype, int64_t K, const int8_t* signs, int block, const uint32_t* codes,
                      const uint16_t* scales, const uint16_t* biases, int64_t N, float* y, hipStream_t st);

bool gemv_fused_eligible(int64_t B, int64_t K, int64_t N, int block);

// tb_ternary_gemv's argument checks (everything but the workspace) and its
// path choice and launches, for entry points that bring their own workspace
int gemv_checked_args(const void* x, int x_dtype, int64_t B, int64_t K, const int8_t* signs, int block,
                      const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t N,
                      const float* y, const char* who);
int gemv_dispatch(const void* x, int x_dtype, int64_t B, int64_t K, const int8_t* signs, int block,
                  const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t N, float* y,
                  void* workspace, size_t ws_bytes, hipStream_t st, const char* who);
void gemv_fused_launch(const void* x, int x_dtype, int64_t B, int64_t K, const int8_t* signs, int block,
                       const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t N,
                       float* y, hipStream_t st);

}  // namespace tb
