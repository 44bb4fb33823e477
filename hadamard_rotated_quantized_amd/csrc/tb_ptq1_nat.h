// The PTQ1_0 kernels' operand image and code operand in natural element
// order [kwkr.cn/news/564617, "packing-format engineering": dense trits, five
// per byte].  The trit table turns a trit byte into its five codes as bytes;
// laid end to end they are the group's codes in natural order, which the
// matmul takes as its int8 operand once the activation's limb rows are in
// natural order too.
#pragma once

#include "tb_xform.h"

namespace tb {

// The operand image in natural element order, for the PTQ1_0 kernels: byte p
// of a (group, limb) row is element p of the group.  xform_chunk (tb_xform.h)
// writes each 16-element block transposed (byte 4 x + t = element x + 4 t),
// the order the 2-bit code-word decode produces; PTQ1_0's trit table gives
// the codes in natural order instead.  Same scaling and limbs as
// xform_chunk; before the stores the lanes of each quad (the four lanes that
// hold one 16-element block) transpose their dwords bytewise (two DPP
// exchanges and two byte permutes per dword).
template <int L, int DT>
__device__ __forceinline__ void xform_chunk_natural(const XformIn<DT>& in, int g0, int lane, const v4u cfirst[2],
                                                    const v4u csecond[2], char* img, float2* xf, int arow_bytes) {
  float v128;
  const v16f U = xform_rotate<L, DT>(in, lane, cfirst, csecond, v128);
  float m = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(U[r]));
#pragma unroll
  for (int j = 0; j < 6; ++j) m = fmaxf(m, xor_lane(m, j, lane));
  const uint32_t mb = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(__float_as_uint(m))));
  int e = static_cast<int>((mb >> 23) & 0xFF) - 127;
  e = mb == 0 ? 0 : (e < -90 ? -90 : e);
  const float sigma = __uint_as_float(static_cast<uint32_t>(29 - e + 127) << 23);
  const float f = __uint_as_float(static_cast<uint32_t>(e - 29 + 127) << 23) * inv_sqrt_block_or_one<L>();
  uint32_t qd[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) qd[r] = static_cast<uint32_t>(static_cast<int>(U[r] * sigma)) + 0x808080u;
  // quad transpose selectors: with lane x ^ 2, then with lane x ^ 1
  const int x = lane & 3;
  const uint32_t sel1 = (x >> 1) ? 0x03020706u : 0x05040100u;
  const uint32_t sel2 = (x & 1) ? 0x03070105u : 0x06020400u;
  auto quad_t = [&](uint32_t d) {
    const uint32_t p = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(d), 0x4E, 0xF, 0xF, false));
    const uint32_t d1 = __builtin_amdgcn_perm(p, d, sel1);
    const uint32_t q = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(d1), 0xB1, 0xF, 0xF, false));
    return __builtin_amdgcn_perm(q, d1, sel2);
  };
  const int h = lane >> 5;
  char* const arow = img + static_cast<int64_t>(g0 + h) * (kXfLimbs * arow_bytes) + (lane & 31) * 4;
#pragma unroll
  for (int Q = 0; Q < 4; ++Q) {
    const uint32_t a0 = qd[4 * Q], a1 = qd[4 * Q + 1], a2 = qd[4 * Q + 2], a3 = qd[4 * Q + 3];
    const uint32_t l0 = (__builtin_amdgcn_perm(a1, a0, 0x0C0C0400u) | __builtin_amdgcn_perm(a3, a2, 0x04000C0Cu)) ^ 0x80808080u;
    const uint32_t l1 = (__builtin_amdgcn_perm(a1, a0, 0x0C0C0501u) | __builtin_amdgcn_perm(a3, a2, 0x05010C0Cu)) ^ 0x80808080u;
    const uint32_t l2 = (__builtin_amdgcn_perm(a1, a0, 0x0C0C0602u) | __builtin_amdgcn_perm(a3, a2, 0x06020C0Cu)) ^ 0x80808080u;
    const uint32_t l3 = __builtin_amdgcn_perm(a1, a0, 0x0C0C0703u) | __builtin_amdgcn_perm(a3, a2, 0x07030C0Cu);
    char* row = arow + static_cast<int64_t>(2 * Q) * (kXfLimbs * arow_bytes);
    *reinterpret_cast<uint32_t*>(row) = quad_t(l0);
    *reinterpret_cast<uint32_t*>(row + arow_bytes) = quad_t(l1);
    *reinterpret_cast<uint32_t*>(row + 2 * arow_bytes) = quad_t(l2);
    *reinterpret_cast<uint32_t*>(row + 3 * arow_bytes) = quad_t(l3);
  }
  xform_group_sums<L>(U, v128, g0, lane, f, xf);
}

// Trit byte -> its five codes (lowest base-3 digit first) as bytes 0-4 of an
// 8-byte entry (256 entries; bytes above 242 decode to whatever digits the
// division gives, which the host-side unpack rejects).
__device__ __forceinline__ uint2 trit_entry(uint32_t b) {
  uint32_t lo = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    lo |= (b % 3u) << (8 * m);
    b /= 3u;
  }
  return make_uint2(lo, b % 3u);
}

// The 128 codes of a PTQ1_0 block as 32 dwords of int8 operand bytes in
// natural order: tb(i) returns trit byte i (0 .. 25), lut the table.  Byte
// dword o (codes 4 o .. 4 o + 3) starts at entry 4 o / 5, byte 4 o % 5.
template <class TritByte>
__device__ __forceinline__ void ptq1_code_bytes(TritByte tb, const uint2* lut, uint32_t cb[32]) {
  uint2 ent[26];
#pragma unroll
  for (int i = 0; i < 26; ++i) ent[i] = lut[tb(i)];
#pragma unroll
  for (int o = 0; o < 32; ++o) {
    const int i = (4 * o) / 5, j = (4 * o) % 5;
    const uint2 a = ent[i];
    const uint2 b = i + 1 < 26 ? ent[i + 1] : make_uint2(0u, 0u);
    if (j == 0) cb[o] = a.x;
    else if (j == 1) cb[o] = __builtin_amdgcn_alignbyte(a.y, a.x, 1);
    else if (j == 2) cb[o] = __builtin_amdgcn_alignbyte(a.y, a.x, 2) | (b.x << 24);
    else if (j == 3) cb[o] = __builtin_amdgcn_alignbyte(a.y, a.x, 3) | (b.x << 16);
    else cb[o] = a.y | (b.x << 8);
  }
}

}  // namespace tb
