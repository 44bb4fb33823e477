// tb_ternary_gemm: the Packed linear for prefill (M activation rows).
//
// Same operation as the GEMV [lpnh.cn/news/2438023, "text model loading";
// kwkr.cn/news/564617, "ternary weights + folded Hadamard rotation" and
// "packing-format engineering"]:
//   y[m][n] = sum_g s[n][g] * (sum_{k in g} c[n][k] xr[m][k]) + b[n][g] * X[m][g]
// with xr = R x[m] and X[m][g] = sum_{k in g} xr[m][k].
//
// gfx950 design: the contraction runs on CDNA4's block-scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4) with fp6 activations and fp4 codes.
//  * The codes need no expansion.  A 2-bit code c in the low half of a 4-bit
//    field is the e2m1 number c / 2, so (w & 0x33333333) and
//    ((w >> 2) & 0x33333333) are two fp4 operand dwords holding the 16 codes
//    of a word; the B block scale 2^1 restores c.
//  * The prep kernel (gemm_prep_mfma_kernel on the matrix cores for blocks
//    0 / 512 / 1024, gemm_prep_kernel with LDS butterflies for 2048 / 4096)
//    rotates each row once per call and writes it as four signed base-16
//    digits per input.  For each run of 32 consecutive inputs
//    of a row, a power-of-two exponent E makes q = round(|xr| 2^-E) a 16-bit
//    integer (the run's largest |xr| maps into [2^15, 2^16)); digit j is
//    (q >> 4j) & 15 with the sign of xr, stored as the e2m3 number digit / 8
//    (the e2m3 bit pattern of d / 8 is the magnitude d itself for d <= 15).
//    Digit j enters the MFMA with the A block scale 2^(E + 4j + 3), byte j of
//    the run's scale dword, so the four digit products of a run sum to
//    c * sign * q * 2^E in the fp32 accumulator.  Each input carries a
//    relative error of at most 2^-16 of its run's largest magnitude.
//  * gemm_mx_kernel tiles the output 64 x 512 per workgroup (8 waves of
//    32 x 128).  Per group of 128 inputs, direct-to-LDS buffer loads bring
//    the activation records, the code words and the scales into a stage of a
//    three-stage LDS ring (one barrier per group); each wave runs 2 k-steps x
//    4 digits x 4 column blocks of MFMAs into a per-group fp32 accumulator
//    and folds y += s * acc in fp32.  The bias term sum_g b[n][g] X[m][g]
//    runs after the loop on fp16 MFMA over the groups, with X (scaled by a
//    per-row power of two) split into an exact-sum fp16 hi + lo pair.
//    Workgroups are mapped so that each XCD walks a contiguous range of an
//    order that covers bands of 8 row tiles column by column: the 32
//    workgroups an XCD runs at once span 8 row tiles x 4 column tiles, so
//    both their activation and their code slices are shared in its L2.
#include <algorithm>
#include <type_traits>

#include "tb_device.h"
#include "tb_xform.h"

namespace tb {

typedef int v8i_g __attribute__((ext_vector_type(8)));
typedef float v16f_g __attribute__((ext_vector_type(16)));
typedef unsigned int v4u_g __attribute__((ext_vector_type(4)));
typedef unsigned int v2u_g __attribute__((ext_vector_type(2)));
typedef float v4f_g __attribute__((ext_vector_type(4)));
typedef _Float16 v8h_g __attribute__((ext_vector_type(8)));

constexpr int kRsrcW3 = 0x00020000;  // buffer resource word 3 (raw buffer, range checked)
constexpr int kOobOff = 0x7FFFFFF0;  // a buffer offset past any size: loads return 0

// Per (row, group) activation record: 4 runs x 4 digits x 24 B (32 fp6
// values each), then the 4 runs' scale dwords.
constexpr int kRunBytes = 96;
constexpr int kScaleOff = 4 * kRunBytes;      // 384
constexpr int kRecBytes = kScaleOff + 16;     // 400
constexpr int kRecUnits = kRecBytes / 16;     // 25

constexpr int kMxBM = 64, kMxBN = 512;        // workgroup tile
constexpr int kMxThreads = 512;               // 8 waves: 2 along M x 4 along N, 32 x 128 each
constexpr int kStageA = kMxBM * kRecBytes;    // 25600 B of activation records
constexpr int kStageC = kMxBN * 32;           // 16384 B of code words (8 per row)
constexpr int kStageS = kMxBN * 4;            // 2048 B: per column the dword holding its scale
constexpr int kStageBytes = kStageA + kStageC + kStageS;  // 44032 B per stage, three stages
constexpr int kADma = kStageA / 1024;         // 25 direct-to-LDS loads of 1 KB (64 lanes x 16 B)
constexpr int kCDma = kADma + kStageC / 1024; // codes: loads 25 .. 40
constexpr int kSDma = kCDma + kStageS / 256;  // scales: loads 41 .. 48 (64 lanes x 4 B)
constexpr int kDmaSlots = 7;                  // load slots per wave and fill (56 slots, 7 of them padding)
constexpr int kPkRec = kMxBN * 32 + kMxBN * 2;  // packed weights: bytes per (column tile, group)
constexpr int kPkScaleOff = kMxBN * 32;         // where the tile's 512 fp16 scales start in that record
// loads per wave and fill: weights as stored (slot 5 issued as two loads) or packed
__host__ __device__ constexpr int fill_loads(bool packed) { return packed ? 6 : 8; }
constexpr int kXcds = 8;
constexpr int kMxBandRows = 8;               // row tiles per band of the tile order
constexpr int kMxMaxSlices = 8;              // K slices per tail tile at most
constexpr uint32_t kFp4Codes = 0x33333333u;
constexpr int kScaleB = 128;                  // E8M0 of 2^1

constexpr int kPrepSuper = 8192;              // inputs per LDS pass of the prep kernel
constexpr int kPrepPadded = kPrepSuper + kPrepSuper / 32;
constexpr int kLdsMaxBytes = 160 * 1024;

static inline int64_t g_align256(int64_t v) { return (v + 255) & ~int64_t(255); }

struct GemmWs {
  int64_t G, Gp;
  int64_t rec_off, xh_off, xl_off, p2_off, total;
};

// Workspace: activation records [M][G][400 B], the scaled group sums as fp16
// hi and lo [M][Gp] (Gp = G rounded up to 16, zero padded), and 2^t per row.
static inline GemmWs gemm_ws_layout(int64_t M, int64_t K) {
  GemmWs w;
  w.G = K / kGroup;
  w.Gp = (w.G + 15) / 16 * 16;
  w.rec_off = 0;
  w.xh_off = g_align256(M * w.G * kRecBytes);
  w.xl_off = w.xh_off + g_align256(M * w.Gp * 2);
  w.p2_off = w.xl_off + g_align256(M * w.Gp * 2);
  w.total = w.p2_off + g_align256(M * 4);
  return w;
}

// Operand value v of a 32-input run multiplies the run's input run_pos(v):
// the B operand dwords of a run are (wa & F), (wa >> 2 & F), (wb & F),
// (wb >> 2 & F) for its two code words wa, wb, so value v is code
// 2 (v & 7) + ((v >> 3) & 1) of word v >> 4.
__host__ __device__ constexpr int run_pos(int v) { return 16 * (v >> 4) + 2 * (v & 7) + ((v >> 3) & 1); }

// LDS index of input i in the prep buffer: one float of padding per 32, so
// the per-thread run reads of 32 threads land on distinct banks.
__device__ __forceinline__ int lpad(int i) { return i + (i >> 5); }

// In-place unnormalized Sylvester transform of every L-chunk of n values in
// the padded buffer (the recurrence H_2n = [[H_n, H_n], [H_n, -H_n]]
// [trdm.cn/news/822023 section 2.2], two butterfly stages per LDS pass).
// Caller has written buf and synchronized; ends with a barrier.
template <int L>
__device__ __forceinline__ void fwht_pad(float* buf, int n) {
  static_assert(L >= 4 && (L & (L - 1)) == 0, "power of two");
  const int tid = threadIdx.x;
  int h = 1;
#pragma unroll
  for (; h * 4 <= L; h *= 4) {
    for (int q = tid; q < n / 4; q += kThreads) {
      const int qc = q & (L / 4 - 1), c = q / (L / 4);
      const int lo = qc & (h - 1), hi = qc / h;
      const int base = c * L + hi * 4 * h + lo;
      const int i0 = lpad(base), i1 = lpad(base + h), i2 = lpad(base + 2 * h), i3 = lpad(base + 3 * h);
      const float a = buf[i0], b = buf[i1], cc = buf[i2], d = buf[i3];
      const float ab0 = a + b, ab1 = a - b, cd0 = cc + d, cd1 = cc - d;
      buf[i0] = ab0 + cd0;
      buf[i1] = ab1 + cd1;
      buf[i2] = ab0 - cd0;
      buf[i3] = ab1 - cd1;
    }
    __syncthreads();
  }
  if (h < L) {  // odd number of index bits: one radix-2 stage left
    for (int q = tid; q < n / 2; q += kThreads) {
      const int qc = q & (L / 2 - 1), c = q / (L / 2);
      const int lo = qc & (h - 1), hi = qc / h;
      const int base = c * L + hi * 2 * h + lo;
      const int i0 = lpad(base), i1 = lpad(base + h);
      const float a = buf[i0], b = buf[i1];
      buf[i0] = a + b;
      buf[i1] = a - b;
    }
    __syncthreads();
  }
}

__device__ __forceinline__ uint16_t half_bits(float v) {
  const _Float16 hv = static_cast<_Float16>(v);
  uint16_t u;
  __builtin_memcpy(&u, &hv, 2);
  return u;
}

// One workgroup per activation row.  Dynamic LDS: kPrepPadded floats of
// transform buffer, then G floats of group sums.
template <int L, int DT>
__global__ __launch_bounds__(kThreads) void gemm_prep_kernel(const void* __restrict__ x,
                                                             const int8_t* __restrict__ signs, int K, int G,
                                                             int Gp, uint8_t* __restrict__ rec,
                                                             uint16_t* __restrict__ xh, uint16_t* __restrict__ xl,
                                                             float* __restrict__ p2) {
  extern __shared__ float prep_lds[];
  float* buf = prep_lds;
  float* xs = prep_lds + kPrepPadded;
  __shared__ float red[kThreads / 64];
  const int tid = threadIdx.x;
  const int64_t m = blockIdx.x;
  float inv = 1.f;
  if constexpr (L > 0) inv = inv_sqrt_block<L>();

  for (int c0 = 0; c0 < K; c0 += kPrepSuper) {
    const int n = min(kPrepSuper, K - c0);  // a multiple of 128 and of L
    // 8 consecutive inputs and their signs per vector load; every load of a
    // thread is issued before any of them is stored
    constexpr int kVec = 8, kIters = kPrepSuper / kVec / kThreads;
    static_assert(kPrepSuper % (kVec * kThreads) == 0, "prep pass tiling");
    float xv[kIters][kVec];
    uint2 sv[kIters];
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int i = (tid + it * kThreads) * kVec;
      sv[it] = make_uint2(0x01010101u, 0x01010101u);  // +1 bytes
      if (i < n) {
        const int64_t e = m * K + c0 + i;  // 8-element aligned: K is a multiple of 128
        if constexpr (DT == TB_F32) {
          const float4 a = reinterpret_cast<const float4*>(x)[e / 4];
          const float4 b = reinterpret_cast<const float4*>(x)[e / 4 + 1];
          xv[it][0] = a.x; xv[it][1] = a.y; xv[it][2] = a.z; xv[it][3] = a.w;
          xv[it][4] = b.x; xv[it][5] = b.y; xv[it][6] = b.z; xv[it][7] = b.w;
        } else {
          const uint4 u = reinterpret_cast<const uint4*>(x)[e / 8];
          const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            xv[it][2 * q] = __uint_as_float(w[q] << 16);
            xv[it][2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
          }
        }
        if constexpr (L > 0) sv[it] = reinterpret_cast<const uint2*>(signs + c0)[i / kVec];
      }
    }
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int i = (tid + it * kThreads) * kVec;
      if (i < n) {
#pragma unroll
        for (int q = 0; q < kVec; ++q) {
          const uint32_t sb = ((q < 4 ? sv[it].x : sv[it].y) >> (8 * (q & 3))) & 0x80u;  // bit 7: -1
          buf[lpad(i + q)] = __uint_as_float(__float_as_uint(xv[it][q]) ^ (sb << 24));
        }
      }
    }
    __syncthreads();
    if constexpr (L > 0) fwht_pad<L>(buf, n);

    // one run of 32 inputs per thread; 4 consecutive threads form a group
    for (int r = tid; r < n / 32; r += kThreads) {
      float v[32];
      float mx = 0.f, part = 0.f;
#pragma unroll
      for (int t = 0; t < 32; ++t) {
        v[t] = buf[33 * r + run_pos(t)] * inv;
        mx = fmaxf(mx, fabsf(v[t]));
        part += v[t];
      }
      int E = 0;
      if (mx > 0.f) E = min(max(__builtin_amdgcn_frexp_expf(mx) - 16, -130), 112);
      uint32_t d[24];
#pragma unroll
      for (int i = 0; i < 24; ++i) d[i] = 0;
#pragma unroll
      for (int t = 0; t < 32; ++t) {
        const float a = ldexpf(fabsf(v[t]), -E);
        const uint32_t q = min(static_cast<uint32_t>(rintf(a)), 65535u);
        const uint32_t sg = (__float_as_uint(v[t]) >> 31) << 5;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t f = sg | ((q >> (4 * j)) & 15u);
          const int bit = 6 * t, dw = 6 * j + bit / 32, sh = bit % 32;
          d[dw] |= f << sh;
          if (sh > 26) d[dw + 1] |= f >> (32 - sh);
        }
      }
      const uint32_t e0 = static_cast<uint32_t>(E + 130);
      const uint32_t sc = e0 | ((e0 + 4) << 8) | ((e0 + 8) << 16) | ((e0 + 12) << 24);
      const int64_t gk = (c0 >> 7) + (r >> 2);
      uint8_t* dst = rec + (m * G + gk) * kRecBytes;
      v4u_g* o = reinterpret_cast<v4u_g*>(dst + (r & 3) * kRunBytes);
#pragma unroll
      for (int u = 0; u < 6; ++u) o[u] = v4u_g{d[4 * u], d[4 * u + 1], d[4 * u + 2], d[4 * u + 3]};
      *reinterpret_cast<uint32_t*>(dst + kScaleOff + 4 * (r & 3)) = sc;
      part += __shfl_xor(part, 1);
      part += __shfl_xor(part, 2);
      if ((r & 3) == 0) xs[gk] = part;
    }
    __syncthreads();
  }

  // per-row power of two for the bias operand: max |X| * 2^-t in [2^14, 2^15)
  float mxx = 0.f;
  for (int g = tid; g < G; g += kThreads) mxx = fmaxf(mxx, fabsf(xs[g]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mxx = fmaxf(mxx, __shfl_xor(mxx, o));
  if ((tid & 63) == 0) red[tid >> 6] = mxx;
  __syncthreads();
  mxx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int t = mxx > 0.f ? __builtin_amdgcn_frexp_expf(mxx) - 15 : 0;
  for (int g = tid; g < Gp; g += kThreads) {
    const float xv = g < G ? ldexpf(xs[g], -t) : 0.f;
    const uint16_t hb = half_bits(xv);
    const float rem = xv - half_bits_to_float(hb);
    xh[m * Gp + g] = hb;
    xl[m * Gp + g] = half_bits(rem);
  }
  if (tid == 0) p2[m] = ldexpf(1.f, t);
}

// The same records from the matrix-core transform (blocks 0, 512, 1024): one
// workgroup of min(chunks, 8) waves per activation row, wave w taking chunks
// w, w + waves, ... of 1024 inputs (at most 128 VGPRs, so several rows share
// a CU).  xform_rotate leaves lane l holding, in registers 4 Q + t,
// inputs (l & 3) | t << 2 | ((l >> 2) & 7) << 4 | (l >> 5) << 7 | Q << 8 of
// the chunk: for each Q a run of 32 inputs sits on 8 consecutive lanes (4
// each), and lane bits b0 = l & 1, b1 = (l >> 1) & 1, b2 = (l >> 2) & 1 put
// its 4 inputs at operand positions 16 b2 + 8 b0 + b1 + 2 t.  So the lane's
// four 6-bit fields of a digit sit at bits 6 b1 + 12 t of the 48-bit window
// starting at bit 96 b2 + 48 b0 of the digit's 24 bytes; lane pairs (b1 = 0,
// 1) merge their fields and the b1 = 0 lane writes the window into the
// wave's LDS copy of the chunk's 8 records (3200 contiguous bytes of the
// workspace), which then goes out as full-wave 16-byte stores.
template <int L, int DT>
__global__ __launch_bounds__(512, 4) void gemm_prep_mfma_kernel(const void* __restrict__ x,
                                                             const int8_t* __restrict__ signs, int K, int G, int Gp,
                                                             uint8_t* __restrict__ rec, uint16_t* __restrict__ xh,
                                                             uint16_t* __restrict__ xl, float* __restrict__ p2) {
  extern __shared__ float2 prep_xs2[];  // (group sum, -) per group of the row's chunks
  __shared__ float red[8];
  __shared__ __attribute__((aligned(16))) uint8_t prep_stage[8][8 * kRecBytes];  // per wave: a chunk's records
  constexpr int ESZ = DT == TB_F32 ? 4 : 2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nthreads = static_cast<int>(blockDim.x), nwaves = nthreads >> 6;
  const int64_t m = blockIdx.x;
  const int nch = (K + 1023) >> 10;
  const auto rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(x) + m * K * ESZ), 0, K * ESZ, kRsrcWord3);
  const auto rsg = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(signs), 0, L > 0 ? K : 0, kRsrcWord3);
  const v4u* cst = reinterpret_cast<const v4u*>(&kXformConst.w[xf_mode<L>()][0][lane][0]);
  const v4u* cst2 = reinterpret_cast<const v4u*>(&kXformConst.w[xf_mode<L>()][1][lane][0]);
  const v4u cf[2] = {cst[0], cst[1]};
  const v4u cs[2] = {cst2[0], cst2[1]};
  const float inv = inv_sqrt_block_or_one<L>();
  const int b0 = lane & 1, b1 = (lane >> 1) & 1, b2 = (lane >> 2) & 1;
  const int rr = (lane >> 3) & 3;  // run of the group
  const int h = lane >> 5;
  uint8_t* const stg = prep_stage[wave];
  for (int c = wave; c < nch; c += nwaves) {
    XformIn<DT> in;
    xform_issue<L, DT>(rx, rsg, static_cast<int64_t>(c) * 1024, c * 1024, lane, in);
    float v128;
    const v16f U = xform_rotate<L, DT>(in, lane, cf, cs, v128);
    xform_group_sums<L>(U, v128, 8 * c, lane, 0.f, prep_xs2);
#pragma unroll
    for (int Q = 0; Q < 4; ++Q) {
      float xr[4];
      float mx = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        xr[t] = U[4 * Q + t] * inv;
        mx = fmaxf(mx, fabsf(xr[t]));
      }
      mx = fmaxf(mx, xor_lane(mx, 0, lane));
      mx = fmaxf(mx, xor_lane(mx, 1, lane));
      mx = fmaxf(mx, xor_lane(mx, 2, lane));
      int E = 0;
      if (mx > 0.f) E = min(max(__builtin_amdgcn_frexp_expf(mx) - 16, -130), 112);
      uint32_t q[4], sg[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        q[t] = min(static_cast<uint32_t>(rintf(ldexpf(fabsf(xr[t]), -E))), 65535u);
        sg[t] = (__float_as_uint(xr[t]) >> 31) << 5;
      }
      uint8_t* const dst = stg + (h + 2 * Q) * kRecBytes;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint64_t w = 0;  // the lane's fields of digit j in the 48-bit window
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint64_t f = sg[t] | ((q[t] >> (4 * j)) & 15u);
          w |= f << (12 * t + 6 * b1);
        }
        uint32_t lo = static_cast<uint32_t>(w), hi = static_cast<uint32_t>(w >> 32);
        lo |= static_cast<uint32_t>(xor_lane_i(static_cast<int>(lo), 1, lane));
        hi |= static_cast<uint32_t>(xor_lane_i(static_cast<int>(hi), 1, lane));
        if (b1 == 0) {
          uint8_t* d = dst + rr * kRunBytes + 24 * j + 12 * b2;
          if (b0 == 0) {
            *reinterpret_cast<uint32_t*>(d) = lo;
            *reinterpret_cast<uint16_t*>(d + 4) = static_cast<uint16_t>(hi);
          } else {
            *reinterpret_cast<uint16_t*>(d + 6) = static_cast<uint16_t>(lo);
            *reinterpret_cast<uint32_t*>(d + 8) = (lo >> 16) | (hi << 16);
          }
        }
      }
      if ((lane & 7) == 0) {
        const uint32_t e0 = static_cast<uint32_t>(E + 130);
        *reinterpret_cast<uint32_t*>(dst + kScaleOff + 4 * rr) = e0 | ((e0 + 4) << 8) | ((e0 + 8) << 16) | ((e0 + 12) << 24);
      }
    }
    // the chunk's records (its groups below G) as 16-byte stores; a wave's
    // LDS accesses complete in order, so the reads see the writes above
    const int units = min(8, G - 8 * c) * (kRecBytes / 16);
    v4u_g* const out = reinterpret_cast<v4u_g*>(rec + (m * G + 8 * c) * kRecBytes);
#pragma unroll
    for (int i = 0; i < (8 * kRecBytes / 16 + 63) / 64; ++i) {
      const int u = 64 * i + lane;
      if (u < units) out[u] = reinterpret_cast<const v4u_g*>(stg)[u];
    }
  }
  __syncthreads();
  // per-row power of two for the bias operand: max |X| * 2^-t in [2^14, 2^15)
  float mxx = 0.f;
  for (int g = tid; g < G; g += nthreads) mxx = fmaxf(mxx, fabsf(prep_xs2[g].x));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mxx = fmaxf(mxx, __shfl_xor(mxx, o));
  if (lane == 0) red[wave] = mxx;
  __syncthreads();
  mxx = red[0];
  for (int w = 1; w < nwaves; ++w) mxx = fmaxf(mxx, red[w]);
  const int t = mxx > 0.f ? __builtin_amdgcn_frexp_expf(mxx) - 15 : 0;
  for (int g = tid; g < Gp; g += nthreads) {
    const float xv = g < G ? ldexpf(prep_xs2[g].x, -t) : 0.f;
    const uint16_t hb = half_bits(xv);
    const float rem = xv - half_bits_to_float(hb);
    xh[m * Gp + g] = hb;
    xl[m * Gp + g] = half_bits(rem);
  }
  if (tid == 0) p2[m] = ldexpf(1.f, t);
}

__device__ __forceinline__ v8h_g as_v8h(v4u_g u) { return __builtin_bit_cast(v8h_g, u); }

// The three LDS stages of the matmul ring.
__shared__ __attribute__((aligned(16))) uint8_t mx_stage0[kStageBytes];
__shared__ __attribute__((aligned(16))) uint8_t mx_stage1[kStageBytes];
__shared__ __attribute__((aligned(16))) uint8_t mx_stage2[kStageBytes];
__shared__ __attribute__((aligned(16))) uint8_t mx_sink[1024];  // target of the padding loads

template <int ST>
__device__ __forceinline__ uint8_t* mx_stage() {
  if constexpr (ST == 0) return mx_stage0;
  else if constexpr (ST == 1) return mx_stage1;
  else return mx_stage2;
}

// Raw buffer resource (stride 0, range checked against `bytes`) as the four
// scalar words the buffer instructions take.
typedef __amdgpu_buffer_rsrc_t v4i_rs;
__device__ __forceinline__ v4i_rs rsrc_words(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcW3);
}

// Direct-to-LDS buffer loads: lane l's 16 (or 4) bytes at voff land at LDS
// address lds + 16 l (4 l).  The destination keeps the provenance of its
// stage array (mx_stage0/1/2 are separate LDS objects), so the compiler's
// wait tracking sees that a fill of one stage does not alias the reads of
// another and the ring's own s_waitcnt vmcnt(n) sets the pace.
typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, lds_u8* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, lds_u8* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 4, voff, 0, 0, 0);
}

// s_waitcnt vmcnt(n) with the other counters left alone
__host__ __device__ constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Operands of one k-step for one wave, read from a stage: the run's 6 units
// (4 digits x 24 B), its scale dword, (first k-step only) the four code
// words of each column block that both k-steps use (words 4h .. 4h + 3 of
// the group: x, y for k-step 0, z, w for k-step 1), and (second k-step only)
// the scale dwords of the lane's columns.
struct MxOps {
  v4u_g a[6];
  v4u_g c[4];
  int sc;
  uint32_t sd[4];
};

// Digit J of a run as an fp6 operand: dwords 6 J .. 6 J + 5 of the run.
template <int J>
__device__ __forceinline__ v8i_g digit_operand(const v4u_g* u) {
  int d[6];
#pragma unroll
  for (int i = 0; i < 6; ++i) d[i] = static_cast<int>(u[(6 * J + i) / 4][(6 * J + i) % 4]);
  return v8i_g{d[0], d[1], d[2], d[3], d[4], d[5], 0, 0};
}

// Digit J against the four column blocks; the A scale is byte J of sc.
template <int J>
__device__ __forceinline__ void mx_digit(const v4u_g* u, const v8i_g* bop, int sc, bool zero, v16f_g* acc) {
  const v8i_g a = digit_operand<J>(u);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    acc[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bop[nb], zero ? v16f_g{} : acc[nb], 2, 4, J, sc,
                                                              0, kScaleB);
}

// First output row and column of tile t of the tile order: bands of
// kMxBandRows row tiles, each walked column by column.
__device__ __forceinline__ void mx_tile_origin(int t, int MT, int NT, int& m0, int& n0) {
  const int band = t / (kMxBandRows * NT), within = t - band * kMxBandRows * NT;
  const int gm = min(kMxBandRows, MT - band * kMxBandRows);
  m0 = (band * kMxBandRows + within % gm) * kMxBM;
  n0 = (within / gm) * kMxBN;
}

// Workgroups [0, 8 per_xcd) compute the first tiles_main tiles of the tile
// order over all of K.  When the tiles do not fill a whole number of rounds
// of the chip, the remaining tiles ("tail") are cut into ks slices of the
// groups each, one workgroup per (tile, slice) after the main ones; a tail
// workgroup writes its 64 x 512 partial sums to part[unit] (slice 0 adds the
// bias term) and gemm_tail_sum_kernel adds the slices in order.
//
// PK: the codes and scales come from the packed copy (gemm_pack_kernel), one
// contiguous kPkRec-byte record per (column tile, group), instead of the
// stored rows: every stage-fill load then reads 1 KB of contiguous memory.
template <bool PK>
__global__ __launch_bounds__(kMxThreads) void gemm_mx_kernel(
    const uint8_t* __restrict__ rec, const uint16_t* __restrict__ xh, const uint16_t* __restrict__ xl,
    const float* __restrict__ p2, const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ wpk, const uint16_t* __restrict__ biases, float* __restrict__ y, int M, int N, int G,
    int Gp, int MT, int NT, int per_xcd, int tiles_main, int ks, float* __restrict__ part, int bvec) {
  constexpr int kFillLoads = fill_loads(PK);
  // XCD-aware tile order: workgroup w runs on XCD w % 8; XCD x owns the
  // contiguous range [x * per_xcd, (x + 1) * per_xcd) of the tile order, so
  // the workgroups an XCD runs at once (8 row tiles x 4 column tiles) share
  // both activation and code slices in its L2.
  const int wg = blockIdx.x;
  int tile, unit = -1, gbeg = 0, gend = G;
  if (wg < per_xcd * kXcds) {
    tile = (wg % kXcds) * per_xcd + wg / kXcds;
    if (tile >= tiles_main) return;
  } else {
    unit = wg - per_xcd * kXcds;
    const int ti = unit / ks, slice = unit - ti * ks;
    tile = tiles_main + ti;
    gbeg = slice * G / ks;
    gend = (slice + 1) * G / ks;
  }
  int m0, n0;
  mx_tile_origin(tile, MT, NT, m0, n0);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int r32 = lane & 31, h = lane >> 5;
  const int W = G * 8;  // code words per weight row

  // Rows past M or N read as zeros through the buffer range checks (sizes
  // computed in 32-bit scalar arithmetic: one tile spans kMxBM / kMxBN rows).
  const int mrows = min(M - m0, kMxBM), nrows = min(N - n0, kMxBN);
  const v4i_rs ra = rsrc_words(rec + static_cast<int64_t>(m0) * G * kRecBytes, mrows * G * kRecBytes);
  const v4i_rs rc = PK ? rsrc_words(wpk + static_cast<int64_t>(n0 / kMxBN) * G * kPkRec, G * kPkRec)
                       : rsrc_words(codes + static_cast<int64_t>(n0) * W, nrows * W * 4);
  const int cstride = PK ? kPkRec : 32;  // code bytes from one group to the next
  // scales: the aligned dword holding s[n][g]; the resource starts at the
  // dword holding s[n0][0] and ends with the dword holding s[N-1][G-1]
  const uint64_t sp = reinterpret_cast<uint64_t>(scales) + static_cast<uint64_t>(n0) * G * 2;
  const uint64_t sbase = sp & ~uint64_t(3);
  const int shalf0 = static_cast<int>((sp - sbase) >> 1);  // 0 or 1
  const v4i_rs rs = rsrc_words(reinterpret_cast<const void*>(sbase), ((shalf0 + (N - n0) * G) * 2 + 3) & ~3);

  // Stage fill: 49 direct-to-LDS loads; wave w issues loads w + 8 i, i < 7.
  // Load q < 25 brings activation units 64 q + lane (unit p is record row
  // p / 25, unit p % 25); loads 25 .. 40 bring code units: LDS unit
  // pos = 64 (q - 25) + lane holds half (pos & 1) ^ x of column n = pos / 2,
  // x = bit 2 ^ bit 3 of n, so that the 16-byte reads of 16 consecutive
  // columns fall on distinct banks; loads 41 .. 48 bring the scale dword of
  // column 64 (q - 41) + lane; loads 49 .. 55 are padding.
  int voff[kDmaSlots];
#pragma unroll
  for (int i = 0; i < kDmaSlots; ++i) {
    const int q = wave + 8 * i;
    if (q < kADma) {
      const int p = 64 * q + lane;
      voff[i] = (p / kRecUnits) * G * kRecBytes + (p % kRecUnits) * 16;
    } else if (q < kCDma) {
      const int pos = 64 * (q - kADma) + lane, n = pos >> 1;
      const int hx = (pos & 1) ^ (((n >> 2) ^ (n >> 3)) & 1);  // the half of column n this unit holds
      voff[i] = PK ? (2 * n + hx) * 16 : n * W * 4 + hx * 16;
    } else if (q < kSDma) {
      // half index of s[n][0] from the resource base; packed: 8 scales per lane
      voff[i] = PK ? kPkScaleOff + 16 * lane : shalf0 + (64 * (q - kCDma) + lane) * G;
    } else {
      voff[i] = kOobOff;
    }
  }
  // lane's own columns: which half of the staged dword is s[n][g] (flips with g)
  int spar[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) spar[nb] = (shalf0 + (wn * 128 + 32 * nb + r32) * G) & 1;

  // Every wave issues exactly kFillLoads loads per fill, so one
  // s_waitcnt vmcnt(kFillLoads) leaves exactly the newest fill in flight.
  // Slots 0-2 are activation units for every wave and slot 4 code units;
  // the kinds of slots 3, 5 and 6 depend on the wave (3: activation for wave
  // 0, codes otherwise; 5: codes for wave 0, scales otherwise; 6: scales for
  // wave 0, padding otherwise) and are chosen with wave-uniform selects of
  // the source and the LDS target, so the fill has no branches: slot 5 is
  // issued as a 16-byte and a 4-byte load, one of them aimed at mx_sink with
  // an out-of-range offset.  Packed weights: slot 5 is codes for wave 0 and
  // the group's 512 scales for wave 1 (one 16-byte load each), slot 6 is not
  // issued.  A fill past the last group loads zeros.
  const bool w0 = wave == 0;
  auto fill = [&](auto stage_tag, int g) {
    constexpr int ST = decltype(stage_tag)::value;
    lds_u8* const dst = (lds_u8*)(mx_stage<ST>());
    lds_u8* const sink = (lds_u8*)(mx_sink);
    const bool live = g < gend;
#pragma unroll
    for (int i = 0; i < 3; ++i) dma16(ra, dst + (wave + 8 * i) * 1024, live ? voff[i] + g * kRecBytes : kOobOff);
    dma16(w0 ? ra : rc, dst + (wave + 24) * 1024, live ? voff[3] + g * (w0 ? kRecBytes : cstride) : kOobOff);
    dma16(rc, dst + (wave + 32) * 1024, live ? voff[4] + g * cstride : kOobOff);
    if constexpr (PK) {
      // slot 5: codes for wave 0, all 512 scales (16 B per lane) for wave 1
      const bool w1 = wave == 1;
      dma16(rc, w0 ? dst + 40 * 1024 : (w1 ? dst + kStageA + kStageC : sink),
            live && (w0 || w1) ? voff[5] + g * kPkRec : kOobOff);
    } else {
      dma16(rc, w0 ? dst + 40 * 1024 : sink, live && w0 ? voff[5] + g * 32 : kOobOff);
      dma4(rs, w0 ? sink : dst + kStageA + kStageC + (wave - 1) * 256,
           live && !w0 ? ((voff[5] + g) >> 1) * 4 : kOobOff);
      dma4(rs, w0 ? dst + kStageA + kStageC + 7 * 256 : sink, live && w0 ? ((voff[6] + g) >> 1) * 4 : kOobOff);
    }
  };

  // LDS read positions of this lane: record row, and the code unit of column
  // block 0 (bits 2 and 3 of the column are those of r32 in every block)
  const int arow = (wm * 32 + r32) * kRecBytes;
  const int cread = kStageA + (2 * (wn * 128 + r32) + (h ^ (((r32 >> 2) ^ (r32 >> 3)) & 1))) * 16;  // + 1024 per block

  v16f_g yv[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) yv[nb] = v16f_g{};

  // Reads of k-step s of the group held by stage ST, in three parts so that
  // they can be spread between the MFMAs of the k-step before.
  auto read_a = [&](auto stage_tag, int s, MxOps& o, int part) {
    constexpr int ST = decltype(stage_tag)::value;
    const uint8_t* S = mx_stage<ST>();
    const int run = 2 * h + s;
#pragma unroll
    for (int u = 3 * part; u < 3 * part + 3; ++u)
      o.a[u] = *reinterpret_cast<const v4u_g*>(S + arow + run * kRunBytes + 16 * u);
    if (part == 1) o.sc = *reinterpret_cast<const int*>(S + arow + kScaleOff + 4 * run);
  };
  auto read_c = [&](auto stage_tag, int s, MxOps& o, bool with_scales) {
    constexpr int ST = decltype(stage_tag)::value;
    const uint8_t* S = mx_stage<ST>();
    if (s == 0) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) o.c[nb] = *reinterpret_cast<const v4u_g*>(S + cread + 1024 * nb);
    }
    if (with_scales) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        o.sd[nb] = PK ? *reinterpret_cast<const uint16_t*>(S + kStageA + kStageC + 2 * (wn * 128 + 32 * nb + r32))
                      : *reinterpret_cast<const uint32_t*>(S + kStageA + kStageC + 4 * (wn * 128 + 32 * nb + r32));
    }
  };
  auto decode = [&](const MxOps& o, v8i_g* bop, int ks) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const uint32_t wa = ks ? o.c[nb].z : o.c[nb].x, wb = ks ? o.c[nb].w : o.c[nb].y;
      bop[nb] = v8i_g{static_cast<int>(wa & kFp4Codes), static_cast<int>((wa >> 2) & kFp4Codes),
                      static_cast<int>(wb & kFp4Codes), static_cast<int>((wb >> 2) & kFp4Codes), 0, 0, 0, 0};
    }
  };

  // Software pipeline at k-step granularity, one barrier per group placed
  // between the group's two k-steps.  Per group g:
  //   MFMAs of k-step 0, with the reads of k-step 1 and the refill of the
  //   stage of group g + 2 issued between them; wait for this wave's part of
  //   the fill of group g + 1 and for its reads; barrier;
  //   MFMAs of k-step 1, with the reads of k-step 0 of group g + 1 between
  //   them; fold group g.
  // The matrix core works through each digit's MFMAs while the reads and
  // loads placed after them are issued.  The refill overwrites the stage of
  // group g - 1, whose reads all completed before the previous barrier.
  fill(std::integral_constant<int, 0>{}, gbeg);
  fill(std::integral_constant<int, 1>{}, gbeg + 1);
  __builtin_amdgcn_s_waitcnt(wait_vm(kFillLoads));
  __builtin_amdgcn_s_barrier();
  MxOps r0;
  read_a(std::integral_constant<int, 0>{}, 0, r0, 0);
  read_a(std::integral_constant<int, 0>{}, 0, r0, 1);
  read_c(std::integral_constant<int, 0>{}, 0, r0, false);

  auto step = [&](auto stage_tag, int g) {
    constexpr int ST = decltype(stage_tag)::value;
    constexpr auto next = std::integral_constant<int, (ST + 1) % 3>{};
    MxOps r1;
    v8i_g bop[4];
    v16f_g acc[4];
    decode(r0, bop, 0);
    mx_digit<0>(r0.a, bop, r0.sc, true, acc);
    __builtin_amdgcn_sched_barrier(0);
    read_a(stage_tag, 1, r1, 0);
    __builtin_amdgcn_sched_barrier(0);
    mx_digit<1>(r0.a, bop, r0.sc, false, acc);
    __builtin_amdgcn_sched_barrier(0);
    read_a(stage_tag, 1, r1, 1);
    __builtin_amdgcn_sched_barrier(0);
    mx_digit<2>(r0.a, bop, r0.sc, false, acc);
    __builtin_amdgcn_sched_barrier(0);
    read_c(stage_tag, 1, r1, true);
    fill(std::integral_constant<int, (ST + 2) % 3>{}, g + 2);
    __builtin_amdgcn_sched_barrier(0);
    mx_digit<3>(r0.a, bop, r0.sc, false, acc);
    // keep this k-step's MFMAs ahead of the barrier: the matrix core works
    // through them while the waves synchronize
    asm volatile("" ::"v"(acc[0]), "v"(acc[1]), "v"(acc[2]), "v"(acc[3]));
    // every read of this wave done (the refill of the next-but-one group
    // targets what other waves read before this barrier) and this wave's
    // part of the next group's stage landed
    __builtin_amdgcn_s_waitcnt(wait_vm(kFillLoads) & ~(0xF << 8));
    __builtin_amdgcn_s_barrier();
    decode(r0, bop, 1);
    mx_digit<0>(r1.a, bop, r1.sc, false, acc);
    __builtin_amdgcn_sched_barrier(0);
    read_a(next, 0, r0, 0);
    __builtin_amdgcn_sched_barrier(0);
    mx_digit<1>(r1.a, bop, r1.sc, false, acc);
    __builtin_amdgcn_sched_barrier(0);
    read_a(next, 0, r0, 1);
    __builtin_amdgcn_sched_barrier(0);
    mx_digit<2>(r1.a, bop, r1.sc, false, acc);
    __builtin_amdgcn_sched_barrier(0);
    read_c(next, 0, r0, false);
    __builtin_amdgcn_sched_barrier(0);
    mx_digit<3>(r1.a, bop, r1.sc, false, acc);
    // per-group scale fold in fp32
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const uint32_t sd = r1.sd[nb];
      const float sv = half_bits_to_float(static_cast<uint16_t>(!PK && (spar[nb] ^ (g & 1)) ? sd >> 16 : sd));
#pragma unroll
      for (int r = 0; r < 16; ++r) yv[nb][r] = fmaf(sv, acc[nb][r], yv[nb][r]);
    }
  };
  for (int g = gbeg; g < gend; g += 3) {
    step(std::integral_constant<int, 0>{}, g);
    if (g + 1 >= gend) break;
    step(std::integral_constant<int, 1>{}, g + 1);
    if (g + 2 >= gend) break;
    step(std::integral_constant<int, 2>{}, g + 2);
  }

  __builtin_amdgcn_s_waitcnt(wait_vm(0));  // the ring's trailing (zero) fills

  // bias term: y += 2^t[m] * sum_g Xs[m][g] * b[n][g] on fp16 MFMA
  const auto rxh = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(xh + static_cast<int64_t>(m0) * Gp), 0,
                                                     mrows * Gp * 2, kRsrcW3);
  const auto rxl = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(xl + static_cast<int64_t>(m0) * Gp), 0,
                                                     mrows * Gp * 2, kRsrcW3);
  const auto rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(biases + static_cast<int64_t>(n0) * G), 0,
                                                    nrows * G * 2, kRsrcW3);
  v16f_g tb4[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) tb4[nb] = v16f_g{};
  // (once per tile: tail slices other than the first skip it).  The loads
  // of step s2 + 1 are issued before the MFMAs of step s2.  When G is a
  // multiple of 8 and the biases are 16-byte aligned (bvec, from the host),
  // the 8 biases an operand needs are one aligned 16-byte load (a block of 8
  // groups lies wholly below G or wholly past it).
  const int nbias = gbeg == 0 ? Gp / 16 : 0;
  auto bias_loads = [&](int s2, v4u_g& ahv, v4u_g& alv, v4u_g* bq) {
    const int g0 = 16 * s2 + 8 * h;
    const int xo = ((wm * 32 + r32) * Gp + g0) * 2;
    ahv = __builtin_amdgcn_raw_buffer_load_b128(rxh, xo, 0, 0);
    alv = __builtin_amdgcn_raw_buffer_load_b128(rxl, xo, 0, 0);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int bo = (wn * 128 + 32 * nb + r32) * G;
      if (bvec) {
        bq[nb] = __builtin_amdgcn_raw_buffer_load_b128(rb, g0 < G ? (bo + g0) * 2 : kOobOff, 0, 0);
      } else {
        uint32_t bw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ga = g0 + 2 * i, gb = ga + 1;
          const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rb, ga < G ? (bo + ga) * 2 : kOobOff, 0, 0);
          const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rb, gb < G ? (bo + gb) * 2 : kOobOff, 0, 0);
          bw[i] = lo | (hi << 16);
        }
        bq[nb] = v4u_g{bw[0], bw[1], bw[2], bw[3]};
      }
    }
  };
  v4u_g ahv, alv, bq[4];
  if (nbias > 0) bias_loads(0, ahv, alv, bq);
  for (int s2 = 0; s2 < nbias; ++s2) {
    const v4u_g ah = ahv, al = alv;
    v4u_g bc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) bc[nb] = bq[nb];
    if (s2 + 1 < nbias) bias_loads(s2 + 1, ahv, alv, bq);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const v8h_g bv = as_v8h(bc[nb]);
      tb4[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_v8h(ah), bv, tb4[nb], 0, 0, 0);
      tb4[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_v8h(al), bv, tb4[nb], 0, 0, 0);
    }
  }
  // D layout of a 32 x 32 block: lane l, register r holds row
  // 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
  const auto rp = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p2 + m0), 0, mrows * 4, kRsrcW3);
  float pr[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const v4f_g u = __builtin_bit_cast(
        v4f_g, __builtin_amdgcn_raw_buffer_load_b128(rp, (wm * 32 + 8 * q + 4 * h) * 4, 0, 0));
    pr[4 * q] = u.x;
    pr[4 * q + 1] = u.y;
    pr[4 * q + 2] = u.z;
    pr[4 * q + 3] = u.w;
  }
  if (unit < 0) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int n = n0 + wn * 128 + 32 * nb + r32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 32 + 8 * (r / 4) + 4 * h + (r % 4);
        const float v = fmaf(pr[r], tb4[nb][r], yv[nb][r]);
        if (m < M && n < N) y[static_cast<int64_t>(m) * N + n] = v;
      }
    }
  } else {
    // the whole 64 x 512 partial tile, row-major (rows past M or N hold
    // sums over zeros)
    float* const pt = part + static_cast<int64_t>(unit) * (kMxBM * kMxBN);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int nn = wn * 128 + 32 * nb + r32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int mm = wm * 32 + 8 * (r / 4) + 4 * h + (r % 4);
        pt[mm * kMxBN + nn] = fmaf(pr[r], tb4[nb][r], yv[nb][r]);
      }
    }
  }
}

// The packed copy of the weights for gemm_mx_kernel<true>: per (column tile
// nt of 512 rows, group g) one record of kPkRec bytes at (nt G + g) kPkRec:
// the 512 rows' 32 code bytes of group g in row order, then their 512 fp16
// scales.  Rows past N are zeros.  Threads [0, code_threads) copy the codes,
// 16 bytes of each of 4 rows: 8 consecutive threads read one row's 128
// bytes of groups 4 g4 .. 4 g4 + 3 (a cache line) and write them to those
// groups' records, so a wave's load reads 8 whole lines and its store
// writes runs of 256 bytes.  The threads
// after them write the scale units, 8 scales (16 bytes) each.
constexpr int kPkRowsPerThread = 4, kPkRowStep = kMxBN / kPkRowsPerThread;
static_assert(kMxBN % kPkRowsPerThread == 0 && (kPkRowStep & (kPkRowStep - 1)) == 0, "pack kernel thread map");
__global__ __launch_bounds__(256) void gemm_pack_kernel(const uint32_t* __restrict__ codes,
                                                        const uint16_t* __restrict__ scales, int N, int G,
                                                        int64_t code_threads, int64_t units, uint8_t* __restrict__ wpk) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int W = G * 8;
  if (i < code_threads) {
    const int G4 = (G + 3) >> 2;
    const int q = static_cast<int>(i & 7), nl0 = static_cast<int>((i >> 3) & (kPkRowStep - 1));
    const int64_t rest = i / (8 * kPkRowStep);  // threads per (column tile, group quad)
    const int nt = static_cast<int>(rest / G4), g4 = static_cast<int>(rest - static_cast<int64_t>(nt) * G4);
    const int g = 4 * g4 + (q >> 1), half = q & 1;
    if (g >= G) return;
    // rows nl0 + kPkRowStep k of the tile: kPkRowsPerThread loads in flight per thread
    v4u_g v[kPkRowsPerThread];
#pragma unroll
    for (int k = 0; k < kPkRowsPerThread; ++k) {
      const int n = nt * kMxBN + nl0 + kPkRowStep * k;
      v[k] = v4u_g{0u, 0u, 0u, 0u};
      if (n < N) v[k] = *reinterpret_cast<const v4u_g*>(codes + static_cast<int64_t>(n) * W + g * 8 + half * 4);
    }
    uint8_t* const dst = wpk + (static_cast<int64_t>(nt) * G + g) * kPkRec + half * 16;
#pragma unroll
    for (int k = 0; k < kPkRowsPerThread; ++k)
      *reinterpret_cast<v4u_g*>(dst + (nl0 + kPkRowStep * k) * 32) = v[k];
    return;
  }
  const int64_t j = i - code_threads;
  if (j >= units) return;
  const int64_t r = j >> 6;  // record (nt, g)
  const int u = static_cast<int>(j & 63);
  const int nt = static_cast<int>(r / G), g = static_cast<int>(r - static_cast<int64_t>(nt) * G);
  const int n0 = nt * kMxBN + 8 * u;
  uint32_t h[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) h[k] = n0 + k < N ? scales[static_cast<int64_t>(n0 + k) * G + g] : 0u;
  *reinterpret_cast<v4u_g*>(wpk + r * kPkRec + kPkScaleOff + u * 16) =
      v4u_g{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// y of the tail tiles: the ks slice partials of each element added in slice
// order.  One thread per 4 consecutive columns of a tile row.
__global__ __launch_bounds__(256) void gemm_tail_sum_kernel(const float* __restrict__ part, float* __restrict__ y,
                                                            int M, int N, int MT, int NT, int tiles_main, int ks) {
  constexpr int kQuads = kMxBM * kMxBN / 4;  // float4 per partial tile
  const int idx = static_cast<int>(blockIdx.x) * 256 + static_cast<int>(threadIdx.x);
  const int ti = idx / kQuads, e4 = idx - ti * kQuads;
  const int r = e4 / (kMxBN / 4), c4 = e4 - r * (kMxBN / 4);
  int m0, n0;
  mx_tile_origin(tiles_main + ti, MT, NT, m0, n0);
  const float4* p = reinterpret_cast<const float4*>(part) + static_cast<int64_t>(ti) * ks * kQuads + e4;
  float4 a = p[0];
  for (int sl = 1; sl < ks; ++sl) {
    const float4 b = p[static_cast<int64_t>(sl) * kQuads];
    a.x += b.x;
    a.y += b.y;
    a.z += b.z;
    a.w += b.w;
  }
  const int m = m0 + r, n = n0 + 4 * c4;
  if (m >= M) return;
  float* const yr = y + static_cast<int64_t>(m) * N;
  if (n < N) yr[n] = a.x;
  if (n + 1 < N) yr[n + 1] = a.y;
  if (n + 2 < N) yr[n + 2] = a.z;
  if (n + 3 < N) yr[n + 3] = a.w;
}

static inline int prep_lds_bytes(int64_t G) { return static_cast<int>((kPrepPadded + G) * 4); }

template <int L>
static void launch_gemm_prep(const void* x, int dt, const int8_t* signs, int64_t M, int64_t K, const GemmWs& lay,
                             char* ws, hipStream_t st) {
  uint8_t* rec = reinterpret_cast<uint8_t*>(ws + lay.rec_off);
  uint16_t* xh = reinterpret_cast<uint16_t*>(ws + lay.xh_off);
  uint16_t* xl = reinterpret_cast<uint16_t*>(ws + lay.xl_off);
  float* p2 = reinterpret_cast<float*>(ws + lay.p2_off);
  if constexpr (L <= 1024) {
    // blocks 0 / 512 / 1024: the matrix-core transform, one wave per chunk
    const int lds_m = static_cast<int>((K + 1023) / 1024 * 8 * sizeof(float2));
    auto km = dt == TB_F32 ? gemm_prep_mfma_kernel<L, TB_F32> : gemm_prep_mfma_kernel<L, TB_BF16>;
    if (lds_m > 64 * 1024)
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(km), hipFuncAttributeMaxDynamicSharedMemorySize, lds_m);
    const int waves = static_cast<int>(std::min<int64_t>((K + 1023) / 1024, 8));
    hipLaunchKernelGGL(km, dim3(static_cast<unsigned>(M)), dim3(64 * waves), static_cast<size_t>(lds_m), st, x, signs,
                       static_cast<int>(K), static_cast<int>(lay.G), static_cast<int>(lay.Gp), rec, xh, xl, p2);
    return;
  }
  const int lds = prep_lds_bytes(lay.G);
  auto kern = dt == TB_F32 ? gemm_prep_kernel<L, TB_F32> : gemm_prep_kernel<L, TB_BF16>;
  if (lds > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(M)), dim3(kThreads), static_cast<size_t>(lds), st, x, signs,
                     static_cast<int>(K), static_cast<int>(lay.G), static_cast<int>(lay.Gp), rec, xh, xl, p2);
}

static int gemm_ws_check(const void* workspace, size_t ws_bytes, int64_t M, int64_t K, const char* who) {
  const GemmWs lay = gemm_ws_layout(M, K);
  if (!workspace || ws_bytes < static_cast<size_t>(lay.total)) {
    set_error("%s: workspace of %zu bytes at %p, need %lld", who, ws_bytes, workspace, (long long)lay.total);
    return TB_ERR_WORKSPACE;
  }
  if (!aligned(workspace, 16)) {
    set_error("%s: workspace must be 16-byte aligned", who);
    return TB_ERR_ALIGN;
  }
  return TB_OK;
}

// the prep kernel reads x and signs with 16- and 8-byte vector loads
static int gemm_align_checks(const void* x, const int8_t* signs, const char* who) {
  if (!aligned(x, 16) || (signs && !aligned(signs, 16))) {
    set_error("%s: x and signs must be 16-byte aligned", who);
    return TB_ERR_ALIGN;
  }
  return TB_OK;
}

static int gemm_shape_checks(int64_t M, int64_t K, int64_t N, const char* who) {
  if (M < 0 || N < 0) {
    set_error("%s: M and N must be >= 0", who);
    return TB_ERR_ARG;
  }
  if (K <= 0) {
    set_error("%s: K must be positive (got %lld)", who, (long long)K);
    return TB_ERR_ARG;
  }
  if (K % kGroup) {
    set_error("%s: K=%lld is not a multiple of the group size %d", who, (long long)K, kGroup);
    return TB_ERR_SHAPE;
  }
  const int64_t G = K / kGroup;
  if (prep_lds_bytes(G) > kLdsMaxBytes || M > 0x7FFFFFFF) {
    set_error("%s: K=%lld or M=%lld too large for the prefill path", who, (long long)K, (long long)M);
    return TB_ERR_SHAPE;
  }
  // 32-bit buffer offsets: one tile's records, the code and scale rows of one
  // call, and the fp16 group sums of all rows
  const int64_t Gp = (G + 15) / 16 * 16;
  if (kMxBM * G * kRecBytes > kOobOff || N * G * 32 > kOobOff || M * Gp * 2 > kOobOff || N > 0x7FFFFFFF) {
    set_error("%s: M=%lld N=%lld K=%lld too large for one call", who, (long long)M, (long long)N, (long long)K);
    return TB_ERR_SHAPE;
  }
  const int64_t MT = (M + kMxBM - 1) / kMxBM, NT = (N + kMxBN - 1) / kMxBN;
  if ((MT * NT + kXcds - 1) / kXcds * kXcds > 0x7FFFFFFF) {
    set_error("%s: M x N too large for one launch", who);
    return TB_ERR_SHAPE;
  }
  return TB_OK;
}

static int gemm_run_checks(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, const float* y,
                           const char* who) {
  TB_TRY(check_container(codes, scales, biases, who));
  if (!y) {
    set_error("%s: y is NULL", who);
    return TB_ERR_ARG;
  }
  if (!aligned(y, 4)) {
    set_error("%s: y must be 4-byte aligned", who);
    return TB_ERR_ALIGN;
  }
  return TB_OK;
}

static void gemm_prepare_launch(const void* x, int x_dtype, int64_t M, int64_t K, const int8_t* signs, int block,
                                void* workspace, hipStream_t st) {
  const GemmWs lay = gemm_ws_layout(M, K);
  char* ws = static_cast<char*>(workspace);
  switch (block) {
    case 0: launch_gemm_prep<0>(x, x_dtype, signs, M, K, lay, ws, st); break;
    case 512: launch_gemm_prep<512>(x, x_dtype, signs, M, K, lay, ws, st); break;
    case 1024: launch_gemm_prep<1024>(x, x_dtype, signs, M, K, lay, ws, st); break;
    case 2048: launch_gemm_prep<2048>(x, x_dtype, signs, M, K, lay, ws, st); break;
    default: launch_gemm_prep<4096>(x, x_dtype, signs, M, K, lay, ws, st); break;
  }
}

// The tail split of one run: with one workgroup per CU, T output tiles take
// ceil(T / CUs) rounds; when the last round is at most half full, its
// T mod CUs tiles are cut into ks = CUs / (T mod CUs) slices of the groups
// (at most kMxMaxSlices, at least 2 groups each), whose partial tiles follow
// the prepared activation in the workspace.
//
// With at least kPkMinRowTiles row tiles (each of which streams all the
// weights), the run also packs the codes and scales into one contiguous
// record per (column tile, group) after the partial tiles (gemm_pack_kernel,
// NT x G x kPkRec bytes) and the matmul reads that copy.
constexpr int kPkMinRowTiles = 4;
struct GemmSplit {
  int64_t tiles_main, tiles_tail, ks, part_off, pk_off, total;
  bool pk;
};
static GemmSplit gemm_split_plan(int64_t M, int64_t K, int64_t N, int cus) {
  const GemmWs lay = gemm_ws_layout(M, K);
  const int64_t MT = (M + kMxBM - 1) / kMxBM, NT = (N + kMxBN - 1) / kMxBN;
  const int64_t T = MT * NT;
  const int64_t rem = cus > 0 ? T % cus : 0;
  const int64_t ks = rem > 0 ? std::min<int64_t>(cus / rem, kMxMaxSlices) : 0;
  GemmSplit sp{T, 0, 1, lay.total, lay.total, lay.total, false};
  if (T > cus && rem > 0 && ks >= 2 && lay.G >= 2 * ks) {
    sp.tiles_main = T - rem;
    sp.tiles_tail = rem;
    sp.ks = ks;
    sp.total = sp.part_off + rem * ks * kMxBM * kMxBN * 4;
  }
  if (MT >= kPkMinRowTiles) {
    sp.pk = true;
    sp.pk_off = g_align256(sp.total);
    sp.total = sp.pk_off + NT * lay.G * kPkRec;
  }
  return sp;
}

static void gemm_run_launch(const void* workspace, size_t ws_bytes, int64_t M, int64_t K, const uint32_t* codes,
                            const uint16_t* scales, const uint16_t* biases, int64_t N, float* y, hipStream_t st) {
  const GemmWs lay = gemm_ws_layout(M, K);
  const char* ws = static_cast<const char*>(workspace);
  const uint8_t* rec = reinterpret_cast<const uint8_t*>(ws + lay.rec_off);
  const uint16_t* xh = reinterpret_cast<const uint16_t*>(ws + lay.xh_off);
  const uint16_t* xl = reinterpret_cast<const uint16_t*>(ws + lay.xl_off);
  const float* p2 = reinterpret_cast<const float*>(ws + lay.p2_off);
  const int64_t MT = (M + kMxBM - 1) / kMxBM, NT = (N + kMxBN - 1) / kMxBN;
  GemmSplit sp = gemm_split_plan(M, K, N, device_cus());
  if (ws_bytes < static_cast<size_t>(sp.total))
    sp = GemmSplit{MT * NT, 0, 1, lay.total, lay.total, lay.total, false};
  float* part = reinterpret_cast<float*>(const_cast<char*>(ws) + sp.part_off);
  uint8_t* wpk = reinterpret_cast<uint8_t*>(const_cast<char*>(ws) + sp.pk_off);
  if (sp.pk) {
    const int64_t code_threads = NT * ((lay.G + 3) / 4) * 8 * kPkRowStep;
    const int64_t units = NT * lay.G * 64;  // scale units
    hipLaunchKernelGGL(gemm_pack_kernel, dim3(static_cast<unsigned>((code_threads + units + 255) / 256)), dim3(256), 0,
                       st, codes, scales, static_cast<int>(N), static_cast<int>(lay.G), code_threads, units, wpk);
  }
  const int64_t per_xcd = (sp.tiles_main + kXcds - 1) / kXcds;
  const int64_t grid = per_xcd * kXcds + sp.tiles_tail * sp.ks;
  hipLaunchKernelGGL(sp.pk ? gemm_mx_kernel<true> : gemm_mx_kernel<false>, dim3(static_cast<unsigned>(grid)),
                     dim3(kMxThreads), 0, st, rec, xh, xl, p2, codes, scales, wpk, biases, y, static_cast<int>(M),
                     static_cast<int>(N), static_cast<int>(lay.G), static_cast<int>(lay.Gp), static_cast<int>(MT),
                     static_cast<int>(NT), static_cast<int>(per_xcd), static_cast<int>(sp.tiles_main),
                     static_cast<int>(sp.ks), part, static_cast<int>(lay.G % 8 == 0 && aligned(biases, 16)));
  if (sp.tiles_tail > 0) {
    const int64_t blocks = sp.tiles_tail * (kMxBM * kMxBN / 4) / 256;
    hipLaunchKernelGGL(gemm_tail_sum_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, part, y,
                       static_cast<int>(M), static_cast<int>(N), static_cast<int>(MT), static_cast<int>(NT),
                       static_cast<int>(sp.tiles_main), static_cast<int>(sp.ks));
  }
}

}  // namespace tb

using namespace tb;

extern "C" size_t tb_ternary_gemm_workspace_size(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || K % kGroup) return 0;
  return static_cast<size_t>(gemm_ws_layout(M, K).total);
}

extern "C" size_t tb_ternary_gemm_workspace_size_n(int64_t M, int64_t K, int64_t N) {
  if (M <= 0 || K <= 0 || K % kGroup || N <= 0) return tb_ternary_gemm_workspace_size(M, K);
  return static_cast<size_t>(gemm_split_plan(M, K, N, device_cus()).total);
}

extern "C" int tb_ternary_gemm_prepare(const void* x, int x_dtype, int64_t M, int64_t K, const int8_t* signs,
                                       int block, void* workspace, size_t ws_bytes, void* stream) {
  const char* who = "tb_ternary_gemm_prepare";
  TB_TRY(gemm_shape_checks(M, K, 0, who));
  TB_TRY(check_rotation(K, block, signs, who));
  if (M == 0) return TB_OK;
  TB_TRY(check_dtype(x_dtype, x, who));
  TB_TRY(gemm_align_checks(x, signs, who));
  TB_TRY(gemm_ws_check(workspace, ws_bytes, M, K, who));
  gemm_prepare_launch(x, x_dtype, M, K, signs, block, workspace, static_cast<hipStream_t>(stream));
  TB_LAUNCH_CHECK(who);
  return TB_OK;
}

extern "C" int tb_ternary_gemm_run(const void* workspace, size_t ws_bytes, int64_t M, int64_t K,
                                   const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t N,
                                   float* y, void* stream) {
  const char* who = "tb_ternary_gemm_run";
  TB_TRY(gemm_shape_checks(M, K, N, who));
  if (M == 0 || N == 0) return TB_OK;
  TB_TRY(gemm_run_checks(codes, scales, biases, y, who));
  TB_TRY(gemm_ws_check(workspace, ws_bytes, M, K, who));
  gemm_run_launch(workspace, ws_bytes, M, K, codes, scales, biases, N, y, static_cast<hipStream_t>(stream));
  TB_LAUNCH_CHECK(who);
  return TB_OK;
}

extern "C" int tb_ternary_gemm(const void* x, int x_dtype, int64_t M, int64_t K, const int8_t* signs, int block,
                               const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t N,
                               float* y, void* workspace, size_t ws_bytes, void* stream) {
  const char* who = "tb_ternary_gemm";
  TB_TRY(gemm_shape_checks(M, K, N, who));
  TB_TRY(check_rotation(K, block, signs, who));
  if (M == 0 || N == 0) return TB_OK;
  TB_TRY(check_dtype(x_dtype, x, who));
  TB_TRY(gemm_align_checks(x, signs, who));
  TB_TRY(gemm_run_checks(codes, scales, biases, y, who));
  TB_TRY(gemm_ws_check(workspace, ws_bytes, M, K, who));
  hipStream_t st = static_cast<hipStream_t>(stream);
  gemm_prepare_launch(x, x_dtype, M, K, signs, block, workspace, st);
  TB_LAUNCH_CHECK(who);
  gemm_run_launch(workspace, ws_bytes, M, K, codes, scales, biases, N, y, st);
  TB_LAUNCH_CHECK(who);
  return TB_OK;
}
