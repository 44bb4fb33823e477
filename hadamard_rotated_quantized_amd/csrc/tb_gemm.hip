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
//  * gemm_prep_kernel rotates each row once per call and writes it as four
//    signed base-16 digits per input.  For each run of 32 consecutive inputs
//    of a row, a power-of-two exponent E makes q = round(|xr| 2^-E) a 16-bit
//    integer (the run's largest |xr| maps into [2^15, 2^16)); digit j is
//    (q >> 4j) & 15 with the sign of xr, stored as the e2m3 number digit / 8
//    (the e2m3 bit pattern of d / 8 is the magnitude d itself for d <= 15).
//    Digit j enters the MFMA with the A block scale 2^(E + 4j + 3), byte j of
//    the run's scale dword, so the four digit products of a run sum to
//    c * sign * q * 2^E in the fp32 accumulator.  Each input carries a
//    relative error of at most 2^-16 of its run's largest magnitude.
//  * gemm_mx_kernel tiles the output 128 x 256 per workgroup (8 waves of
//    32 x 128).  Per group of 128 inputs it stages the activation records and
//    the code words through registers into a double-buffered LDS stage (one
//    barrier per group), runs 2 k-steps x 4 digits x 4 column blocks of MFMAs
//    into a per-group fp32 accumulator and folds y += s * acc in fp32.  The
//    bias term sum_g b[n][g] X[m][g] runs after the loop on fp16 MFMA over
//    the groups, with X (scaled by a per-row power of two) split into an
//    exact-sum fp16 hi + lo pair.  Workgroups are mapped so that each XCD
//    walks contiguous output tiles in M-major order: the XCD's workgroups
//    share one activation row tile in that XCD's L2 while the codes stream.
#include "tb_device.h"

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

constexpr int kMxBM = 128, kMxBN = 256;       // workgroup tile
constexpr int kMxThreads = 512;               // 8 waves: 4 along M x 2 along N
constexpr int kStageA = kMxBM * kRecBytes;    // 51200 B of activation records
constexpr int kStageC = kMxBN * 32;           // 8192 B of code words (8 per row)
constexpr int kStageBytes = kStageA + kStageC;
constexpr int kMxLds = 2 * kStageBytes;       // double-buffered: 118784 B
constexpr int kAUnits = kMxBM * kRecUnits;    // 3200 16-byte units per stage
constexpr int kAUnitLoads = (kAUnits + kMxThreads - 1) / kMxThreads;  // 7
constexpr int kXcds = 8;
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
    for (int i = tid; i < n; i += kThreads) {
      float v = load_x<DT>(x, m * K + c0 + i);
      if constexpr (L > 0) v *= static_cast<float>(signs[c0 + i]);
      buf[lpad(i)] = v;
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

__device__ __forceinline__ v8h_g as_v8h(v4u_g u) { return __builtin_bit_cast(v8h_g, u); }

// Digits 2 JP and 2 JP + 1 of one run (48 B of the record at rp) against the
// four column blocks' fp4 codes; digit j takes byte j of the scale dword.
template <int JP>
__device__ __forceinline__ void mx_digit_pair(const uint8_t* rp, const v8i_g* bop, int sc, bool first,
                                              v16f_g* acc) {
  const v4u_g* ap = reinterpret_cast<const v4u_g*>(rp + 48 * JP);
  const v4u_g u0 = ap[0], u1 = ap[1], u2 = ap[2];
  const v8i_g alo = v8i_g{static_cast<int>(u0.x), static_cast<int>(u0.y), static_cast<int>(u0.z),
                          static_cast<int>(u0.w), static_cast<int>(u1.x), static_cast<int>(u1.y), 0, 0};
  const v8i_g ahi = v8i_g{static_cast<int>(u1.z), static_cast<int>(u1.w), static_cast<int>(u2.x),
                          static_cast<int>(u2.y), static_cast<int>(u2.z), static_cast<int>(u2.w), 0, 0};
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const v16f_g c_in = first ? v16f_g{} : acc[nb];
    acc[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(alo, bop[nb], c_in, 2, 4, 2 * JP, sc, 0, kScaleB);
    acc[nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ahi, bop[nb], acc[nb], 2, 4, 2 * JP + 1, sc, 0,
                                                              kScaleB);
  }
}

__global__ __launch_bounds__(kMxThreads) void gemm_mx_kernel(
    const uint8_t* __restrict__ rec, const uint16_t* __restrict__ xh, const uint16_t* __restrict__ xl,
    const float* __restrict__ p2, const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ biases, float* __restrict__ y, int M, int N, int G, int Gp, int MT, int NT,
    int per_xcd) {
  extern __shared__ __attribute__((aligned(16))) uint8_t mx_lds[];

  // XCD-aware tile order: workgroup w runs on XCD w % 8; XCD x owns the
  // contiguous M-major tile range [x * per_xcd, (x + 1) * per_xcd).
  const int wg = blockIdx.x;
  const int jx = wg / kXcds;
  const int tile = (wg % kXcds) * per_xcd + jx;
  if (jx >= per_xcd || tile >= MT * NT) return;
  const int m0 = (tile / NT) * kMxBM;
  const int n0 = (tile % NT) * kMxBN;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 3, wn = wave >> 2;
  const int r32 = lane & 31, h = lane >> 5;
  const int W = G * 8;  // code words per weight row

  // Rows past M or N read as zeros through the buffer range checks (sizes
  // computed in 32-bit scalar arithmetic: one tile spans at most 128 / 256 rows).
  const int mrows = min(M - m0, kMxBM), nrows = min(N - n0, kMxBN);
  const auto ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(rec + static_cast<int64_t>(m0) * G * kRecBytes), 0, mrows * G * kRecBytes, kRsrcW3);
  const auto rc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(codes + static_cast<int64_t>(n0) * W), 0,
                                                    nrows * W * 4, kRsrcW3);
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales + static_cast<int64_t>(n0) * G), 0,
                                                    nrows * G * 2, kRsrcW3);

  // staging: 4 threads per activation row of the tile, thread t taking the
  // 16-byte units (t % 4) + 4 i of row t / 4; code unit tid is (row tid / 2,
  // half tid % 2).  Offsets differ per unit by constants.
  const int arow_t = tid >> 2, au0 = tid & 3;
  const int aoff = arow_t * G * kRecBytes + au0 * 16;
  const int apos = arow_t * kRecBytes + au0 * 16;
  const bool a_last = au0 + 4 * (kAUnitLoads - 1) < kRecUnits;  // unit 24 exists for au0 == 0 only
  const int crow = tid >> 1, chalf = tid & 1;
  const int coff = crow * W * 4 + chalf * 16;
  const int cpos = 2 * crow + (chalf ^ ((crow >> 2) & 1));  // swizzled LDS unit
  const int soff = (wn * 128 + r32) * G * 2;                 // + 64 G per column block

  v4u_g sa[kAUnitLoads], scw;
  uint32_t sraw[4];
  // g == G loads zeros (every offset out of range): the loop body has no branch
  auto gload = [&](int g) {
    const bool in = g < G;
#pragma unroll
    for (int i = 0; i < kAUnitLoads; ++i) {
      const bool ok = in && (i < kAUnitLoads - 1 || a_last);
      sa[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, ok ? aoff + g * kRecBytes + 64 * i : kOobOff, 0, 0);
    }
    scw = __builtin_amdgcn_raw_buffer_load_b128(rc, in ? coff + g * 32 : kOobOff, 0, 0);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      sraw[nb] = __builtin_amdgcn_raw_buffer_load_b16(rs, in ? soff + nb * 64 * G + 2 * g : kOobOff, 0, 0);
  };
  auto lstore = [&](int st) {
    uint8_t* S = mx_lds + st * kStageBytes;
#pragma unroll
    for (int i = 0; i < kAUnitLoads; ++i)
      if (i < kAUnitLoads - 1 || a_last) *reinterpret_cast<v4u_g*>(S + apos + 64 * i) = sa[i];
    *reinterpret_cast<v4u_g*>(S + kStageA + cpos * 16) = scw;
  };

  // LDS read positions of this lane: record row, and the code unit of
  // column block 0 (bit 2 of the column is that of r32 in every block)
  const int arow = (wm * 32 + r32) * kRecBytes;
  const int cread = kStageA + (2 * (wn * 128 + r32) + (h ^ ((r32 >> 2) & 1))) * 16;  // + 1024 per block

  v16f_g yv[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) yv[nb] = v16f_g{};
  float s_cur[4];

  gload(0);
  lstore(0);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) s_cur[nb] = half_bits_to_float(static_cast<uint16_t>(sraw[nb]));
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const uint8_t* S = mx_lds + (g & 1) * kStageBytes;
    gload(g + 1);

    v16f_g acc[4];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int run = 2 * h + s;
      const int sc = *reinterpret_cast<const int*>(S + arow + kScaleOff + 4 * run);
      v8i_g bop[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const v2u_g cw = *reinterpret_cast<const v2u_g*>(S + cread + 1024 * nb + 8 * s);
        const uint32_t wa = cw.x, wb = cw.y;
        bop[nb] = v8i_g{static_cast<int>(wa & kFp4Codes), static_cast<int>((wa >> 2) & kFp4Codes),
                        static_cast<int>(wb & kFp4Codes), static_cast<int>((wb >> 2) & kFp4Codes), 0, 0, 0, 0};
      }
      mx_digit_pair<0>(S + arow + run * kRunBytes, bop, sc, s == 0, acc);
      mx_digit_pair<1>(S + arow + run * kRunBytes, bop, sc, false, acc);
      // keep the next k-step's LDS reads after these MFMAs (register budget)
      __builtin_amdgcn_sched_barrier(0);
    }
    // per-group scale fold in fp32
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) yv[nb][r] = fmaf(s_cur[nb], acc[nb][r], yv[nb][r]);

    // the stage refill waits for this group's loads: keep it after the MFMAs
    asm volatile("" ::"v"(yv[0]), "v"(yv[1]), "v"(yv[2]), "v"(yv[3]) : "memory");
    lstore((g + 1) & 1);
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) s_cur[nb] = half_bits_to_float(static_cast<uint16_t>(sraw[nb]));
  }

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
  for (int s2 = 0; s2 < Gp / 16; ++s2) {
    const int g0 = 16 * s2 + 8 * h;
    const int xo = ((wm * 32 + r32) * Gp + g0) * 2;
    const v4u_g ahv = __builtin_amdgcn_raw_buffer_load_b128(rxh, xo, 0, 0);
    const v4u_g alv = __builtin_amdgcn_raw_buffer_load_b128(rxl, xo, 0, 0);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int bo = (wn * 128 + 32 * nb + r32) * G;
      uint32_t bw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ga = g0 + 2 * i, gb = ga + 1;
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rb, ga < G ? (bo + ga) * 2 : kOobOff, 0, 0);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rb, gb < G ? (bo + gb) * 2 : kOobOff, 0, 0);
        bw[i] = lo | (hi << 16);
      }
      const v8h_g bv = as_v8h(v4u_g{bw[0], bw[1], bw[2], bw[3]});
      tb4[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_v8h(ahv), bv, tb4[nb], 0, 0, 0);
      tb4[nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_v8h(alv), bv, tb4[nb], 0, 0, 0);
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
}

static inline int prep_lds_bytes(int64_t G) { return static_cast<int>((kPrepPadded + G) * 4); }

template <int L>
static void launch_gemm_prep(const void* x, int dt, const int8_t* signs, int64_t M, int64_t K, const GemmWs& lay,
                             char* ws, hipStream_t st) {
  uint8_t* rec = reinterpret_cast<uint8_t*>(ws + lay.rec_off);
  uint16_t* xh = reinterpret_cast<uint16_t*>(ws + lay.xh_off);
  uint16_t* xl = reinterpret_cast<uint16_t*>(ws + lay.xl_off);
  float* p2 = reinterpret_cast<float*>(ws + lay.p2_off);
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

static void gemm_run_launch(const void* workspace, int64_t M, int64_t K, const uint32_t* codes,
                            const uint16_t* scales, const uint16_t* biases, int64_t N, float* y, hipStream_t st) {
  const GemmWs lay = gemm_ws_layout(M, K);
  const char* ws = static_cast<const char*>(workspace);
  const uint8_t* rec = reinterpret_cast<const uint8_t*>(ws + lay.rec_off);
  const uint16_t* xh = reinterpret_cast<const uint16_t*>(ws + lay.xh_off);
  const uint16_t* xl = reinterpret_cast<const uint16_t*>(ws + lay.xl_off);
  const float* p2 = reinterpret_cast<const float*>(ws + lay.p2_off);
  const int64_t MT = (M + kMxBM - 1) / kMxBM, NT = (N + kMxBN - 1) / kMxBN;
  const int64_t per_xcd = (MT * NT + kXcds - 1) / kXcds;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_mx_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kMxLds);
    attr_set = true;
  }
  hipLaunchKernelGGL(gemm_mx_kernel, dim3(static_cast<unsigned>(per_xcd * kXcds)), dim3(kMxThreads),
                     static_cast<size_t>(kMxLds), st, rec, xh, xl, p2, codes, scales, biases, y,
                     static_cast<int>(M), static_cast<int>(N), static_cast<int>(lay.G), static_cast<int>(lay.Gp),
                     static_cast<int>(MT), static_cast<int>(NT), static_cast<int>(per_xcd));
}

}  // namespace tb

using namespace tb;

extern "C" size_t tb_ternary_gemm_workspace_size(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || K % kGroup) return 0;
  return static_cast<size_t>(gemm_ws_layout(M, K).total);
}

extern "C" int tb_ternary_gemm_prepare(const void* x, int x_dtype, int64_t M, int64_t K, const int8_t* signs,
                                       int block, void* workspace, size_t ws_bytes, void* stream) {
  const char* who = "tb_ternary_gemm_prepare";
  TB_TRY(gemm_shape_checks(M, K, 0, who));
  TB_TRY(check_rotation(K, block, signs, who));
  if (M == 0) return TB_OK;
  TB_TRY(check_dtype(x_dtype, x, who));
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
  gemm_run_launch(workspace, M, K, codes, scales, biases, N, y, static_cast<hipStream_t>(stream));
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
  TB_TRY(gemm_run_checks(codes, scales, biases, y, who));
  TB_TRY(gemm_ws_check(workspace, ws_bytes, M, K, who));
  hipStream_t st = static_cast<hipStream_t>(stream);
  gemm_prepare_launch(x, x_dtype, M, K, signs, block, workspace, st);
  TB_LAUNCH_CHECK(who);
  gemm_run_launch(workspace, M, K, codes, scales, biases, N, y, st);
  TB_LAUNCH_CHECK(who);
  return TB_OK;
}
