// tb_ternary_gemm: the Packed linear for prefill (M activation rows).
//
// Same operation as the GEMV [lpnh.cn/news/2438023, "text model loading";
// kwkr.cn/news/564617, "ternary weights + folded Hadamard rotation" and
// "packing-format engineering"]:
//   y[m][n] = sum_g s[n][g] * (sum_{k in g} c[n][k] xr[m][k]) + b[n][g] * X[m][g]
// with xr = R x[m] and X[m][g] = sum_{k in g} xr[m][k].
//
// gfx950 design: this case is a dense contraction, so it runs on bf16 MFMA.
//  * gemm_prep_kernel rotates every row of x in LDS and writes the rotated
//    activation as an exact-sum pair of bf16 arrays, hi = bf16(xr) and
//    lo = bf16(xr - hi) (16 significant bits), plus X = sum(hi + lo) per group.
//  * gemm_main_kernel tiles the output 128 x 128 per workgroup (4 waves of
//    64 x 64, v_mfma_f32_16x16x32_bf16).  For every group of 128 inputs it
//    stages the hi/lo activation tile and the group's code words through
//    registers into LDS, expanding each 2-bit code to its exact bf16 value
//    {0, 1, 2, 3} in LDS, runs the hi and lo MFMA chains into a per-group
//    fp32 accumulator, then folds the group's fp16 scale and bias in fp32:
//    y += s * acc + b * X.  Global loads of group g+1 are issued before the
//    MFMAs of group g.  Workgroups are mapped so that each XCD walks
//    contiguous output tiles in M-major order, keeping one activation row
//    tile resident in that XCD's L2 while the code tiles stream past it.
#include "tb_device.h"

namespace tb {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kBM = 128, kBN = 128, kBK = kGroup;  // tile and K step (one group)
constexpr int kLdsStride = kBK + 8;                  // bf16 elements per LDS row (padding)
constexpr int kXcds = 8;

static inline int64_t g_align256(int64_t v) { return (v + 255) & ~int64_t(255); }

struct GemmWs {
  int64_t hi_off, lo_off, xg_off, total;
};

static inline GemmWs gemm_ws_layout(int64_t M, int64_t K) {
  GemmWs w;
  w.hi_off = 0;
  w.lo_off = g_align256(M * K * 2);
  w.xg_off = w.lo_off + g_align256(M * K * 2);
  w.total = w.xg_off + g_align256(M * (K / kGroup) * 4);
  return w;
}

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// grid.x = M * nchunks.
template <int L, int CH, int DT>
__global__ __launch_bounds__(kThreads) void gemm_prep_kernel(const void* __restrict__ x,
                                                             const int8_t* __restrict__ signs,
                                                             int64_t K, int64_t nchunks,
                                                             uint16_t* __restrict__ xhi,
                                                             uint16_t* __restrict__ xlo,
                                                             float* __restrict__ xg) {
  __shared__ float buf[CH];
  const int tid = threadIdx.x;
  const int64_t m = blockIdx.x / nchunks;
  const int64_t chunk = blockIdx.x % nchunks;
  const int64_t k0 = chunk * CH;
  const int n = static_cast<int>(min<int64_t>(CH, K - k0));
  for (int i = tid; i < CH; i += kThreads) {
    float v = 0.f;
    if (i < n) {
      v = load_x<DT>(x, m * K + k0 + i);
      if constexpr (L > 0) v *= static_cast<float>(signs[k0 + i]);
    }
    buf[i] = v;
  }
  __syncthreads();
  float sc = 1.f;
  if constexpr (L > 0) {
    fwht_lds<L>(buf);
    sc = inv_sqrt_block<L>();
  }
  const int wave = tid >> 6, lane = tid & 63;
  const int ng = n / kGroup;
  const int64_t G = K / kGroup;
  for (int gl = wave; gl < ng; gl += kThreads / 64) {
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = gl * kGroup + 2 * lane + j;
      const float v = buf[i] * sc;
      const uint16_t h = float_to_bf16_rne(v);
      const float hf = bf16_bits_to_float(h);
      const uint16_t l = float_to_bf16_rne(v - hf);
      xhi[m * K + k0 + i] = h;
      xlo[m * K + k0 + i] = l;
      part += hf + bf16_bits_to_float(l);
    }
    const float tot = wave_sum_f(part);
    if (lane == 0) xg[m * G + k0 / kGroup + gl] = tot;
  }
}

// Exact bf16 bit patterns of the code values 0, 1, 2, 3.
__device__ __forceinline__ uint32_t code_bf16(uint32_t c) {
  return c == 0 ? 0u : (c == 1 ? 0x3F80u : (c == 2 ? 0x4000u : 0x4040u));
}

__device__ __forceinline__ v8bf as_v8bf(uint4 u) { return __builtin_bit_cast(v8bf, u); }

__global__ __launch_bounds__(kThreads) void gemm_main_kernel(
    const uint16_t* __restrict__ xhi, const uint16_t* __restrict__ xlo,
    const float* __restrict__ xg, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases,
    float* __restrict__ y, int64_t M, int64_t N, int64_t K, int64_t MT, int64_t NT,
    int64_t per_xcd) {
  __shared__ __attribute__((aligned(16))) uint16_t sAh[kBM * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t sAl[kBM * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t sB[kBN * kLdsStride];
  __shared__ float sS[kBN], sBi[kBN], sX[kBM];

  // XCD-aware tile order: workgroup w runs on XCD w % 8; XCD x owns the
  // contiguous M-major tile range [x * per_xcd, (x + 1) * per_xcd).
  const int64_t wg = blockIdx.x;
  const int64_t tile = (wg % kXcds) * per_xcd + wg / kXcds;
  if (tile >= MT * NT || wg / kXcds >= per_xcd) return;
  const int64_t m0 = (tile / NT) * kBM;
  const int64_t n0 = (tile % NT) * kBN;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 15, lq = lane >> 4;
  const int64_t G = K / kGroup, W = K / kCodesPerWord;

  // register staging of one group's global data
  uint4 rh[8], rl[8], rc;
  float rs = 0.f, rx = 0.f;
  auto gload = [&](int64_t g) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int u = tid + kThreads * i;  // 0..2047: row u/16, 8-element column u%16
      const int64_t m = m0 + (u >> 4);
      if (m < M) {
        const int64_t off = m * K + g * kBK + (u & 15) * 8;
        rh[i] = *reinterpret_cast<const uint4*>(xhi + off);
        rl[i] = *reinterpret_cast<const uint4*>(xlo + off);
      } else {
        rh[i] = make_uint4(0, 0, 0, 0);
        rl[i] = make_uint4(0, 0, 0, 0);
      }
    }
    {
      const int64_t n = n0 + (tid >> 1);
      rc = (n < N) ? *reinterpret_cast<const uint4*>(codes + n * W + g * 8 + (tid & 1) * 4)
                   : make_uint4(0, 0, 0, 0);
    }
    if (tid < kBN) {
      const int64_t n = n0 + tid;
      rs = (n < N) ? half_bits_to_float(scales[n * G + g]) : 0.f;
      const int64_t m = m0 + tid;
      rx = (m < M) ? xg[m * G + g] : 0.f;
    } else {
      const int64_t n = n0 + tid - kBN;
      rs = (n < N) ? half_bits_to_float(biases[n * G + g]) : 0.f;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int u = tid + kThreads * i;
      *reinterpret_cast<uint4*>(&sAh[(u >> 4) * kLdsStride + (u & 15) * 8]) = rh[i];
      *reinterpret_cast<uint4*>(&sAl[(u >> 4) * kLdsStride + (u & 15) * 8]) = rl[i];
    }
    // expand 4 code words (64 codes) of row tid/2 to exact bf16
    uint16_t* dst = &sB[(tid >> 1) * kLdsStride + (tid & 1) * 64];
    const uint32_t wv[4] = {rc.x, rc.y, rc.z, rc.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t o[8];
#pragma unroll
      for (int p = 0; p < 8; ++p)
        o[p] = code_bf16((wv[w] >> (4 * p)) & 3u) | (code_bf16((wv[w] >> (4 * p + 2)) & 3u) << 16);
      *reinterpret_cast<uint4*>(dst + w * 16) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4*>(dst + w * 16 + 8) = make_uint4(o[4], o[5], o[6], o[7]);
    }
    if (tid < kBN) {
      sS[tid] = rs;
      sX[tid] = rx;
    } else {
      sBi[tid - kBN] = rs;
    }
  };

  v4f yac[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) yac[a][b] = v4f{0.f, 0.f, 0.f, 0.f};

  gload(0);
  for (int64_t g = 0; g < G; ++g) {
    __syncthreads();  // previous group's LDS reads are done
    lstore();
    __syncthreads();
    if (g + 1 < G) gload(g + 1);
    v4f acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      const int kc = kk * 32 + lq * 8;
      uint4 ah[4], al[4], bb[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int r = wm * 64 + a * 16 + li;
        ah[a] = *reinterpret_cast<const uint4*>(&sAh[r * kLdsStride + kc]);
        al[a] = *reinterpret_cast<const uint4*>(&sAl[r * kLdsStride + kc]);
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int r = wn * 64 + b * 16 + li;
        bb[b] = *reinterpret_cast<const uint4*>(&sB[r * kLdsStride + kc]);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(ah[a]), as_v8bf(bb[b]), acc[a][b], 0, 0, 0);
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_v8bf(al[a]), as_v8bf(bb[b]), acc[a][b], 0, 0, 0);
        }
    }
    // per-group affine fold: lane holds D[4 lq + r][li] of tile (a, b)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int nl = wn * 64 + b * 16 + li;
      const float s = sS[nl], bi = sBi[nl];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float xv = sX[wm * 64 + a * 16 + 4 * lq + r];
          yac[a][b][r] += s * acc[a][b][r] + bi * xv;
        }
    }
  }

#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t n = n0 + wn * 64 + b * 16 + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 64 + a * 16 + 4 * lq + r;
        if (m < M && n < N) y[m * N + n] = yac[a][b][r];
      }
    }
}

template <int L, int CH>
static void launch_gemm_prep(const void* x, int dt, const int8_t* signs, int64_t M, int64_t K,
                             uint16_t* xhi, uint16_t* xlo, float* xg, hipStream_t st) {
  const int64_t nchunks = (K + CH - 1) / CH;
  const dim3 grid(static_cast<unsigned>(M * nchunks));
  if (dt == TB_F32)
    hipLaunchKernelGGL((gemm_prep_kernel<L, CH, TB_F32>), grid, dim3(kThreads), 0, st, x, signs, K,
                       nchunks, xhi, xlo, xg);
  else
    hipLaunchKernelGGL((gemm_prep_kernel<L, CH, TB_BF16>), grid, dim3(kThreads), 0, st, x, signs, K,
                       nchunks, xhi, xlo, xg);
}

static int gemm_ws_check(const void* workspace, size_t ws_bytes, int64_t M, int64_t K, const char* who) {
  const GemmWs lay = gemm_ws_layout(M, K);
  if (!workspace || ws_bytes < static_cast<size_t>(lay.total)) {
    set_error("%s: workspace of %zu bytes at %p, need %lld", who, ws_bytes, workspace,
              (long long)lay.total);
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
  const int64_t MT = (M + kBM - 1) / kBM, NT = (N + kBN - 1) / kBN;
  if ((MT * NT + kXcds - 1) / kXcds * kXcds > 0x7FFFFFFF) {
    set_error("%s: M x N too large for one launch", who);
    return TB_ERR_SHAPE;
  }
  return TB_OK;
}

static int gemm_run_checks(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                           const float* y, const char* who) {
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

static void gemm_prepare_launch(const void* x, int x_dtype, int64_t M, int64_t K, const int8_t* signs,
                                int block, void* workspace, hipStream_t st) {
  const GemmWs lay = gemm_ws_layout(M, K);
  char* ws = static_cast<char*>(workspace);
  uint16_t* xhi = reinterpret_cast<uint16_t*>(ws + lay.hi_off);
  uint16_t* xlo = reinterpret_cast<uint16_t*>(ws + lay.lo_off);
  float* xg = reinterpret_cast<float*>(ws + lay.xg_off);
  switch (block) {
    case 0: launch_gemm_prep<0, 512>(x, x_dtype, signs, M, K, xhi, xlo, xg, st); break;
    case 512: launch_gemm_prep<512, 512>(x, x_dtype, signs, M, K, xhi, xlo, xg, st); break;
    case 1024: launch_gemm_prep<1024, 1024>(x, x_dtype, signs, M, K, xhi, xlo, xg, st); break;
    case 2048: launch_gemm_prep<2048, 2048>(x, x_dtype, signs, M, K, xhi, xlo, xg, st); break;
    default: launch_gemm_prep<4096, 4096>(x, x_dtype, signs, M, K, xhi, xlo, xg, st); break;
  }
}

static void gemm_run_launch(const void* workspace, int64_t M, int64_t K, const uint32_t* codes,
                            const uint16_t* scales, const uint16_t* biases, int64_t N, float* y,
                            hipStream_t st) {
  const GemmWs lay = gemm_ws_layout(M, K);
  const char* ws = static_cast<const char*>(workspace);
  const uint16_t* xhi = reinterpret_cast<const uint16_t*>(ws + lay.hi_off);
  const uint16_t* xlo = reinterpret_cast<const uint16_t*>(ws + lay.lo_off);
  const float* xg = reinterpret_cast<const float*>(ws + lay.xg_off);
  const int64_t MT = (M + kBM - 1) / kBM, NT = (N + kBN - 1) / kBN;
  const int64_t per_xcd = (MT * NT + kXcds - 1) / kXcds;
  hipLaunchKernelGGL(gemm_main_kernel, dim3(static_cast<unsigned>(per_xcd * kXcds)), dim3(kThreads), 0,
                     st, xhi, xlo, xg, codes, scales, biases, y, M, N, K, MT, NT, per_xcd);
}

}  // namespace tb

using namespace tb;

extern "C" size_t tb_ternary_gemm_workspace_size(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || K % kGroup) return 0;
  return static_cast<size_t>(gemm_ws_layout(M, K).total);
}

extern "C" int tb_ternary_gemm_prepare(const void* x, int x_dtype, int64_t M, int64_t K,
                                       const int8_t* signs, int block, void* workspace,
                                       size_t ws_bytes, void* stream) {
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
                                   const uint32_t* codes, const uint16_t* scales,
                                   const uint16_t* biases, int64_t N, float* y, void* stream) {
  const char* who = "tb_ternary_gemm_run";
  TB_TRY(gemm_shape_checks(M, K, N, who));
  if (M == 0 || N == 0) return TB_OK;
  TB_TRY(gemm_run_checks(codes, scales, biases, y, who));
  TB_TRY(gemm_ws_check(workspace, ws_bytes, M, K, who));
  gemm_run_launch(workspace, M, K, codes, scales, biases, N, y, static_cast<hipStream_t>(stream));
  TB_LAUNCH_CHECK(who);
  return TB_OK;
}

extern "C" int tb_ternary_gemm(const void* x, int x_dtype, int64_t M, int64_t K,
                               const int8_t* signs, int block, const uint32_t* codes,
                               const uint16_t* scales, const uint16_t* biases, int64_t N, float* y,
                               void* workspace, size_t ws_bytes, void* stream) {
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
