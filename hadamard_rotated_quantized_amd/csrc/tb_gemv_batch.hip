// Decode batches of 2 to 8 rows against one packed weight matrix
// [lpnh.cn/news/2438023, "text model loading" (fwht(x, block, signs), then
// the quantized matmul); kwkr.cn/news/564617, "ternary weights + folded
// Hadamard rotation" and "packing-format engineering"]:
//   y[b][n] = sum_g s[n][g] (sum_{k in g} c[n][k] xr[b][k]) + bias[n][g] X[b][g]
//
// The weights must stream from HBM once for all batch rows, and a decode
// layer is often narrow (N = 5120) but deep (K = 17408): 320 row tiles of 16
// cannot keep 256 CUs streaming, and the exact activation operand of 8 rows
// (4 base-256 limbs each, 557 KB at K = 17408) does not fit one CU's LDS.
// So the contraction is split along K as well:
//
// 1. batch_stream_kernel: one workgroup per (128-row block, K slice of whole
//    chunks).  Its waves first issue the loads of the slice's activation
//    chunks (every batch row), then the first code loads of their tiles, and
//    transform the chunks on the matrix cores (tb_xform.h) straight into the
//    LDS operand image of the slice -- the exact four-limb split and the
//    group terms -- while the codes are in flight.  Each of the 8 waves then
//    streams one 16-row tile through a ring of register slots of 8 groups
//    (8-byte code loads, one 16-byte load for the 8 scales and one for the 8
//    biases of a row).  A group is 2 v_mfma_i32_16x16x64_i8 per 4 batch rows:
//    A row 4 b' + l holds limb l of batch row b', the 4 k-blocks hold 4 of
//    the group's 8 code words, so the accumulator of lane (lane group j, row
//    c) is the 4 limbs of batch row j (+4 for the second set) at output row
//    c.  The limbs are recombined in fp32 and the fp16 scale and bias applied
//    per group.
// 2. batch_reduce_kernel (more than one K slice): the slices' partial rows
//    summed in slice order, so results do not depend on scheduling.
#include <algorithm>

#include "tb_xform.h"

namespace tb {

constexpr int kBatWaves = 8;
constexpr int kBatThreads = 64 * kBatWaves;
constexpr int kBatTile = 16;                    // output rows per wave
constexpr int kBatRows = kBatTile * kBatWaves;  // output rows per work unit
constexpr int kBatArow = 144;                   // LDS bytes per (batch row, group, limb) operand row
constexpr int kBatRing = 2;                     // octets of groups in flight per wave (10 loads each)
constexpr int kBatMaxTasks = 4;                 // chunk transforms per wave
constexpr int64_t kBatLdsMax = 150 * 1024;

// LDS stride between batch rows: 16 mod 32 dwords, so that the two batch rows
// read by lanes 0-3 and 4-7 of an A-operand read land on disjoint banks.
__host__ __device__ inline int batch_bstride(int gps) { return gps * kXfLimbs * kBatArow + ((gps & 1) ? 0 : 64); }
__host__ __device__ inline int64_t batch_lds_bytes(int B, int gps) {
  return static_cast<int64_t>(B) * batch_bstride(gps) + static_cast<int64_t>(B) * gps * 8;
}

struct BatchPlan {
  int nch, cps, S, rbn, grid;
  int64_t lds;
  bool ok;
};

// Work units: ceil(N / 128) row blocks x S slices of cps chunks, about one
// per CU; a slice's operand rows must fit the LDS.
static BatchPlan batch_plan(int64_t B, int64_t K, int64_t N, int cus) {
  BatchPlan p{};
  p.nch = static_cast<int>((K + 1023) / 1024);
  p.rbn = static_cast<int>((N + kBatRows - 1) / kBatRows);
  int cps_max = 0;
  // a slice's chunks are transformed by the 8 waves, kBatMaxTasks each at most
  while (batch_lds_bytes(static_cast<int>(B), 8 * (cps_max + 1)) <= kBatLdsMax &&
         B * (cps_max + 1) <= kBatWaves * kBatMaxTasks)
    ++cps_max;
  const int target = std::max(1, (cus + p.rbn / 2) / p.rbn);
  p.cps = std::min(std::max(1, (p.nch + target - 1) / target), std::max(cps_max, 1));
  p.S = (p.nch + p.cps - 1) / p.cps;
  p.lds = batch_lds_bytes(static_cast<int>(B), 8 * p.cps);
  p.ok = cps_max >= 1 && static_cast<int64_t>(p.rbn) * p.S < (int64_t(1) << 31);
  p.grid = p.rbn * p.S;
  return p;
}

static inline int64_t bat_align256(int64_t v) { return (v + 255) & ~int64_t(255); }
// workspace: the slices' partial rows (none for a single slice)
static int64_t batch_ws_bytes(int64_t B, int64_t N, const BatchPlan& p) {
  return p.S > 1 ? bat_align256(static_cast<int64_t>(p.S) * B * N * 4) : 0;
}

// ---------------------------------------------------------------------------
// 1. transform + stream: one workgroup per (row block, K slice)
// ---------------------------------------------------------------------------
// One ring slot: 8 consecutive groups (an octet) of the lane's row
struct BatchSlot {
  uint2 w[8];  // code words 2 j and 2 j + 1 of (row c, group) for lane group j
  uint4 s, b;  // the 8 fp16 scales / biases of (row c, octet), one 16-byte load each
};

template <int NS, int L, int DT>
__global__ __launch_bounds__(kBatThreads, 1) void batch_stream_kernel(
    const void* __restrict__ x, const int8_t* __restrict__ signs, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases, float* __restrict__ out, int B, int N,
    int K, int cps, int S) {
  extern __shared__ uint4 bat_lds_dyn[];
  char* const lds = reinterpret_cast<char*>(bat_lds_dyn);
  const int unit = blockIdx.x;
  const int rb = unit / S, sl = unit - rb * S;
  const int G = K / kGroup, RBy = K / 4;  // groups, code bytes per weight row
  const int gps = 8 * cps;
  const int g0 = sl * gps;
  const int ng = min(G, g0 + gps) - g0;  // groups of this slice (>= 1)
  const int bstride = batch_bstride(gps);
  float2* const lxf = reinterpret_cast<float2*>(lds + static_cast<int64_t>(B) * bstride);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lg = lane >> 4, c = lane & 15;

  // 1. this wave's tile: rows trow0 .. trow0 + 15; its first code loads
  // (wave-uniform values, kept in scalar registers for the buffer resources)
  const int trow0 = __builtin_amdgcn_readfirstlane(rb * kBatRows + kBatTile * wave);
  const int base_row = __builtin_amdgcn_readfirstlane(min(trow0, N));
  const int nrows = __builtin_amdgcn_readfirstlane(max(0, min(kBatTile, N - trow0)));
  const auto rc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(codes + static_cast<int64_t>(base_row) * (K / 16)),
                                                    0, nrows * RBy, kRsrcWord3);
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales + static_cast<int64_t>(base_row) * G), 0,
                                                    nrows * G * 2, kRsrcWord3);
  const auto rbi = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(biases + static_cast<int64_t>(base_row) * G), 0,
                                                     nrows * G * 2, kRsrcWord3);
  // a slot past the slice loads nothing useful: its offsets lie beyond every
  // buffer and read as zero, so every slot is refilled in one static order.
  // The scale and bias rows are read 8 groups at a time (K % 256 == 0 keeps
  // those 16-byte loads dword aligned).
  auto load = [&](int o, BatchSlot& st) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int gl = 8 * o + j;
      const int oc = gl < ng ? c * RBy + (g0 + gl) * 32 + lg * 8 : kOob;
      const v2u w = __builtin_amdgcn_raw_buffer_load_b64(rc, oc, 0, 0);
      st.w[j] = make_uint2(w.x, w.y);
    }
    const int os = 8 * o < ng ? (c * G + g0 + 8 * o) * 2 : kOob;
    const v4u us = __builtin_amdgcn_raw_buffer_load_b128(rs, os, 0, 0);
    const v4u ub = __builtin_amdgcn_raw_buffer_load_b128(rbi, os, 0, 0);
    st.s = make_uint4(us.x, us.y, us.z, us.w);
    st.b = make_uint4(ub.x, ub.y, ub.z, ub.w);
  };

  // 2. the slice's activation chunks: loads first (they complete before the
  //    code loads issued after them), then the transforms into LDS
  const int ncs = (ng + 7) >> 3;  // chunks of this slice
  const int ntask = B * ncs;      // <= 8 waves x kBatMaxTasks (plan)
  constexpr int ESZ = DT == TB_F32 ? 4 : 2;
  const auto rsg = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(signs), 0, L > 0 ? K : 0, kRsrcWord3);
  // the transform's lane constants are loaded first: the waits for them
  // then do not cover the code loads issued later
  const v4u* cst = reinterpret_cast<const v4u*>(&kXformConst.w[xf_mode<L>()][0][lane][0]);
  const v4u* cst2 = reinterpret_cast<const v4u*>(&kXformConst.w[xf_mode<L>()][1][lane][0]);
  const v4u cf[2] = {cst[0], cst[1]};
  const v4u cs[2] = {cst2[0], cst2[1]};
  XformIn<DT> xin[kBatMaxTasks];
#pragma unroll
  for (int r = 0; r < kBatMaxTasks; ++r) {
    const int t = wave + kBatWaves * r;
    if (t < ntask) {
      const int b = t / ncs, cg = (g0 >> 3) + (t - b * ncs);
      const auto rx = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(static_cast<const char*>(x) + static_cast<int64_t>(b) * K * ESZ), 0, K * ESZ, kRsrcWord3);
      xform_issue<L, DT>(rx, rsg, static_cast<int64_t>(cg) * 1024, cg * 1024, lane, xin[r]);
    }
  }
  BatchSlot ring[kBatRing];
#pragma unroll
  for (int k = 0; k < kBatRing; ++k) load(k, ring[k]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < kBatMaxTasks; ++r) {
    const int t = wave + kBatWaves * r;
    if (t < ntask) {
      const int b = t / ncs, j = t - b * ncs;
      xform_chunk<L, DT>(xin[r], 8 * j, lane, cf, cs, lds + b * bstride, lxf + b * gps, kBatArow);
    }
  }
  __syncthreads();
  if (nrows == 0) return;  // no barrier follows

  // 3. stream the tile's groups
  float yacc[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) yacc[s] = 0.f;
  // lane (j, c) holds A row c = 4 b' + l (batch row b', limb l) of k-block j
  const int ab = c >> 2, al = c & 3;
  auto group = [&](int gl, uint2 w, uint32_t sdw, uint32_t bdw, int hi) {
    const v4i bq0 = decode_word(w.x), bq1 = decode_word(w.y);
    const float sc = half_bits_to_float(static_cast<uint16_t>(sdw >> (16 * hi)));
    const float bi = half_bits_to_float(static_cast<uint16_t>(bdw >> (16 * hi)));
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      v4u a0 = {0u, 0u, 0u, 0u}, a1 = {0u, 0u, 0u, 0u};
      if (4 * s + ab < B) {
        const char* ap = lds + (4 * s + ab) * bstride + (gl * kXfLimbs + al) * kBatArow + 2 * lg * 16;
        a0 = *reinterpret_cast<const v4u*>(ap);
        a1 = *reinterpret_cast<const v4u*>(ap + 16);
      }
      v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, a0), bq0, v4i{0, 0, 0, 0}, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, a1), bq1, acc, 0, 0, 0);
      // lane (j, c): limbs 0..3 of batch row 4 s + j at output row c
      const int bo = 4 * s + lg;
      if (bo < B) {
        const float2 t = lxf[bo * gps + gl];
        const float v = static_cast<float>(acc[3]) * 16777216.f + static_cast<float>(acc[2]) * 65536.f +
                        static_cast<float>(acc[1]) * 256.f + static_cast<float>(acc[0]);
        yacc[s] += sc * (v * t.y) + bi * t.x;
      }
    }
  };
  const int nocts = (ng + 7) >> 3;
  for (int base = 0; base < nocts; base += kBatRing) {
#pragma unroll
    for (int k = 0; k < kBatRing; ++k) {
      const BatchSlot cur = ring[k];
      load(base + k + kBatRing, ring[k]);  // refill the slot before computing on its data
      const int o = base + k;
      if (o < nocts) {
        const uint32_t sd[4] = {cur.s.x, cur.s.y, cur.s.z, cur.s.w};
        const uint32_t bd[4] = {cur.b.x, cur.b.y, cur.b.z, cur.b.w};
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (8 * o + j < ng) group(8 * o + j, cur.w[j], sd[j >> 1], bd[j >> 1], j & 1);
      }
    }
  }

  // 4. the tile's rows: partial sums of this slice, or y itself
  if (c < nrows) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int bo = 4 * s + lg;
      if (bo < B) {
        const int64_t n = trow0 + c;
        float* dst = S > 1 ? out + (static_cast<int64_t>(sl) * B + bo) * N + n : out + static_cast<int64_t>(bo) * N + n;
        *dst = yacc[s];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. the slices' partial rows, summed in slice order
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void batch_reduce_kernel(const float* __restrict__ part, float* __restrict__ y,
                                                           int64_t BN, int S) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= BN) return;
  // eight slices' loads in flight, added in slice order
  float s = 0.f;
  for (int k0 = 0; k0 < S; k0 += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = k0 + j < S ? part[static_cast<int64_t>(k0 + j) * BN + i] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += v[j];
  }
  y[i] = s;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
bool gemv_batch_eligible(int64_t B, int64_t K, int64_t N, int block) {
  if (B < 2 || B > TB_GEMV_MAX_BATCH || !(block == 0 || block == 512 || block == 1024) || K % 256) return false;
  if (N <= 0 || N > (int64_t(1) << 30) || K > (int64_t(1) << 24)) return false;
  return batch_plan(B, K, N, device_cus()).ok;
}

size_t gemv_batch_workspace(int64_t B, int64_t K, int64_t N) {
  const BatchPlan p = batch_plan(B, K, N, device_cus());
  return static_cast<size_t>(batch_ws_bytes(B, N, p));
}

template <int NS, int L, int DT>
static void batch_stream_launch(const BatchPlan& p, const void* x, const int8_t* signs, const uint32_t* codes,
                                const uint16_t* scales, const uint16_t* biases, float* out, int B, int N, int K,
                                hipStream_t st) {
  auto kern = batch_stream_kernel<NS, L, DT>;
  static std::atomic<uint64_t> lds_set{0};
  lds_limit_once(reinterpret_cast<const void*>(kern), static_cast<int>(kBatLdsMax), lds_set);
  hipLaunchKernelGGL(kern, dim3(p.grid), dim3(kBatThreads), static_cast<size_t>(p.lds), st, x, signs, codes, scales,
                     biases, out, B, N, K, p.cps, p.S);
}

template <int NS, int L>
static void batch_launch_dt(int dt, const BatchPlan& p, const void* x, const int8_t* signs, const uint32_t* codes,
                            const uint16_t* scales, const uint16_t* biases, float* out, int B, int N, int K,
                            hipStream_t st) {
  if (dt == TB_F32) batch_stream_launch<NS, L, TB_F32>(p, x, signs, codes, scales, biases, out, B, N, K, st);
  else batch_stream_launch<NS, L, TB_BF16>(p, x, signs, codes, scales, biases, out, B, N, K, st);
}

template <int NS>
static void batch_launch_l(int block, int dt, const BatchPlan& p, const void* x, const int8_t* signs,
                           const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, float* out, int B,
                           int N, int K, hipStream_t st) {
  if (block == 0) batch_launch_dt<NS, 0>(dt, p, x, signs, codes, scales, biases, out, B, N, K, st);
  else if (block == 512) batch_launch_dt<NS, 512>(dt, p, x, signs, codes, scales, biases, out, B, N, K, st);
  else batch_launch_dt<NS, 1024>(dt, p, x, signs, codes, scales, biases, out, B, N, K, st);
}

void gemv_batch_launch(const void* x, int x_dtype, int64_t B, int64_t K, const int8_t* signs, int block,
                       const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t N, float* y,
                       void* workspace, hipStream_t st) {
  const BatchPlan p = batch_plan(B, K, N, device_cus());
  const int b = static_cast<int>(B), k = static_cast<int>(K), n = static_cast<int>(N);
  float* out = p.S > 1 ? static_cast<float*>(workspace) : y;
  if (b <= 4) batch_launch_l<1>(block, x_dtype, p, x, signs, codes, scales, biases, out, b, n, k, st);
  else batch_launch_l<2>(block, x_dtype, p, x, signs, codes, scales, biases, out, b, n, k, st);
  if (p.S > 1) {
    const int64_t BN = B * N;
    hipLaunchKernelGGL(batch_reduce_kernel, dim3(static_cast<unsigned>((BN + 255) / 256)), dim3(256), 0, st, out, y,
                       BN, p.S);
  }
}

}  // namespace tb
