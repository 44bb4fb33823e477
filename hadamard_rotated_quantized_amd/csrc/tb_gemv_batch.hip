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
//    chunks (every batch row; bf16 x and the signs land by direct-to-LDS
//    loads in the LDS rows the chunk's transform will write), then the first
//    code loads of their tiles, and transform the chunks on the matrix cores
//    (tb_xform.h) straight into the LDS operand image of the slice -- the
//    exact four-limb split and the group terms -- while the codes are in
//    flight.  Each of the 8 waves then streams one 16-row tile through a
//    ring of register slots of 8 groups: four 16-byte code loads (each row's
//    64 bytes of two groups as one run, regrouped by one lane swap per
//    dword pair), one 16-byte load for the 8 scales and one for the 8 biases
//    of a row.  A group is 2 v_mfma_i32_16x16x64_i8 per 4 batch rows: A row
//    4 b' + l holds limb l of batch row b', the 4 k-blocks hold 4 of the
//    group's 8 code words, so the accumulator of lane (lane group j, row c)
//    is the 4 limbs of batch row j (+4 for the second set) at output row c.
//    The limbs are recombined (limb pairs exactly in int32, the two halves
//    in one fp32 rounding) and the fp16 scale and bias applied per group; an
//    octet of groups is one branch-free block of MFMAs and fp32 arithmetic.
// 2. batch_reduce_kernel (more than one K slice): the slices' partial rows
//    summed in slice order, so results do not depend on scheduling.
#include <algorithm>

#include "tb_xform.h"

namespace tb {

// A chunk task's transform inputs (XformIn, tb_xform.h) brought in through a
// wave-owned LDS area of at least 3 KB: bf16 x (2 KB) and the signs (1 KB, at byte 2048) land by
// direct-to-LDS loads of 16 bytes per lane, three load instructions per chunk
// instead of eight register loads per lane (fp32 x still comes in registers,
// four 16-byte loads).  The caller waits for these loads (vmcnt) before
// xform_fetch, and may let the chunk's transform overwrite the area: every
// read of it is issued before the transform's first LDS write.
template <int L, int DT>
__device__ __forceinline__ void xform_stage(__amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rsg, int64_t e0, int k0,
                                            int lane, char* stage, XformIn<DT>& in) {
  typedef __attribute__((address_space(3))) void lds_void;
  if constexpr (DT == TB_F32) {
    const int base = xf_lane_base(lane);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int off = base + 32 * (q >> 1) + 16 * (q & 1);
      const v4u u = __builtin_amdgcn_raw_buffer_load_b128(rx, static_cast<int>((e0 + off) * 4), 0, 0);
      in.x[q][0] = u.x; in.x[q][1] = u.y; in.x[q][2] = u.z; in.x[q][3] = u.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(stage + 1024 * i), 16,
                                               static_cast<int>(e0 * 2) + 1024 * i + 16 * lane, 0, 0, 0);
  }
  if constexpr (L > 0)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsg, (lds_void*)(stage + 2048), 16, k0 + 16 * lane, 0, 0, 0);
}

template <int L, int DT>
__device__ __forceinline__ void xform_fetch(const char* stage, int lane, XformIn<DT>& in) {
  const int base = xf_lane_base(lane);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int off = base + 32 * (q >> 1) + 16 * (q & 1);
    if constexpr (DT != TB_F32) {
      const uint2 v = *reinterpret_cast<const uint2*>(stage + 2 * off);
      in.x[q][0] = v.x; in.x[q][1] = v.y;
    }
    if constexpr (L > 0) in.sg[q] = *reinterpret_cast<const uint32_t*>(stage + 2048 + off);
  }
}


constexpr int kBatWaves = 8;
constexpr int kBatThreads = 64 * kBatWaves;
constexpr int kBatTile = 16;                    // output rows per wave
constexpr int kBatRows = kBatTile * kBatWaves;  // output rows per work unit
constexpr int kBatArow = 144;                   // LDS bytes per (batch row, group, limb) operand row
constexpr int kBatRing = 2;                     // octets of groups in flight per wave (10 loads each)
constexpr int kBatMaxTasks = 4;                 // chunk transforms per wave
constexpr int64_t kBatLdsMax = 150 * 1024;
// s_waitcnt vmcnt(n) with the other counters left alone: n = the loads of
// the ring's first slot (4 code loads, scales, biases), issued after the
// staged chunk inputs
constexpr int kBatSlotLoads = 6;
constexpr int kBatWaitStaged = (kBatSlotLoads & 15) | ((kBatSlotLoads >> 4) << 14) | (0x7 << 4) | (0xF << 8);

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
// One ring slot: 8 consecutive groups (an octet) of the lane's row.  Code
// load m brings groups 2 m and 2 m + 1 of the 16 rows: lane group j reads 16
// bytes, half (j & 1) of group 2 m + (j >> 1), so each row's 64 bytes are
// one contiguous run; a lane swap (batch_words) then hands every lane group
// one word pair of each group.
struct BatchSlot {
  v4u w[4];
  uint4 s, b;  // the 8 fp16 scales / biases of (row c, octet), one 16-byte load each
};

// Code words of groups 2 m and 2 m + 1 from a slot's load m.  Before the
// swap lane group j holds words 4 (j & 1) .. + 3 of group 2 m + (j >> 1);
// v_permlane32_swap exchanges the upper lane half of dwords 0, 1 with the
// lower lane half of dwords 2, 3, after which lane group j holds, for both
// groups, word pair p = 2 (j & 1) + (j >> 1) (words 2 p, 2 p + 1).
__device__ __forceinline__ void batch_words(const v4u& w, uint2& g0, uint2& g1) {
  const auto sx = __builtin_amdgcn_permlane32_swap(w.x, w.z, false, false);
  const auto sy = __builtin_amdgcn_permlane32_swap(w.y, w.w, false, false);
  g0 = make_uint2(sx[0], sy[0]);
  g1 = make_uint2(sx[1], sy[1]);
}

template <int NS, int L, int DT>
__global__ __launch_bounds__(kBatThreads, 1) void batch_stream_kernel(
    const void* __restrict__ x, const int8_t* __restrict__ signs, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases, float* __restrict__ out, int B, int N,
    int K, int cps, int S) {
  extern __shared__ uint4 bat_lds_dyn[];
  char* const lds = reinterpret_cast<char*>(bat_lds_dyn);
  const int unit = blockIdx.x;
  // Workgroup w runs on XCD w % 8.  When the row blocks come in eights, all
  // S slices of a row block go to one XCD, so the cache lines of a row's
  // scales and biases that several slices share are fetched into one L2.
  const int rbn = static_cast<int>(gridDim.x) / S;
  int rb, sl;
  if ((rbn & 7) == 0) {
    const int i = unit >> 3;
    rb = (unit & 7) + 8 * (i / S);
    sl = i - (i / S) * S;
  } else {
    rb = unit / S;
    sl = unit - rb * S;
  }
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
    for (int m = 0; m < 4; ++m) {
      const int gl = 8 * o + 2 * m + (lg >> 1);
      const int oc = gl < ng ? c * RBy + (g0 + gl) * 32 + (lg & 1) * 16 : kOob;
      st.w[m] = __builtin_amdgcn_raw_buffer_load_b128(rc, oc, 0, 0);
    }
    const int os = 8 * o < ng ? (c * G + g0 + 8 * o) * 2 : kOob;
    const v4u us = __builtin_amdgcn_raw_buffer_load_b128(rs, os, 0, 0);
    const v4u ub = __builtin_amdgcn_raw_buffer_load_b128(rbi, os, 0, 0);
    st.s = make_uint4(us.x, us.y, us.z, us.w);
    st.b = make_uint4(ub.x, ub.y, ub.z, ub.w);
  };

  // 2. the slice's activation chunks: loads first (they complete before the
  //    code loads issued after them), then the transforms into LDS.  A
  //    task's x and signs are staged in the LDS rows its transform writes.
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
  auto task_rows = [&](int t) {  // LDS operand rows of task t's chunk
    const int b = t / ncs, j = t - b * ncs;
    return lds + b * bstride + j * (8 * kXfLimbs * kBatArow);
  };
#pragma unroll
  for (int r = 0; r < kBatMaxTasks; ++r) {
    const int t = wave + kBatWaves * r;
    if (t < ntask) {
      const int b = t / ncs, cg = (g0 >> 3) + (t - b * ncs);
      const auto rx = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(static_cast<const char*>(x) + static_cast<int64_t>(b) * K * ESZ), 0, K * ESZ, kRsrcWord3);
      xform_stage<L, DT>(rx, rsg, static_cast<int64_t>(cg) * 1024, cg * 1024, lane, task_rows(t), xin[r]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // the ring's loads stay behind the staging loads
  // Only the first slot is loaded ahead of the transforms; the others follow
  // them: fewer loads queued ahead of other waves' activation loads, and the
  // transforms and the barrier cover most of their latency.
  BatchSlot ring[kBatRing];
  load(0, ring[0]);
  __builtin_amdgcn_sched_barrier(0);
  // the staged x and signs have landed once at most the ring's loads remain
  __builtin_amdgcn_s_waitcnt(kBatWaitStaged);
#pragma unroll
  for (int r = 0; r < kBatMaxTasks; ++r) {
    const int t = wave + kBatWaves * r;
    if (t < ntask) {
      const int b = t / ncs, j = t - b * ncs;
      xform_fetch<L, DT>(task_rows(t), lane, xin[r]);
      xform_chunk<L, DT>(xin[r], 8 * j, lane, cf, cs, lds + b * bstride, lxf + b * gps, kBatArow);
    }
  }
#pragma unroll
  for (int k = 1; k < kBatRing; ++k) load(k, ring[k]);
  __syncthreads();
  if (nrows == 0) return;  // no barrier follows

  // 3. stream the tile's groups.  Every lane reads operand rows of real
  //    batch rows (sets past B read row B - 1 and their sums are dropped at
  //    the store), so each octet is one branch-free block of MFMAs and fp32
  //    arithmetic that the compiler can software-pipeline.
  float yacc[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) yacc[s] = 0.f;
  // lane (j, c) holds A row c = 4 b' + l (batch row b', limb l) of the k-block
  // of its code words: word pair wp of each group
  const int ab = c >> 2, al = c & 3;
  const char* arow[NS];
  const float2* trow[NS];
  const int wp = 2 * (lg & 1) + (lg >> 1);  // the word pair (k-block) of lane group lg
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    arow[s] = lds + min(4 * s + ab, B - 1) * bstride + al * kBatArow + 32 * wp;
    trow[s] = lxf + min(4 * s + lg, B - 1) * gps;  // group terms of batch row 4 s + j
  }
  const int nocts = (ng + 7) >> 3;
  for (int base = 0; base < nocts; base += kBatRing) {
#pragma unroll
    for (int k = 0; k < kBatRing; ++k) {
      const BatchSlot cur = ring[k];
      if (base + k + kBatRing < nocts) load(base + k + kBatRing, ring[k]);  // refill before computing
      const int o = base + k;
      if (o < nocts) {
        // groups past the slice have zero codes; the scales and biases read
        // for them belong to the next row and are cleared
        const int nv = ng - 8 * o;
        uint32_t sd[4] = {cur.s.x, cur.s.y, cur.s.z, cur.s.w};
        uint32_t bd[4] = {cur.b.x, cur.b.y, cur.b.z, cur.b.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t keep = (2 * q < nv ? 0xFFFFu : 0u) | (2 * q + 1 < nv ? 0xFFFF0000u : 0u);
          sd[q] &= keep;
          bd[q] &= keep;
        }
        float2 t[NS][8];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 tv = *reinterpret_cast<const float4*>(trow[s] + 8 * o + 2 * q);
            t[s][2 * q] = make_float2(tv.x, tv.y);
            t[s][2 * q + 1] = make_float2(tv.z, tv.w);
          }
        uint2 wd[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) batch_words(cur.w[m], wd[2 * m], wd[2 * m + 1]);
        // the octet is one chunk: its activation scale f (the .y of every
        // group term) multiplies the octet's scaled sums once
        float yo[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) yo[s] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int gl = 8 * o + j;
          const v4i bq0 = decode_word(wd[j].x), bq1 = decode_word(wd[j].y);
          const float sc = half_bits_to_float(static_cast<uint16_t>(sd[j >> 1] >> (16 * (j & 1))));
          const float bi = half_bits_to_float(static_cast<uint16_t>(bd[j >> 1] >> (16 * (j & 1))));
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            const char* ap = arow[s] + gl * (kXfLimbs * kBatArow);
            const v4u a0 = *reinterpret_cast<const v4u*>(ap);
            const v4u a1 = *reinterpret_cast<const v4u*>(ap + 16);
            v4i acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, a0), bq0, v4i{0, 0, 0, 0}, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, a1), bq1, acc, 0, 0, 0);
            // lane (j, c): limbs 0..3 of batch row 4 s + j at output row c.
            // |limb sum| <= 128 * 3 * 128 per group, so limb pairs combine
            // exactly in int32 and in fp32; one rounding joins the halves.
            const int lo = acc[0] + acc[1] * 256, hi = acc[2] + acc[3] * 256;
            const float v = fmaf(static_cast<float>(hi), 65536.f, static_cast<float>(lo));
            yo[s] = fmaf(v, sc, yo[s]);
            yacc[s] = fmaf(bi, t[s][j].x, yacc[s]);
          }
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) yacc[s] = fmaf(yo[s], t[s][0].y, yacc[s]);
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
