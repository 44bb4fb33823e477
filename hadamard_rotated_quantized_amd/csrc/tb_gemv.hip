// tb_ternary_gemv: the Packed linear for decode batches (B <= 8).
//
// What is computed [lpnh.cn/news/2438023, "text model loading";
// kwkr.cn/news/564617, "ternary weights + folded Hadamard rotation" and
// "packing-format engineering"]:
//
//   xr = H (signs .* x) / sqrt(L) per block of L inputs      (rotation)
//   y[b][n] = sum_g s[n][g] * sum_{k in g} c[n][k] xr[b][k]
//                 + b[n][g] * sum_{k in g} xr[b][k]           (affine 2-bit)
//
// which is sum_k (s c + b) xr, i.e. W~ xr, regrouped per 128-weight group.
//
// Design for gfx950 (the weight stream is the cost: 9/32 byte per weight).
// tb_ternary_gemv picks, in order: the K-split batch kernel of
// tb_gemv_batch.hip (batches 2..8), the band kernel of tb_gemv_band.hip
// (batch 1), the single-launch kernel of tb_gemv_fused.hip (a workgroup can
// afford to transform the whole input); otherwise, and always for the
// prepare/run pair, two kernels:
//
// 1. gemv_prep_kernel: one wave per 1024 inputs of one batch row.  Lane l
//    holds inputs 16 l .. 16 l + 15 of the chunk in registers: the transform
//    runs as 4 in-lane butterfly stages and 6 cross-lane stages (DPP and
//    permlane exchanges), with no LDS and no barrier.  The fp32 result is then split exactly into
//    integers: per group of 128 inputs (8 lanes), xr ~= f * q with f = 2^E
//    chosen so |q| <= 2^22 (rounding error below 2^-22 of the group's
//    largest |xr|), and q = h*2^16 + m*2^8 + l with balanced digits h, m, l
//    in [-128, 127].  A lane owns the 16 inputs that meet one 16-code weight
//    word, so it writes its digits ("limbs") directly in the byte order the
//    matmul's MFMA operand needs (three 16-byte stores), and lane 8j writes
//    f and f * sum(q) of its group.
//
// 2. gemv_main_kernel: one workgroup per tile of M output rows (M = 16 for
//    batch 1 with v_mfma_i32_16x16x64_i8, M = 32 for batches 2..8 with
//    v_mfma_i32_32x32x32_i8, which serves 4 batch rows per instruction).
//    The workgroup copies the prepared limbs of its K window into LDS once;
//    its waves split K in spans of GPS = 64 / M groups, one group per lane
//    group of the MFMA.  Lane (lg, c) streams the 8 code words (32 bytes) of
//    row c, group GPS*s + lg with two 128-bit buffer loads, so a row
//    contributes 64 or 128 contiguous bytes per span.  A word becomes the
//    int8 B operand with 7 integer ops: (w >> 2i) & 0x03030303, i = 0..3,
//    gives codes {i, i+4, i+8, i+12} as bytes 0..3 of dword i -- the codes are
//    never expanded to fp16/fp32.  The A operand's rows are (batch j, group
//    lg, limb r); a row is non-zero only in the K range its group's lane
//    group fills, so one MFMA keeps the groups of a span apart.  After the
//    group's 8 words, lane (lg, c) holds the exact int32 limb sums of its
//    (row, group) and applies the fp16 scale and bias in fp32:
//        y += s * f * (S_h 2^16 + S_m 2^8 + S_l) + b * f * sum(q).
//    Integer accumulation is exact, so the only roundings are the limb split
//    and the fp32 sums of per-group terms.  Loads of the next P spans stay in
//    flight while a span computes; the lane groups and waves are reduced at
//    the end and y is written once (no atomics).
#include <algorithm>

#include "tb_gemv.h"

namespace tb {

static inline int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

struct GemvWs {
  int64_t aops_off, xg_off, total;
};

// Workspace: limbs [B][Gp][3][8] x 16 B (groups past K zero-filled), then
// (f * sum q, f) as float2 [B][G].
static inline GemvWs gemv_ws_layout(int64_t B, int64_t K) {
  const int64_t G = K / kGroup;
  GemvWs w;
  w.aops_off = 0;
  w.xg_off = align256(B * padded_groups(K) * kAopsGroupBytes);
  w.total = w.xg_off + align256(B * G * (int64_t)sizeof(float2));
  return w;
}

// Load 16 consecutive activations (16-element aligned) as fp32.
template <int DT>
__device__ __forceinline__ void load16(const void* x, int64_t i0, float v[16]) {
  if constexpr (DT == TB_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + i0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 f = p[j];
      v[4 * j] = f.x; v[4 * j + 1] = f.y; v[4 * j + 2] = f.z; v[4 * j + 3] = f.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + i0);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint4 u = p[j];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * j + 2 * e] = __uint_as_float(w[e] << 16);
        v[8 * j + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    }
  }
}

// One wave per CH-input chunk of one batch row (CH = max(L, 1024); block 0
// uses 1024-input chunks, the last one possibly partial in whole words).
// Lane l holds inputs 1024 u + 16 l + r (u < CH / 1024, r < 16).
template <int L, int DT>
__global__ __launch_bounds__(kThreads) void gemv_prep_kernel(const void* __restrict__ x,
                                                             const int8_t* __restrict__ signs,
                                                             int64_t B, int64_t K, int64_t nchunks,
                                                             int64_t Gp, uint4* __restrict__ aops,
                                                             float2* __restrict__ xg) {
  constexpr int CH = L > 1024 ? L : 1024;
  constexpr int U = CH / 1024;
  const int64_t G = K / kGroup;
  // zero the limbs of the padding groups G .. Gp-1 of every batch row
  if (blockIdx.x == 0) {
    const int64_t npad = (Gp - G) * kLimbs * kWordsPerGroup;
    for (int64_t i = threadIdx.x; i < B * npad; i += kThreads)
      aops[((i / npad) * Gp + G) * kLimbs * kWordsPerGroup + i % npad] = make_uint4(0, 0, 0, 0);
  }
  const int lane = threadIdx.x & 63;
  const int64_t ci = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (ci >= B * nchunks) return;  // whole wave leaves; the kernel has no barrier
  const int64_t b = ci / nchunks;
  const int64_t k0 = (ci % nchunks) * CH;

  float v[U][16];
  bool ok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t kk = k0 + 1024 * u + 16 * lane;
    ok[u] = kk < K;
    if (ok[u]) {
      load16<DT>(x, b * K + kk, v[u]);
      if constexpr (L > 0) {
        const uint4 sg = *reinterpret_cast<const uint4*>(signs + kk);
        const uint32_t sw[4] = {sg.x, sg.y, sg.z, sg.w};
#pragma unroll
        for (int r = 0; r < 16; ++r)
          v[u][r] *= static_cast<float>(static_cast<int8_t>((sw[r >> 2] >> (8 * (r & 3))) & 0xFFu));
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) v[u][r] = 0.f;
    }
  }

  float sc = 1.f;
  if constexpr (L > 0) {
    // index bits 0-9 of a 1024 sub-chunk: in-lane and lane bits; bits 10+
    // of a larger block: u
#pragma unroll
    for (int u = 0; u < U; ++u) fwht_lane16<(L == 512) ? 5 : 6>(v[u], lane);
#pragma unroll
    for (int hu = 1; hu < U; hu <<= 1)
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (!(u & hu))
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float a0 = v[u][r], a1 = v[u + hu][r];
            v[u][r] = a0 + a1;
            v[u + hu][r] = a0 - a1;
          }
    sc = inv_sqrt_block<L>();
  }

#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int r = 0; r < 16; ++r) v[u][r] *= sc;
    uint4 limb[kLimbs];
    float2 xf;
    split_limbs(v[u], lane, limb, xf);
    if (!ok[u]) continue;
    const int64_t g = (k0 + 1024 * u) / kGroup + (lane >> 3);
    const int t = lane & 7;
    if (t == 0) xg[b * G + g] = xf;
#pragma unroll
    for (int l = 0; l < kLimbs; ++l) aops[((b * Gp + g) * kLimbs + l) * kWordsPerGroup + t] = limb[l];
  }
}

// One module of a (possibly multi-module) matmul launch.
struct ModDesc {
  const uint32_t* codes;
  const uint16_t* scales;
  const uint16_t* biases;
  const uint4* aops;   // prepared limbs [NB][Gp][3][8] x 16 B
  const float2* xg;    // (f * sum q, f) [NB][G]
  float* y;            // [NB][N]
  int N, K, Gp, tile0;  // tile0: first global tile index of this module
};

constexpr int kMaxModules = 16;

struct MultiArgs {
  int count;        // modules in this launch
  int total_tiles;  // sum of the modules' tiles
  ModDesc m[kMaxModules];
};

// What one lane streams per span: 8 code words, the group's fp16 scale and
// bias (bits, converted at use so the load does not wait), the batch rows'
// (f * sum q, f), and -- when the limbs do not fit in LDS -- the A operand.
template <int NB, int NBC, bool AG>
struct Span {
  uint4 w0, w1;
  uint16_t s, bias;
  float2 xf[NB];
  v4i a[AG ? NBC : 1][AG ? kWordsPerGroup : 1];
};

__host__ __device__ constexpr int64_t lds_limb_bytes(int nb, int64_t gp) {
  return (int64_t)nb * gp * kLimbs * kLdsRow * 16;
}

// Persistent matmul kernel.  A workgroup has 4 waves; WPT waves share one
// tile of M rows (each taking every WPT-th span of K), so a "tile group" is
// 4 / WPT consecutive tiles.  Workgroup w handles global tile groups w,
// w + grid, ... (each module's tiles are padded to whole groups, so a group
// never straddles two modules).  Each wave keeps its next P (group, span)
// items in flight in a ring of registers, across tile and module
// boundaries; the limbs of the current module sit in LDS.
template <int NB, int M, int WPT, int P, bool AG>
__global__ __launch_bounds__(256) void gemv_main_kernel(const MultiArgs args) {
  using MF = Mfma<M>;
  constexpr int GPS = MF::GPS, BPI = MF::BPI;
  constexpr int NBC = (NB + BPI - 1) / BPI;  // MFMA chains per span
  constexpr int TG = 4 / WPT;                // tiles per group
  using SpanT = Span<NB, NBC, AG>;
  // LDS: 8 zero uint4 (read by lanes whose A operand is zero), then limbs.
  extern __shared__ uint4 lds_dyn[];
  uint4* const lds_zero = lds_dyn;
  uint4* const lds_a = lds_dyn + kWordsPerGroup;
  __shared__ float red[WPT > 1 ? 4 : 1][NB][M];

  const int tid = threadIdx.x;
  // wave index in a scalar register: all loop control below is uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tslot = wave / WPT, kpart = wave % WPT;
  const int lane = tid & 63;
  const int lg = lane / M, c = lane % M;
  // A-operand role of this lane: A row c = (batch jb, group alg, limb ar) is
  // non-zero only in lane group alg == lg, for limbs 0..2.
  const int ar = c & 3;
  const int alg = (c >> 2) & (GPS - 1);
  const int ajb = c / (4 * GPS);
  const bool a_lane = (alg == lg) && (ar < kLimbs);

  const int grid = gridDim.x;
  const int total = args.total_tiles;  // total tile groups of the launch
  const int nmod = args.count;

  // --- prefetch cursor over this wave's (group, span) items --------------
  struct Cursor {
    int q, j, m, cnt, G, W, Gp;
    __amdgpu_buffer_rsrc_t rc, rs, rb, rx, ra;
  };
  auto enter_group = [&](Cursor& cu) {
    while (cu.m + 1 < nmod && cu.q >= args.m[cu.m + 1].tile0) ++cu.m;
    const ModDesc& d = args.m[cu.m];
    const int t = (cu.q - d.tile0) * TG + tslot;  // tile within the module
    const int row0 = t * M;
    const bool valid = cu.q < total && row0 < d.N;
    const int S = d.Gp / GPS;
    cu.G = d.K / kGroup;
    cu.W = d.K / kCodesPerWord;
    cu.cnt = valid ? (S - kpart + WPT - 1) / WPT : 0;
    const int nrows = valid ? min(M, d.N - row0) : 0;
    cu.rc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(d.codes + (int64_t)row0 * cu.W), 0,
                                              nrows * cu.W * 4, kRsrcWord3);
    cu.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(d.scales + (int64_t)row0 * cu.G), 0,
                                              nrows * cu.G * 2, kRsrcWord3);
    cu.rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(d.biases + (int64_t)row0 * cu.G), 0,
                                              nrows * cu.G * 2, kRsrcWord3);
    cu.rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<float2*>(d.xg), 0, valid ? NB * cu.G * 8 : 0,
                                              kRsrcWord3);
    cu.Gp = d.Gp;
    if constexpr (AG)
      cu.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(d.aops), 0,
                                                valid ? NB * d.Gp * (int)kAopsGroupBytes : 0, kRsrcWord3);
  };
  auto advance = [&](Cursor& cu) {
    ++cu.j;
    while (cu.j >= cu.cnt && cu.q < total) {
      cu.q += grid;
      cu.j = 0;
      enter_group(cu);
    }
  };
  auto load_item = [&](const Cursor& cu, SpanT& L) {
    const int g = (kpart + cu.j * WPT) * GPS + lg;
    // an item past the end, a row past N or a group past K reads nothing:
    // buffer loads at an offset past the buffer's size return zero
    const bool gin = g < cu.G;
    const int cw = gin ? c * cu.W * 4 + g * (kWordsPerGroup * 4) : kOob;
    const v4u w0 = __builtin_amdgcn_raw_buffer_load_b128(cu.rc, cw, 0, 0);
    const v4u w1 = __builtin_amdgcn_raw_buffer_load_b128(cu.rc, cw + 16, 0, 0);
    L.w0 = make_uint4(w0.x, w0.y, w0.z, w0.w);
    L.w1 = make_uint4(w1.x, w1.y, w1.z, w1.w);
    const int so = gin ? (c * cu.G + g) * 2 : kOob;
    L.s = __builtin_amdgcn_raw_buffer_load_b16(cu.rs, so, 0, 0);
    L.bias = __builtin_amdgcn_raw_buffer_load_b16(cu.rb, so, 0, 0);
#pragma unroll
    for (int bq = 0; bq < NB; ++bq) {
      const v2u u = __builtin_amdgcn_raw_buffer_load_b64(cu.rx, gin ? (bq * cu.G + g) * 8 : kOob, 0, 0);
      L.xf[bq] = make_float2(__uint_as_float(u.x), __uint_as_float(u.y));
    }
    if constexpr (AG) {
      const int ga = (kpart + cu.j * WPT) * GPS + alg;
#pragma unroll
      for (int bc = 0; bc < NBC; ++bc) {
        const int bq = bc * BPI + ajb;
        const int ao = (a_lane && bq < NB) ? ((bq * cu.Gp + ga) * kLimbs + ar) * kWordsPerGroup * 16 : kOob;
#pragma unroll
        for (int t = 0; t < kWordsPerGroup; ++t) {
          const v4u u = __builtin_amdgcn_raw_buffer_load_b128(cu.ra, ao + 16 * t, 0, 0);
          L.a[bc][t] = v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
        }
      }
    }
  };

  if (tid < kWordsPerGroup) lds_zero[tid] = make_uint4(0, 0, 0, 0);

  SpanT ring[P];
  Cursor pc;
  pc.q = blockIdx.x;
  pc.j = 0;
  pc.m = 0;
  enter_group(pc);
  if (pc.cnt == 0) advance(pc);
#pragma unroll
  for (int i = 0; i < P; ++i) {
    load_item(pc, ring[i]);
    advance(pc);
  }

  float yacc[NB];
  int cur_gp = 0;
  // consume the item in ring slot SL (span s), then refill the slot
  auto consume = [&](auto slot_tag, int s) {
    constexpr int SL = decltype(slot_tag)::value;
    SpanT& cur = ring[SL];
    v4i bop[kWordsPerGroup];
    bop[0] = decode_word(cur.w0.x);
    bop[1] = decode_word(cur.w0.y);
    bop[2] = decode_word(cur.w0.z);
    bop[3] = decode_word(cur.w0.w);
    bop[4] = decode_word(cur.w1.x);
    bop[5] = decode_word(cur.w1.y);
    bop[6] = decode_word(cur.w1.z);
    bop[7] = decode_word(cur.w1.w);
#pragma unroll
    for (int bc = 0; bc < NBC; ++bc) {
      v4i av[kWordsPerGroup];
      if constexpr (AG) {
#pragma unroll
        for (int t = 0; t < kWordsPerGroup; ++t) av[t] = cur.a[bc][t];
      } else {
        const int bq_a = bc * BPI + ajb;
        const int ga = s * GPS + alg;
        const uint4* ap =
            (a_lane && bq_a < NB) ? lds_a + ((bq_a * cur_gp + ga) * kLimbs + ar) * kLdsRow : lds_zero;
#pragma unroll
        for (int t = 0; t < kWordsPerGroup; ++t) {
          const uint4 u = ap[t];
          av[t] = v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
        }
      }
      typename MF::acc_t acc = {};
#pragma unroll
      for (int t = 0; t < kWordsPerGroup; ++t) acc = MF::mac(av[t], bop[t], acc);
      // lane (lg, c) holds D[(4 GPS) j + 4 lg + r][c]: the limb-r sums of
      // row c, group GPS*s + lg, batch row BPI*bc + j  (register 4 j + r)
#pragma unroll
      for (int jj = 0; jj < BPI; ++jj) {
        const int bq = bc * BPI + jj;
        if (bq < NB) {
          // limb 0 = low digit l, limb 1 = m, limb 2 = high digit h
          const float v = static_cast<float>(acc[4 * jj + 2]) * 65536.f +
                          static_cast<float>(acc[4 * jj + 1]) * 256.f + static_cast<float>(acc[4 * jj]);
          yacc[bq] += half_bits_to_float(cur.s) * (v * cur.xf[bq].y) +
                      half_bits_to_float(cur.bias) * cur.xf[bq].x;
        }
      }
    }
    load_item(pc, cur);
    advance(pc);
  };

  int slot = 0;  // ring slot of the next item to consume
  int cur_mod = -1;
  int m = 0;
  for (int q = blockIdx.x; q < total; q += grid) {
    while (m + 1 < nmod && q >= args.m[m + 1].tile0) ++m;
    const ModDesc& d = args.m[m];
    if (!AG && m != cur_mod) {
      // limbs of this module into LDS; the barrier first orders every read
      // of the previous module's limbs before they are overwritten
      __syncthreads();
      const int per_b = d.Gp * kLimbs * kWordsPerGroup;  // uint4 per batch row
#pragma unroll
      for (int bq = 0; bq < NB; ++bq)
        for (int i = tid; i < per_b; i += 256)
          lds_a[bq * d.Gp * kLimbs * kLdsRow + (i >> 3) * kLdsRow + (i & 7)] = d.aops[bq * per_b + i];
      __syncthreads();
      cur_mod = m;
    }
    cur_gp = d.Gp;
    const int row0 = ((q - d.tile0) * TG + tslot) * M;
    const int S = d.Gp / GPS;
    const int cnt = row0 < d.N ? (S - kpart + WPT - 1) / WPT : 0;
#pragma unroll
    for (int bq = 0; bq < NB; ++bq) yacc[bq] = 0.f;
    for (int j = 0; j < cnt; ++j) {
      const int s = kpart + j * WPT;
      if constexpr (P == 2) {
        if (slot == 0) consume(std::integral_constant<int, 0>{}, s);
        else consume(std::integral_constant<int, 1>{}, s);
      } else {
        static_assert(P == 4, "ring depth 2 or 4");
        if (slot == 0) consume(std::integral_constant<int, 0>{}, s);
        else if (slot == 1) consume(std::integral_constant<int, 1>{}, s);
        else if (slot == 2) consume(std::integral_constant<int, 2>{}, s);
        else consume(std::integral_constant<int, 3>{}, s);
      }
      slot = (slot + 1) & (P - 1);
    }
    // reduce this tile: lane groups by shuffles, then (WPT > 1) the waves
    // sharing the tile through LDS
    float part[NB];
#pragma unroll
    for (int bq = 0; bq < NB; ++bq) {
      float v = yacc[bq];
#pragma unroll
      for (int o = M; o < 64; o <<= 1) v += __shfl_xor(v, o);
      part[bq] = v;
    }
    if constexpr (WPT == 1) {
      if (lg == 0 && row0 + c < d.N) {
#pragma unroll
        for (int bq = 0; bq < NB; ++bq) d.y[(int64_t)bq * d.N + row0 + c] = part[bq];
      }
    } else {
      if (lg == 0) {
#pragma unroll
        for (int bq = 0; bq < NB; ++bq) red[wave][bq][c] = part[bq];
      }
      __syncthreads();
      if (kpart == 0 && lg == 0 && row0 + c < d.N) {
#pragma unroll
        for (int bq = 0; bq < NB; ++bq) {
          float a = 0.f;
#pragma unroll
          for (int w = 0; w < WPT; ++w) a += red[wave + w][bq][c];
          d.y[(int64_t)bq * d.N + row0 + c] = a;
        }
      }
      __syncthreads();
    }
  }
}

template <int L>
static void launch_prep(const void* x, int dt, const int8_t* signs, int64_t B, int64_t K, uint4* aops,
                        float2* xg, hipStream_t st) {
  constexpr int CH = L > 1024 ? L : 1024;
  const int64_t nchunks = (K + CH - 1) / CH;
  const int64_t waves = B * nchunks;
  const int64_t Gp = padded_groups(K);
  const dim3 grid(static_cast<unsigned>((waves + 3) / 4));
  if (dt == TB_F32)
    hipLaunchKernelGGL((gemv_prep_kernel<L, TB_F32>), grid, dim3(kThreads), 0, st, x, signs, B, K, nchunks,
                       Gp, aops, xg);
  else
    hipLaunchKernelGGL((gemv_prep_kernel<L, TB_BF16>), grid, dim3(kThreads), 0, st, x, signs, B, K, nchunks,
                       Gp, aops, xg);
}

constexpr int64_t kLdsLimbBudget = 144 * 1024;  // most limbs one workgroup stages in LDS

// Rows per tile: 16 (v_mfma_i32_16x16x64_i8) for batch 1, 32 otherwise.
static inline int tile_rows(int64_t B) { return B == 1 ? 16 : 32; }

// Waves per tile: all four split K when there are too few tiles to give
// every CU several waves of its own; otherwise one wave per tile.
static inline int waves_per_tile(int64_t tiles, int cus) { return tiles >= 8LL * cus ? 1 : 4; }

template <int NB, int WPT, bool AG>
static void launch_main_cfg(const MultiArgs& a, size_t lds, int grid, hipStream_t st) {
  constexpr int M = NB == 1 ? 16 : 32;
  auto kern = gemv_main_kernel<NB, M, WPT, (AG ? 2 : 4), AG>;
  static std::atomic<uint64_t> lds_set{0};
  lds_limit_once(reinterpret_cast<const void*>(kern), 150 * 1024, lds_set);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, st, a);
}

// Limbs are staged in LDS when they fit (kLdsLimbBudget), otherwise every
// span carries its own limbs from the workspace (L2-resident).
template <int NB>
static void launch_main(const MultiArgs& a, int wpt, int64_t max_gp, int grid, hipStream_t st) {
  const bool ag = lds_limb_bytes(NB, max_gp) > kLdsLimbBudget;
  const size_t lds = ag ? kWordsPerGroup * 16 : static_cast<size_t>(lds_limb_bytes(NB, max_gp) + kWordsPerGroup * 16);
  if (ag) {
    if (wpt == 1) launch_main_cfg<NB, 1, true>(a, lds, grid, st);
    else launch_main_cfg<NB, 4, true>(a, lds, grid, st);
  } else {
    if (wpt == 1) launch_main_cfg<NB, 1, false>(a, lds, grid, st);
    else launch_main_cfg<NB, 4, false>(a, lds, grid, st);
  }
}

static int gemv_common_checks(int64_t B, int64_t K, int64_t N, const char* who) {
  if (B < 0 || N < 0) {
    set_error("%s: B and N must be >= 0", who);
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
  if (B > TB_GEMV_MAX_BATCH) {
    set_error("%s: batch %lld exceeds %d (use tb_ternary_gemm)", who, (long long)B, TB_GEMV_MAX_BATCH);
    return TB_ERR_SHAPE;
  }
  if (K > (int64_t(1) << 24)) {  // keeps every buffer offset of the kernels in 32 bits
    set_error("%s: K=%lld exceeds 2^24", who, (long long)K);
    return TB_ERR_SHAPE;
  }
  return TB_OK;
}

static int gemv_ws_check(const void* workspace, size_t ws_bytes, int64_t B, int64_t K, const char* who) {
  const GemvWs lay = gemv_ws_layout(B, K);
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

// The transform kernel reads x and signs with 16-byte vector loads.
static int prep_align_checks(const void* x, const int8_t* signs, const char* who) {
  if (!aligned(x, 16) || (signs && !aligned(signs, 16))) {
    set_error("%s: x and signs must be 16-byte aligned", who);
    return TB_ERR_ALIGN;
  }
  return TB_OK;
}

static void gemv_prepare_launch(const void* x, int x_dtype, int64_t B, int64_t K, const int8_t* signs,
                                int block, void* workspace, hipStream_t st) {
  const GemvWs lay = gemv_ws_layout(B, K);
  char* ws = static_cast<char*>(workspace);
  uint4* aops = reinterpret_cast<uint4*>(ws + lay.aops_off);
  float2* xg = reinterpret_cast<float2*>(ws + lay.xg_off);
  switch (block) {
    case 0: launch_prep<0>(x, x_dtype, signs, B, K, aops, xg, st); break;
    case 512: launch_prep<512>(x, x_dtype, signs, B, K, aops, xg, st); break;
    case 1024: launch_prep<1024>(x, x_dtype, signs, B, K, aops, xg, st); break;
    case 2048: launch_prep<2048>(x, x_dtype, signs, B, K, aops, xg, st); break;
    default: launch_prep<4096>(x, x_dtype, signs, B, K, aops, xg, st); break;
  }
}

static void fill_module(ModDesc& d, const void* workspace, int64_t B, int64_t K, const uint32_t* codes,
                        const uint16_t* scales, const uint16_t* biases, int64_t N, float* y) {
  const GemvWs lay = gemv_ws_layout(B, K);
  const char* ws = static_cast<const char*>(workspace);
  d.codes = codes;
  d.scales = scales;
  d.biases = biases;
  d.aops = reinterpret_cast<const uint4*>(ws + lay.aops_off);
  d.xg = reinterpret_cast<const float2*>(ws + lay.xg_off);
  d.y = y;
  d.N = static_cast<int>(N);
  d.K = static_cast<int>(K);
  d.Gp = static_cast<int>(padded_groups(K));
}

// Launch the matmul over a.count filled modules (tile0 and total_tiles are
// computed here, in tile groups).
static void gemv_launch_multi(MultiArgs& a, int64_t B, hipStream_t st) {
  const int cus = device_cus();
  int64_t tiles = 0, max_gp = 0;
  for (int i = 0; i < a.count; ++i) {
    tiles += (a.m[i].N + tile_rows(B) - 1) / tile_rows(B);
    max_gp = std::max<int64_t>(max_gp, a.m[i].Gp);
  }
  const int wpt = waves_per_tile(tiles, cus);
  const int tg = 4 / wpt;
  int groups = 0;
  for (int i = 0; i < a.count; ++i) {
    a.m[i].tile0 = groups;
    const int t = (a.m[i].N + tile_rows(B) - 1) / tile_rows(B);
    groups += (t + tg - 1) / tg;
  }
  a.total_tiles = groups;
  const int grid = std::min(groups, cus * 4);
  switch (B) {
    case 1: launch_main<1>(a, wpt, max_gp, grid, st); break;
    case 2: launch_main<2>(a, wpt, max_gp, grid, st); break;
    case 3: launch_main<3>(a, wpt, max_gp, grid, st); break;
    case 4: launch_main<4>(a, wpt, max_gp, grid, st); break;
    case 5: launch_main<5>(a, wpt, max_gp, grid, st); break;
    case 6: launch_main<6>(a, wpt, max_gp, grid, st); break;
    case 7: launch_main<7>(a, wpt, max_gp, grid, st); break;
    default: launch_main<8>(a, wpt, max_gp, grid, st); break;
  }
}

static void gemv_run_launch(const void* workspace, int64_t B, int64_t K, const uint32_t* codes,
                            const uint16_t* scales, const uint16_t* biases, int64_t N, float* y,
                            hipStream_t st) {
  MultiArgs a{};
  a.count = 1;
  fill_module(a.m[0], workspace, B, K, codes, scales, biases, N, y);
  gemv_launch_multi(a, B, st);
}

static int run_checks(int64_t N, int64_t K, const uint32_t* codes, const uint16_t* scales, const uint16_t* biases,
                      const float* y, const char* who) {
  TB_TRY(check_container(codes, scales, biases, who, 4));
  if (!y) {
    set_error("%s: y is NULL", who);
    return TB_ERR_ARG;
  }
  if (!aligned(y, 4)) {
    set_error("%s: y must be 4-byte aligned", who);
    return TB_ERR_ALIGN;
  }
  if (N > (int64_t(1) << 30) || N * (K / kCodesPerWord) * 4 > 0x7FFFFFFFll) {
    set_error("%s: N=%lld x K=%lld too large (codes of one call must stay under 2 GiB)", who,
              (long long)N, (long long)K);
    return TB_ERR_SHAPE;
  }
  return TB_OK;
}

}  // namespace tb

using namespace tb;

extern "C" size_t tb_ternary_gemv_workspace_size(int64_t B, int64_t K) {
  if (B <= 0 || K <= 0 || K % kGroup) return 0;
  return static_cast<size_t>(gemv_ws_layout(B, K).total);
}

extern "C" size_t tb_ternary_gemv_workspace_size_n(int64_t B, int64_t K, int64_t N) {
  const size_t base = tb_ternary_gemv_workspace_size(B, K);
  if (base == 0 || N <= 0 || B < 2 || B > TB_GEMV_MAX_BATCH || N > (int64_t(1) << 30) || K > (int64_t(1) << 24))
    return base;
  return std::max(base, gemv_batch_workspace(B, K, N));
}

extern "C" int tb_ternary_gemv_prepare(const void* x, int x_dtype, int64_t B, int64_t K,
                                       const int8_t* signs, int block, void* workspace,
                                       size_t ws_bytes, void* stream) {
  const char* who = "tb_ternary_gemv_prepare";
  TB_TRY(gemv_common_checks(B, K, 0, who));
  TB_TRY(check_rotation(K, block, signs, who));
  if (B == 0) return TB_OK;
  TB_TRY(check_dtype(x_dtype, x, who));
  TB_TRY(prep_align_checks(x, signs, who));
  TB_TRY(gemv_ws_check(workspace, ws_bytes, B, K, who));
  gemv_prepare_launch(x, x_dtype, B, K, signs, block, workspace, static_cast<hipStream_t>(stream));
  TB_LAUNCH_CHECK(who);
  return TB_OK;
}

extern "C" int tb_ternary_gemv_run(const void* workspace, size_t ws_bytes, int64_t B, int64_t K,
                                   const uint32_t* codes, const uint16_t* scales,
                                   const uint16_t* biases, int64_t N, float* y, void* stream) {
  const char* who = "tb_ternary_gemv_run";
  TB_TRY(gemv_common_checks(B, K, N, who));
  if (B == 0 || N == 0) return TB_OK;
  TB_TRY(run_checks(N, K, codes, scales, biases, y, who));
  TB_TRY(gemv_ws_check(workspace, ws_bytes, B, K, who));
  gemv_run_launch(workspace, B, K, codes, scales, biases, N, y, static_cast<hipStream_t>(stream));
  TB_LAUNCH_CHECK(who);
  return TB_OK;
}

namespace tb {

// Host checks of tb_ternary_gemv's arguments other than the workspace.
int gemv_checked_args(const void* x, int x_dtype, int64_t B, int64_t K, const int8_t* signs, int block,
                           const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t N,
                           const float* y, const char* who) {
  TB_TRY(gemv_common_checks(B, K, N, who));
  TB_TRY(check_rotation(K, block, signs, who));
  if (B == 0 || N == 0) return TB_OK;
  TB_TRY(check_dtype(x_dtype, x, who));
  TB_TRY(prep_align_checks(x, signs, who));
  TB_TRY(run_checks(N, K, codes, scales, biases, y, who));
  return TB_OK;
}

// The path choice and launches of tb_ternary_gemv, after gemv_checked_args.
int gemv_dispatch(const void* x, int x_dtype, int64_t B, int64_t K, const int8_t* signs, int block,
                  const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t N, float* y,
                  void* workspace, size_t ws_bytes, hipStream_t st, const char* who) {
  const size_t batch_ws = gemv_batch_eligible(B, K, N, block) ? gemv_batch_workspace(B, K, N) : 0;
  if (gemv_batch_eligible(B, K, N, block) &&
      (batch_ws == 0 || (workspace && aligned(workspace, 16) && ws_bytes >= batch_ws))) {
    gemv_batch_launch(x, x_dtype, B, K, signs, block, codes, scales, biases, N, y, workspace, st);
    TB_LAUNCH_CHECK(who);
    return TB_OK;
  }
  TB_TRY(gemv_ws_check(workspace, ws_bytes, B, K, who));
  // the band kernel stages scales and biases with 16-byte direct-to-LDS loads
  if (gemv_band_eligible(B, K, N, block) && aligned(scales, 16) && aligned(biases, 16)) {
    gemv_band_launch(x, x_dtype, K, signs, block, codes, scales, biases, N, y, st);
    TB_LAUNCH_CHECK(who);
    return TB_OK;
  }
  if (gemv_fused_eligible(B, K, N, block)) {
    gemv_fused_launch(x, x_dtype, B, K, signs, block, codes, scales, biases, N, y, st);
    TB_LAUNCH_CHECK(who);
    return TB_OK;
  }
  gemv_prepare_launch(x, x_dtype, B, K, signs, block, workspace, st);
  TB_LAUNCH_CHECK(who);
  gemv_run_launch(workspace, B, K, codes, scales, biases, N, y, st);
  TB_LAUNCH_CHECK(who);
  return TB_OK;
}

}  // namespace tb

extern "C" int tb_ternary_gemv(const void* x, int x_dtype, int64_t B, int64_t K,
                               const int8_t* signs, int block, const uint32_t* codes,
                               const uint16_t* scales, const uint16_t* biases, int64_t N, float* y,
                               void* workspace, size_t ws_bytes, void* stream) {
  const char* who = "tb_ternary_gemv";
  TB_TRY(gemv_checked_args(x, x_dtype, B, K, signs, block, codes, scales, biases, N, y, who));
  if (B == 0 || N == 0) return TB_OK;
  return gemv_dispatch(x, x_dtype, B, K, signs, block, codes, scales, biases, N, y, workspace, ws_bytes,
                       static_cast<hipStream_t>(stream), who);
}
