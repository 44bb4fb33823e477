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
//   with all of a wave's LDS reads issued before its MFMAs.  The item count
//   per wave is a template parameter, so the items carry no branches (only
//   the last one can be missing; a wave without it skips its reads, since an
//   LDS instruction costs the same whatever its active lanes) and their MFMA
//   chains interleave.  Partial sums meet in LDS and every row of y is
//   written once.
//
// * Remainder blocks.  When the band's last subtile would hold at most 8
//   real rows, those rows (one or two quads of 4) go through
//   v_mfma_i32_4x4x4_16b_i8 instead of 16-row items: a unit is (quad, 8
//   groups); each of the 16 blocks is one (group, half of its words) pair
//   with the group's 4 limb rows as A and the quad's codes as B, so block
//   b's result is the limb sums of its half-group for each row of the quad,
//   row r's in lane 4 b + r.  Units are dealt round robin from the first
//   wave with one 16-row item fewer.
//
// Used for batch 1, blocks 0 / 512 / 1024, at most 3 chunk transforms per
// wave, bands of at most 7 subtiles and an LDS footprint within the limit;
// tb_ternary_gemv takes other paths otherwise.
#include <algorithm>

#include <numeric>

#include "tb_xform.h"

namespace tb {

constexpr int kBandWaves = 8;
constexpr int kBandThreads = 64 * kBandWaves;
constexpr int kBandMaxTasks = 3;      // chunk transforms per wave
constexpr int kBandMaxItems = 4;      // matmul items per wave
constexpr int kBandMaxSub = 7;        // 16-row subtiles per band
constexpr int kBandArow = 144;        // LDS bytes per (group, limb) operand row: 128 + 16 pad
constexpr int kBandSlot = 1024 + 16;  // LDS bytes per staged 1 KB of codes (16 B pad per KB)
constexpr int kBandMaxLoads = 24;     // staging loads per loader wave
constexpr int64_t kBandLdsMax = 150 * 1024;
constexpr int kBandWaitVm0 = (0x7 << 4) | (0xF << 8);  // s_waitcnt vmcnt(0)

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
  l.xf = l.a + nch * 8 * kXfLimbs * kBandArow;
  l.red = l.xf + nch * 8 * 8;
  l.codes = l.red + tsub * kBandWaves * 16 * 4;
  l.sc = l.codes + code_slots * kBandSlot;
  l.bi = l.sc + sb_slots * 1024;
  l.total = l.bi + sb_slots * 1024;
  return l;
}

// rows: output rows per band (the last band may be short); tsq: 16-row
// subtiles per band (bits 0-7) and remainder quads (bits 8-9).
template <int L, int DT, int MI>
__global__ __launch_bounds__(kBandThreads, 1) void gemv_band_kernel(
    const void* __restrict__ x, const int8_t* __restrict__ signs, const uint32_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ biases, int N, int K, int rows,
    int tsq, float* __restrict__ y) {
  constexpr int M = 16, GPS = 4;
  const int tsub = tsq & 0xFF;   // 16-row subtiles per band
  const int quads = tsq >> 8;    // remainder quads (0: none)
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
      if (c < nch) xform_chunk<L, DT>(xin[r], 8 * c, lane, cf, cs, lds_a, lds_xf, kBandArow);
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
  const int items = (tsub - (quads > 0)) * S;
  const uint32_t lane_c = static_cast<uint32_t>(c * RB + lg * 32);
  auto stage_at = [](uint32_t off) { return off + (off >> 10) * (kBandSlot - 1024); };

  // The wave's items are wave + 8 j, j < MI (MI = ceil(items / 8)); only the
  // last can be past the end (it then aliases item 0 and is skipped), so the
  // first MI - 1 items have no branches and their MFMA chains interleave.
  int tt[MI], ss[MI];
  bool iv[MI];
#pragma unroll
  for (int j = 0; j < MI; ++j) {
    const int i = wave + kBandWaves * j;
    iv[j] = i < items;
    const int ic = iv[j] ? i : 0;
    tt[j] = ic / S;
    ss[j] = ic - tt[j] * S;
  }
  // all LDS reads of the wave's items first: codes, scale, bias, the
  // group's (sum, f), and the A operand -- read only by the 16 lanes whose A
  // row is non-zero (the others keep zeros)
  uint4 cw[MI][2];
  uint4 av[MI][kWordsPerGroup];
  float2 xfv[MI];
  uint16_t sraw[MI], braw[MI];
#pragma unroll
  for (int j = 0; j < MI; ++j) {
    cw[j][0] = cw[j][1] = make_uint4(0, 0, 0, 0);
    sraw[j] = braw[j] = 0;
    xfv[j] = make_float2(0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kWordsPerGroup; ++w) av[j][w] = make_uint4(0, 0, 0, 0);
    // LDS instructions cost the same whatever the active lanes: a wave
    // without a last item skips its reads
    if (j < MI - 1 || iv[j]) {
      const int t = tt[j], s = ss[j];
      const uint32_t so = stage_at(lane_c + static_cast<uint32_t>(t * M * RB + s * 128));
      cw[j][0] = *reinterpret_cast<const uint4*>(st_codes + so);
      cw[j][1] = *reinterpret_cast<const uint4*>(st_codes + so + 16);
      const int si = (t * M + c) * G + s * GPS + lg;
      sraw[j] = st_sc[si];
      braw[j] = st_bi[si];
      xfv[j] = lds_xf[s * GPS + lg];
      if (a_lane) {
        const uint4* ap = reinterpret_cast<const uint4*>(lds_a + ((s * GPS + alg) * kXfLimbs + ar) * kBandArow);
#pragma unroll
        for (int w = 0; w < kWordsPerGroup; ++w) av[j][w] = ap[w];
      }
    }
  }
  float part[MI];
#pragma unroll
  for (int j = 0; j < MI; ++j) {
    part[j] = 0.f;
    // only the last item can be invalid; a wave without it skips its work
    if (j < MI - 1 || iv[j]) {
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
    const bool gin = iv[j] && ss[j] * GPS + lg < G;
    const float sc = gin ? half_bits_to_float(sraw[j]) : 0.f;
    const float bi = gin ? half_bits_to_float(braw[j]) : 0.f;
    const float v = static_cast<float>(acc[3]) * 16777216.f + static_cast<float>(acc[2]) * 65536.f +
                    static_cast<float>(acc[1]) * 256.f + static_cast<float>(acc[0]);
    part[j] = sc * (v * xfv[j].y) + bi * xfv[j].x;
    }
  }
  // per subtile: add this wave's items in registers, then over the 4 lane
  // groups, and park the 16 row sums in red[t][wave] (one plain store)
  int tend = tt[0];  // subtile of the wave's last valid item
#pragma unroll
  for (int j = 1; j < MI; ++j) tend = iv[j] ? tt[j] : tend;
  for (int t = tt[0]; t < tsub && t <= tend; ++t) {
    float v = 0.f;
    bool any = false;
#pragma unroll
    for (int j = 0; j < MI; ++j) {
      const bool mine = tt[j] == t && iv[j];
      v += mine ? part[j] : 0.f;
      any |= mine;
    }
    if (any) {
      v += xor_lane(v, 4, lane);
      v += xor_lane(v, 5, lane);
      if (lg == 0) red[(t * kBandWaves + wave) * 16 + c] = v;
    }
  }
  // ---- 3b. remainder blocks (see above): unit u = (quad u / nru, groups
  //          8 (u % nru) ..), this lane block rbk (group 8 (u % nru) +
  //          rbk / 2, half rbk & 1) and quad row rri
  if (quads > 0) {
    const int nru = (G + 7) >> 3;
    const int nunits = quads * nru;
    const int rbk = lane >> 2, rri = lane & 3, h = rbk & 1;
    float yq0 = 0.f, yq1 = 0.f;
    for (int u = (wave - items % kBandWaves + kBandWaves) % kBandWaves; u < nunits; u += kBandWaves) {
      const int qd = u >= nru;
      const int g = (u - qd * nru) * 8 + (rbk >> 1);
      const bool gin = g < G;
      const int row = (tsub - 1) * M + qd * 4 + rri;
      const uint4 cq = gin ? *reinterpret_cast<const uint4*>(
                                 st_codes + stage_at(static_cast<uint32_t>(row * RB + g * 32 + h * 16)))
                           : make_uint4(0, 0, 0, 0);
      // groups past G (a partial last unit) lie within the last chunk's image
      const uint4* ap = reinterpret_cast<const uint4*>(lds_a + (g * kXfLimbs + rri) * kBandArow) + 4 * h;
      const uint32_t wv[4] = {cq.x, cq.y, cq.z, cq.w};
      v4i acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint4 a = ap[t];
        const uint32_t w = wv[t];
        acc0 = __builtin_amdgcn_mfma_i32_4x4x4i8(static_cast<int>(a.x), static_cast<int>(w & 0x03030303u), acc0, 0,
                                                 0, 0);
        acc1 = __builtin_amdgcn_mfma_i32_4x4x4i8(static_cast<int>(a.y), static_cast<int>((w >> 2) & 0x03030303u),
                                                 acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_i32_4x4x4i8(static_cast<int>(a.z), static_cast<int>((w >> 4) & 0x03030303u),
                                                 acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_i32_4x4x4i8(static_cast<int>(a.w), static_cast<int>((w >> 6) & 0x03030303u),
                                                 acc1, 0, 0, 0);
      }
      const v4i acc = acc0 + acc1;
      const float v = static_cast<float>(acc[3]) * 16777216.f + static_cast<float>(acc[2]) * 65536.f +
                      static_cast<float>(acc[1]) * 256.f + static_cast<float>(acc[0]);
      const int si = gin ? row * G + g : 0;
      // the bias term once per group (in its first half)
      const float sc = gin ? half_bits_to_float(st_sc[si]) : 0.f;
      const float bi = (gin && h == 0) ? half_bits_to_float(st_bi[si]) : 0.f;
      const float2 xf = gin ? lds_xf[g] : make_float2(0.f, 0.f);
      const float pr = sc * (v * xf.y) + bi * xf.x;
      if (qd) yq1 += pr;
      else yq0 += pr;
    }
    // add up the 16 blocks of each row (lanes r, r + 4, ..., r + 60)
#pragma unroll
    for (int j = 2; j < 6; ++j) {
      yq0 += xor_lane(yq0, j, lane);
      yq1 += xor_lane(yq1, j, lane);
    }
    if (lane < 4) {
      float* rr = red + ((tsub - 1) * kBandWaves + wave) * 16 + lane;
      rr[0] = yq0;
      if (quads > 1) rr[4] = yq1;
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
struct BandPlan {
  int rows, tsub, grid, mi, quads;
  int64_t lds;
  bool ok;
};

static BandPlan band_plan(int64_t K, int64_t N, int cus) {
  BandPlan p{};
  const int64_t G = K / kGroup, W = K / kCodesPerWord, RB = W * 4;
  const int64_t Gp = (G + 3) / 4 * 4, S = Gp / 4;
  const int64_t nch = (K + 1023) / 1024;
  // rows * G a multiple of 8 keeps every band's scale and bias rows (band0 * G
  // fp16 from a 16-byte aligned base) 16-byte aligned for the direct-to-LDS
  // staging
  const int64_t rq = 8 / std::gcd<int64_t>(G, 8);
  const int64_t rows = (std::max<int64_t>((N + cus - 1) / cus, 16) + rq - 1) / rq * rq;
  const int64_t tsub = (rows + 15) / 16;
  p.rows = static_cast<int>(rows);
  p.tsub = static_cast<int>(tsub);
  p.grid = static_cast<int>((N + rows - 1) / rows);
  // a last subtile of at most 8 real rows goes through remainder blocks
  const int64_t rr = rows - (tsub - 1) * 16;
  p.quads = (tsub >= 2 && rr <= 8) ? static_cast<int>((rr + 3) / 4) : 0;
  p.mi = static_cast<int>(((tsub - (p.quads > 0)) * S + kBandWaves - 1) / kBandWaves);  // 16-row items per wave
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
  return band_plan(K, N, device_cus()).ok;
}

template <int L, int DT, int MI>
static void band_launch_t(const void* x, const int8_t* signs, const uint32_t* codes, const uint16_t* scales,
                          const uint16_t* biases, float* y, int N, int K, const BandPlan& p, hipStream_t st) {
  auto kern = gemv_band_kernel<L, DT, MI>;
  static std::atomic<uint64_t> lds_set{0};
  lds_limit_once(reinterpret_cast<const void*>(kern), static_cast<int>(kBandLdsMax), lds_set);
  hipLaunchKernelGGL(kern, dim3(p.grid), dim3(kBandThreads), static_cast<size_t>(p.lds), st, x, signs, codes, scales,
                     biases, N, K, p.rows, p.tsub | (p.quads << 8), y);
}

template <int L, int DT>
static void band_launch_mi(const void* x, const int8_t* signs, const uint32_t* codes, const uint16_t* scales,
                           const uint16_t* biases, float* y, int N, int K, const BandPlan& p, hipStream_t st) {
  switch (p.mi) {
    case 1: band_launch_t<L, DT, 1>(x, signs, codes, scales, biases, y, N, K, p, st); break;
    case 2: band_launch_t<L, DT, 2>(x, signs, codes, scales, biases, y, N, K, p, st); break;
    case 3: band_launch_t<L, DT, 3>(x, signs, codes, scales, biases, y, N, K, p, st); break;
    default: band_launch_t<L, DT, 4>(x, signs, codes, scales, biases, y, N, K, p, st); break;
  }
}

template <int L>
static void band_launch_l(int dt, const void* x, const int8_t* signs, const uint32_t* codes, const uint16_t* scales,
                          const uint16_t* biases, float* y, int N, int K, const BandPlan& p, hipStream_t st) {
  if (dt == TB_F32) band_launch_mi<L, TB_F32>(x, signs, codes, scales, biases, y, N, K, p, st);
  else band_launch_mi<L, TB_BF16>(x, signs, codes, scales, biases, y, N, K, p, st);
}

void gemv_band_launch(const void* x, int x_dtype, int64_t K, const int8_t* signs, int block, const uint32_t* codes,
                      const uint16_t* scales, const uint16_t* biases, int64_t N, float* y, hipStream_t st) {
  const BandPlan p = band_plan(K, N, device_cus());
  const int n = static_cast<int>(N), k = static_cast<int>(K);
  if (block == 0) band_launch_l<0>(x_dtype, x, signs, codes, scales, biases, y, n, k, p, st);
  else if (block == 512) band_launch_l<512>(x_dtype, x, signs, codes, scales, biases, y, n, k, p, st);
  else band_launch_l<1024>(x_dtype, x, signs, codes, scales, biases, y, n, k, p, st);
}

}  // namespace tb
