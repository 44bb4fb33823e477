// Host container functions of the two block formats [kwkr.cn/news/564617,
// "packing-format engineering": GGUF blocks of 128 ternary weights; PQ2_0
// is a lossless transcode of the MLX container (34 bytes per block), PTQ1_0
// packs the trits densely (28 bytes per block)].  Layouts (a reading): the
// fp16 scale's two bytes (little-endian) first; PQ2_0 then holds code k at
// bits 2 (k % 4) of byte k / 4, PTQ1_0 26 bytes of five base-3 codes each,
// the first code the lowest digit (the last byte three codes).
#include "tb_common.h"

namespace {

constexpr int64_t kPq2Bytes = 34, kPtq1Bytes = 28, kTritBytes = 26;

int check_shape(int64_t N, int64_t K, const char* who) {
  if (N < 0 || K <= 0) {
    tb::set_error("%s: need N >= 0 and K > 0 (got N=%lld, K=%lld)", who, (long long)N, (long long)K);
    return TB_ERR_ARG;
  }
  if (K % tb::kGroup) {
    tb::set_error("%s: K=%lld is not a multiple of %d", who, (long long)K, tb::kGroup);
    return TB_ERR_SHAPE;
  }
  return TB_OK;
}

}  // namespace

extern "C" int tb_pq2_from_mlx(const uint32_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t N,
                               int64_t K, uint8_t* blocks) {
  const char* who = "tb_pq2_from_mlx";
  TB_TRY(check_shape(N, K, who));
  if (N == 0) return TB_OK;
  if (!codes || !scales || !biases || !blocks) {
    tb::set_error("%s: NULL pointer", who);
    return TB_ERR_ARG;
  }
  const int64_t G = K / tb::kGroup, W = K / tb::kCodesPerWord;
  int64_t bad_bias = 0, threes = 0;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t g = 0; g < G; ++g) {
      const uint16_t s = scales[n * G + g];
      bad_bias += biases[n * G + g] != static_cast<uint16_t>(s ^ 0x8000u);
      uint8_t* out = blocks + (n * G + g) * kPq2Bytes;
      out[0] = static_cast<uint8_t>(s & 0xFF);
      out[1] = static_cast<uint8_t>(s >> 8);
      for (int w = 0; w < 8; ++w) {
        const uint32_t word = codes[n * W + g * 8 + w];
        threes += ((word & (word >> 1)) & 0x55555555u) != 0;
        for (int b = 0; b < 4; ++b) out[2 + 4 * w + b] = static_cast<uint8_t>(word >> (8 * b));
      }
    }
  }
  if (bad_bias) {
    tb::set_error("%s: %lld groups have a bias other than the negated scale (PQ2_0 stores no bias)", who,
                  (long long)bad_bias);
    return TB_ERR_CODE;
  }
  if (threes) {
    tb::set_error("%s: %lld code words hold code 3 (not ternary)", who, (long long)threes);
    return TB_ERR_CODE;
  }
  return TB_OK;
}

extern "C" int tb_pq2_to_mlx(const uint8_t* blocks, int64_t N, int64_t K, uint32_t* codes, uint16_t* scales,
                             uint16_t* biases) {
  const char* who = "tb_pq2_to_mlx";
  TB_TRY(check_shape(N, K, who));
  if (N == 0) return TB_OK;
  if (!codes || !scales || !biases || !blocks) {
    tb::set_error("%s: NULL pointer", who);
    return TB_ERR_ARG;
  }
  const int64_t G = K / tb::kGroup, W = K / tb::kCodesPerWord;
  int64_t threes = 0;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t g = 0; g < G; ++g) {
      const uint8_t* in = blocks + (n * G + g) * kPq2Bytes;
      const uint16_t s = static_cast<uint16_t>(in[0] | (in[1] << 8));
      scales[n * G + g] = s;
      biases[n * G + g] = static_cast<uint16_t>(s ^ 0x8000u);
      for (int w = 0; w < 8; ++w) {
        uint32_t word = 0;
        for (int b = 0; b < 4; ++b) word |= static_cast<uint32_t>(in[2 + 4 * w + b]) << (8 * b);
        threes += ((word & (word >> 1)) & 0x55555555u) != 0;
        codes[n * W + g * 8 + w] = word;
      }
    }
  }
  if (threes) {
    tb::set_error("%s: %lld code words hold code 3 (not ternary)", who, (long long)threes);
    return TB_ERR_CODE;
  }
  return TB_OK;
}

extern "C" int tb_ptq1_pack(const int8_t* t, const uint16_t* scales, int64_t N, int64_t K, uint8_t* blocks) {
  const char* who = "tb_ptq1_pack";
  TB_TRY(check_shape(N, K, who));
  if (N == 0) return TB_OK;
  if (!t || !scales || !blocks) {
    tb::set_error("%s: NULL pointer", who);
    return TB_ERR_ARG;
  }
  const int64_t G = K / tb::kGroup;
  int64_t bad = 0;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t g = 0; g < G; ++g) {
      const int8_t* tg = t + n * K + g * tb::kGroup;
      uint8_t* out = blocks + (n * G + g) * kPtq1Bytes;
      const uint16_t s = scales[n * G + g];
      out[0] = static_cast<uint8_t>(s & 0xFF);
      out[1] = static_cast<uint8_t>(s >> 8);
      for (int64_t i = 0; i < kTritBytes; ++i) {
        int v = 0, p3 = 1;
        for (int m = 0; m < 5 && 5 * i + m < tb::kGroup; ++m) {
          const int tv = tg[5 * i + m];
          bad += (tv < -1) | (tv > 1);
          v += ((tv + 1) & 3) % 3 * p3;
          p3 *= 3;
        }
        out[2 + i] = static_cast<uint8_t>(v);
      }
    }
  }
  if (bad) {
    tb::set_error("%s: %lld ternary values outside {-1,0,1}", who, (long long)bad);
    return TB_ERR_CODE;
  }
  return TB_OK;
}

extern "C" int tb_ptq1_unpack(const uint8_t* blocks, int64_t N, int64_t K, int8_t* t, uint16_t* scales) {
  const char* who = "tb_ptq1_unpack";
  TB_TRY(check_shape(N, K, who));
  if (N == 0) return TB_OK;
  if (!t || !scales || !blocks) {
    tb::set_error("%s: NULL pointer", who);
    return TB_ERR_ARG;
  }
  const int64_t G = K / tb::kGroup;
  int64_t bad = 0;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t g = 0; g < G; ++g) {
      const uint8_t* in = blocks + (n * G + g) * kPtq1Bytes;
      scales[n * G + g] = static_cast<uint16_t>(in[0] | (in[1] << 8));
      int8_t* tg = t + n * K + g * tb::kGroup;
      for (int64_t i = 0; i < kTritBytes; ++i) {
        int v = in[2 + i];
        const int ncodes = 5 * i + 5 <= tb::kGroup ? 5 : static_cast<int>(tb::kGroup - 5 * i);
        bad += v > (ncodes == 5 ? 242 : 26);
        for (int m = 0; m < ncodes; ++m) {
          tg[5 * i + m] = static_cast<int8_t>(v % 3 - 1);
          v /= 3;
        }
      }
    }
  }
  if (bad) {
    tb::set_error("%s: %lld trit bytes out of range (not a PTQ1_0 container)", who, (long long)bad);
    return TB_ERR_CODE;
  }
  return TB_OK;
}
