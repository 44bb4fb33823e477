// Host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer:
// the container functions (tb_pack / tb_unpack / tb_signs_validate, the
// PQ2_0 and PTQ1_0 transcodes) and the status strings, on exact-size heap
// buffers so that any read or write past an array is reported.  Built and
// run by tests/test_host_sanitize.py with g++ -fsanitize=address,undefined;
// it links only the two host sources, no HIP runtime.
//
// Checks: round trips are exact (t -> codes -> t, MLX -> PQ2_0 -> MLX,
// t -> PTQ1_0 -> t), each documented error is returned for its bad input,
// and a call on zero rows touches nothing.  Exit status 0 when every check
// holds; the first failed check is printed.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <random>
#include <vector>

#include "tb.h"

static int g_fail = 0;
#define CHECK(cond)                                                 \
  do {                                                              \
    if (!(cond)) {                                                  \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      g_fail = 1;                                                   \
      return;                                                       \
    }                                                               \
  } while (0)

// Exact-size heap arrays (new[] of the element count), so ASan sees the ends.
template <class T>
static std::unique_ptr<T[]> arr(size_t n) {
  return std::unique_ptr<T[]>(new T[n ? n : 1]);
}

static uint16_t scale_bits(std::mt19937& r) {
  // positive normal fp16 in [2^-10, 2): exponent 5..15, any mantissa
  std::uniform_int_distribution<int> e(5, 15), m(0, 1023);
  return static_cast<uint16_t>((e(r) << 10) | m(r));
}

static void round_trips(int64_t N, int64_t K, unsigned seed) {
  std::mt19937 r(seed);
  const int64_t G = K / 128, W = K / 16;
  auto t = arr<int8_t>(N * K);
  auto s = arr<uint16_t>(N * G);
  std::uniform_int_distribution<int> tern(-1, 1);
  for (int64_t i = 0; i < N * K; ++i) t[i] = static_cast<int8_t>(tern(r));
  for (int64_t i = 0; i < N * G; ++i) s[i] = scale_bits(r);

  // MLX container
  auto codes = arr<uint32_t>(N * W);
  auto so = arr<uint16_t>(N * G);
  auto bo = arr<uint16_t>(N * G);
  CHECK(tb_pack(t.get(), s.get(), N, K, codes.get(), so.get(), bo.get()) == TB_OK);
  for (int64_t i = 0; i < N * G; ++i) {
    CHECK(so[i] == s[i]);
    CHECK(bo[i] == static_cast<uint16_t>(s[i] ^ 0x8000u));
  }
  auto t2 = arr<int8_t>(N * K);
  CHECK(tb_unpack(codes.get(), N, K, t2.get()) == TB_OK);
  CHECK(std::memcmp(t.get(), t2.get(), N * K) == 0);

  // PQ2_0: MLX -> blocks -> MLX, bit for bit
  auto pq = arr<uint8_t>(N * G * 34);
  CHECK(tb_pq2_from_mlx(codes.get(), so.get(), bo.get(), N, K, pq.get()) == TB_OK);
  auto c3 = arr<uint32_t>(N * W);
  auto s3 = arr<uint16_t>(N * G);
  auto b3 = arr<uint16_t>(N * G);
  CHECK(tb_pq2_to_mlx(pq.get(), N, K, c3.get(), s3.get(), b3.get()) == TB_OK);
  CHECK(std::memcmp(c3.get(), codes.get(), N * W * 4) == 0);
  CHECK(std::memcmp(s3.get(), so.get(), N * G * 2) == 0);
  CHECK(std::memcmp(b3.get(), bo.get(), N * G * 2) == 0);

  // PTQ1_0: t -> blocks -> t
  auto p1 = arr<uint8_t>(N * G * 28);
  CHECK(tb_ptq1_pack(t.get(), s.get(), N, K, p1.get()) == TB_OK);
  auto t4 = arr<int8_t>(N * K);
  auto s4 = arr<uint16_t>(N * G);
  CHECK(tb_ptq1_unpack(p1.get(), N, K, t4.get(), s4.get()) == TB_OK);
  CHECK(std::memcmp(t4.get(), t.get(), N * K) == 0);
  CHECK(std::memcmp(s4.get(), s.get(), N * G * 2) == 0);
}

static void errors() {
  const int64_t N = 2, K = 256, G = K / 128, W = K / 16;
  auto t = arr<int8_t>(N * K);
  auto s = arr<uint16_t>(N * G);
  auto codes = arr<uint32_t>(N * W);
  auto so = arr<uint16_t>(N * G);
  auto bo = arr<uint16_t>(N * G);
  std::memset(t.get(), 0, N * K);
  for (int64_t i = 0; i < N * G; ++i) s[i] = 0x3C00;  // 1.0

  // shape and pointer errors
  CHECK(tb_pack(t.get(), s.get(), N, 200, codes.get(), so.get(), bo.get()) == TB_ERR_SHAPE);
  CHECK(tb_pack(nullptr, s.get(), N, K, codes.get(), so.get(), bo.get()) == TB_ERR_ARG);
  CHECK(tb_unpack(codes.get(), N, 0, t.get()) != TB_OK);
  CHECK(std::strlen(tb_last_error()) > 0);

  // a ternary value outside {-1, 0, 1}
  t[N * K - 1] = 2;
  CHECK(tb_pack(t.get(), s.get(), N, K, codes.get(), so.get(), bo.get()) == TB_ERR_CODE);
  CHECK(tb_ptq1_pack(t.get(), s.get(), N, K, arr<uint8_t>(N * G * 28).get()) == TB_ERR_CODE);
  t[N * K - 1] = 0;

  // code 3 on unpack and on the PQ2_0 transcode
  CHECK(tb_pack(t.get(), s.get(), N, K, codes.get(), so.get(), bo.get()) == TB_OK);
  codes[N * W - 1] |= 3u << 30;
  auto t2 = arr<int8_t>(N * K);
  CHECK(tb_unpack(codes.get(), N, K, t2.get()) == TB_ERR_CODE);
  auto pq = arr<uint8_t>(N * G * 34);
  CHECK(tb_pq2_from_mlx(codes.get(), so.get(), bo.get(), N, K, pq.get()) == TB_ERR_CODE);
  codes[N * W - 1] &= ~(3u << 30);

  // a bias that is not the negated scale cannot travel as PQ2_0
  bo[N * G - 1] ^= 1;
  CHECK(tb_pq2_from_mlx(codes.get(), so.get(), bo.get(), N, K, pq.get()) == TB_ERR_CODE);
  bo[N * G - 1] ^= 1;

  // a PTQ1_0 trit byte out of range (the last byte of a block holds 3 trits)
  auto p1 = arr<uint8_t>(N * G * 28);
  CHECK(tb_ptq1_pack(t.get(), s.get(), N, K, p1.get()) == TB_OK);
  p1[N * G * 28 - 1] = 27;
  auto s4 = arr<uint16_t>(N * G);
  CHECK(tb_ptq1_unpack(p1.get(), N, K, t2.get(), s4.get()) == TB_ERR_CODE);

  // signs
  auto sg = arr<int8_t>(K);
  for (int64_t k = 0; k < K; ++k) sg[k] = (k & 1) ? 1 : -1;
  CHECK(tb_signs_validate(sg.get(), K) == TB_OK);
  sg[K - 1] = 0;
  CHECK(tb_signs_validate(sg.get(), K) == TB_ERR_SIGN);
  CHECK(tb_signs_validate(nullptr, K) == TB_ERR_ARG);

  // zero rows: nothing is read or written (null outputs are accepted)
  CHECK(tb_pq2_from_mlx(codes.get(), so.get(), bo.get(), 0, K, nullptr) == TB_OK);

  // every status has a string
  for (int st = TB_ERR_WORKSPACE; st <= TB_OK; ++st) CHECK(tb_status_str(st) != nullptr);
  CHECK(tb_abi_version() == TB_ABI_VERSION);
}

int main() {
  round_trips(1, 128, 1);
  round_trips(3, 384, 2);
  round_trips(17, 1024, 3);
  round_trips(5, 5120, 4);
  errors();
  if (g_fail) return 1;
  std::printf("host sanitize driver: all checks passed\n");
  return 0;
}
