// Randomised driver for the host helpers of the C ABI (csrc/host.cpp), built by
// tests/test_sanitize_cpu.py with g++ and AddressSanitizer + UndefinedBehaviorSanitizer.
// Exit code 0 and "ok" on stdout when every check held.
//
// lazyattn_encode_meta: random tables whose entries are in range round-trip through the
// documented word layout (id in the low LAZYATTN_ID_BITS bits, the offset delta
// off - 16 t as a two's-complement field above it); tables with planted out-of-range ids or
// deltas return RANGE, report the first bad entry and zero every bad word while the good
// ones are still written; NULL and SHAPE errors. lazyattn_llama31_inv_freq: every entry is
// finite, the highest frequencies are unchanged, the lowest are divided by the factor, the
// table never increases along k, and bad arguments are refused. lazyattn_status_str gives a
// string for every code.
#include "lazyattn.h"

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

namespace {

uint64_t rng_state = 0x9E3779B97F4A7C15ull;
uint32_t next_u32() {                     // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
int64_t uniform(int64_t lo, int64_t hi) {
  return lo + (int64_t)(((uint64_t)next_u32() << 32 | next_u32()) % (uint64_t)(hi - lo + 1));
}

int fails = 0;
#define CHECK(c, ...)                                   \
  do {                                                  \
    if (!(c)) {                                         \
      std::printf("FAIL line %d: ", __LINE__);          \
      std::printf(__VA_ARGS__);                         \
      std::printf("\n");                                \
      if (++fails > 20) std::exit(1);                   \
    }                                                   \
  } while (0)

constexpr int64_t kIdMax = (1ll << LAZYATTN_ID_BITS) - 1;
constexpr int64_t kDeltaMin = -(1ll << (LAZYATTN_DELTA_BITS - 1));
constexpr int64_t kDeltaMax = (1ll << (LAZYATTN_DELTA_BITS - 1)) - 1;

void encode_case(int case_no, bool plant) {
  const int num_seqs = (int)uniform(0, 12);
  std::vector<int32_t> bt{0};
  for (int s = 0; s < num_seqs; ++s) bt.push_back(bt.back() + (int32_t)uniform(0, 40));
  const int64_t n = bt.back();
  std::vector<int32_t> ids((size_t)n);
  std::vector<int64_t> offs((size_t)n);
  std::vector<uint8_t> bad((size_t)n, 0);
  for (int s = 0; s < num_seqs; ++s)
    for (int64_t e = bt[s]; e < bt[s + 1]; ++e) {
      const int64_t t = e - bt[s];
      ids[(size_t)e] = (int32_t)uniform(0, kIdMax);
      offs[(size_t)e] = 16 * t + uniform(kDeltaMin, kDeltaMax);
      if (plant && uniform(0, 9) == 0) {
        bad[(size_t)e] = 1;
        switch (uniform(0, 3)) {
          case 0: ids[(size_t)e] = (int32_t)(kIdMax + 1 + uniform(0, 1000)); break;
          case 1: ids[(size_t)e] = -(int32_t)uniform(1, 1000); break;
          case 2: offs[(size_t)e] = 16 * t + kDeltaMax + uniform(1, 1000); break;
          default: offs[(size_t)e] = 16 * t + kDeltaMin - uniform(1, 1000); break;
        }
      }
    }
  std::vector<uint32_t> words((size_t)n + 1, 0xDEADBEEFu);
  int64_t first_bad = 12345;
  const int rc = lazyattn_encode_meta(ids.data(), offs.data(), bt.data(), num_seqs, 16,
                                      words.data(), &first_bad);
  int64_t want_first = -1;
  for (int64_t e = 0; e < n && want_first < 0; ++e)
    if (bad[(size_t)e]) want_first = e;
  CHECK(rc == (want_first >= 0 ? LAZYATTN_ERR_RANGE : LAZYATTN_OK) && first_bad == want_first,
        "case %d: rc %d first_bad %lld want %lld", case_no, rc, (long long)first_bad,
        (long long)want_first);
  CHECK(words[(size_t)n] == 0xDEADBEEFu, "case %d: wrote past the table", case_no);
  for (int s = 0; s < num_seqs; ++s)
    for (int64_t e = bt[s]; e < bt[s + 1]; ++e) {
      const uint32_t w = words[(size_t)e];
      if (bad[(size_t)e]) {
        CHECK(w == 0, "case %d: bad entry %lld not zeroed", case_no, (long long)e);
        continue;
      }
      const int64_t id = w & (uint32_t)kIdMax;
      int64_t delta = (int64_t)(w >> LAZYATTN_ID_BITS);
      if (delta > kDeltaMax) delta -= 1ll << LAZYATTN_DELTA_BITS;
      CHECK(id == ids[(size_t)e] && 16 * (e - bt[s]) + delta == offs[(size_t)e],
            "case %d: entry %lld decodes to (%lld, %lld)", case_no, (long long)e, (long long)id,
            (long long)(16 * (e - bt[s]) + delta));
    }
}

void encode_errors() {
  int32_t bt[3] = {0, 2, 3};
  int32_t ids[3] = {1, 2, 3};
  int64_t offs[3] = {0, 16, 0};
  uint32_t w[3];
  int64_t fb = 0;
  CHECK(lazyattn_encode_meta(ids, offs, nullptr, 2, 16, w, &fb) == LAZYATTN_ERR_NULL, "null table");
  CHECK(lazyattn_encode_meta(nullptr, offs, bt, 2, 16, w, &fb) == LAZYATTN_ERR_NULL, "null ids");
  CHECK(lazyattn_encode_meta(ids, offs, bt, 2, 16, nullptr, &fb) == LAZYATTN_ERR_NULL, "null out");
  CHECK(lazyattn_encode_meta(ids, offs, bt, 2, 32, w, &fb) == LAZYATTN_ERR_SHAPE, "B != 16");
  CHECK(lazyattn_encode_meta(ids, offs, bt, -1, 16, w, &fb) == LAZYATTN_ERR_SHAPE, "num_seqs < 0");
  int32_t down[3] = {0, 2, 1};
  CHECK(lazyattn_encode_meta(ids, offs, down, 2, 16, w, &fb) == LAZYATTN_ERR_SHAPE, "decreasing");
  int32_t from1[3] = {1, 2, 3};
  CHECK(lazyattn_encode_meta(ids, offs, from1, 2, 16, w, &fb) == LAZYATTN_ERR_SHAPE, "not from 0");
  CHECK(lazyattn_encode_meta(nullptr, nullptr, bt, 0, 16, nullptr, nullptr) == LAZYATTN_OK,
        "empty table");
}

void llama31_checks() {
  for (int D : {64, 128}) {
    for (double factor : {1.0, 8.0, 32.0}) {
      std::vector<double> t((size_t)D / 2, -1.0);
      const double base = 500000.0, lo = 1.0, hi = 4.0, ctx = 8192.0;
      const int rc = lazyattn_llama31_inv_freq(D, base, factor, lo, hi, ctx, t.data());
      CHECK(rc == LAZYATTN_OK, "llama31 rc %d", rc);
      for (int k = 0; k < D / 2; ++k) {
        const double theta = std::pow(base, -2.0 * k / D);
        const double wave = 6.283185307179586476925286766559 / theta;
        CHECK(std::isfinite(t[(size_t)k]) && t[(size_t)k] > 0.0, "llama31 entry %d", k);
        if (wave < ctx / hi)
          CHECK(t[(size_t)k] == theta, "llama31 short wave %d changed", k);
        if (wave > ctx / lo)
          CHECK(std::fabs(t[(size_t)k] - theta / factor) <= 1e-15 * theta, "llama31 long wave %d", k);
        if (k > 0) CHECK(t[(size_t)k] <= t[(size_t)k - 1], "llama31 not non-increasing at %d", k);
      }
    }
  }
  double t[64];
  CHECK(lazyattn_llama31_inv_freq(128, 500000.0, 8.0, 1.0, 4.0, 8192.0, nullptr) ==
            LAZYATTN_ERR_NULL, "llama31 null");
  CHECK(lazyattn_llama31_inv_freq(130, 500000.0, 8.0, 1.0, 4.0, 8192.0, t) == LAZYATTN_ERR_SHAPE,
        "llama31 D too large");
  CHECK(lazyattn_llama31_inv_freq(63, 500000.0, 8.0, 1.0, 4.0, 8192.0, t) == LAZYATTN_ERR_SHAPE,
        "llama31 odd D");
  CHECK(lazyattn_llama31_inv_freq(128, 0.5, 8.0, 1.0, 4.0, 8192.0, t) == LAZYATTN_ERR_ARG,
        "llama31 base");
  CHECK(lazyattn_llama31_inv_freq(128, 500000.0, 8.0, 4.0, 1.0, 8192.0, t) == LAZYATTN_ERR_ARG,
        "llama31 factors");
  CHECK(lazyattn_llama31_inv_freq(128, 500000.0, NAN, 1.0, 4.0, 8192.0, t) == LAZYATTN_ERR_ARG,
        "llama31 nan factor");
}

}  // namespace

int main(int argc, char** argv) {
  const int cases = argc > 1 ? std::atoi(argv[1]) : 400;
  encode_errors();
  for (int c = 0; c < cases; ++c) encode_case(c, c % 2 == 1);
  llama31_checks();
  for (int code = 1; code >= -12; --code) {
    const char* s = lazyattn_status_str(code);
    CHECK(s != nullptr && std::strlen(s) > 0, "status string for %d", code);
  }
  CHECK(lazyattn_version() != nullptr, "version");
  if (fails) {
    std::printf("%d failures\n", fails);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
