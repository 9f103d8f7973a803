// Randomised driver for the host planner of shared-document decode (csrc/share.cpp), built by
// tests/test_sanitize_cpu.py with g++ and AddressSanitizer + UndefinedBehaviorSanitizer.
// Exit code 0 and "ok" on stdout when every check held.
//
// Each case draws a batch whose rows read runs of a few shared "documents" (consecutive
// block ids) at random entries, plus private blocks, plans it with random members per item
// (through Hq / Hkv), max_chunk and wave counts, and checks what any plan must satisfy:
// every planned (row, entry) is covered exactly once, members of an item read the same ids,
// every member's offset delta is constant inside an item, each row's slots are exactly
// [prefix[r], prefix[r + 1]), and the header describes the plan. Error paths: a size query, a too-small buffer (NOSPACE with the length still
// reported), and rejected arguments.
#include "lazyattn.h"

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

uint64_t rng_state = 0x2545F4914F6CDD1Dull;
uint32_t next_u32() {                     // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
int uniform(int lo, int hi) { return lo + (int)(next_u32() % (uint32_t)(hi - lo + 1)); }

int fails = 0;
long long grouped_items = 0;   // items with more than one member, over all cases
#define CHECK(c, ...)                                   \
  do {                                                  \
    if (!(c)) {                                         \
      std::printf("FAIL line %d: ", __LINE__);          \
      std::printf(__VA_ARGS__);                         \
      std::printf("\n");                                \
      if (++fails > 20) std::exit(1);                   \
    }                                                   \
  } while (0)

constexpr uint32_t kIdMask = (1u << LAZYATTN_ID_BITS) - 1u;

void one_case(int case_no) {
  const int num_seqs = uniform(0, 24);
  const int G = 1 << uniform(0, 5);                 // 1 .. 32 query heads per KV head
  const int Hkv = uniform(1, 4);
  const int Hq = G * Hkv;
  const int n_docs = uniform(1, 6);
  std::vector<int> doc_len(n_docs), doc_base(n_docs);
  int next_id = uniform(0, 1000);
  for (int d = 0; d < n_docs; ++d) {
    doc_len[d] = uniform(1, 40);
    doc_base[d] = next_id;
    next_id += doc_len[d] + uniform(0, 5);
  }
  std::vector<int32_t> q_indptr{0}, block_table{0};
  std::vector<uint32_t> meta;
  for (int s = 0; s < num_seqs; ++s) {
    const int parts = uniform(0, 5);
    for (int k = 0; k < parts; ++k) {
      if (uniform(0, 3) == 0) {                     // private blocks
        const int n = uniform(1, 10);
        for (int i = 0; i < n; ++i) meta.push_back((uint32_t)(next_id++) & kIdMask);
      } else {                                      // a run of a shared document
        const int d = uniform(0, n_docs - 1);
        const int a = uniform(0, doc_len[d] - 1), b = uniform(a, doc_len[d] - 1);
        const uint32_t delta = (uint32_t)uniform(-100, 100) << LAZYATTN_ID_BITS;
        for (int i = a; i <= b; ++i) meta.push_back(((uint32_t)(doc_base[d] + i) & kIdMask) | delta);
      }
    }
    block_table.push_back((int32_t)meta.size());
    q_indptr.push_back(q_indptr.back() + uniform(0, 3));
  }
  const int total_q = q_indptr.back();
  const int single = uniform(0, 1);
  const int max_chunk = uniform(4, 70);
  const int waves = uniform(0, 3) == 0 ? 0 : uniform(1, 600);
  const uint32_t* mp = meta.empty() ? nullptr : meta.data();

  int64_t len = -1;
  int rc = lazyattn_decode_share_plan(q_indptr.data(), block_table.data(), mp, num_seqs,
                                      total_q, Hq, Hkv, single, max_chunk, waves, nullptr, 0,
                                      &len);
  CHECK(rc == LAZYATTN_OK && len >= 9 + total_q, "case %d: size query rc %d len %lld", case_no,
        rc, (long long)len);
  if (rc != LAZYATTN_OK) return;
  if (len > 9) {                                    // too small by one: NOSPACE, length set
    std::vector<int32_t> small((size_t)len - 1);
    int64_t len2 = -1;
    rc = lazyattn_decode_share_plan(q_indptr.data(), block_table.data(), mp, num_seqs, total_q,
                                    Hq, Hkv, single, max_chunk, waves, small.data(),
                                    len - 1, &len2);
    CHECK(rc == LAZYATTN_ERR_NOSPACE && len2 == len, "case %d: short buffer rc %d", case_no, rc);
  }
  std::vector<int32_t> plan((size_t)len);
  int64_t len3 = -1;
  rc = lazyattn_decode_share_plan(q_indptr.data(), block_table.data(), mp, num_seqs, total_q, Hq,
                                  Hkv, single, max_chunk, waves, plan.data(), len, &len3);
  CHECK(rc == LAZYATTN_OK && len3 == len, "case %d: plan rc %d", case_no, rc);
  if (rc != LAZYATTN_OK) return;

  const int M = G <= 16 ? 16 / G : 1, REC = 2 + 4 * M;
  CHECK(plan[0] == 0x5053414C && plan[1] == 2 && plan[2] == M && plan[3] == REC,
        "case %d: header", case_no);
  const int n_items = plan[4], n_slots = plan[5];
  CHECK(plan[6] == total_q && plan[7] == num_seqs, "case %d: header sizes", case_no);
  CHECK((int64_t)len == 8 + total_q + 1 + (int64_t)n_items * REC, "case %d: length", case_no);
  const int32_t* prefix = plan.data() + 8;
  CHECK(prefix[0] == 0 && prefix[total_q] == n_slots, "case %d: prefix ends", case_no);
  std::vector<int> seq_of(total_q > 0 ? total_q : 1, -1);
  for (int s = 0; s < num_seqs; ++s)
    for (int r = q_indptr[s]; r < q_indptr[s + 1]; ++r) seq_of[r] = s;
  std::vector<std::vector<int>> covered(total_q);
  std::vector<std::vector<int>> slots(total_q);
  const int eff_chunk = max_chunk < 128 / M ? max_chunk : 128 / M;
  for (int it = 0; it < n_items; ++it) {
    const int32_t* rec = plan.data() + 8 + total_q + 1 + (size_t)it * REC;
    const int ln = rec[0], nm = rec[1];
    if (nm == 0) {
      CHECK(ln == 0, "case %d: filler item with length %d", case_no, ln);
      continue;
    }
    grouped_items += nm > 1;
    CHECK(nm >= 1 && nm <= M && ln >= 1 && ln <= eff_chunk, "case %d: item %d len %d nm %d",
          case_no, it, ln, nm);
    const int s0 = rec[3], e0 = rec[4];
    for (int k = 0; k < nm && k < M; ++k) {
      const int row = rec[2 + 4 * k], s = rec[3 + 4 * k], e = rec[4 + 4 * k], slot = rec[5 + 4 * k];
      CHECK(row >= 0 && row < total_q && seq_of[row] == s, "case %d: member row", case_no);
      if (!(row >= 0 && row < total_q && seq_of[row] == s)) continue;
      const int T = block_table[s + 1] - block_table[s];
      CHECK(e >= 0 && e + ln <= T, "case %d: member entries", case_no);
      if (!(e >= 0 && e + ln <= T)) continue;
      if (covered[row].empty()) covered[row].assign((size_t)T, 0);
      for (int t = 0; t < ln; ++t) {
        covered[row][(size_t)(e + t)]++;
        const uint32_t a = meta[(size_t)(block_table[s] + e + t)] & kIdMask;
        const uint32_t b = meta[(size_t)(block_table[s0] + e0 + t)] & kIdMask;
        CHECK(a == b, "case %d: member ids differ", case_no);
        CHECK(meta[(size_t)(block_table[s] + e + t)] >> LAZYATTN_ID_BITS ==
                  meta[(size_t)(block_table[s] + e)] >> LAZYATTN_ID_BITS,
              "case %d: member offset delta changes inside an item", case_no);
      }
      slots[row].push_back(slot);
    }
  }
  for (int r = 0; r < total_q; ++r) {
    const int s = seq_of[r];
    const bool planned = !single || q_indptr[s + 1] - q_indptr[s] == 1;
    const int T = block_table[s + 1] - block_table[s];
    if (planned) {
      for (int t = 0; t < T; ++t)
        CHECK(!covered[r].empty() && covered[r][(size_t)t] == 1,
              "case %d: row %d entry %d covered %d times", case_no, r, t,
              covered[r].empty() ? 0 : covered[r][(size_t)t]);
    } else {
      CHECK(covered[r].empty() && prefix[r + 1] == prefix[r], "case %d: unplanned row", case_no);
    }
    std::vector<int> want;
    for (int x = prefix[r]; x < prefix[r + 1]; ++x) want.push_back(x);
    std::vector<int> got = slots[r];
    std::vector<int> sorted(got);
    for (size_t i = 1; i < sorted.size(); ++i)
      for (size_t j = i; j > 0 && sorted[j - 1] > sorted[j]; --j) std::swap(sorted[j - 1], sorted[j]);
    CHECK(sorted == want, "case %d: row %d slots", case_no, r);
  }
}

void error_paths() {
  int32_t qi[2] = {0, 1}, bt[2] = {0, 1};
  uint32_t w[1] = {5};
  int64_t len = 0;
  CHECK(lazyattn_decode_share_plan(nullptr, bt, w, 1, 1, 8, 1, 0, 16, 0, nullptr, 0, &len) ==
            LAZYATTN_ERR_NULL, "null q_indptr");
  CHECK(lazyattn_decode_share_plan(qi, bt, nullptr, 1, 1, 8, 1, 0, 16, 0, nullptr, 0, &len) ==
            LAZYATTN_ERR_NULL, "null words with entries");
  CHECK(lazyattn_decode_share_plan(qi, bt, w, 1, 1, 8, 3, 0, 16, 0, nullptr, 0, &len) ==
            LAZYATTN_ERR_SHAPE, "Hq not a multiple of Hkv");
  CHECK(lazyattn_decode_share_plan(qi, bt, w, 1, 2, 8, 1, 0, 16, 0, nullptr, 0, &len) ==
            LAZYATTN_ERR_SHAPE, "total_q mismatch");
  CHECK(lazyattn_decode_share_plan(qi, bt, w, 1, 1, 8, 1, 0, 3, 0, nullptr, 0, &len) ==
            LAZYATTN_ERR_ARG, "max_chunk below 4");
  CHECK(lazyattn_decode_share_plan(qi, bt, w, 1, 1, 8, 1, 0, 16, -1, nullptr, 0, &len) ==
            LAZYATTN_ERR_ARG, "negative waves");
  int32_t bad[2] = {1, 1};
  CHECK(lazyattn_decode_share_plan(bad, bt, w, 1, 1, 8, 1, 0, 16, 0, nullptr, 0, &len) ==
            LAZYATTN_ERR_SHAPE, "CSR not from 0");
}

}  // namespace

int main(int argc, char** argv) {
  const int cases = argc > 1 ? std::atoi(argv[1]) : 400;
  error_paths();
  for (int c = 0; c < cases; ++c) one_case(c);
  if (fails) {
    std::printf("%d failures\n", fails);
    return 1;
  }
  if (grouped_items == 0) {                        // the layouts must exercise grouping
    std::printf("no grouped item in %d cases\n", cases);
    return 1;
  }
  std::printf("ok (%lld grouped items)\n", grouped_items);
  return 0;
}
