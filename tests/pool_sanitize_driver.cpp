// Randomised driver for the host pool index (csrc/pool.cpp), built by
// tests/test_sanitize_cpu.py with g++ and AddressSanitizer + UndefinedBehaviorSanitizer (the
// single-threaded model check) or ThreadSanitizer (the threaded stress). Exit code 0 and
// "ok" on stdout when every check held.
//
// Model check: a shadow of what the index must guarantee -- documents with a live
// reference keep their blocks (a hit returns the same ids), pinned and private blocks never
// overlap, and free + evictable + pinned + private blocks add up to the pool -- compared
// with lazyattn_pool_stats after every operation. Documents with no reference may be
// evicted at any allocation, so the model only tracks their last block list for the
// hit-returns-same-ids check while they stay cached.
#include "lazyattn.h"

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <set>
#include <thread>
#include <vector>

namespace {

uint64_t rng_state = 0x9E3779B97F4A7C15ull;
uint32_t next_u32() {                     // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
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

constexpr int kBlocks = 200, kB = 16, kDocs = 60;

int32_t doc_tokens(int k) { return kB * (1 + k % 7) - (k % 3); }

struct DocModel {
  std::vector<int32_t> blocks;   // last block list handed out
  int refs = 0;
};

int model_check() {
  void* h = nullptr;
  CHECK(lazyattn_pool_create(0, kB, &h) == LAZYATTN_ERR_ARG, "empty pool accepted");
  CHECK(lazyattn_pool_create(kBlocks, 0, &h) == LAZYATTN_ERR_ARG, "B = 0 accepted");
  CHECK(lazyattn_pool_create(kBlocks, kB, &h) == LAZYATTN_OK && h, "create");
  std::map<int, DocModel> docs;
  std::set<int32_t> priv;
  std::vector<int32_t> buf(64);
  for (int op = 0; op < 40000; ++op) {
    const uint32_t r = next_u32();
    const int k = (int)(next_u32() % kDocs);
    switch (r % 6) {
      case 0:
      case 1: {                                       // acquire
        int32_t n = -1, hit = -1;
        const int cap = (r >> 8) % 16 == 0 ? 1 : 64;  // sometimes too small
        const int rc = lazyattn_pool_acquire(h, (uint64_t)k * 7919u, doc_tokens(k), buf.data(),
                                             cap, &n, &hit);
        const int want_n = (doc_tokens(k) + kB - 1) / kB;
        if (rc == LAZYATTN_ERR_ARG) {
          CHECK(cap < want_n && n == want_n, "ARG with cap %d n %d", cap, n);
          break;
        }
        if (rc == LAZYATTN_ERR_NOSPACE) break;
        CHECK(rc == LAZYATTN_OK, "acquire rc %d", rc);
        CHECK(n == want_n, "acquire n %d want %d", n, want_n);
        DocModel& d = docs[k];
        std::vector<int32_t> got(buf.begin(), buf.begin() + n);
        for (int32_t b : got) {
          CHECK(b >= 0 && b < kBlocks, "block id %d", b);
          CHECK(!priv.count(b), "document block %d is private", b);
        }
        if (d.refs > 0) CHECK(hit == 1 && got == d.blocks, "pinned document not a same-id hit");
        if (hit == 1 && !d.blocks.empty()) CHECK(got == d.blocks, "hit with other ids");
        for (auto& [k2, d2] : docs) {                 // pinned documents stay disjoint
          if (k2 == k || d2.refs == 0) continue;
          for (int32_t b : got)
            for (int32_t b2 : d2.blocks) CHECK(b != b2, "block %d of two live documents", b);
        }
        d.blocks = got;
        d.refs++;
        break;
      }
      case 2:
      case 3: {                                       // release
        DocModel& d = docs[k];
        const int rc = lazyattn_pool_release(h, (uint64_t)k * 7919u);
        if (d.refs > 0) {
          CHECK(rc == LAZYATTN_OK, "release rc %d", rc);
          d.refs--;
        } else {
          CHECK(rc == LAZYATTN_ERR_STATE, "release without reference rc %d", rc);
        }
        break;
      }
      case 4: {                                       // private blocks
        const int n = 1 + (int)(r >> 8) % 4;
        const int rc = lazyattn_pool_alloc_private(h, n, buf.data());
        if (rc == LAZYATTN_ERR_NOSPACE) break;
        CHECK(rc == LAZYATTN_OK, "alloc_private rc %d", rc);
        for (int i = 0; i < n; ++i) {
          CHECK(!priv.count(buf[i]), "private block %d handed out twice", buf[i]);
          for (auto& [k2, d2] : docs)
            for (int32_t b2 : d2.blocks)
              CHECK(d2.refs == 0 || buf[i] != b2, "private block %d of a live document", buf[i]);
          priv.insert(buf[i]);
        }
        break;
      }
      default: {                                      // free private (and a wrong free)
        if (!priv.empty() && (r >> 8) % 2) {
          auto it = priv.begin();
          std::advance(it, (r >> 9) % priv.size());
          const int32_t b = *it;
          CHECK(lazyattn_pool_free_private(h, &b, 1) == LAZYATTN_OK, "free_private");
          priv.erase(it);
          CHECK(lazyattn_pool_free_private(h, &b, 1) == LAZYATTN_ERR_STATE, "double free");
        } else {
          const int32_t b = kBlocks + 3;
          CHECK(lazyattn_pool_free_private(h, &b, 1) == LAZYATTN_ERR_STATE, "free of id past pool");
        }
      }
    }
    LazyattnPoolStats st{};
    CHECK(lazyattn_pool_stats(h, &st) == LAZYATTN_OK, "stats");
    int pinned = 0, pinned_blocks = 0;
    for (auto& [k2, d2] : docs)
      if (d2.refs > 0) {
        pinned++;
        pinned_blocks += (int)d2.blocks.size();
      }
    CHECK(st.num_blocks == kBlocks, "num_blocks");
    CHECK(st.pinned_docs == pinned, "pinned %d model %d", st.pinned_docs, pinned);
    CHECK(st.private_blocks == (int)priv.size(), "private %d model %zu", st.private_blocks,
          priv.size());
    CHECK(st.free_blocks + st.evictable_blocks + pinned_blocks + st.private_blocks == kBlocks,
          "occupancy %d + %d + %d + %d", st.free_blocks, st.evictable_blocks, pinned_blocks,
          st.private_blocks);
  }
  LazyattnPoolStats st{};
  lazyattn_pool_stats(h, &st);
  std::printf("hits %lld misses %lld evictions %lld evicted_blocks %lld\n", (long long)st.hits,
              (long long)st.misses, (long long)st.evictions, (long long)st.evicted_blocks);
  CHECK(st.hits > 0 && st.evictions > 0, "the run exercised no hit or no eviction");
  CHECK(lazyattn_pool_destroy(h) == LAZYATTN_OK, "destroy");
  return fails;
}

// Several threads acquire and release documents and private blocks on one handle; the
// index serialises them. Checks only return codes (the interleaving is not modelled).
int threaded_stress() {
  void* h = nullptr;
  if (lazyattn_pool_create(kBlocks, kB, &h) != LAZYATTN_OK) return 1;
  std::vector<std::thread> ts;
  std::vector<int> bad(4, 0);
  for (int t = 0; t < 4; ++t)
    ts.emplace_back([h, t, &bad] {
      uint64_t s = 0x1234567ull * (t + 1);
      std::vector<int32_t> blocks(64);
      std::vector<int> held;
      for (int i = 0; i < 5000; ++i) {
        s ^= s << 13;
        s ^= s >> 7;
        s ^= s << 17;
        const int k = (int)(s % 40);
        if (s & 0x100) {
          int32_t n, hit;
          const int rc = lazyattn_pool_acquire(h, (uint64_t)k, doc_tokens(k), blocks.data(), 64,
                                               &n, &hit);
          if (rc == LAZYATTN_OK) held.push_back(k);
          else if (rc != LAZYATTN_ERR_NOSPACE) bad[t]++;
        } else if (!held.empty()) {
          if (lazyattn_pool_release(h, (uint64_t)held.back()) != LAZYATTN_OK) bad[t]++;
          held.pop_back();
        }
        if ((s & 0xF000) == 0) {
          if (lazyattn_pool_alloc_private(h, 2, blocks.data()) == LAZYATTN_OK &&
              lazyattn_pool_free_private(h, blocks.data(), 2) != LAZYATTN_OK)
            bad[t]++;
        }
      }
      for (int k : held)
        if (lazyattn_pool_release(h, (uint64_t)k) != LAZYATTN_OK) bad[t]++;
    });
  for (auto& th : ts) th.join();
  LazyattnPoolStats st{};
  lazyattn_pool_stats(h, &st);
  int errs = bad[0] + bad[1] + bad[2] + bad[3];
  if (st.pinned_docs != 0 || st.private_blocks != 0) errs++;
  if (st.free_blocks + st.evictable_blocks != kBlocks) errs++;
  lazyattn_pool_destroy(h);
  if (errs) std::printf("FAIL threaded stress: %d errors\n", errs);
  return errs;
}

}  // namespace

int main(int argc, char** argv) {
  const bool threads = argc > 1 && argv[1][0] == 't';
  const int errs = threads ? threaded_stress() : model_check();
  if (errs == 0) std::printf("ok\n");
  return errs == 0 ? 0 : 1;
}
