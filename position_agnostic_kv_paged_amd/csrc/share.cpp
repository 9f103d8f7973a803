// Host planner of shared-document decode.
//
// Technical summary of LazyAttention (arXiv 2606.04302), "Core Concept" and "Problem
// Statement": cached keys carry no position, so one physical copy of a document's blocks
// serves every request that contains it, at any offset. In a decode batch the same blocks
// therefore sit in many requests' block tables (at different entries and offsets). The
// decode kernel's score and value products take up to 16 columns; with G query heads per KV
// head, 16 / G rows fit side by side. This planner finds runs of blocks that several rows
// read (the same physical block ids at consecutive entries of each row) and makes each such
// run one work item whose rows share the key/value loads; the rest of every row is cut into
// single-row items. Each (item, member row) gets one partial slot; a row's slots are
// consecutive, and the merge folds them.
//
// Plan layout (int32), built here and copied to the device by the caller:
//   [0] magic, [1] version, [2] M = members per item, [3] REC = 2 + 4 M ints per item,
//   [4] n_items, [5] n_slots, [6] total_q, [7] num_seqs,
//   [8 .. 8 + total_q]          row_slot_prefix: row r owns slots [p[r], p[r + 1])
//   then n_items records        {len, n_members, (row, seq, entry_begin, slot) x M}
// Member 0 leads: the item reads blocks entry_begin0 .. entry_begin0 + len - 1 of its
// sequence's table; every member's entries entry_begin_m .. + len - 1 hold the same ids, and
// every member's offset delta is the same over its len entries (its logical offsets advance
// by one block per entry). Items are at most min(max_chunk, 128 / M) blocks long.
#include "lazyattn.h"

#include <algorithm>
#include <cstdint>
#include <vector>

namespace {

constexpr int kMinRun = 4;                   // blocks a shared run must span to be grouped
constexpr uint32_t kIdMask = (1u << LAZYATTN_ID_BITS) - 1u;

struct Row {
  int32_t row, seq, e0, T;
};

}  // namespace

extern "C" int lazyattn_decode_share_plan(const int32_t* q_indptr, const int32_t* block_table,
                                          const uint32_t* block_meta, int32_t num_seqs,
                                          int32_t total_q, int32_t Hq, int32_t Hkv,
                                          int32_t single_row_only, int32_t max_chunk,
                                          int32_t waves, int32_t* plan_out, int64_t plan_cap,
                                          int64_t* plan_len_out) {
  if (!q_indptr || !block_table || !plan_len_out) return LAZYATTN_ERR_NULL;
  if (num_seqs < 0 || total_q < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv) return LAZYATTN_ERR_SHAPE;
  if (max_chunk < kMinRun || waves < 0) return LAZYATTN_ERR_ARG;
  if (q_indptr[0] != 0 || block_table[0] != 0) return LAZYATTN_ERR_SHAPE;
  for (int32_t s = 0; s < num_seqs; ++s)
    if (q_indptr[s + 1] < q_indptr[s] || block_table[s + 1] < block_table[s])
      return LAZYATTN_ERR_SHAPE;
  if (q_indptr[num_seqs] != total_q) return LAZYATTN_ERR_SHAPE;
  if (block_table[num_seqs] > 0 && !block_meta) return LAZYATTN_ERR_NULL;
  const int G = Hq / Hkv;
  const int M = G <= 16 ? 16 / G : 1;          // rows side by side in the 16 columns
  const int REC = 2 + 4 * M;
  // an item's words (length x members) are held in two registers of a wave: at most 128
  max_chunk = std::min(max_chunk, 128 / M);

  // the rows planned: every row of a decode call, or the rows of single-row sequences
  std::vector<Row> rows;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t n = q_indptr[s + 1] - q_indptr[s];
    if (single_row_only && n != 1) continue;
    for (int32_t i = 0; i < n; ++i)
      rows.push_back(Row{q_indptr[s] + i, s, block_table[s], block_table[s + 1] - block_table[s]});
  }
  auto id_of = [&](const Row& r, int32_t e) { return (int32_t)(block_meta[r.e0 + e] & kIdMask); };
  // the offset delta field of an entry's word: within an item it must not change for any
  // member (the kernel scores a group's second block with the first block's rotated query)
  auto delta_of = [&](const Row& r, int32_t e) { return block_meta[r.e0 + e] >> LAZYATTN_ID_BITS; };

  // block id -> (planned row, entry) users, as CSR over the id range, each id's users in
  // ascending (row, entry) order; taken[] flags entries already in an item (flat per row)
  const size_t n_ids = (size_t)kIdMask + 2;
  std::vector<int64_t> row_base(rows.size() + 1, 0);
  for (size_t i = 0; i < rows.size(); ++i) row_base[i + 1] = row_base[i] + rows[i].T;
  const int64_t n_ent = row_base[rows.size()];
  std::vector<int32_t> first(n_ids, 0);
  for (size_t i = 0; i < rows.size(); ++i)
    for (int32_t e = 0; e < rows[i].T; ++e) first[(size_t)id_of(rows[i], e) + 1]++;
  for (size_t k = 1; k < n_ids; ++k) first[k] += first[k - 1];
  std::vector<int32_t> u_row((size_t)n_ent), u_ent((size_t)n_ent);
  {
    std::vector<int32_t> fill(first.begin(), first.end() - 1);
    for (size_t i = 0; i < rows.size(); ++i)
      for (int32_t e = 0; e < rows[i].T; ++e) {
        const int32_t k = fill[(size_t)id_of(rows[i], e)]++;
        u_row[(size_t)k] = (int32_t)i;
        u_ent[(size_t)k] = e;
      }
  }
  std::vector<uint8_t> taken((size_t)n_ent, 0);
  auto is_taken = [&](int32_t i, int32_t e) { return taken[(size_t)(row_base[i] + e)] != 0; };
  // users before cursor[id] are taken (entries never become free again) or belong to rows
  // already planned (an untaken entry of an earlier row found no partner for a run of
  // kMinRun, and runs only shorten as entries are taken): the cursor only moves forward
  std::vector<int32_t> cursor(first.begin(), first.end() - 1);

  struct Member {
    int32_t ri, e;
  };
  struct Item {
    int32_t len;
    std::vector<Member> m;
  };
  std::vector<Item> items;
  // shared runs: for each row in order, each untaken entry looks for up to M - 1 other rows
  // holding the same block at an untaken entry from which at least kMinRun ids agree
  for (int32_t i = 0; M > 1 && i < (int32_t)rows.size(); ++i) {
    const Row& a = rows[i];
    int32_t e = 0;
    while (e < a.T) {
      if (is_taken(i, e)) {
        ++e;
        continue;
      }
      const int32_t id = id_of(a, e);
      int32_t& cur = cursor[(size_t)id];
      const int32_t end = first[(size_t)id + 1];
      while (cur < end && (u_row[(size_t)cur] < i || is_taken(u_row[(size_t)cur], u_ent[(size_t)cur])))
        ++cur;
      std::vector<std::pair<Member, int32_t>> cand;   // (member, run length)
      for (int32_t k = cur; k < end && (int)cand.size() < M - 1; ++k) {
        const int32_t j = u_row[(size_t)k], f = u_ent[(size_t)k];
        if (j <= i || is_taken(j, f)) continue;
        bool dup = false;
        for (const auto& c : cand) dup |= c.first.ri == j;
        if (dup) continue;
        const Row& b = rows[(size_t)j];
        int32_t len = 0;
        while (len < max_chunk && e + len < a.T && f + len < b.T && !is_taken(i, e + len) &&
               !is_taken(j, f + len) && id_of(a, e + len) == id_of(b, f + len) &&
               delta_of(a, e + len) == delta_of(a, e) && delta_of(b, f + len) == delta_of(b, f))
          ++len;
        if (len >= kMinRun) cand.push_back({Member{j, f}, len});
      }
      if (cand.empty()) {
        ++e;
        continue;
      }
      int32_t len = max_chunk;
      for (const auto& c : cand) len = std::min(len, c.second);
      Item it{len, {Member{i, e}}};
      for (const auto& c : cand) it.m.push_back(c.first);
      for (const auto& m : it.m)
        for (int32_t k = 0; k < len; ++k) taken[(size_t)(row_base[m.ri] + m.e + k)] = 1;
      items.push_back(std::move(it));
      e += len;
    }
  }
  // single-row items: each row's untaken entries in runs of at most max_chunk, cut where
  // the offset delta changes
  for (int32_t i = 0; i < (int32_t)rows.size(); ++i) {
    int32_t e = 0;
    while (e < rows[i].T) {
      if (is_taken(i, e)) {
        ++e;
        continue;
      }
      int32_t len = 0;
      while (len < max_chunk && e + len < rows[i].T && !is_taken(i, e + len) &&
             delta_of(rows[i], e + len) == delta_of(rows[i], e))
        ++len;
      items.push_back(Item{len, {Member{i, e}}});
      e += len;
    }
  }

  // Order for the kernel's round-robin dealing (wave-item i runs on wave i mod waves, and
  // each plan item is Hw consecutive wave-items, one per work head): longest items first,
  // each onto the least loaded of the waves / Hw lanes of work, then emitted round by round
  // so that lane k's r-th item lands at position r * lanes + k; lanes with fewer items get
  // empty items (no members). Without a wave count the items keep their order.
  // Items of equal length are dealt in order of their blocks' ids (first, then last id),
  // so that the waves of the chip read neighbouring pool blocks at the same time (a sorted
  // gather runs faster than a random one). Items that read the same run of blocks are also
  // kept on one XCD: lane k's items run on workgroups of XCD class k mod 8 in both decode
  // launches (the standalone kernel deals waves 4 per workgroup with Hw = 8 work heads, the
  // mixed kernel one plan item per workgroup), so the first item of a run fixes a class and
  // the run's later items take the least loaded lane of that class when that costs at most
  // half the item's length in balance. Sorted next to each other they start at about the
  // same time, and the later ones find the blocks in that XCD's L2.
  const int Hw = G <= 16 ? Hkv : Hq / 16;
  const int64_t lanes = waves > 0 ? std::max<int64_t>(1, waves / Hw) : 0;
  if (lanes > 0 && (int64_t)items.size() > 1) {
    const size_t classes = (size_t)std::min<int64_t>(8, lanes);
    auto key = [&](const Item& it) {           // (first id, last id) of the item's blocks
      const Row& r = rows[(size_t)it.m[0].ri];
      return std::make_pair(id_of(r, it.m[0].e), id_of(r, it.m[0].e + it.len - 1));
    };
    std::vector<size_t> order(items.size());
    std::vector<std::pair<int32_t, int32_t>> keys(items.size());
    for (size_t k = 0; k < order.size(); ++k) {
      order[k] = k;
      keys[k] = key(items[k]);
    }
    std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) {
      if (items[a].len != items[b].len) return items[a].len > items[b].len;
      return keys[a] < keys[b];
    });
    std::vector<int64_t> load((size_t)lanes, 0);
    std::vector<std::vector<size_t>> per((size_t)lanes);
    std::pair<int32_t, int32_t> last_key{-1, -1};
    size_t last_class = 0;
    for (size_t k : order) {
      // least loaded lane, ties to the lowest index (a linear scan: lanes is a few hundred)
      size_t best = 0;
      for (size_t x = 1; x < (size_t)lanes; ++x)
        if (load[x] < load[best]) best = x;
      if (keys[k] == last_key) {               // the run's class, if balance allows
        size_t cb = last_class;
        for (size_t x = cb; x < (size_t)lanes; x += classes)
          if (load[x] < load[cb]) cb = x;
        if (2 * (load[cb] - load[best]) <= items[k].len) best = cb;
      }
      last_key = keys[k];
      last_class = best % classes;
      load[best] += items[k].len;
      per[best].push_back(k);
    }
    size_t rounds = 0;
    for (const auto& v : per) rounds = std::max(rounds, v.size());
    std::vector<Item> dealt;
    dealt.reserve(rounds * (size_t)lanes);
    for (size_t r = 0; r < rounds; ++r)
      for (size_t x = 0; x < (size_t)lanes; ++x)
        dealt.push_back(r < per[x].size() ? items[per[x][r]] : Item{0, {}});
    while (!dealt.empty() && dealt.back().m.empty()) dealt.pop_back();
    items.swap(dealt);
  }

  // slots: row-major, in item order within a row
  std::vector<int64_t> nslot((size_t)total_q + 1, 0);
  for (const auto& it : items)
    for (const auto& m : it.m) nslot[(size_t)rows[m.ri].row]++;
  std::vector<int64_t> prefix((size_t)total_q + 1, 0);
  for (int32_t r = 0; r < total_q; ++r) prefix[(size_t)r + 1] = prefix[(size_t)r] + nslot[(size_t)r];
  const int64_t n_slots = prefix[(size_t)total_q];
  const int64_t len_total = 8 + (int64_t)total_q + 1 + (int64_t)items.size() * REC;
  if (n_slots > INT32_MAX || (int64_t)items.size() > INT32_MAX / 2 || len_total > INT32_MAX)
    return LAZYATTN_ERR_SHAPE;
  *plan_len_out = len_total;
  if (!plan_out) return LAZYATTN_OK;           // size query
  if (plan_cap < len_total) return LAZYATTN_ERR_NOSPACE;

  int32_t* p = plan_out;
  p[0] = LAZYATTN_SHARE_PLAN_MAGIC;
  p[1] = LAZYATTN_SHARE_PLAN_VERSION;
  p[2] = M;
  p[3] = REC;
  p[4] = (int32_t)items.size();
  p[5] = (int32_t)n_slots;
  p[6] = total_q;
  p[7] = num_seqs;
  for (int32_t r = 0; r <= total_q; ++r) p[8 + r] = (int32_t)prefix[(size_t)r];
  std::vector<int64_t> next(prefix.begin(), prefix.end() - 1);
  int32_t* rec = p + 8 + total_q + 1;
  for (const auto& it : items) {
    std::fill(rec, rec + REC, 0);
    rec[0] = it.len;
    rec[1] = (int32_t)it.m.size();
    for (size_t k = 0; k < it.m.size(); ++k) {
      const Row& r = rows[(size_t)it.m[k].ri];
      rec[2 + 4 * k] = r.row;
      rec[3 + 4 * k] = r.seq;
      rec[4 + 4 * k] = it.m[k].e;
      rec[5 + 4 * k] = (int32_t)next[(size_t)r.row]++;
    }
    rec += REC;
  }
  return LAZYATTN_OK;
}
