// C ABI of the LazyAttention library: argument validation, RoPE frequency table,
// work sizing and kernel launches. Declarations and contracts: include/lazyattn.h.
#include "lazyattn.h"
#include "lazyattn_common.h"
#include "lazyattn_kernels.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>

using namespace lazyattn;

namespace {


bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool shape_ok(int32_t Hq, int32_t Hkv, int32_t D, int32_t B) {
  if (D != 64 && D != 128) return false;
  if (B != kBlock) return false;
  if (Hkv <= 0 || Hq <= 0 || Hq % Hkv) return false;
  const int G = Hq / Hkv;
  return G == 1 || G == 2 || G == 4 || G == 8 || G % 16 == 0;
}

// Query heads per KV head as the kernels see them: G itself up to 16; G = 16 S splits each
// KV head into S work heads of 16 query heads that read the same pool head.
int work_group(int Hq, int Hkv) { const int G = Hq / Hkv; return G > 16 ? 16 : G; }
int work_heads(int Hq, int Hkv) { return Hq / work_group(Hq, Hkv); }

// Decode split (host): decode_bps for rows_bound rows of about max_entries blocks.
struct DecodeSplit {
  int bps, smax;
};
DecodeSplit decode_split(int rows_bound, int Hkv, int max_entries) {
  const long long T = max_entries > 0 ? max_entries : 1;
  DecodeSplit d;
  d.bps = decode_bps((long long)(rows_bound > 0 ? rows_bound : 1) * Hkv, T,
                     decode_resident_waves());
  d.smax = (int)((T + d.bps - 1) / d.bps);
  return d;
}

// Mixed calls: plan_kernel chooses the decode split from the batch's real decode rows (the
// host sees only num_seqs and the max_entries bound of every sequence); the host bounds
// the splits per row so that the partial buffer holds any such choice.
constexpr int kMixedDecodeMaxSplits = 16;
DecodeSplit mixed_decode_split(int num_seqs, int Hkv, int max_entries) {
  DecodeSplit d = decode_split(num_seqs, Hkv, max_entries);
  const int T = max_entries > 0 ? max_entries : 1;
  d.smax = std::max(d.smax, std::min(kMixedDecodeMaxSplits, (T + 7) / 8));
  return d;
}

// Prefill KV split (mixed calls). Query tiles of 256 (position, head) rows are the natural
// work items; when a batch has too few of them to keep every compute unit busy (one long
// request, say), each tile's key range is cut into splits that run as separate items and
// are merged by the tile's last split. The host cannot see the per-sequence lengths (no
// device reads), so it sizes the split from total_q and the max_entries hint; plan_kernel
// applies the same rule (pf_split) to each sequence's real length.
constexpr int kPfItemsPerCu = 1;    // target prefill items per compute unit (one round)
constexpr int kPfMaxSplits = kMaxPfSplits;
constexpr int kDecChunkWaves = 1;   // decode items per wave in one mixed-kernel claim

struct CallPlan {
  DecodeSplit ds;
  int rows_bound;
  int pf_smax, pf_item_cap;         // prefill KV split bound (mixed calls)
  long long pf_slots;
  WsLayout L;
};

CallPlan plan_call(int mode, int num_seqs, int total_q, int max_entries, int Hq, int Hkv,
                   int D, const DecodeSplit& ds) {
  CallPlan c;
  c.ds = ds;
  c.rows_bound = mode == kPlanDecodeOnly ? total_q : num_seqs;
  c.pf_smax = 1;
  c.pf_item_cap = 0;
  c.pf_slots = 0;
  if (mode == kPlanMixed) {
    // bound of the splits plan_kernel may choose: enough items for one round when the
    // tiles are too few (estimated from total_q)
    const int G = work_group(Hq, Hkv), Hw = work_heads(Hq, Hkv);
    const long long pos = prefill_positions_per_tile(G);
    const long long tiles_est = ((long long)total_q + pos - 1) / pos;
    const long long tiles_bound = tiles_est + num_seqs;
    const long long target = (long long)kPfItemsPerCu * (decode_resident_waves() / 8);
    long long smax = 1;
    if (tiles_est * Hw < target)
      smax = std::max(smax, (target + tiles_est * Hw - 1) / std::max(1ll, tiles_est * Hw));
    c.pf_smax = (int)std::min<long long>(kPfMaxSplits, smax);
    c.pf_item_cap = (int)std::min<long long>(tiles_bound * c.pf_smax, INT32_MAX / 4);
    if (c.pf_smax > 1) c.pf_slots = (long long)Hw * c.pf_item_cap;   // split partials
  }
  c.L = ws_layout(num_seqs, (long long)c.rows_bound * ds.smax, Hq, D, c.pf_slots);
  return c;
}

size_t workspace_for(int mode, int num_seqs, int total_q, int max_entries, int Hq, int Hkv,
                     int D) {
  const DecodeSplit ds = mode == kPlanDecodeOnly
                            ? decode_split(total_q, work_heads(Hq, Hkv), max_entries)
                            : mixed_decode_split(num_seqs, work_heads(Hq, Hkv), max_entries);
  return plan_call(mode, num_seqs, total_q, max_entries, Hq, Hkv, D, ds).L.total;
}

// The split of decode_split, coarsened (longer items, fewer partials) until the workspace
// of a decode call fits `cap` bytes; smax = 0 if even one split per row does not fit.
DecodeSplit decode_split_capped(int num_seqs, int rows_bound, int Hq, int Hkv, int D,
                                int max_entries, size_t cap) {
  DecodeSplit ds = decode_split(rows_bound, work_heads(Hq, Hkv), max_entries);
  const long long T = max_entries > 0 ? max_entries : 1;
  while (ws_layout(num_seqs, (long long)rows_bound * ds.smax, Hq, D).total > cap) {
    if (ds.smax <= 1) {
      ds.smax = 0;
      return ds;
    }
    const long long b = std::min<long long>(2ll * ds.bps, INT32_MAX - 1);
    ds.bps = (int)(b + (b & 1));
    ds.smax = (int)((T + ds.bps - 1) / ds.bps);
  }
  return ds;
}

int run(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
        const uint32_t* block_meta, const int32_t* kv_lens, const int32_t* q_indptr,
        const int32_t* q_positions, double rope_base, int32_t num_seqs, int32_t total_q,
        int32_t Hq, int32_t Hkv, int32_t D, int32_t B, int32_t num_blocks,
        int32_t max_entries, void* out, void* workspace, size_t workspace_bytes,
        void* stream, int mode, int pe, const double* inv_freq = nullptr,
        const float* slopes = nullptr, int rotary_dim = 0,
        const int32_t* stored_offsets = nullptr, bool fit_workspace = false,
        const int32_t* share_plan = nullptr, int32_t plan_items = 0, int32_t plan_slots = 0) {
  if (!q || !k_pool || !v_pool || !block_table || !block_meta || !kv_lens || !q_indptr ||
      !q_positions || !out || !workspace)
    return LAZYATTN_ERR_NULL;
  const bool shared = share_plan != nullptr;  // shared-document decode over a host plan
  if (shared) {
    if (pe != kRope || inv_freq || fit_workspace) return LAZYATTN_ERR_ARG;
    if (plan_items < 0 || plan_slots < 0) return LAZYATTN_ERR_ARG;
    if (!aligned(share_plan, 4)) return LAZYATTN_ERR_ALIGN;
  }
  if (num_seqs < 0 || total_q < 0 || num_blocks < 0 || max_entries < 0 ||
      num_blocks > (1 << kIdBits) || !shape_ok(Hq, Hkv, D, B))
    return LAZYATTN_ERR_SHAPE;
  if (pe == kAlibi) {
    if (!slopes) return LAZYATTN_ERR_NULL;
    if (!aligned(slopes, 4)) return LAZYATTN_ERR_ALIGN;
  } else if (inv_freq) {
    if (!shape_ok(Hq, Hkv, D, B)) return LAZYATTN_ERR_SHAPE;
    for (int k = 0; k < D / 2; ++k)
      if (!(inv_freq[k] >= 0.0) || !std::isfinite(inv_freq[k])) return LAZYATTN_ERR_ARG;
  } else if (!(rope_base > 1.0) || !std::isfinite(rope_base)) {
    return LAZYATTN_ERR_ARG;
  }
  if (pe == kRopePartial && (rotary_dim < 16 || rotary_dim > D || rotary_dim % 16))
    return LAZYATTN_ERR_ARG;
  if (pe == kDocRotated) {
    if (!stored_offsets) return LAZYATTN_ERR_NULL;
    if (!aligned(stored_offsets, 4)) return LAZYATTN_ERR_ALIGN;
  }
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16) ||
      !aligned(workspace, 16) || !aligned(block_table, 4) || !aligned(block_meta, 4) ||
      !aligned(kv_lens, 4) || !aligned(q_indptr, 4) || !aligned(q_positions, 4))
    return LAZYATTN_ERR_ALIGN;
  const int rows_bound = mode == kPlanDecodeOnly ? total_q : num_seqs;
  // fit_workspace: the workspace is a fixed buffer (decode calls), so the split is chosen to
  // fit it
  const DecodeSplit ds =
      fit_workspace
          ? decode_split_capped(num_seqs, rows_bound, Hq, Hkv, D, max_entries, workspace_bytes)
      : mode == kPlanDecodeOnly ? decode_split(rows_bound, work_heads(Hq, Hkv), max_entries)
                                : mixed_decode_split(num_seqs, work_heads(Hq, Hkv), max_entries);
  if (ds.smax <= 0) return LAZYATTN_ERR_WORKSPACE;
  CallPlan cp = plan_call(mode, num_seqs, total_q, max_entries, Hq, Hkv, D, ds);
  if (shared) cp.L = ws_layout(num_seqs, plan_slots, Hq, D, cp.pf_slots);   // a partial per slot
  if (workspace_bytes < cp.L.total) return LAZYATTN_ERR_WORKSPACE;
  if (num_seqs == 0 || total_q == 0) return LAZYATTN_OK;

  hipStream_t st = (hipStream_t)stream;
  const int G = work_group(Hq, Hkv), Hw = work_heads(Hq, Hkv), kv_group = Hw / Hkv;
  const WsLayout& L = cp.L;
  char* ws = (char*)workspace;
  double* freqs = (double*)(ws + L.off_freqs);
  uint32_t* zero = (uint32_t*)(ws + L.off_zero);
  int32_t* pf_prefix = (int32_t*)(ws + L.off_pf_prefix);
  int32_t* dec_prefix = (int32_t*)(ws + L.off_dec_prefix);
  float* partials = (float*)(ws + L.off_partials);
  float* pf_partials = (float*)(ws + L.off_pf_partials);

  // RoPE frequencies in revolutions per position (unused with ALiBi: all zero). Partial
  // rotary: theta_k = base^(-2k/r) for the r/2 rotated pairs, zero for the pass-through
  // pairs of the permuted dim order (nat_chunk).
  RopeFreqs fr{};
  const int r = pe == kRopePartial ? rotary_dim : D;
  for (int k = 0; pe != kAlibi && k < D / 2; ++k)
    fr.f[k] = k < r / 2 ? (inv_freq ? inv_freq[k] : std::pow(rope_base, -2.0 * k / r)) /
                              (2.0 * M_PI)
                        : 0.0;
  const float scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));

  if (mode == kPlanMixed && (long long)cp.pf_item_cap * Hw > INT32_MAX / 2)
    return LAZYATTN_ERR_SHAPE;
  const int ncu = decode_resident_waves() / 8;
  int* pf_kc = (int*)(ws + L.off_zero - 64);                 // the reserved words at 512, 516
  int* dec_bps = pf_kc + 1;
  PlanParams pp{q_indptr, block_table, freqs, pf_prefix, dec_prefix, zero, num_seqs,
                prefill_positions_per_tile(G), ds.bps, ds.smax, mode, D / 2,
                cp.pf_smax, kPfItemsPerCu * ncu, Hw, decode_resident_waves(),
                pf_kc, dec_bps, fr};
  if (launch_plan(pp, st) != hipSuccess) return LAZYATTN_ERR_LAUNCH;

  DecodeParams Dp{(const uint16_t*)q, (const uint16_t*)k_pool, (const uint16_t*)v_pool,
                  block_table, block_meta, kv_lens, q_indptr, q_positions, dec_prefix,
                  (const uint16_t*)zero, partials, num_seqs, Hq, Hw, num_blocks,
                  ds.bps, ds.smax, scale_log2, freqs, slopes, Hkv, kv_group, r / 16,
                  stored_offsets, total_q,
                  (int)std::min<long long>((long long)rows_bound * ds.smax, INT32_MAX)};
  if (mode == kPlanMixed) {
    // prefill tiles and decode chunks of any mix of query lengths: one persistent launch
    PrefillParams P{(const uint16_t*)q, (const uint16_t*)k_pool, (const uint16_t*)v_pool,
                    block_table, block_meta, kv_lens, q_indptr, q_positions,
                    (uint16_t*)out, pf_prefix, (const uint16_t*)zero, num_seqs, Hq, Hw,
                    num_blocks, cp.pf_item_cap, scale_log2, freqs, slopes, Hkv, kv_group,
                    r / 16, stored_offsets, total_q, pf_kc, cp.pf_smax, pf_partials};
    MixedParams Mp{P, dec_prefix, partials, dec_bps, ds.smax, Dp.rowsplit_cap,
                   8 * kDecChunkWaves, share_plan, plan_items, plan_slots};
    if (launch_mixed(Mp, D, G, pe, st) != hipSuccess) return LAZYATTN_ERR_LAUNCH;
    // split tiles: their partials are merged once every split has finished (the launch
    // boundary orders the partial stores before the merge's loads)
    if (cp.pf_smax > 1 && launch_pf_merge(P, D, G, st) != hipSuccess)
      return LAZYATTN_ERR_LAUNCH;
  } else if (shared) {
    if (launch_decode_plan(Dp, share_plan, plan_items, plan_slots, D, G, st) != hipSuccess)
      return LAZYATTN_ERR_LAUNCH;
  } else {
    if (launch_decode(Dp, D, G, pe, st) != hipSuccess) return LAZYATTN_ERR_LAUNCH;
  }
  MergeParams Mp{q_indptr, block_table, dec_prefix, partials, (uint16_t*)out,
                 num_seqs, Hq, dec_bps, ds.smax, mode, total_q,
                 shared ? share_plan + 8 : nullptr, plan_slots, 16 / G};
  if (launch_merge(Mp, total_q, D, st) != hipSuccess) return LAZYATTN_ERR_LAUNCH;
  return LAZYATTN_OK;
}

// ---- the decode entry point that allocates nothing ------------------------------------------
// A fixed device buffer stands in for the workspace (plan prefixes, frequency table, zero
// chunk, split-K partials). Each device that loads the library holds its own copy until the
// process ends. In host code `scratch` names a host-side stand-in, never the device memory:
// its device address comes from hipGetSymbolAddress, once per device, and only that
// address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = (size_t)LAZYATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
static std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];

// Device address of `scratch` on the current device (nullptr if it cannot be had). Host
// threads racing on a device's first call both store the same address.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr)
    return nullptr;
  g_scratch_ptr[dev].store(q, std::memory_order_release);
  return q;
}

}  // namespace

extern "C" {

int lazyattn_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, const uint32_t* block_meta,
                            const int32_t* kv_lens, const int32_t* q_indptr,
                            const int32_t* q_positions, double rope_base, int32_t num_seqs,
                            int32_t total_q, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                            int32_t num_blocks, int32_t max_entries, void* out, void* stream) {
  void* ws = scratch_ptr();
  if (!ws) return LAZYATTN_ERR_LAUNCH;
  return run(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_positions,
             rope_base, num_seqs, total_q, Hq, Hkv, D, B, num_blocks, max_entries, out, ws,
             kNoAllocScratchBytes, stream, kPlanDecodeOnly, kRope, nullptr, nullptr, 0, nullptr,
             true);
}

int lazyattn_prefill(const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_table, const uint32_t* block_meta,
                     const int32_t* kv_lens, const int32_t* q_indptr,
                     const int32_t* q_positions, double rope_base, int32_t num_seqs,
                     int32_t total_q, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                     int32_t num_blocks, int32_t max_entries, void* out, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return run(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_positions,
             rope_base, num_seqs, total_q, Hq, Hkv, D, B, num_blocks, max_entries, out,
             workspace, workspace_bytes, stream, kPlanMixed, kRope);
}

int lazyattn_decode(const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_table, const uint32_t* block_meta,
                    const int32_t* kv_lens, const int32_t* q_indptr,
                    const int32_t* q_positions, double rope_base, int32_t num_seqs,
                    int32_t total_q, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                    int32_t num_blocks, int32_t max_entries, void* out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return run(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_positions,
             rope_base, num_seqs, total_q, Hq, Hkv, D, B, num_blocks, max_entries, out,
             workspace, workspace_bytes, stream, kPlanDecodeOnly, kRope);
}

int lazyattn_decode_shared(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_table, const uint32_t* block_meta,
                           const int32_t* kv_lens, const int32_t* q_indptr,
                           const int32_t* q_positions, double rope_base, int32_t num_seqs,
                           int32_t total_q, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                           int32_t num_blocks, int32_t max_entries, const int32_t* plan,
                           int32_t plan_items, int32_t plan_slots, void* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!plan) return LAZYATTN_ERR_NULL;
  return run(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_positions,
             rope_base, num_seqs, total_q, Hq, Hkv, D, B, num_blocks, max_entries, out,
             workspace, workspace_bytes, stream, kPlanDecodeOnly, kRope, nullptr, nullptr, 0,
             nullptr, false, plan, plan_items, plan_slots);
}

int lazyattn_prefill_shared(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, const uint32_t* block_meta,
                            const int32_t* kv_lens, const int32_t* q_indptr,
                            const int32_t* q_positions, double rope_base, int32_t num_seqs,
                            int32_t total_q, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                            int32_t num_blocks, int32_t max_entries, const int32_t* plan,
                            int32_t plan_items, int32_t plan_slots, void* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan) return LAZYATTN_ERR_NULL;
  return run(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_positions,
             rope_base, num_seqs, total_q, Hq, Hkv, D, B, num_blocks, max_entries, out,
             workspace, workspace_bytes, stream, kPlanMixed, kRope, nullptr, nullptr, 0,
             nullptr, false, plan, plan_items, plan_slots);
}

size_t lazyattn_prefill_shared_workspace_bytes(int32_t num_seqs, int32_t total_q,
                                               int32_t max_entries, int32_t plan_slots,
                                               int32_t Hq, int32_t Hkv, int32_t D) {
  if (num_seqs < 0 || total_q < 0 || max_entries < 0 || plan_slots < 0 ||
      !shape_ok(Hq, Hkv, D, kBlock))
    return 0;
  const DecodeSplit ds = mixed_decode_split(num_seqs, work_heads(Hq, Hkv), max_entries);
  const CallPlan cp = plan_call(kPlanMixed, num_seqs, total_q, max_entries, Hq, Hkv, D, ds);
  return ws_layout(num_seqs, plan_slots, Hq, D, cp.pf_slots).total;
}

size_t lazyattn_decode_shared_workspace_bytes(int32_t num_seqs, int32_t total_q,
                                              int32_t plan_slots, int32_t Hq, int32_t Hkv,
                                              int32_t D) {
  if (num_seqs < 0 || total_q < 0 || plan_slots < 0 || !shape_ok(Hq, Hkv, D, kBlock)) return 0;
  return ws_layout(num_seqs, plan_slots, Hq, D).total;
}

int lazyattn_prefill_rotated_pool(const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_table, const uint32_t* block_meta,
                                  const int32_t* kv_lens, const int32_t* q_indptr,
                                  const int32_t* q_positions, double rope_base,
                                  int32_t num_seqs, int32_t total_q, int32_t Hq, int32_t Hkv,
                                  int32_t D, int32_t B, int32_t num_blocks,
                                  int32_t max_entries, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return run(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_positions,
             rope_base, num_seqs, total_q, Hq, Hkv, D, B, num_blocks, max_entries, out,
             workspace, workspace_bytes, stream, kPlanMixed, kStored);
}

int lazyattn_decode_rotated_pool(const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_table, const uint32_t* block_meta,
                                 const int32_t* kv_lens, const int32_t* q_indptr,
                                 const int32_t* q_positions, double rope_base,
                                 int32_t num_seqs, int32_t total_q, int32_t Hq, int32_t Hkv,
                                 int32_t D, int32_t B, int32_t num_blocks,
                                 int32_t max_entries, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return run(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_positions,
             rope_base, num_seqs, total_q, Hq, Hkv, D, B, num_blocks, max_entries, out,
             workspace, workspace_bytes, stream, kPlanDecodeOnly, kStored);
}

int lazyattn_prefill_freqs(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_table, const uint32_t* block_meta,
                           const int32_t* kv_lens, const int32_t* q_indptr,
                           const int32_t* q_positions, const double* inv_freq,
                           int32_t num_seqs, int32_t total_q, int32_t Hq, int32_t Hkv,
                           int32_t D, int32_t B, int32_t num_blocks, int32_t max_entries,
                           void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!inv_freq) return LAZYATTN_ERR_NULL;
  return run(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_positions, 0.0,
             num_seqs, total_q, Hq, Hkv, D, B, num_blocks, max_entries, out, workspace,
             workspace_bytes, stream, kPlanMixed, kRope, inv_freq);
}

int lazyattn_decode_freqs(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_table, const uint32_t* block_meta,
                          const int32_t* kv_lens, const int32_t* q_indptr,
                          const int32_t* q_positions, const double* inv_freq,
                          int32_t num_seqs, int32_t total_q, int32_t Hq, int32_t Hkv,
                          int32_t D, int32_t B, int32_t num_blocks, int32_t max_entries,
                          void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!inv_freq) return LAZYATTN_ERR_NULL;
  return run(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_positions, 0.0,
             num_seqs, total_q, Hq, Hkv, D, B, num_blocks, max_entries, out, workspace,
             workspace_bytes, stream, kPlanDecodeOnly, kRope, inv_freq);
}

int lazyattn_prefill_alibi(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_table, const uint32_t* block_meta,
                           const int32_t* kv_lens, const int32_t* q_indptr,
                           const int32_t* q_positions, const float* slopes,
                           int32_t num_seqs, int32_t total_q, int32_t Hq, int32_t Hkv,
                           int32_t D, int32_t B, int32_t num_blocks, int32_t max_entries,
                           void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return run(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_positions, 0.0,
             num_seqs, total_q, Hq, Hkv, D, B, num_blocks, max_entries, out, workspace,
             workspace_bytes, stream, kPlanMixed, kAlibi, nullptr, slopes);
}

int lazyattn_decode_alibi(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_table, const uint32_t* block_meta,
                          const int32_t* kv_lens, const int32_t* q_indptr,
                          const int32_t* q_positions, const float* slopes,
                          int32_t num_seqs, int32_t total_q, int32_t Hq, int32_t Hkv,
                          int32_t D, int32_t B, int32_t num_blocks, int32_t max_entries,
                          void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return run(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_positions, 0.0,
             num_seqs, total_q, Hq, Hkv, D, B, num_blocks, max_entries, out, workspace,
             workspace_bytes, stream, kPlanDecodeOnly, kAlibi, nullptr, slopes);
}

int lazyattn_prefill_partial(const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_table, const uint32_t* block_meta,
                             const int32_t* kv_lens, const int32_t* q_indptr,
                             const int32_t* q_positions, double rope_base, int32_t rotary_dim,
                             int32_t num_seqs, int32_t total_q, int32_t Hq, int32_t Hkv,
                             int32_t D, int32_t B, int32_t num_blocks, int32_t max_entries,
                             void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return run(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_positions,
             rope_base, num_seqs, total_q, Hq, Hkv, D, B, num_blocks, max_entries, out,
             workspace, workspace_bytes, stream, kPlanMixed, kRopePartial, nullptr, nullptr,
             rotary_dim);
}

int lazyattn_decode_partial(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, const uint32_t* block_meta,
                            const int32_t* kv_lens, const int32_t* q_indptr,
                            const int32_t* q_positions, double rope_base, int32_t rotary_dim,
                            int32_t num_seqs, int32_t total_q, int32_t Hq, int32_t Hkv,
                            int32_t D, int32_t B, int32_t num_blocks, int32_t max_entries,
                            void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return run(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_positions,
             rope_base, num_seqs, total_q, Hq, Hkv, D, B, num_blocks, max_entries, out,
             workspace, workspace_bytes, stream, kPlanDecodeOnly, kRopePartial, nullptr,
             nullptr, rotary_dim);
}

int lazyattn_prefill_doc_rotated(const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_table, const uint32_t* block_meta,
                                 const int32_t* kv_lens, const int32_t* q_indptr,
                                 const int32_t* q_positions, const int32_t* stored_offsets,
                                 double rope_base, int32_t num_seqs, int32_t total_q,
                                 int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                 int32_t num_blocks, int32_t max_entries, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return run(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_positions,
             rope_base, num_seqs, total_q, Hq, Hkv, D, B, num_blocks, max_entries, out,
             workspace, workspace_bytes, stream, kPlanMixed, kDocRotated, nullptr, nullptr, 0,
             stored_offsets);
}

int lazyattn_decode_doc_rotated(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_table, const uint32_t* block_meta,
                                const int32_t* kv_lens, const int32_t* q_indptr,
                                const int32_t* q_positions, const int32_t* stored_offsets,
                                double rope_base, int32_t num_seqs, int32_t total_q,
                                int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                int32_t num_blocks, int32_t max_entries, void* out,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return run(q, k_pool, v_pool, block_table, block_meta, kv_lens, q_indptr, q_positions,
             rope_base, num_seqs, total_q, Hq, Hkv, D, B, num_blocks, max_entries, out,
             workspace, workspace_bytes, stream, kPlanDecodeOnly, kDocRotated, nullptr,
             nullptr, 0, stored_offsets);
}

size_t lazyattn_prefill_workspace_bytes(int32_t num_seqs, int32_t total_q, int32_t max_entries,
                                        int32_t Hq, int32_t Hkv, int32_t D) {
  if (num_seqs < 0 || total_q < 0 || max_entries < 0 || !shape_ok(Hq, Hkv, D, kBlock)) return 0;
  return workspace_for(kPlanMixed, num_seqs, total_q, max_entries, Hq, Hkv, D);
}

size_t lazyattn_decode_workspace_bytes(int32_t num_seqs, int32_t total_q, int32_t max_entries,
                                       int32_t Hq, int32_t Hkv, int32_t D) {
  if (num_seqs < 0 || total_q < 0 || max_entries < 0 || !shape_ok(Hq, Hkv, D, kBlock)) return 0;
  return workspace_for(kPlanDecodeOnly, num_seqs, total_q, max_entries, Hq, Hkv, D);
}

int lazyattn_materialize_rotated(const void* k_pool, const void* v_pool,
                                 const int32_t* block_table, const uint32_t* block_meta,
                                 const int32_t* kv_lens, double rope_base, int32_t num_seqs,
                                 int32_t n_entries, int32_t Hkv, int32_t D, int32_t B,
                                 int32_t num_blocks, void* dst_k, void* dst_v,
                                 uint32_t* dst_meta, void* stream) {
  if (!k_pool || !v_pool || !block_table || !block_meta || !kv_lens || !dst_k || !dst_v ||
      !dst_meta)
    return LAZYATTN_ERR_NULL;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(dst_k, 16) ||
      !aligned(dst_v, 16) || !aligned(block_table, 4) || !aligned(block_meta, 4) ||
      !aligned(kv_lens, 4) || !aligned(dst_meta, 4))
    return LAZYATTN_ERR_ALIGN;
  if (num_seqs <= 0 || Hkv <= 0 || num_blocks <= 0 || B != kBlock || (D != 64 && D != 128) ||
      n_entries < 0)
    return LAZYATTN_ERR_SHAPE;
  if (n_entries > (int32_t)kIdMask + 1) return LAZYATTN_ERR_RANGE;   // new ids must fit a word
  if (!(rope_base > 1.0)) return LAZYATTN_ERR_ARG;
  MaterializeParams P{(const uint16_t*)k_pool, (const uint16_t*)v_pool, block_table,
                      block_meta, kv_lens, (uint16_t*)dst_k, (uint16_t*)dst_v, dst_meta,
                      num_seqs, n_entries, Hkv, num_blocks, {}};
  for (int k = 0; k < D / 2; ++k)
    P.fr.f[k] = std::pow(rope_base, -2.0 * k / D) / (2.0 * M_PI);
  if (launch_materialize(P, D, 8 * decode_resident_waves() / 8, (hipStream_t)stream) !=
      hipSuccess)
    return LAZYATTN_ERR_LAUNCH;
  return LAZYATTN_OK;
}

int lazyattn_ingest_kv(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                       int32_t n_tokens, int32_t Hkv, int32_t D, int32_t B, int32_t num_blocks,
                       void* k_pool, void* v_pool, void* stream) {
  if (n_tokens < 0 || Hkv <= 0 || num_blocks <= 0) return LAZYATTN_ERR_SHAPE;
  if ((D != 64 && D != 128) || B != kBlock) return LAZYATTN_ERR_SHAPE;
  if (n_tokens == 0) return LAZYATTN_OK;
  if (!k_new || !v_new || !slot_mapping || !k_pool || !v_pool) return LAZYATTN_ERR_NULL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pool, 16) ||
      !aligned(v_pool, 16) || !aligned(slot_mapping, 4))
    return LAZYATTN_ERR_ALIGN;
  IngestParams p{(const uint16_t*)k_new, (const uint16_t*)v_new, slot_mapping,
                 (uint16_t*)k_pool, (uint16_t*)v_pool, n_tokens, Hkv, D, B, num_blocks};
  const long long chunks = (long long)n_tokens * Hkv * (D / 8);
  const long long want = (chunks + 255) / 256;
  const int cap = 8 * (decode_resident_waves() / 8) * 4;      // 4 x (8 workgroups per CU)
  const int num_wg = (int)(want < cap ? want : cap);
  if (launch_ingest(p, num_wg, (hipStream_t)stream) != hipSuccess) return LAZYATTN_ERR_LAUNCH;
  return LAZYATTN_OK;
}

int32_t lazyattn_probe_cus(void) { return decode_resident_waves() / 8; }

int lazyattn_probe_mfma(int32_t iters, void* cycles_out, void* scratch_out, void* stream) {
  if (!cycles_out || !scratch_out) return LAZYATTN_ERR_NULL;
  if (!aligned(cycles_out, 8) || !aligned(scratch_out, 4)) return LAZYATTN_ERR_ALIGN;
  if (iters <= 0) return LAZYATTN_ERR_ARG;
  if (launch_probe_mfma(lazyattn_probe_cus(), iters, (unsigned long long*)cycles_out,
                        (float*)scratch_out, (hipStream_t)stream) != hipSuccess)
    return LAZYATTN_ERR_LAUNCH;
  return LAZYATTN_OK;
}

int lazyattn_probe_read(const void* buf, size_t bytes, void* scratch_out, void* stream) {
  if (!buf || !scratch_out) return LAZYATTN_ERR_NULL;
  if (!aligned(buf, 16) || !aligned(scratch_out, 4)) return LAZYATTN_ERR_ALIGN;
  if (bytes == 0 || bytes % 16) return LAZYATTN_ERR_SHAPE;
  if (launch_probe_read(buf, bytes, 8 * lazyattn_probe_cus(), (uint32_t*)scratch_out,
                        (hipStream_t)stream) != hipSuccess)
    return LAZYATTN_ERR_LAUNCH;
  return LAZYATTN_OK;
}

int lazyattn_probe_gather(const void* buf, size_t bytes, const int32_t* chunk_ids,
                          int32_t n_ids, int32_t chunk_bytes, void* scratch_out, void* stream) {
  if (!buf || !chunk_ids || !scratch_out) return LAZYATTN_ERR_NULL;
  if (!aligned(buf, 16) || !aligned(chunk_ids, 4) || !aligned(scratch_out, 4))
    return LAZYATTN_ERR_ALIGN;
  if (n_ids < 0 || chunk_bytes <= 0 || chunk_bytes % 1024 || bytes < (size_t)chunk_bytes ||
      bytes / (size_t)chunk_bytes > (size_t)INT32_MAX)
    return LAZYATTN_ERR_SHAPE;
  if (n_ids == 0) return LAZYATTN_OK;
  if (launch_probe_gather(buf, bytes, chunk_ids, n_ids, chunk_bytes, 8 * lazyattn_probe_cus(),
                          (uint32_t*)scratch_out, (hipStream_t)stream) != hipSuccess)
    return LAZYATTN_ERR_LAUNCH;
  return LAZYATTN_OK;
}

int lazyattn_debug_decode_meta(const uint32_t* words, const int32_t* block_table,
                               int32_t num_seqs, int32_t n_entries, int32_t B,
                               int32_t* ids_out, int32_t* offsets_out, void* stream) {
  if (!words || !block_table || !ids_out || !offsets_out) return LAZYATTN_ERR_NULL;
  if (num_seqs <= 0 || n_entries < 0 || B != kBlock) return LAZYATTN_ERR_SHAPE;
  if (launch_debug_decode(words, block_table, num_seqs, n_entries, ids_out, offsets_out,
                          (hipStream_t)stream) != hipSuccess)
    return LAZYATTN_ERR_LAUNCH;
  return LAZYATTN_OK;
}

}  // extern "C"
