// Kernel parameter blocks and launchers (internal to the library).
#pragma once

#include "lazyattn_common.h"

namespace lazyattn {

struct PlanParams {
  const int32_t* q_indptr;
  const int32_t* block_table;
  double* freqs_out;         // [D/2] workspace copy of the frequency table
  int32_t* pf_prefix;        // [num_seqs + 1] prefill tiles
  int32_t* dec_prefix;       // [num_seqs + 1] decode row-splits
  uint32_t* zero;            // 192 bytes set to zero here
  int num_seqs;
  int pos_per_tile;          // query positions per prefill tile
  int bps, smax;             // decode split size (blocks) and splits-per-row cap
  int mode;                  // PlanMode
  int half_dim;
  int pf_smax;               // prefill KV split: splits-per-tile cap (workspace bound)
  int num_cus;               // prefill items fill one round of the GPU at least
  int work_heads;            // KV (work) heads
  int dec_waves;             // resident decode waves (decode split of mixed calls)
  int* pf_kc;                // out: key tiles per split (device-chosen, read by prefill)
  int* dec_bps;              // out: decode split size (mixed calls: device-chosen; else bps)
  RopeFreqs fr;              // host-computed table (kernel argument)
};

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_table;
  const uint32_t* block_meta;
  const int32_t* kv_lens;
  const int32_t* q_indptr;
  const int32_t* q_pos;
  uint16_t* out;
  const int32_t* pf_prefix;  // [num_seqs + 1] prefill items (tiles x KV splits) per sequence
  const uint16_t* zero;      // zero bytes: source of V rows that must read as 0
  int num_seqs, Hq, Hkv, num_blocks;
  int pf_item_cap;           // upper bound of prefill items per KV head (grid / buffer sizing)
  float scale_log2;          // log2(e) / sqrt(D)
  const double* freqs;       // [D/2] RoPE frequencies (revolutions per position)
  const float* slopes;       // [Hq] ALiBi slopes (positional encoding kAlibi only)
  int Hkv_pool, kv_group;    // pool KV heads; work heads per pool head (see below)
  int rot_chunks;            // rotary_dim / 16 (kRopePartial only; nat_chunk)
  const int32_t* stored;     // [entries] stored rotation offset of slot 0 (kDocRotated only)
  int total_q;               // rows of q and out: rows at or past it are never touched
  const int* pf_kc;          // KV split: key tiles per split (written by plan_kernel)
  int pf_smax;               // KV split: splits-per-tile cap (pf_split)
  float* pf_partials;        // [Hkv * pf_item_cap][tile rows][D + 4]: split partials (o, m, l)
};

// More than 16 query heads per KV head (G = 16 S): the kernels run Hkv * S "work heads" of
// 16 query heads each; work head v reads pool head v / S (kv_group = S). Otherwise
// kv_group = 1 and Hkv_pool = Hkv.

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_table;
  const uint32_t* block_meta;
  const int32_t* kv_lens;
  const int32_t* q_indptr;
  const int32_t* q_pos;
  const int32_t* dec_prefix;
  const uint16_t* zero;      // zero bytes: source of V rows that must read as 0
  float* partials;           // [row-splits][Hq][D + 4]
  int num_seqs, Hq, Hkv, num_blocks, bps, smax;
  float scale_log2;
  const double* freqs;
  const float* slopes;       // [Hq] ALiBi slopes (positional encoding kAlibi only)
  int Hkv_pool, kv_group;    // as in PrefillParams
  int rot_chunks;            // as in PrefillParams
  const int32_t* stored;     // as in PrefillParams
  int total_q;               // as in PrefillParams
  int rowsplit_cap;          // row-splits the partial buffer holds; items past it are skipped
};

struct MergeParams {
  const int32_t* q_indptr;
  const int32_t* block_table;
  const int32_t* dec_prefix;
  const float* partials;
  uint16_t* out;
  int num_seqs, Hq;
  const int* bps;            // decode split size (written by plan_kernel)
  int smax, mode;
  int total_q;               // rows of out
  const int32_t* slot_prefix;  // shared-document plan: row r's partials are slots
                               // [slot_prefix[r], slot_prefix[r + 1]) (else null)
  int n_slots;                 // partial slots the plan's workspace holds
  int plan_members;            // rows per plan item this call expects (16 / G, or 1)
};

// One launch for a batch of any query lengths: prefill items (query tiles, KV split) and
// decode chunks (dec_chunk consecutive decode items, one wave per item) on one grid, in
// eight per-XCD queues (prefill items first, then decode chunks).
struct MixedParams {
  PrefillParams pf;          // shared fields (pointers, shapes, tables) and the prefill ones
  const int32_t* dec_prefix; // decode-only fields of DecodeParams
  float* partials;
  const int* bps;            // decode split size (written by plan_kernel)
  int smax, rowsplit_cap;
  int dec_chunk;             // decode items per workgroup (a multiple of its 8 waves)
  const int32_t* plan;       // shared-document plan for the decode rows (or null)
  int plan_items, plan_slots;
};
hipError_t launch_mixed(const MixedParams& p, int D, int G, int pe, hipStream_t st);
// merge of the prefill KV-split partials (launched after the mixed kernel when splits may
// have been taken)
hipError_t launch_pf_merge(const PrefillParams& p, int D, int G, hipStream_t st);

hipError_t launch_plan(const PlanParams& p, hipStream_t st);
hipError_t launch_merge(const MergeParams& p, int total_q, int D, hipStream_t st);
hipError_t launch_debug_decode(const uint32_t* words, const int32_t* bt, int num_seqs, int n,
                               int32_t* ids, int32_t* offs, hipStream_t st);
// query positions per prefill tile (256 (position, head) rows)
int prefill_positions_per_tile(int G);
struct MaterializeParams {
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_table;
  const uint32_t* block_meta;
  const int32_t* kv_lens;
  uint16_t* dst_k;           // [n_entries, Hkv, B, D]
  uint16_t* dst_v;
  uint32_t* dst_meta;        // [n_entries]
  int num_seqs, n_entries, Hkv, num_blocks;
  RopeFreqs fr;              // host-computed table (kernel argument)
};
hipError_t launch_materialize(const MaterializeParams& p, int D, int num_wg, hipStream_t st);

struct IngestParams {
  const uint16_t* k_new;     // [n_tokens][Hkv][D] bf16, as projected (no rotation)
  const uint16_t* v_new;
  const int32_t* slot_mapping;   // [n_tokens] block_id * B + slot, or -1
  uint16_t* k_pool;          // [num_blocks][Hkv][B][D]
  uint16_t* v_pool;
  int n_tokens, Hkv, D, B, num_blocks;
};
hipError_t launch_ingest(const IngestParams& p, int num_wg, hipStream_t st);

hipError_t launch_probe_mfma(int num_cus, int iters, unsigned long long* cyc, float* out,
                             hipStream_t st);
hipError_t launch_probe_read(const void* buf, size_t bytes, int num_wg, uint32_t* out,
                             hipStream_t st);
hipError_t launch_probe_gather(const void* buf, size_t bytes, const int32_t* idx, int n_idx,
                               int chunk_bytes, int num_wg, uint32_t* out, hipStream_t st);

// waves of the decode grid (all resident at once); decode items are dealt round-robin to them,
// one contiguous range of items per XCD
int decode_resident_waves();
hipError_t launch_decode(const DecodeParams& p, int D, int G, int pe, hipStream_t st);
// shared-document decode over a host plan (RoPE mode only)
hipError_t launch_decode_plan(const DecodeParams& p, const int32_t* plan, int n_plan,
                              int n_slots, int D, int G, hipStream_t st);

}  // namespace lazyattn
