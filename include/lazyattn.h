/*
 * lazyattn.h -- C ABI of the LazyAttention library for AMD Instinct MI355X (gfx950).
 *
 * LazyAttention (Xia, Pamnani, Fang, Chockchowwat, Park, "LazyAttention: Efficient
 * Retrieval-Augmented Generation with Deferred Positional Encoding", arXiv 2606.04302)
 * keeps a KV cache whose keys carry NO positional encoding, so one physical copy of a
 * document's KV blocks can back many logical requests at arbitrary positions (abstract;
 * technical summary, "Core Concept: Deferred Positional Encoding"). RoPE is applied inside
 * the attention kernels while scores are computed. The technical summary's "Technical
 * Implementation" section describes the two kernels this library provides:
 *   - prefill (compute-bound): cached KV blocks are loaded and each key tile receives ONE
 *     relative rotation per query tile, from the query-to-document offset;
 *   - decode (M = 1, bandwidth-bound): the rotation is fused into the inner loop, the query
 *     is re-rotated only when the relative offset changes (a new document), and block id
 *     and offset are bit-packed in one 32-bit word.
 * "Mathematical Equivalence": the result equals attention over materialised copies whose
 * keys carry RoPE at their absolute logical positions.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Device pointers are owned by the caller; the library never allocates, frees or keeps
 *    them. Compute calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL
 *    is the default stream) and never read device memory on the host, so argument checks
 *    are limited to pointers, alignment and scalar sizes.
 *  - bf16 is IEEE-754 binary32 truncated to its upper 16 bits (round to nearest even).
 *  - Supported shapes: head dim D in {64, 128}; block size B = 16 tokens; Hq % Hkv == 0 with
 *    G = Hq / Hkv in {1, 2, 4, 8} or a multiple of 16 (16, 32, 48, 64, ...: MQA-style
 *    groups); rope_base > 1.
 *  - RoPE: rotate-half pairing (dim k with k + D/2), angle n * theta_k,
 *    theta_k = rope_base^(-2k/D); softmax scale 1/sqrt(D).
 *  - Query head h reads key/value head floor(h / G).
 *  - Causality is on LOGICAL positions: key at position L is visible to a query at p iff
 *    L <= p. A query with no visible key outputs zeros.
 *  - Return value: LAZYATTN_OK (0) or a negative LAZYATTN_ERR_* code; no exception, abort
 *    or other failure leaves the ABI.
 *  - Row arrays: q_indptr must be non-decreasing with q_indptr[0] = 0 and
 *    q_indptr[num_seqs] = total_q. Rows the table places at or past total_q are neither
 *    read nor written, and no partial buffer is written past its size, but their outputs
 *    are then missing: such a call is a caller error the library cannot see (it never reads
 *    device memory on the host).
 *  - Operand range. Rotated queries and keys enter the score products as fp16 (11-bit
 *    significands, 3 more than bf16, at the same matrix-core rate), so every rotate-half
 *    pair (x_k, x_{k+D/2}) of a key must have Euclidean norm below 65504 (then every rotated
 *    element is representable); so must every pair of a query row scaled by log2(e)/sqrt(D)
 *    in the prefill kernel, and of the unscaled query row in the decode kernel. The prefill
 *    kernel keeps its running score maximum (log2 domain, q.k log2(e)/sqrt(D)) as 256 times
 *    an fp16 value: scores must stay below about 1.6e7 in magnitude. Values past these
 *    bounds become inf and the affected rows NaN; bf16 inputs can exceed them, real model
 *    activations (|x| < ~1e3) do not. Probabilities multiply bf16 values in P.V; sums,
 *    maxima and accumulators are fp32.
 */
#ifndef LAZYATTN_H
#define LAZYATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LAZYATTN_OK             0
#define LAZYATTN_ERR_NULL      -1  /* a required pointer is NULL */
#define LAZYATTN_ERR_ALIGN     -2  /* q / pools / out / workspace not 16-byte aligned */
#define LAZYATTN_ERR_SHAPE     -3  /* unsupported D, B, G, or negative / inconsistent sizes */
#define LAZYATTN_ERR_RANGE     -4  /* encoder: block id >= 2^17 or offset delta outside 15 bits */
#define LAZYATTN_ERR_WORKSPACE -5  /* workspace smaller than the matching *_workspace_bytes */
#define LAZYATTN_ERR_LAUNCH    -6  /* a kernel launch failed (hipGetLastError after launch) */
#define LAZYATTN_ERR_ARG       -7  /* other invalid scalar argument (rope_base, counts) */
#define LAZYATTN_ERR_NOSPACE   -8  /* pool index: not enough free or evictable blocks */
#define LAZYATTN_ERR_STATE     -9  /* pool index: unknown document, reference underflow, block not owned */

/*
 * Packed block metadata word (one per block-table entry).
 *   bits [16:0]  physical block id            0 .. 131071
 *   bits [31:17] delta = offset - t * B        15-bit two's complement, -16384 .. 16383
 * t is the entry's index inside its own sequence and offset the logical position of the
 * block's slot 0, so slot j of entry t sits at logical position t*B + delta + j. delta is
 * constant across blocks placed back-to-back, so it changes exactly at document
 * boundaries (where the decode kernel re-anchors its rotated query). The summary only
 * says (block ID, offset) are bit-packed into a single register; this layout is the
 * library's own, chosen because 17 id bits (~128k-block pools) plus an absolute 16-bit
 * position would need 33 bits.
 */
#define LAZYATTN_ID_BITS    17
#define LAZYATTN_DELTA_BITS 15

/*
 * lazyattn_prefill -- attention for a batch of sequences with any number of query rows
 * (technical summary, "Technical Implementation", prefilling phase).
 *
 *  q           bf16 [total_q, Hq, D], contiguous (un-rotated queries)
 *  k_pool      bf16 [num_blocks, Hkv, B, D] UN-ROTATED keys (position-free pool)
 *  v_pool      bf16 [num_blocks, Hkv, B, D]
 *  block_table int32 [num_seqs + 1]: CSR row pointers into block_meta; sequence s owns
 *              entries block_table[s] .. block_table[s+1]-1 (T_s entries, in any order)
 *  block_meta  uint32 [block_table[num_seqs]] packed words (see above)
 *  kv_lens     int32 [num_seqs]: keys of sequence s; (T_s-1)*B < kv_lens[s] <= T_s*B, i.e.
 *              only a sequence's LAST entry may be partial; its unused slots are never read
 *              into the result (they may hold NaN)
 *  q_indptr    int32 [num_seqs + 1]: CSR rows of q per sequence (q_len_s >= 0; mixed OK)
 *  q_positions int32 [total_q]: logical position of each query row
 *  rope_base   RoPE base (e.g. 10000.0)
 *  max_entries an upper bound on T_s used to size split-K work (a wrong bound costs
 *              balance, never memory safety)
 *  out         bf16 [total_q, Hq, D]; every row is written
 *  workspace   device scratch of at least lazyattn_prefill_workspace_bytes(...) bytes,
 *              16-byte aligned; its contents on entry do not matter; concurrent calls must
 *              not share one workspace
 *
 * Sequences with q_len_s > 1 run the tiled prefill kernel (one relative key rotation per
 * query tile); sequences with q_len_s == 1 run the split-K decode kernel and a merge, all
 * inside this call, so a continuous batch mixing prefill and decode requests is one call.
 */
int lazyattn_prefill(const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_table, const uint32_t* block_meta,
                     const int32_t* kv_lens, const int32_t* q_indptr,
                     const int32_t* q_positions, double rope_base,
                     int32_t num_seqs, int32_t total_q, int32_t Hq, int32_t Hkv, int32_t D,
                     int32_t B, int32_t num_blocks, int32_t max_entries,
                     void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * lazyattn_decode -- same arguments and result as lazyattn_prefill, executed entirely by
 * the split-K decode kernel (technical summary, "Technical Implementation", decoding
 * phase): every query row is an M = 1 problem; the query is re-rotated only where the
 * offset delta changes. Intended for q_len_s == 1; larger q_len_s are computed correctly,
 * row by row. Workspace: lazyattn_decode_workspace_bytes(...).
 */
int lazyattn_decode(const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_table, const uint32_t* block_meta,
                    const int32_t* kv_lens, const int32_t* q_indptr,
                    const int32_t* q_positions, double rope_base,
                    int32_t num_seqs, int32_t total_q, int32_t Hq, int32_t Hkv, int32_t D,
                    int32_t B, int32_t num_blocks, int32_t max_entries,
                    void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Shared-document decode (technical summary, "Core Concept": cached keys carry no position,
 * so one physical copy of a document's blocks serves every request that contains it).
 *
 * lazyattn_decode_share_plan -- HOST function. From host copies of a decode batch's tables
 * it finds runs of blocks that several query rows read (the same block ids at consecutive
 * entries, at least 4 blocks) and groups up to M = 16 / G rows (G = Hq / Hkv; M = 1 for
 * G = 16 and above) into one work item that loads each block once; the remaining entries
 * of every row become single-row items of at most max_chunk blocks (grouped runs are also
 * cut at max_chunk). Every item is also cut where a member's offset delta changes, so
 * inside an item each member's logical offsets advance by one block per entry (the kernel
 * relies on it). single_row_only = 1 plans only the rows of sequences with one query
 * row (the decode rows of a mixed batch), 0 plans every row.
 *  q_indptr, block_table  int32 [num_seqs + 1] (host), as for the attention calls
 *  block_meta             uint32 [block_table[num_seqs]] (host) packed words
 *  max_chunk              blocks per item, at most (>= 4; items are also at most 128 / M
 *                         blocks long)
 *  waves                  resident decode waves of the device (8 per compute unit; 0: keep
 *                         the items in planning order). The kernel deals item i to wave
 *                         i mod waves; the planner puts the longest items first on the least
 *                         loaded waves and pads with empty items (no members) to balance them.
 *                         Items of equal length go in order of their block ids, and items
 *                         reading the same run of blocks onto waves of one XCD, balance
 *                         permitting (the order changes speed and rounding order only)
 *  plan_out               int32 [plan_cap] or NULL (size query); *plan_len_out receives the
 *                         plan's length in int32 either way
 * The plan (int32): [0] magic LAZYATTN_SHARE_PLAN_MAGIC, [1] version
 * LAZYATTN_SHARE_PLAN_VERSION, [2] M, [3] 2 + 4 M, [4] items, [5] partial slots, [6]
 * total_q, [7] num_seqs, then total_q + 1 slot offsets (row r owns slots
 * [p[r], p[r + 1])), then one record per item: length in blocks, member count, and per
 * member (query row, sequence, first entry, slot); member 0's entries supply the block ids.
 * Errors: NULL, SHAPE (tables not non-decreasing from 0, q_indptr[num_seqs] != total_q,
 * Hq % Hkv), ARG (max_chunk < 4, waves < 0), NOSPACE (plan_cap too small; *plan_len_out is
 * set).
 *
 * lazyattn_decode_shared -- lazyattn_decode (RoPE) over such a plan, copied to device
 * memory (plan: int32, 4-byte aligned) together with its item and slot counts from the
 * header. The plan must have been built from the same block table, block_meta and q_indptr;
 * a plan whose header does not match the call (magic, version, M, total_q, num_seqs)
 * produces zero rows, and indices inside it are clamped to the call's arrays. Workspace:
 * lazyattn_decode_shared_workspace_bytes(num_seqs, total_q, plan_slots, Hq, Hkv, D).
 * Errors as lazyattn_decode, plus NULL plan and ARG for negative counts.
 *
 * lazyattn_prefill_shared -- lazyattn_prefill (RoPE) with the decode rows of the batch (the
 * rows of single-row sequences) run over a plan built with single_row_only = 1; the prefill
 * rows are computed as by lazyattn_prefill. Workspace:
 * lazyattn_prefill_shared_workspace_bytes(num_seqs, total_q, max_entries, plan_slots, Hq,
 * Hkv, D).
 */
#define LAZYATTN_SHARE_PLAN_MAGIC   0x5053414C  /* "LASP" */
#define LAZYATTN_SHARE_PLAN_VERSION 2           /* 2: one offset delta per member and item */
int lazyattn_decode_share_plan(const int32_t* q_indptr, const int32_t* block_table,
                               const uint32_t* block_meta, int32_t num_seqs, int32_t total_q,
                               int32_t Hq, int32_t Hkv, int32_t single_row_only,
                               int32_t max_chunk, int32_t waves, int32_t* plan_out,
                               int64_t plan_cap, int64_t* plan_len_out);
int lazyattn_decode_shared(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_table, const uint32_t* block_meta,
                           const int32_t* kv_lens, const int32_t* q_indptr,
                           const int32_t* q_positions, double rope_base, int32_t num_seqs,
                           int32_t total_q, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                           int32_t num_blocks, int32_t max_entries, const int32_t* plan,
                           int32_t plan_items, int32_t plan_slots, void* out, void* workspace,
                           size_t workspace_bytes, void* stream);
size_t lazyattn_decode_shared_workspace_bytes(int32_t num_seqs, int32_t total_q,
                                              int32_t plan_slots, int32_t Hq, int32_t Hkv,
                                              int32_t D);
int lazyattn_prefill_shared(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, const uint32_t* block_meta,
                            const int32_t* kv_lens, const int32_t* q_indptr,
                            const int32_t* q_positions, double rope_base, int32_t num_seqs,
                            int32_t total_q, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                            int32_t num_blocks, int32_t max_entries, const int32_t* plan,
                            int32_t plan_items, int32_t plan_slots, void* out,
                            void* workspace, size_t workspace_bytes, void* stream);
size_t lazyattn_prefill_shared_workspace_bytes(int32_t num_seqs, int32_t total_q,
                                               int32_t max_entries, int32_t plan_slots,
                                               int32_t Hq, int32_t Hkv, int32_t D);

/*
 * lazyattn_decode_noalloc -- lazyattn_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * same arguments, result and errors, minus the workspace. The split-K partials, plan
 * prefixes and frequency table live in a fixed device buffer of
 * LAZYATTN_NOALLOC_SCRATCH_BYTES inside the library, one per device, held until the process
 * ends; nothing is allocated or freed by the call. The split is coarsened when the batch's
 * partials would not fit (longer items, same result); a batch whose partials do not fit
 * even with one split per row (about total_q * Hq * (D + 4) * 4 bytes plus 8 bytes per
 * sequence and 1 KB) returns LAZYATTN_ERR_WORKSPACE before any launch. Every call on a
 * device shares that device's buffer: calls that overlap on one device (two streams, or two
 * host threads) race and must be serialised by the caller. The stream must belong to the
 * current device. Returns LAZYATTN_ERR_LAUNCH if the buffer's device address cannot be had.
 */
#define LAZYATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
int lazyattn_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, const uint32_t* block_meta,
                            const int32_t* kv_lens, const int32_t* q_indptr,
                            const int32_t* q_positions, double rope_base, int32_t num_seqs,
                            int32_t total_q, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                            int32_t num_blocks, int32_t max_entries, void* out, void* stream);

/*
 * lazyattn_prefill_rotated_pool / lazyattn_decode_rotated_pool -- the materialised baseline
 * the method is measured against (technical summary: "Mathematical Equivalence"; the
 * "rotate keys twice" copy it avoids). Same arguments, layouts, workspace sizes and errors as
 * lazyattn_prefill / lazyattn_decode, but k_pool must hold keys ALREADY rotated to the
 * absolute logical position they are referenced at (slot j of entry t holds R(off_t + j) k),
 * so each block can serve only one position; queries are rotated by R(p) and keys are used
 * as stored -- plain paged RoPE attention. Same kernels with the per-tile key rotation
 * (prefill) and the per-slot key rotation and query re-anchoring (decode) compiled out; the
 * pair measures what the deferred rotation costs.
 */
int lazyattn_prefill_rotated_pool(const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_table, const uint32_t* block_meta,
                                  const int32_t* kv_lens, const int32_t* q_indptr,
                                  const int32_t* q_positions, double rope_base,
                                  int32_t num_seqs, int32_t total_q, int32_t Hq, int32_t Hkv,
                                  int32_t D, int32_t B, int32_t num_blocks,
                                  int32_t max_entries, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream);
int lazyattn_decode_rotated_pool(const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_table, const uint32_t* block_meta,
                                 const int32_t* kv_lens, const int32_t* q_indptr,
                                 const int32_t* q_positions, double rope_base,
                                 int32_t num_seqs, int32_t total_q, int32_t Hq, int32_t Hkv,
                                 int32_t D, int32_t B, int32_t num_blocks,
                                 int32_t max_entries, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * lazyattn_prefill_freqs / lazyattn_decode_freqs -- the same calls with the RoPE frequency of
 * every rotate-half pair given instead of derived from a base: inv_freq is a HOST array of
 * D/2 doubles, theta_k in radians per position for the pair (k, k + D/2), each finite and
 * >= 0 (0 leaves that pair unrotated). Covers frequency-scaled RoPE variants (technical
 * summary, "Key Contributions": compatibility with RoPE variants), e.g. Llama-3.1's scaled
 * table, position interpolation (theta_k / s), other bases. Read during the call only; the
 * device work is the same. Errors as lazyattn_prefill / lazyattn_decode (NULL if inv_freq
 * is NULL, ARG for a negative or non-finite entry).
 */
int lazyattn_prefill_freqs(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_table, const uint32_t* block_meta,
                           const int32_t* kv_lens, const int32_t* q_indptr,
                           const int32_t* q_positions, const double* inv_freq,
                           int32_t num_seqs, int32_t total_q, int32_t Hq, int32_t Hkv,
                           int32_t D, int32_t B, int32_t num_blocks, int32_t max_entries,
                           void* out, void* workspace, size_t workspace_bytes, void* stream);
int lazyattn_decode_freqs(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_table, const uint32_t* block_meta,
                          const int32_t* kv_lens, const int32_t* q_indptr,
                          const int32_t* q_positions, const double* inv_freq,
                          int32_t num_seqs, int32_t total_q, int32_t Hq, int32_t Hkv,
                          int32_t D, int32_t B, int32_t num_blocks, int32_t max_entries,
                          void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * lazyattn_prefill_partial / lazyattn_decode_partial -- the same calls with partial rotary
 * RoPE (technical summary, "Key Contributions": compatibility with RoPE variants): only the
 * first rotary_dim dims of q and k are rotated, rotate-half inside them (dim k paired with
 * k + rotary_dim/2, theta_k = rope_base^(-2k / rotary_dim), k < rotary_dim/2); dims
 * rotary_dim .. D-1 enter the scores unrotated. This is the convention of GPT-NeoX-style
 * models with a rotary fraction below 1. q and the pool keep the natural dim order; the
 * softmax scale stays 1/sqrt(D). rotary_dim must be a multiple of 16 in [16, D]
 * (LAZYATTN_ERR_ARG otherwise); rotary_dim = D gives lazyattn_prefill / lazyattn_decode.
 * Other arguments, ownership and errors as lazyattn_prefill / lazyattn_decode.
 */
int lazyattn_prefill_partial(const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_table, const uint32_t* block_meta,
                             const int32_t* kv_lens, const int32_t* q_indptr,
                             const int32_t* q_positions, double rope_base, int32_t rotary_dim,
                             int32_t num_seqs, int32_t total_q, int32_t Hq, int32_t Hkv,
                             int32_t D, int32_t B, int32_t num_blocks, int32_t max_entries,
                             void* out, void* workspace, size_t workspace_bytes, void* stream);
int lazyattn_decode_partial(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, const uint32_t* block_meta,
                            const int32_t* kv_lens, const int32_t* q_indptr,
                            const int32_t* q_positions, double rope_base, int32_t rotary_dim,
                            int32_t num_seqs, int32_t total_q, int32_t Hq, int32_t Hkv,
                            int32_t D, int32_t B, int32_t num_blocks, int32_t max_entries,
                            void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * lazyattn_prefill_doc_rotated / lazyattn_decode_doc_rotated -- the same calls over a pool
 * whose keys already carry RoPE at a STORED position, typically their position inside their
 * document as a model produced them when it encoded the document alone (technical summary,
 * "Technical Implementation": a cached key is rotated once by the difference between where
 * it was encoded and where it is used, and decode re-rotates the query only at a new
 * document). stored_offsets: DEVICE int32 [block_table[num_seqs]], caller-owned, one per
 * block-table entry: the position at which slot 0 of that entry's block was rotated when
 * stored (slot j at stored_offsets[e] + j; 16 b for the b-th block of a document encoded from
 * position 0). The key of entry e, slot j, is used as R(off_e - stored_offsets[e]) times the
 * stored key, which equals R(L) k for the key k before rotation; the logical offsets of the
 * packed words still decide causality. With stored_offsets[e] = off_e the call is the
 * materialised baseline. Decode applies no per-key rotation: q' = R(p - off_e +
 * stored_offsets[e]) q is recomputed only where off_e - stored_offsets[e] changes. Errors as
 * lazyattn_prefill / lazyattn_decode (NULL if stored_offsets is NULL, ALIGN if it is not
 * 4-byte aligned).
 */
int lazyattn_prefill_doc_rotated(const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_table, const uint32_t* block_meta,
                                 const int32_t* kv_lens, const int32_t* q_indptr,
                                 const int32_t* q_positions, const int32_t* stored_offsets,
                                 double rope_base, int32_t num_seqs, int32_t total_q,
                                 int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                 int32_t num_blocks, int32_t max_entries, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream);
int lazyattn_decode_doc_rotated(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_table, const uint32_t* block_meta,
                                const int32_t* kv_lens, const int32_t* q_indptr,
                                const int32_t* q_positions, const int32_t* stored_offsets,
                                double rope_base, int32_t num_seqs, int32_t total_q,
                                int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                int32_t num_blocks, int32_t max_entries, void* out,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * lazyattn_prefill_alibi / lazyattn_decode_alibi -- the same calls over the same
 * position-free pool with ALiBi instead of RoPE (technical summary, "Key Contributions":
 * compatibility with ALiBi). Nothing is rotated; a query of head h at logical position p
 * scores key slot j of entry t (logical position L = off_t + j from the packed word) as
 *   q . k / sqrt(D) - slopes[h] * (p - L),
 * with the same causal rule (L <= p), softmax and output. slopes: DEVICE float32 [Hq],
 * caller-owned (e.g. Press et al.'s 2^(-8 i / H)). The bias is computed in fp32 (prefill
 * carries slope * log2(e) for the part within a block, at most 15 slots, as the sum of two
 * fp16 values on the matrix cores). Errors as lazyattn_prefill /
 * lazyattn_decode (NULL if slopes is NULL, ALIGN if it is not 4-byte aligned); rope_base is
 * not an argument.
 */
int lazyattn_prefill_alibi(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_table, const uint32_t* block_meta,
                           const int32_t* kv_lens, const int32_t* q_indptr,
                           const int32_t* q_positions, const float* slopes,
                           int32_t num_seqs, int32_t total_q, int32_t Hq, int32_t Hkv,
                           int32_t D, int32_t B, int32_t num_blocks, int32_t max_entries,
                           void* out, void* workspace, size_t workspace_bytes, void* stream);
int lazyattn_decode_alibi(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_table, const uint32_t* block_meta,
                          const int32_t* kv_lens, const int32_t* q_indptr,
                          const int32_t* q_positions, const float* slopes,
                          int32_t num_seqs, int32_t total_q, int32_t Hq, int32_t Hkv,
                          int32_t D, int32_t B, int32_t num_blocks, int32_t max_entries,
                          void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * lazyattn_materialize_rotated -- the position-adjusted copy the method avoids (technical
 * summary: "Mathematical Equivalence"; reuse schemes that store rotated copies), for
 * measurement. For every block-table entry e (flat index, e < min(n_entries,
 * block_table[num_seqs])) of sequence s with word (id, delta) and offset off_e = t*B + delta
 * it writes private block e of the destination pools:
 *   dst_k[e, g, j, :] = R(off_e + j) k_pool[id, g, j, :]  (bf16, round to nearest even)
 *   dst_v[e, g, j, :] = v_pool[id, g, j, :]
 * for the slots j holding keys of the sequence (slots at or past kv_lens[s], and entries with
 * id >= num_blocks, are written as zeros), and dst_meta[e] = the word with block id e and the
 * same delta. dst_k / dst_v: bf16 [n_entries, Hkv, B, D], dst_meta: uint32 [n_entries], all
 * device memory owned by the caller; n_entries should equal block_table[num_seqs] and must be
 * <= 2^17 (the new ids must fit the word; else LAZYATTN_ERR_RANGE). Then
 * lazyattn_*_rotated_pool over (dst_k, dst_v, dst_meta, block_table, ...) computes the same
 * attention as lazyattn_* over the position-free pool. Asynchronous on `stream`; errors as
 * above (NULL, ALIGN for 16-byte pools / 4-byte arrays, SHAPE, RANGE, ARG, LAUNCH).
 */
int lazyattn_materialize_rotated(const void* k_pool, const void* v_pool,
                                 const int32_t* block_table, const uint32_t* block_meta,
                                 const int32_t* kv_lens, double rope_base, int32_t num_seqs,
                                 int32_t n_entries, int32_t Hkv, int32_t D, int32_t B,
                                 int32_t num_blocks, void* dst_k, void* dst_v,
                                 uint32_t* dst_meta, void* stream);

/*
 * lazyattn_ingest_kv -- writes the keys and values of new tokens (a prefill suffix, a decode
 * token, a document seen for the first time) into the position-free pool, keys exactly as
 * projected, without rotation (technical summary, "Core Concept": the cache holds
 * content-only keys; position is applied later inside the attention kernels).
 *   k_new, v_new   bf16 [n_tokens, Hkv, D], contiguous, 16-byte aligned (device)
 *   slot_mapping   int32 [n_tokens] (device): block_id * B + slot for each token; a negative
 *                  value or a block_id >= num_blocks leaves that token unwritten
 *   k_pool, v_pool bf16 [num_blocks, Hkv, B, D] (device), written in place
 * Tokens must map to distinct slots (two tokens writing one slot race). D in {64, 128}, B = 16.
 * Asynchronous on `stream`; errors: SHAPE, NULL, ALIGN, LAUNCH (n_tokens = 0 is a no-op).
 */
int lazyattn_ingest_kv(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                       int32_t n_tokens, int32_t Hkv, int32_t D, int32_t B, int32_t num_blocks,
                       void* k_pool, void* v_pool, void* stream);

/*
 * Pool index (host only, no device memory): which physical blocks of the position-free pool
 * hold which document. Technical summary, "Core Concept" / "Problem Statement": cached keys
 * carry no position, so one physical copy serves every request containing the document at
 * any offset; the index is keyed by document alone (a caller-chosen 64-bit key, e.g. a
 * content hash). Documents used by no live request stay cached in LRU order and are
 * evicted oldest first when an allocation needs room. The handle is internally locked;
 * calls from several threads are serialised.
 *   lazyattn_pool_create(num_blocks, B, &h) -- all blocks free; ids handed out from 0 up
 *     at first. ARG if num_blocks not in 1 .. 2^17 or B <= 0.
 *   lazyattn_pool_acquire(h, key, n_tokens, blocks_out, cap, &n, &hit) -- n =
 *     ceil(n_tokens / B). Cached: the same block ids, hit = 1 (STATE if n_tokens differs
 *     from the cached document's). Otherwise n blocks are taken (evicting as needed), hit =
 *     0, and the caller writes the document's K/V into them (lazyattn_ingest_kv). Either
 *     way the document gains one reference. ARG if cap < n (n is still returned); NOSPACE if
 *     free plus evictable blocks are fewer than n (nothing is evicted then).
 *   lazyattn_pool_release(h, key) -- drops one reference; at zero the document becomes
 *     evictable (most recently used). STATE for an unknown key or no reference held.
 *   lazyattn_pool_alloc_private / lazyattn_pool_free_private -- blocks owned by one request
 *     (its question, suffix, decode tokens); freeing a block that is not a private block in
 *     use gives STATE and frees nothing.
 *   lazyattn_pool_stats -- counters and occupancy.
 */
typedef struct LazyattnPoolStats {
  int64_t hits, misses, evictions, evicted_blocks;
  int32_t num_blocks, free_blocks, cached_docs, pinned_docs, private_blocks, evictable_blocks;
} LazyattnPoolStats;
int lazyattn_pool_create(int32_t num_blocks, int32_t block_size, void** pool_out);
int lazyattn_pool_destroy(void* pool);
int lazyattn_pool_acquire(void* pool, uint64_t doc_key, int32_t n_tokens, int32_t* blocks_out,
                          int32_t blocks_cap, int32_t* n_blocks_out, int32_t* hit_out);
int lazyattn_pool_release(void* pool, uint64_t doc_key);
int lazyattn_pool_alloc_private(void* pool, int32_t n_blocks, int32_t* blocks_out);
int lazyattn_pool_free_private(void* pool, const int32_t* blocks, int32_t n_blocks);
int lazyattn_pool_stats(void* pool, LazyattnPoolStats* out);

/*
 * Measured ceilings (for reporting; not part of the attention path):
 *  lazyattn_probe_cus -- compute units the probes and the decode grid are sized for.
 *  lazyattn_probe_mfma -- one workgroup of 8 waves per CU; every wave issues iters x 16
 *    independent 32x32x16 fp16 MFMAs (32768 FLOP each) and writes its s_memtime span
 *    (shader cycles) to cycles_out (uint64 [probe_cus * 8]); scratch_out: float
 *    [probe_cus * 512] (results folded there). Time it with events: FLOP / time is the
 *    matrix-core rate reachable in practice; cycles / time is the sustained shader clock.
 *  lazyattn_probe_read -- reads `bytes` (a multiple of 16, 16-byte aligned) of device memory
 *    once with 16-byte non-temporal loads; scratch_out: uint32 [8 * probe_cus * 256].
 *  lazyattn_probe_gather -- reads the chunks chunk_ids[0 .. n_ids) (device int32; chunk c is
 *    bytes [c * chunk_bytes, (c + 1) * chunk_bytes) of buf, chunk_bytes a multiple of 1024)
 *    with ordinary 16-byte loads, one wave per chunk at a time, waves taking the list
 *    round-robin: the access pattern of a paged kernel over randomly placed blocks. Ids
 *    outside the buffer are skipped. scratch_out: uint32 [8 * probe_cus * 256].
 * Errors: NULL, ALIGN, ARG (iters <= 0), SHAPE (bytes, chunk size), LAUNCH.
 */
int32_t lazyattn_probe_cus(void);
int lazyattn_probe_mfma(int32_t iters, void* cycles_out, void* scratch_out, void* stream);
int lazyattn_probe_read(const void* buf, size_t bytes, void* scratch_out, void* stream);
int lazyattn_probe_gather(const void* buf, size_t bytes, const int32_t* chunk_ids,
                          int32_t n_ids, int32_t chunk_bytes, void* scratch_out, void* stream);

/* Workspace sizes (bytes) for the calls above; 0 on invalid sizes. */
size_t lazyattn_prefill_workspace_bytes(int32_t num_seqs, int32_t total_q, int32_t max_entries,
                                        int32_t Hq, int32_t Hkv, int32_t D);
size_t lazyattn_decode_workspace_bytes(int32_t num_seqs, int32_t total_q, int32_t max_entries,
                                       int32_t Hq, int32_t Hkv, int32_t D);

/*
 * lazyattn_llama31_inv_freq -- host helper: the frequency-scaled RoPE table of the Llama 3.1
 * models, D/2 values theta_k (radians per position) for the *_freqs entry points (the
 * summary only claims compatibility with RoPE variants; this is one such table).
 * theta_k = base^(-2k/D); with wavelength w = 2 pi / theta_k, a pair with
 * w < original_context / high_freq_factor keeps theta_k, one with
 * w > original_context / low_freq_factor gets theta_k / factor, and in between
 * s = (original_context / w - low_freq_factor) / (high_freq_factor - low_freq_factor)
 * blends them: (1 - s) theta_k / factor + s theta_k. Llama 3.1 uses base 500000, factor 8,
 * low 1, high 4, original_context 8192.
 *  inv_freq_out  host double [D/2], written in full on success
 * Errors: NULL output (ERR_NULL); D odd, <= 0 or above 128 (ERR_SHAPE); base <= 1,
 * factor < 1, high_freq_factor <= low_freq_factor or a non-positive factor / context
 * (ERR_ARG). Touches no device.
 */
int lazyattn_llama31_inv_freq(int32_t D, double base, double factor, double low_freq_factor,
                              double high_freq_factor, double original_context,
                              double* inv_freq_out);

/*
 * lazyattn_encode_meta -- HOST function: pack per-entry (block id, logical offset) into
 * words (layout above). block_ids int32 [n], offsets int64 [n], block_table int32
 * [num_seqs+1] with n = block_table[num_seqs]; words_out uint32 [n]. On LAZYATTN_ERR_RANGE
 * *first_bad_entry receives the first offending flat entry index (else -1); words_out is
 * then fully written with the in-range entries encoded and the bad ones set to 0.
 * Returns LAZYATTN_ERR_SHAPE if block_table is not non-decreasing from 0.
 */
int lazyattn_encode_meta(const int32_t* block_ids, const int64_t* offsets,
                         const int32_t* block_table, int32_t num_seqs, int32_t B,
                         uint32_t* words_out, int64_t* first_bad_entry);

/*
 * lazyattn_debug_decode_meta -- DEVICE, for tests: decodes every word with the same device
 * routine the attention kernels use. words uint32 [n], block_table int32 [num_seqs+1]
 * (device), ids_out int32 [n], offsets_out int32 [n] (device); n = block_table[num_seqs]
 * must be passed as n_entries.
 */
int lazyattn_debug_decode_meta(const uint32_t* words, const int32_t* block_table,
                               int32_t num_seqs, int32_t n_entries, int32_t B,
                               int32_t* ids_out, int32_t* offsets_out, void* stream);

/* Static description of a status code. */
const char* lazyattn_status_str(int status);

/* Library version string. */
const char* lazyattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LAZYATTN_H */
