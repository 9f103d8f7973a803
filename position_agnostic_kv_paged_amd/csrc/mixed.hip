// One launch for a continuous batch: prefill work items and decode work items on one grid
// of workgroups of 8 waves.
//
// Technical summary of LazyAttention (arXiv 2606.04302), "Technical Implementation": the
// prefilling phase is compute-bound and the decoding phase memory-bandwidth-bound. A batch
// holding both kinds of request runs here as one work list instead of one kernel per kind.
//
// Work items:
//  - prefill: (KV head, item) with item = a query tile of 256 (position, head) rows over one
//    KV split of its key range (prefill_item; splits chosen by plan_kernel);
//  - decode: a chunk of dec_chunk consecutive decode items, one wave per item: (row-split,
//    KV head) pairs (decode_items), or, over a shared-document plan, (plan item, KV head)
//    pairs (decode_plan_items); their partials are merged by merge_kernel.
// Order: workgroup b runs on XCD b mod 8 and the workgroups of an XCD are dispatched in
// index order as compute units free up, so queue q = b mod 8 is worked through in the order
// c = b / 8. Queue q holds a contiguous eighth of the (KV head, prefill item) space first
// (the tiles sharing a head's keys and values share that XCD's L2), then the decode chunks
// q, q + 8, ...: the long prefill items start first and the short decode chunks fill the
// compute units as the prefill items finish. (Spreading the decode chunks evenly between
// the prefill items, or cutting the tiles into KV splits to interleave them more finely,
// measured slower on the mixed 70B-shaped batch.) The grid is sized from host bounds;
// workgroups past their queue's length leave at once.
#include "decode_body.h"
#include "decode_plan.h"
#include "prefill_body.h"

namespace lazyattn {

// A decode wave's value staging, carved out of the prefill arrays (a workgroup runs one
// kind of item): waves 0-3 in Qs, 4-5 in Ks, 6-7 in Vs.
template <int D>
__device__ __forceinline__ uint8_t* decode_wave_buf(const PrefillSmem<D>& SM, int w) {
  constexpr int B = decode_wave_lds_bytes<D>();
  static_assert(4 * B <= (int)sizeof(SM.Qs) && 2 * B <= (int)sizeof(SM.Ks) &&
                    2 * B <= (int)sizeof(SM.Vs),
                "decode staging fits the prefill arrays");
  uint8_t* q = (uint8_t*)&SM.Qs[0][0] + (w & 3) * B;
  uint8_t* k = (uint8_t*)&SM.Ks[0][0] + (w & 1) * B;
  uint8_t* v = (uint8_t*)&SM.Vs[0][0] + (w & 1) * B;
  return w < 4 ? q : w < 6 ? k : v;
}

template <int D, int G, int PE>
__global__ __launch_bounds__(kPrefillWaves * 64, 1) void mixed_kernel(MixedParams M) {
  LAZYATTN_PREFILL_SMEM(D, SM);
  __shared__ DecodeTables<D> TB;
  __shared__ PairTable<D> PT;                                      // shared-document decode
  const PrefillParams& P = M.pf;
  // the decode view of the same call (kernel arguments are passed once)
  const DecodeParams Dp{P.q, P.k_pool, P.v_pool, P.block_table, P.block_meta, P.kv_lens,
                        P.q_indptr, P.q_pos, M.dec_prefix, P.zero, M.partials, P.num_seqs,
                        P.Hq, P.Hkv, P.num_blocks, *M.bps, M.smax, P.scale_log2, P.freqs,
                        P.slopes, P.Hkv_pool, P.kv_group, P.rot_chunks, P.stored, P.total_q,
                        M.rowsplit_cap};
  const int q = blockIdx.x & 7, c = blockIdx.x >> 3;
  const int n_pf = P.pf_prefix[P.num_seqs];                       // prefill items per KV head
  // decode work: the plan's (item, KV head) pairs, or the row-splits of plan_kernel
  const bool shared = M.plan != nullptr;
  const bool plan_ok = shared && share_plan_ok(M.plan, 16 / G, P.total_q, P.num_seqs);
  const int n_plan = plan_ok ? min(M.plan_items, M.plan[4]) : 0;
  const int n_slots = plan_ok ? min(M.plan_slots, M.plan[5]) : 0;
  const int n_dec = shared ? n_plan * P.Hkv
                           : min(M.dec_prefix[P.num_seqs], M.rowsplit_cap) * P.Hkv;
  const int n_dchunks = (n_dec + M.dec_chunk - 1) / M.dec_chunk;
  const long long np_all = (long long)n_pf * P.Hkv;
  const int p_lo = (int)(np_all * q / 8), p_hi = (int)(np_all * (q + 1) / 8);
  const int n_p = p_hi - p_lo;                                    // this queue's prefill items
  // and decode chunks. Row-splits: a contiguous range per queue (items are numbered
  // head-major, so with 8 KV heads queue q reads head q, as its prefill items do). Plan
  // items: chunk q + 8 dc (the planner puts items that read the same blocks in one class
  // mod 8).
  const int d_lo = shared ? 0 : (int)((long long)n_dchunks * q / 8);
  const int n_d = shared ? (q < n_dchunks ? (n_dchunks - q + 7) / 8 : 0)
                         : (int)((long long)n_dchunks * (q + 1) / 8) - d_lo;
  if (c >= n_p + n_d) return;                                     // uniform
  if (c >= n_p) {                                                 // decode chunk
    const int dc = c - n_p;
    const int w = threadIdx.x >> 6;
    const int first = (shared ? q + 8 * dc : d_lo + dc) * M.dec_chunk;
    if constexpr (PE == kRope) {
      if (shared) {                                               // (uniform)
        decode_pair_tables_init<D>(Dp, TB, PT, kPrefillWaves * 64);   // R(j), R(16+j), R(32)
        __syncthreads();
        decode_plan_items<D, G>(Dp, TB, PT, decode_wave_buf<D>(SM, w), M.plan, n_plan, n_slots,
                                first + w, kPrefillWaves, min(first + M.dec_chunk, n_dec));
        return;
      }
    }
    decode_tables_init<D, G, PE>(Dp, TB, kPrefillWaves * 64);
    __syncthreads();
    decode_items<D, G, PE>(Dp, TB, decode_wave_buf<D>(SM, w), first + w, kPrefillWaves,
                           min(first + M.dec_chunk, n_dec));
  } else {                                                       // prefill item
    const int pi = p_lo + c;
    const int kvh = pi / n_pf;
    prefill_item<D, G, PE>(P, SM, kvh, pi - kvh * n_pf);
  }
}

int prefill_positions_per_tile(int G) { return 32 * kPrefillWaves / G; }

// Merge of the KV-split prefill tiles: workgroup (kvh, item) merges its slice of the item's
// tile (pf_merge_slice); items past the batch's count and items of unsplit tiles leave.
template <int D, int G>
__global__ __launch_bounds__(256) void pf_merge_kernel(PrefillParams P) {
  const int kvh = blockIdx.x / P.pf_item_cap, item = blockIdx.x - kvh * P.pf_item_cap;
  if (item >= P.pf_prefix[P.num_seqs]) return;                   // uniform
  pf_merge_slice<D, G>(P, kvh, item, 256);
}

template <int D>
static hipError_t launch_pf_merge_d(const PrefillParams& p, int G, int nwg, hipStream_t st) {
  dim3 grid(nwg), block(256);
  switch (G) {
    case 1: hipLaunchKernelGGL((pf_merge_kernel<D, 1>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((pf_merge_kernel<D, 2>), grid, block, 0, st, p); break;
    case 4: hipLaunchKernelGGL((pf_merge_kernel<D, 4>), grid, block, 0, st, p); break;
    case 8: hipLaunchKernelGGL((pf_merge_kernel<D, 8>), grid, block, 0, st, p); break;
    case 16: hipLaunchKernelGGL((pf_merge_kernel<D, 16>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_pf_merge(const PrefillParams& p, int D, int G, hipStream_t st) {
  const long long nwg = (long long)p.pf_item_cap * p.Hkv;        // every (KV head, item) slot
  if (nwg <= 0) return hipSuccess;
  if (nwg > INT32_MAX / 2) return hipErrorInvalidValue;
  return D == 128 ? launch_pf_merge_d<128>(p, G, (int)nwg, st)
                  : launch_pf_merge_d<64>(p, G, (int)nwg, st);
}

template <int D, int G>
static hipError_t launch_dg(const MixedParams& p, int pe, int nwg, hipStream_t st) {
  dim3 grid(nwg), block(kPrefillWaves * 64);
  switch (pe) {
    case kRope: hipLaunchKernelGGL((mixed_kernel<D, G, kRope>), grid, block, 0, st, p); break;
    case kStored: hipLaunchKernelGGL((mixed_kernel<D, G, kStored>), grid, block, 0, st, p); break;
    case kAlibi: hipLaunchKernelGGL((mixed_kernel<D, G, kAlibi>), grid, block, 0, st, p); break;
    case kRopePartial:
      hipLaunchKernelGGL((mixed_kernel<D, G, kRopePartial>), grid, block, 0, st, p);
      break;
    case kDocRotated:
      hipLaunchKernelGGL((mixed_kernel<D, G, kDocRotated>), grid, block, 0, st, p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const MixedParams& p, int G, int pe, int nwg, hipStream_t st) {
  switch (G) {
    case 1: return launch_dg<D, 1>(p, pe, nwg, st);
    case 2: return launch_dg<D, 2>(p, pe, nwg, st);
    case 4: return launch_dg<D, 4>(p, pe, nwg, st);
    case 8: return launch_dg<D, 8>(p, pe, nwg, st);
    case 16: return launch_dg<D, 16>(p, pe, nwg, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_mixed(const MixedParams& p, int D, int G, int pe, hipStream_t st) {
  // bounds: every (KV head, prefill item) and every decode chunk, spread over 8 queues
  const long long np = (long long)p.pf.pf_item_cap * p.pf.Hkv;
  const long long nd = ((p.plan ? (long long)p.plan_items : (long long)p.rowsplit_cap) *
                            p.pf.Hkv + p.dec_chunk - 1) / p.dec_chunk;
  const long long per_queue = (np + 7) / 8 + (nd + 7) / 8 + 1;
  if (per_queue * 8 > INT32_MAX / 2) return hipErrorInvalidValue;
  const int nwg = (int)(per_queue * 8);
  return D == 128 ? launch_d<128>(p, G, pe, nwg, st) : launch_d<64>(p, G, pe, nwg, st);
}

}  // namespace lazyattn
