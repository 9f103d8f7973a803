// Device-side planning, split-K merge and the debug word decoder.
//
// The host never reads device memory (calls stay asynchronous), so the per-sequence work
// counts are derived on the device: one workgroup scans q_indptr / block_table and writes
// prefix sums that the attention kernels binary-search to find their sequence.
#include "lazyattn_common.h"
#include "lazyattn_kernels.h"
#include "decode_plan.h"
#include "lazyattn.h"
#include <limits.h>

namespace lazyattn {

// the device-side plan check and the host planner agree on the header
static_assert(kSharePlanMagic == LAZYATTN_SHARE_PLAN_MAGIC, "plan magic");
static_assert(kSharePlanVersion == LAZYATTN_SHARE_PLAN_VERSION, "plan version");
static_assert(kSharePlanHeader == 8, "plan header length");

// One workgroup of 256 threads; exclusive scan over sequences in chunks of 256: each wave
// scans its 64 counts with shuffles, the four wave totals go through LDS (two barriers per
// chunk).
__global__ __launch_bounds__(256) void plan_kernel(PlanParams P) {
  __shared__ int wa[4], wb[4];
  __shared__ int s_tiles, s_maxkt, s_kc, s_dec_rows, s_dec_maxT, s_bps;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid < 48) P.zero[tid] = 0u;
  if (tid < P.half_dim) P.freqs_out[tid] = P.fr.f[tid];
  if (tid == 0) {
    s_tiles = 0;
    s_maxkt = 0;
    s_dec_rows = 0;
    s_dec_maxT = 0;
  }
  __syncthreads();
  // pass 1 (mixed calls): prefill query tiles, the longest prefill key range (in 64-key
  // tiles), and the decode rows with their longest block table. The KV split follows:
  // enough prefill items for one round of the GPU when the tiles are too few; and the
  // decode split is sized from the real decode rows.
  for (int base = 0; P.mode == kPlanMixed && base < P.num_seqs; base += 256) {
    const int s = base + tid;
    int tl = 0, kt = 0, dec = 0, dT = 0;
    if (s < P.num_seqs) {
      const int qlen = P.q_indptr[s + 1] - P.q_indptr[s];
      const int T = P.block_table[s + 1] - P.block_table[s];
      if (qlen == 1) {
        dec = 1;
        dT = T;
      } else if (qlen > 1) {
        tl = (qlen + P.pos_per_tile - 1) / P.pos_per_tile;
        kt = (T + 3) / 4;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      tl += __shfl_xor(tl, o);
      kt = max(kt, __shfl_xor(kt, o));
      dec += __shfl_xor(dec, o);
      dT = max(dT, __shfl_xor(dT, o));
    }
    if (lane == 0) {
      atomicAdd(&s_tiles, tl);
      atomicMax(&s_maxkt, kt);
      atomicAdd(&s_dec_rows, dec);
      atomicMax(&s_dec_maxT, dT);
    }
  }
  __syncthreads();
  if (tid == 0) {
    const long long wp = (long long)s_tiles * P.work_heads;
    int sp = 1;
    if (wp > 0 && wp < P.num_cus) sp = (int)((P.num_cus + wp - 1) / wp);
    sp = min(sp, P.pf_smax);
    const int kc = sp > 1 ? max(kPfMinChunk, (s_maxkt + sp - 1) / sp) : INT_MAX / 2;
    s_kc = kc;
    *P.pf_kc = kc;
    // decode split: a mixed call sizes it from its real decode rows (the rows of the
    // single-row sequences and their longest block table), a decode call takes the host's
    const int bps = P.mode == kPlanMixed
                        ? decode_bps((long long)s_dec_rows * P.work_heads, s_dec_maxT,
                                     P.dec_waves)
                        : P.bps;
    s_bps = bps;
    *P.dec_bps = bps;
  }
  __syncthreads();
  const int kc = s_kc;
  const int bps = s_bps;
  int carry_a = 0, carry_b = 0;                 // identical in every thread
  for (int base = 0; base < P.num_seqs; base += 256) {
    const int s = base + tid;
    int a = 0, b = 0;
    if (s < P.num_seqs) {
      const int qlen = P.q_indptr[s + 1] - P.q_indptr[s];
      const int T = P.block_table[s + 1] - P.block_table[s];
      const bool dec = (P.mode == kPlanDecodeOnly) || qlen == 1;
      if (dec) b = qlen * row_splits(T, bps, P.smax);
      else a = (qlen + P.pos_per_tile - 1) / P.pos_per_tile *
               pf_split((T + 3) / 4, kc, P.pf_smax).splits;
    }
    int ia = a, ib = b;                          // inclusive scan within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int xa = __shfl_up(ia, o), xb = __shfl_up(ib, o);
      if (lane >= o) { ia += xa; ib += xb; }
    }
    if (lane == 63) { wa[w] = ia; wb[w] = ib; }
    __syncthreads();
    int oa = 0, ob = 0, ta = 0, tb = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k < w) { oa += wa[k]; ob += wb[k]; }
      ta += wa[k];
      tb += wb[k];
    }
    if (s < P.num_seqs) {
      P.pf_prefix[s] = carry_a + oa + ia - a;
      P.dec_prefix[s] = carry_b + ob + ib - b;
    }
    carry_a += ta;
    carry_b += tb;
    __syncthreads();                             // wa / wb are rewritten next chunk
  }
  if (tid == 0) {
    P.pf_prefix[P.num_seqs] = carry_a;
    P.dec_prefix[P.num_seqs] = carry_b;
  }
}

// Split-K merge: one thread per 4 output dims of one (row, head). Partials hold the
// running max m (log2 domain), the sum l and the unnormalised o of each split. The row's
// sequence is found once per workgroup by its first wave (a 64-way search: one round of
// loads per factor of 64 sequences), and the partials of up to 16 splits are loaded at once
// and folded in with online rescaling, so the kernel waits for a few memory round trips
// rather than one per split.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams P) {
  constexpr int TPH = D / 4;                  // threads per head
  constexpr int HPB = 256 / TPH;              // heads per block
  constexpr int CH = 16;                      // splits loaded together
  __shared__ long long s_item0;
  __shared__ int s_splits, s_row;
  if (P.slot_prefix) {
    // shared-document plan: row r owns slots [prefix[r], prefix[r + 1]) (a plan whose
    // header does not match gives every row zero slots, hence zero output). A decode call
    // runs one workgroup per row; a mixed call one per sequence, and only the row of a
    // single-row sequence is merged here (s_splits = -1: nothing to do)
    if (threadIdx.x == 0) {
      int r = blockIdx.x;
      bool mine = true;
      if (P.mode != kPlanDecodeOnly) {
        const int seq = blockIdx.x;
        r = P.q_indptr[seq];
        mine = (P.q_indptr[seq + 1] - r == 1) & (r < P.total_q);
      }
      const int32_t* hdr = P.slot_prefix - kSharePlanHeader;
      const bool ok = hdr[0] == kSharePlanMagic && hdr[1] == kSharePlanVersion &&
                      hdr[2] == P.plan_members &&
                      hdr[3] == 2 + 4 * P.plan_members && hdr[6] == P.total_q &&
                      hdr[7] == P.num_seqs;
      const int a = ok && mine ? max(P.slot_prefix[r], 0) : 0;
      const int b = ok && mine ? min(P.slot_prefix[r + 1], P.n_slots) : 0;
      s_splits = mine ? max(b - a, 0) : -1;
      s_item0 = a;
      s_row = r;
    }
  } else if (P.mode != kPlanDecodeOnly) {
    // a batch of any query lengths: only single-row sequences have partials, so workgroup
    // x takes sequence x (no search) and prefill sequences leave at once
    if (threadIdx.x == 0) {
      const int seq = blockIdx.x;
      const int q0 = P.q_indptr[seq], qlen = P.q_indptr[seq + 1] - q0;
      const int T = P.block_table[seq + 1] - P.block_table[seq];
      s_splits = (qlen == 1) & (q0 < P.total_q) ? row_splits(T, *P.bps, P.smax) : 0;
      s_item0 = P.dec_prefix[seq];
      s_row = q0;
    }
  } else if (threadIdx.x < 64) {
    const int r = blockIdx.x;
    const int lane = threadIdx.x;
    int lo = 0, hi = P.num_seqs;              // q_indptr[lo] <= r < q_indptr[hi]
    while (hi - lo > 64) {                    // 64 probes spread over [lo, hi)
      const int span = hi - lo;
      const int idx = lo + (int)(((long long)lane * span) / 64);
      const unsigned long long bal = __ballot(P.q_indptr[idx] <= r);   // lane 0 always set
      const int top = 63 - __builtin_clzll(bal);
      const int nlo = lo + (int)(((long long)top * span) / 64);
      if (top < 63) hi = lo + (int)(((long long)(top + 1) * span) / 64);
      lo = nlo;
    }
    {                                         // the last <= 64 candidates, one per lane
      const int span = hi - lo;
      const bool le = lane < span && P.q_indptr[lo + min(lane, span - 1)] <= r;
      lo += 63 - __builtin_clzll(__ballot(le));
    }
    if (lane == 0) {
      const int seq = lo;
      const int q0 = P.q_indptr[seq], qlen = P.q_indptr[seq + 1] - q0;
      const bool dec = (P.mode == kPlanDecodeOnly) || qlen == 1;
      const int T = P.block_table[seq + 1] - P.block_table[seq];
      const int splits = row_splits(T, *P.bps, P.smax);
      s_splits = dec ? splits : 0;            // prefill rows are written by the prefill kernel
      s_item0 = (long long)P.dec_prefix[seq] + (long long)(r - q0) * splits;
      s_row = r;
    }
  }
  __syncthreads();
  const int r = s_row;
  const int splits = s_splits;
  const long long item0 = s_item0;
  const int h = blockIdx.y * HPB + threadIdx.x / TPH;
  const int d0 = (threadIdx.x % TPH) * 4;
  if (h >= P.Hq || splits < 0) return;
  if (splits == 0) {
    if (P.slot_prefix)                        // a row without partials (no key): zero
      *(u32x2*)(P.out + ((size_t)r * P.Hq + h) * D + d0) = u32x2{0u, 0u};
    return;
  }
  auto part = [&](int sp) { return P.partials + ((item0 + sp) * P.Hq + h) * (D + 4); };
  // one pass with online rescaling, CH splits per round of loads
  float M = -INFINITY, L = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += CH) {
    float mm[CH], ll[CH];
    f32x4 vv[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const bool in = s0 + u < splits;
      const float* pp = part(in ? s0 + u : 0);
      mm[u] = in ? pp[D] : -INFINITY;
      ll[u] = in ? pp[D + 1] : 0.f;
      vv[u] = in ? *(const f32x4*)(pp + d0) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float cm = mm[0];
#pragma unroll
    for (int u = 1; u < CH; ++u) cm = fmaxf(cm, mm[u]);
    if (cm == -INFINITY) continue;                // no visible key in these splits
    const float Mn = fmaxf(M, cm);
    const float al = M == -INFINITY ? 0.f : exp2f(M - Mn);
    L *= al;
    o *= al;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      if (mm[u] == -INFINITY) continue;
      const float sc = exp2f(mm[u] - Mn);
      L += ll[u] * sc;
      o += vv[u] * sc;
    }
    M = Mn;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint32_t* dst = (uint32_t*)(P.out + ((size_t)r * P.Hq + h) * D + d0);
  dst[0] = pack_bf16(o[0] * inv, o[1] * inv);
  dst[1] = pack_bf16(o[2] * inv, o[3] * inv);
}

__global__ void debug_decode_meta_kernel(const uint32_t* words, const int32_t* block_table,
                                         int num_seqs, int n, int32_t* ids, int32_t* offs) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const int s = upper_seq(block_table, num_seqs, e);
  const int t = e - block_table[s];
  const uint32_t w = words[e];
  ids[e] = word_id(w);
  offs[e] = word_offset(w, t);
}

hipError_t launch_plan(const PlanParams& p, hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, int total_q, int D, hipStream_t st) {
  if (total_q == 0) return hipSuccess;
  // one workgroup per query row, or per sequence where only single-row sequences merge
  const unsigned rows = p.mode == kPlanDecodeOnly ? (unsigned)total_q : (unsigned)p.num_seqs;
  if (D == 128) {
    hipLaunchKernelGGL(merge_kernel<128>, dim3(rows, (p.Hq + 7) / 8), dim3(256), 0, st, p);
  } else {
    hipLaunchKernelGGL(merge_kernel<64>, dim3(rows, (p.Hq + 15) / 16), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_debug_decode(const uint32_t* words, const int32_t* bt, int num_seqs, int n,
                               int32_t* ids, int32_t* offs, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(debug_decode_meta_kernel, dim3((n + 255) / 256), dim3(256), 0, st,
                     words, bt, num_seqs, n, ids, offs);
  return hipGetLastError();
}

}  // namespace lazyattn
