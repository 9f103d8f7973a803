// LazyAttention decode kernel for gfx950 (M = 1 per query row, split-K over blocks).
//
// Technical summary of LazyAttention (arXiv 2606.04302), "Technical Implementation",
// decoding phase: the query tile has one row; the rotation is fused into the inner loop
// over KV blocks; the query is re-rotated only when the relative offset changes (a new
// document); (block id, offset) come from one packed 32-bit word per block; memory traffic
// stays that of plain paged attention -- only K and V are read.
//
// For entry t with packed word (id, delta): off_t = 16 t + delta and slot j holds logical
// position off_t + j. The score of a query at p is
//   <R(p) q, R(off_t + j) k> = <R(p - off_t) q, R(j) k>.
// R(j), j < 16, is a per-lane constant (lane = slot), so keys are rotated with loop-invariant
// cos/sin. q' = R(p - off_t) q is carried in the 16 columns of a 16x16x32 MFMA as
// (head g, block phase ph) pairs: a group of two consecutive blocks is scored against
// R(p - off_t0) q and R(p - off_t0 - 16) q at once, and from one group to the next (delta
// unchanged) every column advances by the constant R(-32); where delta changes (a document
// boundary) and at the start of each work item q' is recomputed exactly from the
// double-precision phase.
//
// Work: (row-split, kv-head) items, numbered head-major, go in one contiguous range per XCD
// and round-robin to that XCD's waves (decode_kernel; the mixed kernel deals its decode
// chunks the same way); the grid is exactly resident. Each wave first describes all of its items
// at once, one item per lane (sequence, query row and position, entry range), so starting
// an item costs no dependent memory round trips; the first key/value group of the next
// item is fetched while the last group of the current one is multiplied. Keys are
// prefetched one group ahead into registers; values go straight
// from global memory into a double-buffered, XOR-swizzled LDS slice of the wave
// (global_load_lds) and are read back transposed (ds_read_b64_tr_b16) as the A operand of
// O^T += V^T P^T. Rows that must contribute nothing (padding, missing blocks) are fetched
// from a zeroed workspace chunk so that 0 * NaN never enters the sum. Each item writes a
// partial (o, m, l); merge_kernel combines the splits of a row.
#pragma once
#include "lazyattn_common.h"
#include "lazyattn_kernels.h"

namespace lazyattn {

constexpr int kDecodeWaves = 4;        // waves per workgroup (standalone decode kernel)
constexpr int kDecodeWgPerCu = 2;      // workgroups per CU = the resident count (VGPRs, LDS)

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 16-byte global -> LDS copy: lane l writes lds_wave_base + 16 l (the base is wave-uniform).
__device__ __forceinline__ void g2lds16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base,
                                   16, 0, 0);
}

// LDS layout of a group's values (32 rows of D bf16): 16-byte chunk c of row R sits at chunk
// position c ^ swz(R), so the four rows read by one 16-lane transposed read hit disjoint banks.
__device__ __forceinline__ int vswz(int R) { return (R & 3) * 2; }

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// R(j) on two rotate-half pairs at once in packed fp16: a, b hold (x_k, x_k+1) and
// (x_k+D/2, x_k+1+D/2), c and s the pairs' cos and sin; returns {a c - b s, a s + b c}.
// The products are the fp16 score operands themselves (they are rounded to fp16 anyway).
__device__ __forceinline__ u32x2 rot_h2(uint32_t a, uint32_t b, uint32_t c, uint32_t s) {
  const h2 A = __builtin_bit_cast(h2, a), Bv = __builtin_bit_cast(h2, b);
  const h2 C = __builtin_bit_cast(h2, c), S = __builtin_bit_cast(h2, s);
  return u32x2{__builtin_bit_cast(uint32_t, A * C - Bv * S),
               __builtin_bit_cast(uint32_t, A * S + Bv * C)};
}

struct GroupMeta {
  int id[2], delta[2], nval[2];
  int st[2];                   // document-rotated pool: stored offset of the block's slot 0
};

// PE = kStored is the materialised baseline: the pool's keys already carry R(L) at their
// logical positions, so keys are read as stored and q' = R(p) q for the whole item.
// PE = kAlibi rotates nothing (q' = q, keys as stored) and adds slope_h (L - p) to each
// score, L = off_t + j from the packed word.
// PE = kRopePartial is kRope over the permuted dim order of nat_chunk (partial rotary).
// PE = kDocRotated reads keys stored with R(stored_t + j): keys are used as stored and
// q' = R(p - (off_t - stored_t)) q, recomputed where off_t - stored_t changes.
// Loop-invariant rotation constants, shared by a workgroup in LDS: R(j) of slot j for
// frequencies k = 32c + 8 q4 + 2 e2 + u as packed fp16 pairs (cos u = 0, 1; sin u = 0, 1)
// at [c][q4][e2][j] -- the 16 slots of a 16-lane read are consecutive 8-byte words; and
// R(32) (or R(16) for G = 16) for the per-group advance of q', (cos, sin) interleaved.
template <int D>
struct DecodeTables {
  alignas(16) float adv[D];
  alignas(16) u32x2 slot_tab[(D / 64) * 4 * 4 * 16];
};
// Shared-document decode also uses R(16 + j), laid out as slot_tab: the second block of a
// group is scored with the first block's q'.
template <int D>
struct PairTable {
  alignas(16) u32x2 slot_tab16[(D / 64) * 4 * 4 * 16];
};

// One wave's double-buffered value staging (2 groups x 32 rows x D bf16)
template <int D>
constexpr int decode_wave_lds_bytes() { return 2 * 32 * D * 2; }

// Fill the tables (every thread of the workgroup calls it; a barrier must follow).
template <int D, int G, int PE>
__device__ __forceinline__ void decode_tables_init(const DecodeParams& P, DecodeTables<D>& TB,
                                                   int nthreads) {
  constexpr bool ROT = PE == kRope || PE == kRopePartial;
  constexpr bool PHC = 2 * G <= 16;
  constexpr int HC = D / 64;
  for (int i = threadIdx.x; ROT && i < HC * 4 * 4 * 16; i += nthreads) {
    const int j = i & 15, e2 = (i >> 4) & 3, qq = (i >> 6) & 3, c = i >> 8;
    const int f0 = 32 * c + 8 * qq + 2 * e2;
    float c0, s0, c1, s1;
    rope_cos_sin(j, P.freqs[f0], c0, s0);
    rope_cos_sin(j, P.freqs[f0 + 1], c1, s1);
    TB.slot_tab[i] = u32x2{pack_f16(c0, c1), pack_f16(s0, s1)};
  }
  if ((int)threadIdx.x < D / 2) {           // R(32) (PHC) or R(16): q' advance
    float cs, sn;
    rope_cos_sin(PHC ? 32 : 16, P.freqs[threadIdx.x], cs, sn);
    TB.adv[2 * threadIdx.x] = cs;
    TB.adv[2 * threadIdx.x + 1] = sn;
  }
}

// The tables of shared-document decode: R(j) and R(16 + j) per slot, R(32) per group.
template <int D>
__device__ __forceinline__ void decode_pair_tables_init(const DecodeParams& P,
                                                        DecodeTables<D>& TB, PairTable<D>& PT,
                                                        int nthreads) {
  decode_tables_init<D, 8, kRope>(P, TB, nthreads);   // R(j), R(32)
  constexpr int HC = D / 64;
  for (int i = threadIdx.x; i < HC * 4 * 4 * 16; i += nthreads) {
    const int j = i & 15, e2 = (i >> 4) & 3, qq = (i >> 6) & 3, c = i >> 8;
    const int f0 = 32 * c + 8 * qq + 2 * e2;
    float c0, s0, c1, s1;
    rope_cos_sin(16 + j, P.freqs[f0], c0, s0);
    rope_cos_sin(16 + j, P.freqs[f0 + 1], c1, s1);
    PT.slot_tab16[i] = u32x2{pack_f16(c0, c1), pack_f16(s0, s1)};
  }
}

// Decode items gw, gw + W, gw + 2W, ... below n_items, by the calling wave. An item is a
// (row-split, KV head) pair, numbered head-major: item = kvh * R + row_split over the R
// row-splits of the batch, so that a contiguous range of items given to the workgroups of
// one XCD holds one KV head's reads of every row (rows sharing a document then find its
// blocks in that XCD's L2). `lds` is this wave's value staging (decode_wave_lds_bytes).
template <int D, int G, int PE>
__device__ __forceinline__ void decode_items(const DecodeParams& P, const DecodeTables<D>& TB,
                                             uint8_t* lds, const int gw, const int W,
                                             const int n_items) {
  constexpr bool PART = PE == kRopePartial;   // dims in the permuted order of nat_chunk
  constexpr bool ROT = PE == kRope || PART;   // keys get the per-slot rotation R(j)
  constexpr bool ALIBI = PE == kAlibi;
  // DOC: keys carry R(stored + j); q' = R(p - (off - stored)) q is constant over entries with
  // the same off - stored (one document) and keys are used as stored
  constexpr bool DOC = PE == kDocRotated;
  // PHC: the 16 columns of the score MFMA hold (head, block phase) pairs (2 G <= 16), so
  // both blocks of a group are scored against one q' operand. Otherwise (G = 16) the
  // columns are the 16 heads and q' is set to each block's phase in turn.
  constexpr bool PHC = 2 * G <= 16;
  static_assert(PHC || G == 16, "decode supports G in {1, 2, 4, 8, 16}");
  constexpr int NC = D / 32;                  // 32-dim k-steps of the score MFMA
  constexpr int HC = NC / 2;                  // chunk c pairs with chunk c + HC (dims + D/2)
  constexpr int ROWB = D * 2;                 // bytes per value row
  constexpr int BUF = 32 * ROWB;              // one group: 2 blocks x 16 rows
  constexpr int LOADS = BUF / 1024;           // global_load_lds instructions per group
  const float* adv_all = TB.adv;
  const u32x2* slot_tab = TB.slot_tab;
  const int lane = threadIdx.x & 63;
  const int i16 = lane & 15, q4 = lane >> 4;
  const int col = i16, g = col % G, ph = col / G;
  const bool col_ok = col < 2 * G;
  // element offset in a q or key row of the 8 dims this lane holds in 32-dim k-step c
  int dofs[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
    dofs[c] = PART ? 8 * nat_chunk(4 * c + q4, P.rot_chunks, D / 16) : 32 * c + 8 * q4;

  const int nrs = min(P.dec_prefix[P.num_seqs], P.rowsplit_cap);   // row-splits R
  // items gw + i W, i = 0, 1, ...; described 64 at a time, item gw + (64 rd + k) W by lane k
  for (int base = gw; base < n_items; base += 64 * W) {
    int x_rs = 0, x_kvh = 0, x_kvp = 0, x_r = 0, x_p = 0, x_e0 = 0, x_kvlen = 0, x_eb = 0,
        x_ee = 0;
    {
      const int itl = base + lane * W;
      if (itl < n_items) {
        x_kvh = itl / nrs;
        x_rs = itl - x_kvh * nrs;
        x_kvp = x_kvh / P.kv_group;                   // pool head of this work head
        const int seq = upper_seq(P.dec_prefix, P.num_seqs, x_rs);
        const int local = x_rs - P.dec_prefix[seq];
        x_e0 = P.block_table[seq];
        const int T = P.block_table[seq + 1] - x_e0;
        x_kvlen = P.kv_lens[seq];
        const int splits = row_splits(T, P.bps, P.smax);
        const int bpsr = row_bps(T, P.bps, P.smax);
        const int row = local / splits, sp = local - row * splits;
        x_eb = sp * bpsr;
        x_ee = min(T, x_eb + bpsr);
        x_r = P.q_indptr[seq] + row;
        if (x_r >= P.total_q) {                       // past the q array: no work, no partial
          x_r = 0;
          x_ee = x_eb;
        }
        x_p = P.q_pos[x_r];
      }
    }
    const int n_here = min(64, (n_items - base + W - 1) / W);
    int buf = 0;
    bool pre = false;                                 // first group already in flight
    u32x4 kcur[2][NC], knext[2][NC];
    GroupMeta gcur, gnext;
    for (int k = 0; k < n_here; ++k) {
    const int rs = rl(x_rs, k), kvh = rl(x_kvh, k), kvp = rl(x_kvp, k);
    const int e0 = rl(x_e0, k), kvlen = rl(x_kvlen, k);
    const int eb = rl(x_eb, k), ee = rl(x_ee, k);
    const int r = rl(x_r, k), p = rl(x_p, k);
    const int h = kvh * G + g;
    const uint16_t* qrow = P.q + ((size_t)r * P.Hq + h) * D;
    const float sl2 = ALIBI ? P.slopes[h] * 1.4426950408889634f : 0.f;   // log2 units

    float m = -INFINITY, l = 0.f;
    f32x4 o[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{};
    float qr[NC][8];
    bool have_q = false;
    int cur_delta = 0;

    // issue the loads of the group starting at entry t0 of an item (entries below i_ee,
    // words from i_e0, pool head i_kvh, i_kvlen keys) into LDS buffer `buf`
    auto issue = [&](int t0, int i_ee, int i_e0, int i_kvh, int i_kvlen, int buf,
                     u32x4 (&kreg)[2][NC], GroupMeta& gm) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int t = t0 + b;
        const bool blk = t < i_ee;
        const uint32_t wd = blk ? P.block_meta[i_e0 + t] : 0u;
        const int id = word_id(wd);
        const int rem = i_kvlen - t * kBlock;
        gm.id[b] = id;
        gm.delta[b] = word_delta(wd);
        // (used only at the group's turn, after its loads have been waited for)
        gm.st[b] = DOC && blk ? P.stored[i_e0 + t] : 0;
        gm.nval[b] = (blk && id < P.num_blocks) ? (rem < kBlock ? (rem > 0 ? rem : 0) : kBlock) : 0;
        const size_t kb = ((size_t)id * P.Hkv_pool + i_kvh) * kBlock;
#pragma unroll
        for (int c = 0; c < NC; ++c)
          kreg[b][c] = i16 < gm.nval[b]
                           ? *(const u32x4*)(P.k_pool + (kb + i16) * D + dofs[c])
                           : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int off = i * 1024 + 16 * lane;
        const int R = off / ROWB, cs = (off % ROWB) / 16;
        const int b = R >> 4, j = R & 15;
        const int c = cs ^ vswz(R);
        const void* src = P.zero;
        if (j < gm.nval[b])
          src = P.v_pool + (((size_t)gm.id[b] * P.Hkv_pool + i_kvh) * kBlock + j) * D + 8 * c;
        g2lds16(src, lds + buf * BUF + i * 1024);
      }
    };

    if (!pre && eb < ee) issue(eb, ee, e0, kvp, kvlen, buf, knext, gnext);
    pre = false;
    for (int t0 = eb; t0 < ee; t0 += 2) {
      __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0): this group's keys and values
      asm volatile("" ::: "memory");
      wave_sync();
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int c = 0; c < NC; ++c) kcur[b][c] = knext[b][c];
      gcur = gnext;
      if (t0 + 2 < ee) {
        issue(t0 + 2, ee, e0, kvp, kvlen, buf ^ 1, knext, gnext);
      } else if (k + 1 < n_here) {                    // the next item's first group
        const int n_eb = rl(x_eb, k + 1), n_ee = rl(x_ee, k + 1);
        if (n_eb < n_ee) {
          issue(n_eb, n_ee, rl(x_e0, k + 1), rl(x_kvp, k + 1), rl(x_kvlen, k + 1), buf ^ 1,
                knext, gnext);
          pre = true;
        }
      }

      const int d0 = gcur.delta[0];
      const int d1 = (t0 + 1 < ee) ? gcur.delta[1] : d0;
      // rotation still to apply to the stored keys of each block: off - stored
      const int sh0 = t0 * kBlock + d0 - gcur.st[0];
      const int sh1 = (t0 + 1 < ee) ? (t0 + 1) * kBlock + d1 - gcur.st[1] : sh0;
      u32x4 bp;
      if constexpr (PHC) {
        // ---- q' of this lane's column: R(p - off_{t0+ph}) q_g ---------------------------
        if (!ROT && !DOC && have_q) {
          // keys carry their absolute rotation: q' = R(p) q stays fixed
        } else if (DOC && have_q && sh0 == cur_delta && sh1 == cur_delta) {
          // same document as the previous group: q' unchanged
        } else if (ROT && have_q && d0 == cur_delta && d1 == cur_delta) {
#pragma unroll
          for (int c = 0; c < HC; ++c)
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {           // R(-32)
              const f32x4 cs = *(const f32x4*)(adv_all + 2 * (32 * c + 8 * q4 + 2 * e2));
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const int e = 2 * e2 + u;
                const float a = qr[c][e], b = qr[c + HC][e];
                qr[c][e] = a * cs[2 * u] + b * cs[2 * u + 1];
                qr[c + HC][e] = b * cs[2 * u] - a * cs[2 * u + 1];
              }
            }
        } else {
          const int n = ROT ? p - ((t0 + ph) * kBlock + (ph ? d1 : d0))
                        : DOC ? p - (ph ? sh1 : sh0) : (ALIBI ? 0 : p);
#pragma unroll
          for (int c = 0; c < HC; ++c) {
            const u32x4 va = col_ok ? *(const u32x4*)(qrow + dofs[c]) : u32x4{0, 0, 0, 0};
            const u32x4 vb = col_ok ? *(const u32x4*)(qrow + dofs[c + HC]) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              float cs, sn;
              rope_cos_sin(n, P.freqs[32 * c + 8 * q4 + e], cs, sn);
              const float a = (e & 1) ? bf_hi(va[e >> 1]) : bf_lo(va[e >> 1]);
              const float b = (e & 1) ? bf_hi(vb[e >> 1]) : bf_lo(vb[e >> 1]);
              qr[c][e] = a * cs - b * sn;
              qr[c + HC][e] = a * sn + b * cs;
            }
          }
          have_q = ROT ? d0 == d1 : DOC ? sh0 == sh1 : true;
          cur_delta = DOC ? sh1 : d1;
        }
        // ---- scores of both blocks; each lane keeps its own phase's block ------------------
        f32x4 S[2] = {f32x4{}, f32x4{}};
#pragma unroll
        for (int c = 0; c < HC; ++c) {
          u32x4 qlo, qhi;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            qlo[i] = pack_f16(qr[c][2 * i], qr[c][2 * i + 1]);
            qhi[i] = pack_f16(qr[c + HC][2 * i], qr[c + HC][2 * i + 1]);
          }
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            u32x4 lo, hi;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float a0 = bf_lo(kcur[b][c][i]), a1 = bf_hi(kcur[b][c][i]);
              const float b0 = bf_lo(kcur[b][c + HC][i]), b1 = bf_hi(kcur[b][c + HC][i]);
              if (ROT) {
                const u32x2 t = slot_tab[((c * 4 + q4) * 4 + i) * 16 + i16];
                const u32x2 r = rot_h2(pack_f16(a0, a1), pack_f16(b0, b1), t[0], t[1]);
                lo[i] = r[0];
                hi[i] = r[1];
              } else {
                lo[i] = pack_f16(a0, a1);
                hi[i] = pack_f16(b0, b1);
              }
            }
            S[b] = mfma16h(as_f16x8(lo), as_f16x8(qlo), S[b]);
            S[b] = mfma16h(as_f16x8(hi), as_f16x8(qhi), S[b]);
          }
        }
        const int nv = ph ? gcur.nval[1] : gcur.nval[0];
        const int offp = (t0 + ph) * kBlock + (ph ? d1 : d0);
        float sc[4];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * q4 + i;
          const float v = ph ? S[1][i] : S[0][i];
          const bool ok = col_ok && j < nv && offp + j <= p;
          sc[i] = ok ? v * P.scale_log2 + (ALIBI ? sl2 * (float)(offp + j - p) : 0.f) : -INFINITY;
          mx = fmaxf(mx, sc[i]);
        }
        // row max over the 8 lanes of head g: slot groups (q4) and both phases
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        mx = fmaxf(mx, __shfl_xor(mx, G));
        const float m_new = fmaxf(m, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2f(m - m_use);
        float pr[4];
        float rsum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) { pr[i] = exp2f(sc[i] - m_use); rsum += pr[i]; }
        l = l * alpha + rsum;
        m = m_new;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;
        const uint32_t p01 = pack_bf16(pr[0], pr[1]), p23 = pack_bf16(pr[2], pr[3]);
        bp = ph ? u32x4{0u, 0u, p01, p23} : u32x4{p01, p23, 0u, 0u};
      } else {
        // ---- G = 16: q' = R(p - off_b) q_g of lane column g, set for block b in turn ------
        auto qexact = [&](int n) {
#pragma unroll
          for (int c = 0; c < HC; ++c) {
            const u32x4 va = *(const u32x4*)(qrow + dofs[c]);
            const u32x4 vb = *(const u32x4*)(qrow + dofs[c + HC]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              float cs, sn;
              rope_cos_sin(n, P.freqs[32 * c + 8 * q4 + e], cs, sn);
              const float a = (e & 1) ? bf_hi(va[e >> 1]) : bf_lo(va[e >> 1]);
              const float b = (e & 1) ? bf_hi(vb[e >> 1]) : bf_lo(vb[e >> 1]);
              qr[c][e] = a * cs - b * sn;
              qr[c + HC][e] = a * sn + b * cs;
            }
          }
        };
        auto set_q = [&](int off) {              // qr := R(p - off) q (or the fixed q')
          if (!ROT && !DOC) {
            if (!have_q) qexact(ALIBI ? 0 : p);
          } else if (DOC && have_q && off == cur_delta) {
            // same document: q' unchanged
          } else if (ROT && have_q && off == cur_delta + kBlock) {
#pragma unroll
            for (int c = 0; c < HC; ++c)
#pragma unroll
              for (int e2 = 0; e2 < 4; ++e2) {       // R(-16)
                const f32x4 cs = *(const f32x4*)(adv_all + 2 * (32 * c + 8 * q4 + 2 * e2));
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                  const int e = 2 * e2 + u;
                  const float a = qr[c][e], b = qr[c + HC][e];
                  qr[c][e] = a * cs[2 * u] + b * cs[2 * u + 1];
                  qr[c + HC][e] = b * cs[2 * u] - a * cs[2 * u + 1];
                }
              }
          } else {
            qexact(p - off);
          }
          have_q = true;
          cur_delta = off;                         // here: the offset qr is anchored at
        };
        auto scores = [&](int b) {
          f32x4 S = {};
#pragma unroll
          for (int c = 0; c < HC; ++c) {
            u32x4 qlo, qhi, lo, hi;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              qlo[i] = pack_f16(qr[c][2 * i], qr[c][2 * i + 1]);
              qhi[i] = pack_f16(qr[c + HC][2 * i], qr[c + HC][2 * i + 1]);
              const float a0 = bf_lo(kcur[b][c][i]), a1 = bf_hi(kcur[b][c][i]);
              const float b0 = bf_lo(kcur[b][c + HC][i]), b1 = bf_hi(kcur[b][c + HC][i]);
              if (ROT) {
                const u32x2 t = slot_tab[((c * 4 + q4) * 4 + i) * 16 + i16];
                const u32x2 r = rot_h2(pack_f16(a0, a1), pack_f16(b0, b1), t[0], t[1]);
                lo[i] = r[0];
                hi[i] = r[1];
              } else {
                lo[i] = pack_f16(a0, a1);
                hi[i] = pack_f16(b0, b1);
              }
            }
            S = mfma16h(as_f16x8(lo), as_f16x8(qlo), S);
            S = mfma16h(as_f16x8(hi), as_f16x8(qhi), S);
          }
          return S;
        };
        const bool has1 = t0 + 1 < ee;
        set_q(DOC ? sh0 : t0 * kBlock + d0);
        const f32x4 S0 = scores(0);
        f32x4 S1 = {};
        if (has1) {
          set_q(DOC ? sh1 : (t0 + 1) * kBlock + d1);
          S1 = scores(1);
        }
        float sc[8];
        float mx = -INFINITY;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int nv = b ? (has1 ? gcur.nval[1] : 0) : gcur.nval[0];
          const int offb = (t0 + b) * kBlock + (b ? d1 : d0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = 4 * q4 + i;
            const float v = b ? S1[i] : S0[i];
            const bool ok = j < nv && offb + j <= p;
            sc[4 * b + i] = ok ? v * P.scale_log2 + (ALIBI ? sl2 * (float)(offb + j - p) : 0.f)
                               : -INFINITY;
            mx = fmaxf(mx, sc[4 * b + i]);
          }
        }
        // row max over the 4 lanes of head g (slot groups q4)
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2f(m - m_use);
        float pr[8];
        float rsum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) { pr[i] = exp2f(sc[i] - m_use); rsum += pr[i]; }
        l = l * alpha + rsum;
        m = m_new;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;
        bp = u32x4{pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3]), pack_bf16(pr[4], pr[5]),
                   pack_bf16(pr[6], pr[7])};
      }

      // ---- O^T += V^T P^T over the group's 32 keys ------------------------------------------
      const uint8_t* vb = lds + buf * BUF;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const int x = 16 * dt + 4 * (i16 & 3);
        const int cchunk = x >> 3, half = (x >> 2) & 1;
        const int R1 = 4 * q4 + (i16 >> 2), R2 = 16 + R1;
        const u32x2 r1 = lds_read_tr(
            (const uint16_t*)(vb + R1 * ROWB + 16 * (cchunk ^ vswz(R1)) + 8 * half));
        const u32x2 r2 = lds_read_tr(
            (const uint16_t*)(vb + R2 * ROWB + 16 * (cchunk ^ vswz(R2)) + 8 * half));
        const u32x4 a = {r1[0], r1[1], r2[0], r2[1]};
        o[dt] = mfma16(as_bf16x8(a), as_bf16x8(bp), o[dt]);
      }
      buf ^= 1;
    }
    wave_sync();

    // ---- partial of this item: add both phases of head g -----------------------------------
    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    if (PHC) lt += __shfl_xor(lt, G);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int i = 0; PHC && i < 4; ++i) o[dt][i] += __shfl_xor(o[dt][i], G);
    if (col < G) {
      float* part = P.partials + ((size_t)rs * P.Hq + h) * (D + 4);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) *(f32x4*)(part + 16 * dt + 4 * q4) = o[dt];
      if (q4 == 0) { part[D] = m; part[D + 1] = lt; }
    }
    }
  }
}

}  // namespace lazyattn
