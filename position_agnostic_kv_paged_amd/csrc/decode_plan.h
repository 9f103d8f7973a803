// Shared-document decode: work items from a host plan (lazyattn_decode_share_plan), each a
// run of blocks read by up to M = 16 / G query rows at once.
//
// Technical summary of LazyAttention (arXiv 2606.04302), "Core Concept": keys are cached
// without position, so the same physical blocks serve every request that contains a
// document, at any offset. "Technical Implementation", decoding: for entry t with offset
// off_t, <R(p) q, R(off_t + j) k> = <R(p - off_t) q, R(j) k>, keys get the per-slot R(j)
// and the query is re-rotated where the offset changes. Here the 16 columns of the score
// and value products hold (member row m, head g) pairs: the keys and values of a block are
// loaded once (from the leading member's table), rotated by R(j) once, and scored against
// every member's q'_m = R(p_m - off_m,t) q_m, where off_m,t comes from member m's own packed
// word for that block (the same block sits at different entries and offsets in different
// rows). q'_m is set for each block in turn: advanced by R(-16) from the previous block when
// the member's offset moves by 16, recomputed exactly from the double-precision phase
// otherwise. Within an item every member's offset delta is constant (the planner cuts runs
// where it changes), so the second block of a group sits 16 positions after the first for
// every member: <R(p - off - 16) q, R(j) k> = <R(p - off) q, R(16 + j) k>, and that block is
// scored with the first block's q' against keys rotated by R(16 + j). q' is therefore set
// once per group, advanced by R(-32) from the previous group. Masks, the online softmax
// and the partial (o, m, l) are per column; each member writes its partial into its own
// slot, and merge_kernel folds a row's slots.
#pragma once
#include "decode_body.h"

namespace lazyattn {

constexpr int kSharePlanMagic = 0x5053414C;
constexpr int kSharePlanHeader = 8;
constexpr int kSharePlanVersion = 2;         // 2: constant offset delta within an item

// does the plan's header match this call (members per item, rows, sequences)?
__device__ __forceinline__ bool share_plan_ok(const int32_t* plan, int M, int total_q,
                                              int num_seqs) {
  return plan[0] == kSharePlanMagic && plan[1] == kSharePlanVersion && plan[2] == M &&
         plan[3] == 2 + 4 * M &&
         plan[6] == total_q && plan[7] == num_seqs;
}

// Items gw, gw + W, ... below `end` of the n_plan x Hkv (plan item, KV head) pairs, by the
// calling wave. TB must hold R(j) and R(32), PT R(16 + j) (decode_pair_tables_init). Only
// the RoPE mode.
template <int D, int G>
__device__ __forceinline__ void decode_plan_items(const DecodeParams& P,
                                                  const DecodeTables<D>& TB,
                                                  const PairTable<D>& PT, uint8_t* lds,
                                                  const int32_t* plan, const int n_plan,
                                                  const int n_slots, const int gw, const int W,
                                                  const int end) {
  constexpr int M = 16 / G;                    // member rows per item
  constexpr int REC = 2 + 4 * M;
  constexpr int NC = D / 32;
  constexpr int HC = NC / 2;
  constexpr int ROWB = D * 2;
  constexpr int BUF = 32 * ROWB;
  constexpr int LOADS = BUF / 1024;
  const float* adv_all = TB.adv;
  const u32x2* slot_tab = TB.slot_tab;
  const u32x2* slot_tab16 = PT.slot_tab16;
  const int lane = threadIdx.x & 63;
  const int i16 = lane & 15, q4 = lane >> 4;
  const int mi = i16 / G, g = i16 % G;         // this lane's column: member mi, head g
  const int32_t* recs = plan + kSharePlanHeader + P.total_q + 1;
  const int n_items = min(n_plan * P.Hkv, end);
  int dofs[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) dofs[c] = 32 * c + 8 * q4;

  // an item: the leader's table (uniform) and this lane's member (per lane). Member entry
  // t of the item has logical offset o0 + 16 t + delta and kr0 - 16 t keys of its sequence
  // left from its slot 0; entries at or past lim are outside its table. The item's packed
  // words are loaded once, with the description: word w = m len + t (member m, entry t;
  // len * members <= 128) sits in lane w % 64 of w0 (w < 64) or w1.
  struct Desc {
    int len, kvh, kvp, limL;                   // uniform (leader)
    int row, p, slot, lim, o0, kr0;            // per lane (slot < 0: no member)
    uint32_t w0, w1;                           // the item's words
  };
  auto describe = [&](int it) {
    Desc x;
    const int pi = it / P.Hkv;
    x.kvh = it - pi * P.Hkv;
    x.kvp = x.kvh / P.kv_group;
    const int32_t* r = recs + (size_t)pi * REC;
    x.len = __builtin_amdgcn_readfirstlane(r[0]);
    const int nm = min(__builtin_amdgcn_readfirstlane(r[1]), M);
    const int sL = min(max(__builtin_amdgcn_readfirstlane(r[3]), 0), P.num_seqs - 1);
    const int ebL = max(__builtin_amdgcn_readfirstlane(r[4]), 0);
    x.limL = __builtin_amdgcn_readfirstlane(P.block_table[sL + 1]) -
             __builtin_amdgcn_readfirstlane(P.block_table[sL]) - ebL;
    const int row = r[2 + 4 * mi], seq = r[3 + 4 * mi], eb = r[4 + 4 * mi];
    const int slot = r[5 + 4 * mi];
    const bool act = mi < nm && row >= 0 && row < P.total_q && seq >= 0 &&
                     seq < P.num_seqs && slot >= 0 && slot < n_slots && eb >= 0;
    const int s = act ? seq : 0;
    x.row = act ? row : 0;
    x.slot = act ? slot : -1;                  // every member writes its slot
    const int e0 = P.block_table[s];
    x.lim = act ? max(P.block_table[s + 1] - e0 - eb, 0) : 0;
    x.o0 = (act ? eb : 0) * kBlock;
    x.kr0 = P.kv_lens[s] - x.o0;
    x.p = P.q_pos[x.row];
    uint32_t wv[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int w = 64 * k + lane;
      const int m = x.len > 0 ? w / x.len : M, t = x.len > 0 ? w - m * x.len : 0;
      const int sm = m < nm ? r[3 + 4 * m] : -1, em = m < nm ? r[4 + 4 * m] : -1;
      const bool okw = sm >= 0 && sm < P.num_seqs && em >= 0;
      const int b0 = okw ? P.block_table[sm] : 0;
      const int nb = okw ? P.block_table[sm + 1] - b0 : 0;
      wv[k] = okw && em + t < nb ? P.block_meta[b0 + em + t] : 0u;
    }
    x.w0 = wv[0];
    x.w1 = wv[1];
    return x;
  };
  struct Grp {
    int id[2], nl[2], kvp;                     // uniform: block id, rows to load, pool head
    int off[2], nv[2];                         // per lane: member offset, valid keys
  };
  // blocks t0, t0 + 1 of item x: their description into gm and their values into LDS buffer
  // `bb` (the keys follow with issue_k, once the registers they go to are free)
  auto issue = [&](const Desc& x, int t0, int bb, Grp& gm) {
    gm.kvp = x.kvp;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int t = t0 + b;
      const bool okL = t < x.len && t < x.limL;
      // member 0 leads: its word for entry t is word t (uniform); this lane's member's is
      // word mi len + t
      const uint32_t wL = t < 64 ? __builtin_amdgcn_readlane(x.w0, t & 63)
                                 : __builtin_amdgcn_readlane(x.w1, t & 63);
      const int id = word_id(wL);
      const bool idok = okL && id < P.num_blocks;
      const bool okm = t < x.len && t < x.lim;
      const int wi = mi * x.len + t;
      const uint32_t a0 = __shfl(x.w0, wi & 63), a1 = __shfl(x.w1, wi & 63);
      const uint32_t wm = okm && wi < 128 ? (wi < 64 ? a0 : a1) : 0u;
      gm.off[b] = x.o0 + t * kBlock + word_delta(wm);
      const int rem = x.kr0 - t * kBlock;
      gm.nv[b] = okm && idok ? (rem < kBlock ? (rem > 0 ? rem : 0) : kBlock) : 0;
      int nl = gm.nv[b];                       // rows to load: the most any member uses
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) nl = max(nl, __shfl_xor(nl, o));
      gm.nl[b] = __builtin_amdgcn_readfirstlane(nl);
      gm.id[b] = id;
    }
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int off = i * 1024 + 16 * lane;
      const int R = off / ROWB, cs = (off % ROWB) / 16;
      const int b = R >> 4, j = R & 15;
      const int c = cs ^ vswz(R);
      const void* src = P.zero;
      if (j < gm.nl[b])
        src = P.v_pool + (((size_t)gm.id[b] * P.Hkv_pool + x.kvp) * kBlock + j) * D + 8 * c;
      g2lds16(src, lds + bb * BUF + i * 1024);
    }
  };
  // the keys of a described group into registers
  auto issue_k = [&](const Grp& gm, u32x4 (&kreg)[2][NC]) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const size_t kb = ((size_t)gm.id[b] * P.Hkv_pool + gm.kvp) * kBlock;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        kreg[b][c] = i16 < gm.nl[b] ? *(const u32x4*)(P.k_pool + (kb + i16) * D + dofs[c])
                                    : u32x4{0, 0, 0, 0};
    }
  };

  int buf = 0;                                 // LDS buffer of the group in flight
  bool pre = false;                            // the item's first group already in flight
  // one set of key registers: a group's keys are scored first, then the next group's keys
  // are loaded into the same registers while the softmax and value products run
  u32x4 kreg[2][NC];
  Grp gcur, gnext;
  Desc cur = describe(min(gw, max(n_items - 1, 0)));
  for (int it = gw; it < n_items; it += W) {
    const bool has_next = it + W < n_items;
    const Desc nxt = describe(has_next ? it + W : it);
    const int h = cur.kvh * G + g;
    const uint16_t* qrow = P.q + ((size_t)cur.row * P.Hq + h) * D;
    float m = -INFINITY, l = 0.f;
    f32x4 o[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{};
    float qr[NC][8];

    auto qexact = [&](int n) {                 // qr := R(n) q_row
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
    // qr := R(p - off) q for the group at entry t0, per lane: exact at the item's first group;
    // otherwise every member's offset has moved on by two blocks since the previous group
    // (constant delta inside an item), so qr advances by R(-32). t0 is wave-uniform, so the
    // choice is a uniform branch and qr is updated in place.
    auto set_q = [&](int t0, int off) {
      if (t0 != 0) {
#pragma unroll
        for (int c = 0; c < HC; ++c)
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {     // R(-32)
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
        qexact(cur.p - off);
      }
    };
    auto scores = [&](int b, const u32x2* tab) {   // tab: R(j) (b = 0) or R(16 + j) (b = 1)
      f32x4 S = {};
#pragma unroll
      for (int c = 0; c < HC; ++c) {
        u32x4 qlo, qhi, lo, hi;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qlo[i] = pack_f16(qr[c][2 * i], qr[c][2 * i + 1]);
          qhi[i] = pack_f16(qr[c + HC][2 * i], qr[c + HC][2 * i + 1]);
          const float a0 = bf_lo(kreg[b][c][i]), a1 = bf_hi(kreg[b][c][i]);
          const float b0 = bf_lo(kreg[b][c + HC][i]), b1 = bf_hi(kreg[b][c + HC][i]);
          const u32x2 t = tab[((c * 4 + q4) * 4 + i) * 16 + i16];
          const u32x2 r = rot_h2(pack_f16(a0, a1), pack_f16(b0, b1), t[0], t[1]);
          lo[i] = r[0];
          hi[i] = r[1];
        }
        S = mfma16h(as_f16x8(lo), as_f16x8(qlo), S);
        S = mfma16h(as_f16x8(hi), as_f16x8(qhi), S);
      }
      return S;
    };

    if (!pre && cur.len > 0) {
      issue(cur, 0, buf, gnext);
      issue_k(gnext, kreg);
    }
    pre = false;
    for (int t0 = 0; t0 < cur.len; t0 += 2) {
      __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0): this group's keys and values
      asm volatile("" ::: "memory");
      wave_sync();
      gcur = gnext;
      bool more = false;                       // a next group (this item's or the next's)
      if (t0 + 2 < cur.len) {
        issue(cur, t0 + 2, buf ^ 1, gnext);
        more = true;
      } else if (has_next && nxt.len > 0) {    // the next item's first group
        issue(nxt, 0, buf ^ 1, gnext);
        pre = true;
        more = true;
      }
      const bool has1 = t0 + 1 < cur.len;
      set_q(t0, gcur.off[0]);                  // one q' per group (see above)
      const f32x4 S0 = scores(0, slot_tab);
      f32x4 S1 = {};
      if (has1) S1 = scores(1, slot_tab16);
      if (more) issue_k(gnext, kreg);          // this group's keys are read: refill
      float sc[8];
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int nv = b ? (has1 ? gcur.nv[1] : 0) : gcur.nv[0];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * q4 + i;
          const float v = b ? S1[i] : S0[i];
          const bool ok = j < nv && gcur.off[b] + j <= cur.p;
          sc[4 * b + i] = ok ? v * P.scale_log2 : -INFINITY;
          mx = fmaxf(mx, sc[4 * b + i]);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));      // over the 4 lanes of this column
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m - m_use);
      float pr[8];
      float rsum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pr[i] = exp2f(sc[i] - m_use);
        rsum += pr[i];
      }
      l = l * alpha + rsum;
      m = m_new;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;
      const u32x4 bp = {pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3]),
                        pack_bf16(pr[4], pr[5]), pack_bf16(pr[6], pr[7])};
      // O^T += V^T P^T over the group's 32 keys
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
    // partial of this lane's column: the row sum over the column's 4 lanes
    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    if (cur.slot >= 0) {
      float* part = P.partials + ((size_t)cur.slot * P.Hq + h) * (D + 4);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) *(f32x4*)(part + 16 * dt + 4 * q4) = o[dt];
      if (q4 == 0) {
        part[D] = m;
        part[D + 1] = lt;
      }
    }
    cur = nxt;
  }
}

}  // namespace lazyattn
