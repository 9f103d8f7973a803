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
// cos/sin; q' = R(p - off_t) q changes by the constant R(-16) from one block to the next
// while delta stays constant, and is recomputed exactly (double-precision phase) only
// where delta changes and at the start of each split.
//
// One wave per (query row, KV head, split); G query heads are the columns of 16x16x32 bf16
// MFMAs: S^T = K~ q'^T per block, O^T += V^T P^T per pair of blocks (V staged in the
// wave's own LDS slice, transposed on read). Partial (m, l, o) per split go to the
// workspace; merge_kernel combines them.
#include "lazyattn_common.h"
#include "lazyattn_kernels.h"

namespace lazyattn {

constexpr int kDecodeWaves = 4;

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D, int G>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_kernel(DecodeParams P) {
  constexpr int NC = D / 32;                  // 32-dim k-steps (16x16x32)
  constexpr int HC = NC / 2;                  // chunk c pairs with chunk c + HC (dims + D/2)
  constexpr int VS = D + 16;                  // LDS row stride (bf16 elements)
  constexpr int VCH = D / 8;                  // 16-byte chunks per value row
  __shared__ __align__(16) uint16_t Vs_all[kDecodeWaves][32 * VS];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint16_t* Vs = Vs_all[w];
  const long long item = (long long)blockIdx.x * kDecodeWaves + w;
  const int kvh = blockIdx.y;
  if (item >= P.dec_prefix[P.num_seqs]) return;      // per wave; no workgroup barriers below
  const int it = (int)item;
  const int seq = upper_seq(P.dec_prefix, P.num_seqs, it);
  const int local = it - P.dec_prefix[seq];
  const int q0 = P.q_indptr[seq];
  const int e0 = P.block_table[seq], T = P.block_table[seq + 1] - e0;
  const int kvlen = P.kv_lens[seq];
  int splits = T < P.splits ? T : P.splits;
  if (splits < 1) splits = 1;
  const int row = local / splits, sp = local % splits;
  const int bps = (T + splits - 1) / splits;
  const int eb = sp * bps;
  const int ee = min(T, eb + bps);
  const int r = q0 + row;
  const int p = P.q_pos[r];

  const int i16 = lane & 15, q4 = lane >> 4;
  const bool head_ok = i16 < G;
  const int h = kvh * G + (head_ok ? i16 : 0);

  // lane's frequencies: k = 32c + 8 q4 + e for c < HC, e < 8 (same set for K and q')
  // R(j) with j = i16 (slot of this lane's key row) and R(16)
  float cj[HC][8], sj[HC][8], c16[HC][8], s16[HC][8];
#pragma unroll
  for (int c = 0; c < HC; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double f = P.freqs[32 * c + 8 * q4 + e];
      rope_cos_sin(i16, f, cj[c][e], sj[c][e]);
      rope_cos_sin(16, f, c16[c][e], s16[c][e]);
    }
  const uint16_t* qrow = P.q + ((size_t)r * P.Hq + h) * D;

  float qr[NC][8];                 // q' = R(p - off_t) q in fp32
  u32x4 qb[NC];                    // fp16 B operand of q'
  int cur_delta = 0;
  bool anchored = false;

  float m = -INFINITY, l = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{};

  for (int t0 = eb; t0 < ee; t0 += 2) {
    f32x4 sc[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int t = t0 + bb;
      sc[bb] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      const bool blk = t < ee;
      const uint32_t wd = blk ? P.block_meta[e0 + t] : 0u;
      const int id = word_id(wd), delta = word_delta(wd);
      const int off = t * kBlock + delta;
      const int rem = kvlen - t * kBlock;
      const int nval = (blk && id < P.num_blocks) ? (rem < kBlock ? (rem > 0 ? rem : 0) : kBlock)
                                                  : 0;
      const size_t base = ((size_t)id * P.Hkv + kvh) * kBlock;
      // value rows -> LDS slice rows 16*bb .. 16*bb+15 (zero where the slot is not valid)
#pragma unroll
      for (int u0 = 0; u0 < 16 * VCH; u0 += 64) {
        const int u = u0 + lane;
        const int j = u / VCH, c8 = u % VCH;
        u32x4 v = {0, 0, 0, 0};
        if (j < nval) v = *(const u32x4*)(P.v_pool + (base + j) * D + 8 * c8);
        *(u32x4*)(Vs + (16 * bb + j) * VS + 8 * c8) = v;
      }
      if (!blk) continue;                      // uniform
      // q' for this block: exact re-anchor on a delta change, else advance by R(-16)
      if (!anchored || delta != cur_delta) {
        const int n = p - off;
#pragma unroll
        for (int c = 0; c < HC; ++c) {
          const u32x4 va = head_ok ? *(const u32x4*)(qrow + 32 * c + 8 * q4) : u32x4{0, 0, 0, 0};
          const u32x4 vb = head_ok ? *(const u32x4*)(qrow + 32 * (c + HC) + 8 * q4)
                                   : u32x4{0, 0, 0, 0};
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
        anchored = true;
        cur_delta = delta;
      } else {
#pragma unroll
        for (int c = 0; c < HC; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) {   // R(-16): angle -16 theta_k
            const float a = qr[c][e], b = qr[c + HC][e];
            qr[c][e] = a * c16[c][e] + b * s16[c][e];
            qr[c + HC][e] = b * c16[c][e] - a * s16[c][e];
          }
      }
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) qb[c][i] = pack_f16(qr[c][2 * i], qr[c][2 * i + 1]);

      // keys of this block: lane row = slot i16, dims 32c + 8 q4 + e, rotated by R(i16)
      u32x4 kr[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c)
        kr[c] = i16 < nval ? *(const u32x4*)(P.k_pool + (base + i16) * D + 32 * c + 8 * q4)
                           : u32x4{0, 0, 0, 0};
      f32x4 acc = f32x4{};
#pragma unroll
      for (int c = 0; c < HC; ++c) {
        u32x4 lo, hi;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a0 = bf_lo(kr[c][i]), a1 = bf_hi(kr[c][i]);
          const float b0 = bf_lo(kr[c + HC][i]), b1 = bf_hi(kr[c + HC][i]);
          const float c0 = cj[c][2 * i], s0 = sj[c][2 * i], c1 = cj[c][2 * i + 1], s1 = sj[c][2 * i + 1];
          lo[i] = pack_f16(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
          hi[i] = pack_f16(a0 * s0 + b0 * c0, a1 * s1 + b1 * c1);
        }
        acc = mfma16h(as_f16x8(lo), as_f16x8(qb[c]), acc);
        acc = mfma16h(as_f16x8(hi), as_f16x8(qb[c + HC]), acc);
      }
      // acc[i]: slot 4 q4 + i, head column i16
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 4 * q4 + i;
        const bool ok = j < nval && off + j <= p;
        sc[bb][i] = ok ? acc[i] * P.scale_log2 : -INFINITY;
      }
    }
    // online softmax over the 8 scores of this lane's head; row max across the 4 slot groups
    float mx = -INFINITY;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[bb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m - m_use);
    float pr[2][4];
    float rs = 0.f;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i) { pr[bb][i] = exp2f(sc[bb][i] - m_use); rs += pr[bb][i]; }
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;

    const u32x4 bp = {pack_bf16(pr[0][0], pr[0][1]), pack_bf16(pr[0][2], pr[0][3]),
                      pack_bf16(pr[1][0], pr[1][1]), pack_bf16(pr[1][2], pr[1][3])};
    wave_sync();                                 // value rows written by other lanes
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const int n0 = 16 * dt + 4 * (i16 & 3);
      const u32x2 r1 = lds_read_tr(Vs + (4 * q4 + (i16 >> 2)) * VS + n0);
      const u32x2 r2 = lds_read_tr(Vs + (16 + 4 * q4 + (i16 >> 2)) * VS + n0);
      const u32x4 a = {r1[0], r1[1], r2[0], r2[1]};
      o[dt] = mfma16(as_bf16x8(a), as_bf16x8(bp), o[dt]);
    }
    wave_sync();                                 // before the next pair overwrites the slice
  }

  // partial (o, m, l) of this split: lane holds head i16, dims 16 dt + 4 q4 + (0..3)
  float lt = l + __shfl_xor(l, 16);
  lt += __shfl_xor(lt, 32);
  if (head_ok) {
    float* part = P.partials + ((size_t)item * P.Hq + h) * (D + 4);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) *(f32x4*)(part + 16 * dt + 4 * q4) = o[dt];
    if (q4 == 0) { part[D] = m; part[D + 1] = lt; }
  }
}

template <int D>
static hipError_t launch_d(const DecodeParams& p, int G, long long grid_items, hipStream_t st) {
  dim3 grid((unsigned)((grid_items + kDecodeWaves - 1) / kDecodeWaves), p.Hkv);
  dim3 block(kDecodeWaves * 64);
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_kernel<D, 1>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((decode_kernel<D, 2>), grid, block, 0, st, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<D, 4>), grid, block, 0, st, p); break;
    case 8: hipLaunchKernelGGL((decode_kernel<D, 8>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int D, int G, long long grid_items,
                         hipStream_t st) {
  if (grid_items <= 0) return hipSuccess;
  return D == 128 ? launch_d<128>(p, G, grid_items, st) : launch_d<64>(p, G, grid_items, st);
}

}  // namespace lazyattn
