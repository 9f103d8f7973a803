// LazyAttention prefill kernel for gfx950 (bf16 MFMA, online softmax).
//
// Technical summary of LazyAttention (arXiv 2606.04302), "Technical Implementation",
// prefilling phase: cached KV blocks are loaded from the position-free cache and, instead
// of rotating each key twice (back to position zero, then to its target), every key tile is
// rotated ONCE per query tile by the offset between the tile and the key's logical
// position. "Mathematical Equivalence": RoPE scores depend only on n - m, so
//   <R(p) q, R(L) k> = <R(p - p_ref) q, R(L - p_ref) k>
// for any reference position p_ref; the kernel takes p_ref = the tile's first query
// position, rotates the tile's queries by R(p - p_ref) once, and rotates each staged key by
// R(L - p_ref) once per (query tile, key tile) -- the key rotation is shared by all
// 32 * NW rows of the workgroup tile, which is what keeps it a small overhead.
//
// Workgroup tile: NW waves x 32 rows; rows are (query position, head-in-group) pairs so the
// G query heads of one KV head share every staged key/value tile (grouped-query packing).
// Per wave, S^T = K~ Q~^T and O^T += V^T P^T on 32x32x16 bf16 MFMA: each lane owns one
// query row (MFMA column), so row max / row sum are in-lane plus one cross-half exchange.
// V is staged row-major in LDS and transposed on read by ds_read_b64_tr_b16.
#include "lazyattn_common.h"
#include "lazyattn_kernels.h"
#include <limits.h>

namespace lazyattn {

constexpr int kPrefillWaves = 8;

template <int D, int G, bool ROTATE>
__global__ __launch_bounds__(kPrefillWaves * 64, 1) void prefill_kernel(PrefillParams P) {
  constexpr int NW = kPrefillWaves;
  constexpr int NT = NW * 64;
  constexpr int ROWS = 32 * NW;
  constexpr int POS = ROWS / G;               // query positions per tile
  constexpr int NK = 64;                      // keys per key tile (4 blocks)
  constexpr int HALF = D / 2;
  constexpr int NCH = D / 16;                 // 16-dim k-steps of QK^T
  constexpr int KS = D + 8;                   // LDS row strides (bf16 elements)
  constexpr int VS = D + 16;
  constexpr int KU = NK * (HALF / 8);         // key staging units: (key, 8-dim pair chunk)
  constexpr int VU = NK * (D / 8);            // value staging units: (key, 8-dim chunk)

  __shared__ __align__(16) uint16_t Ks[NK * KS];
  __shared__ __align__(16) uint16_t Vs[NK * VS];
  __shared__ double fr_s[HALF];
  __shared__ int pmax_s;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kvh = blockIdx.y;
  const int tile_id = blockIdx.x;
  if (tile_id >= P.pf_prefix[P.num_seqs]) return;          // uniform per workgroup
  const int seq = upper_seq(P.pf_prefix, P.num_seqs, tile_id);
  const int qt = tile_id - P.pf_prefix[seq];
  const int q0 = P.q_indptr[seq], qlen = P.q_indptr[seq + 1] - q0;
  const int e0 = P.block_table[seq], T = P.block_table[seq + 1] - e0;
  const int kvlen = P.kv_lens[seq];
  const int p_ref = ROTATE ? P.q_pos[q0 + qt * POS] : 0;

  for (int i = tid; i < HALF; i += NT) fr_s[i] = P.freqs[i];
  if (tid == 0) pmax_s = INT_MIN;
  __syncthreads();

  // ---- this lane's query row -------------------------------------------------------------
  const int col = lane & 31, hh = lane >> 5;
  const int rho = 32 * w + col;
  const int qi = qt * POS + rho / G;
  const int h = kvh * G + rho % G;
  const bool row_ok = qi < qlen;
  const int p = row_ok ? P.q_pos[q0 + qi] : INT_MIN;       // invalid rows see no key

  // B operand chunks: lane holds dims 16c + 8hh + e (e < 8) of its row; the rotate-half
  // partner of chunk c is chunk c + NCH/2 (dims + D/2), in the same lane.
  u32x4 qb[NCH];
  {
    u32x4 raw[NCH];
    const uint16_t* qrow = P.q + ((size_t)(q0 + (row_ok ? qi : 0)) * P.Hq + h) * D;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      raw[c] = row_ok ? *(const u32x4*)(qrow + 16 * c + 8 * hh) : u32x4{0, 0, 0, 0};
    const int n = row_ok ? p - p_ref : 0;
#pragma unroll
    for (int c = 0; c < NCH / 2; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a0 = bf_lo(raw[c][i]), a1 = bf_hi(raw[c][i]);
        float b0 = bf_lo(raw[c + NCH / 2][i]), b1 = bf_hi(raw[c + NCH / 2][i]);
        float c0, s0, c1, s1;
        rope_cos_sin(n, fr_s[16 * c + 8 * hh + 2 * i], c0, s0);
        rope_cos_sin(n, fr_s[16 * c + 8 * hh + 2 * i + 1], c1, s1);
        qb[c][i] = pack_f16(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
        qb[c + NCH / 2][i] = pack_f16(a0 * s0 + b0 * c0, a1 * s1 + b1 * c1);
      }
    }
  }

  // wave / workgroup extents of the query positions (for tile skipping and masking)
  int pmax_w = p, pmin_w = row_ok ? p : INT_MAX;
  for (int o = 32; o >= 1; o >>= 1) {
    pmax_w = max(pmax_w, __shfl_xor(pmax_w, o));
    pmin_w = min(pmin_w, __shfl_xor(pmin_w, o));
  }
  if (lane == 0) atomicMax(&pmax_s, pmax_w);
  __syncthreads();
  const int pmax_g = pmax_s;

  float m = -INFINITY, l = 0.f;
  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};

  const int n_kt = (T + 3) / 4;
  for (int kt = 0; kt < n_kt; ++kt) {
    // the tile's four words (uniform loads)
    uint32_t wd[4];
    int off[4], nval[4];
    int kmin = INT_MAX, kmax = INT_MIN;
    bool tile_full = true;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int ent = 4 * kt + b;
      if (ent < T) {
        wd[b] = P.block_meta[e0 + ent];
        off[b] = word_offset(wd[b], ent);
        const int rem = kvlen - ent * kBlock;
        nval[b] = rem < kBlock ? (rem > 0 ? rem : 0) : kBlock;
        if (word_id(wd[b]) >= P.num_blocks) nval[b] = 0;      // out-of-pool id: never read
      } else {
        wd[b] = 0; off[b] = 0; nval[b] = 0;
      }
      if (nval[b] > 0) {
        kmin = min(kmin, off[b]);
        kmax = max(kmax, off[b] + nval[b] - 1);
      }
      if (nval[b] != kBlock) tile_full = false;
    }
    if (kmin > pmax_g) continue;                                // nothing visible: skip tile

    // ---- stage: rotated keys and raw values into LDS ---------------------------------
    for (int u = tid; u < KU; u += NT) {
      const int n = u / (HALF / 8), cp = u % (HALF / 8);
      const int b = n >> 4, j = n & 15;
      u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
      if (j < nval[b]) {
        const uint16_t* src = P.k_pool +
            (((size_t)word_id(wd[b]) * P.Hkv + kvh) * kBlock + j) * D + 8 * cp;
        lo = *(const u32x4*)src;
        hi = *(const u32x4*)(src + HALF);
        const int nrel = off[b] + j - p_ref;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float a0 = bf_lo(lo[i]), a1 = bf_hi(lo[i]);
          float b0 = bf_lo(hi[i]), b1 = bf_hi(hi[i]);
          if (ROTATE) {
            float c0, s0, c1, s1;
            rope_cos_sin(nrel, fr_s[8 * cp + 2 * i], c0, s0);
            rope_cos_sin(nrel, fr_s[8 * cp + 2 * i + 1], c1, s1);
            lo[i] = pack_f16(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
            hi[i] = pack_f16(a0 * s0 + b0 * c0, a1 * s1 + b1 * c1);
          } else {
            lo[i] = pack_f16(a0, a1);
            hi[i] = pack_f16(b0, b1);
          }
        }
      }
      *(u32x4*)(Ks + n * KS + 8 * cp) = lo;
      *(u32x4*)(Ks + n * KS + HALF + 8 * cp) = hi;
    }
    for (int u = tid; u < VU; u += NT) {
      const int n = u / (D / 8), c8 = u % (D / 8);
      const int b = n >> 4, j = n & 15;
      u32x4 v = {0, 0, 0, 0};
      if (j < nval[b])
        v = *(const u32x4*)(P.v_pool +
                            (((size_t)word_id(wd[b]) * P.Hkv + kvh) * kBlock + j) * D + 8 * c8);
      *(u32x4*)(Vs + n * VS + 8 * c8) = v;
    }
    __syncthreads();

    // ---- compute (per wave) ---------------------------------------------------------------
    if (kmin <= pmax_w) {
      const bool nomask = tile_full && kmax <= pmin_w;
      f32x16 s[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        s[t] = f32x16{};
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const u32x4 a = *(const u32x4*)(Ks + (32 * t + col) * KS + 16 * c + 8 * hh);
          s[t] = mfma32h(as_f16x8(a), as_f16x8(qb[c]), s[t]);
        }
      }
      // s[t][r]: key n = 32t + (r/4)*8 + 4hh + r%4 of this lane's row
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = s[t][r] * P.scale_log2;
          if (!nomask) {
            const int b = 2 * t + (r >> 3);
            const int j = ((r >> 2) & 1) * 8 + 4 * hh + (r & 3);
            const bool ok = j < nval[b] && off[b] + j <= p;
            v = ok ? v : -INFINITY;
          }
          s[t][r] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m - m_use);
      float rs = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = exp2f(s[t][r] - m_use);
          s[t][r] = e;
          rs += e;
        }
      }
      l = l * alpha + rs;
      m = m_new;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;

      const int gi = lane >> 4, i16 = lane & 15;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          u32x4 bp;
#pragma unroll
          for (int i = 0; i < 4; ++i) bp[i] = pack_bf16(s[t][8 * kk + 2 * i], s[t][8 * kk + 2 * i + 1]);
          const int k0 = 32 * t + 16 * kk + 4 * hh + (i16 >> 2);
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            const int n0 = 32 * dt + 16 * (gi & 1) + 4 * (i16 & 3);
            const u32x2 r1 = lds_read_tr(Vs + k0 * VS + n0);
            const u32x2 r2 = lds_read_tr(Vs + (k0 + 8) * VS + n0);
            const u32x4 a = {r1[0], r1[1], r2[0], r2[1]};
            o[dt] = mfma32(as_bf16x8(a), as_bf16x8(bp), o[dt]);
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue: O / l -> bf16 ----------------------------------------------------------
  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (row_ok) {
    uint16_t* dst = P.out + ((size_t)(q0 + qi) * P.Hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        u32x2 v;
        v[0] = pack_bf16(o[dt][4 * r4] * inv, o[dt][4 * r4 + 1] * inv);
        v[1] = pack_bf16(o[dt][4 * r4 + 2] * inv, o[dt][4 * r4 + 3] * inv);
        *(u32x2*)(dst + 32 * dt + 8 * r4 + 4 * hh) = v;
      }
    }
  }
}

int prefill_positions_per_tile(int G) { return 32 * kPrefillWaves / G; }

template <int D, int G>
static hipError_t launch_dg(const PrefillParams& p, int grid_tiles, bool rotate, hipStream_t st) {
  dim3 grid(grid_tiles, p.Hkv), block(kPrefillWaves * 64);
  if (rotate) hipLaunchKernelGGL((prefill_kernel<D, G, true>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((prefill_kernel<D, G, false>), grid, block, 0, st, p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const PrefillParams& p, int G, int grid_tiles, bool rotate,
                           hipStream_t st) {
  switch (G) {
    case 1: return launch_dg<D, 1>(p, grid_tiles, rotate, st);
    case 2: return launch_dg<D, 2>(p, grid_tiles, rotate, st);
    case 4: return launch_dg<D, 4>(p, grid_tiles, rotate, st);
    case 8: return launch_dg<D, 8>(p, grid_tiles, rotate, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillParams& p, int D, int G, int grid_tiles, bool rotate,
                          hipStream_t st) {
  if (grid_tiles <= 0) return hipSuccess;
  return D == 128 ? launch_d<128>(p, G, grid_tiles, rotate, st)
                  : launch_d<64>(p, G, grid_tiles, rotate, st);
}

}  // namespace lazyattn
