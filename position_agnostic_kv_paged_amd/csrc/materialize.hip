// Materialisation of a position-adjusted KV copy: the work LazyAttention avoids.
//
// Technical summary of LazyAttention (arXiv 2606.04302), "Mathematical Equivalence" and the
// comparison with reuse schemes that store position-dependent copies: placing a cached
// document at a new position normally means writing its keys again with the rotation of
// that position. This kernel does exactly that for a whole batch, so that the copy plus
// plain paged attention over it (the *_rotated_pool entry points) can be timed against the
// deferred rotation. Every block-table entry e gets a private destination block e:
// keys rotated to their absolute logical positions, values copied, and a new packed word
// with block id e and the same offset delta.
//
// Persistent workgroups walk the entries; per entry the workgroup builds cos/sin of
// (off_e theta_k) in LDS and combines it with the loop-invariant slot table R(j), so each
// (key, frequency pair) costs four multiply-adds for the angle and four for the rotation.
#include "lazyattn_common.h"
#include "lazyattn_kernels.h"

namespace lazyattn {

template <int D>
__global__ __launch_bounds__(256) void materialize_kernel(MaterializeParams P) {
  constexpr int HALF = D / 2;
  constexpr int NT = 256;
  __shared__ float2 slot_cs[kBlock * HALF];          // cos/sin(j theta_k), j < 16
  __shared__ float2 blk_cs[HALF];                    // cos/sin(off_e theta_k) of the entry
  const int tid = threadIdx.x;
  for (int i = tid; i < kBlock * HALF; i += NT) {
    float c, s;
    rope_cos_sin(i / HALF, P.fr.f[i % HALF], c, s);
    slot_cs[i] = make_float2(c, s);
  }
  const int total = min(P.n_entries, P.block_table[P.num_seqs]);
  for (int e = blockIdx.x; e < total; e += gridDim.x) {
    const int seq = upper_seq(P.block_table, P.num_seqs, e);
    const int t = e - P.block_table[seq];
    const uint32_t w = P.block_meta[e];
    const int id = word_id(w), off = word_offset(w, t);
    int nv = min(max(P.kv_lens[seq] - t * kBlock, 0), kBlock);
    if (id >= P.num_blocks) nv = 0;                  // out-of-pool id: never read
    __syncthreads();                                 // the previous entry's angles are used
    if (tid < HALF) {
      float c, s;
      rope_cos_sin(off, P.fr.f[tid], c, s);
      blk_cs[tid] = make_float2(c, s);
    }
    if (tid == 0) P.dst_meta[e] = (w & ~kIdMask) | (uint32_t)e;
    __syncthreads();
    // keys: unit = (head g, slot j, 8 frequencies); slots past the sequence are zero
    constexpr int KCH = HALF / 8;
    for (int u = tid; u < P.Hkv * kBlock * KCH; u += NT) {
      const int ch = u % KCH, j = (u / KCH) % kBlock, g = u / (KCH * kBlock);
      u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
      if (j < nv) {
        const uint16_t* src = P.k_pool + (((size_t)id * P.Hkv + g) * kBlock + j) * D + 8 * ch;
        const u32x4 a = *(const u32x4*)src, b = *(const u32x4*)(src + HALF);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float ra[2], rb[2];
#pragma unroll
          for (int v = 0; v < 2; ++v) {
            const int k = 8 * ch + 2 * i + v;
            const float2 bc = blk_cs[k], jc = slot_cs[j * HALF + k];
            const float c = bc.x * jc.x - bc.y * jc.y;      // R(off + j) = R(off) R(j)
            const float s = bc.y * jc.x + bc.x * jc.y;
            const float x = v ? bf_hi(a[i]) : bf_lo(a[i]);
            const float y = v ? bf_hi(b[i]) : bf_lo(b[i]);
            ra[v] = x * c - y * s;
            rb[v] = x * s + y * c;
          }
          lo[i] = pack_bf16(ra[0], ra[1]);
          hi[i] = pack_bf16(rb[0], rb[1]);
        }
      }
      uint16_t* dst = P.dst_k + (((size_t)e * P.Hkv + g) * kBlock + j) * D + 8 * ch;
      *(u32x4*)dst = lo;
      *(u32x4*)(dst + HALF) = hi;
    }
    // values: unit = (head g, slot j, 16-byte chunk), copied as they are
    constexpr int VCH = D / 8;
    for (int u = tid; u < P.Hkv * kBlock * VCH; u += NT) {
      const int ch = u % VCH, j = (u / VCH) % kBlock, g = u / (VCH * kBlock);
      u32x4 v = {0, 0, 0, 0};
      if (j < nv) v = *(const u32x4*)(P.v_pool + (((size_t)id * P.Hkv + g) * kBlock + j) * D + 8 * ch);
      *(u32x4*)(P.dst_v + (((size_t)e * P.Hkv + g) * kBlock + j) * D + 8 * ch) = v;
    }
  }
}

hipError_t launch_materialize(const MaterializeParams& p, int D, int num_wg, hipStream_t st) {
  if (p.n_entries <= 0) return hipSuccess;
  const int nwg = num_wg < p.n_entries ? num_wg : p.n_entries;
  if (D == 128) hipLaunchKernelGGL(materialize_kernel<128>, dim3(nwg), dim3(256), 0, st, p);
  else hipLaunchKernelGGL(materialize_kernel<64>, dim3(nwg), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace lazyattn
