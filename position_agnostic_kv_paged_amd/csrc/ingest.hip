// Ingest of new keys and values into the position-free pool.
//
// Technical summary of LazyAttention (arXiv 2606.04302), "Core Concept": the cache holds
// content-only keys, so the keys a model projects for new tokens (a prefill suffix, a
// decode token, a document seen for the first time) are written into their pool slots
// exactly as projected, with no rotation; position enters only inside the attention
// kernels. One thread moves one 16-byte chunk of one (token, KV head) row of K and of V;
// the 16 threads of a D = 128 row write its 256 contiguous bytes.
#include "lazyattn_common.h"
#include "lazyattn_kernels.h"

namespace lazyattn {

__global__ __launch_bounds__(256) void ingest_kernel(IngestParams P) {
  const int cpr = P.D / 8;                                   // 16-byte chunks per row
  const long long total = (long long)P.n_tokens * P.Hkv * cpr;
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * 256) {
    const int c = (int)(idx % cpr);
    const long long row = idx / cpr;                         // token * Hkv + head
    const int h = (int)(row % P.Hkv);
    const int i = (int)(row / P.Hkv);
    const int s = P.slot_mapping[i];
    const int blk = s >= 0 ? s / P.B : -1, j = s >= 0 ? s % P.B : 0;
    if (blk < 0 || blk >= P.num_blocks) continue;            // unmapped token: skipped
    const size_t src = (size_t)row * P.D + 8 * c;
    const size_t dst = (((size_t)blk * P.Hkv + h) * P.B + j) * P.D + 8 * c;
    const u32x4 k = *(const u32x4*)(P.k_new + src);
    const u32x4 v = *(const u32x4*)(P.v_new + src);
    *(u32x4*)(P.k_pool + dst) = k;
    *(u32x4*)(P.v_pool + dst) = v;
  }
}

hipError_t launch_ingest(const IngestParams& p, int num_wg, hipStream_t st) {
  hipLaunchKernelGGL(ingest_kernel, dim3(num_wg), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace lazyattn
