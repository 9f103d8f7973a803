// Measured ceilings for reporting: an MFMA loop (the matrix-core rate the prefill kernel's
// 32x32x16 fp16/bf16 products can reach, and the shader clock it runs at), a plain stream
// read of device memory and a random gather of fixed-size chunks (the rates the decode
// kernel's traffic can reach, streamed and as a paged kernel reads it).
#include "lazyattn_common.h"
#include "lazyattn_kernels.h"

namespace lazyattn {

constexpr int kProbeWaves = 8;               // two waves per SIMD, as the prefill kernel

// Every wave runs `iters` x 16 independent 32x32x16 fp16 MFMAs (four accumulator chains) and
// records its s_memtime span; results are folded into out so nothing is optimised away.
__global__ __launch_bounds__(kProbeWaves * 64, 1) void probe_mfma_kernel(int iters,
                                                                        unsigned long long* cyc,
                                                                        float* out) {
  __shared__ float pad[24000];                // one workgroup per CU
  const int tid = threadIdx.x;
  if (tid == 0) pad[0] = 0.f;
  f16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)((tid & 7) * 0.01f);
    b[i] = (_Float16)(i * 0.01f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float s = pad[0];
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * kProbeWaves * 64 + tid] = s;
  if ((tid & 63) == 0) cyc[blockIdx.x * kProbeWaves + (tid >> 6)] = t1 - t0;
}

// Grid-stride 16-byte loads over `bytes` (a multiple of 16); XOR folded per thread.
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* buf, size_t n16,
                                                         uint32_t* out) {
  uint32_t x = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(buf + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = x;
}

// Random gather of whole chunks: wave w reads chunks idx[w], idx[w + W], ... (each
// `c16` 16-byte units, read by the 64 lanes together), the access pattern of a paged
// kernel over randomly placed blocks. Chunk ids outside [0, n_total) are skipped.
__global__ __launch_bounds__(256) void probe_gather_kernel(const u32x4* buf, const int32_t* idx,
                                                           int n_idx, int n_total, int c16,
                                                           uint32_t* out) {
  const int lane = threadIdx.x & 63;
  const int wave = (int)((blockIdx.x * 256 + threadIdx.x) >> 6);
  const int nw = (int)(gridDim.x * 4);
  uint32_t x = 0;
  for (int i = wave; i < n_idx; i += nw) {
    const int id = idx[i];
    if ((unsigned)id >= (unsigned)n_total) continue;
    const u32x4* c = buf + (size_t)id * c16;
    for (int k = lane; k < c16; k += 64) {
      const u32x4 v = c[k];
      x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = x;
}

hipError_t launch_probe_gather(const void* buf, size_t bytes, const int32_t* idx, int n_idx,
                               int chunk_bytes, int num_wg, uint32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(probe_gather_kernel, dim3(num_wg), dim3(256), 0, st, (const u32x4*)buf,
                     idx, n_idx, (int)(bytes / (size_t)chunk_bytes), chunk_bytes / 16, out);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int num_cus, int iters, unsigned long long* cyc, float* out,
                             hipStream_t st) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(num_cus), dim3(kProbeWaves * 64), 0, st, iters,
                     cyc, out);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* buf, size_t bytes, int num_wg, uint32_t* out,
                             hipStream_t st) {
  hipLaunchKernelGGL(probe_read_kernel, dim3(num_wg), dim3(256), 0, st, (const u32x4*)buf,
                     bytes / 16, out);
  return hipGetLastError();
}

}  // namespace lazyattn
