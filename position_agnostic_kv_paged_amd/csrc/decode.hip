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
// Work: (row-split, kv-head) items, numbered head-major, are cut into 8 contiguous ranges,
// one per XCD (workgroup b runs on XCD b mod 8), and dealt round-robin to the waves of that
// XCD's workgroups; the grid is exactly resident. With 8 KV heads each XCD reads one head,
// so rows that share a document share that head's blocks in one L2. Each wave first describes all of its items
// at once, one item per lane (sequence, query row and position, entry range), so starting
// an item costs no dependent memory round trips; the first key/value group of the next
// item is fetched while the last group of the current one is multiplied. Keys are
// prefetched one group ahead into registers; values go straight
// from global memory into a double-buffered, XOR-swizzled LDS slice of the wave
// (global_load_lds) and are read back transposed (ds_read_b64_tr_b16) as the A operand of
// O^T += V^T P^T. Rows that must contribute nothing (padding, missing blocks) are fetched
// from a zeroed workspace chunk so that 0 * NaN never enters the sum. Each item writes a
// partial (o, m, l); merge_kernel combines the splits of a row.
#include "decode_body.h"
#include "decode_plan.h"
#include <atomic>

namespace lazyattn {

template <int D, int G, int PE>
__global__ __launch_bounds__(kDecodeWaves * 64, 2) void decode_kernel(DecodeParams P) {
  __shared__ __align__(16) uint8_t lds_all[kDecodeWaves][decode_wave_lds_bytes<D>()];
  __shared__ DecodeTables<D> TB;
  // a call whose batch has no single-row sequence (a pure prefill batch) leaves no work:
  // leave before the per-workgroup constants. Row-splits past the partial buffer (only
  // possible when q_indptr runs past total_q) are never started.
  const int n_items = min(P.dec_prefix[P.num_seqs], P.rowsplit_cap) * P.Hkv;
  if (n_items == 0) return;
  decode_tables_init<D, G, PE>(P, TB, kDecodeWaves * 64);
  __syncthreads();
  const int w = threadIdx.x >> 6;
  // XCD x (of X = 8, or fewer for a grid below 8) takes items [n x / X, n (x + 1) / X)
  const int X = min(8, (int)gridDim.x), x = blockIdx.x % X, bx = blockIdx.x / X;
  const int nbx = ((int)gridDim.x - x + X - 1) / X;              // workgroups on XCD x
  const int lo = (int)((long long)n_items * x / X);
  const int hi = (int)((long long)n_items * (x + 1) / X);
  decode_items<D, G, PE>(P, TB, lds_all[w], lo + bx * kDecodeWaves + w, nbx * kDecodeWaves,
                         hi);
}

// Shared-document decode: items from a host plan (decode_plan.h), dealt round-robin to the
// resident waves like decode_kernel's. A plan whose header does not match the call does
// nothing here (and merge_kernel then writes zero rows).
template <int D, int G>
__global__ __launch_bounds__(kDecodeWaves * 64, 2) void decode_plan_kernel(DecodeParams P,
                                                                          const int32_t* plan,
                                                                          int n_plan,
                                                                          int n_slots) {
  __shared__ __align__(16) uint8_t lds_all[kDecodeWaves][decode_wave_lds_bytes<D>()];
  __shared__ DecodeTables<D> TB;
  __shared__ PairTable<D> PT;
  if (!share_plan_ok(plan, 16 / G, P.total_q, P.num_seqs)) return;
  n_plan = min(n_plan, plan[4]);
  n_slots = min(n_slots, plan[5]);
  if (n_plan <= 0) return;
  decode_pair_tables_init<D>(P, TB, PT, kDecodeWaves * 64);      // R(j), R(16 + j), R(32)
  __syncthreads();
  const int w = threadIdx.x >> 6;
  decode_plan_items<D, G>(P, TB, PT, lds_all[w], plan, n_plan, n_slots,
                          blockIdx.x * kDecodeWaves + w, gridDim.x * kDecodeWaves,
                          n_plan * P.Hkv);
}

// Compute units of each device, queried once per device. Host threads calling at the same
// time may both fill an entry; they store the same value, and the atomics make that race
// well-defined.
constexpr int kMaxDevices = 64;
static std::atomic<int> g_num_cus[kMaxDevices];

static int num_cus() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  if (dev >= 0) {
    const int known = g_num_cus[dev].load(std::memory_order_relaxed);
    if (known > 0) return known;
  }
  int n = 0;
  if (dev < 0 ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    n = 256;                                         // MI355X (also when no device is visible)
  if (dev >= 0) g_num_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

int decode_resident_waves() { return num_cus() * kDecodeWgPerCu * kDecodeWaves; }

template <int D, int PE>
static hipError_t launch_dr(const DecodeParams& p, int G, hipStream_t st) {
  dim3 grid(num_cus() * kDecodeWgPerCu), block(kDecodeWaves * 64);
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_kernel<D, 1, PE>), grid, block, 0, st, p); break;
    case 2: hipLaunchKernelGGL((decode_kernel<D, 2, PE>), grid, block, 0, st, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<D, 4, PE>), grid, block, 0, st, p); break;
    case 8: hipLaunchKernelGGL((decode_kernel<D, 8, PE>), grid, block, 0, st, p); break;
    case 16: hipLaunchKernelGGL((decode_kernel<D, 16, PE>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const DecodeParams& p, int G, int pe, hipStream_t st) {
  switch (pe) {
    case kRope: return launch_dr<D, kRope>(p, G, st);
    case kStored: return launch_dr<D, kStored>(p, G, st);
    case kAlibi: return launch_dr<D, kAlibi>(p, G, st);
    case kRopePartial: return launch_dr<D, kRopePartial>(p, G, st);
    case kDocRotated: return launch_dr<D, kDocRotated>(p, G, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeParams& p, int D, int G, int pe, hipStream_t st) {
  return D == 128 ? launch_d<128>(p, G, pe, st) : launch_d<64>(p, G, pe, st);
}

template <int D>
static hipError_t launch_plan_d(const DecodeParams& p, const int32_t* plan, int n_plan,
                                int n_slots, int G, hipStream_t st) {
  dim3 grid(num_cus() * kDecodeWgPerCu), block(kDecodeWaves * 64);
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_plan_kernel<D, 1>), grid, block, 0, st, p, plan, n_plan, n_slots); break;
    case 2: hipLaunchKernelGGL((decode_plan_kernel<D, 2>), grid, block, 0, st, p, plan, n_plan, n_slots); break;
    case 4: hipLaunchKernelGGL((decode_plan_kernel<D, 4>), grid, block, 0, st, p, plan, n_plan, n_slots); break;
    case 8: hipLaunchKernelGGL((decode_plan_kernel<D, 8>), grid, block, 0, st, p, plan, n_plan, n_slots); break;
    case 16: hipLaunchKernelGGL((decode_plan_kernel<D, 16>), grid, block, 0, st, p, plan, n_plan, n_slots); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_plan(const DecodeParams& p, const int32_t* plan, int n_plan,
                              int n_slots, int D, int G, hipStream_t st) {
  return D == 128 ? launch_plan_d<128>(p, plan, n_plan, n_slots, G, st)
                  : launch_plan_d<64>(p, plan, n_plan, n_slots, G, st);
}

}  // namespace lazyattn
