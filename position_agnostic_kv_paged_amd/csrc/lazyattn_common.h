// Shared device helpers of the LazyAttention kernels (gfx950 only).
//
// Packed words, RoPE phase arithmetic, bf16 packing and MFMA operand types used by the
// prefill, decode and merge kernels. Nothing here is shared with the float64 oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lazyattn {

constexpr int kBlock = 16;                 // tokens per KV block
constexpr int kIdBits = 17;
constexpr uint32_t kIdMask = (1u << kIdBits) - 1u;
constexpr int kMaxHalfDim = 64;            // D <= 128

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// RoPE frequencies in revolutions per position: f_k = base^(-2k/D) / (2 pi), computed on
// the host in double precision and passed by value (kernel argument segment).
struct RopeFreqs {
  double f[kMaxHalfDim];
};

// ---- packed (block id, delta) word ------------------------------------------------------
// bits [16:0] id, bits [31:17] delta = offset - t*B (two's complement). One AND and one
// arithmetic shift; this is the only device decoder, used by every kernel.
__host__ __device__ __forceinline__ int word_id(uint32_t w) { return (int)(w & kIdMask); }
__host__ __device__ __forceinline__ int word_delta(uint32_t w) { return ((int32_t)w) >> kIdBits; }
__host__ __device__ __forceinline__ int word_offset(uint32_t w, int t) {
  return t * kBlock + word_delta(w);
}

// ---- exact RoPE phase --------------------------------------------------------------------
// cos/sin of n * theta_k for an integer n (|n| < 2^31): the angle is reduced in revolutions
// in double precision (n * f_k is exact to ~2^-53 relative, frac() is exact), then the
// hardware sin/cos take the reduced revolution count in [0, 1).
__device__ __forceinline__ void rope_cos_sin(int n, double f, float& c, float& s) {
  double x = (double)n * f;
  x = x - __builtin_floor(x);
  float r = (float)x;
  s = __builtin_amdgcn_sinf(r);
  c = __builtin_amdgcn_cosf(r);
}

// sin(2 pi (frac(n f) + quarter)) from an exact double-precision phase; quarter = 0.25
// gives the cosine.
__device__ __forceinline__ float rope_sin_rev(int n, double f, float quarter) {
  double x = (double)n * f;
  x = x - __builtin_floor(x);
  return __builtin_amdgcn_sinf((float)x + quarter);
}

// ---- bf16 helpers --------------------------------------------------------------------------
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Round two floats to bf16 (nearest even) and pack: a -> low half, b -> high half.
// One v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, h2));
}

// Round two floats to fp16 (nearest even) and pack. The rotated query/key operands of the
// score products are carried in fp16: they come out of fp32 rotation arithmetic anyway,
// and fp16 keeps 3 more mantissa bits than bf16 at the same MFMA rate (element magnitudes
// must stay below 65504).
// One v_cvt_pk_f16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, h2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16h(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16). Within each 16-lane group, lane i
// receives element e = the 16-bit value at (address given by lane 4e + i/4) + (i % 4).
// With lane m supplying &M[k0 + m/4][n0 + 4 (m%4)] of a row-major bf16 matrix M, lane i
// receives M[k0 .. k0+3][n0 + i]: four consecutive rows of one column.
__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// value of v in lane `lane` (a wave-uniform index)
__device__ __forceinline__ int rl(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// c + x.lo + x.hi for two packed bf16 values (v_dot2_f32_bf16 against (1, 1))
__device__ __forceinline__ float sum2_bf16(uint32_t x, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x),
                                         __builtin_bit_cast(bf16x2_t, 0x3F803F80u), c, false);
}

// Combine each lane with lane l ^ 32 (v_permlane32_swap, no LDS round trip). With both
// operands equal, the swap returns {x[l mod 32], x[32 + l mod 32]} in either order, so a
// symmetric combination of the pair needs no lane select.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_add(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max(a, b, c) in one v_max3_f32. Written as inline asm: fmaxf must quiet signalling NaNs,
// so the compiler adds a canonicalising v_max per operand it cannot prove canonical (every
// MFMA result); scores here are finite or -inf.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Max of 16 values: two chains of v_max3.
__device__ __forceinline__ float max16(const f32x16& v) {
  float x = max3f(v[0], v[1], v[2]), y = max3f(v[8], v[9], v[10]);
  x = max3f(x, v[3], v[4]);
  y = max3f(y, v[11], v[12]);
  x = max3f(x, v[5], v[6]);
  y = max3f(y, v[13], v[14]);
  return max3f(max3f(x, v[7], v[15]), y, y);
}

// Max of 32 values: four independent chains of v_max3 (two values per instruction).
__device__ __forceinline__ float max32(const f32x16& a, const f32x16& b) {
  float c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x16& v = j < 2 ? a : b;
    const int o = (j & 1) * 8;
    float x = max3f(v[o], v[o + 1], v[o + 2]);
    x = max3f(x, v[o + 3], v[o + 4]);
    x = max3f(x, v[o + 5], v[o + 6]);
    c[j] = x;
  }
  const float t0 = max3f(c[0], c[1], a[7]), t1 = max3f(c[2], c[3], b[7]);
  return max3f(max3f(t0, t1, a[15]), b[15], b[15]);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Binary search: largest s in [0, n) with prefix[s] <= x (prefix non-decreasing, prefix[0]=0).
__device__ __forceinline__ int upper_seq(const int32_t* prefix, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The same search by one whole wave (every lane calls it; the result is wave-uniform): 64
// probes per round of loads, so up to 64 sequences take one memory round trip instead of
// log2(n) dependent ones. Requires prefix[0] <= x. Returns s and prefix[s].
struct SeqFound {
  int s, start;
};
__device__ __forceinline__ SeqFound wave_upper_seq(const int32_t* prefix, int n, int x,
                                                   int lane) {
  int lo = 0, hi = n;                          // prefix[lo] <= x, answer in [lo, hi)
  while (hi - lo > 64) {
    const int span = hi - lo;
    const int idx = lo + (int)(((long long)lane * span) / 64);
    const unsigned long long bal = __ballot(prefix[idx] <= x);   // lane 0 always set
    const int top = 63 - __builtin_clzll(bal);
    const int nlo = lo + (int)(((long long)top * span) / 64);
    if (top < 63) hi = lo + (int)(((long long)(top + 1) * span) / 64);
    lo = nlo;
  }
  const int span = hi - lo;
  const int v = prefix[lo + min(lane, span - 1)];
  const int top = 63 - __builtin_clzll(__ballot(lane < span && v <= x));
  return SeqFound{__builtin_amdgcn_readfirstlane(lo + top), __builtin_amdgcn_readlane(v, top)};
}

// ---- workspace layout -----------------------------------------------------------------------
// [0, 512)                RoPE frequency table, double [64] (revolutions per position)
// [512, 516)              prefill KV split: key tiles per split (int, written by plan_kernel)
// [516, 768)              reserved; 16-byte zero rows at 576..767
// [768, ...)              prefix arrays: prefill items, decode row-splits, each num_seqs + 1 int32
// aligned 256             split-K partials: float [row-splits][Hq][D + 4]  (o[D], m, l, -, -)
// aligned 256             prefill KV-split partials: float [pf_slots][256 rows][D + 4]
struct WsLayout {
  size_t off_freqs, off_zero, off_pf_prefix, off_dec_prefix, off_partials, off_pf_partials,
      total;
};

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

__host__ __device__ inline WsLayout ws_layout(int num_seqs, long long max_rowsplits, int Hq, int D,
                                              long long pf_slots = 0) {
  WsLayout L;
  L.off_freqs = 0;
  L.off_zero = 576;
  L.off_pf_prefix = 768;
  L.off_dec_prefix = align_up(L.off_pf_prefix + 4ull * (num_seqs + 1), 256);
  L.off_partials = align_up(L.off_dec_prefix + 4ull * (num_seqs + 1), 256);
  L.off_pf_partials =
      align_up(L.off_partials + (size_t)max_rowsplits * Hq * (D + 4) * 4ull, 256);
  L.total = L.off_pf_partials + (size_t)pf_slots * 256ull * (D + 4) * 4ull;
  return L;
}

// KV split of one prefill query tile over n_kt key tiles: at most smax splits of at least kc
// key tiles (the last may be shorter), none empty. n_kt = 0 gives one empty split.
constexpr int kMaxPfSplits = 32;   // splits per prefill tile, at most
constexpr int kPfMinChunk = 8;     // key tiles (of 64 keys) per prefill split, at least

struct PfSplit {
  int splits, chunk;
};
__host__ __device__ inline PfSplit pf_split(int n_kt, int kc, int smax) {
  if (n_kt <= 0) return PfSplit{1, 0};
  int s = n_kt / kc + (n_kt % kc != 0);
  s = s < 1 ? 1 : (s > smax ? smax : s);
  const int chunk = (n_kt + s - 1) / s;
  return PfSplit{(n_kt + chunk - 1) / chunk, chunk};
}

// Decode split size (blocks per item, even, at least 8) for `pairs` (row, KV head) pairs of
// rows holding about T blocks on W resident waves: items are dealt round-robin to the waves
// (within each XCD's eighth of them), so the choice aims at an item count that is a whole
// multiple of W -- every wave gets the same number of equal items. Among 1 .. 8 items per
// wave the candidate with the least idle share wins; ties go to fewer, longer items (fewer
// partials to merge).
__host__ __device__ inline int decode_bps(long long pairs, long long T, long long W) {
  if (T < 1) T = 1;
  if (pairs < 1) pairs = 1;
  long long best_b = 8;
  double best_eff = -1.0;
  for (long long k = 1; k <= 8; ++k) {
    long long s = k * W / pairs;                     // splits per row
    if (s < 1) s = 1;
    long long b = (T + s - 1) / s;
    if (b < 8) b = 8;
    b += b & 1;
    const long long items = pairs * ((T + b - 1) / b);
    const double eff = (double)items / (double)(((items + W - 1) / W) * W);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best_b = b;
    }
  }
  return (int)best_b;
}

// Split-K of a decode row with T block-table entries: the host picks a base split size
// `bps` (even) and a cap `smax` on splits per row; a sequence longer than the caller's
// max_entries bound gets larger splits instead of more, so the partial buffer sized from
// smax is never exceeded.
__host__ __device__ inline int row_bps(int T, int bps, int smax) {
  int need = (T + smax - 1) / smax;
  need += need & 1;
  return need > bps ? need : bps;
}
__host__ __device__ inline int row_splits(int T, int bps, int smax) {
  if (T <= 0) return 1;
  const int b = row_bps(T, bps, smax);
  return (T + b - 1) / b;
}

// Positional encoding applied inside the attention kernels.
//   kRope    position-free pool: keys and queries rotated by RoPE from logical positions
//   kStored  materialised baseline: keys already carry R(L); queries rotated by R(p)
//   kAlibi   position-free pool, no rotation: score + slope_h (L - p) (linear bias)
//   kRopePartial  as kRope, with rotate-half applied inside the first rotary_dim dims only
//   kDocRotated   keys stored with RoPE at a per-entry stored offset (e.g. their position
//                 inside their document): the kernels rotate by off_t - stored_t only
enum PosEnc : int { kRope = 0, kStored = 1, kAlibi = 2, kRopePartial = 3, kDocRotated = 4 };

// Partial rotary (dims k and k + r/2 paired for k < r/2, theta_k = base^(-2k/r), dims r..D-1
// unrotated) is computed as full rotate-half over a permuted dim order whose extra pairs have
// frequency zero: a common permutation of q's and k's dims leaves every score unchanged.
// The permutation moves whole 8-dim chunks. With hc = r/16 and Hc = D/16, the kernels' chunk
// kc holds natural chunk nat_chunk(kc): chunks below hc stay, the pass-through chunks
// r/8 .. r/8 + Hc - hc - 1 fill kernel chunks hc .. Hc - 1, the rotary partners hc .. 2hc - 1
// move to Hc .. Hc + hc - 1, and the rest stays. hc = Hc is the identity.
__host__ __device__ inline int nat_chunk(int kc, int hc, int Hc) {
  return kc < hc ? kc : kc < Hc ? kc + hc : kc < Hc + hc ? kc - Hc + hc : kc;
}

__device__ __forceinline__ uint32_t f16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// The smallest fp16 value >= x, as a float (x finite; values above 65504 give +inf).
__device__ __forceinline__ float f16_round_up(float x) {
  const _Float16 r = (_Float16)x;
  if ((float)r >= x) return (float)r;
  uint16_t b = __builtin_bit_cast(uint16_t, r);
  b = (b & 0x8000u) ? (uint16_t)(b - 1u) : (uint16_t)(b + 1u);   // one ulp towards +inf
  return (float)__builtin_bit_cast(_Float16, b);
}

// Plan modes.
enum PlanMode : int { kPlanMixed = 0, kPlanDecodeOnly = 1 };

}  // namespace lazyattn
