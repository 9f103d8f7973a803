// LazyAttention prefill work item for gfx950 (MFMA, online softmax, pipelined key tiles),
// run by mixed_kernel (mixed.hip).
//
// Technical summary of LazyAttention (arXiv 2606.04302), "Technical Implementation",
// prefilling phase: cached KV blocks are loaded from the position-free cache and, instead
// of rotating each key twice (back to position zero, then to its target), every key tile is
// rotated ONCE per query tile by the offset between the tile and the key's logical
// position. "Mathematical Equivalence": RoPE scores depend only on n - m, so
//   <R(p) q, R(L) k> = <R(p - p_ref) q, R(L - p_ref) k>
// for any reference position p_ref; the kernel takes p_ref = the tile's first query
// position, rotates the tile's queries by R(p - p_ref) once, and rotates each staged key by
// R(L - p_ref) once per (query tile, key tile) -- shared by all 32 * NW rows of the
// workgroup, which is what keeps it a small overhead.
//
// Key rotation cost: for key slot j of a block with offset off_b,
//   R(off_b + j - p_ref) = R(off_b - p_ref) R(j).
// R(j) is a per-thread constant (each thread always stages the same slot and frequencies);
// cos/sin of (off_b - p_ref) theta_k are computed once per (block, frequency) per key tile
// from an exact double-precision phase and shared through LDS; combining the two is four
// multiply-adds per (key, frequency).
//
// Workgroup tile: NW waves x 32 rows; rows are (query position, head-in-group) pairs so the
// G query heads of one KV head share every staged key/value tile (grouped-query packing).
// Per wave, S^T = K~ Q~^T (fp16 operands) and O^T += V^T P^T (bf16) on 32x32x16 MFMA: each
// lane owns one query row (MFMA column), so row max / row sum are in-lane plus one
// cross-half exchange. Values go straight from global memory into a swizzled LDS tile
// (global_load_lds) and are transposed on read (ds_read_b64_tr_b16). The next key tile's
// loads are in flight while the current one is multiplied; one barrier per key tile.
//
// Positional-encoding instances: kRope (above); kStored (keys already carry R(L): no key
// rotation); kAlibi (no rotation, linear bias); kRopePartial (kRope over the permuted dim
// order of nat_chunk); kDocRotated (keys stored with R(stored_b + j): each key tile is
// rotated by R(off_b - stored_b - p_ref) from the block phase table alone).
#pragma once
#include "lazyattn_common.h"
#include "lazyattn_kernels.h"
#include <limits.h>
#include <type_traits>

namespace lazyattn {

constexpr int kPrefillWaves = 8;

__device__ __forceinline__ void g2lds16p(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base,
                                   16, 0, 0);
}


typedef _Float16 h2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t h2_bits(h2 v) { return __builtin_bit_cast(uint32_t, v); }
// two bf16 values -> two fp16 values (one packed word)
__device__ __forceinline__ h2 bf2_to_h2(uint32_t x) {
  return as_h2(pack_f16(__uint_as_float(x << 16), __uint_as_float(x & 0xffff0000u)));
}

struct TileWords {
  int id[4], off[4], nval[4];
  int kmin, kmax;
  bool full;
};

// a[b] for a runtime b in 0..3 without dynamic register indexing
__device__ __forceinline__ int sel4(const int (&a)[4], int b) {
  return b == 0 ? a[0] : b == 1 ? a[1] : b == 2 ? a[2] : a[3];
}

// c ? a : b for pointers as an integer blend: a plain select of an expensive address may be
// turned into a branch, which would split the interleaved MFMA block it sits in
__device__ __forceinline__ const void* blend_ptr(bool c, const void* a, const void* b) {
  const uint64_t m = 0 - (uint64_t)c;
  return (const void*)(((uint64_t)a & m) | ((uint64_t)b & ~m));
}

// Words of key tiles kw .. kw+7 live in one VGPR ("window"): lane i < 32 holds the word of
// entry 4 kw + i. A step needs the words of its tile and the next three, so a window serves
// four steps: the loop loads the next window once per four key tiles, each lane decodes its
// own word (block id, logical offset, valid keys) on the VALU, and the scalars a step needs
// are read out of lanes 4d .. 4d+3 (tile kw + d) with readlane.
constexpr int kWinLanes = 32;
__device__ __forceinline__ uint32_t load_window(const PrefillParams& P, int e0, int T, int kt,
                                                int lane) {
  // every lane loads (no branch): lanes past the table read its last word, which the
  // decode marks empty; a sequence without entries reads the zeroed workspace chunk
  const int ent = min(4 * kt + lane, T - 1);
  return *(const uint32_t*)blend_ptr(T > 0, P.block_meta + e0 + max(ent, 0), P.zero);
}

// stored rotation offsets of the same entries (document-rotated pool)
__device__ __forceinline__ int load_stored(const PrefillParams& P, int e0, int T, int kt,
                                           int lane) {
  const int ent = min(4 * kt + lane, T - 1);
  return *(const int*)blend_ptr(T > 0, P.stored + e0 + max(ent, 0), P.zero);
}

struct WinDec {
  int id, off, nv;                                       // this lane's entry, decoded
  int sh;                                                // rotation still to apply: off - stored
};

__device__ __forceinline__ WinDec decode_window(const PrefillParams& P, uint32_t win, int st,
                                                int T, int kvlen, int kt, int lane) {
  const int ent = 4 * kt + lane;
  WinDec d;
  d.id = word_id(win);
  d.off = word_offset(win, ent);
  d.sh = d.off - st;
  d.nv = ((lane < kWinLanes) & (ent < T) & (d.id < P.num_blocks))   // out-of-pool id: not read
             ? min(max(kvlen - ent * kBlock, 0), kBlock) : 0;
  return d;
}

template <int d>
__device__ __forceinline__ TileWords tile_words(const WinDec& wd) {
  TileWords tw;
  tw.kmin = INT_MAX;
  tw.kmax = INT_MIN;
  tw.full = true;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int id = rl(wd.id, 4 * d + b), off = rl(wd.off, 4 * d + b), nv = rl(wd.nv, 4 * d + b);
    tw.id[b] = id;
    tw.off[b] = off;
    tw.nval[b] = nv;
    tw.kmin = nv > 0 ? min(tw.kmin, off) : tw.kmin;
    tw.kmax = nv > 0 ? max(tw.kmax, off + nv - 1) : tw.kmax;
    tw.full = tw.full & (nv == kBlock);
  }
  return tw;
}

// LDS of one prefill work item (a workgroup of kPrefillWaves waves): references to
// separately declared __shared__ arrays. Keeping them separate variables lets the compiler
// tell the direct-to-LDS value copies (into Vs) from the operand reads of Ks and Qs, so
// operand reads do not wait for the copies in flight.
template <int D>
struct PrefillSmemDims {
  static constexpr int NW = kPrefillWaves, NK = 64, HALF = D / 2, KS = D + 8;
  static constexpr int VBYTES = NK * D * 2;
};
template <int D>
struct PrefillSmem {
  using S = PrefillSmemDims<D>;
  uint16_t (&Ks)[2][S::NK * S::KS];
  uint8_t (&Vs)[2][S::VBYTES];
  // rotation tables as fp16 pairs, one 8-byte entry per two frequencies: {(cos, cos),
  // (sin, sin)}, laid out [block or slot][pair][thread] so that the staging threads of a
  // wave read consecutive 8-byte words
  u32x2 (&tbl)[2][4 * S::HALF / 2];          // (off_b - p_ref) theta_k
  u32x2 (&slot_cs)[16 * S::HALF / 2];        // j theta_k, j < 16
  uint16_t (&Qs)[S::NW][32 * S::KS];         // each wave's rotated queries (fp16)
  double (&fr_s)[S::HALF];
  int& pmax_s;
};

// Declares the arrays of a PrefillSmem in the calling kernel and binds `name` to them.
#define LAZYATTN_PREFILL_SMEM(D, name)                                                       \
  using name##_S = PrefillSmemDims<D>;                                                       \
  __shared__ __align__(16) uint16_t name##_Ks[2][name##_S::NK * name##_S::KS];             \
  __shared__ __align__(16) uint8_t name##_Vs[2][name##_S::VBYTES];                          \
  __shared__ __align__(16) u32x2 name##_tbl[2][4 * name##_S::HALF / 2];                     \
  __shared__ __align__(16) u32x2 name##_slot[16 * name##_S::HALF / 2];                      \
  __shared__ __align__(16) uint16_t name##_Qs[name##_S::NW][32 * name##_S::KS];            \
  __shared__ double name##_fr[name##_S::HALF];                                             \
  __shared__ int name##_pmax;                                                              \
  PrefillSmem<D> name{name##_Ks, name##_Vs, name##_tbl, name##_slot, name##_Qs, name##_fr, \
                      name##_pmax}

// One prefill work item: query tile qt of a sequence for KV (work) head kvh, over the key
// tiles of one KV split. `item` numbers the items of a KV head: each sequence owns
// tiles x splits consecutive items (plan_kernel's prefix sums), tile-major. An item that is
// its tile's only split writes the bf16 output rows; otherwise it writes a partial
// (o, m, l) per row, which pf_merge_slice folds into the output in a later launch.
template <int D, int G, int PE>
__device__ __forceinline__ void prefill_item(const PrefillParams& P, const PrefillSmem<D>& SM,
                                             const int kvh, const int item) {
  constexpr bool PART = PE == kRopePartial;   // dims in the permuted order of nat_chunk
  constexpr bool DOC = PE == kDocRotated;     // keys carry R(stored + j): rotate by off - stored
  constexpr bool ROTATE = PE == kRope || PART || DOC;   // keys rotated per tile
  constexpr bool ALIBI = PE == kAlibi;        // no rotation; linear bias on the scores
  constexpr int NW = kPrefillWaves;
  constexpr int NT = NW * 64;
  constexpr int ROWS = 32 * NW;
  constexpr int POS = ROWS / G;               // query positions per tile
  constexpr int NK = 64;                      // keys per key tile (4 blocks)
  constexpr int HALF = D / 2;
  constexpr int NCH = D / 16;                 // 16-dim k-steps of QK^T
  constexpr int KS = D + 8;                   // K~ LDS row stride (16-bit elements)
  constexpr int ROWB = D * 2;                 // V row bytes
  // value tile in LDS: rows of ROWB bytes; 16-byte chunk c of row R sits at chunk
  // c ^ 2 (R & 3), so the four rows one transposed read touches hit disjoint banks
  constexpr int VBYTES = NK * ROWB;
  constexpr int VINST = VBYTES / 1024;        // wave-wide global_load_lds per tile
  constexpr int RPI = 1024 / ROWB;            // rows per instruction (4 rows of one block)
  constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
  static_assert(VBYTES % 1024 == 0 && 16 % RPI == 0, "value tile = whole wave loads");
  constexpr int FPT = NK * HALF / NT;         // frequencies each thread rotates per key tile
  constexpr int CPT = HALF / FPT;             // threads per key
  static_assert(FPT == 4 || FPT == 8, "staging unit = 4 or 8 frequencies of one key");
  using KRaw = typename std::conditional<FPT == 8, u32x4, u32x2>::type;

  auto& Ks = SM.Ks;
  auto& Vs = SM.Vs;
  auto& tbl = SM.tbl;
  auto& slot_cs = SM.slot_cs;
  auto& Qs = SM.Qs;
  auto& fr_s = SM.fr_s;
  auto& pmax_s = SM.pmax_s;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);    // wave index (uniform)

  // The prologue is a chain of dependent memory round trips (sequence, its CSR entries,
  // then its queries, positions and words, then the first keys); independent loads are
  // issued together so that each link costs one trip.
  const SeqFound sf = wave_upper_seq(P.pf_prefix, P.num_seqs, item, lane);
  const int seq = sf.s;
  const int q0 = __builtin_amdgcn_readfirstlane(P.q_indptr[seq]);
  const int qlen = __builtin_amdgcn_readfirstlane(P.q_indptr[seq + 1] - q0);
  const int e0 = __builtin_amdgcn_readfirstlane(P.block_table[seq]);
  const int T = __builtin_amdgcn_readfirstlane(P.block_table[seq + 1] - e0);
  const int kvlen = __builtin_amdgcn_readfirstlane(P.kv_lens[seq]);
  // this item's query tile and key-tile range (KV split)
  const PfSplit spl = pf_split((T + 3) / 4, *P.pf_kc, P.pf_smax);
  const int local = item - sf.start;
  const int qt = __builtin_amdgcn_readfirstlane(local / spl.splits);
  const int sp = __builtin_amdgcn_readfirstlane(local - qt * spl.splits);
  const int kt_b = sp * spl.chunk;
  const int kt_e = min((T + 3) / 4, kt_b + spl.chunk);
  // (rows at or past total_q -- a q_indptr that runs past the q array -- are not touched)
  const int p_ref =
      ROTATE ? __builtin_amdgcn_readfirstlane(P.q_pos[min(q0 + qt * POS, P.total_q - 1)]) : 0;

  // ---- this lane's query row -------------------------------------------------------------
  const int col = lane & 31, hh = lane >> 5;
  const int rho = 32 * w + col;
  const int qi = qt * POS + rho / G;
  const int h = kvh * G + rho % G;
  const int kvp = kvh / P.kv_group;                          // pool head of this work head
  const bool row_ok = (qi < qlen) & (q0 + qi < P.total_q);
  const int p = row_ok ? P.q_pos[q0 + qi] : INT_MIN;       // invalid rows see no key
  // raw query row (rotated below) and the words of key tiles 0 .. 3, in flight together
  // with the frequency table
  u32x4 qraw[NCH];
  {
    const uint16_t* qrow = P.q + ((size_t)(row_ok ? q0 + qi : 0) * P.Hq + h) * D;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      qraw[c] = row_ok ? *(const u32x4*)(qrow + (PART ? 8 * nat_chunk(2 * c + hh, P.rot_chunks,
                                                                      D / 16)
                                                       : 16 * c + 8 * hh))
                       : u32x4{0, 0, 0, 0};
  }
  uint32_t win = load_window(P, e0, T, kt_b, lane);        // words of tiles kt_b .. kt_b+7
  const int st0 = DOC ? load_stored(P, e0, T, kt_b, lane) : 0;

  for (int i = tid; i < HALF; i += NT) fr_s[i] = P.freqs[i];
  if (tid == 0) pmax_s = INT_MIN;
  __syncthreads();

  // Q~ rows of this wave -> LDS (fp16, row-major): lane holds dims 16c + 8hh + e (e < 8) of
  // its row; the rotate-half partner of chunk c is chunk c + NCH/2 (dims + D/2), same lane.
  uint16_t* qs = Qs[w];
  {
    const u32x4 (&raw)[NCH] = qraw;
    const int n = row_ok ? p - p_ref : 0;
    const float sc = P.scale_log2;                  // softmax scale folded into Q~
#pragma unroll
    for (int c = 0; c < NCH / 2; ++c) {
      u32x4 lo, hi;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a0 = bf_lo(raw[c][i]) * sc, a1 = bf_hi(raw[c][i]) * sc;
        float b0 = bf_lo(raw[c + NCH / 2][i]) * sc, b1 = bf_hi(raw[c + NCH / 2][i]) * sc;
        if (ALIBI) {                                // queries are not rotated
          lo[i] = pack_f16(a0, a1);
          hi[i] = pack_f16(b0, b1);
          continue;
        }
        float c0, s0, c1, s1;
        rope_cos_sin(n, fr_s[16 * c + 8 * hh + 2 * i], c0, s0);
        rope_cos_sin(n, fr_s[16 * c + 8 * hh + 2 * i + 1], c1, s1);
        lo[i] = pack_f16(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
        hi[i] = pack_f16(a0 * s0 + b0 * c0, a1 * s1 + b1 * c1);
      }
      *(u32x4*)(qs + col * KS + 16 * c + 8 * hh) = lo;
      *(u32x4*)(qs + col * KS + 16 * (c + NCH / 2) + 8 * hh) = hi;
    }
  }

  // wave / workgroup extents of the query positions (tile skipping and masking)
  int pmax_w = p, pmin_w = row_ok ? p : INT_MAX;
  for (int o = 32; o >= 1; o >>= 1) {
    pmax_w = max(pmax_w, __shfl_xor(pmax_w, o));
    pmin_w = min(pmin_w, __shfl_xor(pmin_w, o));
  }
  if (lane == 0) atomicMax(&pmax_s, pmax_w);
  pmax_w = __builtin_amdgcn_readfirstlane(pmax_w);           // wave-uniform after the reduction
  pmin_w = __builtin_amdgcn_readfirstlane(pmin_w);

  // ---- this thread's key staging unit: key kn (slot kj of block kb), frequencies
  // FPT*cp .. FPT*cp+FPT-1 (a wave's 64 threads stage keys of one block: kb is uniform)
  const int kn = tid / CPT, cp = tid % CPT;
  const int kb = __builtin_amdgcn_readfirstlane((kn >> 4) & 3), kj = kn & 15;
  // where those dims sit in a pool row (and their rotate-half partners, k_dhi further on)
  const int k_lo = PART ? 8 * nat_chunk(FPT * cp / 8, P.rot_chunks, D / 16) + FPT * cp % 8
                        : FPT * cp;
  const int k_dhi = PART ? 8 * nat_chunk(FPT * cp / 8 + D / 16, P.rot_chunks, D / 16) +
                               FPT * cp % 8 - k_lo
                         : HALF;
  // fp16 position of the cosine of frequency f of row r (a block or a slot) in the tables;
  // its sine sits 2 further on
  auto tpos = [&](int r, int f) {
    return ((r * (FPT / 2) + (f % FPT) / 2) * CPT + f / FPT) * 4 + (f & 1);
  };
  for (int i = tid; !DOC && i < 16 * HALF; i += NT) {       // R(j) table, loop invariant
    float c, sn;
    rope_cos_sin(i / HALF, fr_s[i % HALF], c, sn);
    _Float16* t = (_Float16*)slot_cs + tpos(i / HALF, i % HALF);
    t[0] = (_Float16)c;
    t[2] = (_Float16)sn;
  }

  // The running max m rides on the matrix cores: an extra 16-wide k-step with
  // K~ = (256, 0, ...) and Q~ = (-m / 256, 0, ...) makes S^T = K~ Q~^T - m directly. m is
  // kept a multiple of 256 times an fp16 value, so the product is exact in the fp32
  // accumulator and m may reach 256 * 65504 (~1.7e7) in the log2 domain before it
  // overflows. With ALiBi the same k-step also carries the bias within a block:
  // K~ = (256, j, j, 0, ...) for slot j and Q~ = (-m / 256, c_hi, c_lo, 0, ...) with
  // c = slope_h log2(e) = c_hi + c_lo split into two fp16 values, so S^T gets + c j; the
  // rest of the bias, c (off_b - p) per block b, is added on the vector ALUs in fp32.
  const bool e0lane = hh == 0;
  const float cslope = ALIBI ? P.slopes[h] * 1.4426950408889634f : 0.f;
  const float c_hi = (float)(_Float16)cslope;
  const uint32_t slope_hi = ALIBI ? f16_bits(c_hi) << 16 : 0u;
  const uint32_t jbits = ALIBI ? f16_bits((float)(col & 15)) : 0u;
  const u32x4 ones_a = e0lane ? u32x4{0x5C00u | (jbits << 16), jbits, 0u, 0u}
                              : u32x4{0u, 0u, 0u, 0u};      // fp16 (256, j, j, 0, ...)
  float m = -INFINITY, l = 0.f;                              // l: this lane's half of the row sum
  u32x4 qm = {e0lane ? slope_hi : 0u,                        // (-m/256, c_hi, c_lo, 0...) fp16
              e0lane && ALIBI ? f16_bits(cslope - c_hi) : 0u, 0u, 0u};
  const int p_bias = row_ok ? p : 0;                         // rows past the tile see no key
  // ALiBi bias of score half t of the tile whose words are at window index d of wd
  auto add_bias = [&](f32x16& s, const WinDec& wd, int d, int t) __attribute__((always_inline)) {
    if (!ALIBI) return;
    const float b0 = cslope * (float)(rl(wd.off, 4 * d + 2 * t) - p_bias);
    const float b1 = cslope * (float)(rl(wd.off, 4 * d + 2 * t + 1) - p_bias);
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] += (r < 8) ? b0 : b1;
  };
  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};

  // table of a key tile: cos and sin((off_b - p_ref) theta_k) for 4 blocks x HALF
  // frequencies = 8 HALF values, one per thread (threads beyond repeat a value and store
  // the same bits): value v is entry v / 2, cosine if v is even (cos x = sin(x + 1/4 rev)).
  // Branch-free so that it can sit between MFMAs of one basic block.
  const int tab_v = tid % (8 * HALF);
  const int tab_b = __builtin_amdgcn_readfirstlane((tab_v >> 1) / HALF);   // wave-uniform
  const double tab_f = fr_s[(tab_v >> 1) % HALF];          // this thread's frequency
  const float tab_quarter = (tab_v & 1) ? 0.f : 0.25f;
  const int tab_pos = tpos(tab_b, (tab_v >> 1) % HALF) + 2 * (tab_v & 1);
  // (the per-lane block choice selects among readlane results, never indexes an array)
  auto make_table = [&](const WinDec& wd, int d, int buf) __attribute__((always_inline)) {
    if (!ROTATE) return;                                    // keys need no phase table
    const int o = rl(DOC ? wd.sh : wd.off, 4 * d + tab_b);
    ((_Float16*)tbl[buf])[tab_pos] = (_Float16)rope_sin_rev(o - p_ref, tab_f, tab_quarter);
  };
  // values of tile kt + d straight into LDS, wave-wide instruction i of this wave: rows
  // R0 .. R0 + RPI - 1 of one block (block id and valid count are wave-uniform); lane l
  // fetches the chunk that belongs at its LDS slot (swizzle above); rows past the block's
  // valid keys read the zeroed chunk
  constexpr int VPW = VINST / NW;                           // value loads every wave issues
  static_assert(VPW >= 1 && VPW <= 3 && VINST % NW == 0,
                "value loads are placed in the first score k-steps");
  const int v_r = lane / CPR;                               // row within an instruction
  const int v_lc = (lane % CPR) ^ (2 * (v_r & 3));          // logical chunk this lane fetches
  auto issue_v = [&](const WinDec& wd, int d, int buf, int i) __attribute__((always_inline)) {
    const int R0 = (w * VPW + i) * RPI;                     // uniform
    const int b = R0 >> 4;
    const int nv = rl(wd.nv, 4 * d + b), id = rl(wd.id, 4 * d + b);
    const int j = (R0 & 15) + v_r;
    const void* src = blend_ptr(j < nv,
                                P.v_pool + (((size_t)id * P.Hkv_pool + kvp) * kBlock + j) * D +
                                    8 * v_lc,
                                P.zero);
    g2lds16p(src, Vs[buf] + R0 * ROWB);
  };

  KRaw klo{}, khi{};
  // raw keys of a tile into (klo, khi); empty slots read as zero
  // (key staging reads block kb of tile kt + d: lane 4 d + kb of the decoded window)
  auto load_k_to = [&](const WinDec& wd, int d, KRaw& lo, KRaw& hi) {
    const int nv = rl(wd.nv, 4 * d + kb), id = rl(wd.id, 4 * d + kb);
    // branch-free: empty slots load from the zeroed workspace chunk (0 < k_dhi <= D/2)
    const uint16_t* src = (const uint16_t*)blend_ptr(
        kj < nv, P.k_pool + (((size_t)id * P.Hkv_pool + kvp) * kBlock + kj) * D + k_lo, P.zero);
    lo = *(const KRaw*)src;
    hi = *(const KRaw*)(src + k_dhi);
  };
  auto load_k = [&](const WinDec& wd, int d) { load_k_to(wd, d, klo, khi); };
  // rotation of frequencies 2 i2, 2 i2 + 1 of the staged key by R(off_b - p_ref) R(kj),
  // in packed fp16 from the (cos, sin) pairs of the tables (the result is an fp16 operand)
  auto rot_pair = [&](const u32x2 cs, const u32x2 js, uint32_t xlo, uint32_t xhi) -> u32x2 {
    h2 c = as_h2(cs[0]), sn = as_h2(cs[1]);
    if (!DOC) {
      const h2 cj = as_h2(js[0]), sj = as_h2(js[1]);
      const h2 cc = c * cj - sn * sj;
      sn = sn * cj + c * sj;
      c = cc;
    }
    const h2 a = bf2_to_h2(xlo), b = bf2_to_h2(xhi);
    return u32x2{h2_bits(a * c - b * sn), h2_bits(a * sn + b * c)};
  };

  // Software pipeline over key tiles. Iteration kt holds S(kt) on entry; it
  //   A) exponentiates S(kt) into P(kt) while the matrix cores compute S(kt+1);
  //   B) runs O += V(kt)^T P(kt)^T while the vector ALUs rotate keys of tile kt+2;
  // keys are staged two tiles ahead, values one tile ahead (both double-buffered), the
  // (block, frequency) phase tables three tiles ahead. Work on tiles past the end reads
  // empty blocks (zeros) and is discarded. Inside A and B the order of matrix, vector,
  // memory and LDS instructions is fixed by scheduling fences: each MFMA is followed by the
  // vector work that hides under it, LDS operands are fetched one MFMA group ahead, and the
  // loads for later tiles are spread over A's k-steps so that the vector memory path
  // overlaps the matrix cores instead of stalling every wave right after the barrier.
  if (kt_e > kt_b) {
    const WinDec wd = decode_window(P, win, st0, T, kvlen, kt_b, lane);
    KRaw kraw[2][2];                                         // raw keys of tiles 0 and 1
    load_k_to(wd, 0, kraw[0][0], kraw[0][1]);
    load_k_to(wd, 1, kraw[1][0], kraw[1][1]);
    make_table(wd, 0, 0);
    make_table(wd, 1, 1);
#pragma unroll
    for (int i = 0; i < VPW; ++i) issue_v(wd, 0, 0, i);
    __syncthreads();                                         // tables 0, 1 visible
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {                         // keys of tiles 0 and 1
      const KRaw& klo = kraw[tt][0];
      const KRaw& khi = kraw[tt][1];
      KRaw ol, oh;
      if (ROTATE) {
        const u32x2* t4 = &tbl[tt][kb * (FPT / 2) * CPT + cp];
        const u32x2* j4 = &slot_cs[kj * (FPT / 2) * CPT + cp];
#pragma unroll
        for (int i2 = 0; i2 < FPT / 2; ++i2) {
          const u32x2 r = rot_pair(t4[i2 * CPT], DOC ? u32x2{} : j4[i2 * CPT], klo[i2],
                                   khi[i2]);
          ol[i2] = r[0];
          oh[i2] = r[1];
        }
      } else {
#pragma unroll
        for (int i2 = 0; i2 < FPT / 2; ++i2) {
          ol[i2] = pack_f16(bf_lo(klo[i2]), bf_hi(klo[i2]));
          oh[i2] = pack_f16(bf_lo(khi[i2]), bf_hi(khi[i2]));
        }
      }
      *(KRaw*)(Ks[tt] + kn * KS + FPT * cp) = ol;
      *(KRaw*)(Ks[tt] + kn * KS + HALF + FPT * cp) = oh;
    }
    __syncthreads();                                         // tables 0, 1 consumed
    make_table(wd, 2, 0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);                        // vmcnt(0)
  __syncthreads();
  const int pmax_g = __builtin_amdgcn_readfirstlane(pmax_s);
  // Does tile d of a decoded window (lanes 4d .. 4d+3) need the causal / ragged mask for
  // this wave's rows? It does not when its four blocks are full, none reaches past the
  // wave's first row, and at least one starts at or before the last row of the wave and of
  // the workgroup. Two ballots per window give every tile's answer (no per-block scalar
  // reads): `bad` marks blocks not full or reaching past the first row, `late` blocks that
  // start after the last row.
  const int pm_vis = min(pmax_w, pmax_g);
  struct WinMask { uint64_t bad, late; };
  auto window_mask = [&](const WinDec& wd) __attribute__((always_inline)) {
    return WinMask{__ballot((wd.nv != kBlock) | (wd.off + (kBlock - 1) > pmin_w)),
                   __ballot(wd.off > pm_vis)};
  };
  auto needs_mask = [&](const WinMask& wm, int d) __attribute__((always_inline)) {
    return (((wm.bad >> (4 * d)) & 0xFull) != 0) | (((wm.late >> (4 * d)) & 0xFull) == 0xFull);
  };
  f32x16 S0[2], S1[2];

  // S^T = K~ Q~^T - m for the key tile in Ks[buf] (prologue only; the loop interleaves it)
  auto qk = [&](int buf, f32x16 (&sc)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) sc[t] = mfma32h(as_f16x8(ones_a), as_f16x8(qm), f32x16{});
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const u32x4 b = *(const u32x4*)(qs + col * KS + 16 * c + 8 * hh);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 a = *(const u32x4*)(Ks[buf] + (32 * t + col) * KS + 16 * c + 8 * hh);
        sc[t] = mfma32h(as_f16x8(a), as_f16x8(b), sc[t]);
      }
    }
  };
  if (kt_e > kt_b) qk(0, S0);
  WinDec wdc = decode_window(P, win, st0, T, kvlen, kt_b, lane);
  WinMask wmc = window_mask(wdc);
  add_bias(S0[0], wdc, 0, 0);
  add_bias(S0[1], wdc, 0, 1);
  bool maskc = needs_mask(wmc, 0);
  uint32_t win_nx = 0;                                       // the next window, in flight
  int st_nx = 0;
  float mxc = xor32_max(max32(S0[0], S0[1]));

  const int gi = lane >> 4, i16 = lane & 15;
  // transposed value reads: this lane's row is 4 hh + i16 / 4 (+ 32 t + 16 kk, + 8), so its
  // swizzle 2 (R & 3) = 2 (i16 / 4) is fixed; the chunk of dim step dt is
  // (4 dt + 2 (gi & 1) + (i16 & 3) / 2) ^ 2 (i16 / 4)
  const int v_sw = 2 * (i16 >> 2);
  const uint8_t* vlane = (const uint8_t*)Vs + (4 * hh + (i16 >> 2)) * ROWB + 8 * (i16 & 1);
  auto vchunk = [&](int dt) { return 16 * ((4 * dt + 2 * (gi & 1) + ((i16 & 3) >> 1)) ^ v_sw); };
  const uint16_t* klane = Ks[0] + col * KS + 8 * hh;        // + buf * NK * KS
  const uint16_t* qlane = qs + col * KS + 8 * hh;

  // one pipeline iteration: S(kt) in Sc on entry, S(kt+1) left in Sn. PH = (kt - kt_b) % 4 is
  // the step's place in its window: wdc holds the decoded words of tiles kt - PH .. kt - PH + 7
  // (tile kt + d at window index PH + d); the next window is loaded in step PH = 0 and decoded
  // in step PH = 3. mxc (row max of S(kt) before masking) was computed under the MFMAs of
  // the previous iteration.
  auto step = [&](auto ph, const int kt, f32x16 (&Sc)[2], f32x16 (&Sn)[2]) {
    constexpr int PH = decltype(ph)::value;
    const int cur = PH & 1, nxt = cur ^ 1;                   // buffers of tiles kt, kt+1
    const WinDec wd = wdc;
    WinDec wdn = wdc;
    WinMask wmn = wmc;
    bool maskn = false;
    float h0 = 0.f, h1 = 0.f;
    float mx = mxc;
    // ---- rare paths: causal / ragged mask of S(kt) ------------------------------------
    if (maskc) {
      const TileWords tw = tile_words<PH>(wd);
      const bool visible = tw.kmin <= pmax_w && tw.kmin <= pmax_g;
      {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int b = 2 * t + (r >> 3);
            const int j = ((r >> 2) & 1) * 8 + 4 * hh + (r & 3);
            const bool ok = visible & (j < tw.nval[b]) & (tw.off[b] + j <= p);
            Sc[t][r] = ok ? Sc[t][r] : -INFINITY;
          }
        mx = xor32_max(max32(Sc[0], Sc[1]));
      }
    }
    // the running max moves only when a row's max exceeds it by 2^8 (or on the row's first
    // visible key), so P = exp2(S) stays below 256; m is kept as the exact value the
    // matrix cores subtract (256 times an fp16 number, rounded up so that m is never below
    // the row max it is set from), so the offset cancels in O / l
    const bool first = (m == -INFINITY) & (mx != -INFINITY);
    if (__any(first | (mx > 8.f))) {
      const float m_old = m == -INFINITY ? 0.f : m;
      float m_new = m;
      if (first | (mx > 0.f)) m_new = 256.f * f16_round_up((m_old + mx) * (1.f / 256.f));
      const float delta = m_new == -INFINITY ? 0.f : m_new - m_old;
      const float alpha = first ? 1.f : __builtin_amdgcn_exp2f(-delta);
      m = m_new;
      qm[0] = e0lane ? f16_bits(m == -INFINITY ? 0.f : m * (-1.f / 256.f)) | slope_hi : 0u;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) Sc[t][r] -= delta;
    }
    __builtin_amdgcn_sched_barrier(0);

    // Waves w and w + NW/2 share a SIMD and run the same phase; the issue arbiter favours
    // the older one, which then idles at the barrier while the other finishes alone.
    // Alternating wave priorities between the two blocks lets both finish together.
    if (w < NW / 2) __builtin_amdgcn_s_setprio(2); else __builtin_amdgcn_s_setprio(1);
    // ---- A: S(kt+1) on the matrix cores, P(kt) = exp2(S(kt)) on the VALU ---------------
    // score pair q (0..15) of this lane: t = q / 8, kk = (q / 4) % 2, i = q % 4
    u32x4 bp[2][2];
    float rs0 = 0.f, rs1 = 0.f;
    constexpr int SLOTS = 2 * NCH + 2;                        // MFMAs of S(kt+1)
    constexpr int PPS = (16 + SLOTS - 1) / SLOTS;             // score pairs per MFMA slot
    auto exp_slot = [&](const int slot) {
#pragma unroll
      for (int u = 0; u < PPS; ++u) {
        const int q = slot * PPS + u;
        if (q < 16) {
          const int t = q >> 3, kk = (q >> 2) & 1, i = q & 3;
          const float x0 = __builtin_amdgcn_exp2f(Sc[t][8 * kk + 2 * i]);
          const float x1 = __builtin_amdgcn_exp2f(Sc[t][8 * kk + 2 * i + 1]);
          bp[t][kk][i] = pack_bf16(x0, x1);
          if (i & 1) rs1 = sum2_bf16(bp[t][kk][i], rs1);
          else rs0 = sum2_bf16(bp[t][kk][i], rs0);
          asm volatile("" ::"v"(bp[t][kk][i]));                // keep it in this MFMA slot
        }
      }
    };
    {
      const uint16_t* ka = klane + nxt * (NK * KS);
      u32x4 a0 = *(const u32x4*)ka, a1 = *(const u32x4*)(ka + 32 * KS);
      u32x4 b = *(const u32x4*)qlane;
      Sn[0] = mfma32h(as_f16x8(ones_a), as_f16x8(qm), f32x16{});
      exp_slot(0);
      load_k(wd, PH + 2);                                   // raw keys of tile kt+2
      Sn[1] = mfma32h(as_f16x8(ones_a), as_f16x8(qm), f32x16{});
      exp_slot(1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        u32x4 na0 = a0, na1 = a1, nb = b;
        if (c + 1 < NCH) {
          na0 = *(const u32x4*)(ka + 16 * (c + 1));
          na1 = *(const u32x4*)(ka + 32 * KS + 16 * (c + 1));
          nb = *(const u32x4*)(qlane + 16 * (c + 1));
        }
        Sn[0] = mfma32h(as_f16x8(a0), as_f16x8(b), Sn[0]);
        exp_slot(2 + 2 * c);
        // staging for later tiles, spread over the k-steps so that the vector memory
        // path works while the matrix cores do: values of tile kt+1 (k-steps 0..2), the
        // next word window (k-step 2), the phase table of tile kt+3 (k-step 3)
        if (c < VPW) issue_v(wd, PH + 1, nxt, c);
        if (PH == 0 && c == 2) {                            // the window of tiles kt+4 ..
          win_nx = load_window(P, e0, T, kt + 4, lane);
          if (DOC) st_nx = load_stored(P, e0, T, kt + 4, lane);
        }
        if (c == 3) make_table(wd, PH + 3, nxt);
        Sn[1] = mfma32h(as_f16x8(a1), as_f16x8(b), Sn[1]);
        exp_slot(3 + 2 * c);
        __builtin_amdgcn_sched_barrier(0);
        a0 = na0;
        a1 = na1;
        b = nb;
      }
    }
    l += rs0 + rs1;

    if (w < NW / 2) __builtin_amdgcn_s_setprio(1); else __builtin_amdgcn_s_setprio(2);
    // ---- B: O += V(kt)^T P(kt)^T on the matrix cores, keys of tile kt+2 on the VALU -----
    // MFMA group g = (t, kk) = (g / 2, g % 2) takes D/32 MFMAs; rotation chunk g (two
    // frequencies of the staged key) is cut into four pieces spread over those MFMAs.
    {
      const uint8_t* vb = vlane + cur * VBYTES;
      auto vread = [&](int g, u32x4 (&va)[D / 32]) {
        const int t = g >> 1, kk = g & 1;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const uint8_t* a1 = vb + (32 * t + 16 * kk) * ROWB + vchunk(dt);
          const u32x2 r1 = lds_read_tr((const uint16_t*)a1);
          const u32x2 r2 = lds_read_tr((const uint16_t*)(a1 + 8 * ROWB));
          va[dt] = u32x4{r1[0], r1[1], r2[0], r2[1]};
        }
      };
      const u32x2* t4 = &tbl[cur][kb * (FPT / 2) * CPT + cp];
      const u32x2* j4 = &slot_cs[kj * (FPT / 2) * CPT + cp];
      KRaw ol, oh;
      h2 rc, rsn, xa, xb;
      // chunk g (two frequencies) in packed fp16, four pieces: 0 the angle R(off_b - p_ref)
      // R(kj), 1 and 2 the key halves to fp16, 3 the rotation
      auto piece = [&](const int g, const int pc, const u32x2 cs, const u32x2 js) {
        if (pc == 0) {
          rc = as_h2(cs[0]);
          rsn = as_h2(cs[1]);
          if (!DOC) {
            const h2 cj = as_h2(js[0]), sj = as_h2(js[1]);
            const h2 cc = rc * cj - rsn * sj;
            rsn = rsn * cj + rc * sj;
            rc = cc;
          }
          asm volatile("" ::"v"(rc), "v"(rsn));
        } else if (pc == 1) {
          xa = bf2_to_h2(klo[g]);
          asm volatile("" ::"v"(xa));
        } else if (pc == 2) {
          xb = bf2_to_h2(khi[g]);
          asm volatile("" ::"v"(xb));
        } else {
          ol[g] = h2_bits(xa * rc - xb * rsn);
          oh[g] = h2_bits(xa * rsn + xb * rc);
          asm volatile("" ::"v"(ol[g]), "v"(oh[g]));
        }
      };
      auto plain = [&](const int g) {
        ol[g] = pack_f16(bf_lo(klo[g]), bf_hi(klo[g]));
        oh[g] = pack_f16(bf_lo(khi[g]), bf_hi(khi[g]));
        asm volatile("" ::"v"(ol[g]), "v"(oh[g]));
      };
      u32x4 va[D / 32];
      vread(0, va);
      u32x2 cs = ROTATE ? t4[0] : u32x2{}, js = ROTATE && !DOC ? j4[0] : u32x2{};
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x4 vn[D / 32];
        u32x2 csn = cs, jsn = js;
        if (g + 1 < 4) {
          vread(g + 1, vn);
          if (ROTATE && g + 1 < FPT / 2) {
            csn = t4[(g + 1) * CPT];
            if (!DOC) jsn = j4[(g + 1) * CPT];
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        // next iteration's inputs, under these MFMAs: the mask decision of tile kt+1 and,
        // in the window's last step, the next window decoded (group 1); the row max of
        // S(kt+1) (groups 2, 3)
        if (g == 1) {
          maskn = needs_mask(wmc, PH + 1);
          if (PH == 3) {
            wdn = decode_window(P, win_nx, st_nx, T, kvlen, kt + 1, lane);
            asm volatile("" ::"v"(wdn.id), "v"(wdn.off), "v"(wdn.nv));
            wmn = window_mask(wdn);
          }
        }
        if (g == 2) {
          add_bias(Sn[0], wd, PH + 1, 0);
          h0 = max16(Sn[0]);
          asm volatile("" ::"v"(h0));
        }
        if (g == 3) {
          add_bias(Sn[1], wd, PH + 1, 1);
          h1 = max16(Sn[1]);
          asm volatile("" ::"v"(h1));
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          o[dt] = mfma32(as_bf16x8(va[dt]), as_bf16x8(bp[g >> 1][g & 1]), o[dt]);
          if (g < FPT / 2) {
            if (ROTATE) {
#pragma unroll
              for (int pc = dt * 4 / (D / 32); pc < (dt + 1) * 4 / (D / 32); ++pc)
                piece(g, pc, cs, js);
            } else if (dt == 0) {
              plain(g);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (g + 1 < 4) {
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) va[dt] = vn[dt];
          cs = csn;
          js = jsn;
        }
      }
      *(KRaw*)(Ks[cur] + kn * KS + FPT * cp) = ol;           // keys of tile kt+2
      *(KRaw*)(Ks[cur] + kn * KS + HALF + FPT * cp) = oh;
    }
    __builtin_amdgcn_s_setprio(0);
    wdc = wdn;
    wmc = wmn;
    maskc = maskn;
    mxc = xor32_max(max3f(h0, h1, h1));
    __builtin_amdgcn_s_waitcnt(0x0F70);                      // vmcnt(0): values of tile kt+1
    __syncthreads();
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  for (int kt = kt_b; kt < kt_e; kt += 4) {                  // one window; S0 <-> S1
    step(P0{}, kt, S0, S1);
    if (kt + 1 < kt_e) step(P1{}, kt + 1, S1, S0);
    if (kt + 2 < kt_e) step(P2{}, kt + 2, S0, S1);
    if (kt + 3 < kt_e) step(P3{}, kt + 3, S1, S0);
  }

  // ---- epilogue: O / l -> bf16 ----------------------------------------------------------
  const float lt = xor32_add(l);
  if (spl.splits == 1) {
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
    return;
  }
  // KV split: partial (o, m, l) of each row of the tile, [slot][row rho][D + 4] floats
  constexpr int RS = D + 4;
  const size_t cap = (size_t)P.pf_item_cap;
  float* part = P.pf_partials + ((size_t)kvh * cap + item) * (size_t)(ROWS * RS);
  {
    float* pr = part + (size_t)rho * RS;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *(f32x4*)(pr + 32 * dt + 8 * r4 + 4 * hh) =
            f32x4{o[dt][4 * r4], o[dt][4 * r4 + 1], o[dt][4 * r4 + 2], o[dt][4 * r4 + 3]};
    if (hh == 0) {
      pr[D] = lt > 0.f ? m : -INFINITY;
      pr[D + 1] = lt;
    }
  }
}

// Merge of a split query tile (after every split item has written its partial): the rows
// of the tile are shared among its split items' slots, so item sp of a tile with s splits
// merges rows [sp 256 / s, (sp + 1) 256 / s). One thread per (row, 4 dims) in turn:
// M = max m, L = sum l 2^(m - M), O = sum o 2^(m - M), out = O / L (0 where L = 0). A split
// with no visible key has m = -inf, l = 0, o = 0, weight 0. Every wave of the workgroup
// calls it with the same (kvh, item).
template <int D, int G>
__device__ __forceinline__ void pf_merge_slice(const PrefillParams& P, const int kvh,
                                               const int item, const int nthreads) {
  constexpr int ROWS = 32 * kPrefillWaves;
  constexpr int POS = ROWS / G;
  constexpr int RS = D + 4;
  constexpr int CH = D / 4;                                  // 4-dim chunks per row
  constexpr size_t SPLIT = (size_t)ROWS * RS;                // floats per split partial
  const int lane = threadIdx.x & 63;
  const SeqFound sf = wave_upper_seq(P.pf_prefix, P.num_seqs, item, lane);
  const int seq = sf.s;
  const int q0 = P.q_indptr[seq], qlen = P.q_indptr[seq + 1] - q0;
  const int T = P.block_table[seq + 1] - P.block_table[seq];
  const PfSplit spl = pf_split((T + 3) / 4, *P.pf_kc, P.pf_smax);
  const int ns = spl.splits;
  if (ns == 1) return;                                       // written by the item itself
  const int local = item - sf.start;
  const int qt = local / ns, sp = local - qt * ns;
  const int first = item - sp;
  const int r0 = sp * ROWS / ns, r1 = (sp + 1) * ROWS / ns;
  const float* tile = P.pf_partials + ((size_t)kvh * P.pf_item_cap + first) * SPLIT;
  for (int x = threadIdx.x; x < (r1 - r0) * CH; x += nthreads) {
    const int row = r0 + x / CH, c = x % CH;
    const int rq = qt * POS + row / G;                       // query row in the sequence
    const int rh = kvh * G + row % G;                        // query head
    if (!((rq < qlen) & (q0 + rq < P.total_q))) continue;
    const float* base = tile + (size_t)row * RS;
    float M = -INFINITY;
    for (int s0 = 0; s0 < ns; s0 += 8) {                     // eight m values per round
      float mv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) mv[u] = s0 + u < ns ? base[(s0 + u) * SPLIT + D] : -INFINITY;
#pragma unroll
      for (int u = 0; u < 8; ++u) M = fmaxf(M, mv[u]);
    }
    const float Mu = M == -INFINITY ? 0.f : M;               // all -inf: weights 0, row 0
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < ns; s0 += 4) {                     // four splits per round
      f32x4 ov[4];
      float ms[4], ls[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool ok = s0 + u < ns;
        const float* ps = base + (size_t)(ok ? s0 + u : s0) * SPLIT;
        ov[u] = *(const f32x4*)(ps + 4 * c);
        ms[u] = ok ? ps[D] : -INFINITY;
        ls[u] = ps[D + 1];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wgt = __builtin_amdgcn_exp2f(ms[u] - Mu);
        L += ls[u] * wgt;
        acc += ov[u] * wgt;
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    u32x2 v;
    v[0] = pack_bf16(acc[0] * inv, acc[1] * inv);
    v[1] = pack_bf16(acc[2] * inv, acc[3] * inv);
    *(u32x2*)(P.out + ((size_t)(q0 + rq) * P.Hq + rh) * D + 4 * c) = v;
  }
}

}  // namespace lazyattn
