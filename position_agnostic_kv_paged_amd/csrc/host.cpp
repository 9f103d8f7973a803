// Host helpers of the C ABI that touch no device: the packed block-word encoder, the Llama 3.1
// frequency table, status strings and the version. Plain C++ (built with the HIP sources,
// and on its own by the sanitizer tests). Declarations and contracts: include/lazyattn.h.
#include "lazyattn.h"

#include <cmath>
#include <cstdint>

namespace {

constexpr int kBlockTokens = 16;              // tokens per pool block (the calls require B = 16)
constexpr int kMaxHeadDim = 128;              // largest head dim of the attention calls
constexpr uint32_t kIdMask = (1u << LAZYATTN_ID_BITS) - 1u;
constexpr double kTwoPi = 6.283185307179586476925286766559;

}  // namespace

extern "C" {

int lazyattn_encode_meta(const int32_t* block_ids, const int64_t* offsets,
                         const int32_t* block_table, int32_t num_seqs, int32_t B,
                         uint32_t* words_out, int64_t* first_bad_entry) {
  if (first_bad_entry) *first_bad_entry = -1;
  if (!block_table || num_seqs < 0) return !block_table ? LAZYATTN_ERR_NULL : LAZYATTN_ERR_SHAPE;
  if (B != kBlockTokens) return LAZYATTN_ERR_SHAPE;
  if (block_table[0] != 0) return LAZYATTN_ERR_SHAPE;
  for (int s = 0; s < num_seqs; ++s)
    if (block_table[s + 1] < block_table[s]) return LAZYATTN_ERR_SHAPE;
  const int64_t n = block_table[num_seqs];
  if (n > 0 && (!block_ids || !offsets || !words_out)) return LAZYATTN_ERR_NULL;
  int rc = LAZYATTN_OK;
  const int64_t dmin = -(1ll << (LAZYATTN_DELTA_BITS - 1)), dmax = (1ll << (LAZYATTN_DELTA_BITS - 1)) - 1;
  for (int s = 0; s < num_seqs; ++s) {
    for (int64_t e = block_table[s]; e < block_table[s + 1]; ++e) {
      const int64_t t = e - block_table[s];
      const int64_t id = block_ids[e];
      const int64_t delta = offsets[e] - t * B;
      if (id < 0 || id > (int64_t)kIdMask || delta < dmin || delta > dmax) {
        words_out[e] = 0;
        if (rc == LAZYATTN_OK && first_bad_entry) *first_bad_entry = e;
        rc = LAZYATTN_ERR_RANGE;
        continue;
      }
      words_out[e] = (uint32_t)id | ((uint32_t)(delta & ((1 << LAZYATTN_DELTA_BITS) - 1)) << LAZYATTN_ID_BITS);
    }
  }
  return rc;
}

int lazyattn_llama31_inv_freq(int32_t D, double base, double factor, double low_freq_factor,
                              double high_freq_factor, double original_context,
                              double* inv_freq_out) {
  if (!inv_freq_out) return LAZYATTN_ERR_NULL;
  if (D <= 0 || D % 2 || D > kMaxHeadDim) return LAZYATTN_ERR_SHAPE;
  if (!(base > 1.0) || !(factor >= 1.0) || !(low_freq_factor > 0.0) ||
      !(high_freq_factor > low_freq_factor) || !(original_context > 0.0) ||
      !std::isfinite(base) || !std::isfinite(factor) || !std::isfinite(high_freq_factor) ||
      !std::isfinite(original_context))
    return LAZYATTN_ERR_ARG;
  // wavelength 2 pi / theta against the context the model was trained on: short waves keep
  // theta, long waves are slowed by `factor`, the band between is a linear blend in
  // original_context / wavelength
  const double short_wave = original_context / high_freq_factor;
  const double long_wave = original_context / low_freq_factor;
  for (int k = 0; k < D / 2; ++k) {
    const double theta = std::pow(base, -2.0 * k / D);
    const double wave = kTwoPi / theta;
    double t = theta;
    if (wave > long_wave) {
      t = theta / factor;
    } else if (wave >= short_wave) {
      const double w = (original_context / wave - low_freq_factor) /
                       (high_freq_factor - low_freq_factor);
      t = (1.0 - w) * theta / factor + w * theta;
    }
    inv_freq_out[k] = t;
  }
  return LAZYATTN_OK;
}

const char* lazyattn_status_str(int status) {
  switch (status) {
    case LAZYATTN_OK: return "ok";
    case LAZYATTN_ERR_NULL: return "null pointer argument";
    case LAZYATTN_ERR_ALIGN: return "misaligned pointer argument";
    case LAZYATTN_ERR_SHAPE: return "unsupported or inconsistent shape";
    case LAZYATTN_ERR_RANGE: return "block id or offset delta out of the packed word's range";
    case LAZYATTN_ERR_WORKSPACE: return "workspace too small";
    case LAZYATTN_ERR_LAUNCH: return "kernel launch failed";
    case LAZYATTN_ERR_ARG: return "invalid scalar argument";
    case LAZYATTN_ERR_NOSPACE: return "pool index: not enough free or evictable blocks";
    case LAZYATTN_ERR_STATE: return "pool index: unknown document, reference underflow or block not owned";
  }
  return "unknown status";
}

const char* lazyattn_version(void) { return "lazyattn-gfx950 0.1"; }

}  // extern "C"
