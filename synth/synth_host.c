/*
 * Host side of the synthetic-input generator (see synth_gen.h).
 * Plain C; every function fills `n` consecutive elements starting at flat
 * element `start` of the named tensor.
 */
#include <stddef.h>
#include <stdint.h>

#include "synth_gen.h"

uint64_t synth_stream_key(uint64_t seed, uint64_t cfg, uint64_t tensor,
                          uint64_t step) {
  return synth_key(seed, cfg, tensor, step);
}

/* bf16 tensor with N(0, sigma^2) entries (x, router weights). */
void synth_fill_bf16(uint64_t seed, uint64_t cfg, uint64_t tensor,
                     uint64_t step, uint64_t start, uint64_t n, double sigma,
                     uint16_t *out) {
  uint64_t key = synth_key(seed, cfg, tensor, step);
  for (uint64_t i = 0; i < n; ++i)
    out[i] = synth_f32_to_bf16(synth_normal_f32(key, start + i, sigma));
}

/* fp32 tensor with N(0, sigma^2) entries (router bias). */
void synth_fill_f32(uint64_t seed, uint64_t cfg, uint64_t tensor,
                    uint64_t step, uint64_t start, uint64_t n, double sigma,
                    float *out) {
  uint64_t key = synth_key(seed, cfg, tensor, step);
  for (uint64_t i = 0; i < n; ++i)
    out[i] = synth_normal_f32(key, start + i, sigma);
}

/* fp32 expert weights with the x10 outliers of stream tensor+100. */
void synth_fill_weight_f32(uint64_t seed, uint64_t cfg, uint64_t tensor,
                           uint64_t start, uint64_t n, double sigma,
                           float *out) {
  uint64_t key = synth_key(seed, cfg, tensor, 0);
  uint64_t mkey = synth_key(seed, cfg, tensor + SYNTH_MASK_OFFSET, 0);
  for (uint64_t i = 0; i < n; ++i)
    out[i] = synth_weight_f32(key, mkey, start + i, sigma);
}

/* Outlier flags (1 = scaled x10) of the same elements, for tests. */
void synth_fill_outlier_mask(uint64_t seed, uint64_t cfg, uint64_t tensor,
                             uint64_t start, uint64_t n, uint8_t *out) {
  uint64_t mkey = synth_key(seed, cfg, tensor + SYNTH_MASK_OFFSET, 0);
  for (uint64_t i = 0; i < n; ++i)
    out[i] = (uint8_t)synth_is_outlier(mkey, start + i);
}

/* Raw standard-normal deviates in double, for distribution tests. */
void synth_fill_std_normal(uint64_t key, uint64_t start, uint64_t n,
                           double *out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = synth_std_normal(key, start + i);
}
