/*
 * synth_gen.h -- seeded, counter-based generator of the synthetic inputs of
 * the routed-expert MoE layer (activations, router weights, router bias,
 * expert weights with sparse x10 outliers).
 *
 * This module holds input generation only, none of the layer's arithmetic.
 * The same source is compiled for the host (gcc, C) and for the GPU (hipcc),
 * so both sides of a test draw bit-identical tensors:
 *   - every draw is SplitMix64 (Steele, Lea, Flood, "Fast splittable
 *     pseudorandom number generators", OOPSLA 2014) evaluated at a counter,
 *     so element n of a tensor can be produced on its own, in any order;
 *   - a standard normal deviate is the Irwin-Hall sum of twelve 32-bit
 *     uniforms minus 6 (mean 0, variance 1, support [-6, 6]).  The sum is an
 *     integer and its conversion to double is exact, so the deviate is
 *     identical on any IEEE-754 machine; no transcendental function (whose
 *     last bit differs between libm and the GPU math library) is involved;
 *   - each later step is one correctly rounded IEEE operation (a double
 *     multiply, double->float, float->bf16 round-to-nearest-even).
 *
 * Tensor element n is always the row-major flat index of the tensor's
 * logical shape, so a tensor may be generated whole, by rows or by samples.
 */
#ifndef SYNTH_GEN_H
#define SYNTH_GEN_H

#include <stdint.h>

#if defined(__HIPCC__)
#define SYNTH_FN __host__ __device__ static inline
#else
#define SYNTH_FN static inline
#endif

#if defined(__clang__)
#pragma clang fp contract(off)
#endif

/* tensor ids of the stream key */
#define SYNTH_T_X 1          /* activations x [T][d], bf16, N(0,1)          */
#define SYNTH_T_WR 2         /* router weights [E][d], bf16, N(0,1/d)       */
#define SYNTH_T_BIAS 3       /* router logit bias [E], fp32, N(0,sb^2)      */
#define SYNTH_T_W_GATE_UP 4  /* gate|up weights [E][2f][d], fp32             */
#define SYNTH_T_W_DOWN 6     /* down weights [E][d][f], fp32                 */
#define SYNTH_MASK_OFFSET 100 /* outlier-mask stream of tensor t is t+100    */

#define SYNTH_GOLDEN 0x9E3779B97F4A7C15ULL
/* floor(0.001 * 2^64): a draw below it marks an outlier (probability 1e-3) */
#define SYNTH_OUTLIER_THRESHOLD 18446744073709551ULL

SYNTH_FN uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Stream key of one tensor: (master seed, config id, tensor id, step). */
SYNTH_FN uint64_t synth_key(uint64_t seed, uint64_t cfg, uint64_t tensor,
                            uint64_t step) {
  uint64_t k = synth_mix64(seed + SYNTH_GOLDEN);
  k = synth_mix64(k + SYNTH_GOLDEN * (cfg + 1));
  k = synth_mix64(k + SYNTH_GOLDEN * (tensor + 1));
  k = synth_mix64(k + SYNTH_GOLDEN * (step + 1));
  return k;
}

/* Draw i of the stream with key `key`: SplitMix64 output i for state key. */
SYNTH_FN uint64_t synth_u64(uint64_t key, uint64_t i) {
  return synth_mix64(key + SYNTH_GOLDEN * (i + 1));
}

/* Standard normal deviate for element n (Irwin-Hall, 12 uniforms). */
SYNTH_FN double synth_std_normal(uint64_t key, uint64_t n) {
  uint64_t s = 0;
  for (uint64_t j = 0; j < 6; ++j) {
    uint64_t r = synth_u64(key, 6 * n + j);
    s += (r & 0xFFFFFFFFULL) + (r >> 32);
  }
  /* s < 12 * 2^32 < 2^36: exact in double, and so are the scale and shift */
  return (double)s * (1.0 / 4294967296.0) - 6.0;
}

SYNTH_FN int synth_is_outlier(uint64_t mask_key, uint64_t n) {
  return synth_u64(mask_key, n) < SYNTH_OUTLIER_THRESHOLD;
}

SYNTH_FN float synth_normal_f32(uint64_t key, uint64_t n, double sigma) {
  return (float)(synth_std_normal(key, n) * sigma);
}

/* Expert weight: N(0, sigma^2), and x10 with probability 1e-3. */
SYNTH_FN float synth_weight_f32(uint64_t key, uint64_t mask_key, uint64_t n,
                                double sigma) {
  double z = synth_std_normal(key, n);
  double sc = synth_is_outlier(mask_key, n) ? sigma * 10.0 : sigma;
  return (float)(z * sc);
}

/* float -> bfloat16 bits, round to nearest even (inputs here are finite). */
SYNTH_FN uint16_t synth_f32_to_bf16(float f) {
  union {
    float f;
    uint32_t u;
  } v;
  v.f = f;
  uint32_t u = v.u;
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

#endif /* SYNTH_GEN_H */
