/*
 * oracle.h -- plain, slow CPU definition of the routed-expert W4A16 MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU library; its inputs come from the
 * seeded generator, never from the GPU path.
 *
 * Sources (the five web pages on quantized MoE experts):
 *  - "Every Expert Counts: ExactMoE for Memory-Efficient W4A16 Inference",
 *    Abstract: symmetric group-128 4-bit weights on routed experts only, BF16
 *    router, unchanged top-k routing, every selected expert executed.
 *  - "PagedMoE: Cross-Precision Expert Caching for Token-Level Dynamic
 *    Precision in SSD-Resident MoE Inference", abstract: each expert stored
 *    once in a bitplane layout whose lower precisions are prefixes of higher
 *    ones, executed directly at 1-8-bit prefixes chosen per token.
 *  - "MatMoE: Matryoshka Mixture-of-Experts with Dynamic Mixed-Precision
 *    Quantization for Efficient Inference", abstract: floor-and-compensation
 *    dequantization of a nested representation; bit-width from routing score.
 * The exact layer definition (softmax, tie-break, quantizer rounding, SwiGLU,
 * combine) fills in what the pages leave open; each reading is stated at the
 * function that takes it.
 *
 * Precision: integer decisions are taken exactly as defined (router logits in
 * fp32 in a fixed order, quantizer quotients in fp64 = exact rounding);
 * everything else is accumulated in fp64.
 *
 * All functions return 0 on success, -1 on an invalid argument.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Router logits [T][E] (fp32), fixed lane-group summation order. */
int oracle_router_logits(const uint16_t *x_bf16, const uint16_t *wr_bf16,
                         const float *bias, int T, int d, int E, float *logits);
/* Top-k selection on logits and renormalised softmax weights (fp64). */
int oracle_topk(const float *logits, int T, int E, int k, int32_t *topk_idx,
                double *topk_w);
/* Grouping of the T*k token-expert pairs by expert (counting sort). */
int oracle_permute(const int32_t *topk_idx, int T, int k, int E,
                   int32_t *expert_offsets, int32_t *sorted_pair,
                   int32_t *pair_pos);
/* Quantizers of one [R][K] fp32 matrix, groups of 128 along K. */
int oracle_quantize_w4(const float *w, int64_t R, int K, uint8_t *codes,
                       uint16_t *scales_f16);
int oracle_quantize_bp8(const float *w, int64_t R, int K, uint8_t *planes,
                        uint16_t *scales_f16);
/* Dequantized weights s*q (exact) of one [R][K] matrix, as fp64. */
int oracle_dequant_w4(const uint8_t *codes, const uint16_t *scales_f16,
                      int64_t R, int K, double *w);
int oracle_dequant_bp(const uint8_t *planes, const uint16_t *scales_f16,
                      int64_t R, int K, int bits, double *w);
/* Weight-space distortion of one bitplane expert at prefix widths 1..8
 * (dist[8]), fixed fp64 summation order (see oracle.c). */
int oracle_bp_distortion(const uint8_t *gu_planes, const uint16_t *gu_scales,
                         const uint8_t *dn_planes, const uint16_t *dn_scales,
                         int d, int f, double *dist);
/* Read-budget bit allocation: per-expert Lagrangian choice, bisection on the
 * multiplier (see oracle.c).  dist [E][8], counts [E] routing counts. */
int oracle_allocate_bits(const double *dist, const int32_t *counts, int E, int d,
                         int f, int bmin, int bmax, int64_t budget, uint8_t *bits,
                         double *lambda_out, int64_t *read_out);
/* Bit-width of every pair [T*k] from a bits mode (see oracle.c). */
int oracle_pair_bits(int T, int k, int E, const int32_t *topk_idx,
                     int bits_mode, const uint8_t *bits, uint8_t *pair_bits);
/* SwiGLU expert FFN for n token rows of one expert. */
int oracle_expert_ffn(const uint16_t *x_rows_bf16, int n, int d, int f,
                      const double *w_gate_up, const double *w_down,
                      double *h_out, double *y_out);
/* Weighted combine of the pair outputs y [T*k][d] (sorted order). */
int oracle_combine(const double *y_pairs, const int32_t *pair_pos,
                   const double *topk_w, int T, int k, int d, double *o,
                   uint16_t *out_bf16);

/* Rounding helpers exposed for the tests (the oracle's own). */
uint16_t oracle_f64_to_bf16(double v);
uint16_t oracle_f64_to_f16(double v);
double oracle_f16_to_f64(uint16_t h);

#ifdef __cplusplus
}
#endif
#endif /* MOE_ORACLE_H */
