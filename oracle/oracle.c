/*
 * oracle.c -- plain, slow CPU definition of the routed-expert W4A16 MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the CPU
 * baseline of the benchmark, never by the GPU library (they share no code).
 * Built with gcc -O2 -ffp-contract=off, no fast-math; OpenMP only splits
 * independent rows, so results do not depend on the thread count.
 *
 * Every function states the passage it follows; "reading" marks a choice
 * made where the pages are silent (see oracle.h for the page titles).
 *
 * Parity pins: every function here is checked by the CPU tests against an
 * independent fact (hand-derived worked examples, closed forms, library
 * routines, brute force, invariants).  No function is "parity unpinned".
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ floats */

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round v to p significant bits, round-half-even, with a subnormal range
 * below 2^emin (the IEEE binary formats bf16: p=8, emin=-126; fp16: p=11,
 * emin=-14).  v / q is exact (power-of-two scaling), nearbyint is RNE. */
static double round_sig(double v, int p, int emin) {
  if (v == 0.0 || isnan(v) || isinf(v)) return v;
  int e;
  frexp(fabs(v), &e); /* |v| in [2^(e-1), 2^e) */
  int lead = e - 1;
  if (lead < emin) lead = emin;
  double q = ldexp(1.0, lead - (p - 1));
  return nearbyint(v / q) * q;
}

uint16_t oracle_f64_to_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double r = round_sig(v, 8, -126);
  if (fabs(r) > 3.3895313892515355e38) return sign | 0x7F80;
  float f = (float)r; /* exact: r has <= 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

uint16_t oracle_f64_to_f16(double v) {
  if (isnan(v)) return 0x7E00;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(round_sig(v, 11, -14));
  if (a > 65504.0) return sign | 0x7C00;
  if (a == 0.0) return sign;
  if (a < ldexp(1.0, -14)) /* subnormal: multiple of 2^-24 */
    return sign | (uint16_t)(a / ldexp(1.0, -24));
  int e;
  double m = frexp(a, &e); /* a = (2m) * 2^(e-1), 2m in [1,2) */
  uint16_t mant = (uint16_t)((2.0 * m - 1.0) * 1024.0);
  return sign | (uint16_t)((e - 1 + 15) << 10) | mant;
}

double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1, ex = (h >> 10) & 0x1F, man = h & 0x3FF;
  double v;
  if (ex == 0)
    v = ldexp((double)man, -24);
  else if (ex == 31)
    v = man ? NAN : INFINITY;
  else
    v = ldexp(1.0 + man / 1024.0, ex - 15);
  return sign ? -v : v;
}

/* ------------------------------------------------------------------ router */

/* Router logits (ExactMoE, Abstract: the router stays BF16 and the top-k
 * routing procedure is unchanged).  x and W_r are bf16; logits accumulate in
 * fp32.  Reading: because the top-k indices are compared bit for bit, the
 * fp32 summation order is fixed as part of the definition.  Sixteen partial
 * sums acc_0..acc_15 start at +0; acc_l adds, in this order, the products of
 * elements i = 128c + 8l + r for c = 0, 1, ... and r = 0..7.  The partials
 * are then combined pairwise, acc_l <- acc_l + acc_(l xor o) for o = 8, 4, 2,
 * 1, and the logit is acc_0 + b_e (b_e = 0 without a bias).  A bf16*bf16
 * product is exact in fp32, so only the order of the additions matters.
 * Requires d % 128 == 0. */
int oracle_router_logits(const uint16_t *x_bf16, const uint16_t *wr_bf16,
                         const float *bias, int T, int d, int E,
                         float *logits) {
  if (T < 0 || d <= 0 || d % 128 || E <= 0 || !logits) return -1;
  if (T == 0) return 0;
  if (!x_bf16 || !wr_bf16) return -1;
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const uint16_t *x = x_bf16 + (int64_t)t * d;
    for (int e = 0; e < E; ++e) {
      const uint16_t *w = wr_bf16 + (int64_t)e * d;
      float acc[16];
      for (int l = 0; l < 16; ++l) acc[l] = 0.0f;
      for (int c = 0; c < d / 128; ++c)
        for (int l = 0; l < 16; ++l)
          for (int r = 0; r < 8; ++r) {
            int i = 128 * c + 8 * l + r;
            float prod = bf16_to_f32(x[i]) * bf16_to_f32(w[i]);
            acc[l] = acc[l] + prod;
          }
      for (int o = 8; o >= 1; o >>= 1) {
        float nxt[16];
        for (int l = 0; l < 16; ++l) nxt[l] = acc[l] + acc[l ^ o];
        for (int l = 0; l < 16; ++l) acc[l] = nxt[l];
      }
      float b = bias ? bias[e] : 0.0f;
      logits[(int64_t)t * E + e] = acc[0] + b;
    }
  }
  return 0;
}

/* Top-k and routing weights (ExactMoE, Abstract: unchanged top-k routing).
 * Reading: experts are ranked by logit, larger first, equal logits toward
 * the lower expert index (softmax is monotone, so this is the order of the
 * scores); rank 1 is written first.  The weights are the softmax over all E
 * experts renormalised over the k selected ones, here in fp64. */
int oracle_topk(const float *logits, int T, int E, int k, int32_t *topk_idx,
                double *topk_w) {
  if (T < 0 || E <= 0 || k <= 0 || k > E) return -1;
  if (T == 0) return 0;
  if (!logits || !topk_idx || !topk_w) return -1;
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const float *l = logits + (int64_t)t * E;
    char *taken = (char *)calloc((size_t)E, 1);
    int32_t *idx = topk_idx + (int64_t)t * k;
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
      taken[best] = 1;
      idx[j] = best;
    }
    free(taken);
    double m = l[idx[0]], z = 0.0;
    for (int e = 0; e < E; ++e) z += exp((double)l[e] - m);
    double sel = 0.0;
    for (int j = 0; j < k; ++j) sel += exp((double)l[idx[j]] - m) / z;
    for (int j = 0; j < k; ++j)
      topk_w[(int64_t)t * k + j] = (exp((double)l[idx[j]] - m) / z) / sel;
  }
  return 0;
}

/* ----------------------------------------------------------------- permute */

/* Grouping of the pairs by expert for grouped execution (ExactMoE, Abstract:
 * fused grouped MoE kernels run all selected experts).  Pair p = t*k + j.
 * Reading: the group order is deterministic -- a counting sort: counts per
 * expert, exclusive prefix sum into expert_offsets[0..E], then the pairs in
 * ascending p are appended to their expert's segment.  pair_pos is the
 * inverse map (slot of pair p). */
int oracle_permute(const int32_t *topk_idx, int T, int k, int E,
                   int32_t *expert_offsets, int32_t *sorted_pair,
                   int32_t *pair_pos) {
  if (T < 0 || k <= 0 || E <= 0 || !expert_offsets) return -1;
  int64_t P = (int64_t)T * k;
  if (P && (!topk_idx || !sorted_pair || !pair_pos)) return -1;
  int32_t *count = (int32_t *)calloc((size_t)E, sizeof(int32_t));
  for (int64_t p = 0; p < P; ++p) {
    if (topk_idx[p] < 0 || topk_idx[p] >= E) {
      free(count);
      return -1;
    }
    count[topk_idx[p]]++;
  }
  expert_offsets[0] = 0;
  for (int e = 0; e < E; ++e) expert_offsets[e + 1] = expert_offsets[e] + count[e];
  for (int e = 0; e < E; ++e) count[e] = 0;
  for (int64_t p = 0; p < P; ++p) {
    int e = topk_idx[p];
    int32_t slot = expert_offsets[e] + count[e]++;
    sorted_pair[slot] = (int32_t)p;
    pair_pos[p] = slot;
  }
  free(count);
  return 0;
}

/* --------------------------------------------------------------- quantize */

static float group_absmax(const float *w) {
  float a = 0.0f;
  for (int i = 0; i < 128; ++i)
    if (fabsf(w[i]) > a) a = fabsf(w[i]);
  return a;
}

/* Symmetric group-128 4-bit quantization of routed-expert weights (ExactMoE,
 * Abstract).  Per row and per group of 128 consecutive input-dimension
 * elements: s = fp16(max|w| / 7), rounded to nearest even from the exact
 * quotient; q = clamp(round_half_even(w / s), -7, 7), or 0 when s == 0.
 * Reading: both quotients are taken in fp64, whose rounding to fp16 / to an
 * integer equals the rounding of the exact quotient for fp32 inputs.
 * Packing: byte (r, j) holds element 2j in its low nibble and 2j+1 in its
 * high nibble, two's complement. */
int oracle_quantize_w4(const float *w, int64_t R, int K, uint8_t *codes,
                       uint16_t *scales_f16) {
  if (R < 0 || K <= 0 || K % 128) return -1;
  if (R == 0) return 0;
  if (!w || !codes || !scales_f16) return -1;
  int G = K / 128;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    for (int g = 0; g < G; ++g) {
      const float *wg = w + r * K + 128 * g;
      uint16_t s16 = oracle_f64_to_f16((double)group_absmax(wg) / 7.0);
      double s = oracle_f16_to_f64(s16);
      scales_f16[r * G + g] = s16;
      for (int i = 0; i < 128; i += 2) {
        int q[2];
        for (int h = 0; h < 2; ++h) {
          double v = (s == 0.0) ? 0.0 : nearbyint((double)wg[i + h] / s);
          if (v > 7.0) v = 7.0;
          if (v < -7.0) v = -7.0;
          q[h] = (int)v;
        }
        codes[r * (K / 2) + (128 * g + i) / 2] =
            (uint8_t)((q[0] & 0xF) | ((q[1] & 0xF) << 4));
      }
    }
  }
  return 0;
}

/* Bitplane storage of one 8-bit offset code per weight (PagedMoE, abstract:
 * each expert stored once in a bitplane layout so that lower precisions are
 * prefixes of higher ones).  Per group of 128: s = fp16(max|w| / 127) from
 * the exact quotient, u = clamp(round_half_even(w / s) + 128, 0, 255), or 128
 * when s == 0.  Layout of an [R][K] matrix: 8 plane slabs [8][R][K/8], slab
 * p holding bit 7-p of u (most significant first), so the top b planes are
 * the first b slabs; bit i of byte (r, j) belongs to element 8j + i. */
int oracle_quantize_bp8(const float *w, int64_t R, int K, uint8_t *planes,
                        uint16_t *scales_f16) {
  if (R < 0 || K <= 0 || K % 128) return -1;
  if (R == 0) return 0;
  if (!w || !planes || !scales_f16) return -1;
  int G = K / 128;
  int64_t slab = R * (K / 8);
  memset(planes, 0, (size_t)(8 * slab));
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    for (int g = 0; g < G; ++g) {
      const float *wg = w + r * K + 128 * g;
      uint16_t s16 = oracle_f64_to_f16((double)group_absmax(wg) / 127.0);
      double s = oracle_f16_to_f64(s16);
      scales_f16[r * G + g] = s16;
      for (int i = 0; i < 128; ++i) {
        double v = (s == 0.0) ? 128.0 : nearbyint((double)wg[i] / s) + 128.0;
        if (v > 255.0) v = 255.0;
        if (v < 0.0) v = 0.0;
        int u = (int)v, el = 128 * g + i;
        for (int p = 0; p < 8; ++p)
          if ((u >> (7 - p)) & 1)
            planes[p * slab + r * (K / 8) + el / 8] |= (uint8_t)(1u << (el % 8));
      }
    }
  }
  return 0;
}

/* Dequantized int4 weight s * q, exact (ExactMoE, Abstract: W4A16). */
int oracle_dequant_w4(const uint8_t *codes, const uint16_t *scales_f16,
                      int64_t R, int K, double *w) {
  if (R < 0 || K <= 0 || K % 128) return -1;
  if (R == 0) return 0;
  if (!codes || !scales_f16 || !w) return -1;
  int G = K / 128;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r)
    for (int i = 0; i < K; ++i) {
      uint8_t byte = codes[r * (K / 2) + i / 2];
      int nib = (i % 2) ? (byte >> 4) : (byte & 0xF);
      int q = nib >= 8 ? nib - 16 : nib;
      w[r * K + i] = oracle_f16_to_f64(scales_f16[r * G + i / 128]) * q;
    }
  return 0;
}

/* Dequantized weight of a b-bit prefix (PagedMoE, abstract: a b-bit prefix
 * is executed directly from the top b planes; MatMoE, abstract:
 * floor-and-compensation).  Only slabs 0..b-1 are read: u_b is u with its
 * 8-b low bits cleared (the floor), and the compensation adds half of the
 * dropped range, 2^(7-b); v = u_b + 2^(7-b) - 128 for b < 8 and v = u - 128
 * for b = 8; the weight is s * v (exact). */
int oracle_dequant_bp(const uint8_t *planes, const uint16_t *scales_f16,
                      int64_t R, int K, int bits, double *w) {
  if (R < 0 || K <= 0 || K % 128 || bits < 1 || bits > 8) return -1;
  if (R == 0) return 0;
  if (!planes || !scales_f16 || !w) return -1;
  int G = K / 128;
  int64_t slab = R * (K / 8);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r)
    for (int i = 0; i < K; ++i) {
      int ub = 0;
      for (int p = 0; p < bits; ++p)
        ub |= ((planes[p * slab + r * (K / 8) + i / 8] >> (i % 8)) & 1) << (7 - p);
      int v = (bits == 8) ? ub - 128 : ub + (1 << (7 - bits)) - 128;
      w[r * K + i] = oracle_f16_to_f64(scales_f16[r * G + i / 128]) * v;
    }
  return 0;
}

/* Bit-width of every pair p = t*k + j.  bits_mode 0: none (8-bit codes read
 * in full); 1: bits[p] per pair; 2: bits[e] per expert; 3: the rank rule of
 * the dynamic-precision workload (rank 1 -> 8 bits, ranks 2-4 -> 4, ranks
 * 5-8 -> 2; requires k == 8).  Precision per token-expert pair and per
 * expert follows PagedMoE (abstract) and MatMoE (abstract). */
int oracle_pair_bits(int T, int k, int E, const int32_t *topk_idx,
                     int bits_mode, const uint8_t *bits, uint8_t *pair_bits) {
  if (T < 0 || k <= 0 || E <= 0) return -1;
  int64_t P = (int64_t)T * k;
  if (P == 0) return 0;
  if (!pair_bits) return -1;
  if (bits_mode == 3 && k != 8) return -1;
  if ((bits_mode == 1 || bits_mode == 2) && !bits) return -1;
  if (bits_mode == 2 && !topk_idx) return -1;
  for (int64_t p = 0; p < P; ++p) {
    int b;
    switch (bits_mode) {
      case 0: b = 8; break;
      case 1: b = bits[p]; break;
      case 2: b = bits[topk_idx[p]]; break;
      case 3: {
        int j = (int)(p % k);
        b = (j == 0) ? 8 : (j < 4 ? 4 : 2);
        break;
      }
      default: return -1;
    }
    if (b < 1 || b > 8) return -1;
    pair_bits[p] = (uint8_t)b;
  }
  return 0;
}

/* ---------------------------------------------------------------- expert */

/* SwiGLU expert FFN in W4A16 form (ExactMoE, Abstract).  w_gate_up is the
 * dequantized [2f][d] matrix (gate rows 0..f-1, up rows f..2f-1), w_down the
 * dequantized [d][f] matrix.  For every token row: g = Wg x, u = Wu x (fp64
 * sums); silu(g) = g / (1 + exp(-g)).  Reading of "A16": the intermediate
 * activation is bf16, h = bf16_rne(silu(g) * u); then y = Wd h (fp64).
 * h_out (optional) receives h as fp64 values, y_out is [n][d]. */
int oracle_expert_ffn(const uint16_t *x_rows_bf16, int n, int d, int f,
                      const double *w_gate_up, const double *w_down,
                      double *h_out, double *y_out) {
  if (n < 0 || d <= 0 || f <= 0) return -1;
  if (n == 0) return 0;
  if (!x_rows_bf16 || !w_gate_up || !w_down || !y_out) return -1;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < n; ++r) {
    double *x = (double *)malloc(sizeof(double) * (size_t)d);
    double *h = (double *)malloc(sizeof(double) * (size_t)f);
    for (int i = 0; i < d; ++i)
      x[i] = bf16_to_f32(x_rows_bf16[(int64_t)r * d + i]);
    for (int j = 0; j < f; ++j) {
      const double *wg = w_gate_up + (int64_t)j * d;
      const double *wu = w_gate_up + (int64_t)(f + j) * d;
      double g = 0.0, u = 0.0;
      for (int i = 0; i < d; ++i) {
        g += wg[i] * x[i];
        u += wu[i] * x[i];
      }
      double silu = g / (1.0 + exp(-g));
      uint16_t hb = oracle_f64_to_bf16(silu * u);
      h[j] = bf16_to_f32(hb);
      if (h_out) h_out[(int64_t)r * f + j] = h[j];
    }
    for (int m = 0; m < d; ++m) {
      const double *wd = w_down + (int64_t)m * f;
      double acc = 0.0;
      for (int j = 0; j < f; ++j) acc += wd[j] * h[j];
      y_out[(int64_t)r * d + m] = acc;
    }
    free(x);
    free(h);
  }
  return 0;
}

/* Combine (ExactMoE, Abstract: every selected expert contributes): the layer
 * output of token t is o_t = sum over ranks j of w_tj * y_(t,j), summed in
 * rank order (fp64), and the bf16 output is bf16_rne(o_t).  y_pairs is in
 * grouped order, pair p = t*k + j lives at slot pair_pos[p]. */
int oracle_combine(const double *y_pairs, const int32_t *pair_pos,
                   const double *topk_w, int T, int k, int d, double *o,
                   uint16_t *out_bf16) {
  if (T < 0 || k <= 0 || d <= 0) return -1;
  if (T == 0) return 0;
  if (!y_pairs || !pair_pos || !topk_w || !o) return -1;
  for (int t = 0; t < T; ++t)
    for (int m = 0; m < d; ++m) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) {
        int64_t slot = pair_pos[(int64_t)t * k + j];
        acc += topk_w[(int64_t)t * k + j] * y_pairs[slot * d + m];
      }
      o[(int64_t)t * d + m] = acc;
      if (out_bf16) out_bf16[(int64_t)t * d + m] = oracle_f64_to_bf16(acc);
    }
  return 0;
}

/* Read-side bit allocation (DuoRate, "Two-Rate Per-Expert Precision
 * Allocation for Mixture-of-Experts Serving": the routing-weighted read rate
 * sum_e f_e R(M_e); a Lagrangian relaxation whose per-expert minimizer does
 * not depend on f_e; selection by one evaluation per expert and a bisection
 * on the multiplier to meet a read budget).  The distortion is taken in
 * weight space from the stored codes (no calibration data), and the
 * precisions are the prefixes of the bitplane codes (PagedMoE, abstract;
 * MatMoE, abstract: floor-and-compensation).
 *
 * Distortion of one expert at prefix width b (1..8): the squared error of
 * its b-bit prefix weights against its 8-bit weights, over gate/up ([2f][d])
 * and down ([d][f]).  Per element, v_b - v_8 = 2^(7-b) - (u mod 2^(8-b)),
 * an integer; per 128-group the squared differences sum to an exact integer
 * I; the group contributes (s*s)*I (s*s exact in fp64, one rounding).  The
 * sum order is fixed: groups ascending within a row from +0 (a row partial),
 * then the row partials of gate/up rows 0..2f-1 followed by down rows
 * 0..d-1, from +0.  Planes are the oracle's slab layout [8][R][K/8]. */
static double bp_row_distortion(const uint8_t *planes, int64_t slab, int64_t r,
                                int K, const uint16_t *scales, int b) {
  int G = K / 128;
  double acc = 0.0;
  for (int g = 0; g < G; ++g) {
    int64_t I = 0;
    for (int i = 128 * g; i < 128 * (g + 1); ++i) {
      int u = 0;
      for (int p = 0; p < 8; ++p)
        u |= ((planes[p * slab + r * (K / 8) + i / 8] >> (i % 8)) & 1) << (7 - p);
      int64_t diff = (b == 8) ? 0 : (1 << (7 - b)) - (u & ((1 << (8 - b)) - 1));
      I += diff * diff;
    }
    double s = oracle_f16_to_f64(scales[r * G + g]);
    acc = acc + (s * s) * (double)I;
  }
  return acc;
}

int oracle_bp_distortion(const uint8_t *gu_planes, const uint16_t *gu_scales,
                         const uint8_t *dn_planes, const uint16_t *dn_scales,
                         int d, int f, double *dist) {
  if (d <= 0 || f <= 0 || d % 128 || f % 128) return -1;
  if (!gu_planes || !gu_scales || !dn_planes || !dn_scales || !dist) return -1;
  int64_t gu_slab = (int64_t)2 * f * (d / 8), dn_slab = (int64_t)d * (f / 8);
  for (int b = 1; b <= 8; ++b) {
    double tot = 0.0;
    for (int64_t r = 0; r < 2 * (int64_t)f; ++r)
      tot = tot + bp_row_distortion(gu_planes, gu_slab, r, d, gu_scales, b);
    for (int64_t r = 0; r < d; ++r)
      tot = tot + bp_row_distortion(dn_planes, dn_slab, r, f, dn_scales, b);
    dist[b - 1] = tot;
  }
  return 0;
}

/* Bytes read for one expert at prefix width b: b planes of gate/up and down
 * (3df/8 bytes each) plus the fp16 scales (3df/64 bytes). */
static int64_t bp_read_bytes(int d, int f, int b) {
  return (int64_t)b * 3 * d * f / 8 + (int64_t)3 * d * f / 64;
}

/* The per-expert Lagrangian choice: b in [bmin, bmax] minimizing
 * D_e(b) + lambda * R(b), evaluated as fma(lambda, R(b), D_e(b)); ties go to
 * the larger b.  The routing count of the expert does not enter. */
static int alloc_choose(const double *dist_e, int bmin, int bmax, int d, int f,
                        double lambda) {
  int best = bmax;
  double key = fma(lambda, (double)bp_read_bytes(d, f, bmax), dist_e[bmax - 1]);
  for (int b = bmax - 1; b >= bmin; --b) {
    double kb = fma(lambda, (double)bp_read_bytes(d, f, b), dist_e[b - 1]);
    if (kb < key) {
      key = kb;
      best = b;
    }
  }
  return best;
}

/* Read rate at a multiplier: sum_e counts_e * R(b_e(lambda)), exact. */
static int64_t alloc_read(const double *dist, const int32_t *counts, int E, int bmin,
                          int bmax, int d, int f, double lambda) {
  int64_t tot = 0;
  for (int e = 0; e < E; ++e)
    tot += (int64_t)counts[e] *
           bp_read_bytes(d, f, alloc_choose(dist + 8 * e, bmin, bmax, d, f, lambda));
  return tot;
}

/* Bisection on the multiplier.  lambda = 0 when the widest choice already
 * meets the budget.  Otherwise hi starts at 1 and doubles (at most 2^1023)
 * until its read meets the budget; then 64 halvings of [lo, hi] keep read(hi)
 * within the budget and read(lo) above it; the result is b_e(hi).  When even
 * the narrowest choice exceeds the budget every expert gets bmin (the
 * returned read then exceeds the budget). */
int oracle_allocate_bits(const double *dist, const int32_t *counts, int E, int d,
                         int f, int bmin, int bmax, int64_t budget, uint8_t *bits,
                         double *lambda_out, int64_t *read_out) {
  if (E <= 0 || d <= 0 || f <= 0 || bmin < 1 || bmax > 8 || bmin > bmax) return -1;
  if (!dist || !counts || !bits) return -1;
  for (int e = 0; e < E; ++e)
    if (counts[e] < 0) return -1;
  double lambda = 0.0;
  if (alloc_read(dist, counts, E, bmin, bmax, d, f, 0.0) > budget) {
    double lo = 0.0, hi = 1.0;
    int n = 0;
    while (alloc_read(dist, counts, E, bmin, bmax, d, f, hi) > budget && n < 1023) {
      lo = hi;
      hi = hi * 2.0;
      ++n;
    }
    if (alloc_read(dist, counts, E, bmin, bmax, d, f, hi) > budget) {
      hi = INFINITY;
    } else {
      for (int it = 0; it < 64; ++it) {
        double mid = 0.5 * (lo + hi);
        if (alloc_read(dist, counts, E, bmin, bmax, d, f, mid) <= budget)
          hi = mid;
        else
          lo = mid;
      }
    }
    lambda = hi;
  }
  for (int e = 0; e < E; ++e)
    bits[e] = (uint8_t)(isinf(lambda) ? bmin
                                      : alloc_choose(dist + 8 * e, bmin, bmax, d, f, lambda));
  if (lambda_out) *lambda_out = lambda;
  if (read_out) {
    int64_t tot = 0;
    for (int e = 0; e < E; ++e) tot += (int64_t)counts[e] * bp_read_bytes(d, f, bits[e]);
    *read_out = tot;
  }
  return 0;
}

