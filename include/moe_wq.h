/*
 * moe_wq.h -- C ABI of the MI355X (gfx950) routed-expert MoE FFN with
 * low-bit weight-only quantized experts (W4A16 and bitplane prefixes).
 *
 * One forward pass of the layer is four calls on one HIP stream:
 *
 *   moe_route          x, router weights -> top-k expert ids and weights
 *   moe_permute        top-k ids -> pairs grouped by expert
 *   moe_expert_ffn_wq  grouped pairs -> per-pair SwiGLU expert outputs
 *   moe_combine        per-pair outputs -> layer output
 *
 * plus the offline quantizers moe_quantize_w4 / moe_quantize_bitplane8.
 *
 * The pages this follows:
 *  [ExactMoE] "Every Expert Counts: ExactMoE for Memory-Efficient W4A16
 *    Inference", Abstract: symmetric group-128 four-bit quantization of the
 *    routed experts only; router in BF16; unchanged top-k routing; all
 *    selected experts executed (none pruned or substituted) by fused grouped
 *    MoE kernels.
 *  [PagedMoE] "PagedMoE: Cross-Precision Expert Caching for Token-Level
 *    Dynamic Precision in SSD-Resident MoE Inference", abstract: each expert
 *    stored once as bitplanes whose lower precisions are prefixes of higher
 *    ones; 1-8-bit prefixes executed directly, chosen per token from the
 *    routing.
 *  [MatMoE] "MatMoE: Matryoshka Mixture-of-Experts with Dynamic
 *    Mixed-Precision Quantization for Efficient Inference", abstract:
 *    floor-and-compensation dequantization of the nested representation;
 *    per-expert bit-width from routing scores.
 *
 * Conventions (all calls):
 *  - Every pointer is a DEVICE pointer (hipMalloc / torch CUDA memory) unless
 *    stated otherwise.  The caller owns all memory; the library allocates
 *    nothing.  Scratch memory is a caller-provided workspace whose size the
 *    *_ws_bytes queries return.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work; they never synchronise the host.  Kernel faults surface at
 *    the caller's next synchronisation.
 *  - Arguments are validated before anything is enqueued: a call that
 *    returns an error has written nothing.  T == 0 is a valid no-op.
 *  - Integer results (top-k ids, grouping, codes, scales) are deterministic
 *    and bit-identical to the plain CPU definition; floating-point results
 *    are deterministic run to run (no floating-point atomics).
 *  - Calls are re-entrant; concurrent calls must use distinct outputs and
 *    workspaces.
 */
#ifndef MOE_WQ_H
#define MOE_WQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG 1 /* null / misaligned pointer, bad size      */
#define MOE_ERR_UNSUPPORTED 2 /* valid but outside the supported shapes   */
#define MOE_ERR_WORKSPACE 3   /* workspace missing or too small           */
#define MOE_ERR_HIP 4         /* the HIP runtime rejected a launch        */

/* ---- enumerations ---------------------------------------------------- */
#define MOE_FMT_W4_SYM 0    /* int4 codes, two per byte, fp16 group scales */
#define MOE_FMT_BITPLANE8 1 /* 8 bitplanes of an 8-bit offset code         */

#define MOE_BITS_NONE 0       /* int4 format: no bit-width argument         */
#define MOE_BITS_PER_PAIR 1   /* bits[T*k], pair p = t*k + j                */
#define MOE_BITS_PER_EXPERT 2 /* bits[E]                                    */
#define MOE_BITS_RANK_RULE 3  /* rank 1 -> 8, ranks 2-4 -> 4, 5-8 -> 2; k=8 */

#define MOE_OUT_BF16 0 /* layer output as bf16 (round to nearest even)     */
#define MOE_OUT_F32 1  /* layer output as fp32 (same sum, before rounding)  */

#define MOE_PATH_AUTO 0    /* DECODE if T*k <= 8*E or T <= 16, else PREFILL */
#define MOE_PATH_DECODE 1  /* weight-streaming kernels (small batches)     */
#define MOE_PATH_PREFILL 2 /* LDS-tiled grouped MFMA kernels               */

/* ---- limits ---------------------------------------------------------- */
#define MOE_GROUP 128     /* quantization group along the input dimension */
#define MOE_MAX_EXPERTS 512
#define MOE_MAX_TOPK 16
#define MOE_MAX_D 8192   /* router stages eight activation rows in LDS */
/* d and f must be multiples of 128, d <= MOE_MAX_D; T*k below 2^31. */

/* Human-readable name of a status code. */
const char *moe_status_str(int status);
/* Detail of the last error returned on the calling thread ("" if none). */
const char *moe_last_error(void);

/* ---------------------------------------------------------------------
 * moe_route -- router logits, softmax, top-k, renormalised weights.
 * [ExactMoE] Abstract: the router stays BF16 and the top-k procedure is
 * unchanged.  Definition:
 *   logit[t][e] = sum_i x[t][i] * wr[e][i] in fp32, in a FIXED order: 16
 *     partial sums, partial l adding elements i = 128c + 8l + r for c = 0,1,..
 *     and r = 0..7 in that order; partials combined as acc_l += acc_(l^o) for
 *     o = 8,4,2,1; then + bias[e] (one fp32 add; no add term if bias NULL
 *     other than +0).  bf16*bf16 products are exact in fp32, so the logits
 *     are bit-identical to the CPU definition.
 *   topk_idx[t][0..k-1]: the k experts with the largest logits, larger
 *     first, equal logits toward the lower index (= order of the softmax
 *     scores).
 *   topk_w[t][j] = softmax(logit[t])[idx_j] / sum_j softmax(logit[t])[idx_j]
 *     (fp32; computed as the softmax over the k selected logits).
 * Arguments:
 *   x      bf16 [T][d] row-major, 16-byte aligned.
 *   wr     bf16 [E][d] (router matrix stored expert-major), 16-byte aligned.
 *   bias   fp32 [E] logit bias, or NULL.
 *   topk_idx int32 [T][k]; topk_w fp32 [T][k]  (outputs).
 *   ws / ws_bytes: workspace of at least moe_route_ws_bytes(T, E) bytes
 *     (small batches keep the fp32 logits there; may be 0 bytes / NULL
 *     when the query returns 0).
 * Requires d % 128 == 0, d <= 8192, 1 <= k <= min(E, 16), E <= 512.
 * ------------------------------------------------------------------- */
size_t moe_route_ws_bytes(int T, int E);
int moe_route(const void *x_bf16, const void *wr_bf16, const float *bias,
              int T, int d, int E, int k, int32_t *topk_idx, float *topk_w,
              void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------
 * moe_permute -- group the P = T*k token-expert pairs by expert.
 * [ExactMoE] Abstract: fused grouped execution of all selected experts.
 * Deterministic counting sort: pair p = t*k + j; expert_offsets[e] =
 * number of pairs with expert < e (so expert_offsets[E] = P); within an
 * expert, pairs keep ascending p.  sorted_pair[slot] = p and pair_pos[p] =
 * slot (inverse maps).
 * Arguments:
 *   topk_idx int32 [T][k] with values in [0, E).  Out-of-range ids make the
 *     kernels skip the pair (results then undefined; not checked on host).
 *   expert_offsets int32 [E+1]; sorted_pair, pair_pos int32 [T*k] (outputs).
 *   ws / ws_bytes: workspace of at least moe_permute_ws_bytes(T, k, E).
 * ------------------------------------------------------------------- */
size_t moe_permute_ws_bytes(int T, int k, int E);
int moe_permute(const int32_t *topk_idx, int T, int k, int E,
                int32_t *expert_offsets, int32_t *sorted_pair,
                int32_t *pair_pos, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------
 * moe_route_permute -- moe_route followed by moe_permute, with the same
 * outputs bit for bit, in fewer launches for small batches (T <= 512: the
 * logits kernel, then one block that selects every token's top-k and
 * groups the pairs).  Arguments as for the two calls; ws / ws_bytes: at
 * least moe_route_permute_ws_bytes(T, k, E).  T = 0 writes expert_offsets
 * (all zero) and nothing else.
 * ------------------------------------------------------------------- */
size_t moe_route_permute_ws_bytes(int T, int k, int E);
int moe_route_permute(const void *x_bf16, const void *wr_bf16, const float *bias,
                      int T, int d, int E, int k, int32_t *topk_idx, float *topk_w,
                      int32_t *expert_offsets, int32_t *sorted_pair, int32_t *pair_pos,
                      void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------
 * moe_expert_ffn_wq -- SwiGLU FFN of every grouped pair with quantized,
 * in-kernel dequantized expert weights.
 * [ExactMoE] Abstract (W4A16, grouped kernels); [PagedMoE] abstract
 * (bitplane prefixes executed directly); [MatMoE] abstract (floor and
 * compensation).  For the pair in slot r (token t = sorted_pair[r] / k,
 * expert e):
 *   g = Wg' x_t, u = Wu' x_t   (fp32 sums over d)
 *   h = bf16_rne(silu(g) * u),  silu(g) = g / (1 + exp(-g))     ("A16")
 *   y_pairs[r] = Wd' h          (fp32 sums over f)
 * with dequantized weights W' = s * q (int4) or W' = s * v_b(u) (bitplane,
 * b = the pair's bit-width): v_b = (u with its 8-b low bits cleared)
 * + 2^(7-b) - 128 for b < 8, and u - 128 for b = 8.  Only the top max_b(e)
 * planes of expert e are read, where max_b(e) is the largest b among its
 * pairs.  Dequantized weights are never rounded: integer codes enter the
 * bf16 MFMA exactly and the fp16 scale multiplies each 128-group partial sum
 * in fp32.
 * Weight layouts (K = input dimension, contiguous; groups of 128 along K):
 *   MOE_FMT_W4_SYM (codes tiled for streaming, as moe_quantize_w4 writes
 *   them): a matrix of R rows (R = E*2f gate/up, E*d down; rows of expert e
 *   start at e*2f resp. e*d; gate rows 0..f-1 then up rows f..2f-1 of each
 *   expert) and K inputs is stored as u8 [R/16][K/128][16][64]: the codes of
 *   row n, elements 128g .. 128g+127, are the 64 bytes at
 *   (((n/16)*(K/128) + g)*16 + n%16)*64, read as 16 little-endian 32-bit
 *   words; word j holds elements 128g+8j .. +7: element 8j+2i in nibble i
 *   (bits 4i..4i+3) and element 8j+2i+1 in nibble 4+i, for i = 0..3; each
 *   nibble is two's complement in [-7, 7].  (One 16-row tile's group is
 *   1 KiB contiguous.)
 *     gate_up_codes: R = E*2f, K = d (E*f*d bytes);  gate_up_scales fp16
 *     [E][2f][d/128];  down_codes: R = E*d, K = f;  down_scales fp16
 *     [E][d][f/128].
 *   MOE_FMT_BITPLANE8 (u = 8-bit offset code, w ~ s * (u - 128)): a matrix
 *   of R rows (as for int4) and K inputs is stored as u8
 *   [R/16][K/128][4][16][4][2][4]: for 16-row tile n/16 and group g a 2 KiB
 *   block holds the 8 planes (plane p = bit 7-p of u, most significant
 *   first) as 4 plane pairs c of 512 bytes (planes 2c, 2c+1); within pair c
 *   row r = n%16 takes 32 bytes at 32 r, its quarter q (elements
 *   128g + 32q .. 128g + 32q + 31) being the 4-byte word of plane 2c then
 *   that of plane 2c+1, and bit i of a word belongs to element
 *   128g + 32q + i.  Byte j of row r's 16 bytes of plane p is at
 *   512 (p/2) + 32 r + 8 (j/4) + 4 (p%2) + j%4.  The top b planes of every
 *   block lie in its first 512 ceil(b/2) bytes: a b-bit read loads only
 *   those (an odd b brings plane b along).
 *     gate_up_codes: R = E*2f, K = d;  down_codes: R = E*d, K = f;
 *     scales as for int4.
 * Bit-widths (bitplane only): bits_mode MOE_BITS_PER_PAIR (bits u8 [T*k],
 *   indexed by pair p), MOE_BITS_PER_EXPERT (bits u8 [E]) or
 *   MOE_BITS_RANK_RULE (bits NULL; requires k == 8); values in [1, 8].
 *   The int4 format takes MOE_BITS_NONE and bits NULL.
 * Other arguments:
 *   x bf16 [T][d]; expert_offsets, sorted_pair as from moe_permute.
 *   E counts the experts whose weights this call receives (E may be below
 *     k).  Slot positions in expert_offsets are absolute, so experts
 *     [e0, e0+E) of a larger grouping are run by passing expert_offsets + e0
 *     and each weight/scale pointer advanced by e0 experts (and bits + e0
 *     for MOE_BITS_PER_EXPERT); y_pairs rows of the other experts are left
 *     untouched.
 *   y_pairs fp32 [T*k][d] in grouped (slot) order (output).
 *   ws / ws_bytes: at least moe_ffn_ws_bytes(T, k, E, d, f, format).
 *   path_hint: MOE_PATH_AUTO / _DECODE / _PREFILL (all give results within
 *     the same tolerance of the CPU definition).
 * Alignment: x, codes and y_pairs 16-byte aligned; scales 4-byte aligned.
 * Requires d % 128 == 0, d <= 8192, f % 128 == 0, E <= 512, 1 <= k <= 16.
 * On the prefill path (chosen, or taken by MOE_PATH_AUTO when T > 16 and
 * T*k > 8E) T * max(d, f) * 2 must not exceed 2^32 - 1 bytes (e.g. T <=
 * 262143 at d = 8192); larger batches return MOE_ERR_UNSUPPORTED before any
 * launch and are run as several calls.
 * ------------------------------------------------------------------- */
size_t moe_ffn_ws_bytes(int T, int k, int E, int d, int f, int format);
int moe_expert_ffn_wq(const void *x_bf16, const int32_t *expert_offsets,
                      const int32_t *sorted_pair, int T, int k, int E, int d,
                      int f, int format, int group_size,
                      const uint8_t *gate_up_codes,
                      const uint16_t *gate_up_scales_f16,
                      const uint8_t *down_codes,
                      const uint16_t *down_scales_f16, const uint8_t *bits,
                      int bits_mode, float *y_pairs, void *ws,
                      size_t ws_bytes, int path_hint, void *stream);

/* ---------------------------------------------------------------------
 * moe_combine -- weighted sum of each token's k expert outputs.
 * [ExactMoE] Abstract: every selected expert contributes.
 *   o[t][m] = sum_{j<k} topk_w[t][j] * y_pairs[pair_pos[t*k+j]][m]
 * summed in rank order in fp32 from +0; out = o (MOE_OUT_F32) or
 * bf16_rne(o) (MOE_OUT_BF16).  out is [T][d], 16-byte aligned.
 * ------------------------------------------------------------------- */
int moe_combine(const float *y_pairs, const int32_t *pair_pos,
                const float *topk_w, int T, int k, int d, void *out,
                int out_dtype, void *stream);

/* ---------------------------------------------------------------------
 * moe_layer_forward_wq -- one routed-expert MoE layer step in one call:
 * the composition moe_route_permute -> moe_expert_ffn_wq -> moe_combine
 * with the same arguments, producing the same outputs bit for bit
 * (topk_idx, topk_w, expert_offsets, sorted_pair, pair_pos, y_pairs, out).
 * [ExactMoE] Abstract: unchanged top-k routing, every selected expert
 * executed by grouped kernels, outputs combined.
 * When the decode path applies to an int4 layer with T <= 16 and
 * 2 T k >= E, the grouping is computed inside the expert gate/up kernel
 * (expert-major work items; no separate permute launch); otherwise the
 * three steps run as listed.
 * ws / ws_bytes: at least moe_layer_ws_bytes(T, k, E, d, f, format),
 *   256-byte aligned, caller-owned, no contents carried between calls.
 * Every argument is checked as by the three entry points before anything
 * is enqueued; error codes as there.  Timing events armed with
 * moe_set_ffn_events apply to its gate/up and down kernels.
 * ------------------------------------------------------------------- */
size_t moe_layer_ws_bytes(int T, int k, int E, int d, int f, int format);
int moe_layer_forward_wq(const void *x_bf16, const void *wr_bf16, const float *bias,
                         int T, int d, int E, int k, int f, int format,
                         int group_size, const uint8_t *gate_up_codes,
                         const uint16_t *gate_up_scales_f16,
                         const uint8_t *down_codes,
                         const uint16_t *down_scales_f16, const uint8_t *bits,
                         int bits_mode, int32_t *topk_idx, float *topk_w,
                         int32_t *expert_offsets, int32_t *sorted_pair,
                         int32_t *pair_pos, float *y_pairs, void *out,
                         int out_dtype, void *ws, size_t ws_bytes, int path_hint,
                         void *stream);

/* ---------------------------------------------------------------------
 * moe_layer_forward_wq_noalloc -- for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The step of moe_layer_forward_wq with the same
 * arguments except the workspace, whose place is taken by a fixed array of
 * MOE_NOALLOC_SCRATCH_BYTES in device memory inside the library.  Outputs
 * (bit for bit) and error codes as for moe_layer_forward_wq.
 * Limit: moe_layer_ws_bytes(T, k, E, d, f, format) must not exceed
 *   MOE_NOALLOC_SCRATCH_BYTES (32 MiB: every decode batch of up to 64 tokens
 *   of the d = 4096, E = 256, f = 2048 layer fits in 16.1 MiB; a 4096-token
 *   prefill of the OLMoE-shaped layer needs 67 MiB); a larger step returns
 *   MOE_ERR_WORKSPACE before touching the device.
 * Ownership: each GPU holds its own copy of the array, from the library's
 *   load on that device until the process ends.  The first call on a device
 *   looks up the array's address there (the device current at the call);
 *   no call allocates or frees memory.  stream must belong to the current
 *   device.
 * Sharing: every call on one GPU uses that GPU's array, which keeps the last
 *   call's contents; nothing in it needs to start at zero (each kernel
 *   writes what it reads within the call).  Calls on one stream are ordered;
 *   calls that overlap in time on one GPU (other streams or threads without
 *   ordering between them) race on the array and give undefined results.
 * ------------------------------------------------------------------- */
#define MOE_NOALLOC_SCRATCH_BYTES (32 << 20)
int moe_layer_forward_wq_noalloc(const void *x_bf16, const void *wr_bf16, const float *bias,
                                 int T, int d, int E, int k, int f, int format,
                                 int group_size, const uint8_t *gate_up_codes,
                                 const uint16_t *gate_up_scales_f16,
                                 const uint8_t *down_codes,
                                 const uint16_t *down_scales_f16, const uint8_t *bits,
                                 int bits_mode, int32_t *topk_idx, float *topk_w,
                                 int32_t *expert_offsets, int32_t *sorted_pair,
                                 int32_t *pair_pos, float *y_pairs, void *out,
                                 int out_dtype, int path_hint, void *stream);

/* ---------------------------------------------------------------------
 * moe_bp_distortion -- weight-space distortion of bitplane experts, the
 * offline half of read-budget bit allocation.
 * [DuoRate] "Two-Rate Per-Expert Precision Allocation for Mixture-of-Experts
 * Serving": a distortion table is computed once, offline, per expert and
 * precision; [PagedMoE] abstract and [MatMoE] abstract: the precisions are
 * prefixes of one stored code with floor-and-compensation.
 *   dist[e][b-1], b = 1..8 (fp64, device, [E][8]) = sum over the expert's
 *   gate/up and down weights of (s * (v_b(u) - v_8(u)))^2, where
 *   v_b(u) - v_8(u) = 2^(7-b) - (u mod 2^(8-b)) and s is the group's fp16
 *   scale.  Order: per 128-group the integer sum I of squared prefix errors;
 *   row partial = groups in ascending order from +0 of fp64 (s*s)*I; total =
 *   row partials of gate/up rows 0..2f-1 then down rows 0..d-1 from +0; every
 *   product and sum rounded separately (reproducible bit for bit).
 * Planes and scales: as written by moe_quantize_bitplane8 for [E][2f][d]
 * (gate rows then up rows) and [E][d][f].  ws: moe_bp_distortion_ws_bytes
 * (8-byte aligned).  Requires d % 128 == 0, f % 128 == 0, E <= 512.
 * ------------------------------------------------------------------- */
size_t moe_bp_distortion_ws_bytes(int E, int d, int f);
int moe_bp_distortion(const uint8_t *gate_up_planes,
                      const uint16_t *gate_up_scales_f16,
                      const uint8_t *down_planes, const uint16_t *down_scales_f16,
                      int E, int d, int f, double *dist, void *ws,
                      size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------
 * moe_allocate_bits -- per-expert prefix width under a read budget, the
 * online half.
 * [DuoRate]: read rate sum_e f_e R(b_e); in the Lagrangian relaxation the
 * routing frequency cancels from each expert's decision, which is
 *   b_e(lambda) = argmin_{b_min <= b <= b_max} fma(lambda, R(b), dist[e][b-1])
 * (ties to the larger b), with R(b) = b*3df/8 + 3df/64 bytes read (planes
 * plus scales; the b planes a b-bit prefix needs -- the bitplane layout
 * fetches whole plane pairs, so an odd b moves one more plane of bytes);
 * a bisection on lambda meets the budget:
 *   read(lambda) = sum_e counts[e] * R(b_e(lambda)) (exact int64);
 *   lambda = 0 if read(0) <= budget_bytes; otherwise hi = 1, doubled (at
 *   most 1023 times) until read(hi) <= budget, then 64 halvings of [lo, hi]
 *   (mid = 0.5*(lo+hi)); the result is b_e(hi).  If even b_min everywhere
 *   exceeds the budget, lambda = +inf and every expert gets b_min.
 * counts: int32 [E] routing counts of a profiling window (>= 0).  bits: u8
 * [E] output, usable as MOE_BITS_PER_EXPERT.  lambda (fp64) and read_bytes
 * (int64): optional device outputs (NULL to skip); a read above the budget
 * signals an infeasible budget.  One 512-thread block; device pointers.
 * ------------------------------------------------------------------- */
int moe_allocate_bits(const double *dist, const int32_t *counts, int E, int d, int f,
                      int b_min, int b_max, int64_t budget_bytes, uint8_t *bits,
                      double *lambda, int64_t *read_bytes, void *stream);

/* ---------------------------------------------------------------------
 * moe_set_ffn_events -- optional timing instrumentation (no page defines
 * it; it serves throughput measurement).  Arms, for the NEXT
 * moe_expert_ffn_wq call made by the calling thread only, four hipEvent_t
 * handles (any may be NULL): the start and stop events of its gate/up
 * kernel and of its down kernel, attached to those kernel dispatches
 * (hipExtLaunchKernel), so that they time exactly the kernels and add no
 * separate marker to the stream.  The events are created and owned by the
 * caller.  Returns MOE_OK.
 * ------------------------------------------------------------------- */
int moe_set_ffn_events(void *gateup_begin, void *gateup_end,
                       void *down_begin, void *down_end);

/* ---------------------------------------------------------------------
 * HBM expert slot cache.  [ExactMoE] Abstract: the routed-expert bank sits
 * in pinned host memory in front of a device-side expert cache; [PagedMoE]
 * abstract: per-step precision is chosen from routing before any transfer,
 * and a step fetches only the bitplanes it is missing.
 *
 * moe_cache_create -- a cache of `slots` device slots (2 <= slots <= E) over
 * a bank of E experts of the given format.
 *   host_*: the whole bank, in the layouts above ([E] experts), in PINNED
 *     host memory (hipHostMalloc; checked, MOE_ERR_INVALID_ARG otherwise).
 *   slot_*: device arrays of `slots` experts in the same per-expert layout.
 *   Both stay owned by the caller and must outlive the cache.  The cache
 *   itself (host state, four copy streams, their events, small pinned
 *   buffers that its kernels read and write directly, and a device copy of
 *   all E experts' scales -- 1/32 of an int4 bank -- from which slots take
 *   their scales) is allocated here and freed by moe_cache_destroy.
 * moe_cache_forward -- one MoE layer step (as moe_layer_forward_wq: routing,
 *   grouping, expert FFN, combine) with the experts read from the slots:
 *   routes on `stream`, writes the per-expert request to pinned host memory
 *   and WAITS for it (the one host synchronisation of a step), assigns
 *   slots, issues the
 *   host-to-device copies of missing experts (bitplane: missing plane
 *   ranges of resident experts, whole prefixes of new ones) on the copy
 *   streams, and runs the FFN on `stream` after them.  Resident experts keep
 *   their slot; new ones take empty slots, then the least recently used.
 *   When a step routes to more experts than there are slots, the FFN runs in
 *   chunks: chunk 0 on all slots, then slot halves in turn, copies of the
 *   next chunk overlapping the FFN of the current one.
 *   Outputs: topk_idx, topk_w (as moe_route), pair_pos [T*k] and y_pairs
 *   [T*k][d] fp32 (grouped order of this step's internal grouping; pair p's
 *   output row is y_pairs[pair_pos[p]]), out [T][d] as moe_combine.
 *   ws: moe_cache_ws_bytes(cache, T, k) bytes, 256-byte aligned.  Calls
 *   that share a cache must not overlap (one stream, one thread at a time).
 * moe_cache_stats -- int64[6]: steps, expert hits, experts loaded whole,
 *   experts extended by missing planes, bytes copied from the host, FFN
 *   chunks.
 * moe_cache_slots -- the resident expert (-1: empty) and plane count of each
 *   slot (host arrays [slots]).
 * moe_cache_reset -- forget every resident expert and the statistics.
 * moe_cache_destroy -- waits for the last step's work, then frees the
 *   cache's own resources (never the caller's bank or slots).
 * A moe_cache_forward that fails with MOE_ERR_HIP leaves the cache with
 *   every slot empty.
 * moe_cache_plan -- the slot assignment of one step alone, on host state
 *   (no device work; for checking the policy): slot_expert/slot_bits/
 *   slot_last [slots] in/out, need [E] (widest prefix per routed expert,
 *   int4: 8; 0 = not routed).  Outputs vmap [E] (virtual expert id, -1),
 *   chunks [n][4] = {first virtual id, count, first slot, FFN chunk the
 *   copies wait for or -1}, loads [n][6] = {expert, slot, first plane, end
 *   plane, chunk, scales copied}, V = number of virtual experts.
 * ------------------------------------------------------------------- */
typedef struct moe_cache moe_cache;
int moe_cache_create(int E, int d, int f, int format, int slots,
                     const uint8_t *host_gate_up_codes, const uint16_t *host_gate_up_scales_f16,
                     const uint8_t *host_down_codes, const uint16_t *host_down_scales_f16,
                     uint8_t *slot_gate_up_codes, uint16_t *slot_gate_up_scales_f16,
                     uint8_t *slot_down_codes, uint16_t *slot_down_scales_f16,
                     moe_cache **cache);
void moe_cache_destroy(moe_cache *cache);
size_t moe_cache_ws_bytes(const moe_cache *cache, int T, int k);
int moe_cache_forward(moe_cache *cache, const void *x_bf16, const void *wr_bf16,
                      const float *bias, int T, int k, const uint8_t *bits, int bits_mode,
                      int32_t *topk_idx, float *topk_w, int32_t *pair_pos, float *y_pairs,
                      void *out, int out_dtype, void *ws, size_t ws_bytes, void *stream);
int moe_cache_stats(const moe_cache *cache, int64_t *stats6);
int moe_cache_slots(const moe_cache *cache, int32_t *slot_expert, int32_t *slot_bits);
int moe_cache_reset(moe_cache *cache);
int moe_cache_plan(int E, int slots, int format, int32_t *slot_expert, int32_t *slot_bits,
                   int64_t *slot_last, int64_t step, const int32_t *need, int32_t *vmap,
                   int32_t *chunks, int max_chunks, int *n_chunks, int32_t *loads,
                   int max_loads, int *n_loads, int *V);

/* ---------------------------------------------------------------------
 * Offline quantizers (untimed packing of fp32 expert weights on the GPU).
 * w is fp32 [E][N][K] (K = input dimension); groups of 128 along K.
 * moe_quantize_w4 ([ExactMoE] Abstract, symmetric group-128 4-bit):
 *   s = fp16_rne(max|w| / 7) (exact quotient), q = clamp(rne(w / s), -7, 7),
 *   q = 0 when s == 0.  codes: E*N*K/2 bytes in the tiled int4 layout above
 *   (R = E*N rows; requires N % 16 == 0), scales fp16 [E][N][K/128].
 * moe_quantize_bitplane8 ([PagedMoE] abstract, bitplane prefixes):
 *   s = fp16_rne(max|w| / 127), u = clamp(rne(w / s) + 128, 0, 255), u = 128
 *   when s == 0.  planes: E*N*K bytes in the bitplane layout above (R = E*N
 *   rows; requires N % 16 == 0), scales fp16 [E][N][K/128].
 * Codes and scales are bit-identical to the CPU definition.  Weights with
 * max|w| above 7 * 65504 (fp16 overflow of the scale) are unsupported.
 * ------------------------------------------------------------------- */
int moe_quantize_w4(const float *w, int E, int N, int K, int group_size,
                    uint8_t *codes, uint16_t *scales_f16, void *stream);
int moe_quantize_bitplane8(const float *w, int E, int N, int K,
                           int group_size, uint8_t *planes,
                           uint16_t *scales_f16, void *stream);

/* ---------------------------------------------------------------------
 * Canonical code layouts -> the streaming layouts above (a pure
 * rearrangement of bits, bit-exact; scales are already [E][N][K/128] in
 * both and need no conversion).  For codes produced elsewhere in the plain
 * row-major forms:
 * moe_retile_w4 ([ExactMoE] Abstract: symmetric 4-bit codes, two per byte):
 *   in  codes_canonical u8 [E][N][K/2]: byte (e, n, j) holds element 2j in
 *       its low nibble and 2j + 1 in its high nibble (two's complement);
 *   out codes, E*N*K/2 bytes in the tiled int4 layout of moe_expert_ffn_wq.
 * moe_retile_bitplane8 ([PagedMoE] abstract: one 8-bit code per weight as
 *   bitplanes whose lower precisions are prefixes):
 *   in  planes_canonical u8 [E][8][N][K/8]: per expert 8 plane slabs, slab p
 *       holding bit 7 - p of u (most significant first), bit i of byte
 *       (n, j) for element 8j + i;
 *   out planes, E*N*K bytes in the bitplane layout of moe_expert_ffn_wq.
 * Requires N % 16 == 0, K % 128 == 0; device pointers 16-byte aligned; the
 * input and output must not overlap (MOE_ERR_INVALID_ARG).  Gate/up codes
 * are converted with N = 2f (gate rows, then up rows), down codes with
 * N = d.  Stream-ordered; allocates nothing.
 * ------------------------------------------------------------------- */
int moe_retile_w4(const uint8_t *codes_canonical, int E, int N, int K, uint8_t *codes,
                  void *stream);
int moe_retile_bitplane8(const uint8_t *planes_canonical, int E, int N, int K,
                         uint8_t *planes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_WQ_H */
