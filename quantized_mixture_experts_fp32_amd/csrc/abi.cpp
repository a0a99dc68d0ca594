// C ABI of the MoE layer library: argument validation (before anything is
// enqueued), status codes and dispatch to the gfx950 kernel launchers.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include "../../include/moe_wq.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_ffn_ev[4] = {nullptr, nullptr, nullptr, nullptr};

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return MOE_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// k <= E holds for routing; the expert FFN may receive a slice of the
// experts (fewer than k of them), so it skips that check.
int check_dims(int T, int d, int E, int k, bool k_le_E = true) {
  if (T < 0 || d <= 0 || E <= 0 || k <= 0)
    return fail(MOE_ERR_INVALID_ARG, "negative or zero size (T=%d d=%d E=%d k=%d)",
                T, d, E, k);
  if (k_le_E && k > E) return fail(MOE_ERR_INVALID_ARG, "k=%d > E=%d", k, E);
  if (E > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_UNSUPPORTED, "E=%d > %d", E, MOE_MAX_EXPERTS);
  if (k > MOE_MAX_TOPK) return fail(MOE_ERR_UNSUPPORTED, "k=%d > %d", k, MOE_MAX_TOPK);
  if ((long long)T * k >= (1LL << 31))
    return fail(MOE_ERR_UNSUPPORTED, "T*k must be below 2^31");
  if (d % MOE_GROUP) return fail(MOE_ERR_UNSUPPORTED, "d=%d not a multiple of 128", d);
  if (d > MOE_MAX_D) return fail(MOE_ERR_UNSUPPORTED, "d=%d > %d", d, MOE_MAX_D);
  return MOE_OK;
}

}  // namespace

namespace moe {
int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}
}  // namespace moe

extern "C" {

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_err; }

size_t moe_route_ws_bytes(int T, int E) {
  if (T < 0 || E <= 0) return 0;
  return moe::route_ws_bytes(T, E);
}

int moe_route(const void* x_bf16, const void* wr_bf16, const float* bias,
              int T, int d, int E, int k, int32_t* topk_idx, float* topk_w,
              void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(T, d, E, k);
  if (rc) return rc;
  if (T == 0) return ok();
  if (!x_bf16 || !wr_bf16 || !topk_idx || !topk_w)
    return fail(MOE_ERR_INVALID_ARG, "moe_route: null pointer");
  const size_t need = moe::route_ws_bytes(T, E);
  if (need && (!ws || ws_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "moe_route: workspace %zu < %zu bytes",
                ws ? ws_bytes : (size_t)0, need);
  if (!aligned(x_bf16, 16) || !aligned(wr_bf16, 16) || !aligned(topk_idx, 4) ||
      !aligned(topk_w, 4) || (bias && !aligned(bias, 4)) || (need && !aligned(ws, 16)))
    return fail(MOE_ERR_INVALID_ARG, "moe_route: misaligned pointer");
  return hip_status(moe::launch_route(x_bf16, wr_bf16, bias, T, d, E, k,
                                      topk_idx, topk_w, ws, (hipStream_t)stream),
                    "moe_route");
}

size_t moe_permute_ws_bytes(int T, int k, int E) {
  if (T < 0 || k <= 0 || E <= 0) return 0;
  return moe::permute_ws_bytes(T, k, E);
}

int moe_permute(const int32_t* topk_idx, int T, int k, int E,
                int32_t* expert_offsets, int32_t* sorted_pair,
                int32_t* pair_pos, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(T, MOE_GROUP, E, k);
  if (rc) return rc;
  if (!expert_offsets) return fail(MOE_ERR_INVALID_ARG, "moe_permute: null offsets");
  if (T > 0 && (!topk_idx || !sorted_pair || !pair_pos))
    return fail(MOE_ERR_INVALID_ARG, "moe_permute: null pointer");
  const size_t need = moe::permute_ws_bytes(T, k, E);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_permute: workspace %zu < %zu bytes",
                ws ? ws_bytes : (size_t)0, need);
  if (!aligned(ws, 16) || !aligned(expert_offsets, 4) ||
      (T > 0 && (!aligned(topk_idx, 4) || !aligned(sorted_pair, 4) ||
                 !aligned(pair_pos, 4))))
    return fail(MOE_ERR_INVALID_ARG, "moe_permute: misaligned pointer");
  return hip_status(moe::launch_permute(topk_idx, T, k, E, expert_offsets,
                                        sorted_pair, pair_pos, ws,
                                        (hipStream_t)stream),
                    "moe_permute");
}

size_t moe_route_permute_ws_bytes(int T, int k, int E) {
  if (T < 0 || k <= 0 || E <= 0) return 0;
  return moe::route_permute_ws_bytes(T, k, E);
}

static int route_permute_check(const void* x_bf16, const void* wr_bf16, const float* bias,
                               int T, int d, int E, int k, int32_t* topk_idx, float* topk_w,
                               int32_t* expert_offsets, int32_t* sorted_pair,
                               int32_t* pair_pos, void* ws, size_t ws_bytes) {
  int rc = check_dims(T, d, E, k);
  if (rc) return rc;
  if (!expert_offsets) return fail(MOE_ERR_INVALID_ARG, "moe_route_permute: null offsets");
  if (T > 0 && (!x_bf16 || !wr_bf16 || !topk_idx || !topk_w || !sorted_pair || !pair_pos))
    return fail(MOE_ERR_INVALID_ARG, "moe_route_permute: null pointer");
  const size_t need = moe::route_permute_ws_bytes(T, k, E);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_route_permute: workspace %zu < %zu bytes",
                ws ? ws_bytes : (size_t)0, need);
  if (!aligned(ws, 16) || !aligned(expert_offsets, 4) ||
      (T > 0 && (!aligned(x_bf16, 16) || !aligned(wr_bf16, 16) || !aligned(topk_idx, 4) ||
                 !aligned(topk_w, 4) || (bias && !aligned(bias, 4)) ||
                 !aligned(sorted_pair, 4) || !aligned(pair_pos, 4))))
    return fail(MOE_ERR_INVALID_ARG, "moe_route_permute: misaligned pointer");
  return MOE_OK;
}

int moe_route_permute(const void* x_bf16, const void* wr_bf16, const float* bias, int T,
                      int d, int E, int k, int32_t* topk_idx, float* topk_w,
                      int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_pos,
                      void* ws, size_t ws_bytes, void* stream) {
  int rc = route_permute_check(x_bf16, wr_bf16, bias, T, d, E, k, topk_idx, topk_w,
                               expert_offsets, sorted_pair, pair_pos, ws, ws_bytes);
  if (rc) return rc;
  return hip_status(moe::launch_route_permute(x_bf16, wr_bf16, bias, T, d, E, k, topk_idx,
                                              topk_w, expert_offsets, sorted_pair, pair_pos,
                                              ws, (hipStream_t)stream),
                    "moe_route_permute");
}

size_t moe_ffn_ws_bytes(int T, int k, int E, int d, int f, int format) {
  if (T < 0 || k <= 0 || E <= 0 || d <= 0 || f <= 0) return 0;
  return moe::ffn_ws_bytes(T, k, E, d, f, format);
}

// Checks of moe_expert_ffn_wq; *path receives the resolved path.
static int ffn_check(const void* x_bf16, const int32_t* expert_offsets,
                     const int32_t* sorted_pair, int T, int k, int E, int d, int f,
                     int format, int group_size, const uint8_t* gate_up_codes,
                     const uint16_t* gate_up_scales_f16, const uint8_t* down_codes,
                     const uint16_t* down_scales_f16, const uint8_t* bits, int bits_mode,
                     float* y_pairs, void* ws, size_t ws_bytes, int path_hint, int* path) {
  int rc = check_dims(T, d, E, k, false);
  if (rc) return rc;
  if (f <= 0) return fail(MOE_ERR_INVALID_ARG, "f=%d", f);
  if (f % MOE_GROUP) return fail(MOE_ERR_UNSUPPORTED, "f=%d not a multiple of 128", f);
  if (group_size != MOE_GROUP)
    return fail(MOE_ERR_UNSUPPORTED, "group_size=%d (only 128)", group_size);
  if (format != MOE_FMT_W4_SYM && format != MOE_FMT_BITPLANE8)
    return fail(MOE_ERR_INVALID_ARG, "unknown format %d", format);
  if (path_hint < MOE_PATH_AUTO || path_hint > MOE_PATH_PREFILL)
    return fail(MOE_ERR_INVALID_ARG, "unknown path_hint %d", path_hint);
  if (format == MOE_FMT_W4_SYM) {
    if (bits_mode != MOE_BITS_NONE || bits)
      return fail(MOE_ERR_INVALID_ARG, "int4 format takes MOE_BITS_NONE and bits NULL");
  } else {
    if (bits_mode == MOE_BITS_RANK_RULE) {
      if (k != 8)
        return fail(MOE_ERR_UNSUPPORTED, "the rank bit-width rule needs k == 8");
    } else if (bits_mode == MOE_BITS_PER_PAIR || bits_mode == MOE_BITS_PER_EXPERT) {
      if (T > 0 && !bits) return fail(MOE_ERR_INVALID_ARG, "bits is NULL");
    } else {
      return fail(MOE_ERR_INVALID_ARG, "bitplane format needs a bits mode");
    }
  }
  if (T == 0) return ok();
  if (!x_bf16 || !expert_offsets || !sorted_pair || !gate_up_codes ||
      !gate_up_scales_f16 || !down_codes || !down_scales_f16 || !y_pairs)
    return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn_wq: null pointer");
  if (!aligned(x_bf16, 16) || !aligned(gate_up_codes, 16) ||
      !aligned(down_codes, 16) || !aligned(y_pairs, 16) ||
      !aligned(gate_up_scales_f16, 4) || !aligned(down_scales_f16, 4) ||
      !aligned(expert_offsets, 4) || !aligned(sorted_pair, 4))
    return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn_wq: misaligned pointer");
  const size_t need = moe::ffn_ws_bytes(T, k, E, d, f, format);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_expert_ffn_wq: workspace %zu < %zu bytes",
                ws ? ws_bytes : (size_t)0, need);
  if (!aligned(ws, 256))
    return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn_wq: workspace not 256-byte aligned");
  const long long P = (long long)T * k;
  *path = path_hint;
  // weight streaming while experts receive few pairs on average; an expert
  // receives at most T pairs (one per token), so T <= 16 always streams
  if (*path == MOE_PATH_AUTO)
    *path = (P <= 8LL * E || T <= 16) ? MOE_PATH_DECODE : MOE_PATH_PREFILL;
  // the prefill kernels address a gathered activation row (gate/up: one of
  // T tokens; down: one of an expert's at most T pairs) by a 32-bit byte
  // offset of row * K * 2 from a uniform base
  if (*path == MOE_PATH_PREFILL && (long long)T * (d > f ? d : f) * 2 > 0xFFFFFFFFLL)
    return fail(MOE_ERR_UNSUPPORTED,
                "prefill: T * max(d, f) * 2 = %lld bytes exceeds 2^32 - 1; split the batch",
                (long long)T * (d > f ? d : f) * 2);
  return MOE_OK;
}

int moe_expert_ffn_wq(const void* x_bf16, const int32_t* expert_offsets,
                      const int32_t* sorted_pair, int T, int k, int E, int d,
                      int f, int format, int group_size,
                      const uint8_t* gate_up_codes,
                      const uint16_t* gate_up_scales_f16,
                      const uint8_t* down_codes,
                      const uint16_t* down_scales_f16, const uint8_t* bits,
                      int bits_mode, float* y_pairs, void* ws, size_t ws_bytes,
                      int path_hint, void* stream) {
  int path = 0;
  int rc = ffn_check(x_bf16, expert_offsets, sorted_pair, T, k, E, d, f, format, group_size,
                     gate_up_codes, gate_up_scales_f16, down_codes, down_scales_f16, bits,
                     bits_mode, y_pairs, ws, ws_bytes, path_hint, &path);
  if (rc || T == 0) return rc;
  moe::FfnArgs a{(const uint16_t*)x_bf16, expert_offsets, sorted_pair, T, k, E,
                 d, f, format, gate_up_codes, gate_up_scales_f16, down_codes,
                 down_scales_f16, bits, bits_mode, y_pairs, ws, path,
                 {g_ffn_ev[0], g_ffn_ev[1], g_ffn_ev[2], g_ffn_ev[3]}};
  for (auto& ev : g_ffn_ev) ev = nullptr;  // one-shot
  return hip_status(moe::launch_ffn(a, (hipStream_t)stream), "moe_expert_ffn_wq");
}

int moe_set_ffn_events(void* gateup_begin, void* gateup_end, void* down_begin,
                       void* down_end) {
  g_ffn_ev[0] = (hipEvent_t)gateup_begin;
  g_ffn_ev[1] = (hipEvent_t)gateup_end;
  g_ffn_ev[2] = (hipEvent_t)down_begin;
  g_ffn_ev[3] = (hipEvent_t)down_end;
  return ok();
}

static int combine_check(const float* y_pairs, const int32_t* pair_pos, const float* topk_w,
                         int T, int k, int d, void* out, int out_dtype) {
  if (T < 0 || k <= 0 || d <= 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_combine: bad size");
  if (k > MOE_MAX_TOPK) return fail(MOE_ERR_UNSUPPORTED, "k=%d > %d", k, MOE_MAX_TOPK);
  if (d % 4) return fail(MOE_ERR_UNSUPPORTED, "d must be a multiple of 4");
  if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_F32)
    return fail(MOE_ERR_INVALID_ARG, "unknown out_dtype %d", out_dtype);
  if (T == 0) return ok();
  if (!y_pairs || !pair_pos || !topk_w || !out)
    return fail(MOE_ERR_INVALID_ARG, "moe_combine: null pointer");
  if (!aligned(y_pairs, 16) || !aligned(out, 16) || !aligned(pair_pos, 4) ||
      !aligned(topk_w, 4))
    return fail(MOE_ERR_INVALID_ARG, "moe_combine: misaligned pointer");
  return MOE_OK;
}

int moe_combine(const float* y_pairs, const int32_t* pair_pos,
                const float* topk_w, int T, int k, int d, void* out,
                int out_dtype, void* stream) {
  int rc = combine_check(y_pairs, pair_pos, topk_w, T, k, d, out, out_dtype);
  if (rc || T == 0) return rc;
  return hip_status(moe::launch_combine(y_pairs, pair_pos, topk_w, T, k, d, out,
                                        out_dtype == MOE_OUT_F32,
                                        (hipStream_t)stream),
                    "moe_combine");
}

static int quantize_common(const float* w, int E, int N, int K, int group,
                           uint8_t* codes, uint16_t* scales, int bitplane,
                           void* stream) {
  if (E < 0 || N < 0 || K <= 0)
    return fail(MOE_ERR_INVALID_ARG, "quantize: bad size");
  if (group != MOE_GROUP) return fail(MOE_ERR_UNSUPPORTED, "group_size=%d", group);
  if (K % MOE_GROUP) return fail(MOE_ERR_UNSUPPORTED, "K=%d not a multiple of 128", K);
  if (N % 16)
    return fail(MOE_ERR_UNSUPPORTED, "quantize: N=%d not a multiple of 16 (tiled rows)", N);
  if ((long long)E * N == 0) return ok();
  if (!w || !codes || !scales) return fail(MOE_ERR_INVALID_ARG, "quantize: null pointer");
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 2))
    return fail(MOE_ERR_INVALID_ARG, "quantize: misaligned pointer");
  return hip_status(moe::launch_quantize(w, E, N, K, bitplane, codes, scales,
                                         (hipStream_t)stream),
                    "quantize");
}

int moe_quantize_w4(const float* w, int E, int N, int K, int group_size,
                    uint8_t* codes, uint16_t* scales_f16, void* stream) {
  return quantize_common(w, E, N, K, group_size, codes, scales_f16, 0, stream);
}

int moe_quantize_bitplane8(const float* w, int E, int N, int K, int group_size,
                           uint8_t* planes, uint16_t* scales_f16, void* stream) {
  return quantize_common(w, E, N, K, group_size, planes, scales_f16, 1, stream);
}

static int retile_check(const uint8_t* in, int E, int N, int K, const uint8_t* out,
                        size_t bytes, const char* what) {
  if (E < 0 || N < 0 || K <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: bad size", what);
  if (K % MOE_GROUP) return fail(MOE_ERR_UNSUPPORTED, "%s: K=%d not a multiple of 128", what, K);
  if (N % 16) return fail(MOE_ERR_UNSUPPORTED, "%s: N=%d not a multiple of 16", what, N);
  if ((long long)E * N == 0) return ok();
  if (!in || !out) return fail(MOE_ERR_INVALID_ARG, "%s: null pointer", what);
  if (!aligned(in, 16) || !aligned(out, 16))
    return fail(MOE_ERR_INVALID_ARG, "%s: misaligned pointer", what);
  const uintptr_t a = (uintptr_t)in, b = (uintptr_t)out;
  if (a < b + bytes && b < a + bytes)
    return fail(MOE_ERR_INVALID_ARG, "%s: input and output overlap", what);
  return MOE_OK;
}

int moe_retile_w4(const uint8_t* codes_canonical, int E, int N, int K, uint8_t* codes,
                  void* stream) {
  const size_t bytes = (size_t)E * N * (K > 0 ? K : 0) / 2;
  int rc = retile_check(codes_canonical, E, N, K, codes, bytes, "moe_retile_w4");
  if (rc || (long long)E * N == 0) return rc;
  return hip_status(moe::launch_retile_w4(codes_canonical, (long long)E * N, K, codes,
                                          (hipStream_t)stream),
                    "moe_retile_w4");
}

int moe_retile_bitplane8(const uint8_t* planes_canonical, int E, int N, int K,
                         uint8_t* planes, void* stream) {
  const size_t bytes = (size_t)E * N * (K > 0 ? K : 0);
  int rc = retile_check(planes_canonical, E, N, K, planes, bytes, "moe_retile_bitplane8");
  if (rc || (long long)E * N == 0) return rc;
  return hip_status(moe::launch_retile_bp(planes_canonical, E, N, K, planes,
                                          (hipStream_t)stream),
                    "moe_retile_bitplane8");
}

}  // extern "C"

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t moe_layer_ws_bytes(int T, int k, int E, int d, int f, int format) {
  if (T < 0 || k <= 0 || E <= 0 || d <= 0 || f <= 0) return 0;
  const size_t ffn = moe::ffn_ws_bytes(T, k, E, d, f, format);
  const size_t em = moe::em_h_bytes(E, f);
  return align256(moe::route_permute_ws_bytes(T, k, E)) + (ffn > em ? ffn : em);
}

int moe_layer_forward_wq(const void* x_bf16, const void* wr_bf16, const float* bias, int T,
                         int d, int E, int k, int f, int format, int group_size,
                         const uint8_t* gate_up_codes, const uint16_t* gate_up_scales_f16,
                         const uint8_t* down_codes, const uint16_t* down_scales_f16,
                         const uint8_t* bits, int bits_mode, int32_t* topk_idx,
                         float* topk_w, int32_t* expert_offsets, int32_t* sorted_pair,
                         int32_t* pair_pos, float* y_pairs, void* out, int out_dtype,
                         void* ws, size_t ws_bytes, int path_hint, void* stream) {
  const size_t need = moe_layer_ws_bytes(T, k, E, d, f, format);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_layer_forward_wq: workspace %zu < %zu bytes",
                ws ? ws_bytes : (size_t)0, need);
  if (!aligned(ws, 256))
    return fail(MOE_ERR_INVALID_ARG, "moe_layer_forward_wq: workspace not 256-byte aligned");
  const size_t rp_b = align256(moe::route_permute_ws_bytes(T, k, E));
  void* ws_ffn = (char*)ws + rp_b;
  int path = 0;
  int rc = route_permute_check(x_bf16, wr_bf16, bias, T, d, E, k, topk_idx, topk_w,
                               expert_offsets, sorted_pair, pair_pos, ws, rp_b);
  if (!rc)
    rc = ffn_check(x_bf16, expert_offsets, sorted_pair, T, k, E, d, f, format, group_size,
                   gate_up_codes, gate_up_scales_f16, down_codes, down_scales_f16, bits,
                   bits_mode, y_pairs, ws_ffn, ws_bytes - rp_b, path_hint, &path);
  if (!rc) rc = combine_check(y_pairs, pair_pos, topk_w, T, k, d, out, out_dtype);
  if (rc) return rc;
  const hipStream_t s = (hipStream_t)stream;
  if (T == 0)  // no tokens: expert_offsets becomes all zero, as from moe_route_permute
    return hip_status(moe::launch_route_permute(x_bf16, wr_bf16, bias, 0, d, E, k, topk_idx,
                                                topk_w, expert_offsets, sorted_pair,
                                                pair_pos, ws, s),
                      "moe_layer_forward_wq");
  moe::FfnArgs a{(const uint16_t*)x_bf16, expert_offsets, sorted_pair, T, k, E,
                 d, f, format, gate_up_codes, gate_up_scales_f16, down_codes,
                 down_scales_f16, bits, bits_mode, y_pairs, ws_ffn, path,
                 {g_ffn_ev[0], g_ffn_ev[1], g_ffn_ev[2], g_ffn_ev[3]}};
  for (auto& ev : g_ffn_ev) ev = nullptr;  // one-shot
  hipError_t e;
  if (path == MOE_PATH_DECODE && moe::em_applies(T, k, E, d, f, format)) {
    // the grouping comes out of the expert-major kernels; for E <= 64 they
    // take the routing (and select the top-k) from logits that the routing
    // launch spreads over (token, 16 experts) blocks
    // (the logits variant needs a gate/up block b for every token b < T, i.e.
    // E * f / 128 >= T; smaller layers route first and take topk_idx)
    if (moe::em_selects_topk(T, k, E) && (long long)E * (f / 128) >= T) {
      float* logits = (float*)ws;  // route_ws_bytes(T, E) <= rp_b
      e = moe::launch_route_logits(x_bf16, wr_bf16, bias, T, d, E, logits, s);
      if (e == hipSuccess)
        e = moe::launch_ffn_decode_em(a, nullptr, expert_offsets, sorted_pair, pair_pos,
                                      (uint16_t*)ws_ffn, s, logits, topk_idx, topk_w);
    } else {
      e = moe::launch_route(x_bf16, wr_bf16, bias, T, d, E, k, topk_idx, topk_w, ws, s);
      if (e == hipSuccess)
        e = moe::launch_ffn_decode_em(a, topk_idx, expert_offsets, sorted_pair, pair_pos,
                                      (uint16_t*)ws_ffn, s);
    }
  } else if (path == MOE_PATH_DECODE && moe::decode_selects_topk(T, k, E, d, f, format)) {
    // at most 64 pairs: the decode gate/up routes the batch from the logits
    float* logits = (float*)ws;  // route_ws_bytes(T, E) <= rp_b
    a.logits = logits;
    a.topk_idx_out = topk_idx;
    a.topk_w_out = topk_w;
    a.offsets_out = expert_offsets;
    a.sorted_pair_out = sorted_pair;
    a.pair_pos_out = pair_pos;
    e = moe::launch_route_logits(x_bf16, wr_bf16, bias, T, d, E, logits, s);
    if (e == hipSuccess) e = moe::launch_ffn(a, s);
  } else {
    e = moe::launch_route_permute(x_bf16, wr_bf16, bias, T, d, E, k, topk_idx, topk_w,
                                  expert_offsets, sorted_pair, pair_pos, ws, s);
    if (e == hipSuccess) e = moe::launch_ffn(a, s);
  }
  if (e == hipSuccess)
    e = moe::launch_combine(y_pairs, pair_pos, topk_w, T, k, d, out, out_dtype == MOE_OUT_F32,
                            s);
  return hip_status(e, "moe_layer_forward_wq");
}

size_t moe_bp_distortion_ws_bytes(int E, int d, int f) {
  if (E <= 0 || d <= 0 || f <= 0) return 0;
  return moe::bp_distortion_ws_bytes(E, d, f);
}

int moe_bp_distortion(const uint8_t* gate_up_planes, const uint16_t* gate_up_scales_f16,
                      const uint8_t* down_planes, const uint16_t* down_scales_f16, int E,
                      int d, int f, double* dist, void* ws, size_t ws_bytes, void* stream) {
  if (E <= 0 || d <= 0 || f <= 0) return fail(MOE_ERR_INVALID_ARG, "moe_bp_distortion: bad size");
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "E=%d > %d", E, MOE_MAX_EXPERTS);
  if (d % MOE_GROUP || f % MOE_GROUP)
    return fail(MOE_ERR_UNSUPPORTED, "d=%d, f=%d must be multiples of 128", d, f);
  if (!gate_up_planes || !gate_up_scales_f16 || !down_planes || !down_scales_f16 || !dist)
    return fail(MOE_ERR_INVALID_ARG, "moe_bp_distortion: null pointer");
  if (!aligned(gate_up_planes, 16) || !aligned(down_planes, 16) || !aligned(dist, 8) ||
      !aligned(gate_up_scales_f16, 2) || !aligned(down_scales_f16, 2))
    return fail(MOE_ERR_INVALID_ARG, "moe_bp_distortion: misaligned pointer");
  const size_t need = moe::bp_distortion_ws_bytes(E, d, f);
  if (!ws || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_bp_distortion: workspace %zu < %zu bytes",
                ws ? ws_bytes : (size_t)0, need);
  if (!aligned(ws, 8)) return fail(MOE_ERR_INVALID_ARG, "moe_bp_distortion: misaligned workspace");
  return hip_status(moe::launch_bp_distortion(gate_up_planes, gate_up_scales_f16, down_planes,
                                              down_scales_f16, E, d, f, dist, ws,
                                              (hipStream_t)stream),
                    "moe_bp_distortion");
}

int moe_allocate_bits(const double* dist, const int32_t* counts, int E, int d, int f,
                      int b_min, int b_max, int64_t budget_bytes, uint8_t* bits,
                      double* lambda, int64_t* read_bytes, void* stream) {
  if (E <= 0 || d <= 0 || f <= 0) return fail(MOE_ERR_INVALID_ARG, "moe_allocate_bits: bad size");
  if (E > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "E=%d > %d", E, MOE_MAX_EXPERTS);
  if (d % MOE_GROUP || f % MOE_GROUP)
    return fail(MOE_ERR_UNSUPPORTED, "d=%d, f=%d must be multiples of 128", d, f);
  if (b_min < 1 || b_max > 8 || b_min > b_max)
    return fail(MOE_ERR_INVALID_ARG, "bit range [%d, %d] outside 1..8", b_min, b_max);
  if (!dist || !counts || !bits)
    return fail(MOE_ERR_INVALID_ARG, "moe_allocate_bits: null pointer");
  if (!aligned(dist, 8) || !aligned(counts, 4) || (lambda && !aligned(lambda, 8)) ||
      (read_bytes && !aligned(read_bytes, 8)))
    return fail(MOE_ERR_INVALID_ARG, "moe_allocate_bits: misaligned pointer");
  return hip_status(moe::launch_allocate_bits(dist, counts, E, d, f, b_min, b_max, budget_bytes,
                                              bits, lambda, read_bytes, (hipStream_t)stream),
                    "moe_allocate_bits");
}

