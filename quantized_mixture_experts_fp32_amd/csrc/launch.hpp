// Host-side launchers of the gfx950 kernels (called by the C ABI in abi.cpp
// after argument validation).  Each returns the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Launch a kernel; when start/stop events are given they are attached to the
// dispatch itself (hipExtLaunchKernel), so they time exactly this kernel and
// put no separate marker into the stream.
template <typename... KArgs, typename... Args>
inline void launch_k(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds,
                     hipStream_t s, hipEvent_t start, hipEvent_t stop, Args... args) {
  if (start || stop)
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, start, stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}


size_t route_ws_bytes(int T, int E);
hipError_t launch_route(const void* x, const void* wr, const float* bias,
                        int T, int d, int E, int k, int32_t* topk_idx,
                        float* topk_w, void* ws, hipStream_t s);

// Router logits [T][E] fp32 into `logits` (T <= 512; route_ws_bytes(T, E)).
hipError_t launch_route_logits(const void* x, const void* wr, const float* bias, int T, int d,
                               int E, float* logits, hipStream_t s);
size_t route_permute_ws_bytes(int T, int k, int E);
hipError_t launch_route_permute(const void* x, const void* wr, const float* bias, int T,
                                int d, int E, int k, int32_t* topk_idx, float* topk_w,
                                int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                                void* ws, hipStream_t s);
size_t permute_ws_bytes(int T, int k, int E);
hipError_t launch_permute(const int32_t* topk_idx, int T, int k, int E,
                          int32_t* offsets, int32_t* sorted_pair,
                          int32_t* pair_pos, void* ws, hipStream_t s);

hipError_t launch_quantize(const float* w, long long E, long long N, int K,
                           int bitplane, uint8_t* codes, uint16_t* scales,
                           hipStream_t s);

struct FfnArgs {
  const uint16_t* x;
  const int32_t* offsets;
  const int32_t* sorted_pair;
  int T, k, E, d, f, format;
  const uint8_t* gu_codes;
  const uint16_t* gu_scales;
  const uint8_t* dn_codes;
  const uint16_t* dn_scales;
  const uint8_t* bits;
  int bits_mode;
  float* y;
  void* ws;
  int path;  // resolved: 1 decode, 2 prefill
  hipEvent_t ev[4];  // optional: gate/up begin/end, down begin/end
  // Optional (decode, at most 64 pairs): the router logits [T][E]; the
  // decode gate/up then selects the top-k and groups the pairs itself and
  // stores them to the routing outputs below (offsets and sorted_pair above
  // point to the same buffers as offsets_out and sorted_pair_out).
  const float* logits = nullptr;
  int32_t* topk_idx_out = nullptr;
  float* topk_w_out = nullptr;
  int32_t* offsets_out = nullptr;
  int32_t* sorted_pair_out = nullptr;
  int32_t* pair_pos_out = nullptr;
};
size_t ffn_ws_bytes(int T, int k, int E, int d, int f, int format);
hipError_t launch_ffn(const FfnArgs& a, hipStream_t s);
// decode path for int4 experts (ffn_decode.hip); h = bf16 [P][f] scratch
// Bitplane experts, small batches: true when every wave can stream a whole
// K range (the single-slice decode kernels apply).
bool ffn_decode_bp_applies(long long P, int E, int f);
hipError_t launch_ffn_decode_bp(const FfnArgs& a, uint16_t* h, hipStream_t s);
hipError_t launch_ffn_decode_w4(const FfnArgs& a, uint16_t* h, hipStream_t s);
// The int4 decode path can take the routing from logits (FfnArgs::logits):
// at most 64 pairs, E <= 64, with the K-split gate/up kernel.
bool decode_selects_topk(int T, int k, int E, int d, int f, int format);
// prefill path for int4 experts (ffn_prefill.hip); ws: its own scratch
size_t ffn_prefill_ws_bytes(int T, int k, int E, int d, int f);
hipError_t launch_ffn_prefill_w4(const FfnArgs& a, uint16_t* h, void* ws, hipStream_t s);
// prefill path for bitplane experts (ffn_prefill.hip), same workspace
hipError_t launch_ffn_prefill_bp(const FfnArgs& a, uint16_t* h, void* ws, hipStream_t s);

// expert-major decode of at most 16 tokens, int4 (ffn_decode.hip): the
// grouping comes out of its gate/up kernel; hE: em_h_bytes(E, f) of scratch
size_t em_h_bytes(int E, int f);
bool em_applies(int T, int k, int E, int d, int f, int format);
bool em_selects_topk(int T, int k, int E);
// topk_idx: the pairs' experts; or, with logits ([T][E] fp32) not null and
// em_selects_topk, the kernels take each token's choice from the logits and
// store the top-k to idx_out / w_out (topk_idx unused).
hipError_t launch_ffn_decode_em(const FfnArgs& a, const int32_t* topk_idx, int32_t* offsets,
                                int32_t* sorted_pair, int32_t* pair_pos, uint16_t* hE,
                                hipStream_t s, const float* logits = nullptr,
                                int32_t* idx_out = nullptr, float* w_out = nullptr);

// read-budget bit allocation (alloc.hip)
size_t bp_distortion_ws_bytes(int E, int d, int f);
hipError_t launch_bp_distortion(const uint8_t* gu_planes, const uint16_t* gu_scales,
                                const uint8_t* dn_planes, const uint16_t* dn_scales, int E,
                                int d, int f, double* dist, void* ws, hipStream_t s);
hipError_t launch_allocate_bits(const double* dist, const int32_t* counts, int E, int d, int f,
                                int bmin, int bmax, int64_t budget, uint8_t* bits,
                                double* lambda, int64_t* read, hipStream_t s);

// status code + message of the calling thread's last error (abi.cpp)
int set_error(int code, const char* fmt, ...);

// expert slot cache (cache.hip): need_cnt = [need[E] | cnt[E]] int32
hipError_t launch_cache_need(const int32_t* topk_idx, int P, int k, int E, int format,
                             int bits_mode, const uint8_t* bits, int32_t* need_cnt,
                             hipStream_t s);
// items [n][2] = (expert, slot); scale bytes per expert multiples of 16
hipError_t launch_cache_scale_gather(const int32_t* items, int n, const void* bank_gu,
                                     const void* bank_dn, void* slot_gu, void* slot_dn,
                                     size_t gu_bytes, size_t dn_bytes, hipStream_t s);
hipError_t launch_cache_remap(const int32_t* topk_idx, int P, int E, const int32_t* vmap,
                              int32_t* vidx, const uint8_t* bits_e, uint8_t* bits_v,
                              hipStream_t s);

hipError_t launch_combine(const float* y, const int32_t* pair_pos,
                          const float* topk_w, int T, int k, int d, void* out,
                          int out_f32, hipStream_t s);

// Canonical -> streaming code layouts (retile.hip).
hipError_t launch_retile_w4(const uint8_t* canon, long long R, int K, uint8_t* tiled,
                            hipStream_t s);
hipError_t launch_retile_bp(const uint8_t* canon, int E, int N, int K, uint8_t* tiled,
                            hipStream_t s);

}  // namespace moe
