// moe_layer_forward_wq_noalloc: the layer step for callers that cannot
// allocate device memory.  It runs the kernels of moe_layer_forward_wq,
// whose workspace here is a fixed array in device memory owned by the
// library instead of a caller buffer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/moe_wq.h"
#include "launch.hpp"

namespace {

// The scratch of every call on a GPU.  Each device that loads the library
// holds its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, looked up once per device with that device current,
// and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_lookup[kMaxDevices];

}  // namespace

extern "C" int moe_layer_forward_wq_noalloc(
    const void* x_bf16, const void* wr_bf16, const float* bias, int T, int d, int E, int k,
    int f, int format, int group_size, const uint8_t* gate_up_codes,
    const uint16_t* gate_up_scales_f16, const uint8_t* down_codes,
    const uint16_t* down_scales_f16, const uint8_t* bits, int bits_mode, int32_t* topk_idx,
    float* topk_w, int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_pos,
    float* y_pairs, void* out, int out_dtype, int path_hint, void* stream) {
  // size limit first: a step that does not fit touches no device state
  const size_t need = moe_layer_ws_bytes(T, k, E, d, f, format);
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return moe::set_error(MOE_ERR_WORKSPACE,
                          "moe_layer_forward_wq_noalloc: this step needs %zu bytes of "
                          "scratch, more than the fixed %d; use moe_layer_forward_wq "
                          "with a workspace",
                          need, MOE_NOALLOC_SCRATCH_BYTES);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return moe::set_error(MOE_ERR_HIP, "moe_layer_forward_wq_noalloc: hipGetDevice: %s",
                          hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return moe::set_error(MOE_ERR_UNSUPPORTED,
                          "moe_layer_forward_wq_noalloc: device %d beyond %d", dev,
                          kMaxDevices);
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_lookup[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = p;
  });
  if (g_lookup[dev] != hipSuccess || !g_scratch[dev])
    return moe::set_error(MOE_ERR_HIP,
                          "moe_layer_forward_wq_noalloc: scratch address on device %d: %s",
                          dev, hipGetErrorString(g_lookup[dev]));
  return moe_layer_forward_wq(x_bf16, wr_bf16, bias, T, d, E, k, f, format, group_size,
                              gate_up_codes, gate_up_scales_f16, down_codes, down_scales_f16,
                              bits, bits_mode, topk_idx, topk_w, expert_offsets, sorted_pair,
                              pair_pos, y_pairs, out, out_dtype, g_scratch[dev],
                              (size_t)MOE_NOALLOC_SCRATCH_BYTES, path_hint, stream);
}
