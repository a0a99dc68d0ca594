// GPU side of the synthetic-input generator (see synth_gen.h): the same
// element-wise definitions, evaluated by a grid-stride kernel straight into
// device memory, so multi-GB weight sets never pass through the host.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "synth_gen.h"

namespace {

__global__ void fill_bf16_k(uint64_t key, uint64_t start, uint64_t n,
                            double sigma, uint16_t* out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += stride)
    out[i] = synth_f32_to_bf16(synth_normal_f32(key, start + i, sigma));
}

__global__ void fill_f32_k(uint64_t key, uint64_t start, uint64_t n,
                           double sigma, float* out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += stride)
    out[i] = synth_normal_f32(key, start + i, sigma);
}

__global__ void fill_weight_k(uint64_t key, uint64_t mkey, uint64_t start,
                              uint64_t n, double sigma, float* out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += stride)
    out[i] = synth_weight_f32(key, mkey, start + i, sigma);
}

unsigned grid_for(uint64_t n) {
  uint64_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  if (b == 0) b = 1;
  return (unsigned)b;
}

}  // namespace

extern "C" {

int synth_dev_fill_bf16(uint64_t seed, uint64_t cfg, uint64_t tensor,
                        uint64_t step, uint64_t start, uint64_t n,
                        double sigma, void* out, void* stream) {
  if (n == 0) return 0;
  uint64_t key = synth_key(seed, cfg, tensor, step);
  hipLaunchKernelGGL(fill_bf16_k, dim3(grid_for(n)), dim3(256), 0,
                     (hipStream_t)stream, key, start, n, sigma,
                     (uint16_t*)out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

int synth_dev_fill_f32(uint64_t seed, uint64_t cfg, uint64_t tensor,
                       uint64_t step, uint64_t start, uint64_t n, double sigma,
                       void* out, void* stream) {
  if (n == 0) return 0;
  uint64_t key = synth_key(seed, cfg, tensor, step);
  hipLaunchKernelGGL(fill_f32_k, dim3(grid_for(n)), dim3(256), 0,
                     (hipStream_t)stream, key, start, n, sigma, (float*)out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

int synth_dev_fill_weight_f32(uint64_t seed, uint64_t cfg, uint64_t tensor,
                              uint64_t start, uint64_t n, double sigma,
                              void* out, void* stream) {
  if (n == 0) return 0;
  uint64_t key = synth_key(seed, cfg, tensor, 0);
  uint64_t mkey = synth_key(seed, cfg, tensor + SYNTH_MASK_OFFSET, 0);
  hipLaunchKernelGGL(fill_weight_k, dim3(grid_for(n)), dim3(256), 0,
                     (hipStream_t)stream, key, mkey, start, n, sigma,
                     (float*)out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
