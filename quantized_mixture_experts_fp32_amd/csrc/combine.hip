// Combine: out[t] = sum over ranks j of topk_w[t][j] * y_pairs[pair_pos[t*k+j]]
// (fp32, rank order), stored as fp32 or as bf16 (round to nearest even).
// ExactMoE ("Every Expert Counts ...", Abstract): every selected expert
// contributes to the token's output.  HBM-bound: 16-byte loads and stores.
#include "kcommon.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;

// K > 0: top-k fixed at compile time (all K slots, weights and rows are
// loaded together: two round trips); K = 0: any k, one rank at a time.
template <bool kF32Out, int K>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const float* __restrict__ y, const int32_t* __restrict__ pair_pos,
    const float* __restrict__ topk_w, int k, int d, void* __restrict__ out) {
  const int nch = (d / 4 + kThreads - 1) / kThreads;
  const int t = blockIdx.x / nch;
  const int m = ((blockIdx.x % nch) * kThreads + threadIdx.x) * 4;
  if (m >= d) return;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  if (K > 0) {
    int64_t slot[K > 0 ? K : 1];
    float w[K > 0 ? K : 1];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      slot[j] = pair_pos[(int64_t)t * K + j];
      w[j] = topk_w[(int64_t)t * K + j];
    }
    f32x4 v[K > 0 ? K : 1];
#pragma unroll
    for (int j = 0; j < K; ++j) v[j] = *(const f32x4*)(y + slot[j] * d + m);
#pragma unroll
    for (int j = 0; j < K; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(w[j], v[j][q], acc[q]);
    }
  } else {
    for (int j = 0; j < k; ++j) {
      const int64_t slot = pair_pos[(int64_t)t * k + j];
      const float w = topk_w[(int64_t)t * k + j];
      const f32x4 v = *(const f32x4*)(y + slot * d + m);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(w, v[q], acc[q]);
    }
  }
  if (kF32Out) {
    *(f32x4*)((float*)out + (int64_t)t * d + m) = acc;
  } else {
    uint2 pk;
    pk.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
    pk.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
    *(uint2*)((uint16_t*)out + (int64_t)t * d + m) = pk;
  }
}

}  // namespace

hipError_t launch_combine(const float* y, const int32_t* pair_pos,
                          const float* topk_w, int T, int k, int d, void* out,
                          int out_f32, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)T * ((d / 4 + kThreads - 1) / kThreads));
  auto kern = out_f32 ? (k == 8 ? combine_kernel<true, 8> : combine_kernel<true, 0>)
                      : (k == 8 ? combine_kernel<false, 8> : combine_kernel<false, 0>);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s, y, pair_pos, topk_w, k, d, out);
  return hipGetLastError();
}

}  // namespace moe
