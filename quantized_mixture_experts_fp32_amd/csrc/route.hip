// Router: fp32 logits in the fixed lane-group order, top-k by wavefront
// shuffles, renormalised softmax weights.
// ExactMoE ("Every Expert Counts ...", Abstract): the router stays BF16 and
// the top-k routing procedure is unchanged; the summation order below is the
// fixed order that makes the selected expert ids reproducible bit for bit.
#include <float.h>

#include "kcommon.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kTokPerBlock = 8;   // tokens sharing each router-row load
constexpr int kThreads = 256;     // 16 lane groups of 16
constexpr int kInvalid = 0x7FFFFFFF;

__device__ __forceinline__ bool better(float av, int ae, float bv, int be) {
  if (ae == kInvalid) return false;
  if (be == kInvalid) return true;
  return av > bv || (av == bv && ae < be);
}

// One block: kTokPerBlock tokens x all E experts.
// Phase 1: lane group G (16 lanes, lane l) evaluates experts G, G+16, ...;
//   lane l accumulates elements 128c + 8l + r (c ascending, r = 0..7) for
//   each of the block's tokens, then the xor-butterfly (8, 4, 2, 1) combines
//   the 16 partials; lane 0 adds the bias and stores the logit in LDS.
// Phase 2: wave w selects the top-k of tokens w and w+4 by k rounds of a
//   wave-wide (logit desc, index asc) arg-max; the weights are the softmax
//   over the k selected logits (equal to the renormalised full softmax).
__global__ __launch_bounds__(kThreads) void route_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int d, int E, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  extern __shared__ float lds[];
  float* logit_sh = lds;                            // [kTokPerBlock][E]

  const int tid = threadIdx.x;
  const int G = tid >> 4, l = tid & 15;
  const int t0 = blockIdx.x * kTokPerBlock;
  const int nchunk = d >> 7;

  const int n_iter = (E + 15) >> 4;  // uniform trip count for the shuffles
  for (int it = 0; it < n_iter; ++it) {
    const int e = G + 16 * it;
    const bool ok = e < E;
    const uint16_t* wrow = wr + (size_t)(ok ? e : 0) * d + 8 * l;
    float acc[kTokPerBlock];
#pragma unroll
    for (int tt = 0; tt < kTokPerBlock; ++tt) acc[tt] = 0.0f;
    for (int c = 0; c < nchunk; ++c) {
      const u32x4 wv = *(const u32x4*)(wrow + 128 * c);
      float wf[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wf[2 * q] = __uint_as_float(wv[q] << 16);
        wf[2 * q + 1] = __uint_as_float(wv[q] & 0xFFFF0000u);
      }
#pragma unroll
      for (int tt = 0; tt < kTokPerBlock; ++tt) {
        u32x4 xv = {0u, 0u, 0u, 0u};
        if (t0 + tt < T)
          xv = *(const u32x4*)(x + (size_t)(t0 + tt) * d + 128 * c + 8 * l);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // bf16 * bf16 is exact in fp32, so fma == multiply-then-add here
          acc[tt] = fmaf(__uint_as_float(xv[q] << 16), wf[2 * q], acc[tt]);
          acc[tt] = fmaf(__uint_as_float(xv[q] & 0xFFFF0000u), wf[2 * q + 1],
                         acc[tt]);
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < kTokPerBlock; ++tt) {
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) acc[tt] = acc[tt] + __shfl_xor(acc[tt], o, kWave);
    }
    if (ok && l == 0) {
      const float b = bias ? bias[e] : 0.0f;
#pragma unroll
      for (int tt = 0; tt < kTokPerBlock; ++tt) logit_sh[tt * E + e] = acc[tt] + b;
    }
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  for (int tt = wave; tt < kTokPerBlock; tt += kThreads / kWave) {
    const int t = t0 + tt;
    if (t >= T) break;
    const float* lg = logit_sh + tt * E;
    uint32_t taken = 0;
    float m = 0.0f, ssum = 0.0f, my_ex = 0.0f;
    for (int j = 0; j < k; ++j) {
      float bv = -FLT_MAX;
      int be = kInvalid;
      for (int i = 0; 64 * i + lane < E; ++i) {
        const int e = 64 * i + lane;
        if (!((taken >> i) & 1u) && better(lg[e], e, bv, be)) {
          bv = lg[e];
          be = e;
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oe = __shfl_xor(be, o, kWave);
        if (better(ov, oe, bv, be)) {
          bv = ov;
          be = oe;
        }
      }
      // every lane now holds the rank-(j+1) expert (bv, be)
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      if (j == 0) m = bv;
      const float ex = expf(bv - m);  // softmax over the selected logits
      ssum += ex;                      // rank order, identical in all lanes
      if (lane == j) {
        my_ex = ex;
        topk_idx[(size_t)t * k + j] = be;
      }
    }
    if (lane < k) topk_w[(size_t)t * k + lane] = my_ex / ssum;
  }
}

}  // namespace

hipError_t launch_route(const void* x, const void* wr, const float* bias,
                        int T, int d, int E, int k, int32_t* topk_idx,
                        float* topk_w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int blocks = (T + kTokPerBlock - 1) / kTokPerBlock;
  const size_t lds = sizeof(float) * (size_t)kTokPerBlock * E;
  hipLaunchKernelGGL(route_kernel, dim3(blocks), dim3(kThreads), lds, s,
                     (const uint16_t*)x, (const uint16_t*)wr, bias, T, d, E,
                     k, topk_idx, topk_w);
  return hipGetLastError();
}

}  // namespace moe
