// Router: fp32 logits in the fixed lane-group order, top-k by wavefront
// ballots or arg-max rounds (route_common.hpp), renormalised softmax weights.
// ExactMoE ("Every Expert Counts ...", Abstract): the router stays BF16 and
// the top-k routing procedure is unchanged; the fixed summation order below
// makes the selected expert ids reproducible bit for bit:
//   partial l (0..15) of logit (t, e) adds x[t][i] * wr[e][i] for
//   i = 128c + 8l + r, c ascending, r = 0..7, from +0 in fp32; the partials
//   are combined with acc_l += acc_(l xor o) for o = 8, 4, 2, 1; the logit
//   is acc_0 + bias[e].  bf16 * bf16 products are exact in fp32, so fma and
//   multiply-then-add give the same sums.
// Three launch shapes share that order: for few tokens, (one or two tokens,
// 16 experts) blocks write logits to the workspace, and a second launch (or
// the decode FFN kernels themselves) selects the top-k (many blocks even for
// one token); one 1024-thread block per token with the top-k fused
// (moe_route at up to 16 tokens); for many tokens, eight tokens per
// 256-thread block, four experts per lane group at a time, with the top-k
// fused.  Activation rows are staged in LDS; router rows are streamed with
// several outstanding 16-byte loads per lane.
#include <float.h>

#include "kcommon.hpp"
#include "launch.hpp"
#include "permute_common.hpp"
#include "route_common.hpp"

namespace moe {
namespace {

constexpr int kInvalid = 0x7FFFFFFF;
constexpr int kWindow = 16;  // router-row chunks in flight per lane

__device__ __forceinline__ bool better(float av, int ae, float bv, int be) {
  if (ae == kInvalid) return false;
  if (be == kInvalid) return true;
  return av > bv || (av == bv && ae < be);
}

__device__ __forceinline__ float lo_bf16(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t v) {
  return __uint_as_float(v & 0xFFFF0000u);
}

// Top-k of one token from its E logits in LDS, by one wave: k rounds of a
// wave-wide (logit desc, index asc) arg-max; weights = softmax over the k
// selected logits (equal to the renormalised full softmax).
__device__ void select_topk(const float* __restrict__ lg, int E, int k,
                            int32_t* __restrict__ idx_out,
                            float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
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
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (j == 0) m = bv;
    const float ex = expf(bv - m);
    ssum += ex;  // rank order, identical in every lane
    if (lane == j) {
      my_ex = ex;
      idx_out[j] = be;
    }
  }
  if (lane < k) w_out[lane] = my_ex / ssum;
}

// The same selection for E <= 64 (one logit per lane) by ballots instead of
// k arg-max rounds (select_topk_radix64), from the token's logits in memory.
__device__ __forceinline__ void select_topk_64(const float* __restrict__ lg, int E, int k,
                                               int32_t* __restrict__ idx_out,
                                               float* __restrict__ w_out,
                                               int32_t* __restrict__ idx_copy) {
  const int lane = threadIdx.x & 63;
  select_topk_radix64(lane < E ? lg[lane] : 0.0f, E, k, idx_out, w_out, idx_copy);
}

// Stage TB activation rows (bf16) into LDS; rows past T are zero.
template <int TB, int NTHR>
__device__ __forceinline__ void stage_x(const uint16_t* __restrict__ x, int T,
                                        int d, int t0, uint16_t* xs) {
  const int n16 = TB * d / 8;  // 16-byte units
  for (int i = threadIdx.x; i < n16; i += NTHR) {
    const int tt = (8 * i) / d, c = 8 * i - tt * d;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (t0 + tt < T) v = *(const u32x4*)(x + (size_t)(t0 + tt) * d + c);
    *(u32x4*)(xs + tt * d + c) = v;
  }
}

// Logits of TB tokens (rows of xs) for the experts of this lane group; the
// group's 16 lanes are lanes 16*(tid/16) .. +15 of one wave.  Router-row
// chunks are loaded kWindow at a time; load_window fills one window and
// group_logits_from consumes a first window already loaded.
__device__ __forceinline__ void load_window(const uint16_t* __restrict__ wrow, bool ok,
                                            int nchunk, int c0, u32x4 (&wv)[kWindow]) {
  const int l = threadIdx.x & 15;
#pragma unroll
  for (int q = 0; q < kWindow; ++q)
    wv[q] = (ok && c0 + q < nchunk) ? *(const u32x4*)(wrow + 128 * (c0 + q) + 8 * l)
                                    : u32x4{0u, 0u, 0u, 0u};
}

template <int TB>
__device__ __forceinline__ void group_logits_from(const uint16_t* xs, int d,
                                                  const uint16_t* __restrict__ wrow, bool ok,
                                                  u32x4 (&wv)[kWindow], float acc[TB]) {
  const int l = threadIdx.x & 15;
  const int nchunk = d >> 7;
#pragma unroll
  for (int tt = 0; tt < TB; ++tt) acc[tt] = 0.0f;
  for (int c0 = 0; c0 < nchunk; c0 += kWindow) {
    if (c0 > 0) load_window(wrow, ok, nchunk, c0, wv);
#pragma unroll
    for (int q = 0; q < kWindow; ++q) {
      if (c0 + q >= nchunk) break;
      const int off = 128 * (c0 + q) + 8 * l;
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) {
        const u32x4 xv = *(const u32x4*)(xs + tt * d + off);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          acc[tt] = fmaf(lo_bf16(xv[p]), lo_bf16(wv[q][p]), acc[tt]);
          acc[tt] = fmaf(hi_bf16(xv[p]), hi_bf16(wv[q][p]), acc[tt]);
        }
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < TB; ++tt) {
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) acc[tt] = acc[tt] + __shfl_xor(acc[tt], o, kWave);
  }
}

template <int TB>
__device__ __forceinline__ void group_logits(const uint16_t* xs, int d,
                                             const uint16_t* __restrict__ wrow,
                                             bool ok, float acc[TB]) {
  u32x4 wv[kWindow];
  load_window(wrow, ok, d >> 7, 0, wv);
  group_logits_from<TB>(xs, d, wrow, ok, wv, acc);
}

// The same logits for NE experts per lane group at once: every activation
// chunk read from LDS is unpacked once and used for the NE experts, and
// every router chunk once for the TB tokens (per (token, expert) the
// summation order is the one above).  W router chunks per expert are in
// flight; a slot is refilled right after it is unpacked.  Loads past the
// row's end, and rows of experts past E (given as any valid row), read
// valid addresses and feed only unstored logits.
template <int NE, int W>
__device__ __forceinline__ void logits_prefetch(const uint16_t* const (&wrow)[NE], int nchunk,
                                                u32x4 (&wv)[W][NE]) {
  const int l = threadIdx.x & 15;
#pragma unroll
  for (int q = 0; q < W; ++q) {
    const int c = q < nchunk ? q : nchunk - 1;
#pragma unroll
    for (int j = 0; j < NE; ++j) wv[q][j] = *(const u32x4*)(wrow[j] + 128 * c + 8 * l);
  }
}

template <int TB, int NE, int W>
__device__ __forceinline__ void group_logits_ne(const uint16_t* xs, int d,
                                                const uint16_t* const (&wrow)[NE],
                                                u32x4 (&wv)[W][NE], float (&acc)[TB][NE]) {
  const int l = threadIdx.x & 15;
  const int nchunk = d >> 7;
#pragma unroll
  for (int tt = 0; tt < TB; ++tt)
#pragma unroll
    for (int j = 0; j < NE; ++j) acc[tt][j] = 0.0f;
  for (int c0 = 0; c0 < nchunk; c0 += W) {
#pragma unroll
    for (int q = 0; q < W; ++q) {
      const int c = c0 + q;
      if (c >= nchunk) break;
      float wf[NE][8];
#pragma unroll
      for (int j = 0; j < NE; ++j)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          wf[j][2 * p] = lo_bf16(wv[q][j][p]);
          wf[j][2 * p + 1] = hi_bf16(wv[q][j][p]);
        }
      {
        const int cn = c + W < nchunk ? c + W : nchunk - 1;
#pragma unroll
        for (int j = 0; j < NE; ++j) wv[q][j] = *(const u32x4*)(wrow[j] + 128 * cn + 8 * l);
      }
      const int off = 128 * c + 8 * l;
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) {
        const u32x4 xv = *(const u32x4*)(xs + tt * d + off);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float x0 = lo_bf16(xv[p]), x1 = hi_bf16(xv[p]);
#pragma unroll
          for (int j = 0; j < NE; ++j) {
            acc[tt][j] = fmaf(x0, wf[j][2 * p], acc[tt][j]);
            acc[tt][j] = fmaf(x1, wf[j][2 * p + 1], acc[tt][j]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < TB; ++tt)
#pragma unroll
    for (int j = 0; j < NE; ++j)
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) acc[tt][j] = acc[tt][j] + __shfl_xor(acc[tt][j], o, kWave);
}

// Many tokens: 8 per 256-thread block, 16 lane groups over the experts, four
// experts per lane group at a time.
constexpr int kTbNE = 4;

__global__ __launch_bounds__(256) void route_tb8(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int d, int E, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  constexpr int TB = 8;
  extern __shared__ float lds[];
  float* logit_sh = lds;                               // [TB][E]
  uint16_t* xs = (uint16_t*)(lds + TB * E);            // [TB][d]
  const int t0 = blockIdx.x * TB;
  stage_x<TB, 256>(x, T, d, t0, xs);
  __syncthreads();
  const int G = threadIdx.x >> 4, l = threadIdx.x & 15;
  constexpr int NE = kTbNE;
  const int n_iter = (E + 16 * NE - 1) / (16 * NE);  // uniform trip count (shuffles inside)
  for (int it = 0; it < n_iter; ++it) {
    int e[NE];
    const uint16_t* wrow[NE];
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      e[j] = G + 16 * (j + NE * it);
      wrow[j] = wr + (size_t)(e[j] < E ? e[j] : 0) * d;
    }
    u32x4 wv[4][NE];
    logits_prefetch<NE, 4>(wrow, d >> 7, wv);
    float acc[TB][NE];
    group_logits_ne<TB, NE, 4>(xs, d, wrow, wv, acc);
    if (l == 0) {
#pragma unroll
      for (int j = 0; j < NE; ++j) {
        if (e[j] >= E) continue;
        const float b = bias ? bias[e[j]] : 0.0f;
#pragma unroll
        for (int tt = 0; tt < TB; ++tt) logit_sh[tt * E + e[j]] = acc[tt][j] + b;
      }
    }
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6;
  for (int tt = wave; tt < TB; tt += 4) {
    const int t = t0 + tt;
    if (t >= T) break;
    select_topk(logit_sh + tt * E, E, k, topk_idx + (size_t)t * k,
                topk_w + (size_t)t * k);
  }
}

// Few tokens: block (token, 16 experts) with one lane group per expert
// writes fp32 logits to the workspace; a second launch selects the top-k.
constexpr int kSmallT = 512;

__global__ __launch_bounds__(256) void route_logits_small(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int d, int E,
    float* __restrict__ logits) {
  extern __shared__ uint16_t xs[];  // [d]
  const int neb = (E + 15) >> 4;
  const int t = blockIdx.x / neb, eb = blockIdx.x % neb;
  const int G = threadIdx.x >> 4, l = threadIdx.x & 15;
  const int e = 16 * eb + G;
  const bool ok = e < E;
  const uint16_t* wrow = wr + (size_t)(ok ? e : 0) * d;
  // the router row's first window is requested before the activation row,
  // so the two loads share one memory round trip
  u32x4 wv[kWindow];
  load_window(wrow, ok, d >> 7, 0, wv);
  stage_x<1, 256>(x, T, d, t, xs);
  __syncthreads();
  float acc[1];
  group_logits_from<1>(xs, d, wrow, ok, wv, acc);
  if (ok && l == 0) logits[(size_t)t * E + e] = acc[0] + (bias ? bias[e] : 0.0f);
}

// Few tokens, more than one per block: block (TB tokens, 16 experts), one
// lane group per expert; each router chunk serves the TB tokens, so the
// router rows are read T / TB times instead of T times.
template <int TB, int W>
__global__ __launch_bounds__(256) void route_logits_tile(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int d, int E, float* __restrict__ logits) {
  extern __shared__ uint16_t xs[];  // [TB][d]
  const int neb = (E + 15) >> 4;
  const int t0 = (blockIdx.x / neb) * TB, eb = blockIdx.x % neb;
  const int G = threadIdx.x >> 4, l = threadIdx.x & 15;
  const int e = 16 * eb + G;
  const bool ok = e < E;
  const uint16_t* wrow[1] = {wr + (size_t)(ok ? e : 0) * d};
  // the router rows' first chunks are requested before the activation rows
  u32x4 wv[W][1];
  logits_prefetch<1, W>(wrow, d >> 7, wv);
  stage_x<TB, 256>(x, T, d, t0, xs);
  __syncthreads();
  float acc[TB][1];
  group_logits_ne<TB, 1, W>(xs, d, wrow, wv, acc);
  if (ok && l == 0) {
    const float b = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int tt = 0; tt < TB; ++tt)
      if (t0 + tt < T) logits[(size_t)(t0 + tt) * E + e] = acc[tt][0] + b;
  }
}

__global__ __launch_bounds__(256) void route_topk(const float* __restrict__ logits,
                                                  int T, int E, int k,
                                                  int32_t* __restrict__ topk_idx,
                                                  float* __restrict__ topk_w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  if (E <= 64)
    select_topk_64(logits + (size_t)t * E, E, k, topk_idx + (size_t)t * k,
                   topk_w + (size_t)t * k, topk_idx + (size_t)t * k);
  else
    select_topk_reg(logits + (size_t)t * E, E, k, topk_idx + (size_t)t * k,
                    topk_w + (size_t)t * k, topk_idx + (size_t)t * k);
}

// Very few tokens: one 1024-thread block per token computes all E logits
// (64 lane groups, one expert each per pass, same order as above) into LDS
// and selects the token's top-k there: one launch, no logits round trip.
constexpr int kTokenBlockT = 16;

__global__ __launch_bounds__(1024) void route_token_block(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int d, int E, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  extern __shared__ float lds[];
  float* lg = lds;                                  // [E]
  uint16_t* xs = (uint16_t*)(lds + ((E + 3) & ~3));  // [d]
  const int t = blockIdx.x;
  stage_x<1, 1024>(x, T, d, t, xs);
  __syncthreads();
  const int G = threadIdx.x >> 4, l = threadIdx.x & 15;
  for (int e0 = 0; e0 < E; e0 += 64) {  // uniform trip count (shuffles inside)
    const int e = e0 + G;
    const bool ok = e < E;
    float acc[1];
    group_logits<1>(xs, d, wr + (size_t)(ok ? e : 0) * d, ok, acc);
    if (ok && l == 0) lg[e] = acc[0] + (bias ? bias[e] : 0.0f);
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    if (E <= 64)
      select_topk_64(lg, E, k, topk_idx + (size_t)t * k, topk_w + (size_t)t * k,
                     topk_idx + (size_t)t * k);
    else
      select_topk_reg(lg, E, k, topk_idx + (size_t)t * k, topk_w + (size_t)t * k,
                      topk_idx + (size_t)t * k);
  }
}

// Few tokens: top-k of every token (one wave per token) and the grouping of
// the T*k pairs by expert, in one block: 1024 threads, or for at most 64
// pairs one wave per token (at most 16) with the grouping by wave 0 alone.
__global__ __launch_bounds__(1024) void route_topk_permute(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos) {
  extern __shared__ int32_t sh[];
  const int P = T * k;
  const int nw = blockDim.x >> 6;
  int32_t* idx_lds = sh;
  for (int t = threadIdx.x >> 6; t < T; t += nw) {
    if (E <= 64)
      select_topk_64(logits + (size_t)t * E, E, k, topk_idx + (size_t)t * k,
                     topk_w + (size_t)t * k, idx_lds + t * k);
    else
      select_topk_reg(logits + (size_t)t * E, E, k, topk_idx + (size_t)t * k,
                      topk_w + (size_t)t * k, idx_lds + t * k);
  }
  __syncthreads();
  if (P <= 64) {
    if (threadIdx.x < 64)
      permute_wave_small(idx_lds, P, E, offsets, sorted_pair, pair_pos, sh + ((P + 3) & ~3));
  } else {
    permute_block(idx_lds, P, E, offsets, sorted_pair, pair_pos, sh + ((P + 3) & ~3));
  }
}

}  // namespace

// fp32 logits [T][E] of up to kSmallT tokens into `logits`: two tokens per
// block when that still gives at least 256 (token pair, 16-expert) blocks,
// else one (measured at E = 256: T = 64, 200 and 512 route in 15.1, 24.9 and
// 42.7 us with two tokens per block, 16.7, 31.0 and 58.9 with one; four or
// eight tokens per block were slower than one).
static void launch_logits_small(const void* x, const void* wr, const float* bias, int T, int d,
                                int E, float* logits, hipStream_t s) {
  const int neb = (E + 15) / 16;
  const int tb = ((T + 1) / 2) * neb >= 256 ? 2 : 1;
  const uint16_t* xp = (const uint16_t*)x;
  const uint16_t* wp = (const uint16_t*)wr;
  const size_t lds = sizeof(uint16_t) * (size_t)tb * d;
  const dim3 grid(((T + tb - 1) / tb) * neb), blk(256);
  if (tb == 2)
    hipLaunchKernelGGL((route_logits_tile<2, 8>), grid, blk, lds, s, xp, wp, bias, T, d, E, logits);
  else
    hipLaunchKernelGGL(route_logits_small, grid, blk, lds, s, xp, wp, bias, T, d, E, logits);
}

// fp32 logits [T][E] only (T <= kSmallT), for a consumer that selects the
// top-k itself.
hipError_t launch_route_logits(const void* x, const void* wr, const float* bias, int T, int d,
                               int E, float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T > kSmallT) return hipErrorInvalidValue;
  launch_logits_small(x, wr, bias, T, d, E, logits, s);
  return hipGetLastError();
}

size_t route_ws_bytes(int T, int E) {
  return T <= kSmallT ? sizeof(float) * (size_t)T * E : 0;
}

hipError_t launch_route(const void* x, const void* wr, const float* bias,
                        int T, int d, int E, int k, int32_t* topk_idx,
                        float* topk_w, void* ws, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T <= kTokenBlockT) {
    const size_t lds = sizeof(float) * ((E + 3) & ~3) + sizeof(uint16_t) * d;
    hipLaunchKernelGGL(route_token_block, dim3(T), dim3(1024), lds, s, (const uint16_t*)x,
                       (const uint16_t*)wr, bias, T, d, E, k, topk_idx, topk_w);
  } else if (T <= kSmallT) {
    float* logits = (float*)ws;
    launch_logits_small(x, wr, bias, T, d, E, logits, s);
    hipLaunchKernelGGL(route_topk, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k,
                       topk_idx, topk_w);
  } else {
    const size_t lds = sizeof(float) * 8 * E + sizeof(uint16_t) * 8 * d;
    hipLaunchKernelGGL(route_tb8, dim3((T + 7) / 8), dim3(256), lds, s,
                       (const uint16_t*)x, (const uint16_t*)wr, bias, T, d, E, k,
                       topk_idx, topk_w);
  }
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

size_t route_permute_ws_bytes(int T, int k, int E) {
  const size_t a = route_ws_bytes(T, E), b = permute_ws_bytes(T, k, E);
  return a > b ? a : b;
}

hipError_t launch_route_permute(const void* x, const void* wr, const float* bias, int T,
                                int d, int E, int k, int32_t* topk_idx, float* topk_w,
                                int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                                void* ws, hipStream_t s) {
  // One block selecting every token's top-k and grouping the pairs saves a
  // launch, but its sequential selections cost more than the launch past 64
  // pairs with more than 64 experts (measured at E = 256, T = 64: 31 us
  // against 6.9 us for one wave per token over 16 blocks plus 3.8 us for a
  // separate one-block grouping) and past 16 tokens with 64 experts (route
  // and permute at E = 64, T = 32 / 64 / 128 / 512: 11.0 / 12.3 / 13.2 /
  // 23.1 us separately, 14.4 / 21.6 / 35.4 / 118.6 us in one block); those
  // shapes route, then permute.
  const int P = T * k;
  if (T > 0 && T <= kSmallT && (P <= 64 || (E <= 64 && T <= 16))) {
    float* logits = (float*)ws;
    launch_logits_small(x, wr, bias, T, d, E, logits, s);
    const size_t lds = sizeof(int32_t) * ((P + 3) & ~3) + permute_block_lds_bytes(E);
    const int threads = P <= 64 ? 64 * (T < 16 ? T : 16) : 1024;
    hipLaunchKernelGGL(route_topk_permute, dim3(1), dim3(threads), lds, s, logits, T, E, k,
                       topk_idx, topk_w, offsets, sorted_pair, pair_pos);
    return hipGetLastError();
  }
  hipError_t e = launch_route(x, wr, bias, T, d, E, k, topk_idx, topk_w, ws, s);
  if (e != hipSuccess) return e;
  return launch_permute(topk_idx, T, k, E, offsets, sorted_pair, pair_pos, ws, s);
}

}  // namespace moe
