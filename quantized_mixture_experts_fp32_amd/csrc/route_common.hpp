// Top-k selection of one token by one wave, shared by the routing kernels and
// the decode gate/up kernels that route a few tokens themselves from the
// logits (the expert-major one ranks its own expert per token; the K-split
// one selects the whole batch).
// ExactMoE ("Every Expert Counts ...", Abstract): the top-k routing procedure
// is unchanged; experts are ranked by logit, larger first, equal logits to
// the lower index, and the k weights are the softmax over the selected
// logits (equal to the renormalised full softmax).
#pragma once

#include "kcommon.hpp"

namespace moe {

// Order-preserving unsigned image of an fp32 value (-0 orders as +0).
__device__ __forceinline__ uint32_t ordered_f32(float f) {
  const uint32_t u = (f == 0.0f) ? 0u : __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unordered_f32(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Rank of expert e among the token's E <= 64 logits (lane l < E holds logit
// l; e uniform): the number of keys above e's key (order-preserving logit
// bits ol, then the lower index first).  e is among the top k when it is
// below k, and then it is e's position in the token's rank order.
__device__ __forceinline__ int expert_rank64(float logit, int E, int e) {
  const int lane = threadIdx.x & 63;
  const uint32_t ol = ordered_f32(logit);
  const uint32_t oe = (uint32_t)__builtin_amdgcn_readlane((int)ol, e);
  return __popcll(__ballot(lane < E && (ol > oe || (ol == oe && lane < e))));
}

// E <= 64, k <= E: lane l < E holds logit l of the token; one wave selects
// its top-k with ballots and lane reads, no LDS.  Keys are distinct (ol,
// then the lower index first).  A bitwise search for the largest v with
// #{ol >= v} >= k gives the k-th largest ol; lanes above it are selected,
// and among lanes equal to it the lowest indices fill the remaining places.
// A selected lane's rank counts the selected keys above its own.  Weights:
// m is the rank-0 logit, ex = exp(logit - m), and the ex are summed in rank
// order from 0 (the same fp32 steps as the arg-max selection).  Returns
// whether this lane is selected, with its rank and weight.
__device__ __forceinline__ bool topk_radix64(float logit, int E, int k, int& rank, float& w) {
  const int lane = threadIdx.x & 63;
  const bool ok = lane < E;
  const uint32_t ol = ordered_f32(logit);
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    if (__popcll(__ballot(ok && ol >= cand)) >= k) thr = cand;
  }
  const uint64_t above = __ballot(ok && ol > thr), tied = __ballot(ok && ol == thr);
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const bool sel = ok && (ol > thr || (ol == thr && __popcll(tied & lt) < k - __popcll(above)));
  rank = 0;
  for (uint64_t m = __ballot(sel); m; m &= m - 1) {
    const int j = __ffsll((unsigned long long)m) - 1;
    const uint32_t oj = (uint32_t)__builtin_amdgcn_readlane((int)ol, j);
    rank += (oj > ol || (oj == ol && j < lane)) ? 1 : 0;
  }
  const float v = unordered_f32(ol);
  const int top = __ffsll((unsigned long long)__ballot(sel && rank == 0)) - 1;
  const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), top));
  const float ex = expf(v - m);
  float ssum = 0.0f;
  for (int r = 0; r < k; ++r) {  // rank order
    const int jr = __ffsll((unsigned long long)__ballot(sel && rank == r)) - 1;
    ssum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), jr));
  }
  w = ex / ssum;
  return sel;
}

// The same, storing idx_out[r], w_out[r] and idx_copy[r] (each when not
// null) for r < k.
__device__ __forceinline__ void select_topk_radix64(float logit, int E, int k,
                                                    int32_t* __restrict__ idx_out,
                                                    float* __restrict__ w_out,
                                                    int32_t* __restrict__ idx_copy) {
  const int lane = threadIdx.x & 63;
  int rank;
  float w;
  if (topk_radix64(logit, E, k, rank, w)) {
    if (idx_copy) idx_copy[rank] = lane;
    if (idx_out) idx_out[rank] = lane;
    if (w_out) w_out[rank] = w;
  }
}

// E <= 512: the token's logits from memory into registers (up to 8 per
// lane), each as a 64-bit key (order-preserving logit bits, inverted index):
// the largest key is the largest logit, ties to the lower index.  k rounds
// of a wave-wide arg-max, with the same weights as above.  The wave arg-max of each round is four DPP steps within rows of
// 16 lanes and four readlanes.  Stores idx_out[j], w_out[j] and idx_copy[j]
// (each when not null) for j < k.
template <int kCtrl>
__device__ __forceinline__ uint64_t dpp_max(uint64_t v) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, kCtrl, 0xF, 0xF, false);
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, kCtrl, 0xF, 0xF, false);
  const uint64_t o = ((uint64_t)ohi << 32) | olo;
  return o > v ? o : v;
}

__device__ __forceinline__ uint64_t wave_max_key(uint64_t v) {
  v = dpp_max<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_max<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_max<0x141>(v);  // row_half_mirror
  v = dpp_max<0x140>(v);  // row_mirror: every lane holds its row's maximum
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  uint64_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint64_t k = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, 16 * r) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)lo, 16 * r);
    m = k > m ? k : m;
  }
  return m;
}

__device__ inline void select_topk_reg(const float* __restrict__ lg, int E, int k,
                                int32_t* __restrict__ idx_out, float* __restrict__ w_out,
                                int32_t* __restrict__ idx_copy) {
  const int lane = threadIdx.x & 63;
  uint64_t key[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int e = 64 * i + lane;
    key[i] = (e < E) ? (((uint64_t)ordered_f32(lg[e]) << 32) | (uint32_t)~(uint32_t)e) : 0ull;
  }
  float m = 0.0f, ssum = 0.0f, my_ex = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t loc = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) loc = key[i] > loc ? key[i] : loc;
    const uint64_t win = wave_max_key(loc);
    const int be = (int)~(uint32_t)win;
    const float bv = unordered_f32((uint32_t)(win >> 32));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (64 * i + lane == be) key[i] = 0;
    if (j == 0) m = bv;
    const float ex = expf(bv - m);
    ssum += ex;  // rank order, identical in every lane
    if (lane == j) {
      my_ex = ex;
      if (idx_out) idx_out[j] = be;
      if (idx_copy) idx_copy[j] = be;
    }
  }
  if (lane < k && w_out) w_out[lane] = my_ex / ssum;
}

}  // namespace moe
