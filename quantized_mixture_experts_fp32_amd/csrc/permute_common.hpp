// Single-block grouping of token-expert pairs by expert, shared by the
// permute kernels and the fused small-batch router: a deterministic
// counting sort (histogram -> exclusive scan -> stable scatter).
#pragma once
#include "kcommon.hpp"

namespace moe {

// Histogram, exclusive scan and stable scatter of P <= kSmallP pairs by one
// 1024-thread block (idx may live in global memory or in LDS; sh is LDS of
// permute_block_lds_bytes(E)).  Same order as the multi-block path.
constexpr int kSmallP = 8192;

__host__ __device__ constexpr size_t permute_block_lds_bytes(int E) {
  return (size_t)(17 * E) * sizeof(int32_t);
}

__device__ inline void permute_block(const int32_t* idx, int P, int E,
                                     int32_t* __restrict__ offsets,
                                     int32_t* __restrict__ sorted_pair,
                                     int32_t* __restrict__ pair_pos, int32_t* sh) {
  int32_t* base = sh;               // [E]: counts, then next slot per expert
  int32_t* wave_cnt = sh + E;       // [16][E]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += 1024) {
    base[e] = 0;
    for (int w = 0; w < 16; ++w) wave_cnt[w * E + e] = 0;
  }
  __syncthreads();
  for (int p = tid; p < P; p += 1024) {
    const int e = idx[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&base[e], 1);
  }
  __syncthreads();
  // exclusive scan of the counts by one wave: lane l owns experts
  // l*per .. l*per + per - 1 (per = ceil(E / 64) <= 8)
  if (wave == 0) {
    const int per = (E + 63) >> 6;
    int c[8], sum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = lane * per + i;
      c[i] = (i < per && e < E) ? base[e] : 0;
      sum += c[i];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    int run = incl - sum;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = lane * per + i;
      if (i < per && e < E) {
        base[e] = run;
        offsets[e] = run;
        run += c[i];
      }
    }
    if (lane == 63) offsets[E] = incl;
  }
  __syncthreads();
  for (int r = 0; r < P; r += 1024) {
    const int p = r + tid;
    int e = (p < P) ? idx[p] : -1;
    if ((unsigned)e >= (unsigned)E) e = -1;
    const uint32_t key = (uint32_t)(e < 0 ? 0x3FF : e);
    uint64_t peers = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 10; ++bit) {
      const bool set = (key >> bit) & 1u;
      const uint64_t m = __ballot(set);
      peers &= set ? m : ~m;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(peers & below);
    if (e >= 0 && (peers & below) == 0) wave_cnt[wave * E + e] = __popcll(peers);
    __syncthreads();
    if (e >= 0) {
      int slot = base[e] + rank;
      for (int w = 0; w < wave; ++w) slot += wave_cnt[w * E + e];
      sorted_pair[slot] = p;
      pair_pos[p] = slot;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += 1024) {
      int add = 0;
      for (int w = 0; w < 16; ++w) {
        add += wave_cnt[w * E + ee];
        wave_cnt[w * E + ee] = 0;
      }
      base[ee] += add;
    }
    __syncthreads();
  }
}

// The same grouping of P <= 64 pairs by one wave (wave 0 of the block; no
// block barrier): LDS atomics count the pairs of each expert, the wave scans
// the counts (as above), and a pair's slot is its expert's start plus the
// number of lower lanes with the same expert (ballots over the expert id
// bits).  idx may live in global memory or in LDS; cnt is LDS of E ints.
__device__ inline void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline void permute_wave_small(const int32_t* idx, int P, int E,
                                          int32_t* __restrict__ offsets,
                                          int32_t* __restrict__ sorted_pair,
                                          int32_t* __restrict__ pair_pos, int32_t* cnt) {
  const int lane = threadIdx.x & 63;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  int e = lane < P ? idx[lane] : -1;
  if ((unsigned)e >= (unsigned)E) e = -1;
  wave_sync_lds();
  if (e >= 0) atomicAdd(&cnt[e], 1);
  wave_sync_lds();
  const int per = (E + 63) >> 6;
  int c[8], sum = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ee = lane * per + i;
    c[i] = (i < per && ee < E) ? cnt[ee] : 0;
    sum += c[i];
  }
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += v;
  }
  wave_sync_lds();  // every count is read before the starts overwrite them
  int run = incl - sum;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ee = lane * per + i;
    if (i < per && ee < E) {
      cnt[ee] = run;
      offsets[ee] = run;
      run += c[i];
    }
  }
  if (lane == 63) offsets[E] = incl;
  wave_sync_lds();
  const uint32_t key = (uint32_t)(e < 0 ? 0x3FF : e);
  uint64_t peers = ~0ull;
#pragma unroll
  for (int bit = 0; bit < 10; ++bit) {
    const bool set = (key >> bit) & 1u;
    const uint64_t m = __ballot(set);
    peers &= set ? m : ~m;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (e >= 0) {
    const int slot = cnt[e] + __popcll(peers & below);
    sorted_pair[slot] = lane;
    pair_pos[lane] = slot;
  }
}

}  // namespace moe
