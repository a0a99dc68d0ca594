// Grouping of the P = T*k token-expert pairs by expert: a deterministic
// counting sort (histogram -> exclusive scan -> stable scatter), the data
// structure behind ExactMoE's fused grouped execution ("Every Expert Counts
// ...", Abstract).  Integer-only, so the result is bit-exact by construction.
// Small batches use one single-block launch; large ones three kernels
// (per-chunk LDS histograms, one scan block, per-chunk stable scatter).
#include "kcommon.hpp"
#include "launch.hpp"
#include "permute_common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 1024;  // pairs per block (4 rounds of 256)

// counts[b][e]: number of pairs of expert e in chunk b (LDS histogram).
__global__ __launch_bounds__(kThreads) void perm_count(
    const int32_t* __restrict__ idx, int P, int E, int32_t* __restrict__ counts) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += kThreads) hist[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kChunk;
  for (int i = threadIdx.x; i < kChunk; i += kThreads) {
    const int p = base + i;
    if (p < P) {
      const int e = idx[p];
      if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads)
    counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// One block, one thread per expert (E <= 512 < 1024 threads):
// offsets[e] = exclusive scan of the totals; counts[b][e] is replaced in
// place by the first slot of chunk b's pairs of expert e.  Each thread
// reads its column kScanBatch chunks at a time (independent loads in
// flight instead of one dependent load per chunk).
constexpr int kScanBatch = 16;

__global__ __launch_bounds__(1024) void perm_scan(int nblocks, int E,
                                                  int32_t* __restrict__ counts,
                                                  int32_t* __restrict__ offsets) {
  __shared__ int32_t tot[1024];
  const int e = threadIdx.x;
  int32_t t = 0;
  if (e < E) {
    int b = 0;
    for (; b + kScanBatch <= nblocks; b += kScanBatch) {
      int32_t v[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) v[i] = counts[(size_t)(b + i) * E + e];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) t += v[i];
    }
    for (; b < nblocks; ++b) t += counts[(size_t)b * E + e];
  }
  tot[e] = (e < E) ? t : 0;
  __syncthreads();
  // Hillis-Steele inclusive scan over 1024 entries (integers: exact)
  for (int off = 1; off < 1024; off <<= 1) {
    int32_t v = (e >= off) ? tot[e - off] : 0;
    __syncthreads();
    tot[e] += v;
    __syncthreads();
  }
  if (e < E) {
    int32_t run = tot[e] - t;  // exclusive prefix
    offsets[e] = run;
    if (e == E - 1) offsets[E] = tot[e];
    int b = 0;
    for (; b + kScanBatch <= nblocks; b += kScanBatch) {
      int32_t v[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) v[i] = counts[(size_t)(b + i) * E + e];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) {
        counts[(size_t)(b + i) * E + e] = run;
        run += v[i];
      }
    }
    for (; b < nblocks; ++b) {
      const int32_t c = counts[(size_t)b * E + e];
      counts[(size_t)b * E + e] = run;
      run += c;
    }
  }
}

// Stable scatter: block b walks its chunk in rounds of 256 pairs.  Within a
// wave, the lanes holding the same expert are found with 9 ballots (one per
// bit of the expert id) and ranked by lane; waves are ordered through LDS
// per-wave counts; a per-expert running base carries across rounds.
__global__ __launch_bounds__(kThreads) void perm_scatter(
    const int32_t* __restrict__ idx, int P, int E,
    const int32_t* __restrict__ first_slot, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_pos) {
  extern __shared__ int32_t sh[];
  int32_t* base = sh;             // [E] next slot per expert
  int32_t* wave_cnt = sh + E;     // [4][E] pairs per wave in this pass
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += kThreads) {
    base[e] = first_slot[(size_t)blockIdx.x * E + e];
    for (int w = 0; w < 4; ++w) wave_cnt[w * E + e] = 0;
  }
  __syncthreads();
  const int chunk0 = blockIdx.x * kChunk;
  for (int r = 0; r < kChunk; r += kThreads) {
    const int p = chunk0 + r + tid;
    int e = (p < P) ? idx[p] : -1;
    if ((unsigned)e >= (unsigned)E) e = -1;  // skipped pair
    const uint32_t key = (uint32_t)(e < 0 ? 0x3FF : e);  // 10-bit key
    uint64_t peers = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 10; ++bit) {
      const bool set = (key >> bit) & 1u;
      const uint64_t m = __ballot(set);
      peers &= set ? m : ~m;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(peers & below);
    const bool leader = (peers & below) == 0;
    if (e >= 0 && leader) wave_cnt[wave * E + e] = __popcll(peers);
    __syncthreads();
    if (e >= 0) {
      int slot = base[e] + rank;
      for (int w = 0; w < wave; ++w) slot += wave_cnt[w * E + e];
      sorted_pair[slot] = p;
      pair_pos[p] = slot;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += kThreads) {
      int add = 0;
      for (int w = 0; w < 4; ++w) {
        add += wave_cnt[w * E + ee];
        wave_cnt[w * E + ee] = 0;
      }
      base[ee] += add;
    }
    __syncthreads();
  }
}

// Small batches (P <= kSmallP): one block, one launch (one wave for at most
// 64 pairs, else 1024 threads).
__global__ __launch_bounds__(1024) void perm_small(const int32_t* __restrict__ idx,
                                                   int P, int E,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ sorted_pair,
                                                   int32_t* __restrict__ pair_pos) {
  extern __shared__ int32_t sh[];
  if (P <= 64) {
    if (threadIdx.x < 64) permute_wave_small(idx, P, E, offsets, sorted_pair, pair_pos, sh);
  } else {
    permute_block(idx, P, E, offsets, sorted_pair, pair_pos, sh);
  }
}

}  // namespace

size_t permute_ws_bytes(int T, int k, int E) {
  const long long P = (long long)T * k;
  const long long nb = (P + kChunk - 1) / kChunk;
  return (size_t)((nb > 0 ? nb : 1) * E * sizeof(int32_t));
}

hipError_t launch_permute(const int32_t* topk_idx, int T, int k, int E,
                          int32_t* offsets, int32_t* sorted_pair,
                          int32_t* pair_pos, void* ws, hipStream_t s) {
  const int P = T * k;
  if (P <= kSmallP) {
    hipLaunchKernelGGL(perm_small, dim3(1), dim3(P <= 64 ? 64 : 1024),
                       permute_block_lds_bytes(E), s, topk_idx, P, E, offsets, sorted_pair,
                       pair_pos);
    return hipGetLastError();
  }
  const int nb = (P + kChunk - 1) / kChunk;
  int32_t* counts = (int32_t*)ws;
  if (nb > 0) {
    hipLaunchKernelGGL(perm_count, dim3(nb), dim3(kThreads),
                       E * sizeof(int32_t), s, topk_idx, P, E, counts);
  }
  hipLaunchKernelGGL(perm_scan, dim3(1), dim3(1024), 0, s, nb, E, counts,
                     offsets);
  if (nb > 0) {
    hipLaunchKernelGGL(perm_scatter, dim3(nb), dim3(kThreads),
                       5 * E * sizeof(int32_t), s, topk_idx, P, E, counts,
                       sorted_pair, pair_pos);
  }
  return hipGetLastError();
}

}  // namespace moe
