// Device side of the HBM expert slot cache: the per-step residency request
// (which experts the routed pairs touch, and the widest bitplane prefix each
// needs) and the renaming of routed experts to virtual ids whose weights sit
// in device slots.  ExactMoE ("Every Expert Counts ...", Abstract) keeps
// the expert bank in pinned host memory with a device cache; PagedMoE
// (abstract) fetches only the bitplanes a step is missing.
#include "kcommon.hpp"
#include "launch.hpp"

namespace moe {
namespace {

// need[e] = widest prefix (1..8) over the pairs routed to e (int4: 8), 0 when
// no pair is; cnt[e] = number of pairs of e.  One block, LDS tallies.
__global__ __launch_bounds__(1024) void cache_need_kernel(const int32_t* __restrict__ topk_idx,
                                                          int P, int k, int E, int format,
                                                          int bits_mode,
                                                          const uint8_t* __restrict__ bits,
                                                          int32_t* __restrict__ need_cnt) {
  extern __shared__ int32_t sh[];
  int32_t* need = sh;
  int32_t* cnt = sh + E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) need[e] = cnt[e] = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    const int e = topk_idx[p];
    if ((unsigned)e >= (unsigned)E) continue;
    const int b = format == 0 ? 8 : pair_bit_width(p, e, k, bits_mode, bits);
    atomicMax(&need[e], b);
    atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    need_cnt[e] = need[e];
    need_cnt[E + e] = cnt[e];
  }
}

// vidx[p] = vmap[topk_idx[p]]; with per-expert widths also bits_v[vmap[e]]
// = bits[e] for every routed expert (the FFN reads widths by virtual id).
__global__ __launch_bounds__(256) void cache_remap_kernel(const int32_t* __restrict__ topk_idx,
                                                          int P, int E,
                                                          const int32_t* __restrict__ vmap,
                                                          int32_t* __restrict__ vidx,
                                                          const uint8_t* __restrict__ bits_e,
                                                          uint8_t* __restrict__ bits_v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < P) {
    const int e = topk_idx[i];
    vidx[i] = (unsigned)e < (unsigned)E ? vmap[e] : -1;
  }
  if (bits_v && i < E) {
    const int v = vmap[i];
    if (v >= 0) bits_v[v] = bits_e[i];
  }
}

// Scales of experts new to their slots, from the device-resident scale
// bank: item i = (expert, slot); block (i, part) copies a 1/8 share of the
// expert's gate/up and down scales in 16-byte words.
__global__ __launch_bounds__(256) void cache_scale_gather_kernel(
    const int32_t* __restrict__ items, const uint4* __restrict__ bank_gu,
    const uint4* __restrict__ bank_dn, uint4* __restrict__ slot_gu, uint4* __restrict__ slot_dn,
    int gu_words, int dn_words) {
  const int e = items[2 * blockIdx.x], s = items[2 * blockIdx.x + 1];
  const int part = blockIdx.y, nparts = gridDim.y;
  for (int i = part * 256 + threadIdx.x; i < gu_words; i += nparts * 256)
    slot_gu[(size_t)s * gu_words + i] = bank_gu[(size_t)e * gu_words + i];
  for (int i = part * 256 + threadIdx.x; i < dn_words; i += nparts * 256)
    slot_dn[(size_t)s * dn_words + i] = bank_dn[(size_t)e * dn_words + i];
}

}  // namespace

hipError_t launch_cache_scale_gather(const int32_t* items, int n, const void* bank_gu,
                                     const void* bank_dn, void* slot_gu, void* slot_dn,
                                     size_t gu_bytes, size_t dn_bytes, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(cache_scale_gather_kernel, dim3(n, 8), dim3(256), 0, s, items,
                     (const uint4*)bank_gu, (const uint4*)bank_dn, (uint4*)slot_gu,
                     (uint4*)slot_dn, (int)(gu_bytes / 16), (int)(dn_bytes / 16));
  return hipGetLastError();
}

hipError_t launch_cache_need(const int32_t* topk_idx, int P, int k, int E, int format,
                             int bits_mode, const uint8_t* bits, int32_t* need_cnt,
                             hipStream_t s) {
  hipLaunchKernelGGL(cache_need_kernel, dim3(1), dim3(1024), 2 * E * sizeof(int32_t), s,
                     topk_idx, P, k, E, format, bits_mode, bits, need_cnt);
  return hipGetLastError();
}

hipError_t launch_cache_remap(const int32_t* topk_idx, int P, int E, const int32_t* vmap,
                              int32_t* vidx, const uint8_t* bits_e, uint8_t* bits_v,
                              hipStream_t s) {
  const int n = P > E ? P : E;
  hipLaunchKernelGGL(cache_remap_kernel, dim3((n + 255) / 256), dim3(256), 0, s, topk_idx, P,
                     E, vmap, vidx, bits_e, bits_v);
  return hipGetLastError();
}

}  // namespace moe
