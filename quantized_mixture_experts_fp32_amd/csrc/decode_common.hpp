// Helpers shared by the decode-path (small batch) expert FFN kernels:
// locating a work item's token tile from expert_offsets, staging routing
// and group scales in LDS.
#pragma once
#include "kcommon.hpp"

namespace moe {
namespace dec {

struct TileInfo {
  int e, r0, cnt;
};

// Tile b of the list "every expert's slot range cut into tiles of tok
// pairs, experts in ascending order".  Wave-cooperative (all lanes call it
// with the same b and get the same answer); returns false past the end.
__device__ inline bool find_tile(const int32_t* __restrict__ offsets, int E, int tok,
                          int b, TileInfo& t) {
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    const int lo = (e < E) ? offsets[e] : 0;
    const int n = (e < E) ? offsets[e + 1] - lo : 0;
    const int c = (n + tok - 1) / tok;
    int s = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(s, o, kWave);
      if (lane >= o) s += v;
    }
    const int total = __shfl(s, 63, kWave);
    if (b < carry + total) {
      const uint64_t m = __ballot(carry + s > b);
      const int L = __ffsll((unsigned long long)m) - 1;
      const int sL = __shfl(s, L, kWave), cL = __shfl(c, L, kWave);
      const int loL = __shfl(lo, L, kWave), nL = __shfl(n, L, kWave);
      const int chunk = b - (carry + sL - cL);
      t.e = base + L;
      t.r0 = loL + chunk * tok;
      t.cnt = min(tok, nL - chunk * tok);
      return true;
    }
    carry += total;
  }
  return false;
}

__device__ __forceinline__ bf16x8 bf16_splat(uint32_t bits16) {
  const uint32_t p = bits16 | (bits16 << 16);
  u32x4 r = {p, p, p, p};
  return __builtin_bit_cast(bf16x8, r);
}

// The kernels below stage expert_offsets and (when it fits) sorted_pair in
// LDS once per persistent block; a work item then needs one round trip to
// HBM: all of a wave's code, scale and activation loads are issued together.
constexpr int kPairsInLds = 4096;

// For 256-thread blocks.  Loads are issued four per thread at a time
// (indices clamped in range), then stored, so that staging takes one round
// trip per 1024 entries instead of one per 256.
__device__ __forceinline__ int stage_routing(const int32_t* __restrict__ offsets,
                                             const int32_t* __restrict__ sorted_pair,
                                             int E, int P, int32_t* off_lds,
                                             int32_t* sp_lds) {
  const int np = P <= kPairsInLds ? P : 0;
  constexpr int bd = 256;
  for (int i0 = threadIdx.x; i0 <= E || i0 < np; i0 += 4 * bd) {
    int32_t vo[4], vs[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * bd;
      vo[u] = offsets[i <= E ? i : E];
      vs[u] = np ? sorted_pair[i < np ? i : np - 1] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * bd;
      if (i <= E) off_lds[i] = vo[u];
      if (i < np) sp_lds[i] = vs[u];
    }
  }
  return np;
}




// Scales of 64 rows per matrix staged as fp32 in LDS, [matrix][group][row],
// for a 256-thread block: thread t owns row t % 64 (of matrix (t / 64) % NMAT)
// and every (256 / (64 NMAT))-th group.
template <int NMAT>
__device__ __forceinline__ void stage_scales_rows64(const uint16_t* __restrict__ rows_src,
                                                    size_t mat_stride, int G,
                                                    float* __restrict__ dst) {
  constexpr int kStep = 256 / (64 * NMAT);
  const int r = threadIdx.x & 63, m = (threadIdx.x >> 6) % NMAT, g0 = (threadIdx.x >> 6) / NMAT;
  const uint16_t* src = rows_src + ((size_t)m * mat_stride + r) * G;
  float* d = dst + (size_t)m * G * 64 + r;
  for (int g = g0; g < G; g += kStep) d[g * 64] = f16_bits_to_f32(src[g]);
}

// The same staging in two phases for G % 8 == 0 and 16-byte aligned scale
// rows: fetch() issues one 16-byte load (8 consecutive groups of one row)
// per chunk, kSC chunks per thread, before the code loads; store() converts
// and writes them to LDS after those loads are issued, so the scales share
// their round trip instead of queueing before it.  Chunk c covers row c % 64
// of matrix c / (64 G/8), groups 8 ((c / 64) % (G/8)) + 0..7; threads past
// the last chunk take chunk c mod total and store the same values to the same
// places as its owner (an unconditional store keeps the fetch where it is).
template <int NMAT, int kSC>
struct ScaleStage {
  u32x4 v[kSC];
  int c0;
  __device__ __forceinline__ void fetch(const uint16_t* __restrict__ rows_src,
                                        size_t mat_stride, int G) {
    const int cpr = G >> 3, total = NMAT * 64 * cpr;
    c0 = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kSC; ++i) {
      int c = c0 + 256 * i;
      c = c < total ? c : c % total;
      const int r = c & 63, m = (c >> 6) / cpr, cc = (c >> 6) % cpr;
      v[i] = *(const u32x4*)(rows_src + ((size_t)m * mat_stride + r) * G + 8 * cc);
    }
  }
  __device__ __forceinline__ void store(int G, float* __restrict__ dst) const {
    const int cpr = G >> 3, total = NMAT * 64 * cpr;
#pragma unroll
    for (int i = 0; i < kSC; ++i) {
      int c = c0 + 256 * i;
      c = c < total ? c : c % total;
      const int r = c & 63, m = (c >> 6) / cpr, cc = (c >> 6) % cpr;
      float* d = dst + ((size_t)m * G + 8 * cc) * 64 + r;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        d[(2 * q) * 64] = f16_bits_to_f32(v[i][q] & 0xFFFFu);
        d[(2 * q + 1) * 64] = f16_bits_to_f32(v[i][q] >> 16);
      }
    }
  }
};

// kSC for a staging of NMAT matrices x 64 rows x G groups (0: G % 8 != 0 or
// unaligned scales, use stage_scales_rows64).
inline int scale_chunks(int nmat, int G, const void* scales) {
  if (G % 8 || ((uintptr_t)scales & 15)) return 0;
  const int per = (nmat * 64 * (G / 8) + 255) / 256;
  return per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : 0;
}

constexpr int kXRow = 136;  // bf16 per staged activation row (128 + 8 pad)

}  // namespace dec
}  // namespace moe
