// Conversion of expert codes from the canonical row-major layouts into the
// streaming layouts the FFN kernels read (a pure rearrangement of bits).
//  int4 (ExactMoE, Abstract: symmetric group-128 4-bit codes, two per
//    byte): canonical byte (r, j) holds element 2j in its low nibble and
//    2j + 1 in its high nibble.  Streaming: 16-row tiles [R/16][K/128][16]
//    [64] bytes; 32-bit word j of a row's group holds elements 8j .. 8j + 7,
//    element 8j + 2i in nibble i and 8j + 2i + 1 in nibble 4 + i.
//  bitplane8 (PagedMoE, abstract: one 8-bit code per weight stored as
//    bitplanes whose lower precisions are prefixes): canonical per expert 8
//    plane slabs [8][N][K/8], slab p holding bit 7 - p, bit i of byte (n, j)
//    for element 8j + i.  Streaming: [N/16][K/128][8][16][16] bytes per
//    expert, the same bytes regrouped per 16-row tile and 128-group.
#include "kcommon.hpp"
#include "launch.hpp"

namespace moe {
namespace {

// One thread per output 32-bit word (8 elements of one row).
__global__ __launch_bounds__(256) void retile_w4_kernel(const uint32_t* __restrict__ canon,
                                                        long long R, int K,
                                                        uint32_t* __restrict__ tiled) {
  const long long wpr = K / 8;  // words per row
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= R * wpr) return;
  // tiled word i: tile t, group g, row rr of the tile, word j of the row
  const int G = K >> 7;
  const int j = (int)(i & 15);
  const int rr = (int)((i >> 4) & 15);
  const long long tg = i >> 8;  // tile * G + g
  const long long t = tg / G;
  const int g = (int)(tg % G);
  const long long r = 16 * t + rr;
  const uint32_t cw = canon[r * wpr + 16 * g + j];  // bytes: elements (2m, 2m+1)
  uint32_t out = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    out |= ((cw >> (8 * m)) & 0xFu) << (4 * m);          // element 2m -> nibble m
    out |= ((cw >> (8 * m + 4)) & 0xFu) << (16 + 4 * m);  // element 2m+1 -> nibble 4+m
  }
  tiled[i] = out;
}

// One thread per 16-byte piece of the output (one plane of one row of one
// tile and group).
__global__ __launch_bounds__(256) void retile_bp_kernel(const u32x4* __restrict__ canon,
                                                        int E, int N, int K,
                                                        u32x4* __restrict__ tiled) {
  const int G = K >> 7;
  const long long per_e = (long long)N * G * 8;  // 16-byte pieces per expert
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)E * per_e) return;
  const long long e = i / per_e;
  const long long w = i % per_e;
  // tiled piece w of expert e: [N/16][G][8][16]
  const int rr = (int)(w & 15);
  const int p = (int)((w >> 4) & 7);
  const long long tg = w >> 7;
  const long long t = tg / G;
  const int g = (int)(tg % G);
  const long long n = 16 * t + rr;
  // canonical piece: slab p, row n, bytes 16 g .. 16 g + 15
  tiled[i] = canon[e * per_e + ((long long)p * N + n) * G + g];
}

}  // namespace

hipError_t launch_retile_w4(const uint8_t* canon, long long R, int K, uint8_t* tiled,
                            hipStream_t s) {
  const long long n = R * (K / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(retile_w4_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     (const uint32_t*)canon, R, K, (uint32_t*)tiled);
  return hipGetLastError();
}

hipError_t launch_retile_bp(const uint8_t* canon, int E, int N, int K, uint8_t* tiled,
                            hipStream_t s) {
  const long long n = (long long)E * N * (K / 128) * 8;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(retile_bp_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     (const u32x4*)canon, E, N, K, (u32x4*)tiled);
  return hipGetLastError();
}

}  // namespace moe
