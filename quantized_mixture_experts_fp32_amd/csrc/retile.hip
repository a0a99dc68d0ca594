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
//    for element 8j + i.  Streaming: per 16-row tile and 128-group a 2 KiB
//    block of four plane pairs, a row's two words of one pair and quarter
//    side by side (kcommon.hpp); the same bytes regrouped.
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

// One thread per 16-byte piece of the output: half hf of row rr's 32 bytes
// of plane pair c in one tile and group, i.e. quarters 2 hf and 2 hf + 1 of
// planes 2c and 2c + 1 (bytes 8 hf .. 8 hf + 7 of each plane's 16).
__global__ __launch_bounds__(256) void retile_bp_kernel(const uint2* __restrict__ canon,
                                                        int E, int N, int K,
                                                        u32x4* __restrict__ tiled) {
  const int G = K >> 7;
  const long long per_e = (long long)N * G * 8;  // 16-byte pieces per expert
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)E * per_e) return;
  const long long e = i / per_e;
  const long long w = i % per_e;
  // piece w of expert e: block tg = w / 128, then pair, row, half
  const int hf = (int)(w & 1);
  const int rr = (int)((w >> 1) & 15);
  const int c = (int)((w >> 5) & 3);
  const long long tg = w >> 7;
  const long long t = tg / G;
  const int g = (int)(tg % G);
  const long long n = 16 * t + rr;
  // canonical: slab p, row n, bytes 16 g + 8 hf .. 16 g + 8 hf + 7
  const uint2* ce = canon + 2 * e * per_e;
  const uint2 a = ce[(((long long)(2 * c) * N + n) * G + g) * 2 + hf];
  const uint2 b = ce[(((long long)(2 * c + 1) * N + n) * G + g) * 2 + hf];
  tiled[i] = u32x4{a.x, b.x, a.y, b.y};
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
                     (const uint2*)canon, E, N, K, (u32x4*)tiled);
  return hipGetLastError();
}

}  // namespace moe
