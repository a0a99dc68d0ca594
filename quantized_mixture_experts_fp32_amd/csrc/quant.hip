// Offline quantizers (untimed packing of fp32 expert weights on the GPU).
//  int4 (ExactMoE, "Every Expert Counts ...", Abstract: symmetric group-128
//    four-bit): s = fp16_rne(max|w|/7), q = clamp(rne(w/s), -7, 7), q = 0 if
//    s == 0; in the tiled layout the FFN kernels stream: [rows/16][K/128]
//    [16 rows][64 bytes], so one 16-row tile's 128-group is 1 KiB
//    contiguous; 32-bit word j of a row's group holds elements 8j..8j+7,
//    the even ones in nibbles 0-3 and the odd ones in nibbles 4-7, so that
//    the kernels' nibble-to-bf16 conversion yields them in order.
//  bitplane8 (PagedMoE, abstract: one stored state, bitplane prefixes):
//    s = fp16_rne(max|w|/127), u = clamp(rne(w/s) + 128, 0, 255), u = 128 if
//    s == 0; per 16-row tile and 128-group a 2 KiB block holds the 8 planes
//    (plane p = bit 7-p) of 16 rows x 16 bytes; bit i of byte j is element
//    8j + i of the group.
// Both quotients are evaluated in fp64, so each rounding is the rounding of
// the exact quotient; codes and scales are bit-exact.
#include "kcommon.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;  // 4 waves, one 128-element group per wave

template <bool kBitplane>
__global__ __launch_bounds__(kThreads) void quant_kernel(
    const float* __restrict__ w, long long ngroups, long long N, int K,
    uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int G = K >> 7;
  for (long long grp = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
       grp < ngroups; grp += (long long)gridDim.x * 4) {
    const float2 v = *(const float2*)(w + grp * 128 + 2 * lane);
    float a = fmaxf(fabsf(v.x), fabsf(v.y));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, kWave));
    const uint32_t s16 = f64_to_f16_rne((double)a / (kBitplane ? 127.0 : 7.0));
    const double s = (double)f16_bits_to_f32(s16);
    if (lane == 0) scales[grp] = (uint16_t)s16;
    if (!kBitplane) {
      int q[2];
      const float vv[2] = {v.x, v.y};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        double r = (s == 0.0) ? 0.0 : rint((double)vv[h] / s);
        r = fmin(fmax(r, -7.0), 7.0);
        q[h] = (int)r;
      }
      // elements 2*lane (even) and 2*lane+1 (odd) of the group sit in word
      // lane/4: even elements in the low half-word, odd ones in the high
      // half-word, at nibble lane % 4 of each half
      const long long row = grp / G;  // over all E*N rows; N % 16 == 0
      const long long g = grp % G;
      uint32_t wv = ((uint32_t)(q[0] & 0xF) << (4 * (lane & 3))) |
                    ((uint32_t)(q[1] & 0xF) << (16 + 4 * (lane & 3)));
      wv |= __shfl_xor(wv, 1, kWave);
      wv |= __shfl_xor(wv, 2, kWave);
      if ((lane & 3) == 0)
        *(uint32_t*)(codes + (((row >> 4) * G + g) * 16 + (row & 15)) * 64 + lane) = wv;
    } else {
      int u[2];
      const float vv[2] = {v.x, v.y};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        double r = (s == 0.0) ? 128.0 : rint((double)vv[h] / s) + 128.0;
        r = fmin(fmax(r, 0.0), 255.0);
        u[h] = (int)r;
      }
      // elements 2*lane and 2*lane+1 of the group: byte lane/4 of the row's
      // 16 bytes of each plane, bit positions 2*(lane%4) and +1, stored in
      // the 2 KiB block of the row's 16-row tile and group (kcommon.hpp)
      const long long row = grp / G;  // over all E*N rows; N % 16 == 0
      const long long g = grp % G;
      uint8_t* blk = codes + ((row >> 4) * G + g) * kBpBlock;
      const int r16 = (int)(row & 15), j = lane >> 2;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        uint32_t bits = (((u[0] >> (7 - p)) & 1) | (((u[1] >> (7 - p)) & 1) << 1))
                        << (2 * (lane & 3));
        bits |= __shfl_xor(bits, 1, kWave);
        bits |= __shfl_xor(bits, 2, kWave);
        if ((lane & 3) == 0) blk[bp_byte(p, r16, j)] = (uint8_t)bits;
      }
    }
  }
}

}  // namespace

hipError_t launch_quantize(const float* w, long long E, long long N, int K,
                           int bitplane, uint8_t* codes, uint16_t* scales,
                           hipStream_t s) {
  const long long ngroups = E * N * (K / 128);
  if (ngroups == 0) return hipSuccess;
  long long blocks = (ngroups + 3) / 4;
  if (blocks > 262144) blocks = 262144;
  if (bitplane)
    hipLaunchKernelGGL(quant_kernel<true>, dim3((unsigned)blocks),
                       dim3(kThreads), 0, s, w, ngroups, N, K, codes, scales);
  else
    hipLaunchKernelGGL(quant_kernel<false>, dim3((unsigned)blocks),
                       dim3(kThreads), 0, s, w, ngroups, N, K, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
