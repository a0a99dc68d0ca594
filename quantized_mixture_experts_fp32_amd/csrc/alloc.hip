// Read-budget bit allocation for bitplane experts.
// DuoRate ("Two-Rate Per-Expert Precision Allocation for Mixture-of-Experts
// Serving"): the read rate is routing-weighted, sum_e f_e R(b_e); in the
// Lagrangian relaxation the routing frequency cancels from each expert's
// decision, so the selection is one evaluation per expert plus a bisection
// on the multiplier to meet a read budget.  The distortion is taken in weight
// space from the stored bitplane codes (PagedMoE, abstract: prefixes of one
// stored code; MatMoE, abstract: floor-and-compensation), no calibration
// data.
//
// Distortion D_e(b), b = 1..8: per element the prefix error v_b - v_8 is the
// integer 2^(7-b) - (u mod 2^(8-b)); a 128-group's squared errors sum to an
// exact integer I, weighted by s^2 (exact in fp64) with one rounding.  Row
// partials add the groups in ascending order from +0; the expert total adds
// the row partials of gate/up rows 0..2f-1 then down rows 0..d-1 from +0.
// Every fp64 operation is explicit (no contraction), so the totals are
// reproducible bit for bit.
#include "kcommon.hpp"
#include "launch.hpp"

// Products and sums stay separate roundings here (the fixed order above);
// the allocator's key is an explicit fma.
#pragma clang fp contract(off)

namespace moe {
namespace {


__device__ __forceinline__ double dmul(double a, double b) { return a * b; }
__device__ __forceinline__ double dadd(double a, double b) { return a + b; }

// Row partials of one matrix of E experts ([E][R] rows, K inputs, tiled
// bitplane layout) into part[e][row0 + r][8].
__global__ __launch_bounds__(256) void bp_row_distortion(const uint8_t* __restrict__ planes,
                                                         const uint16_t* __restrict__ scales,
                                                         int E, int R, int K, int rows_e,
                                                         int row0, double* __restrict__ part) {
  const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // global row
  if (n >= (int64_t)E * R) return;
  const int G = K / 128;
  const int e = (int)(n / R), r = (int)(n % R);
  double acc[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) acc[b] = 0.0;
  for (int g = 0; g < G; ++g) {
    // row n's 32 bytes of each plane pair: quarters 0, 1 then 2, 3, each
    // the word of the even plane followed by the word of the odd one
    const uint8_t* blk = planes + ((n >> 4) * G + g) * kBpBlock + (n & 15) * 32;
    u32x4 pw[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 lo = *(const u32x4*)(blk + kBpPair * c);
      const u32x4 hi = *(const u32x4*)(blk + kBpPair * c + 16);
      pw[2 * c] = u32x4{lo[0], lo[2], hi[0], hi[2]};
      pw[2 * c + 1] = u32x4{lo[1], lo[3], hi[1], hi[3]};
    }
    int I[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int w = 0; w < 4; ++w)
      for (int i = 0; i < 32; ++i) {  // element 32 w + i of the group
        int u = 0;
#pragma unroll
        for (int p = 0; p < 8; ++p) u |= (int)((pw[p][w] >> i) & 1u) << (7 - p);
#pragma unroll
        for (int b = 1; b < 8; ++b) {
          const int df = (1 << (7 - b)) - (u & ((1 << (8 - b)) - 1));
          I[b - 1] += df * df;
        }
      }
    const double s = (double)f16_bits_to_f32(scales[n * G + g]);
    const double s2 = dmul(s, s);
#pragma unroll
    for (int b = 0; b < 7; ++b) acc[b] = dadd(acc[b], dmul(s2, (double)I[b]));
  }
  double* o = part + ((int64_t)e * rows_e + row0 + r) * 8;
#pragma unroll
  for (int b = 0; b < 8; ++b) o[b] = acc[b];
}

// dist[e][b] = row partials of expert e summed in row order.
__global__ void bp_expert_distortion(const double* __restrict__ part, int E, int rows_e,
                                     double* __restrict__ dist) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= E * 8) return;
  const int e = i / 8, b = i % 8;
  const double* p = part + (int64_t)e * rows_e * 8 + b;
  double tot = 0.0;
  for (int r = 0; r < rows_e; ++r) tot = dadd(tot, p[(int64_t)r * 8]);
  dist[i] = tot;
}

__device__ __forceinline__ int64_t read_bytes(int d, int f, int b) {
  return (int64_t)b * 3 * d * f / 8 + (int64_t)3 * d * f / 64;
}

// The per-expert choice: b in [bmin, bmax] minimizing fma(lambda, R(b),
// D_e(b)); ties go to the larger b.
__device__ int choose(const double* __restrict__ de, int bmin, int bmax, int d, int f,
                      double lambda) {
  int best = bmax;
  double key = fma(lambda, (double)read_bytes(d, f, bmax), de[bmax - 1]);
  for (int b = bmax - 1; b >= bmin; --b) {
    const double kb = fma(lambda, (double)read_bytes(d, f, b), de[b - 1]);
    if (kb < key) {
      key = kb;
      best = b;
    }
  }
  return best;
}

constexpr int kAllocThreads = 512;

// Exact int64 block sum (every thread returns the total).
__device__ int64_t block_sum(int64_t v, int64_t* sh) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();  // sh is reused by consecutive calls
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  int64_t t = 0;
  for (int w = 0; w < kAllocThreads / 64; ++w) t += sh[w];
  return t;
}

__device__ int64_t read_at(const double* __restrict__ dist, const int32_t* __restrict__ counts,
                           int E, int bmin, int bmax, int d, int f, double lambda,
                           int64_t* sh) {
  int64_t v = 0;
  for (int e = threadIdx.x; e < E; e += kAllocThreads)
    v += (int64_t)counts[e] * read_bytes(d, f, choose(dist + 8 * e, bmin, bmax, d, f, lambda));
  return block_sum(v, sh);
}

// One block: the same sequence of multipliers as the plain definition (lambda
// = 0 if the widest choice fits; else hi = 1, doubled at most 1023 times
// until it fits, then 64 halvings of [lo, hi]; infinite if nothing fits).
__global__ __launch_bounds__(kAllocThreads) void allocate_bits_kernel(
    const double* __restrict__ dist, const int32_t* __restrict__ counts, int E, int d, int f,
    int bmin, int bmax, int64_t budget, uint8_t* __restrict__ bits,
    double* __restrict__ lambda_out, int64_t* __restrict__ read_out) {
  __shared__ int64_t sh[kAllocThreads / 64];
  double lambda = 0.0;
  if (read_at(dist, counts, E, bmin, bmax, d, f, 0.0, sh) > budget) {
    double lo = 0.0, hi = 1.0;
    int n = 0;
    while (read_at(dist, counts, E, bmin, bmax, d, f, hi, sh) > budget && n < 1023) {
      lo = hi;
      hi = hi * 2.0;
      ++n;
    }
    if (read_at(dist, counts, E, bmin, bmax, d, f, hi, sh) > budget) {
      hi = __longlong_as_double(0x7FF0000000000000LL);  // +inf
    } else {
      for (int it = 0; it < 64; ++it) {
        const double mid = dmul(0.5, dadd(lo, hi));
        if (read_at(dist, counts, E, bmin, bmax, d, f, mid, sh) <= budget)
          hi = mid;
        else
          lo = mid;
      }
    }
    lambda = hi;
  }
  const bool inf = __builtin_isinf(lambda);
  int64_t v = 0;
  for (int e = threadIdx.x; e < E; e += kAllocThreads) {
    const int b = inf ? bmin : choose(dist + 8 * e, bmin, bmax, d, f, lambda);
    bits[e] = (uint8_t)b;
    v += (int64_t)counts[e] * read_bytes(d, f, b);
  }
  const int64_t tot = block_sum(v, sh);
  if (threadIdx.x == 0) {
    if (lambda_out) *lambda_out = lambda;
    if (read_out) *read_out = tot;
  }
}

}  // namespace

size_t bp_distortion_ws_bytes(int E, int d, int f) {
  return sizeof(double) * 8 * (size_t)E * (2 * (size_t)f + d);
}

hipError_t launch_bp_distortion(const uint8_t* gu_planes, const uint16_t* gu_scales,
                                const uint8_t* dn_planes, const uint16_t* dn_scales, int E,
                                int d, int f, double* dist, void* ws, hipStream_t s) {
  double* part = (double*)ws;
  const int rows_e = 2 * f + d;
  const int64_t ngu = (int64_t)E * 2 * f, ndn = (int64_t)E * d;
  hipLaunchKernelGGL(bp_row_distortion, dim3((unsigned)((ngu + 255) / 256)), dim3(256), 0, s,
                     gu_planes, gu_scales, E, 2 * f, d, rows_e, 0, part);
  hipLaunchKernelGGL(bp_row_distortion, dim3((unsigned)((ndn + 255) / 256)), dim3(256), 0, s,
                     dn_planes, dn_scales, E, d, f, rows_e, 2 * f, part);
  hipLaunchKernelGGL(bp_expert_distortion, dim3((E * 8 + 255) / 256), dim3(256), 0, s, part, E,
                     rows_e, dist);
  return hipGetLastError();
}

hipError_t launch_allocate_bits(const double* dist, const int32_t* counts, int E, int d, int f,
                                int bmin, int bmax, int64_t budget, uint8_t* bits,
                                double* lambda, int64_t* read, hipStream_t s) {
  hipLaunchKernelGGL(allocate_bits_kernel, dim3(1), dim3(kAllocThreads), 0, s, dist, counts, E,
                     d, f, bmin, bmax, budget, bits, lambda, read);
  return hipGetLastError();
}

}  // namespace moe
