// Prefill-path expert FFN for int4 experts: grouped GEMMs on bf16 MFMA.
//  ExactMoE ("Every Expert Counts ...", Abstract): symmetric group-128 W4A16
//  routed experts, every selected pair computed by grouped kernels.
//
// Layout of the product.  Tokens are the MFMA M dimension (A operand, from
// LDS), output features the N dimension (B operand, int4 codes dequantized
// in registers), so that each lane of a 32x32 accumulator tile owns one
// output feature and needs one fp16 scale per 128-group.
//
// Arithmetic.  As in the decode path, a nibble becomes bf16(24 + q) with one
// v_bitop3, and each group's partial sum starts from -24 * sum_k x_k: that
// term enters as one extra MFMA per group whose A column holds the exact
// three-part bf16 split (hi + mid + lo) of the fp32 group sum of the token's
// activations, and whose B column holds -24.  The running fp32 total is kept
// in units of the current group's fp16 scale: before a group with a new
// scale is accumulated, the total is multiplied by s_prev / s_g, and after
// the last group by the final scale, so every group's sum is weighted by its
// own scale without a separate partial accumulator.
// A pre-pass kernel computes the group sums (and their splits) of x per
// token and of h per grouped pair.
//
// Tiling.  Block = 4 waves = 128 tokens x 64 features (gate/up: 64 features
// of gate and the same 64 of up).  Wave (wt, wf) owns tokens [64 wt, +64)
// and 32 features.  Per 128-group the block stages the 128 x 128 bf16
// activation tile in LDS (double buffered, rows padded by 16 bytes, stored in
// the nibble order 0,4,1,5,2,6,3,7 of the conversion), while every wave
// streams its own code rows from HBM one group ahead.
#include "kcommon.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBT = 128;      // tokens per block tile
constexpr int kRowB = 272;    // LDS bytes per token row: 256 + 16 padding
constexpr int kBufB = kBT * kRowB;
constexpr int kPfWaves = 2;   // waves per SIMD the register allocation is held to

struct PTile {
  int e, r0, cnt, maxb;
};

// 8 nibbles -> bf16 (136 + q), element order 0,4,1,5,2,6,3,7 (the same
// conversion as the decode path: q + 8 lands in the low mantissa bits of
// 128.0, unshifted for elements 0 and 4).
__device__ __forceinline__ bf16x8 w4_magic_pf(uint32_t w) {
  const uint32_t B = 0x000F000Fu, D = 0x43084308u;
  u32x4 r;
  r[0] = __builtin_amdgcn_bitop3_b32(w, B, D, 0x6A);
  r[1] = __builtin_amdgcn_bitop3_b32(w >> 4, B, D, 0x6A);
  r[2] = __builtin_amdgcn_bitop3_b32(w >> 8, B, D, 0x6A);
  r[3] = __builtin_amdgcn_bitop3_b32(w >> 12, B, D, 0x6A);
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ u32x4 perm8(u32x4 v) {
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(v[2], v[0], 0x05040100u);
  r[1] = __builtin_amdgcn_perm(v[2], v[0], 0x07060302u);
  r[2] = __builtin_amdgcn_perm(v[3], v[1], 0x05040100u);
  r[3] = __builtin_amdgcn_perm(v[3], v[1], 0x07060302u);
  return r;
}

// ---------------------------------------------------------------- pre-pass
// For row r (token t of x, or grouped slot of h) and group g: s = fp32 sum
// of the 128 bf16 elements, split exactly into three bf16 parts
// (hi = bf16_rne(s), mid = bf16_rne(s - hi), lo = bf16_rne(s - hi - mid)),
// stored as uint2 {hi | mid << 16, lo}.
__global__ __launch_bounds__(256) void group_sums(const uint16_t* __restrict__ rows,
                                                  long long R, int K,
                                                  uint2* __restrict__ out) {
  const int G = K >> 7;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= R * G) return;
  const long long r = i / G;
  const int g = (int)(i % G);
  const uint16_t* p = rows + r * K + 128 * g;
  float s = 0.0f;
#pragma unroll 4
  for (int c = 0; c < 16; ++c) {
    const u32x4 v = *(const u32x4*)(p + 8 * c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s += __uint_as_float(v[q] << 16);
      s += __uint_as_float(v[q] & 0xFFFF0000u);
    }
  }
  const uint32_t hi = f32_to_bf16_rne(s);
  const float r1 = s - __uint_as_float(hi << 16);
  const uint32_t mid = f32_to_bf16_rne(r1);
  const float r2 = r1 - __uint_as_float(mid << 16);
  const uint32_t lo = f32_to_bf16_rne(r2);
  out[i] = uint2{hi | (mid << 16), lo};
}

// ------------------------------------------------------------- GEMM core
// One block = one tile of up to 128 grouped rows (tokens) x one feature
// block; every wave owns all 128 tokens (four 32-token blocks) and two
// 32-feature B blocks, i.e. eight 32x32 fp32 accumulators, so that each
// converted code fragment feeds four MFMAs.
//   gate/up (kGateUp): feature block fb covers features [128 fb, +128);
//     wave w's B blocks are gate rows n = 128 fb + 32 w + c32 and the up
//     rows N + n, so h = silu(gate) * up is formed in the lane.
//   down: feature block fb covers [256 fb, +256); wave w's B blocks are rows
//     256 fb + 64 w + c32 and + 32 (blocks at or past N are computed on a
//     clamped row and not stored).
// Pipeline per 128-group g: the block's barrier publishes the staged
// activation tile of g; activations of g + 1 are then loaded into registers
// while g is computed and written to the other LDS buffer afterwards; each
// wave's codes run two groups ahead of the MFMAs.
template <bool kGateUp>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kPfWaves, kPfWaves)))
void pf_w4_kernel(const uint16_t* __restrict__ act,       // x [T][K] or h [P][K]
                  const int32_t* __restrict__ sorted_pair,  // gate/up: gather
                  int k_top, int K, int N,                  // N: features per matrix
                  const uint8_t* __restrict__ codes,        // tiled [E*rows/16][K/128][16][64]
                  const uint16_t* __restrict__ scales,      // [E][rows][K/128]
                  const uint2* __restrict__ gsum,           // [rows of act][K/128]
                  const PTile* __restrict__ tiles, const int* __restrict__ num_tiles,
                  int nfb,                                  // feature blocks per tile
                  uint16_t* __restrict__ h_out,             // gate/up: [P][N]
                  float* __restrict__ y_out) {              // down:    [P][N]
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ uint2 xs_sum[2][kBT];  // group sums of the staged tile

  // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin by
  // linear id, so XCD c runs tiles c, c + 8, ...; within an XCD all nfb
  // feature blocks of a tile are consecutive and run together, and the
  // tile's gathered activation rows are fetched into that XCD's L2 once.
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int tile = (local / nfb) * 8 + xcd, fblk = local % nfb;
  if (tile >= *num_tiles) return;
  const PTile tl = tiles[tile];
  const int G = K >> 7;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c32 = lane & 31, hh = lane >> 5;
  const int nrows = kGateUp ? 2 * N : N;
  const size_t ebase = (size_t)tl.e * nrows;

  int brow[2];
  bool bstore[2];
  if (kGateUp) {
    const int n = fblk * 128 + wave * 32 + c32;
    brow[0] = n;
    brow[1] = N + n;
    bstore[0] = bstore[1] = true;
  } else {
    const int n0 = fblk * 256 + wave * 64;
    bstore[0] = n0 < N;
    bstore[1] = n0 + 32 < N;
    brow[0] = bstore[0] ? n0 + c32 : c32;
    brow[1] = bstore[1] ? n0 + 32 + c32 : c32;
  }
  const uint8_t* cb[2];
  const uint16_t* sb[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const size_t row = ebase + brow[m];  // tiled codes: 16-row tiles, 1 KiB per group
    cb[m] = codes + (row & ~(size_t)15) * (size_t)(K >> 1) + 64 * (row & 15) + 32 * hh;
    sb[m] = scales + row * (size_t)G;
  }

  // staging assignment: thread -> (token row, half of the group)
  const int st_row = tid & (kBT - 1), st_half = tid >> 7;
  const bool st_valid = st_row < tl.cnt;
  const int st_slot = tl.r0 + (st_valid ? st_row : 0);
  const long long st_src_row = kGateUp ? (long long)(sorted_pair[st_slot] / k_top) : st_slot;
  const uint16_t* st_src = act + st_src_row * K + 64 * st_half;
  const uint2* st_sum = gsum + st_src_row * G;

  // Activations are staged through registers in two halves of four
  // 16-byte chunks each, so that only 16 registers hold them in flight.
  u32x4 stv[4];
  uint2 st_s = {0u, 0u};
  auto stage_load = [&](int g, int half) {
#pragma unroll
    for (int c = 0; c < 4; ++c) stv[c] = *(const u32x4*)(st_src + 128 * g + 32 * half + 8 * c);
    if (half == 0 && st_half == 0) st_s = st_sum[g];
  };
  auto stage_store = [&](int buf, int half) {
    uint8_t* rowp = lds + buf * kBufB + st_row * kRowB + 128 * st_half + 64 * half;
#pragma unroll
    for (int c = 0; c < 4; ++c) *(u32x4*)(rowp + 16 * c) = perm8(stv[c]);
    if (half == 0 && st_half == 0) xs_sum[buf][st_row] = st_s;
  };
  auto codes_load = [&](int g, u32x4 (&q)[2][2], uint32_t (&sc)[2]) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      q[m][0] = *(const u32x4*)(cb[m] + 1024 * g);
      q[m][1] = *(const u32x4*)(cb[m] + 1024 * g + 16);
      sc[m] = sb[m][g];
    }
  };

  // Running totals are kept in units of the current group's scale: before
  // group g is added, acc *= s_prev / s_g (1 when unchanged); after the last
  // group acc *= s.  All-zero groups (s_g == 0) contribute nothing and keep
  // s_prev.
  f32x16 acc[4][2];  // [token block][B block]
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][m][i] = 0.0f;
  float s_cur[2] = {0.0f, 0.0f};

  // B column of the offset MFMA: -136 in K rows 0..2 (lanes of half 0)
  u32x4 negv = {0u, 0u, 0u, 0u};
  if (hh == 0) {
    negv[0] = 0xC308C308u;  // -136, -136
    negv[1] = 0x0000C308u;  // -136, 0
  }
  const bf16x8 negB = __builtin_bit_cast(bf16x8, negv);

  auto group_step = [&](int g, u32x4 (&q)[2][2], uint32_t (&sc)[2]) {
    const int buf = g & 1;
    __syncthreads();  // tile g staged; every wave is done reading buffer buf ^ 1
    const bool more = g + 1 < G;
    if (more) stage_load(g + 1, 0);
    const uint8_t* abase = lds + buf * kBufB + c32 * kRowB + 128 * hh;
    float r[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float sg = f16_bits_to_f32(sc[m]);
      const bool upd = sg != 0.0f;
      r[m] = upd ? ((s_cur[m] == 0.0f) ? 0.0f : s_cur[m] / sg) : 1.0f;
      s_cur[m] = upd ? sg : s_cur[m];
    }
    // offset term and rescale, token block by token block
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (hh == 0) {
        const uint2 ss = xs_sum[buf][t * 32 + c32];
        v[0] = ss.x;
        v[1] = ss.y;
      }
      const bf16x8 sumA = __builtin_bit_cast(bf16x8, v);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][m][i] *= r[m];
        acc[t][m] = mfma32(sumA, negB, acc[t][m]);
      }
    }
    bf16x8 af[2][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      af[0][t] = __builtin_bit_cast(bf16x8, *(const u32x4*)(abase + t * 32 * kRowB));
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) {
      const int cur = s2 & 1;
      if (s2 + 1 < 8) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          af[cur ^ 1][t] = __builtin_bit_cast(
              bf16x8, *(const u32x4*)(abase + t * 32 * kRowB + 16 * (s2 + 1)));
      }
      bf16x8 bfr[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) bfr[m] = w4_magic_pf(q[m][s2 >> 2][s2 & 3]);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int m = 0; m < 2; ++m) acc[t][m] = mfma32(af[cur][t], bfr[m], acc[t][m]);
      if (s2 == 3 && more) {
        stage_store(buf ^ 1, 0);
        stage_load(g + 1, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (g + 2 < G) codes_load(g + 2, q, sc);
    if (more) stage_store(buf ^ 1, 1);
  };

  u32x4 qa[2][2], qb[2][2];  // [B block][16-byte half] codes of groups g, g + 1
  uint32_t sca[2], scb[2];
  codes_load(0, qa, sca);
  if (G > 1) codes_load(1, qb, scb);
  stage_load(0, 0);
  stage_store(0, 0);
  stage_load(0, 1);
  stage_store(0, 1);
  for (int g = 0; g < G; g += 2) {
    group_step(g, qa, sca);
    if (g + 1 < G) group_step(g + 1, qb, scb);
  }
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][m][i] *= s_cur[m];

  // ---- epilogue: lane owns feature brow (per B block) for 16 token rows
  // of each token block: rows 8*(i/4) + 4*hh + i%4 of the 32-row block.
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tok = t * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
      if (tok >= tl.cnt) continue;
      const size_t slot = (size_t)(tl.r0 + tok);
      if (kGateUp) {
        const float hv = silu_f32(acc[t][0][i]) * acc[t][1][i];
        h_out[slot * N + brow[0]] = (uint16_t)f32_to_bf16_rne(hv);
      } else {
        if (bstore[0]) y_out[slot * N + brow[0]] = acc[t][0][i];
        if (bstore[1]) y_out[slot * N + brow[1]] = acc[t][1][i];
      }
    }
}

__global__ __launch_bounds__(1024) void pf_prep(const int32_t* __restrict__ offsets, int E,
                                                PTile* __restrict__ tiles,
                                                int* __restrict__ num_tiles) {
  __shared__ int sc[1024];
  const int e = threadIdx.x;
  int lo = 0, n = 0;
  if (e < E) {
    lo = offsets[e];
    n = offsets[e + 1] - lo;
  }
  const int nt = (n + kBT - 1) / kBT;
  sc[e] = nt;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = (e >= off) ? sc[e - off] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  const int base = sc[e] - nt;
  for (int c = 0; c < nt; ++c)
    tiles[base + c] = PTile{e, lo + c * kBT, min(kBT, n - c * kBT), 8};
  if (e == 1023) *num_tiles = sc[1023];
}

}  // namespace

size_t ffn_prefill_ws_bytes(int T, int k, int E, int d, int f) {
  const long long P = (long long)T * k;
  const size_t tiles = (size_t)((P + kBT - 1) / kBT + (P < E ? P : E));
  auto a256 = [](size_t v) { return (v + 255) & ~(size_t)255; };
  return 256 + a256(tiles * sizeof(PTile)) + a256((size_t)T * (d / 128) * 8) +
         a256((size_t)P * (f / 128) * 8);
}

hipError_t launch_ffn_prefill_w4(const FfnArgs& a, uint16_t* h, void* ws, hipStream_t s) {
  const long long P = (long long)a.T * a.k;
  auto a256 = [](size_t v) { return (v + 255) & ~(size_t)255; };
  char* w = (char*)ws;
  int* num_tiles = (int*)w;
  PTile* tiles = (PTile*)(w + 256);
  const size_t mt = (size_t)((P + kBT - 1) / kBT + (P < a.E ? P : a.E));
  uint2* xsum = (uint2*)(w + 256 + a256(mt * sizeof(PTile)));
  uint2* hsum = (uint2*)((char*)xsum + a256((size_t)a.T * (a.d / 128) * 8));
  const size_t lds = 2 * (size_t)kBufB;

  hipLaunchKernelGGL(pf_prep, dim3(1), dim3(1024), 0, s, a.offsets, a.E, tiles, num_tiles);
  {
    const long long n = (long long)a.T * (a.d / 128);
    hipLaunchKernelGGL(group_sums, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.x,
                       (long long)a.T, a.d, xsum);
  }
  if (a.ev[0]) hipEventRecord(a.ev[0], s);
  const unsigned mt8 = (unsigned)((mt + 7) & ~(size_t)7);
  hipLaunchKernelGGL((pf_w4_kernel<true>), dim3(mt8 * (a.f / 128)), dim3(kThreads), lds, s,
                     a.x, a.sorted_pair, a.k, a.d, a.f, a.gu_codes, a.gu_scales, xsum, tiles,
                     num_tiles, a.f / 128, h, (float*)nullptr);
  if (a.ev[1]) hipEventRecord(a.ev[1], s);
  {
    const long long n = P * (a.f / 128);
    hipLaunchKernelGGL(group_sums, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, h, P,
                       a.f, hsum);
  }
  if (a.ev[2]) hipEventRecord(a.ev[2], s);
  const int dn_fb = (a.d + 255) / 256;
  hipLaunchKernelGGL((pf_w4_kernel<false>), dim3(mt8 * dn_fb), dim3(kThreads), lds,
                     s, h, a.sorted_pair, a.k, a.f, a.d, a.dn_codes, a.dn_scales, hsum, tiles,
                     num_tiles, dn_fb, (uint16_t*)nullptr, a.y);
  if (a.ev[3]) hipEventRecord(a.ev[3], s);
  return hipGetLastError();
}

}  // namespace moe
