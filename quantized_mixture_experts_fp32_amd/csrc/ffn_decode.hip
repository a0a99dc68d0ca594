// Decode-path expert FFN for int4 experts (small batches, HBM-bound).
//  ExactMoE ("Every Expert Counts ...", Abstract): symmetric group-128 W4A16
//  routed experts executed by grouped kernels; decode is bound by moving the
//  expert weights, so each selected expert's packed codes stream from HBM
//  once per token tile with 16-byte loads and are dequantized in registers.
//
// Arithmetic.  A code nibble n (two's complement q) is turned into the bf16
// value 136 + q with one v_bitop3 (128.0 with q + 8 in the low four
// mantissa bits); 136 + q is an exact bf16 integer.  The MFMA accumulator of
// every 128-group starts from -136 * sum(x over the group), produced by four
// MFMAs with a constant -136 A-operand, so the group's sum is
// sum((136+q) x) - 136 sum(x) = sum(q x) with fp32 accumulation only.  The
// fp16 scale then multiplies the group sum (fp32) and the product is added to
// the running fp32 total.  Dequantized weights are never rounded.
//
// Layout.  Codes are stored in 16-row tiles (see the ABI header): lane
// (col, kq) of a wave reads bytes [16kq, 16kq + 16) of row col of its tile's
// 128-group, so one wave-wide 16-byte load covers the tile's group, 1 KiB
// contiguous, and consecutive groups are consecutive kilobytes.
//
// K order.  Word j of a row's group holds elements 8j..8j+7 with the even
// elements in its low half-word and the odd ones in the high half-word, so
// the conversion yields them in natural order and activation fragments are
// used as loaded.
//
// Work decomposition.  Work item = (token tile of up to 16*NT grouped
// pairs of one expert, 4/KS row tiles of 16 output features).  Each wave
// streams one row tile over one of KS slices of K, keeping kDepth 128-groups
// of codes and activations in flight; the K slices are reduced through LDS in
// a fixed order.  Blocks are persistent: they walk the work items with a
// grid stride and decode their tile from expert_offsets staged in LDS (no
// separate preparation launch).
#include <algorithm>
#include <type_traits>

#include "kcommon.hpp"
#include "launch.hpp"
#include "route_common.hpp"
#include "permute_common.hpp"
#include "decode_common.hpp"

namespace moe {
namespace {
using namespace dec;

constexpr int kTileGroupBytes = 16 * 64;  // one 16-row tile x one 128-group

// Code loads carry the nontemporal hint: a decode step reads each activated
// expert's codes once, and streaming them past the caches keeps the
// activations, h, the scales and the routing resident in L2 and the
// Infinity Cache.  (The one-token kernel's direct-to-LDS code loads keep
// the default policy, which measured faster there.)

// One code word (elements 8j..8j+7, even ones in nibbles 0-3, odd ones in
// nibbles 4-7) -> bf16 (136 + q) of the 8 elements in order.
// bitop3 LUT 0x6A: out = B ? (x ^ D) : D.  B selects bits 0-3 of each half,
// the low mantissa bits of 128.0 (whose ulp is 1): nibble m and nibble m + 4
// (elements 2m and 2m + 1) land there after a shift by 4m; D = 0x4308 per
// half is 128.0 plus the inversion of the nibble's top bit, which maps
// two's complement q to q + 8.
__device__ __forceinline__ bf16x8 w4_magic(uint32_t w) {
  const uint32_t B = 0x000F000Fu, D = 0x43084308u;
  u32x4 r;
  r[0] = __builtin_amdgcn_bitop3_b32(w, B, D, 0x6A);
  r[1] = __builtin_amdgcn_bitop3_b32(w >> 4, B, D, 0x6A);
  r[2] = __builtin_amdgcn_bitop3_b32(w >> 8, B, D, 0x6A);
  r[3] = __builtin_amdgcn_bitop3_b32(w >> 12, B, D, 0x6A);
  return __builtin_bit_cast(bf16x8, r);
}

constexpr uint32_t kBf16NegOff = 0xC308u;  // -136.0, the conversion offset


// Scales of a work item, staged once as fp32 in LDS: [matrix][group][row].
// rows_src: first scale row of matrix 0; matrices are mat_stride rows apart.
__device__ __forceinline__ void stage_scales_f32(const uint16_t* __restrict__ rows_src,
                                                 size_t mat_stride, int nmat, int rows,
                                                 int G, float* __restrict__ dst) {
  const int total = nmat * rows * G;
  for (int i = threadIdx.x; i < total; i += blockDim.x) {
    const int g = i % G, r = (i / G) % rows, m = i / (G * rows);
    dst[(m * G + g) * rows + r] =
        f16_bits_to_f32(rows_src[(size_t)m * mat_stride * G + (size_t)r * G + g]);
  }
}


// One 128-group of one 16-row matrix tile: offset-corrected MFMA sum,
// scaled and accumulated.  xp/seed are shared by the tiles of a group.
__device__ __forceinline__ void tile_group(const bf16x8 (&xp)[4], const f32x4 seed,
                                           const u32x4 q, const f32x4 sv, f32x4& acc) {
  f32x4 p = seed;
#pragma unroll
  for (int j = 0; j < 4; ++j) p = mfma16(w4_magic(q[j]), xp[j], p);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = fmaf(sv[i], p[i], acc[i]);
}

// Routing of a K-split gate/up block.  With kLg the block selects and
// groups the batch itself from the router logits [T][E] (block 0 stores
// every routing output; scratch: 128 + E ints of LDS); otherwise it stages
// expert_offsets and sorted_pair.  Returns the pairs staged in sp_lds (0:
// sorted_pair is read from global memory).
template <bool kLg>
__device__ __forceinline__ int ks_route(const int32_t* __restrict__ offsets,
                                        const int32_t* __restrict__ sorted_pair, int E, int k,
                                        int P, const float* __restrict__ logits,
                                        int32_t* __restrict__ idx_out, float* __restrict__ w_out,
                                        int32_t* __restrict__ offsets_out,
                                        int32_t* __restrict__ sorted_pair_out,
                                        int32_t* __restrict__ pair_pos_out, int32_t* off_lds,
                                        int32_t* sp_lds, int32_t* scratch) {
  if constexpr (kLg) {
    int32_t* idx_lds = scratch;      // [64] experts of the pairs
    int32_t* pp_lds = idx_lds + 64;  // [64] slot of each pair
    int32_t* cnt_lds = pp_lds + 64;  // [E]
    const bool store = blockIdx.x == 0;
    const int T = P / k, lane = threadIdx.x & 63;
    for (int t = threadIdx.x >> 6; t < T; t += 4) {  // wave-uniform
      int32_t* io = store ? idx_out + (size_t)t * k : nullptr;
      float* wo = store ? w_out + (size_t)t * k : nullptr;
      select_topk_radix64(lane < E ? logits[(size_t)t * E + lane] : 0.0f, E, k, io, wo,
                          idx_lds + t * k);
    }
    __syncthreads();
    if (threadIdx.x < 64) permute_wave_small(idx_lds, P, E, off_lds, sp_lds, pp_lds, cnt_lds);
    __syncthreads();
    if (store) {
      for (int i = threadIdx.x; i <= E; i += blockDim.x) offsets_out[i] = off_lds[i];
      for (int i = threadIdx.x; i < P; i += blockDim.x) {
        sorted_pair_out[i] = sp_lds[i];
        pair_pos_out[i] = pp_lds[i];
      }
    }
    return P;
  } else {
    const int np = stage_routing(offsets, sorted_pair, E, P, off_lds, sp_lds);
    __syncthreads();
    return np;
  }
}

// ------------------------------------------------------------- gate / up
// Work item = (token tile of up to 16*NT pairs, row group of RT = 4/KS row
// tiles of 16 features).  Wave (rt, ks) streams gate and up codes of its row
// tile over K slice ks with kDepth groups of codes and activations in flight.
// With kLg (at most 64 pairs, E <= 64) the block routes the batch itself
// from the router logits [T][E]: wave w selects the top-k of tokens w,
// w + 4, ... (the routing kernels' ballot selection), wave 0 groups the
// pairs (the one-wave counting sort), and block 0 stores every routing
// output; the routing launch before it only computes logits.  (With E = 256
// the arg-max selection in every block cost more than the launch it saves.)
template <int KS, int NT, int kDepth, int kWaves, bool kLg>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWaves, 8)))
void gateup_w4_decode(const uint16_t* __restrict__ x, const int32_t* __restrict__ offsets,
                      const int32_t* __restrict__ sorted_pair, int E, int k, int P,
                      int d, int f, const uint8_t* __restrict__ codes,
                      const uint16_t* __restrict__ scales, uint16_t* __restrict__ h,
                      const float* __restrict__ logits, int32_t* __restrict__ idx_out,
                      float* __restrict__ w_out, int32_t* __restrict__ offsets_out,
                      int32_t* __restrict__ sorted_pair_out,
                      int32_t* __restrict__ pair_pos_out) {
  constexpr int RT = 4 / KS;
  extern __shared__ int32_t lds_i[];
  const int G = d >> 7, RG = f / (16 * RT);
  int32_t* off_lds = lds_i;
  int32_t* sp_lds = lds_i + ((E + 1 + 3) & ~3);
  float* sc_lds = (float*)(sp_lds + ((min(P, kPairsInLds) + 3) & ~3));  // [2][G][16 RT]
  f32x4* red = (f32x4*)(sc_lds + 2 * G * 16 * RT);                       // [4][NT][2][64]
  const int np = ks_route<kLg>(offsets, sorted_pair, E, k, P, logits, idx_out, w_out,
                               offsets_out, sorted_pair_out, pair_pos_out, off_lds, sp_lds,
                               (int32_t*)(red + 4 * NT * 2 * 64));

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int rt = wave / KS, ks = wave % KS;
  const int gps = (G + KS - 1) / KS;
  const int gb = ks * gps, ge = min(G, gb + gps);
  const bf16x8 negoff = bf16_splat(kBf16NegOff);

  for (int w = blockIdx.x;; w += gridDim.x) {
    TileInfo tl;
    if (!find_tile(off_lds, E, 16 * NT, w / RG, tl)) break;
    const int nb = (w % RG) * 16 * RT, n0 = nb + 16 * rt;
    const size_t erow = (size_t)tl.e * 2 * f;
    const int nch = (tl.cnt + 15) >> 4;

    // Token columns past the tile's end read the tile's first row instead:
    // a B column only feeds its own output column, which is not stored.
    const uint16_t* xr[NT];
    bool valid[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      const int j = 16 * c + col;
      valid[c] = j < tl.cnt;
      const int jj = valid[c] ? j : 0;
      const int p = np ? sp_lds[tl.r0 + jj] : sorted_pair[tl.r0 + jj];
      xr[c] = x + (size_t)(p / k) * d + 32 * kq;
    }
    const uint8_t* cg = codes + (erow + n0) * (size_t)(d >> 1) + 64 * col + 16 * kq;
    const uint8_t* cu = cg + (size_t)f * (d >> 1);

    u32x4 qg[kDepth], qu[kDepth], xv[kDepth][NT][4];
    auto load = [&](int g, u32x4& a, u32x4& b, u32x4 (&v)[NT][4]) {
      a = __builtin_nontemporal_load((const u32x4*)(cg + kTileGroupBytes * g));
      b = __builtin_nontemporal_load((const u32x4*)(cu + kTileGroupBytes * g));
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        if (c >= nch) break;
        const uint16_t* xg = xr[c] + 128 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[c][j] = *(const u32x4*)(xg + 8 * j);
      }
    };
    // The item's scales: with at most 1024 of them, G % 4 == 0 and 8-byte
    // aligned rows, one 8-byte piece (4 groups of one row) per thread,
    // fetched before the code loads so that both share one round trip
    // (staging them one by one after the barrier costs a round trip per
    // 256 scales); otherwise staged one by one.
    const int nsc = 2 * 16 * RT * G;
    const bool vsc = (G & 3) == 0 && nsc <= 4 * 256 && ((uintptr_t)scales & 7) == 0;
    const int scc = min((int)threadIdx.x, nsc / 4 - 1);
    const int sc_m = (4 * scc) / (16 * RT * G), sc_rem = 4 * scc - sc_m * 16 * RT * G;
    uint2 scv = {0u, 0u};
    if (vsc)
      scv = *(const uint2*)(scales + (erow + nb + (size_t)sc_m * f) * G + sc_rem);
#pragma unroll
    for (int i = 0; i < kDepth; ++i)
      if (gb + i < ge) load(gb + i, qg[i], qu[i], xv[i]);

    __syncthreads();  // previous item is done with sc_lds / red
    if (vsc) {
      if ((int)threadIdx.x < nsc / 4) {
        const int r = sc_rem / G, g0 = sc_rem % G;
        float* dd = sc_lds + (sc_m * G + g0) * (16 * RT) + r;
        dd[0] = f16_bits_to_f32(scv.x & 0xFFFFu);
        dd[16 * RT] = f16_bits_to_f32(scv.x >> 16);
        dd[32 * RT] = f16_bits_to_f32(scv.y & 0xFFFFu);
        dd[48 * RT] = f16_bits_to_f32(scv.y >> 16);
      }
    } else {
      stage_scales_f32(scales + (erow + nb) * G, (size_t)f, 2, 16 * RT, G, sc_lds);
    }
    __syncthreads();

    f32x4 tg[NT], tu[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) tg[c] = tu[c] = f32x4{0, 0, 0, 0};
    for (int g = gb; g < ge; g += kDepth) {
#pragma unroll
      for (int i = 0; i < kDepth; ++i) {
        const int gi = g + i;
        if (gi >= ge) break;
        const f32x4 sg = *(const f32x4*)(sc_lds + gi * (16 * RT) + 16 * rt + 4 * kq);
        const f32x4 su = *(const f32x4*)(sc_lds + (G + gi) * (16 * RT) + 16 * rt + 4 * kq);
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          if (c >= nch) break;
          bf16x8 xp[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) xp[j] = __builtin_bit_cast(bf16x8, xv[i][c][j]);
          f32x4 seed = {0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < 4; ++j) seed = mfma16(negoff, xp[j], seed);
          tile_group(xp, seed, qg[i], sg, tg[c]);
          tile_group(xp, seed, qu[i], su, tu[c]);
        }
        if (gi + kDepth < ge) load(gi + kDepth, qg[i], qu[i], xv[i]);
      }
    }

    if (KS > 1) {
      if (ks > 0) {
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          red[((wave * NT + c) * 2 + 0) * 64 + lane] = tg[c];
          red[((wave * NT + c) * 2 + 1) * 64 + lane] = tu[c];
        }
      }
      __syncthreads();
      if (ks == 0) {
        for (int s2 = 1; s2 < KS; ++s2)
#pragma unroll
          for (int c = 0; c < NT; ++c) {
            const f32x4 g2 = red[(((wave + s2) * NT + c) * 2 + 0) * 64 + lane];
            const f32x4 u2 = red[(((wave + s2) * NT + c) * 2 + 1) * 64 + lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              tg[c][i] = tg[c][i] + g2[i];
              tu[c][i] = tu[c][i] + u2[i];
            }
          }
      }
    }
    if (ks == 0) {
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        if (!valid[c]) continue;
        uint32_t hb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          hb[i] = f32_to_bf16_rne(silu_f32(tg[c][i]) * tu[c][i]);
        uint2 pk;
        pk.x = hb[0] | (hb[1] << 16);
        pk.y = hb[2] | (hb[3] << 16);
        *(uint2*)(h + (size_t)(tl.r0 + 16 * c + col) * f + n0 + 4 * kq) = pk;
      }
    }
  }
}

// ------------------------------------------------- gate / up, one token
// The K-split gate/up of a one-token batch (every tile holds one pair
// unless the caller's top-k ids repeat an expert) streams its codes through
// LDS: direct-to-LDS loads hold no registers, so each wave keeps three
// groups of codes in flight at four waves per SIMD (the register kernel
// above holds one), and the token's activations for the wave's K slice are
// staged once per item instead of loaded per group.  Each step refills the
// slot it has just read, with the group three ahead (groups past the slice
// re-read its last group), so that the loads in flight after any step's
// codes are exactly the two later groups' four: a step waits with
// vmcnt(4) for its codes and reads its slot, scales and activations with
// inline LDS reads that wait for themselves (the compiler would wait for
// every direct-to-LDS load in flight before any LDS read it emits, which
// leaves nothing in flight).  Work items, operands, MFMA order and the
// K-slice reduction are those of the kernel above (the same fp32
// results).  A tile of several pairs (repeated ids) reads its columns'
// activations from global memory instead.
constexpr int kT1MaxGps = 8;  // groups per K slice that the staged activations hold

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

template <int KS, bool kLg>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8)))
void gateup_w4_decode_t1(const uint16_t* __restrict__ x, const int32_t* __restrict__ offsets,
                         const int32_t* __restrict__ sorted_pair, int E, int k, int P,
                         int d, int f, const uint8_t* __restrict__ codes,
                         const uint16_t* __restrict__ scales, uint16_t* __restrict__ h,
                         const float* __restrict__ logits, int32_t* __restrict__ idx_out,
                         float* __restrict__ w_out, int32_t* __restrict__ offsets_out,
                         int32_t* __restrict__ sorted_pair_out,
                         int32_t* __restrict__ pair_pos_out) {
  constexpr int RT = 4 / KS;
  constexpr int kSlot = 2 * kTileGroupBytes;  // gate and up tiles of one group
  // [slot][wave] codes in flight
  __shared__ __attribute__((aligned(16))) uint8_t ring[3 * 4 * kSlot];
  // [wave][kT1MaxGps * 128] activations of the wave's K slice; after the
  // group loop the K-slice partial sums [wave][2][64] (f32x4) of the reduction
  __shared__ __attribute__((aligned(16))) uint16_t xsl[4 * kT1MaxGps * 128];
  extern __shared__ int32_t lds_i[];
  const int G = d >> 7, RG = f / (16 * RT);
  int32_t* off_lds = lds_i;
  int32_t* sp_lds = lds_i + ((E + 1 + 3) & ~3);
  float* sc_lds = (float*)(sp_lds + ((min(P, kPairsInLds) + 3) & ~3));  // [2][G][16 RT]
  const int np = ks_route<kLg>(offsets, sorted_pair, E, k, P, logits, idx_out, w_out,
                               offsets_out, sorted_pair_out, pair_pos_out, off_lds, sp_lds,
                               (int32_t*)(sc_lds + 2 * G * 16 * RT));
  f32x4* red = (f32x4*)xsl;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int rt = wave / KS, ks = wave % KS;
  const int gps = G / KS;  // the launch requires G % KS == 0 and gps <= kT1MaxGps
  const int gb = ks * gps;
  const bf16x8 negoff = bf16_splat(kBf16NegOff);
  uint8_t* const slot0 = ring + wave * kSlot;  // slot j at + j * 4 * kSlot
  uint16_t* const xw = xsl + wave * (kT1MaxGps * 128);
  // LDS byte addresses of the lane's reads: its 16 bytes of a slot, its
  // activations of group gb, its scales of group 0 (gate; up G * 16 RT
  // floats further)
  const uint32_t a_slot = lds_addr(slot0) + 16 * lane;
  const uint32_t a_x = lds_addr(xw) + 2 * (32 * kq);
  const uint32_t a_sc = lds_addr(sc_lds) + 4 * (16 * rt + 4 * kq);
  const uint32_t sc_up = 4 * (G * 16 * RT);

  for (int w = blockIdx.x;; w += gridDim.x) {
    TileInfo tl;
    if (!find_tile(off_lds, E, 16, w / RG, tl)) break;
    const int nb = (w % RG) * 16 * RT, n0 = nb + 16 * rt;
    const size_t erow = (size_t)tl.e * 2 * f;
    // the lane's column (past the tile's end: its first row, not stored)
    const int jj = col < tl.cnt ? col : 0;
    const int pcol = np ? sp_lds[tl.r0 + jj] : sorted_pair[tl.r0 + jj];
    const int p0 = __shfl(pcol, 0, kWave);
    const uint16_t* xrow = x + (size_t)(p0 / k) * d;
    const uint16_t* xr = x + (size_t)(pcol / k) * d + 32 * kq;
    const uint8_t* cg = codes + (erow + n0) * (size_t)(d >> 1) + 64 * col + 16 * kq;
    const uint8_t* cu = cg + (size_t)f * (d >> 1);
    // group g (clamped to the slice) of gate and up codes into slot j
    auto dma = [&](int j, int g) {
      g = min(g, gb + gps - 1);
      uint8_t* dst = slot0 + j * 4 * kSlot;
      __builtin_amdgcn_global_load_lds(cg + kTileGroupBytes * g,
                                       (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(cu + kTileGroupBytes * g,
                                       (__attribute__((address_space(3))) void*)(dst + kTileGroupBytes),
                                       16, 0, 0);
    };

    // scales as in the kernel above
    const int nsc = 2 * 16 * RT * G;
    const bool vsc = (G & 3) == 0 && nsc <= 4 * 256 && ((uintptr_t)scales & 7) == 0;
    const int scc = min((int)threadIdx.x, nsc / 4 - 1);
    const int sc_m = (4 * scc) / (16 * RT * G), sc_rem = 4 * scc - sc_m * 16 * RT * G;
    uint2 scv = {0u, 0u};
    if (vsc)
      scv = *(const uint2*)(scales + (erow + nb + (size_t)sc_m * f) * G + sc_rem);
    // Every wave is done with the previous item's scales and reduction
    // (xsl): their LDS reads have returned.  A bare barrier: a fence would
    // wait for the scale load.
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    {
      // the token's activations of the slice in element order (2 KiB: lane
      // l of load i brings elements 8 (l + 64 i) .. + 7 of the slice;
      // elements past it repeat its last 8 and are never read)
      const int lim = (gb + gps) * 128 - 8;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int el = min(gb * 128 + 8 * (lane + 64 * i), lim);
        __builtin_amdgcn_global_load_lds(xrow + el,
                                         (__attribute__((address_space(3))) void*)(xw + 512 * i),
                                         16, 0, 0);
      }
    }
    dma(0, gb);
    dma(1, gb + 1);
    dma(2, gb + 2);
    if (vsc) {
      if ((int)threadIdx.x < nsc / 4) {
        const int r = sc_rem / G, g0 = sc_rem % G;
        float* dd = sc_lds + (sc_m * G + g0) * (16 * RT) + r;
        dd[0] = f16_bits_to_f32(scv.x & 0xFFFFu);
        dd[16 * RT] = f16_bits_to_f32(scv.x >> 16);
        dd[32 * RT] = f16_bits_to_f32(scv.y & 0xFFFFu);
        dd[48 * RT] = f16_bits_to_f32(scv.y >> 16);
      }
    } else {
      stage_scales_f32(scales + (erow + nb) * G, (size_t)f, 2, 16 * RT, G, sc_lds);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the scales are written
    __builtin_amdgcn_s_barrier();

    f32x4 tg = {0, 0, 0, 0}, tu = {0, 0, 0, 0};
    auto run = [&](auto one_c) {
      constexpr bool kOne = decltype(one_c)::value;
      for (int i = 0; i < gps; ++i) {
        const int gi = gb + i, j = i % 3;
        const uint32_t as = a_slot + j * 4 * kSlot, ac = a_sc + 4 * (gi * 16 * RT);
        u32x4 qg, qu;
        f32x4 sg, su;
        bf16x8 xp[4];
        if constexpr (kOne) {
          const uint32_t ax = a_x + 256 * i;
          asm volatile(
              "s_waitcnt vmcnt(4)\n\t"
              "ds_read_b128 %0, %8\n\t"
              "ds_read_b128 %1, %8 offset:1024\n\t"
              "ds_read_b128 %2, %9\n\t"
              "ds_read_b128 %3, %10\n\t"
              "ds_read_b128 %4, %11\n\t"
              "ds_read_b128 %5, %11 offset:16\n\t"
              "ds_read_b128 %6, %11 offset:32\n\t"
              "ds_read_b128 %7, %11 offset:48\n\t"
              "s_waitcnt lgkmcnt(0)"
              : "=&v"(qg), "=&v"(qu), "=&v"(sg), "=&v"(su), "=&v"(xp[0]), "=&v"(xp[1]),
                "=&v"(xp[2]), "=&v"(xp[3])
              : "v"(as), "v"(ac), "v"(ac + sc_up), "v"(ax)
              : "memory");
        } else {
          asm volatile(
              "s_waitcnt vmcnt(4)\n\t"
              "ds_read_b128 %0, %4\n\t"
              "ds_read_b128 %1, %4 offset:1024\n\t"
              "ds_read_b128 %2, %5\n\t"
              "ds_read_b128 %3, %6\n\t"
              "s_waitcnt lgkmcnt(0)"
              : "=&v"(qg), "=&v"(qu), "=&v"(sg), "=&v"(su)
              : "v"(as), "v"(ac), "v"(ac + sc_up)
              : "memory");
#pragma unroll
          for (int q = 0; q < 4; ++q) xp[q] = *(const bf16x8*)(xr + 128 * gi + 8 * q);
        }
        f32x4 seed = {0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < 4; ++q) seed = mfma16(negoff, xp[q], seed);
        tile_group(xp, seed, qg, sg, tg);
        tile_group(xp, seed, qu, su, tu);
        dma(j, gi + 3);
      }
    };
    if (tl.cnt == 1)
      run(std::true_type{});
    else
      run(std::false_type{});
    // the re-reads past the slice land before xsl and the slots are reused
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    if (KS > 1) {
      if (ks > 0) {
        red[(wave * 2 + 0) * 64 + lane] = tg;
        red[(wave * 2 + 1) * 64 + lane] = tu;
      }
      __syncthreads();
      if (ks == 0) {
        for (int s2 = 1; s2 < KS; ++s2) {
          const f32x4 g2 = red[((wave + s2) * 2 + 0) * 64 + lane];
          const f32x4 u2 = red[((wave + s2) * 2 + 1) * 64 + lane];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            tg[q] = tg[q] + g2[q];
            tu[q] = tu[q] + u2[q];
          }
        }
      }
    }
    if (ks == 0 && col < tl.cnt) {
      uint32_t hb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) hb[q] = f32_to_bf16_rne(silu_f32(tg[q]) * tu[q]);
      uint2 pk;
      pk.x = hb[0] | (hb[1] << 16);
      pk.y = hb[2] | (hb[3] << 16);
      *(uint2*)(h + (size_t)(tl.r0 + col) * f + n0 + 4 * kq) = pk;
    }
  }
}

// ------------------------------------------------------------------ down
template <int KS, int NT, int kDepth, int kWaves>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWaves, 8)))
void down_w4_decode(const uint16_t* __restrict__ h, const int32_t* __restrict__ offsets,
                    int E, int d, int f, const uint8_t* __restrict__ codes,
                    const uint16_t* __restrict__ scales, float* __restrict__ y) {
  constexpr int RT = 4 / KS;
  extern __shared__ int32_t lds_i[];
  const int G = f >> 7, RG = d / (16 * RT);
  int32_t* off_lds = lds_i;
  float* sc_lds = (float*)(lds_i + ((E + 1 + 3) & ~3));  // [G][16 RT]
  f32x4* red = (f32x4*)(sc_lds + G * 16 * RT);           // [4][NT][64]
  for (int i = threadIdx.x; i <= E; i += blockDim.x) off_lds[i] = offsets[i];
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int rt = wave / KS, ks = wave % KS;
  const int gps = (G + KS - 1) / KS;
  const int gb = ks * gps, ge = min(G, gb + gps);
  const bf16x8 negoff = bf16_splat(kBf16NegOff);

  for (int w = blockIdx.x;; w += gridDim.x) {
    TileInfo tl;
    if (!find_tile(off_lds, E, 16 * NT, w / RG, tl)) break;
    const int mb = (w % RG) * 16 * RT, m0 = mb + 16 * rt;
    const size_t erow = (size_t)tl.e * d;
    const int nch = (tl.cnt + 15) >> 4;

    const uint16_t* hr[NT];  // columns past the tile read its first row
    bool valid[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      const int j = 16 * c + col;
      valid[c] = j < tl.cnt;
      hr[c] = h + (size_t)(tl.r0 + (valid[c] ? j : 0)) * f + 32 * kq;
    }
    const uint8_t* cd = codes + (erow + m0) * (size_t)(f >> 1) + 64 * col + 16 * kq;

    u32x4 q[kDepth], hv[kDepth][NT][4];
    auto load = [&](int g, u32x4& a, u32x4 (&v)[NT][4]) {
      a = __builtin_nontemporal_load((const u32x4*)(cd + kTileGroupBytes * g));
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        if (c >= nch) break;
        const uint16_t* hg = hr[c] + 128 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[c][j] = *(const u32x4*)(hg + 8 * j);
      }
    };
#pragma unroll
    for (int i = 0; i < kDepth; ++i)
      if (gb + i < ge) load(gb + i, q[i], hv[i]);

    __syncthreads();
    stage_scales_f32(scales + (erow + mb) * G, 0, 1, 16 * RT, G, sc_lds);
    __syncthreads();

    f32x4 acc[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[c] = f32x4{0, 0, 0, 0};
    for (int g = gb; g < ge; g += kDepth) {
#pragma unroll
      for (int i = 0; i < kDepth; ++i) {
        const int gi = g + i;
        if (gi >= ge) break;
        const f32x4 sv = *(const f32x4*)(sc_lds + gi * (16 * RT) + 16 * rt + 4 * kq);
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          if (c >= nch) break;
          bf16x8 hp[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) hp[j] = __builtin_bit_cast(bf16x8, hv[i][c][j]);
          f32x4 seed = {0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < 4; ++j) seed = mfma16(negoff, hp[j], seed);
          tile_group(hp, seed, q[i], sv, acc[c]);
        }
        if (gi + kDepth < ge) load(gi + kDepth, q[i], hv[i]);
      }
    }

    if (KS > 1) {
      if (ks > 0) {
#pragma unroll
        for (int c = 0; c < NT; ++c) red[(wave * NT + c) * 64 + lane] = acc[c];
      }
      __syncthreads();
      if (ks == 0) {
        for (int s2 = 1; s2 < KS; ++s2)
#pragma unroll
          for (int c = 0; c < NT; ++c) {
            const f32x4 v = red[((wave + s2) * NT + c) * 64 + lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[c][i] = acc[c][i] + v[i];
          }
      }
    }
    if (ks == 0) {
#pragma unroll
      for (int c = 0; c < NT; ++c)
        if (valid[c])
          *(f32x4*)(y + (size_t)(tl.r0 + 16 * c + col) * d + m0 + 4 * kq) = acc[c];
    }
  }
}



// ------------------------------------------- single K slice, one token tile
// When every wave streams the whole K range of its own 16-feature row tile
// (KS = 1, tiles of up to 16 pairs), the four waves of a block share one
// token tile.  The block then stages each 128-group of the tile's
// activation rows in LDS once (one 16-byte piece per thread), and the waves
// read their B fragments from there.  Compared with per-wave activation
// loads this cuts activation registers by four and leaves the global-load
// counter to the codes alone, so the code stream can run kDQ groups ahead
// of the MFMAs.  The arithmetic (operands,
// MFMA order, scaling) is the same as in the kernels above.
// The group loop keeps every global load unconditional (addresses of rows
// past the tile, and of groups past the end, are clamped to valid ones) and
// refills every slot in its steady state without a branch, so the compiler's
// wait before each use counts exactly the loads issued after it: kDQ groups
// stay in flight across the loop edge.
// kRT row tiles per wave and matrix: the item covers 64 kRT features, wave w
// those at 16 (w + 4 r), r < kRT, of its gate and up matrices, all fed by
// one staging of the tile's activations per 128-group.
template <int kDQ, int kWaves, int kSC, int kRT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWaves, 8)))
void gateup_w4_decode_lds(const uint16_t* __restrict__ x, const int32_t* __restrict__ offsets,
                          const int32_t* __restrict__ sorted_pair, int E, int k, int P,
                          int d, int f, const uint8_t* __restrict__ codes,
                          const uint16_t* __restrict__ scales, uint16_t* __restrict__ h) {
  extern __shared__ int32_t lds_i[];
  const int G = d >> 7, RG = f / (64 * kRT);
  int32_t* off_lds = lds_i;
  int32_t* sp_lds = lds_i + ((E + 1 + 3) & ~3);
  // [gate, up][kRT][G][64]
  float* sc_lds = (float*)(sp_lds + ((min(P, kPairsInLds) + 3) & ~3));
  uint16_t* xs = (uint16_t*)(sc_lds + 2 * kRT * G * 64);  // [2][16][kXRow]
  const int np = stage_routing(offsets, sorted_pair, E, P, off_lds, sp_lds);
  __syncthreads();

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int st_tok = tid >> 4, st_pc = tid & 15;  // staged row and 16-byte piece
  const bf16x8 negoff = bf16_splat(kBf16NegOff);
  const size_t rt_stride = (size_t)64 * (d >> 1);  // 64 rows apart

  for (int w = blockIdx.x;; w += gridDim.x) {
    TileInfo tl;
    if (!find_tile(off_lds, E, 16, w / RG, tl)) break;
    const int nb = (w % RG) * 64 * kRT;
    const size_t erow = (size_t)tl.e * 2 * f;
    // rows past the tile stage a copy of its first row (never stored)
    const int sj = tl.r0 + (st_tok < tl.cnt ? st_tok : 0);
    const int sp = np ? sp_lds[sj] : sorted_pair[sj];
    // take the routing value here, before any weight load is issued: a wait
    // for it after those loads would also wait for them
    asm volatile("" ::"v"(sp) : "memory");
    const uint16_t* xsrc = x + (size_t)(sp / k) * d + 8 * st_pc;
    const uint8_t* cg = codes + (erow + nb + 16 * wave) * (size_t)(d >> 1) + 64 * col + 16 * kq;
    const uint8_t* cu = cg + (size_t)f * (d >> 1);

    u32x4 qg[kDQ][kRT], qu[kDQ][kRT], xv[kDQ];
    auto load = [&](int g, int i) {
      xv[i] = *(const u32x4*)(xsrc + 128 * g);
#pragma unroll
      for (int r = 0; r < kRT; ++r) {
        qg[i][r] = __builtin_nontemporal_load((const u32x4*)(cg + r * rt_stride + kTileGroupBytes * g));
        qu[i][r] = __builtin_nontemporal_load((const u32x4*)(cu + r * rt_stride + kTileGroupBytes * g));
      }
    };
    // the previous item's last barrier precedes these LDS writes; the first
    // barrier of the group loop orders them before any read.  Scale rows of
    // one matrix are consecutive: kRT "matrices" of 64 rows each.
    ScaleStage<kRT, kSC ? kSC : 1> ssg, ssu;
    if (kSC) {
      ssg.fetch(scales + (erow + nb) * G, 64, G);
      ssu.fetch(scales + (erow + f + nb) * G, 64, G);
    }
    __builtin_amdgcn_sched_barrier(0);  // scales first: their wait skips the codes
#pragma unroll
    for (int i = 0; i < kDQ; ++i) load(i < G ? i : G - 1, i);
    __builtin_amdgcn_sched_barrier(0);
    if (kSC) {
      ssg.store(G, sc_lds);
      ssu.store(G, sc_lds + kRT * G * 64);
    } else {
      for (int r = 0; r < kRT; ++r) {
        stage_scales_rows64<1>(scales + (erow + nb + 64 * r) * G, 0, G, sc_lds + r * G * 64);
        stage_scales_rows64<1>(scales + (erow + f + nb + 64 * r) * G, 0, G,
                               sc_lds + (kRT + r) * G * 64);
      }
    }

    f32x4 tg[kRT], tu[kRT];
#pragma unroll
    for (int r = 0; r < kRT; ++r) tg[r] = tu[r] = f32x4{0, 0, 0, 0};
    auto step = [&](int gi, int i) {
      // slot gi & 1 was last read in step gi - 2, before the barrier of step gi - 1
      uint16_t* slot = xs + (gi & 1) * 16 * kXRow;
      *(u32x4*)(slot + st_tok * kXRow + 8 * st_pc) = xv[i];
      __syncthreads();
      bf16x8 xp[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) xp[j] = *(const bf16x8*)(slot + col * kXRow + 32 * kq + 8 * j);
      f32x4 seed = {0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 4; ++j) seed = mfma16(negoff, xp[j], seed);
#pragma unroll
      for (int r = 0; r < kRT; ++r) {
        const f32x4 sg = *(const f32x4*)(sc_lds + (r * G + gi) * 64 + 16 * wave + 4 * kq);
        const f32x4 su =
            *(const f32x4*)(sc_lds + ((kRT + r) * G + gi) * 64 + 16 * wave + 4 * kq);
        tile_group(xp, seed, qg[i][r], sg, tg[r]);
        tile_group(xp, seed, qu[i][r], su, tu[r]);
      }
    };
    // steady state: slot i is refilled right after its codes are used (the
    // new loads reuse its registers: no copy, hence no wait, at the edge)
    int g = 0;
    for (; g + 2 * kDQ <= G; g += kDQ) {
#pragma unroll
      for (int i = 0; i < kDQ; ++i) {
        step(g + i, i);
        load(g + i + kDQ, i);
        // keep the refill ahead of the next step's waits
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the last (fewer than 2 kDQ) groups
#pragma unroll
    for (int i = 0; i < kDQ; ++i) {
      if (g + i >= G) break;
      step(g + i, i);
      if (g + i + kDQ < G) load(g + i + kDQ, i);
    }
#pragma unroll
    for (int i = 0; i < kDQ; ++i)
      if (g + kDQ + i < G) step(g + kDQ + i, i);

    if (col < tl.cnt) {
#pragma unroll
      for (int r = 0; r < kRT; ++r) {
        uint32_t hb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hb[i] = f32_to_bf16_rne(silu_f32(tg[r][i]) * tu[r][i]);
        uint2 pk;
        pk.x = hb[0] | (hb[1] << 16);
        pk.y = hb[2] | (hb[3] << 16);
        *(uint2*)(h + (size_t)(tl.r0 + col) * f + nb + 16 * (wave + 4 * r) + 4 * kq) = pk;
      }
    }
    __syncthreads();  // the next item rewrites the scales and the slots
  }
}

// Work item = (token tile of up to 16 pairs, 64 kRT output rows): wave w
// streams the kRT row tiles at rows 16 (w + 4 r), r < kRT, of the item, all
// fed by one staging of the tile's h per 128-group (the h staging, its
// barrier and the seed MFMAs are shared by kRT row tiles); kDQ groups of
// codes per row tile stay in flight.
template <int kDQ, int kWaves, int kSC, int kRT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWaves, 8)))
void down_w4_decode_lds(const uint16_t* __restrict__ h, const int32_t* __restrict__ offsets,
                        int E, int d, int f, const uint8_t* __restrict__ codes,
                        const uint16_t* __restrict__ scales, float* __restrict__ y) {
  extern __shared__ int32_t lds_i[];
  const int G = f >> 7, RG = d / (64 * kRT);
  int32_t* off_lds = lds_i;
  float* sc_lds = (float*)(lds_i + ((E + 1 + 3) & ~3));  // [kRT][G][64]
  uint16_t* xs = (uint16_t*)(sc_lds + kRT * G * 64);     // [2][16][kXRow]
  for (int i = threadIdx.x; i <= E; i += blockDim.x) off_lds[i] = offsets[i];
  __syncthreads();

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int st_tok = tid >> 4, st_pc = tid & 15;
  const bf16x8 negoff = bf16_splat(kBf16NegOff);

  for (int w = blockIdx.x;; w += gridDim.x) {
    TileInfo tl;
    if (!find_tile(off_lds, E, 16, w / RG, tl)) break;
    const int mb = (w % RG) * 64 * kRT;
    const size_t erow = (size_t)tl.e * d;
    const uint16_t* hsrc = h + (size_t)(tl.r0 + (st_tok < tl.cnt ? st_tok : 0)) * f + 8 * st_pc;
    const uint8_t* cd = codes + (erow + mb + 16 * wave) * (size_t)(f >> 1) + 64 * col + 16 * kq;
    const size_t rt_stride = (size_t)64 * (f >> 1);  // 64 rows apart

    u32x4 q[kDQ][kRT], hv[kDQ];
    auto load = [&](int g, int i) {
      hv[i] = *(const u32x4*)(hsrc + 128 * g);
#pragma unroll
      for (int r = 0; r < kRT; ++r)
        q[i][r] = __builtin_nontemporal_load((const u32x4*)(cd + r * rt_stride + kTileGroupBytes * g));
    };
    // scale rows mb .. mb + 64 kRT - 1 are consecutive: kRT "matrices" of
    // 64 rows, 64 rows apart
    ScaleStage<kRT, kSC ? kSC : 1> sst;
    if (kSC) sst.fetch(scales + (erow + mb) * G, 64, G);
    __builtin_amdgcn_sched_barrier(0);  // scales first: their wait skips the codes
#pragma unroll
    for (int i = 0; i < kDQ; ++i) load(i < G ? i : G - 1, i);
    __builtin_amdgcn_sched_barrier(0);
    if (kSC)
      sst.store(G, sc_lds);
    else
      for (int r = 0; r < kRT; ++r)
        stage_scales_rows64<1>(scales + (erow + mb + 64 * r) * G, 0, G, sc_lds + r * G * 64);

    f32x4 acc[kRT];
#pragma unroll
    for (int r = 0; r < kRT; ++r) acc[r] = f32x4{0, 0, 0, 0};
    auto step = [&](int gi, int i) {
      uint16_t* slot = xs + (gi & 1) * 16 * kXRow;
      *(u32x4*)(slot + st_tok * kXRow + 8 * st_pc) = hv[i];
      __syncthreads();
      bf16x8 xp[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) xp[j] = *(const bf16x8*)(slot + col * kXRow + 32 * kq + 8 * j);
      f32x4 seed = {0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < 4; ++j) seed = mfma16(negoff, xp[j], seed);
#pragma unroll
      for (int r = 0; r < kRT; ++r) {
        const f32x4 sv = *(const f32x4*)(sc_lds + (r * G + gi) * 64 + 16 * wave + 4 * kq);
        tile_group(xp, seed, q[i][r], sv, acc[r]);
      }
    };
    int g = 0;
    for (; g + 2 * kDQ <= G; g += kDQ) {
#pragma unroll
      for (int i = 0; i < kDQ; ++i) {
        step(g + i, i);
        load(g + i + kDQ, i);
        // keep the refill ahead of the next step's waits
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int i = 0; i < kDQ; ++i) {
      if (g + i >= G) break;
      step(g + i, i);
      if (g + i + kDQ < G) load(g + i + kDQ, i);
    }
#pragma unroll
    for (int i = 0; i < kDQ; ++i)
      if (g + kDQ + i < G) step(g + kDQ + i, i);

    if (col < tl.cnt) {
#pragma unroll
      for (int r = 0; r < kRT; ++r)
        *(f32x4*)(y + (size_t)(tl.r0 + col) * d + mb + 16 * (wave + 4 * r) + 4 * kq) = acc[r];
    }
    __syncthreads();
  }
}

// kDepth: 128-groups of codes + activations in flight per wave; kWaves:
// the occupancy the register allocation is held to (measured on MI355X:
// occupancy matters more than prefetch depth, and spilling variants lose;
// the single-tile K-split gate/up at three waves per SIMD was 33 % slower
// than at four).
template <int KS, int NT> constexpr int gu_depth() { return 1; }
template <int KS, int NT> constexpr int gu_waves() { return NT == 1 ? 4 : 2; }
template <int KS, int NT> constexpr int dn_depth() { return NT == 1 ? 2 : 1; }
template <int KS, int NT> constexpr int dn_waves() { return NT == 1 ? 4 : 2; }

template <int KS, int NT>
void launch_gu_pair(const FfnArgs& a, uint16_t* h, long long P, hipStream_t s) {
  constexpr int RT = 4 / KS;
  const int tok = 16 * NT;
  const long long mt = (P + tok - 1) / tok + (P < a.E ? P : a.E);
  const size_t off_b = sizeof(int32_t) * ((a.E + 1 + 3) & ~3);
  const long long cap = 256LL * 8;
  const int G = a.d / 128;
  const long long work = mt * (a.f / (16 * RT));
  const int grid = (int)(work < cap ? work : cap);
  const size_t lds = off_b + sizeof(int32_t) * ((std::min<long long>(P, kPairsInLds) + 3) & ~3) +
                     sizeof(float) * 2 * G * 16 * RT + sizeof(f32x4) * 4 * NT * 2 * 64 +
                     (a.logits ? sizeof(int32_t) * (128 + a.E) : 0);
  auto kern = a.logits ? gateup_w4_decode<KS, NT, gu_depth<KS, NT>(), gu_waves<KS, NT>(), true>
                       : gateup_w4_decode<KS, NT, gu_depth<KS, NT>(), gu_waves<KS, NT>(), false>;
  launch_k(kern, dim3(grid), dim3(256), lds, s, a.ev[0], a.ev[1], a.x, a.offsets,
           a.sorted_pair, a.E, a.k, (int)P, a.d, a.f, a.gu_codes, a.gu_scales, h, a.logits,
           a.topk_idx_out, a.topk_w_out, a.offsets_out, a.sorted_pair_out, a.pair_pos_out);
}

// The one-token K-split gate/up (LDS-streamed codes) applies when every K
// slice is full and fits the staged activations.
static bool gu_t1_applies(const FfnArgs& a, int KS) {
  const int G = a.d / 128;
  return a.T == 1 && (KS == 2 || KS == 4) && G % KS == 0 && G / KS <= kT1MaxGps;
}

template <int KS>
void launch_gu_t1(const FfnArgs& a, uint16_t* h, long long P, hipStream_t s) {
  constexpr int RT = 4 / KS;
  const long long mt = (P + 15) / 16 + (P < a.E ? P : a.E);
  const size_t off_b = sizeof(int32_t) * ((a.E + 1 + 3) & ~3);
  const long long cap = 256LL * 8;
  const int G = a.d / 128;
  const long long work = mt * (a.f / (16 * RT));
  const int grid = (int)(work < cap ? work : cap);
  const size_t lds = off_b + sizeof(int32_t) * ((std::min<long long>(P, kPairsInLds) + 3) & ~3) +
                     sizeof(float) * 2 * G * 16 * RT +
                     (a.logits ? sizeof(int32_t) * (128 + a.E) : 0);
  auto kern = a.logits ? gateup_w4_decode_t1<KS, true> : gateup_w4_decode_t1<KS, false>;
  launch_k(kern, dim3(grid), dim3(256), lds, s, a.ev[0], a.ev[1], a.x, a.offsets,
           a.sorted_pair, a.E, a.k, (int)P, a.d, a.f, a.gu_codes, a.gu_scales, h, a.logits,
           a.topk_idx_out, a.topk_w_out, a.offsets_out, a.sorted_pair_out, a.pair_pos_out);
}

template <int KS, int NT>
void launch_dn_pair(const FfnArgs& a, uint16_t* h, long long P, hipStream_t s) {
  constexpr int RT = 4 / KS;
  const int tok = 16 * NT;
  const long long mt = (P + tok - 1) / tok + (P < a.E ? P : a.E);
  const size_t off_b = sizeof(int32_t) * ((a.E + 1 + 3) & ~3);
  const long long cap = 256LL * 8;
  const int G = a.f / 128;
  const long long work = mt * (a.d / (16 * RT));
  const int grid = (int)(work < cap ? work : cap);
  const size_t lds = off_b + sizeof(float) * G * 16 * RT + sizeof(f32x4) * 4 * NT * 64;
  launch_k(down_w4_decode<KS, NT, dn_depth<KS, NT>(), dn_waves<KS, NT>()>, dim3(grid),
           dim3(256), lds, s, a.ev[2], a.ev[3], h, a.offsets, a.E, a.d, a.f, a.dn_codes,
           a.dn_scales, a.y);
}

// Code groups in flight and occupancy of the LDS-staged kernels (measured
// on MI355X: deeper code prefetch in gate/up costs the fourth wave).
constexpr int kGuDQ = 2, kGuWaves = 4, kDnDQ = 4, kDnWaves = 4;
// row tiles per wave of the single-slice down kernel, and its code groups in
// flight per row tile
constexpr int kDnLdsRT = 2, kDnLdsDQ = 2;
// the same for the single-slice gate/up kernel
constexpr int kGuLdsRT = 1, kGuLdsDQ = 2;
// row tiles per wave of the expert-major down kernel: one h staging per
// group serves four row tiles (measured at the OLMoE decode shape: 16.7 us
// with one, 14.5 with two, 14.1 with four, 18.5 with eight; one group of
// codes in flight per row tile, deeper was slower)
constexpr int kDnRT = 4;

template <int kDQ, int kRT>
void launch_gu_lds_rt(const FfnArgs& a, uint16_t* h, long long P, hipStream_t s) {
  const long long mt = (P + 15) / 16 + (P < a.E ? P : a.E);
  const size_t off_b = sizeof(int32_t) * ((a.E + 1 + 3) & ~3);
  const size_t xs_b = sizeof(uint16_t) * 2 * 16 * kXRow;
  const long long cap = 256LL * 8;
  const int G = a.d / 128;
  const long long work = mt * (a.f / (64 * kRT));
  const int grid = (int)(work < cap ? work : cap);
  const size_t lds = off_b + sizeof(int32_t) * ((std::min<long long>(P, kPairsInLds) + 3) & ~3) +
                     sizeof(float) * 2 * kRT * G * 64 + xs_b;
  const int sc = scale_chunks(kRT, G, a.gu_scales);
  auto kern = sc == 1   ? gateup_w4_decode_lds<kDQ, kGuWaves, 1, kRT>
              : sc == 2 ? gateup_w4_decode_lds<kDQ, kGuWaves, 2, kRT>
              : sc == 4 ? gateup_w4_decode_lds<kDQ, kGuWaves, 4, kRT>
                        : gateup_w4_decode_lds<kDQ, kGuWaves, 0, kRT>;
  launch_k(kern, dim3(grid), dim3(256), lds, s, a.ev[0], a.ev[1], a.x, a.offsets,
           a.sorted_pair, a.E, a.k, (int)P, a.d, a.f, a.gu_codes, a.gu_scales, h);
}

void launch_gu_lds(const FfnArgs& a, uint16_t* h, long long P, hipStream_t s) {
  if (a.f % (64 * kGuLdsRT) == 0)
    launch_gu_lds_rt<kGuLdsDQ, kGuLdsRT>(a, h, P, s);
  else
    launch_gu_lds_rt<kGuDQ, 1>(a, h, P, s);
}

template <int kDQ, int kRT>
void launch_dn_lds_rt(const FfnArgs& a, uint16_t* h, long long P, hipStream_t s) {
  const long long mt = (P + 15) / 16 + (P < a.E ? P : a.E);
  const size_t off_b = sizeof(int32_t) * ((a.E + 1 + 3) & ~3);
  const size_t xs_b = sizeof(uint16_t) * 2 * 16 * kXRow;
  const long long cap = 256LL * 8;
  const int G = a.f / 128;
  const long long work = mt * (a.d / (64 * kRT));
  const int grid = (int)(work < cap ? work : cap);
  const size_t lds = off_b + sizeof(float) * kRT * G * 64 + xs_b;
  const int sc = scale_chunks(kRT, G, a.dn_scales);
  auto kern = sc == 1   ? down_w4_decode_lds<kDQ, kDnWaves, 1, kRT>
              : sc == 2 ? down_w4_decode_lds<kDQ, kDnWaves, 2, kRT>
              : sc == 4 ? down_w4_decode_lds<kDQ, kDnWaves, 4, kRT>
                        : down_w4_decode_lds<kDQ, kDnWaves, 0, kRT>;
  launch_k(kern, dim3(grid), dim3(256), lds, s, a.ev[2], a.ev[3], h, a.offsets, a.E, a.d,
           a.f, a.dn_codes, a.dn_scales, a.y);
}

// kDnLdsRT row tiles per wave, unless that leaves fewer than two blocks per
// CU (a token or two: then one row tile per wave with kDnDQ groups in
// flight; measured at E = 256, T = 1: 11.8 -> 11.2 us, OLMoE-shaped T = 1:
// 6.2 -> 5.7 us; at E = 256, T = 64 two row tiles stay faster, 82.6 against
// 95.7 us).
void launch_dn_lds(const FfnArgs& a, uint16_t* h, long long P, hipStream_t s) {
  const long long mt = (P + 15) / 16 + (P < a.E ? P : a.E);
  const bool few = mt * (a.d / (64 * kDnLdsRT)) < 512;
  if (a.d % (64 * kDnLdsRT) == 0 && !few)
    launch_dn_lds_rt<kDnLdsDQ, kDnLdsRT>(a, h, P, s);
  else
    launch_dn_lds_rt<kDnDQ, 1>(a, h, P, s);
}
// ------------------------------------ expert-major, at most 16 tokens
// With at most 16 tokens every expert receives at most 16 pairs (a token's
// k experts are distinct), so each expert needs one token tile and a work
// item (expert e, 64 features) follows from blockIdx alone.  The gate/up
// block issues its first scale, code and activation loads (the rows of all
// T tokens) together with topk_idx and derives the grouping itself: ballots
// over the T*k pairs give expert e's slot range [r0, r0 + cnt) (pairs
// ordered by expert, then by pair index: the counting sort of the permute
// step) and the pair of each of its columns.  Block (e, 0) stores expert
// e's part of expert_offsets, sorted_pair and pair_pos.  h is kept per
// expert, [E][16][f] bf16, so the down block loads its rows without waiting
// for the grouping; its slot range comes from expert_offsets, loaded beside
// its first code loads.  Per group, operands and MFMA order are those of
// the LDS-staged kernels above (the same fp32 results).
// With kLg (E <= 64, k <= 16) the block takes the router logits [T][E]
// instead of topk_idx: e's rank among each token's logits says whether the
// token chose e (rank < k) and at which place (the pair t k + rank), which
// is all the block's columns need.  The grouping is finished by the down
// kernel from the per-expert counts and pair lists that the (e, 0) blocks
// store; block b < T also selects token b's top-k (one wave, while its first
// loads are in flight) and stores topk_idx and topk_w.  The routing launch
// thus only computes logits, over many more blocks than one per token.
constexpr int kEmMaxT = 16;

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// kW waves per block (4 or 8), one 16-feature row tile each: blocks of 16 kW
// features; every group of four waves stages the whole activation tile
// (waves 4-7 write the same values to the same places as waves 0-3).
template <int kDQ, int kWaves, int kSC, int kW, bool kLg>
__global__ __launch_bounds__(64 * kW) __attribute__((amdgpu_waves_per_eu(kWaves, 8)))
void gateup_w4_em(const uint16_t* __restrict__ x, const int32_t* __restrict__ topk_idx,
                  int T, int k, int E, int d, int f, const uint8_t* __restrict__ codes,
                  const uint16_t* __restrict__ scales, uint16_t* __restrict__ hE,
                  int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
                  int32_t* __restrict__ pair_pos, const float* __restrict__ logits,
                  int32_t* __restrict__ em_cnt, int32_t* __restrict__ em_list,
                  int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  static_assert(!kLg || kEmMaxT % kW == 0, "tokens per wave");
  constexpr int kTokW = kLg ? kEmMaxT / kW : 1;  // tokens whose top-k a wave selects
  constexpr int kRows = 16 * kW, kMat = kW / 4;  // 64-row scale chunks per matrix
  extern __shared__ int32_t lds_i[];
  __shared__ int32_t wcnt[kW][2];
  __shared__ int32_t colpair[kEmMaxT];
  const int G = d >> 7, RG = f / kRows, P = T * k;
  float* sc_lds = (float*)lds_i;                          // [gate, up][kMat][G][64]
  uint16_t* xs = (uint16_t*)(sc_lds + 2 * kMat * G * 64);  // [2][16][kXRow]

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int st_tok = (tid >> 4) & 15, st_pc = tid & 15;  // staged token row, 16-byte piece
  const bf16x8 negoff = bf16_splat(kBf16NegOff);
  const int e = blockIdx.x / RG, rg = blockIdx.x % RG;
  const int nb = rg * kRows, n0 = nb + 16 * wave;
  const int sc_g = ((wave >> 2) * G) * 64 + 16 * (wave & 3) + 4 * kq;  // gate scale slot
  const int sc_u = sc_g + kMat * G * 64;                              // up scale slot
  const size_t erow = (size_t)e * 2 * f;

  // t = 0: every pair's expert (or this wave's tokens' logits), then
  // scales, codes and activations
  int pe = -1;
  float lgv[kTokW];
  if constexpr (kLg) {
#pragma unroll
    for (int j = 0; j < kTokW; ++j) {
      const int t = wave + kW * j;
      lgv[j] = (t < T && lane < E) ? logits[(size_t)t * E + lane] : 0.0f;
    }
  } else {
    pe = tid < P ? topk_idx[tid] : -1;
  }
  const uint16_t* xsrc = x + (size_t)(st_tok < T ? st_tok : 0) * d + 8 * st_pc;
  const uint8_t* cg = codes + (erow + n0) * (size_t)(d >> 1) + 64 * col + 16 * kq;
  const uint8_t* cu = cg + (size_t)f * (d >> 1);
  u32x4 qg[kDQ], qu[kDQ], xv[kDQ];
  auto load = [&](int g, int i) {
    xv[i] = *(const u32x4*)(xsrc + 128 * g);
    qg[i] = __builtin_nontemporal_load((const u32x4*)(cg + kTileGroupBytes * g));
    qu[i] = __builtin_nontemporal_load((const u32x4*)(cu + kTileGroupBytes * g));
  };
  // scales: 4 waves take gate and up as two 64-row matrices; 8 or 16 waves
  // take gate then up as runs of kMat 64-row chunks
  const uint16_t* sc_src = scales + (erow + nb) * G;
  const size_t sc_stride = kW == 4 ? (size_t)f : 64;
  constexpr int kStageMat = kW == 4 ? 2 : kMat;
  ScaleStage<kStageMat, kSC ? kSC : 1> sst, sst2;
  if (kSC) {
    sst.fetch(sc_src, sc_stride, G);
    if (kW > 4) sst2.fetch(sc_src + (size_t)f * G, 64, G);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kDQ; ++i) load(i < G ? i : G - 1, i);
  __builtin_amdgcn_sched_barrier(0);
  if (kSC) {
    sst.store(G, sc_lds);
    if (kW > 4) sst2.store(G, sc_lds + kMat * G * 64);
  } else if (tid < 256) {
    stage_scales_rows64<kStageMat>(sc_src, sc_stride, G, sc_lds);
    if (kW > 4)
      stage_scales_rows64<kStageMat>(sc_src + (size_t)f * G, 64, G, sc_lds + kMat * G * 64);
  }

  int cnt = 0, xrow = 0;  // columns; staged row (token) of column col
  if constexpr (kLg) {
    __shared__ int32_t trank[kEmMaxT];  // e's place in token t's top-k, or -1
#pragma unroll
    for (int j = 0; j < kTokW; ++j) {
      const int t = wave + kW * j;
      if (t < T) {  // wave-uniform
        const int r = expert_rank64(lgv[j], E, e);
        if (lane == 0) trank[t] = r < k ? r : -1;
        if (t == (int)blockIdx.x)
          select_topk_radix64(lgv[j], E, k, idx_out + (size_t)t * k, w_out + (size_t)t * k,
                              nullptr);
      }
    }
    __syncthreads();
    // the columns are the tokens that chose e, in token (= pair) order
    const int tr = lane < T ? trank[lane] : -1;
    const uint64_t bm = __ballot(tr >= 0);
    cnt = __popcll(bm);
    if (rg == 0 && wave == 0) {
      if (tr >= 0) em_list[e * kEmMaxT + __popcll(bm & lanemask_lt())] = lane * k + tr;
      if (lane == 0) em_cnt[e] = cnt;
    }
    if (cnt == 0) return;  // block-uniform
    uint64_t mcol = bm;
    for (int i = 0; i < col && i + 1 < cnt; ++i) mcol &= mcol - 1;
    xrow = __ffsll((unsigned long long)mcol) - 1;
  } else {
    // the grouping of the pairs, as far as expert e is concerned
    const bool mine = pe == e;
    const bool below = (unsigned)pe < (unsigned)E && pe < e;
    const uint64_t bm = __ballot(mine), bb = __ballot(below);
    if (lane == 0) {
      wcnt[wave][0] = __popcll(bm);
      wcnt[wave][1] = __popcll(bb);
    }
    __syncthreads();
    int r0 = 0, rank = __popcll(bm & lanemask_lt());
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      cnt += wcnt[w][0];
      r0 += wcnt[w][1];
      rank += w < wave ? wcnt[w][0] : 0;
    }
    if (mine && rank < kEmMaxT) colpair[rank] = tid;
    if (rg == 0) {
      if (mine) {
        sorted_pair[r0 + rank] = tid;
        pair_pos[tid] = r0 + rank;
      }
      if (tid == 0) {
        offsets[e] = r0;
        if (e == E - 1) offsets[E] = r0 + cnt;
      }
    }
    __syncthreads();
    if (cnt == 0) return;  // block-uniform
    xrow = colpair[col < cnt ? col : 0] / k;
  }
  const int ncol = cnt < kEmMaxT ? cnt : kEmMaxT;

  f32x4 tg = {0, 0, 0, 0}, tu = {0, 0, 0, 0};
  auto step = [&](int gi, int i) {
    // slot gi & 1 was last read in step gi - 2, before the barrier of step gi - 1
    uint16_t* slot = xs + (gi & 1) * 16 * kXRow;
    *(u32x4*)(slot + st_tok * kXRow + 8 * st_pc) = xv[i];
    __syncthreads();
    bf16x8 xp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xp[j] = *(const bf16x8*)(slot + xrow * kXRow + 32 * kq + 8 * j);
    const f32x4 sg = *(const f32x4*)(sc_lds + sc_g + gi * 64);
    const f32x4 su = *(const f32x4*)(sc_lds + sc_u + gi * 64);
    f32x4 seed = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) seed = mfma16(negoff, xp[j], seed);
    tile_group(xp, seed, qg[i], sg, tg);
    tile_group(xp, seed, qu[i], su, tu);
  };
  // the first groups' loads were issued at the start (their one wait at the
  // loop entry covers loads issued together); each slot is refilled after use
  int g = 0;
  for (; g + 2 * kDQ <= G; g += kDQ) {
#pragma unroll
    for (int i = 0; i < kDQ; ++i) {
      step(g + i, i);
      load(g + i + kDQ, i);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int i = 0; i < kDQ; ++i) {
    if (g + i >= G) break;
    step(g + i, i);
    if (g + i + kDQ < G) load(g + i + kDQ, i);
  }
#pragma unroll
  for (int i = 0; i < kDQ; ++i)
    if (g + kDQ + i < G) step(g + kDQ + i, i);

  if (col < ncol) {
    uint32_t hb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hb[i] = f32_to_bf16_rne(silu_f32(tg[i]) * tu[i]);
    uint2 pk;
    pk.x = hb[0] | (hb[1] << 16);
    pk.y = hb[2] | (hb[3] << 16);
    *(uint2*)(hE + ((size_t)e * kEmMaxT + col) * f + n0 + 4 * kq) = pk;
  }
}

// Down, expert-major: block = (expert e, 64 kRT features); wave w owns the
// row tiles 64 r + 16 w (r < kRT) of the block, so one staging of h per
// group (and one seed) serves kRT row tiles of codes.  With kLg the slot
// range comes from the per-expert counts of the gate/up kernel (a wave sum
// over the experts below e) and the (e, 0) blocks store expert_offsets,
// sorted_pair and pair_pos from the experts' pair lists.
template <int kDQ, int kWaves, int kSC, int kRT, bool kLg>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWaves, 8)))
void down_w4_em(const uint16_t* __restrict__ hE, const int32_t* __restrict__ offsets,
                int E, int d, int f, const uint8_t* __restrict__ codes,
                const uint16_t* __restrict__ scales, float* __restrict__ y,
                const int32_t* __restrict__ em_cnt, const int32_t* __restrict__ em_list,
                int32_t* __restrict__ offsets_out, int32_t* __restrict__ sorted_pair,
                int32_t* __restrict__ pair_pos) {
  extern __shared__ int32_t lds_i[];
  constexpr int kRows = 64 * kRT;
  const int G = f >> 7, RG = d / kRows;
  float* sc_lds = (float*)lds_i;                      // [kRT][G][64]
  uint16_t* xs = (uint16_t*)(sc_lds + kRT * G * 64);  // [2][16][kXRow]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int st_tok = tid >> 4, st_pc = tid & 15;
  const bf16x8 negoff = bf16_splat(kBf16NegOff);
  const int e = blockIdx.x / RG, rg = blockIdx.x % RG;
  const int mb = rg * kRows;
  const size_t erow = (size_t)e * d;

  // t = 0: the slot range (or every expert's count and e's pair list),
  // scales, codes and all 16 rows of h (rows past the expert's count hold
  // stale values that feed only unstored columns)
  int lo = 0, hi = 0, cv = 0, pv = 0;
  if constexpr (kLg) {
    cv = lane < E ? em_cnt[lane] : 0;
    pv = em_list[e * kEmMaxT + (tid & (kEmMaxT - 1))];
  } else {
    lo = offsets[e];
    hi = offsets[e + 1];
  }
  const uint16_t* hsrc = hE + ((size_t)e * kEmMaxT + st_tok) * f + 8 * st_pc;
  const uint8_t* cd[kRT];
#pragma unroll
  for (int r = 0; r < kRT; ++r)
    cd[r] = codes + (erow + mb + 64 * r + 16 * wave) * (size_t)(f >> 1) + 64 * col + 16 * kq;
  u32x4 q[kDQ][kRT], hv[kDQ];
  auto load = [&](int g, int i) {
    hv[i] = *(const u32x4*)(hsrc + 128 * g);
#pragma unroll
    for (int r = 0; r < kRT; ++r) q[i][r] = __builtin_nontemporal_load((const u32x4*)(cd[r] + kTileGroupBytes * g));
  };
  ScaleStage<kRT, kSC ? kSC : 1> sst;
  if (kSC) sst.fetch(scales + (erow + mb) * G, 64, G);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kDQ; ++i) load(i < G ? i : G - 1, i);
  __builtin_amdgcn_sched_barrier(0);
  if (kSC)
    sst.store(G, sc_lds);
  else
    stage_scales_rows64<kRT>(scales + (erow + mb) * G, 64, G, sc_lds);
  if constexpr (kLg) {
    // sum of the counts below e (each at most 16) bit by bit with ballots
    int below = 0;
#pragma unroll
    for (int b = 0; b < 5; ++b)
      below += __popcll(__ballot(lane < e && ((cv >> b) & 1))) << b;
    lo = below;
    hi = lo + __builtin_amdgcn_readlane(cv, e);
    if (rg == 0) {
      if (tid < hi - lo) {
        sorted_pair[lo + tid] = pv;
        pair_pos[pv] = lo + tid;
      }
      if (tid == 0) {
        offsets_out[e] = lo;
        if (e == E - 1) offsets_out[E] = hi;
      }
    }
  }
  const int cnt = hi - lo;
  if (cnt <= 0) return;  // block-uniform
  const int ncol = cnt < kEmMaxT ? cnt : kEmMaxT;

  f32x4 acc[kRT];
#pragma unroll
  for (int r = 0; r < kRT; ++r) acc[r] = f32x4{0, 0, 0, 0};
  auto step = [&](int gi, int i) {
    uint16_t* slot = xs + (gi & 1) * 16 * kXRow;
    *(u32x4*)(slot + st_tok * kXRow + 8 * st_pc) = hv[i];
    __syncthreads();
    bf16x8 xp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xp[j] = *(const bf16x8*)(slot + col * kXRow + 32 * kq + 8 * j);
    f32x4 seed = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) seed = mfma16(negoff, xp[j], seed);
#pragma unroll
    for (int r = 0; r < kRT; ++r) {
      const f32x4 sv = *(const f32x4*)(sc_lds + (r * G + gi) * 64 + 16 * wave + 4 * kq);
      tile_group(xp, seed, q[i][r], sv, acc[r]);
    }
  };
  // the first groups' loads were issued at the start (their one wait at the
  // loop entry covers loads issued together); each slot is refilled after use
  int g = 0;
  for (; g + 2 * kDQ <= G; g += kDQ) {
#pragma unroll
    for (int i = 0; i < kDQ; ++i) {
      step(g + i, i);
      load(g + i + kDQ, i);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int i = 0; i < kDQ; ++i) {
    if (g + i >= G) break;
    step(g + i, i);
    if (g + i + kDQ < G) load(g + i + kDQ, i);
  }
#pragma unroll
  for (int i = 0; i < kDQ; ++i)
    if (g + kDQ + i < G) step(g + kDQ + i, i);
  if (col < ncol) {
#pragma unroll
    for (int r = 0; r < kRT; ++r)
      *(f32x4*)(y + (size_t)(lo + col) * d + mb + 64 * r + 16 * wave + 4 * kq) = acc[r];
  }
}

}  // namespace

// Waves per K split for a kernel of row_tiles 16-row tiles.
static int ks_of(long long row_tiles) {
  return row_tiles < 2048 ? 4 : (row_tiles < 4096 ? 2 : 1);
}

bool decode_selects_topk(int T, int k, int E, int d, int f, int format) {
  const long long P = (long long)T * k;
  const long long active = P < E ? P : E;
  return format == 0 /* int4 */ && T >= 1 && P <= 64 && E <= 64 && d % 128 == 0 &&
         f % 128 == 0 && ks_of(active * (f / 16)) > 1;
}

// Split K over 1, 2 or 4 waves so that few active experts (a single
// token touches k of them) still put enough waves on every CU.
hipError_t launch_ffn_decode_w4(const FfnArgs& a, uint16_t* h, hipStream_t s) {
  const long long P = (long long)a.T * a.k;
  const long long active = P < a.E ? P : a.E;
  // K split per kernel from its own row-tile count (gate/up: f rows per
  // matrix; down: d rows).  Down, whose K (= f) is the shorter one, runs
  // one K slice per wave from 1024 row tiles up (measured: E = 256, T = 1
  // down 18.4 us with four slices, 14.6 with two, 11.5 with one); gate/up
  // keeps the split (forcing one or two slices at T = 1 was slower).
  const int KSg = ks_of(active * (a.f / 16));
  const long long rt_d = active * (a.d / 16);
  const int KSd = rt_d < 1024 ? ks_of(rt_d) : 1;
  const bool nt2 = P > 2LL * a.E;
  if (a.logits && (KSg == 1 || !decode_selects_topk(a.T, a.k, a.E, a.d, a.f, a.format)))
    return hipErrorInvalidValue;
  if (nt2) {
    if (KSg == 4) launch_gu_pair<4, 2>(a, h, P, s);
    else if (KSg == 2) launch_gu_pair<2, 2>(a, h, P, s);
    else launch_gu_pair<1, 2>(a, h, P, s);
    if (KSd == 4) launch_dn_pair<4, 2>(a, h, P, s);
    else if (KSd == 2) launch_dn_pair<2, 2>(a, h, P, s);
    else launch_dn_pair<1, 2>(a, h, P, s);
  } else {
    if (gu_t1_applies(a, KSg)) {
      if (KSg == 4) launch_gu_t1<4>(a, h, P, s);
      else launch_gu_t1<2>(a, h, P, s);
    } else if (KSg == 4) {
      launch_gu_pair<4, 1>(a, h, P, s);
    } else if (KSg == 2) {
      launch_gu_pair<2, 1>(a, h, P, s);
    } else {
      launch_gu_lds(a, h, P, s);
    }
    if (KSd == 4) launch_dn_pair<4, 1>(a, h, P, s);
    else if (KSd == 2) launch_dn_pair<2, 1>(a, h, P, s);
    else launch_dn_lds(a, h, P, s);
  }
  return hipGetLastError();
}

// Expert-major decode of at most 16 tokens (int4): gate/up also produces the
// grouping (expert_offsets, sorted_pair, pair_pos) from topk_idx; hE is the
// per-expert scratch of em_h_bytes(E, f) bytes: h [E][16][f] bf16, then the
// per-expert pair counts [E] and pair lists [E][16] of the logits variant.
static size_t em_a256(size_t b) { return (b + 255) & ~(size_t)255; }
size_t em_h_bytes(int E, int f) {
  return em_a256((size_t)E * kEmMaxT * f * sizeof(uint16_t)) + em_a256(sizeof(int32_t) * E) +
         sizeof(int32_t) * (size_t)E * kEmMaxT;
}

// Every expert's blocks issue their first loads before knowing whether the
// expert has pairs, so the path needs most experts active: 2 T k >= E.
// The expert-major kernels can take the routing from the logits: E <= 64,
// k <= 16.
bool em_selects_topk(int T, int k, int E) { return T <= kEmMaxT && E <= 64 && k <= 16; }

bool em_applies(int T, int k, int E, int d, int f, int format) {
  return format == 0 && T >= 1 && T <= kEmMaxT && 2LL * T * k >= E && d % 128 == 0 &&
         f % 128 == 0;
}

hipError_t launch_ffn_decode_em(const FfnArgs& a, const int32_t* topk_idx, int32_t* offsets,
                                int32_t* sorted_pair, int32_t* pair_pos, uint16_t* hE,
                                hipStream_t s, const float* logits, int32_t* idx_out,
                                float* w_out) {
  if (logits && (!em_selects_topk(a.T, a.k, a.E) || (int)(a.E * (a.f / 128)) < a.T))
    return hipErrorInvalidValue;
  int32_t* em_cnt =
      (int32_t*)((char*)hE + em_a256((size_t)a.E * kEmMaxT * a.f * sizeof(uint16_t)));
  int32_t* em_list = em_cnt + em_a256(sizeof(int32_t) * a.E) / sizeof(int32_t);
  {
    // 8-wave blocks of 128 features (f % 128 == 0 always holds here; 16-wave
    // blocks of 256 features measured slower: 29.4 against 25.2 us); at most
    // four tokens, whose few active experts leave CUs idle, take 4-wave
    // blocks of 64 features (OLMoE-shaped layer, same-box A/B: T = 4 step
    // 39.1 -> 38.0 us; T = 8 and 16 were 2-4 % slower that way)
    const int G = a.d / 128;
    const size_t lds = sizeof(float) * 4 * G * 64 + sizeof(uint16_t) * 2 * 16 * kXRow;
    const int sc = scale_chunks(2, G, a.gu_scales);
    const bool w4 = a.T <= 4;
    auto pick = [&](auto lg, auto kw) {
      constexpr bool L = decltype(lg)::value;
      constexpr int W = decltype(kw)::value;
      return sc == 1   ? gateup_w4_em<kGuDQ, kGuWaves, 1, W, L>
             : sc == 2 ? gateup_w4_em<kGuDQ, kGuWaves, 2, W, L>
             : sc == 4 ? gateup_w4_em<kGuDQ, kGuWaves, 4, W, L>
                       : gateup_w4_em<kGuDQ, kGuWaves, 0, W, L>;
    };
    using W4 = std::integral_constant<int, 4>;
    using W8 = std::integral_constant<int, 8>;
    auto kern = logits ? (w4 ? pick(std::true_type{}, W4{}) : pick(std::true_type{}, W8{}))
                       : (w4 ? pick(std::false_type{}, W4{}) : pick(std::false_type{}, W8{}));
    launch_k(kern, dim3(a.E * (a.f / (w4 ? 64 : 128))), dim3(w4 ? 256 : 512), lds, s, a.ev[0],
             a.ev[1], a.x, topk_idx,
             a.T, a.k, a.E, a.d, a.f, a.gu_codes, a.gu_scales, hE, offsets, sorted_pair,
             pair_pos, logits, em_cnt, em_list, idx_out, w_out);
  }
  {
    // kDnRT row tiles per wave when d allows (d % 128 == 0 always holds)
    constexpr int RT = kDnRT;
    const int rt = a.d % (64 * RT) == 0 ? RT : 1;
    const int G = a.f / 128;
    const size_t lds = sizeof(float) * rt * G * 64 + sizeof(uint16_t) * 2 * 16 * kXRow;
    const int sc = scale_chunks(rt, G, a.dn_scales);
    if (rt == RT) {
      constexpr int DQ = kDnDQ / RT > 0 ? kDnDQ / RT : 1;  // same bytes in flight per wave
      auto pick = [&](auto lg) {
        constexpr bool L = decltype(lg)::value;
        return sc == 1   ? down_w4_em<DQ, kDnWaves, 1, RT, L>
               : sc == 2 ? down_w4_em<DQ, kDnWaves, 2, RT, L>
               : sc == 4 ? down_w4_em<DQ, kDnWaves, 4, RT, L>
                         : down_w4_em<DQ, kDnWaves, 0, RT, L>;
      };
      auto kern = logits ? pick(std::true_type{}) : pick(std::false_type{});
      launch_k(kern, dim3(a.E * (a.d / (64 * RT))), dim3(256), lds, s, a.ev[2], a.ev[3], hE,
               offsets, a.E, a.d, a.f, a.dn_codes, a.dn_scales, a.y, em_cnt, em_list, offsets,
               sorted_pair, pair_pos);
    } else {
      auto pick = [&](auto lg) {
        constexpr bool L = decltype(lg)::value;
        return sc == 1   ? down_w4_em<kDnDQ, kDnWaves, 1, 1, L>
               : sc == 2 ? down_w4_em<kDnDQ, kDnWaves, 2, 1, L>
               : sc == 4 ? down_w4_em<kDnDQ, kDnWaves, 4, 1, L>
                         : down_w4_em<kDnDQ, kDnWaves, 0, 1, L>;
      };
      auto kern = logits ? pick(std::true_type{}) : pick(std::false_type{});
      launch_k(kern, dim3(a.E * (a.d / 64)), dim3(256), lds, s, a.ev[2], a.ev[3], hE, offsets,
               a.E, a.d, a.f, a.dn_codes, a.dn_scales, a.y, em_cnt, em_list, offsets,
               sorted_pair, pair_pos);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
