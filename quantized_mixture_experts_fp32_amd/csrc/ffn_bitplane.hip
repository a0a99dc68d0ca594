// Decode-path expert FFN for bitplane experts at per-pair bit-widths.
//  PagedMoE (abstract): one stored 8-bit state per weight, laid out as
//    bitplanes so that every lower precision is a prefix; a pair at b bits
//    executes the b-plane prefix directly and only the planes an expert
//    needs (its largest b) are read.
//  MatMoE (abstract): floor-and-compensation dequantization of a prefix:
//    v_b(u) = (u with its 8-b low bits cleared) + 2^(7-b) - 128 (b < 8),
//    v_8(u) = u - 128.
//
// Arithmetic.  With bit_p the plane-p bit of u (p = 0 most significant),
//   sum_k v_b(u_k) x_k = sum_{p<b} 2^(7-p) S_p + c_b X,
//   S_p = sum_k bit_p(u_k) x_k,  X = sum_k x_k,  c_b = v_b(0).
// Per 128-group every plane p < max b is one chain of four MFMAs on exact
// bf16 operands: the A value of a weight is 1 + bit * 2^(j-4) (1.0 with the
// bit placed in mantissa bit j + 3, one v_bitop3 from a shifted plane word),
// where j = k mod 4 is also the MFMA of the chain the element belongs to,
// and the staged activation is x * 2^(4-j) (a power-of-two scaling, exact;
// the bit sits as high in the mantissa as the four shifts allow, which
// keeps the cancelled term X' small).
// Each chain starts from -X' (X' = sum_k x_k 2^(4 - k mod 4), four MFMAs with
// A = -1 shared by all planes and both matrices), so it ends at S_p.  Every
// lane owns one token column, so it weights S_p by 2^(7-p) when p is below
// its pair's bit-width and by 0 otherwise, adds c_b X (X from four more
// MFMAs), and the fp16 group scale multiplies the group sum in fp32.
// Dequantized weights are never rounded.
//
// Layout (ABI header): per 16-row tile and 128-group a 2 KiB block holds
// the 8 planes (most significant first) of 256 bytes, row r's 16 bytes at
// 16 r; bit i of byte j is element 8j + i.  Lane (row, kq) reads the word
// kq of its row: elements 32 kq .. 32 kq + 31.  A b-plane read touches the
// first 256 b bytes of each block.
//
// Work decomposition as for the int4 decode kernels with a single K slice:
// block = token tile of up to 16 pairs of one expert x 4 row tiles of 16
// features; the tile's activations are staged in LDS per group by the
// block (scaled and ordered for the B fragments); plane words stream kDQ
// groups ahead.
#include "kcommon.hpp"
#include "launch.hpp"
#include "decode_common.hpp"

namespace moe {
namespace {
using namespace dec;

constexpr int kBlockBytes = 8 * 256;  // 8 planes of one 16-row tile, one group

// Plane word (elements 32kq + s, s = 0..31) -> A operands of the 4 MFMAs
// of a chain: MFMA j, word d holds elements s = j + 4d (low half) and
// s + 16 (high half) as 1 + bit * 2^(j-4): bit s moves to bit j + 3.
__device__ __forceinline__ void bp_frags(uint32_t w, bf16x8 (&a)[4]) {
  const uint32_t C = 0x3F803F80u;  // 1.0, 1.0
  const uint32_t sh[4] = {w << 3, w >> 1, w >> 5, w >> 9};  // 4d - 3 to the right
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t M = (1u << (j + 3)) | (1u << (19 + j));
    u32x4 r;
#pragma unroll
    for (int d = 0; d < 4; ++d) r[d] = __builtin_amdgcn_bitop3_b32(sh[d], M, C, 0xEA);  // (sh & M) | C
    a[j] = __builtin_bit_cast(bf16x8, r);
  }
}

// B fragment order of one staged token row (128 bf16): element k = 32 kq + r
// goes to slot ((kq * 4 + j) * 4 + d) * 2 + h with j = r % 4, d = (r % 16) / 4,
// h = r / 16, scaled by 2^(4 - j).
__device__ __forceinline__ int bp_slot(int k) {
  const int kq = k >> 5, r = k & 31;
  return (((kq * 4 + (r & 3)) * 4 + ((r & 15) >> 2)) << 1) + (r >> 4);
}

// Stage 8 consecutive activations (16 bytes at element k0, k0 % 8 == 0).
__device__ __forceinline__ void bp_stage8(uint16_t* __restrict__ row, int k0, u32x4 v) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t b = (v[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
    const float f = __uint_as_float(b << 16) * (float)(1 << (4 - (i & 3)));
    row[bp_slot(k0 + i)] = (uint16_t)(__float_as_uint(f) >> 16);
  }
}

__device__ __forceinline__ bf16x8 splat2(uint32_t bits16) {
  const uint32_t p = bits16 | (bits16 << 16);
  return __builtin_bit_cast(bf16x8, u32x4{p, p, p, p});
}

// Per-lane (token column) plane weights and compensation of bit-width b.
struct ColWeights {
  float wp[8];
  float cb;
};

__device__ __forceinline__ ColWeights col_weights(int b) {
  ColWeights c;
#pragma unroll
  for (int p = 0; p < 8; ++p) c.wp[p] = (p < b) ? (float)(1 << (7 - p)) : 0.0f;
  c.cb = (b < 8) ? (float)((1 << (7 - b)) - 128) : -128.0f;
  return c;
}

// One group of one 16-row matrix tile: sum over planes p < nb of the
// weighted chains, plus c_b X, times the group scale, into acc.
__device__ __forceinline__ void bp_group(const bf16x8 (&xf)[4], const f32x4 seed, const f32x4 dx,
                                         const uint32_t (&pw)[8], int nb, const ColWeights& cw,
                                         const f32x4 sv, f32x4& acc) {
  f32x4 comb;
#pragma unroll
  for (int i = 0; i < 4; ++i) comb[i] = cw.cb * dx[i];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    if (p >= nb) break;
    bf16x8 a[4];
    bp_frags(pw[p], a);
    f32x4 d = seed;
#pragma unroll
    for (int j = 0; j < 4; ++j) d = mfma16(a[j], xf[j], d);
#pragma unroll
    for (int i = 0; i < 4; ++i) comb[i] = fmaf(cw.wp[p], d[i], comb[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = fmaf(sv[i], comb[i], acc[i]);
}

// Seeds of a group: -X' (A = -1) and X (A = 2^(j-4) in MFMA j).
__device__ __forceinline__ void bp_seeds(const bf16x8 (&xf)[4], f32x4& seed, f32x4& dx) {
  seed = f32x4{0, 0, 0, 0};
  dx = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    seed = mfma16(splat2(0xBF80u), xf[j], seed);
    dx = mfma16(splat2((uint32_t)(123 + j) << 7), xf[j], dx);
  }
}

// Bit-width of the tile's column col and the tile's largest bit-width.
__device__ __forceinline__ int tile_bits(const int32_t* __restrict__ sp, int r0, int cnt, int col,
                                         int e, int k, int mode, const uint8_t* __restrict__ bits,
                                         int& maxb) {
  const int b = col < cnt ? pair_bit_width(sp[r0 + col], e, k, mode, bits) : 1;
  int m = b;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) m = max(m, __shfl_xor(m, o, kWave));
  maxb = __builtin_amdgcn_readfirstlane(m);
  return b;
}

// ------------------------------------------------------------- gate / up
template <int kDQ, int kWaves>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWaves, 8)))
void gateup_bp_decode(const uint16_t* __restrict__ x, const int32_t* __restrict__ offsets,
                      const int32_t* __restrict__ sorted_pair, int E, int k, int P, int d,
                      int f, const uint8_t* __restrict__ planes,
                      const uint16_t* __restrict__ scales, int bits_mode,
                      const uint8_t* __restrict__ bits, uint16_t* __restrict__ h) {
  extern __shared__ int32_t lds_i[];
  const int G = d >> 7, RG = f / 64;
  int32_t* off_lds = lds_i;
  int32_t* sp_lds = lds_i + ((E + 1 + 3) & ~3);
  float* sc_lds = (float*)(sp_lds + ((min(P, kPairsInLds) + 3) & ~3));  // [2][G][64]
  uint16_t* xs = (uint16_t*)(sc_lds + 2 * G * 64);                      // [2][16][kXRow]
  const int np = stage_routing(offsets, sorted_pair, E, P, off_lds, sp_lds);
  __syncthreads();
  const int32_t* spp = np ? sp_lds : sorted_pair;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int st_tok = tid >> 4, st_pc = tid & 15;

  for (int w = blockIdx.x;; w += gridDim.x) {
    TileInfo tl;
    if (!find_tile(off_lds, E, 16, w / RG, tl)) break;
    const int nb = (w % RG) * 64, n0 = nb + 16 * wave;
    int maxb;
    const int b = tile_bits(spp, tl.r0, tl.cnt, col, tl.e, k, bits_mode, bits, maxb);
    const ColWeights cw = col_weights(b);
    const bool st_ok = st_tok < tl.cnt;
    const int sj = tl.r0 + (st_ok ? st_tok : 0);
    const uint16_t* xsrc = x + (size_t)(spp[sj] / k) * d + 8 * st_pc;
    // plane words: tiles of 16 rows; row n0 + col of gate, f + n0 + col of up
    const size_t rg = (size_t)tl.e * 2 * f + n0, ru = rg + f;
    const uint8_t* pg = planes + (rg >> 4) * (size_t)G * kBlockBytes + 16 * col + 4 * kq;
    const uint8_t* pu = planes + (ru >> 4) * (size_t)G * kBlockBytes + 16 * col + 4 * kq;

    uint32_t wg[kDQ][8], wu[kDQ][8];
    u32x4 xv[kDQ];
    auto load = [&](int g, int i) {
      if (st_ok) xv[i] = *(const u32x4*)(xsrc + 128 * g);
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        if (p >= maxb) break;
        wg[i][p] = *(const uint32_t*)(pg + (size_t)g * kBlockBytes + 256 * p);
        wu[i][p] = *(const uint32_t*)(pu + (size_t)g * kBlockBytes + 256 * p);
      }
    };
#pragma unroll
    for (int i = 0; i < kDQ; ++i)
      if (i < G) load(i, i);
    stage_scales_rows64<2>(scales + ((size_t)tl.e * 2 * f + nb) * G, (size_t)f, G, sc_lds);

    f32x4 tg = {0, 0, 0, 0}, tu = {0, 0, 0, 0};
    const int rd_tok = col < tl.cnt ? col : 0;
    for (int g = 0; g < G; g += kDQ) {
#pragma unroll
      for (int i = 0; i < kDQ; ++i) {
        const int gi = g + i;
        if (gi >= G) break;
        uint16_t* slot = xs + (gi & 1) * 16 * kXRow;
        if (st_ok) bp_stage8(slot + st_tok * kXRow, 8 * st_pc, xv[i]);
        __syncthreads();
        bf16x8 xf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xf[j] = *(const bf16x8*)(slot + rd_tok * kXRow + 8 * (kq * 4 + j));
        const f32x4 sg = *(const f32x4*)(sc_lds + gi * 64 + 16 * wave + 4 * kq);
        const f32x4 su = *(const f32x4*)(sc_lds + (G + gi) * 64 + 16 * wave + 4 * kq);
        f32x4 seed, dx;
        bp_seeds(xf, seed, dx);
        bp_group(xf, seed, dx, wg[i], maxb, cw, sg, tg);
        bp_group(xf, seed, dx, wu[i], maxb, cw, su, tu);
        if (gi + kDQ < G) load(gi + kDQ, i);
      }
    }
    if (col < tl.cnt) {
      uint32_t hb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) hb[i] = f32_to_bf16_rne(silu_f32(tg[i]) * tu[i]);
      uint2 pk;
      pk.x = hb[0] | (hb[1] << 16);
      pk.y = hb[2] | (hb[3] << 16);
      *(uint2*)(h + (size_t)(tl.r0 + col) * f + n0 + 4 * kq) = pk;
    }
    __syncthreads();  // the next item rewrites the scales and the slots
  }
}

// ------------------------------------------------------------------ down
template <int kDQ, int kWaves>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWaves, 8)))
void down_bp_decode(const uint16_t* __restrict__ h, const int32_t* __restrict__ offsets,
                    const int32_t* __restrict__ sorted_pair, int E, int k, int d, int f,
                    const uint8_t* __restrict__ planes, const uint16_t* __restrict__ scales,
                    int bits_mode, const uint8_t* __restrict__ bits, float* __restrict__ y) {
  extern __shared__ int32_t lds_i[];
  const int G = f >> 7, RG = d / 64;
  int32_t* off_lds = lds_i;
  float* sc_lds = (float*)(lds_i + ((E + 1 + 3) & ~3));  // [G][64]
  uint16_t* xs = (uint16_t*)(sc_lds + G * 64);           // [2][16][kXRow]
  for (int i = threadIdx.x; i <= E; i += blockDim.x) off_lds[i] = offsets[i];
  __syncthreads();

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int st_tok = tid >> 4, st_pc = tid & 15;

  for (int w = blockIdx.x;; w += gridDim.x) {
    TileInfo tl;
    if (!find_tile(off_lds, E, 16, w / RG, tl)) break;
    const int mb = (w % RG) * 64, m0 = mb + 16 * wave;
    int maxb;
    const int b = tile_bits(sorted_pair, tl.r0, tl.cnt, col, tl.e, k, bits_mode, bits, maxb);
    const ColWeights cw = col_weights(b);
    const bool st_ok = st_tok < tl.cnt;
    const uint16_t* hsrc = h + (size_t)(tl.r0 + (st_ok ? st_tok : 0)) * f + 8 * st_pc;
    const size_t rd0 = (size_t)tl.e * d + m0;
    const uint8_t* pd = planes + (rd0 >> 4) * (size_t)G * kBlockBytes + 16 * col + 4 * kq;

    uint32_t wd[kDQ][8];
    u32x4 hv[kDQ];
    auto load = [&](int g, int i) {
      if (st_ok) hv[i] = *(const u32x4*)(hsrc + 128 * g);
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        if (p >= maxb) break;
        wd[i][p] = *(const uint32_t*)(pd + (size_t)g * kBlockBytes + 256 * p);
      }
    };
#pragma unroll
    for (int i = 0; i < kDQ; ++i)
      if (i < G) load(i, i);
    stage_scales_rows64<1>(scales + ((size_t)tl.e * d + mb) * G, 0, G, sc_lds);

    f32x4 acc = {0, 0, 0, 0};
    const int rd_tok = col < tl.cnt ? col : 0;
    for (int g = 0; g < G; g += kDQ) {
#pragma unroll
      for (int i = 0; i < kDQ; ++i) {
        const int gi = g + i;
        if (gi >= G) break;
        uint16_t* slot = xs + (gi & 1) * 16 * kXRow;
        if (st_ok) bp_stage8(slot + st_tok * kXRow, 8 * st_pc, hv[i]);
        __syncthreads();
        bf16x8 xf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xf[j] = *(const bf16x8*)(slot + rd_tok * kXRow + 8 * (kq * 4 + j));
        const f32x4 sv = *(const f32x4*)(sc_lds + gi * 64 + 16 * wave + 4 * kq);
        f32x4 seed, dx;
        bp_seeds(xf, seed, dx);
        bp_group(xf, seed, dx, wd[i], maxb, cw, sv, acc);
        if (gi + kDQ < G) load(gi + kDQ, i);
      }
    }
    if (col < tl.cnt) *(f32x4*)(y + (size_t)(tl.r0 + col) * d + m0 + 4 * kq) = acc;
    __syncthreads();
  }
}

#ifndef BP_DQ
#define BP_DQ 2
#define BP_WAVES 3
#endif
constexpr int kBpDQ = BP_DQ, kBpWaves = BP_WAVES;

}  // namespace

bool ffn_decode_bp_applies(long long P, int E, int f) {
  const long long active = P < E ? P : E;
  return P <= 2LL * E && active * (f / 16) >= 4096;
}

hipError_t launch_ffn_decode_bp(const FfnArgs& a, uint16_t* h, hipStream_t s) {
  const long long P = (long long)a.T * a.k;
  const long long mt = (P + 15) / 16 + (P < a.E ? P : a.E);
  const size_t off_b = sizeof(int32_t) * ((a.E + 1 + 3) & ~3);
  const size_t xs_b = sizeof(uint16_t) * 2 * 16 * kXRow;
  const long long cap = 256LL * 8;
  {
    const int G = a.d / 128;
    const long long work = mt * (a.f / 64);
    const int grid = (int)(work < cap ? work : cap);
    const size_t lds = off_b + sizeof(int32_t) * ((std::min<long long>(P, kPairsInLds) + 3) & ~3) +
                       sizeof(float) * 2 * G * 64 + xs_b;
    launch_k(gateup_bp_decode<kBpDQ, kBpWaves>, dim3(grid), dim3(256), lds, s, a.ev[0], a.ev[1],
             a.x,
                       a.offsets, a.sorted_pair, a.E, a.k, (int)P, a.d, a.f, a.gu_codes,
                       a.gu_scales, a.bits_mode, a.bits, h);
  }
  {
    const int G = a.f / 128;
    const long long work = mt * (a.d / 64);
    const int grid = (int)(work < cap ? work : cap);
    const size_t lds = off_b + sizeof(float) * G * 64 + xs_b;
    launch_k(down_bp_decode<kBpDQ, kBpWaves>, dim3(grid), dim3(256), lds, s, a.ev[2], a.ev[3],
             h,
                       a.offsets, a.sorted_pair, a.E, a.k, a.d, a.f, a.dn_codes, a.dn_scales,
                       a.bits_mode, a.bits, a.y);
  }
  return hipGetLastError();
}

}  // namespace moe
