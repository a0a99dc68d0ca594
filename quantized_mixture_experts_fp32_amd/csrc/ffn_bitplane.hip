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
template <int NB>
__device__ __forceinline__ void bp_group(const bf16x8 (&xf)[4], const f32x4 seed, const f32x4 dx,
                                         const uint32_t (&pw)[NB], const ColWeights& cw,
                                         const f32x4 sv, f32x4& acc) {
  f32x4 comb;
#pragma unroll
  for (int i = 0; i < 4; ++i) comb[i] = cw.cb * dx[i];
#pragma unroll
  for (int p = 0; p < NB; ++p) {
    bf16x8 a[4];
    bp_frags(pw[p], a);
    f32x4 d = seed;
#pragma unroll
    for (int j = 0; j < 4; ++j) d = mfma16(a[j], xf[j], d);
#pragma unroll
    for (int i = 0; i < 4; ++i) comb[i] = fmaf(cw.wp[p], d[i], comb[i]);
    __builtin_amdgcn_sched_barrier(0);  // one plane's fragments live at a time
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
// One work item reading the NB planes of its tile's largest bit-width (NB is
// a compile-time constant, chosen per item by a block-uniform switch, so
// every load of the group loop is unconditional).  The loop refills each
// slot right after its use in a branch-free steady state: the compiler's
// waits then count exactly the loads issued after the one needed, and kDQ
// groups stay in flight across the loop edge.  Scales are fetched before
// the plane words and written to LDS after them.  Rows past the tile stage a
// copy of its first row (they feed only unstored columns).
template <int NB, int kDQ, int kSC>
__device__ __forceinline__ void bp_gu_item(const uint16_t* __restrict__ xsrc,
                                           const uint8_t* __restrict__ pg,
                                           const uint8_t* __restrict__ pu, int G,
                                           const uint16_t* __restrict__ sc_src, size_t f,
                                           float* sc_lds, uint16_t* xs, const ColWeights& cw,
                                           f32x4& tg, f32x4& tu) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int st_tok = tid >> 4, st_pc = tid & 15;
  uint32_t wg[kDQ][NB], wu[kDQ][NB];
  u32x4 xv[kDQ];
  auto load = [&](int g, int i) {
    xv[i] = *(const u32x4*)(xsrc + 128 * g);
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      wg[i][p] = *(const uint32_t*)(pg + (size_t)g * kBlockBytes + 256 * p);
      wu[i][p] = *(const uint32_t*)(pu + (size_t)g * kBlockBytes + 256 * p);
    }
  };
  ScaleStage<2, kSC ? kSC : 1> sst;
  if (kSC) sst.fetch(sc_src, f, G);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kDQ; ++i) load(i < G ? i : G - 1, i);
  __builtin_amdgcn_sched_barrier(0);
  if (kSC)
    sst.store(G, sc_lds);
  else
    stage_scales_rows64<2>(sc_src, f, G, sc_lds);
  auto step = [&](int gi, int i) {
    // slot gi & 1 was last read in step gi - 2, before the barrier of step gi - 1
    uint16_t* slot = xs + (gi & 1) * 16 * kXRow;
    bp_stage8(slot + st_tok * kXRow, 8 * st_pc, xv[i]);
    __syncthreads();
    bf16x8 xf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xf[j] = *(const bf16x8*)(slot + col * kXRow + 8 * (kq * 4 + j));
    const f32x4 sg = *(const f32x4*)(sc_lds + gi * 64 + 16 * wave + 4 * kq);
    const f32x4 su = *(const f32x4*)(sc_lds + (G + gi) * 64 + 16 * wave + 4 * kq);
    f32x4 seed, dx;
    bp_seeds(xf, seed, dx);
    bp_group<NB>(xf, seed, dx, wg[i], cw, sg, tg);
    bp_group<NB>(xf, seed, dx, wu[i], cw, su, tu);
  };
  int g = 0;
  for (; g + 2 * kDQ <= G; g += kDQ) {
#pragma unroll
    for (int i = 0; i < kDQ; ++i) {
      step(g + i, i);
      __builtin_amdgcn_sched_barrier(0);  // the slot's words are consumed first
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
}

template <int kDQ, int kWaves, int kSC>
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
    const int sj = tl.r0 + (st_tok < tl.cnt ? st_tok : 0);
    const int sp = spp[sj];
    asm volatile("" ::"v"(sp) : "memory");  // routing value taken before any plane load
    const uint16_t* xsrc = x + (size_t)(sp / k) * d + 8 * st_pc;
    // plane words: tiles of 16 rows; row n0 + col of gate, f + n0 + col of up
    const size_t rg = (size_t)tl.e * 2 * f + n0, ru = rg + f;
    const uint8_t* pg = planes + (rg >> 4) * (size_t)G * kBlockBytes + 16 * col + 4 * kq;
    const uint8_t* pu = planes + (ru >> 4) * (size_t)G * kBlockBytes + 16 * col + 4 * kq;
    const uint16_t* sc_src = scales + ((size_t)tl.e * 2 * f + nb) * G;
    f32x4 tg = {0, 0, 0, 0}, tu = {0, 0, 0, 0};
    switch (maxb) {  // block-uniform
#define BP_GU_CASE(N) \
  case N:             \
    bp_gu_item<N, kDQ, kSC>(xsrc, pg, pu, G, sc_src, (size_t)f, sc_lds, xs, cw, tg, tu); \
    break;
      BP_GU_CASE(1) BP_GU_CASE(2) BP_GU_CASE(3) BP_GU_CASE(4)
      BP_GU_CASE(5) BP_GU_CASE(6) BP_GU_CASE(7)
      default:
        bp_gu_item<8, kDQ, kSC>(xsrc, pg, pu, G, sc_src, (size_t)f, sc_lds, xs, cw, tg, tu);
#undef BP_GU_CASE
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
template <int NB, int kDQ, int kSC>
__device__ __forceinline__ void bp_dn_item(const uint16_t* __restrict__ hsrc,
                                           const uint8_t* __restrict__ pd, int G,
                                           const uint16_t* __restrict__ sc_src, float* sc_lds,
                                           uint16_t* xs, const ColWeights& cw, f32x4& acc) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int st_tok = tid >> 4, st_pc = tid & 15;
  uint32_t wd[kDQ][NB];
  u32x4 hv[kDQ];
  auto load = [&](int g, int i) {
    hv[i] = *(const u32x4*)(hsrc + 128 * g);
#pragma unroll
    for (int p = 0; p < NB; ++p)
      wd[i][p] = *(const uint32_t*)(pd + (size_t)g * kBlockBytes + 256 * p);
  };
  ScaleStage<1, kSC ? kSC : 1> sst;
  if (kSC) sst.fetch(sc_src, 0, G);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kDQ; ++i) load(i < G ? i : G - 1, i);
  __builtin_amdgcn_sched_barrier(0);
  if (kSC)
    sst.store(G, sc_lds);
  else
    stage_scales_rows64<1>(sc_src, 0, G, sc_lds);
  auto step = [&](int gi, int i) {
    uint16_t* slot = xs + (gi & 1) * 16 * kXRow;
    bp_stage8(slot + st_tok * kXRow, 8 * st_pc, hv[i]);
    __syncthreads();
    bf16x8 xf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xf[j] = *(const bf16x8*)(slot + col * kXRow + 8 * (kq * 4 + j));
    const f32x4 sv = *(const f32x4*)(sc_lds + gi * 64 + 16 * wave + 4 * kq);
    f32x4 seed, dx;
    bp_seeds(xf, seed, dx);
    bp_group<NB>(xf, seed, dx, wd[i], cw, sv, acc);
  };
  int g = 0;
  for (; g + 2 * kDQ <= G; g += kDQ) {
#pragma unroll
    for (int i = 0; i < kDQ; ++i) {
      step(g + i, i);
      __builtin_amdgcn_sched_barrier(0);  // the slot's words are consumed first
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
}

template <int kDQ, int kWaves, int kSC>
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
    const uint16_t* hsrc = h + (size_t)(tl.r0 + (st_tok < tl.cnt ? st_tok : 0)) * f + 8 * st_pc;
    const size_t rd0 = (size_t)tl.e * d + m0;
    const uint8_t* pd = planes + (rd0 >> 4) * (size_t)G * kBlockBytes + 16 * col + 4 * kq;
    const uint16_t* sc_src = scales + ((size_t)tl.e * d + mb) * G;
    f32x4 acc = {0, 0, 0, 0};
    switch (maxb) {  // block-uniform
#define BP_DN_CASE(N) \
  case N:             \
    bp_dn_item<N, kDQ, kSC>(hsrc, pd, G, sc_src, sc_lds, xs, cw, acc); \
    break;
      BP_DN_CASE(1) BP_DN_CASE(2) BP_DN_CASE(3) BP_DN_CASE(4)
      BP_DN_CASE(5) BP_DN_CASE(6) BP_DN_CASE(7)
      default:
        bp_dn_item<8, kDQ, kSC>(hsrc, pd, G, sc_src, sc_lds, xs, cw, acc);
#undef BP_DN_CASE
    }
    if (col < tl.cnt) *(f32x4*)(y + (size_t)(tl.r0 + col) * d + m0 + 4 * kq) = acc;
    __syncthreads();
  }
}

// Plane-word groups in flight and occupancy (measured on MI355X): both
// kernels keep two groups ahead at two waves per SIMD (gate/up with one
// group ahead at three waves was 8-15 % slower).
constexpr int kBpGuDQ = 2, kBpGuWaves = 2, kBpDnDQ = 2, kBpDnWaves = 2;

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
    const int sc = scale_chunks(2, G, a.gu_scales);
    auto kern = sc == 1   ? gateup_bp_decode<kBpGuDQ, kBpGuWaves, 1>
                : sc == 2 ? gateup_bp_decode<kBpGuDQ, kBpGuWaves, 2>
                : sc == 4 ? gateup_bp_decode<kBpGuDQ, kBpGuWaves, 4>
                          : gateup_bp_decode<kBpGuDQ, kBpGuWaves, 0>;
    launch_k(kern, dim3(grid), dim3(256), lds, s, a.ev[0], a.ev[1], a.x, a.offsets,
             a.sorted_pair, a.E, a.k, (int)P, a.d, a.f, a.gu_codes, a.gu_scales, a.bits_mode,
             a.bits, h);
  }
  {
    const int G = a.f / 128;
    const long long work = mt * (a.d / 64);
    const int grid = (int)(work < cap ? work : cap);
    const size_t lds = off_b + sizeof(float) * G * 64 + xs_b;
    const int sc = scale_chunks(1, G, a.dn_scales);
    auto kern = sc == 1   ? down_bp_decode<kBpDnDQ, kBpDnWaves, 1>
                : sc == 2 ? down_bp_decode<kBpDnDQ, kBpDnWaves, 2>
                : sc == 4 ? down_bp_decode<kBpDnDQ, kBpDnWaves, 4>
                          : down_bp_decode<kBpDnDQ, kBpDnWaves, 0>;
    launch_k(kern, dim3(grid), dim3(256), lds, s, a.ev[2], a.ev[3], h, a.offsets,
             a.sorted_pair, a.E, a.k, a.d, a.f, a.dn_codes, a.dn_scales, a.bits_mode, a.bits,
             a.y);
  }
  return hipGetLastError();
}

}  // namespace moe
