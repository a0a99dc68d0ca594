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
// Planes are taken in pairs (2c, 2c + 1): the two-bit field
// f = 2 bit_2c + bit_2c+1 of every weight gives
//   2^(7-2c) S_2c + 2^(6-2c) S_2c+1 = 2^(6-2c) F_c,  F_c = sum_k f_k x_k,
// so one MFMA chain per plane pair covers both planes.  The A value of a
// weight is 2^(7-pos) + f: 2^(7-pos) with the field in mantissa bits pos
// and pos + 1 (pos = 0, 2 or 4 by the weight's place in the operand; the
// mantissa ulp of 2^(7-pos) is 2^(pos-7), so the field adds f exactly),
// placed by one v_bitop3 per two weights from a word holding the fields of
// 16 weights (two v_bitop3 merge the two plane words into such words for
// the even and the odd weights).  The product with the staged activation
// is x 2^(7-pos) + f x.  Each chain starts from -X' (X' = sum_k x_k
// 2^(7-pos_k), four MFMAs with A = -2^(7-pos) shared by all chains and both
// matrices), so it ends at F_c.  A pair that
// a column's odd width splits (b = 2c + 1) uses the half chain H_c of plane
// 2c alone (field 2 bit_2c, the same scheme with a zero second plane), which
// gives 2 S_2c.  Every lane owns one token column: it weights F_c by
// 2^(6-2c) when b >= 2c + 2 and H_c by 2^(6-2c) when b = 2c + 1, adds c_b X
// (X from four more MFMAs whose A is 1), and the fp16 group scale
// multiplies the group sum in fp32.  Dequantized weights are never rounded.
// Activations are staged in the operand order (a permutation of each
// 128-group, bp_run) and unscaled.
//
// Layout (ABI header, kcommon.hpp): per 16-row tile and 128-group a 2 KiB
// block holds four plane pairs of 512 bytes (most significant first); row
// r's quarter kq of pair c is the 8 bytes at 512 c + 32 r + 8 kq, the word
// of plane 2c then that of plane 2c + 1, bit i of a word being element
// 32 kq + i.  Lane (row, kq) fetches a pair with one 8-byte load (an odd
// width's last plane with a 4-byte one); a b-plane read touches the first
// 512 ceil(b / 2) bytes of each block.
//
// Work decomposition as for the int4 decode kernels with a single K slice:
// block = token tile of up to 16 pairs of one expert x 4 waves, each wave
// two 16-row tiles (gate/up: the gate and up tiles of 16 features; down:
// two row tiles 64 rows apart); the tile's activations are staged in LDS
// per group by the block (scaled and ordered for the B fragments); plane
// words stream kDQ groups ahead.  Blocks take the tiles widest first (see
// "work item order" below).
#include "kcommon.hpp"
#include "launch.hpp"
#include "decode_common.hpp"

namespace moe {
namespace {
using namespace dec;

constexpr int kBlockBytes = kBpBlock;  // 8 planes of one 16-row tile, one group

// Operand slot o = 4 j + d (MFMA j, 32-bit word d of the lane's A operand)
// holds the fields at bits 2 i, 2 i + 1 (low half) and 2 i + 16, 2 i + 17
// (high half) of the merged word of parity o / 8, i = o % 8: the weights
// 2 i + par (low) and 2 i + 16 + par (high) of the lane's 32-weight slice.
// The word is shifted right by kShift[i] so that the field sits at
// mantissa bit kPos[i] = 2 i - kShift[i].
constexpr int kShift[8] = {0, 0, 0, 6, 6, 6, 12, 12};
constexpr int kPos[8] = {0, 2, 4, 0, 2, 4, 0, 2};

// Plane words of planes p (high) and q (low) -> the field words of the even
// (E) and odd (O) weights of the slice (bitop3 LUT 0xE4: a & c | b & ~c).
__device__ __forceinline__ void bp_merge(uint32_t wp, uint32_t wq, uint32_t& E, uint32_t& O) {
  E = __builtin_amdgcn_bitop3_b32(wp << 1, wq, 0xAAAAAAAAu, 0xE4);
  O = __builtin_amdgcn_bitop3_b32(wp, wq >> 1, 0xAAAAAAAAu, 0xE4);
}
// Plane p alone (a zero second plane): fields 2 bit_p.
__device__ __forceinline__ void bp_merge_half(uint32_t wp, uint32_t& E, uint32_t& O) {
  E = (wp << 1) & 0xAAAAAAAAu;
  O = wp & 0xAAAAAAAAu;
}

// bf16 2^(7 - pos) of operand slot i in both halves (sign bit: negated).
__device__ constexpr uint32_t bp_pow2(int i, uint32_t sign = 0) {
  return (sign | (uint32_t)(134 - kPos[i]) << 7) * 0x10001u;
}

// Field words -> the A operands of the chain's four MFMAs (LUT 0xEA:
// (a & b) | c; c = 2^(7 - pos) in both halves).
__device__ __forceinline__ void bp_frags(uint32_t E, uint32_t O, bf16x8 (&a)[4]) {
  const uint32_t w[2][3] = {{E, E >> 6, E >> 12}, {O, O >> 6, O >> 12}};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x4 r;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int o = 4 * j + d, par = o >> 3, i = o & 7;
      const uint32_t M = (3u << kPos[i]) | (3u << (kPos[i] + 16));
      r[d] = __builtin_amdgcn_bitop3_b32(w[par][kShift[i] / 6], M, bp_pow2(i), 0xEA);
    }
    a[j] = __builtin_bit_cast(bf16x8, r);
  }
}

// Staged order of a 128-group (the B fragment order): weight k sits at
// slot 32 (k / 32) + 8 j + 2 d + h, with h = (k / 16) % 2 and operand index
// o = 4 j + d = 8 (k % 2) + (k % 16) / 2.  The weights k0 + t and
// k0 + 16 + t (k0 % 32 = 4 m, m < 4, t < 4) fill the two 8-byte runs at
// s0 = 32 (k0 / 32) + 8 (m / 2) + 4 (m % 2) and s0 + 16: run s0 holds
// k0, k0 + 16, k0 + 2, k0 + 18 and run s0 + 16 holds k0 + 1, k0 + 17,
// k0 + 3, k0 + 19.
__device__ __forceinline__ int bp_run(int k0) {
  const int m = (k0 & 15) >> 2;
  return 32 * (k0 >> 5) + 8 * (m >> 1) + 4 * (m & 1);
}

// Stage the 8 weights of one thread: lo = weights k0 .. k0 + 3, hi =
// k0 + 16 .. k0 + 19 (bf16 pairs), into the runs at s0 and s0 + 16.
__device__ __forceinline__ void bp_stage8(uint16_t* __restrict__ row, int s0, u32x4 v) {
  const uint32_t lx = v[0], ly = v[1], hx = v[2], hy = v[3];
  *(uint2*)(row + s0) = uint2{(lx & 0xFFFFu) | (hx << 16), (ly & 0xFFFFu) | (hy << 16)};
  *(uint2*)(row + s0 + 16) = uint2{(lx >> 16) | (hx & 0xFFFF0000u), (ly >> 16) | (hy & 0xFFFF0000u)};
}

__device__ __forceinline__ bf16x8 splat2(uint32_t bits16) {
  const uint32_t p = bits16 | (bits16 << 16);
  return __builtin_bit_cast(bf16x8, u32x4{p, p, p, p});
}

// Per-lane (token column) chain weights and compensation of bit-width b:
// wF[c] for the pair chain F_c, wH[c] for the half chain H_c.
struct ColWeights {
  float wF[4], wH[4];
  float cb;
};

__device__ __forceinline__ ColWeights col_weights(int b) {
  ColWeights c;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    c.wF[q] = (b >= 2 * q + 2) ? (float)(1 << (6 - 2 * q)) : 0.0f;
    c.wH[q] = (b == 2 * q + 1) ? (float)(1 << (6 - 2 * q)) : 0.0f;
  }
  c.cb = (b < 8) ? (float)((1 << (7 - b)) - 128) : -128.0f;
  return c;
}

// Seeds of a group: -X' (A = -2^(7-pos) per operand slot) and X (A = 1).
__device__ __forceinline__ void bp_seeds(const bf16x8 (&xf)[4], f32x4& seed, f32x4& dx) {
  seed = f32x4{0, 0, 0, 0};
  dx = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x4 r;
#pragma unroll
    for (int d = 0; d < 4; ++d) r[d] = bp_pow2((4 * j + d) & 7, 0x8000u);
    seed = mfma16(__builtin_bit_cast(bf16x8, r), xf[j], seed);
    dx = mfma16(splat2(0x3F80u), xf[j], dx);
  }
}

// Chain t of a group of NB planes: the pair chains F_0 .. F_(NB/2 - 1), then
// (odd NB) the half chain of the top plane.
template <int NB>
__device__ __forceinline__ void bp_chain_words(const uint32_t (&pw)[NB], int t, uint32_t& E,
                                               uint32_t& O) {
  if (2 * t + 1 < NB)
    bp_merge(pw[2 * t], pw[2 * t + 1], E, O);
  else
    bp_merge_half(pw[2 * t], E, O);
}
template <int NB>
__device__ __forceinline__ float bp_chain_weight(const ColWeights& cw, int t) {
  return (2 * t + 1 < NB) ? cw.wF[t] : cw.wH[t];
}

// Gate and up tiles of one group, software-pipelined: the chains of step t
// (gate and up, independent) run on the matrix core while the A operands of
// step t + 1 are built and step t - 1's sums are weighted into the column
// totals.  Half chains of odd widths below the tile's largest (hmask bit
// c: some column has b = 2c + 1) come first, one at a time.
template <int NB>
__device__ __forceinline__ void bp_group2(const bf16x8 (&xf)[4], const f32x4 seed,
                                          const f32x4 dx, const uint32_t (&pg)[NB],
                                          const uint32_t (&pu)[NB], const ColWeights& cw,
                                          uint32_t hmask, const f32x4 sg, const f32x4 su,
                                          f32x4& tg, f32x4& tu) {
  constexpr int NC = (NB + 1) / 2;
  f32x4 cg, cu;
#pragma unroll
  for (int i = 0; i < 4; ++i) cg[i] = cu[i] = cw.cb * dx[i];
#pragma unroll
  for (int t = 0; t < NC + NB / 2; ++t) {
    const bool half = t >= NC;
    const int c = half ? t - NC : t;
    if (half && !((hmask >> c) & 1u)) continue;
    bf16x8 ag[4], au[4];
    uint32_t E, O;
    if (half) bp_merge_half(pg[2 * c], E, O); else bp_chain_words<NB>(pg, c, E, O);
    bp_frags(E, O, ag);
    if (half) bp_merge_half(pu[2 * c], E, O); else bp_chain_words<NB>(pu, c, E, O);
    bp_frags(E, O, au);
    f32x4 dg = seed, du = seed;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dg = mfma16(ag[j], xf[j], dg);
      du = mfma16(au[j], xf[j], du);
    }
    const float w = half ? cw.wH[c] : bp_chain_weight<NB>(cw, c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      cg[i] = fmaf(w, dg[i], cg[i]);
      cu[i] = fmaf(w, du[i], cu[i]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    tg[i] = fmaf(sg[i], cg[i], tg[i]);
    tu[i] = fmaf(su[i], cu[i], tu[i]);
  }
}

// Bit-width of the tile's column col, the tile's largest bit-width, and the
// half-chain mask (bit c: some column has the odd width 2c + 1 below maxb).
__device__ __forceinline__ int tile_bits(const int32_t* __restrict__ sp, int r0, int cnt, int col,
                                         int e, int k, int mode, const uint8_t* __restrict__ bits,
                                         int& maxb, uint32_t& hmask) {
  const int b = col < cnt ? pair_bit_width(sp[r0 + col], e, k, mode, bits) : 1;
  int m = b;
  uint32_t odd = (col < cnt && (b & 1)) ? 1u << (b >> 1) : 0u;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    m = max(m, __shfl_xor(m, o, kWave));
    odd |= (uint32_t)__shfl_xor((int)odd, o, kWave);
  }
  maxb = __builtin_amdgcn_readfirstlane(m);
  // the top plane of an odd largest width is a chain of its own already
  hmask = (uint32_t)__builtin_amdgcn_readfirstlane((int)odd) & ((1u << (maxb >> 1)) - 1u);
  return b;
}

// ------------------------------------------------------ work item order
// An item's cost grows with the planes it reads, which under a mixed
// bit-width rule differ up to eightfold between experts.  Blocks therefore
// take the tiles in the order of their keys, largest first (key: the
// largest bit-width among the expert's pairs; experts ascending within a
// key), so that the widest items start in the first residency round and
// the narrow ones fill the tail (measured at the OLMoE-shaped layer, T = 16,
// rank rule: gate/up 52.3 -> 45.8 us, outputs unchanged, since every item
// computes the same values wherever it runs).  Every block computes the key
// of every expert (key[e], 0 without pairs) and the tile count of every key
// (ktiles[v]) in LDS: slot i raises the key of the expert owning it, the
// last e with off[e] <= i, to its pair's width.
__device__ __forceinline__ void stage_tile_keys(const int32_t* __restrict__ off,
                                                const int32_t* __restrict__ sp, int E, int k,
                                                int mode, const uint8_t* __restrict__ bits,
                                                int32_t* __restrict__ key,
                                                int32_t* __restrict__ ktiles) {
  const int tid = threadIdx.x;
  if (tid < 9) ktiles[tid] = 0;
  const bool per_pair = mode == 1 || mode == 3;  // otherwise one width per expert
  for (int e = tid; e < E; e += blockDim.x)
    key[e] = (!per_pair && off[e + 1] > off[e]) ? pair_bit_width(0, e, k, mode, bits) : 0;
  __syncthreads();
  if (per_pair) {
    const int np = off[E];
    for (int i = tid; i < np; i += blockDim.x) {
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= i) lo = mid; else hi = mid - 1;
      }
      atomicMax(&key[lo], pair_bit_width(sp[i], lo, k, mode, bits));
    }
    __syncthreads();
  }
  for (int e = tid; e < E; e += blockDim.x)
    if (key[e] > 0) atomicAdd(&ktiles[key[e]], (off[e + 1] - off[e] + 15) >> 4);
  __syncthreads();
}
// Tile b of the list "tiles of 16 pairs of the experts of key 8, then of
// key 7, ... 1" (wave-cooperative, as find_tile; false past the end).
__device__ inline bool find_tile_by_key(const int32_t* __restrict__ offsets,
                                        const int32_t* __restrict__ key,
                                        const int32_t* __restrict__ ktiles, int E, int b,
                                        TileInfo& t) {
  const int lane = threadIdx.x & 63;
  int carry = 0, v = 8;
  for (; v >= 1; --v) {
    if (b < carry + ktiles[v]) break;
    carry += ktiles[v];
  }
  if (v < 1) return false;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    const int lo = (e < E) ? offsets[e] : 0;
    const int n = (e < E && key[e] == v) ? offsets[e + 1] - lo : 0;
    const int c = (n + 15) >> 4;
    int s = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(s, o, kWave);
      if (lane >= o) s += u;
    }
    const int total = __shfl(s, 63, kWave);
    if (b < carry + total) {
      const uint64_t m = __ballot(carry + s > b);
      const int L = __ffsll((unsigned long long)m) - 1;
      const int sL = __shfl(s, L, kWave), cL = __shfl(c, L, kWave);
      const int loL = __shfl(lo, L, kWave), nL = __shfl(n, L, kWave);
      const int chunk = b - (carry + sL - cL);
      t.e = base + L;
      t.r0 = loL + chunk * 16;
      t.cnt = min(16, nL - chunk * 16);
      return true;
    }
    carry += total;
  }
  return false;
}
// LDS bytes of the keys and the key tile counts.
inline size_t tile_key_bytes(int E) { return sizeof(int32_t) * ((size_t)E + 16); }

// ------------------------------------------------------------- gate / up
// One work item reading the NB planes of its tile's largest bit-width (NB is
// a compile-time constant, chosen per item by a block-uniform switch, so
// every load of the group loop is unconditional).  Each wave computes two
// 16-row tiles that share the staged activations and whose chains
// interleave on the matrix core: the gate and up tiles of the same
// features (gate/up), or two row tiles 64 rows apart (down).  Tile t starts
// at pt[t]; its scale rows start t mat_stride rows past sc_src.  The loop refills each
// slot right after its use in a branch-free steady state: the compiler's
// waits then count exactly the loads issued after the one needed, and kDQ
// groups stay in flight across the loop edge.  Scales are fetched before
// the plane words and written to LDS after them.  Rows past the tile stage a
// copy of its first row (they feed only unstored columns).  kStaged: the
// activation rows are stored already in the staged order (h as the gate/up
// kernel writes it): xsrc points at the thread's 16 bytes of group 0 and
// staging is a plain copy.  Otherwise xsrc points at weight k0 of group 0
// (k0 = 32 (st_pc / 4) + 4 (st_pc % 4)) and the thread loads weights
// k0 .. k0 + 3 and k0 + 16 .. k0 + 19 and stores them as two runs.
template <int NB, int kDQ, int kSC, bool kStaged>
__device__ __forceinline__ void bp_item(const uint16_t* __restrict__ xsrc,
                                        const uint8_t* const (&pt)[2], int G,
                                        const uint16_t* __restrict__ sc_src, size_t mat_stride,
                                        float* sc_lds, uint16_t* xs, const ColWeights& cw,
                                        uint32_t hmask, f32x4 (&acc)[2]) {
  constexpr int NT = 2;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int st_tok = tid >> 4, st_pc = tid & 15;
  uint32_t wv[kDQ][NT][NB];
  u32x4 xv[kDQ];
  auto load = [&](int g, int i) {
    if (kStaged) {
      xv[i] = *(const u32x4*)(xsrc + 128 * g);
    } else {
      const uint2 lo = *(const uint2*)(xsrc + 128 * g), hi = *(const uint2*)(xsrc + 128 * g + 16);
      xv[i] = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
#pragma unroll
    for (int c = 0; c < NB / 2; ++c)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        // plane words are read once per step: nontemporal, as the int4 codes
        const u32x2 a =
            __builtin_nontemporal_load((const u32x2*)(pt[t] + (size_t)g * kBlockBytes + kBpPair * c));
        wv[i][t][2 * c] = a.x;
        wv[i][t][2 * c + 1] = a.y;
      }
    if (NB & 1)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        wv[i][t][NB - 1] =
            __builtin_nontemporal_load((const uint32_t*)(pt[t] + (size_t)g * kBlockBytes + kBpPair * (NB / 2)));
  };
  ScaleStage<2, kSC ? kSC : 1> sst;
  if (kSC) sst.fetch(sc_src, mat_stride, G);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kDQ; ++i) load(i < G ? i : G - 1, i);
  __builtin_amdgcn_sched_barrier(0);
  if (kSC)
    sst.store(G, sc_lds);
  else
    stage_scales_rows64<2>(sc_src, mat_stride, G, sc_lds);
  auto step = [&](int gi, int i) {
    // slot gi & 1 was last read in step gi - 2, before the barrier of step gi - 1
    uint16_t* slot = xs + (gi & 1) * 16 * kXRow;
    if (kStaged)
      *(u32x4*)(slot + st_tok * kXRow + 8 * st_pc) = xv[i];
    else
      bp_stage8(slot + st_tok * kXRow, bp_run(32 * (st_pc >> 2) + 4 * (st_pc & 3)), xv[i]);
    __syncthreads();
    bf16x8 xf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xf[j] = *(const bf16x8*)(slot + col * kXRow + 8 * (kq * 4 + j));
    f32x4 sv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
      sv[t] = *(const f32x4*)(sc_lds + (t * G + gi) * 64 + 16 * wave + 4 * kq);
    f32x4 seed, dx;
    bp_seeds(xf, seed, dx);
    bp_group2<NB>(xf, seed, dx, wv[i][0], wv[i][1], cw, hmask, sv[0], sv[1], acc[0], acc[1]);
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

// Gate/up: item = (token tile of up to 16 pairs, 64 features); wave w
// computes features 16 w .. 16 w + 15 of the gate and up matrices.  (Two
// such feature tiles per wave, one group of planes in flight instead of
// two, read the same bytes per wave but were slower: 56.3 against 52.2 us
// at the OLMoE-shaped layer, T = 16.)
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
  int32_t* ktiles = (int32_t*)(xs + 2 * 16 * kXRow);                     // [16]
  int32_t* key = ktiles + 16;                                            // [E]
  const int np = stage_routing(offsets, sorted_pair, E, P, off_lds, sp_lds);
  __syncthreads();
  const int32_t* spp = np ? sp_lds : sorted_pair;
  stage_tile_keys(off_lds, spp, E, k, bits_mode, bits, key, ktiles);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int st_tok = tid >> 4, st_pc = tid & 15;

  for (int w = blockIdx.x;; w += gridDim.x) {
    TileInfo tl;
    if (!find_tile_by_key(off_lds, key, ktiles, E, w / RG, tl)) break;
    const int nb = (w % RG) * 64, n0 = nb + 16 * wave;
    int maxb;
    uint32_t hmask;
    const int b = tile_bits(spp, tl.r0, tl.cnt, col, tl.e, k, bits_mode, bits, maxb, hmask);
    const ColWeights cw = col_weights(b);
    const int sj = tl.r0 + (st_tok < tl.cnt ? st_tok : 0);
    const int sp = spp[sj];
    asm volatile("" ::"v"(sp) : "memory");  // routing value taken before any plane load
    const uint16_t* xsrc = x + (size_t)(sp / k) * d + 32 * (st_pc >> 2) + 4 * (st_pc & 3);
    // plane words: tiles of 16 rows, (gate n0, up n0) = rows n0 and f + n0
    const size_t rg = (size_t)tl.e * 2 * f + n0;
    const uint8_t* pt[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
      pt[t] = planes + ((rg + t * (size_t)f) >> 4) * (size_t)G * kBlockBytes + 32 * col + 8 * kq;
    const uint16_t* sc_src = scales + ((size_t)tl.e * 2 * f + nb) * G;
    f32x4 acc[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
    switch (maxb) {  // block-uniform
#define BP_GU_CASE(N) \
  case N:             \
    bp_item<N, kDQ, kSC, false>(xsrc, pt, G, sc_src, f, sc_lds, xs, cw, hmask, acc); \
    break;
      BP_GU_CASE(1) BP_GU_CASE(2) BP_GU_CASE(3) BP_GU_CASE(4)
      BP_GU_CASE(5) BP_GU_CASE(6) BP_GU_CASE(7)
      default:
        bp_item<8, kDQ, kSC, false>(xsrc, pt, G, sc_src, f, sc_lds, xs, cw, hmask, acc);
#undef BP_GU_CASE
    }
    if (col < tl.cnt) {
      // h is stored per 128-group of the down pass's K in that pass's staged
      // order, so the down kernel stages it with plain copies.  The lane's
      // features k4 .. k4 + 3 (k4 % 4 == 0) sit at s + 0, 16, 2, 18 with
      // s = bp_run(k4) + (k4 / 16) % 2.
      uint16_t* hr = h + (size_t)(tl.r0 + col) * f + ((n0 >> 7) << 7);
      const int k4 = (n0 + 4 * kq) & 127, s = bp_run(k4) + ((k4 >> 4) & 1);
      uint16_t hb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        hb[i] = (uint16_t)f32_to_bf16_rne(silu_f32(acc[0][i]) * acc[1][i]);
      hr[s] = hb[0];
      hr[s + 16] = hb[1];
      hr[s + 2] = hb[2];
      hr[s + 18] = hb[3];
    }
    __syncthreads();  // the next item rewrites the scales and the slots
  }
}

// ------------------------------------------------------------------ down
// Down with two row tiles per wave: item = (token tile of up to 16 pairs,
// 128 output rows); wave w computes rows 16 w .. 16 w + 15 and 64 + 16 w ..
// of the item through the gate/up item loop, so the h staging, its barrier
// and the seed MFMAs of a group serve two row tiles, and the two tiles'
// chains interleave on the matrix core.
template <int kDQ, int kWaves, int kSC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWaves, 8)))
void down_bp_decode(const uint16_t* __restrict__ h, const int32_t* __restrict__ offsets,
                     const int32_t* __restrict__ sorted_pair, int E, int k, int P, int d, int f,
                     const uint8_t* __restrict__ planes, const uint16_t* __restrict__ scales,
                     int bits_mode, const uint8_t* __restrict__ bits, float* __restrict__ y) {
  extern __shared__ int32_t lds_i[];
  const int G = f >> 7, RG = d / 128;
  int32_t* off_lds = lds_i;
  int32_t* sp_lds = lds_i + ((E + 1 + 3) & ~3);
  float* sc_lds = (float*)(sp_lds + ((min(P, kPairsInLds) + 3) & ~3));  // [2][G][64]
  uint16_t* xs = (uint16_t*)(sc_lds + 2 * G * 64);                      // [2][16][kXRow]
  int32_t* ktiles = (int32_t*)(xs + 2 * 16 * kXRow);                    // [16]
  int32_t* key = ktiles + 16;                                           // [E]
  const int np = stage_routing(offsets, sorted_pair, E, P, off_lds, sp_lds);
  __syncthreads();
  const int32_t* spp = np ? sp_lds : sorted_pair;
  stage_tile_keys(off_lds, spp, E, k, bits_mode, bits, key, ktiles);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int st_tok = tid >> 4, st_pc = tid & 15;

  for (int w = blockIdx.x;; w += gridDim.x) {
    TileInfo tl;
    if (!find_tile_by_key(off_lds, key, ktiles, E, w / RG, tl)) break;
    const int mb = (w % RG) * 128, m0 = mb + 16 * wave;
    int maxb;
    uint32_t hmask;
    const int b = tile_bits(spp, tl.r0, tl.cnt, col, tl.e, k, bits_mode, bits, maxb, hmask);
    const ColWeights cw = col_weights(b);
    const uint16_t* hsrc = h + (size_t)(tl.r0 + (st_tok < tl.cnt ? st_tok : 0)) * f + 8 * st_pc;
    const size_t r0 = (size_t)tl.e * d + m0;
    const uint8_t* pt[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
      pt[t] = planes + ((r0 + 64 * t) >> 4) * (size_t)G * kBlockBytes + 32 * col + 8 * kq;
    const uint16_t* sc_src = scales + ((size_t)tl.e * d + mb) * G;
    f32x4 acc[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
    switch (maxb) {  // block-uniform
#define BP_DN_CASE(N) \
  case N:             \
    bp_item<N, kDQ, kSC, true>(hsrc, pt, G, sc_src, 64, sc_lds, xs, cw, hmask, acc); \
    break;
      BP_DN_CASE(1) BP_DN_CASE(2) BP_DN_CASE(3) BP_DN_CASE(4)
      BP_DN_CASE(5) BP_DN_CASE(6) BP_DN_CASE(7)
      default:
        bp_item<8, kDQ, kSC, true>(hsrc, pt, G, sc_src, 64, sc_lds, xs, cw, hmask, acc);
#undef BP_DN_CASE
    }
    if (col < tl.cnt) {
      float* yr = y + (size_t)(tl.r0 + col) * d + m0 + 4 * kq;
      *(f32x4*)yr = acc[0];
      *(f32x4*)(yr + 64) = acc[1];
    }
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
                       sizeof(float) * 2 * G * 64 + xs_b + tile_key_bytes(a.E);
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
    const long long work = mt * (a.d / 128);
    const int grid = (int)(work < cap ? work : cap);
    const size_t lds = off_b + sizeof(int32_t) * ((std::min<long long>(P, kPairsInLds) + 3) & ~3) +
                       sizeof(float) * 2 * G * 64 + xs_b + tile_key_bytes(a.E);
    const int sc = scale_chunks(2, G, a.dn_scales);
    auto kern = sc == 1   ? down_bp_decode<kBpDnDQ, kBpDnWaves, 1>
                : sc == 2 ? down_bp_decode<kBpDnDQ, kBpDnWaves, 2>
                : sc == 4 ? down_bp_decode<kBpDnDQ, kBpDnWaves, 4>
                          : down_bp_decode<kBpDnDQ, kBpDnWaves, 0>;
    launch_k(kern, dim3(grid), dim3(256), lds, s, a.ev[2], a.ev[3], h, a.offsets,
             a.sorted_pair, a.E, a.k, (int)P, a.d, a.f, a.dn_codes, a.dn_scales, a.bits_mode,
             a.bits, a.y);
  }
  return hipGetLastError();
}

}  // namespace moe
