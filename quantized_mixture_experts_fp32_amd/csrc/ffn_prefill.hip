// Prefill-path expert FFN for int4 experts: grouped GEMMs on bf16 MFMA.
//  ExactMoE ("Every Expert Counts ...", Abstract): symmetric group-128 W4A16
//  routed experts, every selected pair computed by grouped kernels.
//
// Layout of the product.  Tokens are the MFMA M dimension (A operand, from
// LDS), output features the N dimension (B operand, int4 codes dequantized
// in registers), so that each lane of a 32x32 accumulator tile owns one
// output feature and needs one fp16 scale per 128-group.
//
// Arithmetic.  A code word becomes eight bf16 values 192 + 8 q (in element
// order) with shifts and v_bitop3: the code, sign bit flipped, lands in the
// top four mantissa bits of 128.0, so that the MFMA sums x * (192 + 8 q)
// and each group's partial sum is corrected by -192 * sum_k x_k.  (Codes in
// the top mantissa bits keep the exact part of every MFMA partial sum small
// next to its signal: the offset is 24 code steps, not the 136 of codes in
// the low bits, so fp32 rounding of the partial sums costs about 6x less.)
// The correction enters as one extra MFMA per group whose A column holds
// the exact three-part bf16 split (hi + mid + lo) of the fp32 group sum of
// the token's activations, and whose B column holds -192.  The running fp32
// total is kept in units of the current group's fp16 scale / 8: before a
// group is accumulated, the total is multiplied by s_prev / s_g, and after
// the last group by the final scale, so every group's sum is weighted by its
// own scale without a separate partial accumulator.  A pre-pass kernel computes the group sums
// (and their splits) of x per token and of h per grouped pair.
//
// Tiling and pipeline: see the GEMM core below.
#include "kcommon.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBT = 128;      // tokens per block tile
constexpr int kRowB = 256;    // LDS bytes per staged token row (chunks swizzled)
constexpr int kBufB = kBT * kRowB;
constexpr int kPfWaves = 2;   // waves per SIMD the register allocation is held to


struct PTile {
  int e, r0, cnt, maxb;
};

// Compile-time count of 32-token blocks in a tile (1..4).
template <int N>
struct TokBlocks {
  static constexpr int value = N;
};

// One code word (elements 8j..8j+7, element 2i in nibble i, 2i+1 in
// nibble 4+i) -> eight bf16 in element order: nibble c goes to mantissa
// bits 3..6 and is XORed into D there.  D = 0x4340 (192.0): two's
// complement codes q -> 192 + 8 q.  D = 0x4300 (128.0): unsigned nibbles
// c -> 128 + 8 c; D = 0x4500 (2048.0): 16 (128 + 8 c).
__device__ __forceinline__ bf16x8 w4_top(uint32_t w, uint32_t D) {
  const uint32_t B = 0x00780078u;
  u32x4 r;
  r[0] = __builtin_amdgcn_bitop3_b32(w << 3, B, D, 0x6A);
  r[1] = __builtin_amdgcn_bitop3_b32(w >> 1, B, D, 0x6A);
  r[2] = __builtin_amdgcn_bitop3_b32(w >> 5, B, D, 0x6A);
  r[3] = __builtin_amdgcn_bitop3_b32(w >> 9, B, D, 0x6A);
  return __builtin_bit_cast(bf16x8, r);
}

// ---------------------------------------------------------------- pre-pass
// For row r (token t of x, or grouped slot of h) and group g: s = fp32 sum
// of the 128 bf16 elements, split exactly into three bf16 parts
// (hi = bf16_rne(s), mid = bf16_rne(s - hi), lo = bf16_rne(s - hi - mid)),
// stored as uint2 {hi | mid << 16, lo}.
__device__ __forceinline__ uint2 split3_bf16(float s) {
  const uint32_t hi = f32_to_bf16_rne(s);
  const float r1 = s - __uint_as_float(hi << 16);
  const uint32_t mid = f32_to_bf16_rne(r1);
  const float r2 = r1 - __uint_as_float(mid << 16);
  const uint32_t lo = f32_to_bf16_rne(r2);
  return uint2{hi | (mid << 16), lo};
}

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
  out[i] = split3_bf16(s);
}

// Barrier that opens a 128-group: every wave's direct-to-LDS loads of the
// group's tile (issued one group earlier) must have landed before any wave
// reads it, and s_barrier does not wait for vector memory by itself, so the
// wait is explicit (it also covers the codes loaded one group ahead, which
// the group consumes right after the barrier anyway).
__device__ __forceinline__ void staged_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt untouched
  __syncthreads();
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
// Pipeline: right after the block barrier that opens 128-group g, the block
// issues the direct-to-LDS loads of group g+1's activation tile (and its
// group sums) into the other buffer, and every wave issues its codes of
// group g+1; all of them have the whole of group g's MFMA work to land
// before the barrier that opens g+1 waits for them.
// Staged tile: row t (256 bytes) holds the token's 128 activations as
// 16-byte chunks, chunk c at position c ^ (t & 15), so that the 32 rows a
// fragment read touches fall on distinct banks.
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
                  float* __restrict__ y_out,                // down:    [P][N]
                  uint2* __restrict__ hsum_out) {           // gate/up: [P][N/128]
  // two staging buffers as distinct objects, so that reads of one are not
  // ordered behind the in-flight direct-to-LDS loads of the other
  __shared__ __attribute__((aligned(16))) uint8_t abuf0[kBufB];
  __shared__ __attribute__((aligned(16))) uint8_t abuf1[kBufB];
  __shared__ uint2 sbuf0[kBT];
  __shared__ uint2 sbuf1[kBT];

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

  // Direct-to-LDS staging: load instruction i of wave w fills rows
  // 32 w + 4 i .. + 3 (1 KiB), lane l writing position l % 16 of row
  // 32 w + 4 i + l / 16; it reads the row's logical chunk (l % 16) ^ (t % 16).
  // Rows past the tile's end read the tile's first row (never stored).
  // Lane offsets are 32-bit and relative to a uniform 64-bit base row: the
  // token row 0 (gate/up: rows < T) or the tile's first slot (down: its
  // slots are consecutive), so they stay below T * K * 2 bytes, which the
  // host checks against 2^32.
  const size_t row0 = kGateUp ? 0 : (size_t)tl.r0;
  const char* act_b = (const char*)(act + row0 * (size_t)K);
  const uint2* gsum_b = gsum + row0 * (size_t)G;
  uint32_t srcoff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = wave * 32 + 4 * i + (lane >> 4);
    const int slot = tl.r0 + (t < tl.cnt ? t : 0);
    const uint32_t src_row =
        kGateUp ? (uint32_t)(sorted_pair[slot] / k_top) : (uint32_t)(slot - (int)row0);
    srcoff[i] = src_row * (uint32_t)K * 2u + 16u * (uint32_t)((lane & 15) ^ (t & 15));
  }
  // group sums: wave w stages tokens 32 w .. + 31, two dwords per token
  uint32_t sumoff;
  {
    const int t = wave * 32 + (lane >> 1);
    const int slot = tl.r0 + (t < tl.cnt ? t : 0);
    const uint32_t src_row =
        kGateUp ? (uint32_t)(sorted_pair[slot] / k_top) : (uint32_t)(slot - (int)row0);
    sumoff = src_row * (uint32_t)G * 8u + 4u * (uint32_t)(lane & 1);
  }
  // (the empty asm hides the offsets' loop invariance, so that the loads
  // keep the uniform-base + 32-bit offset form instead of eight hoisted
  // 64-bit addresses held across the loop)
  auto stage = [&](int g, uint8_t* ab, uint2* sbp) {
    const char* gbase = act_b + 256 * g;  // uniform; per-lane 32-bit offsets
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t o = srcoff[i];
      asm volatile("" : "+v"(o));
      __builtin_amdgcn_global_load_lds(gbase + o,
                                       (__attribute__((address_space(3))) void*)(ab + (wave * 32 + 4 * i) * kRowB),
                                       16, 0, 0);
    }
    __builtin_amdgcn_global_load_lds((const char*)(gsum_b + g) + sumoff,
                                     (__attribute__((address_space(3))) void*)(sbp + wave * 32),
                                     4, 0, 0);
  };
  auto codes_load = [&](int g, u32x4 (&q)[2][2], uint32_t (&sc)[2]) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      q[m][0] = *(const u32x4*)(cb[m] + 1024 * g);
      q[m][1] = *(const u32x4*)(cb[m] + 1024 * g + 16);
      sc[m] = sb[m][g];
    }
  };

  // The tile's group loop is specialised for its count of 32-token blocks:
  // a ragged last tile of an expert runs (and stages) only the token
  // blocks it holds.
  auto run = [&](auto ntb_c) {
    constexpr int NTB = decltype(ntb_c)::value;
    // Running totals are kept in units of the current group's scale / 8:
    // before group g is added, acc *= s_prev / s_g (1 when unchanged); after
    // the last group acc *= s / 8.  All-zero groups (s_g == 0) contribute nothing and keep
    // s_prev.
    f32x16 acc[NTB][2];  // [token block][B block]
#pragma unroll
    for (int t = 0; t < NTB; ++t)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][m][i] = 0.0f;
    float s_cur[2] = {0.0f, 0.0f};

    // B column of the offset MFMA: -192 in K rows 0..2 (lanes of half 0)
    u32x4 negv = {0u, 0u, 0u, 0u};
    if (hh == 0) {
      negv[0] = 0xC340C340u;  // -192, -192
      negv[1] = 0x0000C340u;  // -192, 0
    }
    const bf16x8 negB = __builtin_bit_cast(bf16x8, negv);

    // fragment address of (token block 0, K step 0) in a staged buffer, and
    // the chunk swizzle of K steps 1..7
    const int x16 = c32 & 15;
    const int rd_base = c32 * kRowB + 16 * ((8 * hh) ^ (x16 & 8));
    const int rd_x = 16 * (x16 & 7);

    auto group_step = [&](int g, const uint8_t* ab, const uint2* sbp, uint8_t* ab_next,
                          uint2* sb_next, const u32x4 (&q)[2][2], const uint32_t (&sc)[2],
                          u32x4 (&qn)[2][2], uint32_t (&scn)[2]) {
      staged_barrier();  // group g staged; every wave is done with the other buffer
      if (g + 1 < G) {
        if (wave < NTB) stage(g + 1, ab_next, sb_next);
        codes_load(g + 1, qn, scn);
      }
      // a zero-scale group contributes nothing: the row keeps its running
      // scale and its codes are masked to 0 (which convert to the offset 192
      // that the offset MFMA cancels), whatever codes it holds
      float r[2];
      uint32_t qmask[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const float sg = 0.125f * f16_bits_to_f32(sc[m]);
        const bool upd = sg != 0.0f;
        r[m] = upd ? ((s_cur[m] == 0.0f) ? 0.0f : s_cur[m] / sg) : 1.0f;
        s_cur[m] = upd ? sg : s_cur[m];
        qmask[m] = upd ? 0xFFFFFFFFu : 0u;
      }
      // offset term and rescale, token block by token block
#pragma unroll
      for (int t = 0; t < NTB; ++t) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (hh == 0) {
          const uint2 ss = sbp[t * 32 + c32];
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
      const uint8_t* rd = ab + rd_base;
      bf16x8 af[2][NTB];
#pragma unroll
      for (int t = 0; t < NTB; ++t)
        af[0][t] = __builtin_bit_cast(bf16x8, *(const u32x4*)(rd + t * 32 * kRowB + rd_x));
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) {
        const int cur = s2 & 1;
        if (s2 + 1 < 8) {
          const int off = rd_x ^ (16 * (s2 + 1));
#pragma unroll
          for (int t = 0; t < NTB; ++t)
            af[cur ^ 1][t] =
                __builtin_bit_cast(bf16x8, *(const u32x4*)(rd + t * 32 * kRowB + off));
        }
        bf16x8 bfr[2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
          bfr[m] = w4_top(q[m][s2 >> 2][s2 & 3] & qmask[m], 0x43404340u);
#pragma unroll
        for (int t = 0; t < NTB; ++t)
#pragma unroll
          for (int m = 0; m < 2; ++m) acc[t][m] = mfma32(af[cur][t], bfr[m], acc[t][m]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    u32x4 qa[2][2], qb[2][2];  // [B block][16-byte half] codes of groups g, g + 1
    uint32_t sca[2], scb[2];
    codes_load(0, qa, sca);
    if (wave < NTB) stage(0, abuf0, sbuf0);
    for (int g = 0; g < G; g += 2) {
      group_step(g, abuf0, sbuf0, abuf1, sbuf1, qa, sca, qb, scb);
      if (g + 1 < G) group_step(g + 1, abuf1, sbuf1, abuf0, sbuf0, qb, scb, qa, sca);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int t = 0; t < NTB; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][m][i] *= s_cur[m];

    // ---- epilogue: lane owns feature brow (per B block) for 16 token rows
    // of each token block: rows 8*(i/4) + 4*hh + i%4 of the 32-row block.
    // gate/up also stages its bf16 h in LDS (row tok: the block's 128
    // features, 16-byte chunks swizzled as the activation tile) for the
    // group sums the down pass needs: the block's features are exactly one
    // 128-group of the down GEMM's K.
    uint16_t* hst = (uint16_t*)abuf0;
    if (kGateUp) __syncthreads();  // every wave is done with the staging buffers
    const int lf = wave * 32 + c32;  // gate/up: the lane's feature within the block
#pragma unroll
    for (int t = 0; t < NTB; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tok = t * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
        if (tok >= tl.cnt) continue;
        const size_t slot = (size_t)(tl.r0 + tok);
        if (kGateUp) {
          const float hv = silu_f32(acc[t][0][i]) * acc[t][1][i];
          const uint16_t hb = (uint16_t)f32_to_bf16_rne(hv);
          h_out[slot * N + brow[0]] = hb;
          hst[tok * 128 + 8 * ((lf >> 3) ^ (tok & 15)) + (lf & 7)] = hb;
        } else {
          // y rows are read once, by the combine: streamed past the caches
          if (bstore[0]) __builtin_nontemporal_store(acc[t][0][i], y_out + slot * N + brow[0]);
          if (bstore[1]) __builtin_nontemporal_store(acc[t][1][i], y_out + slot * N + brow[1]);
        }
      }
    if (kGateUp) {
      // the group sum of token tok's 128 h values, in element order (the
      // same fp32 steps as group_sums), split into three bf16 parts
      __syncthreads();
      const int tok = tid;
      if (tok < tl.cnt && tok < kBT) {
        float sum = 0.0f;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const u32x4 v = *(const u32x4*)(hst + tok * 128 + 8 * (c ^ (tok & 15)));
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            sum += __uint_as_float(v[q] << 16);
            sum += __uint_as_float(v[q] & 0xFFFF0000u);
          }
        }
        hsum_out[(size_t)(tl.r0 + tok) * (size_t)(N >> 7) + fblk] = split3_bf16(sum);
      }
    }
  };
  const int ntb = (tl.cnt + 31) >> 5;
  if (ntb >= 4)
    run(TokBlocks<4>{});
  else if (ntb == 3)
    run(TokBlocks<3>{});
  else if (ntb == 2)
    run(TokBlocks<2>{});
  else
    run(TokBlocks<1>{});
}

// Block-wide exclusive scan of v over the 1024 threads (sc: 1024 ints of
// LDS); returns the sum over threads below, and the total in *total.
__device__ __forceinline__ int pf_scan(int v, int* sc, int* total) {
  const int e = threadIdx.x;
  sc[e] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int u = (e >= off) ? sc[e - off] : 0;
    __syncthreads();
    sc[e] += u;
    __syncthreads();
  }
  const int r = sc[e] - v;
  *total = sc[1023];
  __syncthreads();
  return r;
}

// Tiles of up to 128 slots of one expert, heaviest first: every expert's
// full tiles (experts ascending), then the ragged last tiles by their count
// of 32-token blocks, 4 down to 1, so that the lighter blocks fill the tail.
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
  const int nf = n / kBT, rem = n - nf * kBT, nb = (rem + 31) >> 5;
  int total;
  const int basef = pf_scan(nf, sc, &total);
  for (int c = 0; c < nf; ++c) tiles[basef + c] = PTile{e, lo + c * kBT, kBT, 8};
  int base = total;
  for (int v = 4; v >= 1; --v) {
    int tv;
    const int pos = pf_scan(nb == v ? 1 : 0, sc, &tv);
    if (nb == v) tiles[base + pos] = PTile{e, lo + nf * kBT, rem, 8};
    base += tv;
  }
  if (e == 0) *num_tiles = base;
}

// ============================================ bitplane experts, prefill
// PagedMoE (abstract): a pair at width b runs the b-plane prefix of its
// expert directly.  MatMoE (abstract): the b-bit prefix of the 8-bit code u
// dequantizes to v_b(u) = (u with its 8 - b low bits cleared) + 2^(7-b) - 128
// for b < 8, and u - 128 for b = 8.  With planes P0 (most significant) ..
// P7 and unsigned nibbles placed by w4_top (nibble c -> 128 + 8 c):
//   b <= 4: one pass over the nibble (P0, .., P(b-1), zeros), code
//     C = 128 + 2^(7-b) t for the top b bits t, and v_b = 2 (C - 192 +
//     2^(6-b));
//   b > 4: two passes, (P0..P3) converted to 16 C0 and (P4..P7, planes at or
//     past b read as 0) to C1, and 8 v_b = 16 C0 + C1 - 3200 + 8 c_b with
//     c_b = 2^(7-b) for b < 8 and 0 for b = 8.
// So a tile of width b runs the int4 pipeline once or twice over the same
// staged activations, with the group scale times 2 (b <= 4) or 1/8 (b > 4)
// and the constant terms in the one offset MFMA of the group: K rows 0..2
// carry the split group sum against -192 + 2^(6-b) (or -3200), rows 3..5
// the same sum against 0 (or 8 c_b).  Every code sits in the top mantissa
// bits, so the exact part of an MFMA partial sum stays within a few times
// its signal at every width (with codes in the low mantissa bits a 1-bit
// prefix would carry 270 times its signal).
// Codes come from plane words by an in-register bit transpose: four source
// bytes (nibble bits 0..3 of eight elements, bit i = element i) become one
// code word with two delta swaps, which w4_top_bp expands to eight bf16.  Tiles hold pairs of one expert and one width
// (an expert's slots are listed by width, then slot, in `bslot`), so the
// codes of a tile serve all of its token rows.

// Code word of eight elements from the 32-bit word x whose byte b holds
// nibble bit (0, 2, 1, 3)[b] of elements 0..7 (bit i = element i): with
// the bits of x indexed by (byte b1 b0, element e2 e1 e0), the two delta
// swaps exchange index bits 0 <-> 4 and 1 <-> 3, which leaves element e's
// nibble (bit k at 4 n + k) at nibble n = 4 e0 + 2 e1 + e2.
__device__ __forceinline__ uint32_t nib_transpose2(uint32_t x) {
  uint32_t t;
  t = __builtin_amdgcn_bitop3_b32(x >> 15, x, 0x0000AAAAu, 0x28);  // (a ^ b) & c
  x = __builtin_amdgcn_bitop3_b32(x, t, t << 15, 0x96);            // a ^ b ^ c
  t = __builtin_amdgcn_bitop3_b32(x >> 6, x, 0x00CC00CCu, 0x28);
  x = __builtin_amdgcn_bitop3_b32(x, t, t << 6, 0x96);
  return x;
}

// nib_transpose2's word -> eight bf16 in element order (elements 2j, 2j+1
// sit in nibbles n, n + 4 with n = 0, 2, 1, 3 for j = 0..3); the nibble goes
// to mantissa bits 3..6 of D, as w4_top.
__device__ __forceinline__ bf16x8 w4_top_bp(uint32_t w, uint32_t D) {
  const uint32_t B = 0x00780078u;
  u32x4 r;
  r[0] = __builtin_amdgcn_bitop3_b32(w << 3, B, D, 0x6A);
  r[1] = __builtin_amdgcn_bitop3_b32(w >> 5, B, D, 0x6A);
  r[2] = __builtin_amdgcn_bitop3_b32(w >> 1, B, D, 0x6A);
  r[3] = __builtin_amdgcn_bitop3_b32(w >> 9, B, D, 0x6A);
  return __builtin_bit_cast(bf16x8, r);
}

// Pairs of one expert grouped by width, in two launches of one 256-thread
// block per expert.  bp_pf_count: cnt[8 e + w] = pairs of expert e with
// width w + 1 (ballots over the expert's slots).  bp_pf_scatter: the
// expert's slots listed by width, each width in slot order (stable), and
// the 128-pair tiles of every (expert, width), listed in (expert, width)
// order for the down pass and widest first for the gate/up pass; the block
// of the last expert stores the tile count.
__global__ __launch_bounds__(256) void bp_pf_count(const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ sorted_pair,
                                                   int k, int mode,
                                                   const uint8_t* __restrict__ bits,
                                                   int32_t* __restrict__ cnt) {
  __shared__ int32_t part[4][8];
  const int e = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lo = offsets[e], n = offsets[e + 1] - lo;
  int c[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int i0 = 0; i0 < n; i0 += 256) {
    const int i = i0 + (int)threadIdx.x;
    const int b = i < n ? pair_bit_width(sorted_pair[lo + i], e, k, mode, bits) : 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) c[w] += __popcll(__ballot(b == w + 1));
  }
  if (lane < 8) {
    int v = c[0];
#pragma unroll
    for (int w = 1; w < 8; ++w) v = lane == w ? c[w] : v;
    part[wave][lane] = v;
  }
  __syncthreads();
  if (threadIdx.x < 8) {
    const int w = threadIdx.x;
    cnt[8 * e + w] = part[0][w] + part[1][w] + part[2][w] + part[3][w];
  }
}

__global__ __launch_bounds__(256) void bp_pf_scatter(const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ sorted_pair,
                                                     int E, int k, int mode,
                                                     const uint8_t* __restrict__ bits,
                                                     const int32_t* __restrict__ cnt,
                                                     int32_t* __restrict__ bslot,
                                                     PTile* __restrict__ tiles,
                                                     PTile* __restrict__ tiles_wide,
                                                     int* __restrict__ num_tiles) {
  __shared__ int32_t redb[4][8], redt[4][8];
  __shared__ int32_t sbase[8];
  __shared__ int32_t chunk[4][8];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Two lists of the same tiles.  tiles: expert-major (experts ascending,
  // widths ascending within an expert), so that an expert's tiles of
  // different widths, which read the same leading planes, run close
  // together.  tiles_wide: widest first (width 8 down to 1, experts
  // ascending within a width), so that the two-pass tiles of widths above
  // 4 start first and one-pass tiles fill the tail.  Thread tid counts the
  // tiles of width tid % 8 + 1 of the experts below e and of all experts.
  int tb_below = 0, tb_all = 0;
  for (int j = tid; j < 8 * E; j += 256) {
    const int tl = (cnt[j] + kBT - 1) / kBT;
    tb_all += tl;
    if ((j >> 3) < e) tb_below += tl;
  }
#pragma unroll
  for (int o = 8; o < 64; o <<= 1) {
    tb_below += __shfl_xor(tb_below, o, kWave);
    tb_all += __shfl_xor(tb_all, o, kWave);
  }
  if (lane < 8) {
    redb[wave][lane] = tb_below;
    redt[wave][lane] = tb_all;
  }
  __syncthreads();
  if (tid < 8) {
    // expert-major: tiles of all widths of the experts below e, then of
    // the narrower widths of e; widest first: tiles of the wider widths,
    // then of this width of the experts below e
    int sb = offsets[e], tb = 0, tw = 0;
    for (int w = 0; w < 8; ++w) {
      const int below = redb[0][w] + redb[1][w] + redb[2][w] + redb[3][w];
      tb += below;
      if (w < tid) {
        sb += cnt[8 * e + w];
        tb += (cnt[8 * e + w] + kBT - 1) / kBT;
      }
      if (w > tid) tw += redt[0][w] + redt[1][w] + redt[2][w] + redt[3][w];
      if (w == tid) tw += below;
    }
    sbase[tid] = sb;
    const int nw = cnt[8 * e + tid];
    for (int c2 = 0; c2 * kBT < nw; ++c2) {
      const PTile t = PTile{e, sb + c2 * kBT, min(kBT, nw - c2 * kBT), tid + 1};
      tiles[tb + c2] = t;
      tiles_wide[tw + c2] = t;
    }
    if (e == E - 1 && tid == 7) *num_tiles = tb + (nw + kBT - 1) / kBT;
  }
  __syncthreads();
  // slot lists: 256 slots per round; a slot's place within its width is the
  // count of earlier slots of that width (earlier rounds, earlier waves of
  // this round, lower lanes of its wave)
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const int lo = offsets[e], n = offsets[e + 1] - lo;
  int run[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int i0 = 0; i0 < n; i0 += 256) {
    const int i = i0 + tid;
    const int b = i < n ? pair_bit_width(sorted_pair[lo + i], e, k, mode, bits) : 0;
    uint64_t mine = 0;
    int cw = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint64_t m = __ballot(b == w + 1);
      if (b == w + 1) mine = m;
      if (lane == w) cw = __popcll(m);
    }
    if (lane < 8) chunk[wave][lane] = cw;
    __syncthreads();
    if (b) {
      int pos = sbase[b - 1] + run[b - 1] + __popcll(mine & below);
      for (int v = 0; v < wave; ++v) pos += chunk[v][b - 1];
      bslot[pos] = lo + i;
    }
#pragma unroll
    for (int w = 0; w < 8; ++w) run[w] += chunk[0][w] + chunk[1][w] + chunk[2][w] + chunk[3][w];
    __syncthreads();  // the next round rewrites chunk
  }
}

template <bool kGateUp>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kPfWaves, kPfWaves)))
void pf_bp_kernel(const uint16_t* __restrict__ act,       // x [T][K] or h [P][K]
                  const int32_t* __restrict__ sorted_pair,  // gate/up: gather
                  const int32_t* __restrict__ bslot,        // tile rows -> slots
                  int k_top, int K, int N,
                  const uint8_t* __restrict__ planes,       // [E*rows/16][K/128] 2 KiB blocks
                  const uint16_t* __restrict__ scales,      // [E][rows][K/128]
                  const uint2* __restrict__ gsum,           // [rows of act][K/128]
                  const PTile* __restrict__ tiles, const int* __restrict__ num_tiles, int nfb,
                  uint16_t* __restrict__ h_out, float* __restrict__ y_out,
                  uint2* __restrict__ hsum_out) {  // gate/up: [P][N/128]
  __shared__ __attribute__((aligned(16))) uint8_t abuf0[kBufB];
  __shared__ __attribute__((aligned(16))) uint8_t abuf1[kBufB];
  __shared__ uint2 sbuf0[kBT];
  __shared__ uint2 sbuf1[kBT];

  // same XCD-aware tile order as the int4 kernel
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int tile = (local / nfb) * 8 + xcd, fblk = local % nfb;
  if (tile >= *num_tiles) return;
  const PTile tl = tiles[tile];
  const int nb = tl.maxb;  // the tile's width, 1..8
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
  // lane half hh reads quarters 2 hh and 2 hh + 1 of its row in each plane
  // pair (one 16-byte load at 512 c + 32 r + 16 hh of the group's block:
  // both planes' words of the two quarters): elements 64 hh .. 64 hh + 63
  // of the group, the int4 lane split.  Addresses are a uniform base
  // (expert, group, pair) plus a 32-bit lane offset within the expert (its
  // nrows * K bytes).
  const uint8_t* pe = planes + ebase * (size_t)K;  // 2 KiB blocks: 16 rows x 4 plane pairs
  const uint16_t* se = scales + ebase * (size_t)G;
  uint32_t lo_p[2], lo_s[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    lo_p[m] = (uint32_t)(brow[m] >> 4) * (uint32_t)G * 2048u + 32u * (uint32_t)(brow[m] & 15) +
              16u * (uint32_t)hh;
    lo_s[m] = (uint32_t)brow[m] * (uint32_t)G;
  }

  // 32-bit lane offsets from a uniform base row, as in the int4 kernel; a
  // tile lists slots of one (expert, width) in ascending order, so its
  // first slot is the smallest and the offsets stay below T * K * 2 bytes
  // (an expert receives at most T pairs).
  const size_t row0 = kGateUp ? 0 : (size_t)bslot[tl.r0];
  const char* act_b = (const char*)(act + row0 * (size_t)K);
  const uint2* gsum_b = gsum + row0 * (size_t)G;
  uint32_t srcoff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = wave * 32 + 4 * i + (lane >> 4);
    const int slot = bslot[tl.r0 + (t < tl.cnt ? t : 0)];
    const uint32_t src_row =
        kGateUp ? (uint32_t)(sorted_pair[slot] / k_top) : (uint32_t)(slot - (int)row0);
    srcoff[i] = src_row * (uint32_t)K * 2u + 16u * (uint32_t)((lane & 15) ^ (t & 15));
  }
  uint32_t sumoff;
  {
    const int t = wave * 32 + (lane >> 1);
    const int slot = bslot[tl.r0 + (t < tl.cnt ? t : 0)];
    const uint32_t src_row =
        kGateUp ? (uint32_t)(sorted_pair[slot] / k_top) : (uint32_t)(slot - (int)row0);
    sumoff = src_row * (uint32_t)G * 8u + 4u * (uint32_t)(lane & 1);
  }
  // (empty asm: as in the int4 kernel)
  auto stage = [&](int g, uint8_t* ab, uint2* sbp) {
    const char* gbase = act_b + 256 * g;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t o = srcoff[i];
      asm volatile("" : "+v"(o));
      __builtin_amdgcn_global_load_lds(gbase + o,
                                       (__attribute__((address_space(3))) void*)(ab + (wave * 32 + 4 * i) * kRowB),
                                       16, 0, 0);
    }
    __builtin_amdgcn_global_load_lds((const char*)(gsum_b + g) + sumoff,
                                     (__attribute__((address_space(3))) void*)(sbp + wave * 32),
                                     4, 0, 0);
  };

  // A pass reads four plane words per B block: nibble bit kb of pass j is
  // plane 4 j + 3 - kb, from pair 2 j + pi (pi = 0: planes 4 j, 4 j + 1;
  // pi = 1: planes 4 j + 2, 4 j + 3) at byte offset poff[j][pi] of the
  // group's 2 KiB block; pairs at or past the width read the last present
  // one and planes at or past the width are masked to zero (keep[j] holds
  // 0xFF in the bytes kept).
  uint32_t poff[2][2], keep[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int pi = 0; pi < 2; ++pi)
      poff[j][pi] = (uint32_t)kBpPair * (uint32_t)min(2 * j + pi, (nb - 1) >> 1);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      keep[j] |= 4 * j + 3 - kb < nb ? 0xFFu << (8 * kb) : 0u;
  }
  // U[m][pi] keeps the loaded order: words (plane 4 j + 2 pi, quarter
  // 2 hh), (plane 4 j + 2 pi + 1, quarter 2 hh), then the same for quarter
  // 2 hh + 1; nibble bit kb's plane 4 j + 3 - kb is pi = (3 - kb) / 2,
  // s = (3 - kb) % 2, its words U[m][pi][s] and U[m][pi][2 + s].
  auto unit_load = [&](int g, int pass, u32x4 (&U)[2][2]) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int pi = 0; pi < 2; ++pi) {
        uint32_t o = lo_p[m];
        asm volatile("" : "+v"(o));  // keep the uniform-base + offset form
        U[m][pi] = *(const u32x4*)(pe + ((size_t)g * 2048 + poff[pass][pi]) + o);
      }
  };
  // A group whose scale is 0 contributes nothing (its weights s * v are 0
  // whatever the planes hold; the quantizer stores u = 128 there, whose
  // b-bit prefix is 2^(7-b), not 0).  The lane's row keeps its running scale
  // for such a group, all its plane words are masked to 0, and its offset
  // column (offZ below) cancels what zero nibbles convert to, so the group
  // adds exactly 0 up to the fp32 rounding of that cancellation.
  bool zrow[2] = {false, false};
  // zero the absent planes of a pass (keep mask uniform per pass) and every
  // plane of a zero-scale row
  auto unit_fix = [&](u32x4 (&U)[2][2], uint32_t kp) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint32_t km = ((kp >> (8 * kb)) & 0xFFu) && !zrow[m] ? 0xFFFFFFFFu : 0u;
        const int pi = (3 - kb) >> 1, s = (3 - kb) & 1;
        U[m][pi][s] &= km;
        U[m][pi][2 + s] &= km;
      }
  };
  // step s2's word: byte b = byte s2 of the source of nibble bit (0, 2,
  // 1, 3)[b]
  auto code_word = [&](const u32x4 (&S)[2], int s2) {
    const int sh = 8 * (s2 & 3);
    auto byte = [&](int kb) {
      const int pi = (3 - kb) >> 1, s = (3 - kb) & 1;
      return (S[pi][(s2 < 4 ? 0 : 2) + s] >> sh) & 0xFFu;
    };
    return nib_transpose2(byte(0) | (byte(2) << 8) | (byte(1) << 16) | (byte(3) << 24));
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][m][i] = 0.0f;
  float s_cur[2] = {0.0f, 0.0f};

  // group scale multiplier and the offset MFMA's B column (all constants
  // are exact in bf16)
  const float smul = nb > 4 ? 0.125f : 2.0f;
  uint32_t hi3, lo3;  // bf16 constants of K rows 0..2 and 3..5
  if (nb > 4) {
    hi3 = f32_to_bf16_rne(-3200.0f);
    lo3 = f32_to_bf16_rne((float)(nb == 8 ? 0 : 8 << (7 - nb)));
  } else {
    hi3 = f32_to_bf16_rne((float)(-192 + (1 << (6 - nb))));
    lo3 = 0u;
  }
  u32x4 offv = {0u, 0u, 0u, 0u};
  if (hh == 0) {
    offv[0] = hi3 | (hi3 << 16);
    offv[1] = hi3 | (lo3 << 16);
    offv[2] = lo3 | (lo3 << 16);
  }
  const bf16x8 offB = __builtin_bit_cast(bf16x8, offv);
  // offset column of a zero-scale row: zero nibbles convert to 2048 + 128
  // (two passes) or 128 (one pass) per element, cancelled in K rows 0..2
  u32x4 offz = {0u, 0u, 0u, 0u};
  if (hh == 0) {
    const uint32_t z3 = f32_to_bf16_rne(nb > 4 ? -2176.0f : -128.0f);
    offz[0] = z3 | (z3 << 16);
    offz[1] = z3;
  }
  const bf16x8 offZ = __builtin_bit_cast(bf16x8, offz);
  const uint32_t D0 = nb > 4 ? 0x45004500u : 0x43004300u;

  const int x16 = c32 & 15;
  const int rd_base = c32 * kRowB + 16 * ((8 * hh) ^ (x16 & 8));
  const int rd_x = 16 * (x16 & 7);

  // rescale to group g's scale and add its offset term
  auto group_head = [&](const uint2* sbp, const uint32_t (&sc)[2]) {
    float r[2];
    bf16x8 ob[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float sg = smul * f16_bits_to_f32(sc[m]);
      const bool upd = sg != 0.0f;
      r[m] = upd ? ((s_cur[m] == 0.0f) ? 0.0f : s_cur[m] / sg) : 1.0f;
      s_cur[m] = upd ? sg : s_cur[m];
      zrow[m] = !upd;
      ob[m] = upd ? offB : offZ;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (hh == 0) {
        const uint2 ss = sbp[t * 32 + c32];  // {hi | mid << 16, lo}
        v[0] = ss.x;
        v[1] = ss.y | (ss.x << 16);          // lo, hi
        v[2] = (ss.x >> 16) | (ss.y << 16);  // mid, lo
      }
      const bf16x8 sumA = __builtin_bit_cast(bf16x8, v);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][m][i] *= r[m];
        acc[t][m] = mfma32(sumA, ob[m], acc[t][m]);
      }
    }
  };
  // The B fragments of K step s2 + 1 are converted in the same scheduling
  // region as the MFMAs of step s2 (independent work the VALU does while
  // the matrix core runs).
  auto run_pass = [&](const uint8_t* ab, const u32x4 (&U)[2][2], uint32_t D) {
    const uint8_t* rd = ab + rd_base;
    bf16x8 af[2][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      af[0][t] = __builtin_bit_cast(bf16x8, *(const u32x4*)(rd + t * 32 * kRowB + rd_x));
    bf16x8 bfr[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m) bfr[0][m] = w4_top_bp(code_word(U[m], 0), D);
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) {
      const int cur = s2 & 1;
      if (s2 + 1 < 8) {
        const int off = rd_x ^ (16 * (s2 + 1));
#pragma unroll
        for (int t = 0; t < 4; ++t)
          af[cur ^ 1][t] = __builtin_bit_cast(bf16x8, *(const u32x4*)(rd + t * 32 * kRowB + off));
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int m = 0; m < 2; ++m) acc[t][m] = mfma32(af[cur][t], bfr[cur][m], acc[t][m]);
      if (s2 + 1 < 8) {
#pragma unroll
        for (int m = 0; m < 2; ++m) bfr[cur ^ 1][m] = w4_top_bp(code_word(U[m], s2 + 1), D);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto scales_load = [&](int g, uint32_t (&sc)[2]) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      uint32_t o = lo_s[m];
      asm volatile("" : "+v"(o));
      sc[m] = (se + g)[o];
    }
  };

  if (nb > 4) {
    // two passes per group: UA = planes 0..3 of group g (loaded one group
    // ahead), UB = planes 4..7 (loaded at the group's start)
    u32x4 UA[2][2], UB[2][2];
    uint32_t sc[2];
    unit_load(0, 0, UA);
    scales_load(0, sc);
    stage(0, abuf0, sbuf0);
    auto gstep = [&](int g, uint8_t* ab, uint2* sbp, uint8_t* ab_next, uint2* sb_next) {
      staged_barrier();
      if (g + 1 < G) stage(g + 1, ab_next, sb_next);
      unit_load(g, 1, UB);
      group_head(sbp, sc);
      unit_fix(UA, keep[0]);
      run_pass(ab, UA, D0);
      if (g + 1 < G) {
        unit_load(g + 1, 0, UA);
        scales_load(g + 1, sc);
      }
      unit_fix(UB, keep[1]);
      run_pass(ab, UB, 0x43004300u);
    };
    for (int g = 0; g < G; g += 2) {
      gstep(g, abuf0, sbuf0, abuf1, sbuf1);
      if (g + 1 < G) gstep(g + 1, abuf1, sbuf1, abuf0, sbuf0);
    }
  } else {
    u32x4 UA[2][2], UB[2][2];
    uint32_t sca[2], scb[2];
    unit_load(0, 0, UA);
    scales_load(0, sca);
    stage(0, abuf0, sbuf0);
    auto gstep = [&](int g, uint8_t* ab, uint2* sbp, uint8_t* ab_next, uint2* sb_next,
                     u32x4 (&U)[2][2], const uint32_t (&sc)[2], u32x4 (&Un)[2][2],
                     uint32_t (&scn)[2]) {
      staged_barrier();
      if (g + 1 < G) {
        stage(g + 1, ab_next, sb_next);
        unit_load(g + 1, 0, Un);
        scales_load(g + 1, scn);
      }
      group_head(sbp, sc);
      unit_fix(U, keep[0]);
      run_pass(ab, U, D0);
    };
    for (int g = 0; g < G; g += 2) {
      gstep(g, abuf0, sbuf0, abuf1, sbuf1, UA, sca, UB, scb);
      if (g + 1 < G) gstep(g + 1, abuf1, sbuf1, abuf0, sbuf0, UB, scb, UA, sca);
    }
  }
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][m][i] *= s_cur[m];

  // gate/up also writes the down pass's group sums of h, as the int4
  // kernel does (the block's features are one 128-group of the down K)
  uint16_t* hst = (uint16_t*)abuf0;
  if (kGateUp) __syncthreads();  // every wave is done with the staging buffers
  const int lf = wave * 32 + c32;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tok = t * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
      if (tok >= tl.cnt) continue;
      const size_t slot = (size_t)bslot[tl.r0 + tok];
      if (kGateUp) {
        const float hv = silu_f32(acc[t][0][i]) * acc[t][1][i];
        const uint16_t hb = (uint16_t)f32_to_bf16_rne(hv);
        h_out[slot * N + brow[0]] = hb;
        hst[tok * 128 + 8 * ((lf >> 3) ^ (tok & 15)) + (lf & 7)] = hb;
      } else {
        // y rows are read once, by the combine: streamed past the caches
        if (bstore[0]) __builtin_nontemporal_store(acc[t][0][i], y_out + slot * N + brow[0]);
        if (bstore[1]) __builtin_nontemporal_store(acc[t][1][i], y_out + slot * N + brow[1]);
      }
    }
  if (kGateUp) {
    __syncthreads();
    const int tok = tid;
    if (tok < tl.cnt && tok < kBT) {
      float sum = 0.0f;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const u32x4 v = *(const u32x4*)(hst + tok * 128 + 8 * (c ^ (tok & 15)));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          sum += __uint_as_float(v[q] << 16);
          sum += __uint_as_float(v[q] & 0xFFFF0000u);
        }
      }
      const size_t slot = (size_t)bslot[tl.r0 + tok];
      hsum_out[slot * (size_t)(N >> 7) + fblk] = split3_bf16(sum);
    }
  }
}

}  // namespace

// Tiles: at most one partial tile per (expert, width) beyond P / 128.
static size_t pf_max_tiles(long long P, int E) {
  const long long nonempty = P < 8LL * E ? P : 8LL * E;
  return (size_t)((P + kBT - 1) / kBT + nonempty);
}

size_t ffn_prefill_ws_bytes(int T, int k, int E, int d, int f) {
  const long long P = (long long)T * k;
  const size_t tiles = pf_max_tiles(P, E);
  auto a256 = [](size_t v) { return (v + 255) & ~(size_t)255; };
  return 256 + a256(tiles * sizeof(PTile)) + a256((size_t)T * (d / 128) * 8) +
         a256((size_t)P * (f / 128) * 8) + a256((size_t)P * sizeof(int32_t)) +
         a256((size_t)E * 8 * sizeof(int32_t)) + a256(tiles * sizeof(PTile));
}

hipError_t launch_ffn_prefill_w4(const FfnArgs& a, uint16_t* h, void* ws, hipStream_t s) {
  const long long P = (long long)a.T * a.k;
  auto a256 = [](size_t v) { return (v + 255) & ~(size_t)255; };
  char* w = (char*)ws;
  int* num_tiles = (int*)w;
  PTile* tiles = (PTile*)(w + 256);
  const size_t mt = (size_t)((P + kBT - 1) / kBT + (P < a.E ? P : a.E));
  uint2* xsum = (uint2*)(w + 256 + a256(pf_max_tiles(P, a.E) * sizeof(PTile)));
  uint2* hsum = (uint2*)((char*)xsum + a256((size_t)a.T * (a.d / 128) * 8));

  hipLaunchKernelGGL(pf_prep, dim3(1), dim3(1024), 0, s, a.offsets, a.E, tiles, num_tiles);
  {
    const long long n = (long long)a.T * (a.d / 128);
    hipLaunchKernelGGL(group_sums, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.x,
                       (long long)a.T, a.d, xsum);
  }
  const unsigned mt8 = (unsigned)((mt + 7) & ~(size_t)7);
  // gate/up writes h and its group sums (the down pass's offset terms)
  launch_k(pf_w4_kernel<true>, dim3(mt8 * (a.f / 128)), dim3(kThreads), 0, s, a.ev[0], a.ev[1],
           a.x, a.sorted_pair, a.k, a.d, a.f, a.gu_codes, a.gu_scales, xsum,
           (const PTile*)tiles, (const int*)num_tiles, a.f / 128, h, (float*)nullptr, hsum);
  const int dn_fb = (a.d + 255) / 256;
  launch_k(pf_w4_kernel<false>, dim3(mt8 * dn_fb), dim3(kThreads), 0, s, a.ev[2], a.ev[3],
           (const uint16_t*)h, a.sorted_pair, a.k, a.f, a.d, a.dn_codes, a.dn_scales,
           (const uint2*)hsum, (const PTile*)tiles, (const int*)num_tiles, dn_fb,
           (uint16_t*)nullptr, a.y, (uint2*)nullptr);
  return hipGetLastError();
}

// Bitplane experts, prefill: tiles of one expert and one width (bp_pf_count,
// bp_pf_scatter),
// then the same two GEMM launches with plane words in place of codes.
hipError_t launch_ffn_prefill_bp(const FfnArgs& a, uint16_t* h, void* ws, hipStream_t s) {
  const long long P = (long long)a.T * a.k;
  auto a256 = [](size_t v) { return (v + 255) & ~(size_t)255; };
  char* w = (char*)ws;
  int* num_tiles = (int*)w;
  PTile* tiles = (PTile*)(w + 256);
  const size_t mt = pf_max_tiles(P, a.E);
  uint2* xsum = (uint2*)(w + 256 + a256(mt * sizeof(PTile)));
  uint2* hsum = (uint2*)((char*)xsum + a256((size_t)a.T * (a.d / 128) * 8));
  int32_t* bslot = (int32_t*)((char*)hsum + a256((size_t)P * (a.f / 128) * 8));
  int32_t* cnt = (int32_t*)((char*)bslot + a256((size_t)P * sizeof(int32_t)));
  PTile* tiles_wide = (PTile*)((char*)cnt + a256((size_t)a.E * 8 * sizeof(int32_t)));

  hipLaunchKernelGGL(bp_pf_count, dim3(a.E), dim3(256), 0, s, a.offsets, a.sorted_pair, a.k,
                     a.bits_mode, a.bits, cnt);
  hipLaunchKernelGGL(bp_pf_scatter, dim3(a.E), dim3(256), 0, s, a.offsets, a.sorted_pair, a.E,
                     a.k, a.bits_mode, a.bits, (const int32_t*)cnt, bslot, tiles, tiles_wide,
                     num_tiles);
  {
    const long long n = (long long)a.T * (a.d / 128);
    hipLaunchKernelGGL(group_sums, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.x,
                       (long long)a.T, a.d, xsum);
  }
  const unsigned mt8 = (unsigned)((mt + 7) & ~(size_t)7);
  launch_k(pf_bp_kernel<true>, dim3(mt8 * (a.f / 128)), dim3(kThreads), 0, s, a.ev[0], a.ev[1],
           a.x, a.sorted_pair, (const int32_t*)bslot, a.k, a.d, a.f, a.gu_codes, a.gu_scales,
           (const uint2*)xsum, (const PTile*)tiles_wide, (const int*)num_tiles, a.f / 128, h,
           (float*)nullptr, hsum);
  const int dn_fb = (a.d + 255) / 256;
  launch_k(pf_bp_kernel<false>, dim3(mt8 * dn_fb), dim3(kThreads), 0, s, a.ev[2], a.ev[3],
           (const uint16_t*)h, a.sorted_pair, (const int32_t*)bslot, a.k, a.f, a.d, a.dn_codes,
           a.dn_scales, (const uint2*)hsum, (const PTile*)tiles, (const int*)num_tiles, dn_fb,
           (uint16_t*)nullptr, a.y, (uint2*)nullptr);
  return hipGetLastError();
}

}  // namespace moe
