// Expert SwiGLU FFN over the grouped pairs with in-kernel dequantization:
// dispatch of the int4 paths (decode and prefill kernels in their own files)
// and the kernels for bitplane-prefix experts.
//  ExactMoE ("Every Expert Counts ...", Abstract): symmetric group-128 W4A16
//    routed experts, executed by grouped kernels, every pair computed.
//  PagedMoE (abstract): bitplane prefixes executed directly at the pair's
//    bit-width, reading only the top planes the expert needs.
//  MatMoE (abstract): floor-and-compensation dequantization of a prefix.
//
// Arithmetic (bitplane): the prefix value v_b in [-128,127] is exact in bf16 and enter a bf16 MFMA with bf16 activations;
// each 128-element group's fp32 partial sum is multiplied by its fp16 scale
// (exact in fp32) and added to the fp32 accumulator.  Dequantized weights
// are therefore never rounded.  h = bf16_rne(silu(g) * u).
//
// Work decomposition: a prep kernel cuts every expert's slot range
// [offsets[e], offsets[e+1]) into tiles of up to 16*NT tokens; block
// (tile, row tile of 16 output features) computes 16 features x the tile's
// tokens with v_mfma_f32_16x16x32_bf16 (weights on M, tokens on N), the four
// waves splitting the K dimension and reducing through LDS in a fixed order.
#include "kcommon.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;

struct Tile {
  int e, r0, cnt, maxb;
};

// Bit-width of pair p (values outside [1, 8] are clamped into it).

// One block of up to 1024 threads, one thread per expert.
__global__ __launch_bounds__(1024) void ffn_prep(
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pair,
    int E, int k, int tok, int bits_mode, const uint8_t* __restrict__ bits,
    Tile* __restrict__ tiles, int* __restrict__ num_tiles) {
  __shared__ int sc[1024];
  const int e = threadIdx.x;
  int lo = 0, n = 0;
  if (e < E) {
    lo = offsets[e];
    n = offsets[e + 1] - lo;
  }
  const int nt = (n + tok - 1) / tok;
  sc[e] = nt;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = (e >= off) ? sc[e - off] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  const int base = sc[e] - nt;
  for (int c = 0; c < nt; ++c) {
    Tile t;
    t.e = e;
    t.r0 = lo + c * tok;
    t.cnt = min(tok, n - c * tok);
    int mb = 0;
    if (bits_mode != 0) {
      for (int r = 0; r < t.cnt; ++r) {
        const int p = sorted_pair[t.r0 + r];
        mb = max(mb, pair_bit_width(p, e, k, bits_mode, bits));
      }
    } else {
      mb = 8;
    }
    t.maxb = mb;
    tiles[base + c] = t;
  }
  if (e == 1023) *num_tiles = sc[1023];
}

// ---------------------------------------------------------------- weights
// bitplane: one dword per plane p < maxb holds bit 7-p of the lane's 32
// elements (bit position = element offset).  Planes are stored per 16-row
// tile and 128-group as a 2 KiB block of plane pairs (kcommon.hpp);
// tb = codes + (row / 16) * G * 2048 + 32 * (row % 16).  For class b the
// K-values are v_b = (u with 8-b low bits cleared) + 2^(7-b) - 128, or
// u - 128 for b = 8.
__device__ __forceinline__ const uint8_t* bp_tile(const uint8_t* codes, size_t row, int G) {
  return codes + (row >> 4) * (size_t)G * kBpBlock + 32 * (row & 15);
}

__device__ __forceinline__ void bp_load(const uint8_t* tb, int g, int kq, int maxb,
                                        uint32_t pl[8]) {
#pragma unroll
  for (int p = 0; p < 8; ++p)
    pl[p] = (p < maxb) ? *(const uint32_t*)(tb + (size_t)g * kBpBlock + kBpPair * (p >> 1) +
                                           8 * kq + 4 * (p & 1))
                       : 0u;
}

__device__ __forceinline__ void bp_frags(const uint32_t pl[8], int b,
                                         bf16x8 a[4]) {
  const int keep = (0xFF << (8 - b)) & 0xFF;
  const int comp = (b == 8) ? -128 : (1 << (7 - b)) - 128;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int u = 0;
#pragma unroll
      for (int p = 0; p < 8; ++p) u |= ((pl[p] >> (8 * j + i)) & 1u) << (7 - p);
      a[j][i] = (__bf16)(float)((u & keep) + comp);
    }
  }
}

// -------------------------------------------------------------- gate / up
template <int NT>
__global__ __launch_bounds__(kThreads) void gateup_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ sorted_pair,
    int k, int d, int f, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, int bits_mode,
    const uint8_t* __restrict__ bits, const Tile* __restrict__ tiles,
    const int* __restrict__ num_tiles, uint16_t* __restrict__ h) {
  if ((int)blockIdx.x >= *num_tiles) return;
  const Tile tl = tiles[blockIdx.x];
  const int n0 = blockIdx.y * 16;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int G = d >> 7;

  const uint16_t* xrow[NT];
  bool valid[NT];
  int tb[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    const int j = 16 * c + col;
    valid[c] = j < tl.cnt;
    const int p = valid[c] ? sorted_pair[tl.r0 + j] : 0;
    xrow[c] = x + (size_t)(p / k) * d;
    tb[c] = valid[c] ? pair_bit_width(p, tl.e, k, bits_mode, bits) : 0;
  }

  const size_t rows2f = (size_t)2 * f;
  const uint16_t* sg = scales + ((size_t)tl.e * rows2f + n0 + 4 * kq) * G;
  const uint16_t* su = sg + (size_t)f * G;

  f32x4 accg[NT], accu[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    accg[c] = f32x4{0, 0, 0, 0};
    accu[c] = f32x4{0, 0, 0, 0};
  }

  // classes of bit-width present in the tile
  uint32_t cls = 0;
  {
#pragma unroll
    for (int c = 0; c < NT; ++c) cls |= valid[c] ? (1u << tb[c]) : 0u;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) cls |= __shfl_xor(cls, o, kWave);
  }

  const int gpw = (G + 3) >> 2;
  const int g0 = wave * gpw, g1 = min(G, g0 + gpw);
  for (int g = g0; g < g1; ++g) {
    float s_g[4], s_u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s_g[i] = f16_bits_to_f32(sg[(size_t)i * G + g]);
      s_u[i] = f16_bits_to_f32(su[(size_t)i * G + g]);
    }
    f32x4 pg[NT], pu[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      pg[c] = f32x4{0, 0, 0, 0};
      pu[c] = f32x4{0, 0, 0, 0};
    }
    {
      uint32_t plg[8], plu[8];
      bp_load(bp_tile(codes, (size_t)tl.e * rows2f + n0 + col, G), g, kq, tl.maxb, plg);
      bp_load(bp_tile(codes, (size_t)tl.e * rows2f + f + n0 + col, G), g, kq, tl.maxb, plu);
      for (int b = 1; b <= 8; ++b) {
        if (!((cls >> b) & 1u)) continue;
        bf16x8 ag[4], au[4];
        bp_frags(plg, b, ag);
        bp_frags(plu, b, au);
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          if (16 * c >= tl.cnt) break;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            u32x4 xb = {0u, 0u, 0u, 0u};
            if (valid[c] && tb[c] == b)
              xb = *(const u32x4*)(xrow[c] + 128 * g + 32 * kq + 8 * j);
            pg[c] = mfma16(ag[j], as_bf16x8(xb), pg[c]);
            pu[c] = mfma16(au[j], as_bf16x8(xb), pu[c]);
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        accg[c][i] = fmaf(s_g[i], pg[c][i], accg[c][i]);
        accu[c][i] = fmaf(s_u[i], pu[c][i], accu[c][i]);
      }
  }

  // fixed-order reduction of the four waves' K-slices
  __shared__ f32x4 red[4][NT][2][64];
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    red[wave][c][0][lane] = accg[c];
    red[wave][c][1][lane] = accu[c];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    if (!valid[c]) continue;
    f32x4 gs = red[0][c][0][lane], us = red[0][c][1][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const f32x4 g2 = red[w][c][0][lane], u2 = red[w][c][1][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gs[i] = gs[i] + g2[i];
        us[i] = us[i] + u2[i];
      }
    }
    uint32_t hb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hb[i] = f32_to_bf16_rne(silu_f32(gs[i]) * us[i]);
    uint2 pk;
    pk.x = hb[0] | (hb[1] << 16);
    pk.y = hb[2] | (hb[3] << 16);
    *(uint2*)(h + (size_t)(tl.r0 + 16 * c + col) * f + n0 + 4 * kq) = pk;
  }
}

// ------------------------------------------------------------------- down
template <int NT>
__global__ __launch_bounds__(kThreads) void down_kernel(
    const uint16_t* __restrict__ h, const int32_t* __restrict__ sorted_pair,
    int k, int d, int f, const uint8_t* __restrict__ codes,
    const uint16_t* __restrict__ scales, int bits_mode,
    const uint8_t* __restrict__ bits, const Tile* __restrict__ tiles,
    const int* __restrict__ num_tiles, float* __restrict__ y) {
  if ((int)blockIdx.x >= *num_tiles) return;
  const Tile tl = tiles[blockIdx.x];
  const int m0 = blockIdx.y * 16;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, kq = lane >> 4;
  const int G = f >> 7;

  const uint16_t* hrow[NT];
  bool valid[NT];
  int tb[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    const int j = 16 * c + col;
    valid[c] = j < tl.cnt;
    hrow[c] = h + (size_t)(tl.r0 + (valid[c] ? j : 0)) * f;
    const int p = valid[c] ? sorted_pair[tl.r0 + j] : 0;
    tb[c] = valid[c] ? pair_bit_width(p, tl.e, k, bits_mode, bits) : 0;
  }
  const uint16_t* sd = scales + ((size_t)tl.e * d + m0 + 4 * kq) * G;

  f32x4 acc[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) acc[c] = f32x4{0, 0, 0, 0};
  uint32_t cls = 0;
  {
#pragma unroll
    for (int c = 0; c < NT; ++c) cls |= valid[c] ? (1u << tb[c]) : 0u;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) cls |= __shfl_xor(cls, o, kWave);
  }

  const int gpw = (G + 3) >> 2;
  const int g0 = wave * gpw, g1 = min(G, g0 + gpw);
  for (int g = g0; g < g1; ++g) {
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = f16_bits_to_f32(sd[(size_t)i * G + g]);
    f32x4 pa[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) pa[c] = f32x4{0, 0, 0, 0};
    {
      uint32_t pl[8];
      bp_load(bp_tile(codes, (size_t)tl.e * d + m0 + col, G), g, kq, tl.maxb, pl);
      for (int b = 1; b <= 8; ++b) {
        if (!((cls >> b) & 1u)) continue;
        bf16x8 a[4];
        bp_frags(pl, b, a);
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          if (16 * c >= tl.cnt) break;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            u32x4 hb = {0u, 0u, 0u, 0u};
            if (valid[c] && tb[c] == b)
              hb = *(const u32x4*)(hrow[c] + 128 * g + 32 * kq + 8 * j);
            pa[c] = mfma16(a[j], as_bf16x8(hb), pa[c]);
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[c][i] = fmaf(s[i], pa[c][i], acc[c][i]);
  }

  __shared__ f32x4 red[4][NT][64];
#pragma unroll
  for (int c = 0; c < NT; ++c) red[wave][c][lane] = acc[c];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    if (!valid[c]) continue;
    f32x4 v = red[0][c][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const f32x4 v2 = red[w][c][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = v[i] + v2[i];
    }
    *(f32x4*)(y + (size_t)(tl.r0 + 16 * c + col) * d + m0 + 4 * kq) = v;
  }
}

constexpr size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t max_tiles(long long P, int E, int tok) {
  return (size_t)((P + tok - 1) / tok + (P < E ? P : E));
}

template <int NT>
hipError_t run_ffn(const FfnArgs& a, hipStream_t s) {
  const long long P = (long long)a.T * a.k;
  const int tok = 16 * NT;
  const size_t mt = max_tiles(P, a.E, tok);
  char* ws = (char*)a.ws;
  int* num_tiles = (int*)ws;
  Tile* tiles = (Tile*)(ws + 256);
  uint16_t* h = (uint16_t*)(ws + 256 + align256(mt * sizeof(Tile)));
  hipLaunchKernelGGL(ffn_prep, dim3(1), dim3(1024), 0, s, a.offsets,
                     a.sorted_pair, a.E, a.k, tok, a.bits_mode,
                     a.bits, tiles, num_tiles);
  dim3 g1((unsigned)mt, a.f / 16), g2((unsigned)mt, a.d / 16);
  launch_k(gateup_kernel<NT>, g1, dim3(kThreads), 0, s, a.ev[0], a.ev[1],
           a.x, a.sorted_pair, a.k, a.d, a.f, a.gu_codes,
                     a.gu_scales, a.bits_mode, a.bits, tiles, num_tiles, h);
  launch_k(down_kernel<NT>, g2, dim3(kThreads), 0, s, a.ev[2], a.ev[3],
           h,
                     a.sorted_pair, a.k, a.d, a.f, a.dn_codes, a.dn_scales,
                     a.bits_mode, a.bits, tiles, num_tiles, a.y);
  return hipGetLastError();
}

}  // namespace

// Workspace: [256 B header | tile list | h bf16 [P][f] | prefill scratch]
size_t ffn_ws_bytes(int T, int k, int E, int d, int f, int format) {
  (void)format;
  const long long P = (long long)T * k;
  const size_t mt = max_tiles(P, E, 16);  // smallest tile -> most tiles
  return 256 + align256(mt * sizeof(Tile)) + align256((size_t)P * f * 2) +
         ffn_prefill_ws_bytes(T, k, E, d, f);
}

hipError_t launch_ffn(const FfnArgs& a, hipStream_t s) {
  const long long P = (long long)a.T * a.k;
  if (P == 0) return hipSuccess;
  uint16_t* h = (uint16_t*)((char*)a.ws + 256 + align256(max_tiles(P, a.E, 16) * sizeof(Tile)));
  if (a.format == 0 && a.path == 1) return launch_ffn_decode_w4(a, h, s);
  if (a.format == 0 && a.path == 2) {
    void* pws = (char*)h + align256((size_t)P * a.f * 2);
    return launch_ffn_prefill_w4(a, h, pws, s);
  }
  // bitplane prefixes (int4 always resolves to one of the two paths above)
  if (a.path == 1 && ffn_decode_bp_applies(P, a.E, a.f)) return launch_ffn_decode_bp(a, h, s);
  if (a.path == 2) {
    void* pws = (char*)h + align256((size_t)P * a.f * 2);
    return launch_ffn_prefill_bp(a, h, pws, s);
  }
  return run_ffn<2>(a, s);
}

}  // namespace moe
