// HBM expert slot cache: the host runtime.  The expert bank lives in
// pinned host memory; S device slots hold experts (or, for bitplane
// experts, a prefix of their planes).  Each step routes on the device, reads
// back which experts the routed pairs touch and how many planes each needs,
// assigns slots (resident experts stay; free slots go empty-first, then
// least recently used), copies what is missing on a copy stream, and runs the
// expert FFN over "virtual experts" whose weights are contiguous slot ranges.
//   ExactMoE ("Every Expert Counts ...", Abstract): the routed-expert bank in
//   pinned host memory in front of a device-side expert cache.
//   PagedMoE (abstract): a step fetches only the bitplanes it is missing,
//   and the precision is chosen from routing before any transfer.
// When a step touches more experts than there are slots, chunk 0 runs on
// all S slots (resident experts in place, missing ones loaded into the free
// slots) and the remaining experts stream through the two slot halves:
// chunk c >= 1 loads into half (c - 1) % 2 after the FFN of the last chunk
// that used those slots, so copies of chunk c + 1 overlap the FFN of chunk c.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/moe_wq.h"
#include "launch.hpp"

namespace moe {

struct CacheLoad {
  int e, slot, p0, p1, chunk;  // planes [p0, p1) (int4: the whole expert)
  bool scales;                 // copy the expert's scales too (new slot)
};
struct CacheChunk {
  int v0, n, slot0, wait;  // virtual ids [v0, v0 + n) in slots [slot0, +n);
};                         // wait: FFN chunk the loads follow (-1: none)

struct SlotState {
  int E = 0, S = 0, format = 0;
  std::vector<int32_t> slot_expert;  // -1: empty
  std::vector<int32_t> slot_bits;    // planes resident (int4: 8)
  std::vector<int64_t> slot_last;    // last step that used the slot
  std::vector<int32_t> expert_slot;  // -1: not resident
  void reset() {
    slot_expert.assign(S, -1);
    slot_bits.assign(S, 0);
    slot_last.assign(S, -1);
    expert_slot.assign(E, -1);
  }
};

struct CachePlan {
  std::vector<int32_t> vmap;  // [E] virtual id of each routed expert, -1 else
  std::vector<CacheChunk> chunks;
  std::vector<CacheLoad> loads;
  int V = 0;
  int64_t hits = 0, loads_full = 0, loads_partial = 0;
};

// One step's slot assignment.  need[e]: widest prefix the step uses for e
// (int4: 8), 0 when e has no pair.
void plan_step(SlotState& st, const int32_t* need, int64_t step, CachePlan& pl) {
  const int E = st.E, S = st.S;
  pl.vmap.assign(E, -1);
  pl.chunks.clear();
  pl.loads.clear();
  pl.hits = pl.loads_full = pl.loads_partial = 0;
  auto width = [&](int e) { return st.format == MOE_FMT_W4_SYM ? 8 : need[e]; };
  auto assign = [&](int e, int s, int chunk) {
    const int old = st.slot_expert[s];
    if (old >= 0) st.expert_slot[old] = -1;
    st.slot_expert[s] = e;
    st.slot_bits[s] = width(e);
    st.slot_last[s] = step;
    st.expert_slot[e] = s;
    pl.loads.push_back({e, s, 0, width(e), chunk, true});
    ++pl.loads_full;
  };

  std::vector<char> used(S, 0);
  std::vector<int> misses;
  for (int e = 0; e < E; ++e) {
    if (need[e] <= 0) continue;
    const int s = st.expert_slot[e];
    if (s < 0) {
      misses.push_back(e);
      continue;
    }
    used[s] = 1;
    pl.vmap[e] = s;
    ++pl.hits;
    st.slot_last[s] = step;
    if (width(e) > st.slot_bits[s]) {  // a longer prefix: the missing planes only
      pl.loads.push_back({e, s, st.slot_bits[s], width(e), 0, false});
      st.slot_bits[s] = width(e);
      ++pl.loads_partial;
    }
  }
  std::vector<int> freel;
  for (int s = 0; s < S; ++s)
    if (!used[s]) freel.push_back(s);
  std::stable_sort(freel.begin(), freel.end(), [&](int a, int b) {
    const bool ea = st.slot_expert[a] < 0, eb = st.slot_expert[b] < 0;
    if (ea != eb) return ea;
    return st.slot_last[a] < st.slot_last[b];
  });
  size_t i = 0;
  for (size_t j = 0; j < freel.size() && i < misses.size(); ++j, ++i) {
    assign(misses[i], freel[j], 0);
    pl.vmap[misses[i]] = freel[j];
  }
  pl.chunks.push_back({0, S, 0, -1});
  pl.V = S;
  const int H = S / 2;
  for (int c = 1; i < misses.size(); ++c) {
    const int slot0 = ((c - 1) % 2) * H;
    const int n = (int)std::min<size_t>(H, misses.size() - i);
    pl.chunks.push_back({pl.V, n, slot0, c >= 3 ? c - 2 : 0});
    for (int j = 0; j < n; ++j, ++i) {
      assign(misses[i], slot0 + j, c);
      pl.vmap[misses[i]] = pl.V + j;
    }
    pl.V += n;
  }
}

// Largest virtual id count a step can produce.
int max_virtual(int E, int S) {
  const int H = S / 2;
  const int rest = E > S ? E - S : 0;
  return S + (rest + H - 1) / H * H;
}

}  // namespace moe

struct moe_cache {
  moe::SlotState st;
  int d = 0, f = 0, format = 0;
  const uint8_t* h_gu = nullptr;
  const uint16_t* h_gus = nullptr;
  const uint8_t* h_dn = nullptr;
  const uint16_t* h_dns = nullptr;
  uint8_t* s_gu = nullptr;
  uint16_t* s_gus = nullptr;
  uint8_t* s_dn = nullptr;
  uint16_t* s_dns = nullptr;
  size_t gu_b = 0, gus_b = 0, dn_b = 0, dns_b = 0;  // bytes per expert
  int Vmax = 0;
  static constexpr int kCopyStreams = 4;  // copy engines fed in parallel
  hipStream_t copy[kCopyStreams] = {};
  std::vector<hipEvent_t> copy_done;  // [chunk][stream]
  std::vector<hipEvent_t> ffn_done;   // [chunk]
  hipEvent_t last = nullptr;          // end of the last step on its stream
  // pinned host memory that the kernels read or write directly (device
  // aliases beside): no copy launches on the step's critical path
  int32_t* host_need = nullptr;   // [2E]: need | cnt, written by the need kernel
  int32_t* host_vmap = nullptr;   // [E], read by the remap kernel
  int32_t* host_items = nullptr;  // [E][2]: (expert, slot) needing scales, read by the gather
  int32_t* dev_need = nullptr;
  int32_t* dev_vmap = nullptr;
  int32_t* dev_items = nullptr;
  std::vector<int> item_begin;    // per chunk, into host_items
  uint8_t* d_gus = nullptr;       // device-resident scale bank [E] (1/32 of
  uint8_t* d_dns = nullptr;       // the int4 bank): slots take theirs by gather
  moe::CachePlan plan;
  int64_t step = 0;
  int64_t stats[6] = {0, 0, 0, 0, 0, 0};  // steps, hits, full loads, partial loads, bytes, chunks
};

namespace {

int cfail(int code, const char* msg) { return moe::set_error(code, "%s", msg); }

bool pinned_host(const void* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return a.type == hipMemoryTypeHost;
}

size_t a256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace: route | need_cnt [2E] | vmap [E] | items [E][2] | vidx [P] |
// bits_v [Vmax] | offsets [Vmax + 1] | sorted_pair [P] | permute | ffn (or
// em scratch)
struct CacheWs {
  void* route;
  int32_t *vidx, *offsets, *sorted_pair;
  uint8_t* bits_v;
  void* perm;
  void* ffn;
  size_t total;
};

CacheWs cache_ws(const moe_cache* c, int T, int k, char* base) {
  const int E = c->st.E, V = c->Vmax;
  const long long P = (long long)T * k;
  CacheWs w{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + o : nullptr;
    o += a256(bytes);
    return p;
  };
  w.route = take(moe::route_ws_bytes(T, E) + 16);
  w.vidx = (int32_t*)take(sizeof(int32_t) * (P + 1));
  w.bits_v = (uint8_t*)take(V + 1);
  w.offsets = (int32_t*)take(sizeof(int32_t) * (V + 1));
  w.sorted_pair = (int32_t*)take(sizeof(int32_t) * (P + 1));
  w.perm = take(moe::permute_ws_bytes(T, k, V) + 16);
  const size_t ffn = moe::ffn_ws_bytes(T, k, V, c->d, c->f, c->format);
  const size_t em = moe::em_h_bytes(c->st.S, c->f);
  w.ffn = take(ffn > em ? ffn : em);
  w.total = o;
  return w;
}

}  // namespace

extern "C" {

int moe_cache_create(int E, int d, int f, int format, int slots,
                     const uint8_t* host_gate_up_codes, const uint16_t* host_gate_up_scales_f16,
                     const uint8_t* host_down_codes, const uint16_t* host_down_scales_f16,
                     uint8_t* slot_gate_up_codes, uint16_t* slot_gate_up_scales_f16,
                     uint8_t* slot_down_codes, uint16_t* slot_down_scales_f16,
                     moe_cache** cache) {
  if (!cache) return cfail(MOE_ERR_INVALID_ARG, "moe_cache_create: null handle pointer");
  *cache = nullptr;
  if (E <= 0 || d <= 0 || f <= 0 || slots < 2)
    return cfail(MOE_ERR_INVALID_ARG, "moe_cache_create: bad size (E, d, f > 0, slots >= 2)");
  if (E > MOE_MAX_EXPERTS) return cfail(MOE_ERR_UNSUPPORTED, "moe_cache_create: E too large");
  if (slots > E) return cfail(MOE_ERR_INVALID_ARG, "moe_cache_create: more slots than experts");
  if (d % MOE_GROUP || f % MOE_GROUP || d > MOE_MAX_D)
    return cfail(MOE_ERR_UNSUPPORTED, "moe_cache_create: d, f must be multiples of 128");
  if (format != MOE_FMT_W4_SYM && format != MOE_FMT_BITPLANE8)
    return cfail(MOE_ERR_INVALID_ARG, "moe_cache_create: unknown format");
  if (!host_gate_up_codes || !host_gate_up_scales_f16 || !host_down_codes ||
      !host_down_scales_f16 || !slot_gate_up_codes || !slot_gate_up_scales_f16 ||
      !slot_down_codes || !slot_down_scales_f16)
    return cfail(MOE_ERR_INVALID_ARG, "moe_cache_create: null pointer");
  if (!pinned_host(host_gate_up_codes) || !pinned_host(host_gate_up_scales_f16) ||
      !pinned_host(host_down_codes) || !pinned_host(host_down_scales_f16))
    return cfail(MOE_ERR_INVALID_ARG,
                 "moe_cache_create: the host expert bank must be pinned host memory");
  moe_cache* c = new (std::nothrow) moe_cache;
  if (!c) return cfail(MOE_ERR_INVALID_ARG, "moe_cache_create: out of host memory");
  c->st.E = E;
  c->st.S = slots;
  c->st.format = format;
  c->st.reset();
  c->d = d;
  c->f = f;
  c->format = format;
  c->h_gu = host_gate_up_codes;
  c->h_gus = host_gate_up_scales_f16;
  c->h_dn = host_down_codes;
  c->h_dns = host_down_scales_f16;
  c->s_gu = slot_gate_up_codes;
  c->s_gus = slot_gate_up_scales_f16;
  c->s_dn = slot_down_codes;
  c->s_dns = slot_down_scales_f16;
  c->gu_b = format == MOE_FMT_W4_SYM ? (size_t)2 * f * d / 2 : (size_t)2 * f * d;
  c->dn_b = format == MOE_FMT_W4_SYM ? (size_t)d * f / 2 : (size_t)d * f;
  c->gus_b = (size_t)2 * f * (d / MOE_GROUP) * 2;
  c->dns_b = (size_t)d * (f / MOE_GROUP) * 2;
  c->Vmax = moe::max_virtual(E, slots);
  const int max_chunks = 1 + (c->Vmax - slots) / (slots / 2) + 1;
  hipError_t e = hipSuccess;
  for (int i = 0; i < moe_cache::kCopyStreams && e == hipSuccess; ++i)
    e = hipStreamCreateWithFlags(&c->copy[i], hipStreamNonBlocking);
  c->copy_done.assign((size_t)max_chunks * moe_cache::kCopyStreams, nullptr);
  c->ffn_done.assign(max_chunks, nullptr);
  for (auto& ev : c->copy_done)
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  for (auto& ev : c->ffn_done)
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->last, hipEventDisableTiming);
  if (e == hipSuccess) e = hipHostMalloc((void**)&c->host_need, sizeof(int32_t) * 2 * E);
  if (e == hipSuccess) e = hipHostMalloc((void**)&c->host_vmap, sizeof(int32_t) * E);
  if (e == hipSuccess) e = hipHostMalloc((void**)&c->host_items, sizeof(int32_t) * 2 * E);
  if (e == hipSuccess) e = hipHostGetDevicePointer((void**)&c->dev_need, c->host_need, 0);
  if (e == hipSuccess) e = hipHostGetDevicePointer((void**)&c->dev_vmap, c->host_vmap, 0);
  if (e == hipSuccess) e = hipHostGetDevicePointer((void**)&c->dev_items, c->host_items, 0);
  if (e == hipSuccess) e = hipMalloc((void**)&c->d_gus, (size_t)E * c->gus_b);
  if (e == hipSuccess) e = hipMalloc((void**)&c->d_dns, (size_t)E * c->dns_b);
  if (e == hipSuccess)
    e = hipMemcpy(c->d_gus, c->h_gus, (size_t)E * c->gus_b, hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy(c->d_dns, c->h_dns, (size_t)E * c->dns_b, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    moe_cache_destroy(c);
    return moe::set_error(MOE_ERR_HIP, "moe_cache_create: %s", hipGetErrorString(e));
  }
  *cache = c;
  return moe::set_error(MOE_OK, "%s", "");
}

void moe_cache_destroy(moe_cache* c) {
  if (!c) return;
  // the last step's kernels read the scale bank and its uploads read the
  // pinned staging buffers: let them finish before anything is freed
  if (c->last) (void)hipEventSynchronize(c->last);
  for (auto st : c->copy)
    if (st) (void)hipStreamSynchronize(st);
  if (c->last) (void)hipEventDestroy(c->last);
  for (auto ev : c->copy_done)
    if (ev) (void)hipEventDestroy(ev);
  for (auto ev : c->ffn_done)
    if (ev) (void)hipEventDestroy(ev);
  for (auto st : c->copy)
    if (st) (void)hipStreamDestroy(st);
  if (c->host_need) (void)hipHostFree(c->host_need);
  if (c->host_vmap) (void)hipHostFree(c->host_vmap);
  if (c->host_items) (void)hipHostFree(c->host_items);
  if (c->d_gus) (void)hipFree(c->d_gus);
  if (c->d_dns) (void)hipFree(c->d_dns);
  delete c;
}

int moe_cache_reset(moe_cache* c) {
  if (!c) return cfail(MOE_ERR_INVALID_ARG, "moe_cache_reset: null cache");
  c->st.reset();
  for (auto& s : c->stats) s = 0;
  c->step = 0;
  return MOE_OK;
}

size_t moe_cache_ws_bytes(const moe_cache* c, int T, int k) {
  if (!c || T < 0 || k <= 0) return 0;
  return cache_ws(c, T, k, nullptr).total;
}

int moe_cache_stats(const moe_cache* c, int64_t* stats6) {
  if (!c || !stats6) return cfail(MOE_ERR_INVALID_ARG, "moe_cache_stats: null pointer");
  for (int i = 0; i < 6; ++i) stats6[i] = c->stats[i];
  return MOE_OK;
}

int moe_cache_slots(const moe_cache* c, int32_t* slot_expert, int32_t* slot_bits) {
  if (!c || !slot_expert || !slot_bits)
    return cfail(MOE_ERR_INVALID_ARG, "moe_cache_slots: null pointer");
  for (int s = 0; s < c->st.S; ++s) {
    slot_expert[s] = c->st.slot_expert[s];
    slot_bits[s] = c->st.slot_bits[s];
  }
  return MOE_OK;
}

// Host-only planner entry point (no device work): one step's assignment on
// caller-held slot state, as moe_cache_forward makes it.
int moe_cache_plan(int E, int slots, int format, int32_t* slot_expert, int32_t* slot_bits,
                   int64_t* slot_last, int64_t step, const int32_t* need, int32_t* vmap,
                   int32_t* chunks, int max_chunks, int* n_chunks, int32_t* loads,
                   int max_loads, int* n_loads, int* V) {
  if (E <= 0 || slots < 2 || slots > E || (format != MOE_FMT_W4_SYM && format != MOE_FMT_BITPLANE8))
    return cfail(MOE_ERR_INVALID_ARG, "moe_cache_plan: bad size or format");
  if (!slot_expert || !slot_bits || !slot_last || !need || !vmap || !chunks || !n_chunks ||
      !loads || !n_loads || !V)
    return cfail(MOE_ERR_INVALID_ARG, "moe_cache_plan: null pointer");
  moe::SlotState st;
  st.E = E;
  st.S = slots;
  st.format = format;
  st.slot_expert.assign(slot_expert, slot_expert + slots);
  st.slot_bits.assign(slot_bits, slot_bits + slots);
  st.slot_last.assign(slot_last, slot_last + slots);
  st.expert_slot.assign(E, -1);
  for (int s = 0; s < slots; ++s) {
    const int e = slot_expert[s];
    if (e >= E || e < -1) return cfail(MOE_ERR_INVALID_ARG, "moe_cache_plan: bad slot table");
    if (e >= 0) {
      if (st.expert_slot[e] >= 0)
        return cfail(MOE_ERR_INVALID_ARG, "moe_cache_plan: expert in two slots");
      st.expert_slot[e] = s;
    }
  }
  for (int e = 0; e < E; ++e)
    if (need[e] < 0 || need[e] > 8) return cfail(MOE_ERR_INVALID_ARG, "moe_cache_plan: need");
  moe::CachePlan pl;
  moe::plan_step(st, need, step, pl);
  if ((int)pl.chunks.size() > max_chunks || (int)pl.loads.size() > max_loads)
    return cfail(MOE_ERR_WORKSPACE, "moe_cache_plan: output arrays too small");
  for (int s = 0; s < slots; ++s) {
    slot_expert[s] = st.slot_expert[s];
    slot_bits[s] = st.slot_bits[s];
    slot_last[s] = st.slot_last[s];
  }
  std::memcpy(vmap, pl.vmap.data(), sizeof(int32_t) * E);
  for (size_t i = 0; i < pl.chunks.size(); ++i) {
    const auto& ch = pl.chunks[i];
    chunks[4 * i + 0] = ch.v0;
    chunks[4 * i + 1] = ch.n;
    chunks[4 * i + 2] = ch.slot0;
    chunks[4 * i + 3] = ch.wait;
  }
  for (size_t i = 0; i < pl.loads.size(); ++i) {
    const auto& l = pl.loads[i];
    int32_t* o = loads + 6 * i;
    o[0] = l.e;
    o[1] = l.slot;
    o[2] = l.p0;
    o[3] = l.p1;
    o[4] = l.chunk;
    o[5] = l.scales ? 1 : 0;
  }
  *n_chunks = (int)pl.chunks.size();
  *n_loads = (int)pl.loads.size();
  *V = pl.V;
  return MOE_OK;
}

}  // extern "C"

namespace {

// Copies of a run of n loads (experts e.., slots s.., the same plane range)
// on copy stream `st`: whole int4 experts, or the plane pairs that hold the
// plane range [p0, p1) of every 2 KiB bitplane block (512 bytes per pair, a
// strided 2-D copy; an odd bound brings its pair's other plane along).  Scales come from the
// device-resident scale bank (cache_scale_gather on the compute stream).
hipError_t enqueue_run(moe_cache* c, const moe::CacheLoad& l, int n, hipStream_t st,
                       int64_t* bytes) {
  const size_t e = (size_t)l.e, s = (size_t)l.slot, m = (size_t)n;
  hipError_t r = hipSuccess;
  auto copy = [&](void* dst, const void* src, size_t len) {
    if (r == hipSuccess) r = hipMemcpyAsync(dst, src, len, hipMemcpyHostToDevice, st);
    *bytes += (int64_t)len;
  };
  if (c->format == MOE_FMT_W4_SYM) {
    copy(c->s_gu + s * c->gu_b, c->h_gu + e * c->gu_b, m * c->gu_b);
    copy(c->s_dn + s * c->dn_b, c->h_dn + e * c->dn_b, m * c->dn_b);
  } else if (l.p1 > l.p0) {
    const size_t c0 = (size_t)l.p0 / 2, c1 = ((size_t)l.p1 + 1) / 2;
    const size_t w = 512 * (c1 - c0), off = 512 * c0;
    auto copy2d = [&](uint8_t* dst, const uint8_t* src, size_t blocks) {
      if (w == 2048) {  // all eight planes: the blocks are contiguous
        copy(dst, src, 2048 * blocks);
        return;
      }
      if (r == hipSuccess)
        r = hipMemcpy2DAsync(dst + off, 2048, src + off, 2048, w, blocks, hipMemcpyHostToDevice,
                             st);
      *bytes += (int64_t)(w * blocks);
    };
    copy2d(c->s_gu + s * c->gu_b, c->h_gu + e * c->gu_b, m * (c->gu_b / 2048));
    copy2d(c->s_dn + s * c->dn_b, c->h_dn + e * c->dn_b, m * (c->dn_b / 2048));
  }
  return r;
}

// The loads of one chunk: runs of up to kMaxRun consecutive experts into
// consecutive slots become single copies, spread over the copy streams (the
// least loaded first); each stream first waits for the FFN chunk that last
// used the slots, and records the chunk's copy_done event.  (Measured with
// 16 and 32 slots: one stream or four, whole runs or runs of 1-2 experts
// all move 33-41 GB/s; short runs over four streams were at the top.)
constexpr int kMaxRun = 2;

hipError_t enqueue_chunk_loads(moe_cache* c, int chunk) {
  const auto& ch = c->plan.chunks[chunk];
  constexpr int NS = moe_cache::kCopyStreams;
  hipError_t r = hipSuccess;
  std::vector<const moe::CacheLoad*> ls;
  for (const auto& l : c->plan.loads)
    if (l.chunk == chunk) ls.push_back(&l);
  for (int i = 0; i < NS && r == hipSuccess; ++i)
    if (ch.wait >= 0) r = hipStreamWaitEvent(c->copy[i], c->ffn_done[ch.wait], 0);
  int64_t load[NS] = {};
  for (size_t i = 0; i < ls.size() && r == hipSuccess;) {
    size_t j = i + 1;
    while (j < ls.size() && (int)(j - i) < kMaxRun && ls[j]->e == ls[j - 1]->e + 1 &&
           ls[j]->slot == ls[j - 1]->slot + 1 && ls[j]->p0 == ls[i]->p0 &&
           ls[j]->p1 == ls[i]->p1)
      ++j;
    const int st = (int)(std::min_element(load, load + NS) - load);
    int64_t b = 0;
    r = enqueue_run(c, *ls[i], (int)(j - i), c->copy[st], &b);
    load[st] += b;
    c->stats[4] += b;
    i = j;
  }
  for (int i = 0; i < NS && r == hipSuccess; ++i)
    r = hipEventRecord(c->copy_done[(size_t)chunk * NS + i], c->copy[i]);
  return r;
}

// The compute stream waits for every copy stream's part of a chunk.
hipError_t wait_chunk_loads(moe_cache* c, int chunk, hipStream_t s) {
  hipError_t r = hipSuccess;
  for (int i = 0; i < moe_cache::kCopyStreams && r == hipSuccess; ++i)
    r = hipStreamWaitEvent(s, c->copy_done[(size_t)chunk * moe_cache::kCopyStreams + i], 0);
  return r;
}

}  // namespace

extern "C" int moe_cache_forward(moe_cache* c, const void* x_bf16, const void* wr_bf16,
                                 const float* bias, int T, int k, const uint8_t* bits,
                                 int bits_mode, int32_t* topk_idx, float* topk_w,
                                 int32_t* pair_pos, float* y_pairs, void* out, int out_dtype,
                                 void* ws, size_t ws_bytes, void* stream) {
  if (!c) return cfail(MOE_ERR_INVALID_ARG, "moe_cache_forward: null cache");
  const int E = c->st.E, d = c->d, f = c->f;
  if (T < 0 || k <= 0 || k > E || k > MOE_MAX_TOPK || (long long)T * k >= (1LL << 31))
    return cfail(MOE_ERR_INVALID_ARG, "moe_cache_forward: bad T or k");
  if (c->format == MOE_FMT_W4_SYM) {
    if (bits_mode != MOE_BITS_NONE || bits)
      return cfail(MOE_ERR_INVALID_ARG, "moe_cache_forward: int4 takes MOE_BITS_NONE");
  } else if (bits_mode == MOE_BITS_RANK_RULE) {
    if (k != 8) return cfail(MOE_ERR_UNSUPPORTED, "the rank bit-width rule needs k == 8");
  } else if (bits_mode == MOE_BITS_PER_PAIR || bits_mode == MOE_BITS_PER_EXPERT) {
    if (T > 0 && !bits) return cfail(MOE_ERR_INVALID_ARG, "moe_cache_forward: bits is NULL");
  } else {
    return cfail(MOE_ERR_INVALID_ARG, "moe_cache_forward: bitplane format needs a bits mode");
  }
  if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_F32)
    return cfail(MOE_ERR_INVALID_ARG, "moe_cache_forward: unknown out_dtype");
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !wr_bf16 || !topk_idx || !topk_w || !pair_pos || !y_pairs || !out)
    return cfail(MOE_ERR_INVALID_ARG, "moe_cache_forward: null pointer");
  auto al = [](const void* p, size_t a) { return ((uintptr_t)p % a) == 0; };
  if (!al(x_bf16, 16) || !al(wr_bf16, 16) || !al(y_pairs, 16) || !al(out, 16) ||
      !al(topk_idx, 4) || !al(topk_w, 4) || !al(pair_pos, 4) || (bias && !al(bias, 4)))
    return cfail(MOE_ERR_INVALID_ARG, "moe_cache_forward: misaligned pointer");
  const size_t need_b = cache_ws(c, T, k, nullptr).total;
  if (!ws || ws_bytes < need_b || !al(ws, 256))
    return cfail(MOE_ERR_WORKSPACE, "moe_cache_forward: workspace missing, small or misaligned");

  const hipStream_t s = (hipStream_t)stream;
  const CacheWs w = cache_ws(c, T, k, (char*)ws);
  const long long P = (long long)T * k;
  hipError_t r = moe::launch_route(x_bf16, wr_bf16, bias, T, d, E, k, topk_idx, topk_w,
                                   w.route, s);
  if (r == hipSuccess)  // straight into pinned host memory
    r = moe::launch_cache_need(topk_idx, (int)P, k, E, c->format, bits_mode, bits, c->dev_need,
                               s);
  if (r == hipSuccess) r = hipStreamSynchronize(s);  // the routing decides the copies
  if (r != hipSuccess) goto hip_error;
  {
    moe::plan_step(c->st, c->host_need, c->step, c->plan);
    const auto& pl = c->plan;
    ++c->step;
    c->stats[0] += 1;
    c->stats[1] += pl.hits;
    c->stats[2] += pl.loads_full;
    c->stats[3] += pl.loads_partial;
    c->stats[5] += (int64_t)pl.chunks.size();
    std::memcpy(c->host_vmap, pl.vmap.data(), sizeof(int32_t) * E);
    // experts new to their slots, chunk by chunk: their scales are gathered
    // from the resident scale bank right before the chunk's FFN
    const int nch_all = (int)pl.chunks.size();
    c->item_begin.assign(nch_all + 1, 0);
    int ni = 0;
    for (int ci = 0; ci < nch_all; ++ci) {
      c->item_begin[ci] = ni;
      for (const auto& l : pl.loads)
        if (l.chunk == ci && l.scales) {
          c->host_items[2 * ni] = l.e;
          c->host_items[2 * ni + 1] = l.slot;
          ++ni;
        }
    }
    c->item_begin[nch_all] = ni;
    // the remap and gather kernels read the map and the items from pinned
    // host memory, which the host rewrites only after the next step's sync
    const bool per_expert = bits_mode == MOE_BITS_PER_EXPERT;
    r = moe::launch_cache_remap(topk_idx, (int)P, E, c->dev_vmap, w.vidx,
                                per_expert ? bits : nullptr, per_expert ? w.bits_v : nullptr, s);
    if (r == hipSuccess) r = enqueue_chunk_loads(c, 0);
    if (r == hipSuccess) r = wait_chunk_loads(c, 0, s);
    if (r != hipSuccess) goto hip_error;

    const int nch = (int)pl.chunks.size();
    const uint8_t* fbits = per_expert ? w.bits_v : bits;
    auto ffn_args = [&](int ci, int path) {
      const auto& ch = pl.chunks[ci];
      moe::FfnArgs a{(const uint16_t*)x_bf16, w.offsets + ch.v0, w.sorted_pair, T, k, ch.n,
                     d, f, c->format, c->s_gu + (size_t)ch.slot0 * c->gu_b,
                     (const uint16_t*)((const char*)c->s_gus + (size_t)ch.slot0 * c->gus_b),
                     c->s_dn + (size_t)ch.slot0 * c->dn_b,
                     (const uint16_t*)((const char*)c->s_dns + (size_t)ch.slot0 * c->dns_b),
                     per_expert ? fbits + ch.v0 : fbits, bits_mode, y_pairs, w.ffn, path,
                     {nullptr, nullptr, nullptr, nullptr}};
      return a;
    };
    auto chunk_pairs = [&](int ci) {
      long long n = 0;
      for (int e = 0; e < E; ++e) {
        const int v = pl.vmap[e];
        if (v >= pl.chunks[ci].v0 && v < pl.chunks[ci].v0 + pl.chunks[ci].n)
          n += c->host_need[E + e];
      }
      return n;
    };
    auto gather_scales = [&](int ci) {
      const int i0 = c->item_begin[ci], n = c->item_begin[ci + 1] - i0;
      return moe::launch_cache_scale_gather(c->dev_items + 2 * i0, n, c->d_gus, c->d_dns, c->s_gus,
                                            c->s_dns, c->gus_b, c->dns_b, s);
    };
    auto path_of = [&](int ci) {
      const long long pc = chunk_pairs(ci);
      return (pc <= 8LL * pl.chunks[ci].n || T <= 16) ? MOE_PATH_DECODE : MOE_PATH_PREFILL;
    };
    if (nch == 1 && path_of(0) == MOE_PATH_DECODE &&
        moe::em_applies(T, k, c->st.S, d, f, c->format)) {
      // expert-major decode over the slots: grouping inside its gate/up
      moe::FfnArgs a = ffn_args(0, MOE_PATH_DECODE);
      r = gather_scales(0);
      if (r == hipSuccess)
        r = moe::launch_ffn_decode_em(a, w.vidx, w.offsets, w.sorted_pair, pair_pos,
                                      (uint16_t*)w.ffn, s);
    } else {
      r = moe::launch_permute(w.vidx, T, k, pl.V, w.offsets, w.sorted_pair, pair_pos, w.perm,
                              s);
      for (int ci = 0; ci < nch && r == hipSuccess; ++ci) {
        if (ci > 0) r = wait_chunk_loads(c, ci, s);
        if (r == hipSuccess) r = gather_scales(ci);
        if (r == hipSuccess) r = moe::launch_ffn(ffn_args(ci, path_of(ci)), s);
        if (r == hipSuccess) r = hipEventRecord(c->ffn_done[ci], s);
        // loads that follow this chunk's FFN: chunks 1 and 2 after chunk 0,
        // chunk ci + 2 after chunk ci
        for (int nx = (ci == 0 ? 1 : ci + 2); nx <= ci + 2 && nx < nch && r == hipSuccess; ++nx)
          r = enqueue_chunk_loads(c, nx);
      }
    }
  }
  if (r == hipSuccess)
    r = moe::launch_combine(y_pairs, pair_pos, topk_w, T, k, d, out, out_dtype == MOE_OUT_F32,
                            s);
  if (r == hipSuccess) r = hipEventRecord(c->last, s);
  if (r == hipSuccess) return moe::set_error(MOE_OK, "%s", "");
hip_error:
  // the slot table may name copies that never ran: start from empty slots
  c->st.reset();
  return moe::set_error(MOE_ERR_HIP, "moe_cache_forward: %s", hipGetErrorString(r));
}
