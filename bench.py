#!/usr/bin/env python3
"""Throughput of the routed-expert W4A16 MoE layer on one MI355X.

One step = one forward pass of the whole layer (route -> group pairs by
expert -> expert SwiGLU FFN with in-kernel dequantization -> combine) over
one batch of synthetic tokens, through the C ABI, with inputs and weights
already resident in HBM.  The headline workload is the largest layer: d=4096,
E=256 experts, top-8, f=2048, symmetric int4 group-128 experts (3.3 GB
packed), router bias N(0,1), decoding T=64 tokens per step; its 8192-token
prefill is reported beside it against the bf16 MFMA peak.

Honest HBM numbers: weight sets that fit the 256 MB Infinity Cache (the
OLMoE-shaped layers, 207.6 MB) are rotated over several device copies of
the packed experts (>= 1 GiB touched between reuses of a copy); every
workload rotates over distinct token batches.

Prints ONE JSON line (rank 0).  --gpus must be 1: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "MoE-layer tokens/s; decode HBM GB/s on expert bytes; prefill MFMA util %"


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only-headline", action="store_true",
                    help="skip the secondary workloads")
    ap.add_argument("--no-headline", action="store_true",
                    help="run only the selected secondary workloads (for profiling one "
                         "workload; the JSON line then has no headline value)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=32,
                    help="tokens of the headline batch in the one-thread oracle run")
    ap.add_argument("--workloads", default="",
                    help="comma list of name filters (spaces as _) for secondary workloads")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the workloads, run one plain device-to-device copy "
                         "of this many MiB (reference dispatch for HBM byte counters)")
    return ap.parse_args()


class Hip:
    """hipEvent helpers from the HIP runtime torch already loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, ev, stream):
        assert self.lib.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) == 0

    def ms(self, a, b):
        t = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(a),
                                            ctypes.c_void_p(b)) == 0
        return t.value

    def destroy(self, ev):
        self.lib.hipEventDestroy(ctypes.c_void_p(ev))


def expert_bytes(cfg, planes=None):
    """Packed bytes of one expert: (gate/up, down) = codes + fp16 scales."""
    d, f = cfg.d, cfg.f
    if cfg.fmt == "w4":
        return 2 * f * d // 2 + 2 * f * (d // 128) * 2, d * f // 2 + d * (f // 128) * 2
    b = 8 if planes is None else planes
    return b * 2 * f * d // 8 + 2 * f * (d // 128) * 2, b * d * f // 8 + d * (f // 128) * 2


class Workload:
    """mode: "fused" (one grouped FFN call per step), "seq-active" (one FFN
    call per activated expert, ids read back from the routing) or "seq-all"
    (one FFN call per expert, no read-back).  budget_bits (bitplane layers):
    per-expert widths from the read-budget allocator at that many bits per
    weight on average over the routing counts of the workload's batches,
    instead of the rank rule."""

    def __init__(self, name, cid, T, steps, path=0, mode="fused", budget_bits=None,
                 slots=None):
        self.name, self.cid, self.T, self.steps, self.path = name, cid, T, steps, path
        self.mode, self.budget_bits, self.slots = mode, budget_bits, slots


def run_cache_workload(wl, warmup, hip, torch, np, synth, moe):
    """Layer steps with the expert bank in pinned host memory behind
    `wl.slots` HBM slots (moe_cache_forward): each step routes a fresh batch,
    copies the experts (bitplane: the planes) it is missing, then computes.
    The step time includes the host round trip of the routing result and the
    host-to-device copies."""
    cfg = synth.CONFIGS[wl.cid]
    T, d, E, k, f = wl.T, cfg.d, cfg.E, cfg.k, cfg.f
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    bp = cfg.fmt == "bp8"
    quant = moe.moe_quantize_bitplane8 if bp else moe.moe_quantize_w4
    w = torch.empty((E, 2 * f, d), dtype=torch.float32, device=dev)
    synth.dev_fill_weight(cfg, synth.T_W_GATE_UP, w.data_ptr(), stream)
    gu = quant(w)
    del w
    w = torch.empty((E, d, f), dtype=torch.float32, device=dev)
    synth.dev_fill_weight(cfg, synth.T_W_DOWN, w.data_ptr(), stream)
    dn = quant(w)
    del w
    wr = torch.empty((E, d), dtype=torch.int16, device=dev)
    synth.dev_fill_router(cfg, wr.data_ptr(), stream)
    bias = None
    if cfg.bias_sigma is not None:
        bias = torch.empty((E,), dtype=torch.float32, device=dev)
        synth.dev_fill_bias(cfg, bias.data_ptr(), stream)
    nx = 16
    xs = []
    for i in range(nx):
        x = torch.empty((T, d), dtype=torch.int16, device=dev)
        synth.dev_fill_x(cfg, x.data_ptr(), T, stream, step=i)
        xs.append(x)
    fmt = moe.MOE_FMT_BITPLANE8 if bp else moe.MOE_FMT_W4_SYM
    bmode = moe.MOE_BITS_RANK_RULE if bp else moe.MOE_BITS_NONE
    cache = moe.ExpertCache(wr, bias, k, f, gu[0], gu[1], dn[0], dn[1], fmt, wl.slots)
    del gu, dn
    # host-to-device rate of one plain 256 MiB copy from pinned memory
    src = torch.empty(256 << 20, dtype=torch.uint8).pin_memory()
    dst = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    c0, c1 = hip.event(), hip.event()
    hip.record(c0, stream)
    dst.copy_(src, non_blocking=True)
    hip.record(c1, stream)
    torch.cuda.synchronize()
    h2d_cal = (256 << 20) / (hip.ms(c0, c1) * 1e-3) / 1e9
    hip.destroy(c0)
    hip.destroy(c1)
    del src, dst
    out = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    # warm-up: one pass over the batches (the first host-to-device reads of
    # each pinned page are slower; timed on its own)
    wu = max(warmup, nx)
    w0 = time.perf_counter()
    for i in range(wu):
        cache.forward(xs[i % nx], out=out, bits_mode=bmode)
    torch.cuda.synchronize()
    warm_ms = 1e3 * (time.perf_counter() - w0) / wu
    st0 = cache.stats()
    t_start, t_end = hip.event(), hip.event()
    hip.record(t_start, stream)
    wall0 = time.perf_counter()
    for i in range(wl.steps):
        cache.forward(xs[(wu + i) % nx], out=out, bits_mode=bmode)
    hip.record(t_end, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = hip.ms(t_start, t_end) / wl.steps
    hip.destroy(t_start)
    hip.destroy(t_end)
    st = {key: v - st0[key] for key, v in cache.stats().items()}
    n = max(st["steps"], 1)
    routed = st["hits"] + st["loads_full"]
    rec = {"workload": wl.name, "config": cfg.name, "T": T, "d": d, "E": E, "k": k, "f": f,
           "format": "bitplane8-rank" if bp else "int4-g128", "slots": wl.slots,
           "ms_per_step": round(ms, 5), "tokens_per_s": round(T / (ms * 1e-3), 1),
           "wall_ms_per_step": round(1e3 * wall / wl.steps, 5),
           "first_pass_ms_per_step": round(warm_ms, 4),
           "hit_rate": round(st["hits"] / max(routed, 1), 4),
           "experts_routed_per_step": round(routed / n, 2),
           "experts_loaded_per_step": round(st["loads_full"] / n, 2),
           "experts_extended_per_step": round(st["loads_partial"] / n, 2),
           "h2d_MB_per_step": round(st["bytes"] / n / 1e6, 3),
           "h2d_GBps_of_step_time": round(st["bytes"] / n / (ms * 1e-3) / 1e9, 2),
           "h2d_plain_copy_GBps": round(h2d_cal, 2),
           "ffn_chunks_per_step": round(st["chunks"] / n, 2),
           "note": "bank in pinned host memory; step time includes the routing "
                   "read-back and the host-to-device copies"}
    cache.close()
    return rec


def run_workload(wl, warmup, hip, torch, np, synth, moe):
    cfg = synth.CONFIGS[wl.cid]
    T, d, E, k, f = wl.T, cfg.d, cfg.E, cfg.k, cfg.f
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    bp = cfg.fmt == "bp8"
    quant = moe.moe_quantize_bitplane8 if bp else moe.moe_quantize_w4

    # packed experts (offline, untimed), then copies for cache-cold rotation
    w = torch.empty((E, 2 * f, d), dtype=torch.float32, device=dev)
    synth.dev_fill_weight(cfg, synth.T_W_GATE_UP, w.data_ptr(), stream)
    gu = quant(w)
    del w
    w = torch.empty((E, d, f), dtype=torch.float32, device=dev)
    synth.dev_fill_weight(cfg, synth.T_W_DOWN, w.data_ptr(), stream)
    dn = quant(w)
    del w
    set_bytes = sum(t.numel() * t.element_size() for t in (*gu, *dn))
    ncopies = max(1, min(8, math.ceil(1.1 * 2**30 / set_bytes)))
    copies = [(gu[0], gu[1], dn[0], dn[1])]
    for _ in range(ncopies - 1):
        copies.append(tuple(t.clone() for t in copies[0]))

    wr = torch.empty((E, d), dtype=torch.int16, device=dev)
    synth.dev_fill_router(cfg, wr.data_ptr(), stream)
    bias = None
    if cfg.bias_sigma is not None:
        bias = torch.empty((E,), dtype=torch.float32, device=dev)
        synth.dev_fill_bias(cfg, bias.data_ptr(), stream)
    nx = 16 if T <= 64 else 2
    xs = []
    for i in range(nx):
        x = torch.empty((T, d), dtype=torch.int16, device=dev)
        synth.dev_fill_x(cfg, x.data_ptr(), T, stream, step=i)
        xs.append(x)
    fmt = moe.MOE_FMT_BITPLANE8 if bp else moe.MOE_FMT_W4_SYM
    bmode = moe.MOE_BITS_RANK_RULE if (bp and cfg.bits_rule == "rank") else moe.MOE_BITS_NONE
    layer = moe.MoeLayer(wr, bias, k, f, *copies[0], fmt, bmode, None)
    out = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    alloc = None
    if bp and wl.budget_bits is not None:
        # offline distortion table, routing counts of the workload's batches,
        # then the allocator kernel (each timed on its own, outside the steps)
        ev = [hip.event() for _ in range(4)]
        hip.record(ev[0], stream)
        dist = moe.moe_bp_distortion(gu[0], gu[1], dn[0], dn[1], d, f)
        hip.record(ev[1], stream)
        counts = torch.zeros((E,), dtype=torch.int32, device=dev)
        for x in xs:
            layer.forward(x, out=out, path=wl.path)
            counts += torch.diff(layer.offsets).to(torch.int32)
        lo_b = expert_bytes(cfg, int(wl.budget_bits))
        hi_b = expert_bytes(cfg, int(wl.budget_bits) + 1)
        frac = wl.budget_bits - int(wl.budget_bits)
        per = (1 - frac) * (lo_b[0] + lo_b[1]) + frac * (hi_b[0] + hi_b[1])
        budget = int(int(counts.sum().item()) * per)
        for _ in range(3):
            bits_t, lam_t, read_t = moe.moe_allocate_bits(dist, counts, d, f, 2, 8, budget)
        hip.record(ev[2], stream)
        bits_t, lam_t, read_t = moe.moe_allocate_bits(dist, counts, d, f, 2, 8, budget)
        hip.record(ev[3], stream)
        torch.cuda.synchronize()
        bits_np = bits_t.cpu().numpy()
        dist_np = dist.cpu().numpy()
        cnt_np = counts.cpu().numpy()
        uni = int(wl.budget_bits)
        # the storage layout fetches whole plane pairs: an odd width also
        # brings its pair's other plane
        fetched = sum(int(c) * sum(expert_bytes(cfg, 2 * ((int(b) + 1) // 2)))
                      for c, b in zip(cnt_np, bits_np))
        alloc = {"budget_bits_per_weight": wl.budget_bits, "budget_bytes": budget,
                 "read_bytes": int(read_t.cpu()[0]), "read_bytes_fetched_pairs": fetched,
                 "lambda": float(lam_t.cpu()[0]),
                 "bits_histogram": {int(b): int((bits_np == b).sum()) for b in np.unique(bits_np)},
                 "distortion_table_ms": round(hip.ms(ev[0], ev[1]), 3),
                 "allocator_us": round(1e3 * hip.ms(ev[2], ev[3]), 2),
                 "weighted_distortion_allocated": float(np.sum(cnt_np * dist_np[np.arange(E), bits_np - 1])),
                 "weighted_distortion_uniform_%d" % uni: float(np.sum(cnt_np * dist_np[:, uni - 1])),
                 "weighted_distortion_uniform_%d" % (uni + 1): float(np.sum(cnt_np * dist_np[:, uni]))}
        for h in ev:
            hip.destroy(h)
        layer = moe.MoeLayer(wr, bias, k, f, *copies[0], fmt, moe.MOE_BITS_PER_EXPERT, bits_t)
        bmode = moe.MOE_BITS_PER_EXPERT

    # algorithmic work of each x batch (routing is re-run here, untimed)
    gu_bytes, dn_bytes, active, indep = [], [], [], []
    for x in xs:
        layer.forward(x, out=out, path=wl.path)
        torch.cuda.synchronize()
        idx = layer.topk_idx.cpu().numpy()
        experts = np.unique(idx)
        active.append(len(experts))
        if bp:
            rank_bits = np.array([8, 4, 4, 4, 2, 2, 2, 2])[:k]
            gsum = dsum = isum = 0
            for e in experts:
                widths = ({int(bits_np[e])} if alloc is not None
                          else set(rank_bits[np.nonzero(idx == e)[1]].tolist()))
                g1, d1 = expert_bytes(cfg, max(widths))
                gsum, dsum = gsum + g1, dsum + d1
                # a design keeping each precision as its own object reads one
                # object per distinct (expert, width) (PagedMoE, abstract)
                isum += sum(sum(expert_bytes(cfg, b)) for b in widths)
            gu_bytes.append(gsum)
            dn_bytes.append(dsum)
            indep.append(isum)
        else:
            g1, d1 = expert_bytes(cfg)
            gu_bytes.append(len(experts) * g1)
            dn_bytes.append(len(experts) * d1)
    P = T * k
    flops_gu, flops_dn = 4.0 * P * d * f, 2.0 * P * d * f

    seq_ws = torch.empty((max(moe.moe_ffn_ws_bytes(T, k, 1, d, f, fmt), 256),),
                         dtype=torch.uint8, device=dev)
    launches = []

    bound = {}

    def step(i):
        x, wts = xs[i % nx], copies[i % ncopies]
        if wl.mode == "fused":
            key = (i % nx, i % ncopies)
            if key not in bound:
                bound[key] = layer.bind(x, out, weights=wts, path=wl.path)
            bound[key]()
            return
        # the sequential baseline: same routing, same kernels, one expert FFN
        # call per expert, then the same combine
        moe.moe_route_permute(x, wr, bias, k, layer.ws_rp, layer.topk_idx, layer.topk_w,
                              layer.offsets, layer.sorted_pair, layer.pair_pos)
        experts = None
        if wl.mode == "seq-active":
            experts = np.nonzero(np.diff(layer.offsets.cpu().numpy()))[0]
        launches.append(E if experts is None else len(experts))
        moe.expert_ffn_per_expert(x, layer.offsets, layer.sorted_pair, k, f, *wts,
                                  layer.y_pairs, seq_ws, fmt, path=wl.path,
                                  experts=experts)
        moe.moe_combine(layer.y_pairs, layer.pair_pos, layer.topk_w, out,
                        moe.MOE_OUT_BF16)

    steps = wl.steps
    if wl.mode == "fused":  # marshal every (batch, weight copy) pair up front
        for i in range(min(max(steps, warmup), nx * ncopies)):
            key = (i % nx, i % ncopies)
            bound.setdefault(key, layer.bind(xs[key[0]], out, weights=copies[key[1]],
                                             path=wl.path))
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # pass 1, the measurement: `steps` eager layer steps (argument marshalling
    # done up front) between two events
    t_start, t_end = hip.event(), hip.event()
    hip.record(t_start, stream)
    wall0 = time.perf_counter()
    for i in range(steps):
        step(i)
    hip.record(t_end, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = hip.ms(t_start, t_end)
    # the same steps replayed from HIP graphs (one per batch / weight-copy
    # pair), reported beside the eager rate
    graph_ms = None
    if wl.mode == "fused":
        graphs = {key: layer.capture(xs[key[0]], out, weights=copies[key[1]], path=wl.path)
                  for key in bound}
        for i in range(warmup):
            graphs[(i % nx, i % ncopies)].replay()
        torch.cuda.synchronize()
        hip.record(t_start, stream)
        for i in range(steps):
            graphs[(i % nx, i % ncopies)].replay()
        hip.record(t_end, stream)
        torch.cuda.synchronize()
        graph_ms = hip.ms(t_start, t_end) / steps
        del graphs
    if wl.mode != "fused":
        hip.destroy(t_start)
        hip.destroy(t_end)
        # pass 2: kernel durations of every per-expert call (attached events)
        kern_us = []
        for i in range(steps):
            x, wts = xs[i % nx], copies[i % ncopies]
            moe.moe_route_permute(x, wr, bias, k, layer.ws_rp, layer.topk_idx,
                                  layer.topk_w, layer.offsets, layer.sorted_pair,
                                  layer.pair_pos)
            experts = (np.nonzero(np.diff(layer.offsets.cpu().numpy()))[0]
                       if wl.mode == "seq-active" else range(E))
            ev = [[hip.event() for _ in range(4)] for _ in experts]
            moe.expert_ffn_per_expert(x, layer.offsets, layer.sorted_pair, k, f, *wts,
                                      layer.y_pairs, seq_ws, fmt, path=wl.path,
                                      experts=experts, events=ev)
            torch.cuda.synchronize()
            kern_us.append(1e3 * sum(hip.ms(e[0], e[1]) + hip.ms(e[2], e[3]) for e in ev))
            for e in ev:
                for h in e:
                    hip.destroy(h)
        ms_step = total_ms / steps
        rec = {"workload": wl.name, "config": cfg.name, "T": T, "d": d, "E": E, "k": k,
               "f": f, "format": "int4-g128", "mode": wl.mode,
               "ms_per_step": round(ms_step, 5),
               "tokens_per_s": round(T / (ms_step / 1e3), 1),
               "wall_s": round(wall, 3), "weight_copies": ncopies,
               "ffn_calls_per_step": round(float(np.mean(launches[-steps:])), 2),
               "ffn_kernel_us_per_step": round(float(np.mean(kern_us)), 2),
               "active_experts_avg": round(float(np.mean(active)), 2)}
        del copies, layer, xs
        torch.cuda.empty_cache()
        return rec

    # pass 2, the same steps again with start/stop events attached to the two
    # expert-FFN kernel dispatches (per-kernel durations for the roofline)
    ev = [[hip.event() for _ in range(4)] for _ in range(steps)]
    i0, i1 = hip.event(), hip.event()
    hip.record(i0, stream)
    for i in range(steps):
        moe.moe_set_ffn_events(*ev[i])
        layer.forward(xs[i % nx], out=out, path=wl.path, weights=copies[i % ncopies])
    hip.record(i1, stream)
    torch.cuda.synchronize()
    instr_ms = hip.ms(i0, i1)
    gu_ms = [hip.ms(e[0], e[1]) for e in ev]
    dn_ms = [hip.ms(e[2], e[3]) for e in ev]
    gu_b = sum(gu_bytes[i % nx] for i in range(steps))
    dn_b = sum(dn_bytes[i % nx] for i in range(steps))
    for e in ev:
        for h in e:
            hip.destroy(h)
    for h in (t_start, t_end, i0, i1):
        hip.destroy(h)

    ms_step = total_ms / steps
    rec = {
        "workload": wl.name, "config": cfg.name, "T": T, "d": d, "E": E, "k": k,
        "f": f, "format": ("bitplane8-allocated" if alloc else "bitplane8-rank") if bp else "int4-g128",
        "ms_per_step": round(ms_step, 5), "tokens_per_s": round(T / (ms_step / 1e3), 1),
        "ms_per_step_instrumented": round(instr_ms / steps, 5),
        "graph_replay_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
        "wall_s": round(wall, 3), "weight_copies": ncopies,
        "active_experts_avg": round(float(np.mean(active)), 2),
        "gateup_us": round(1e3 * float(np.mean(gu_ms)), 3),
        "down_us": round(1e3 * float(np.mean(dn_ms)), 3),
        "gateup_bytes_avg": int(gu_b / steps), "down_bytes_avg": int(dn_b / steps),
        "gateup_GBps": round(gu_b / (sum(gu_ms) * 1e-3) / 1e9, 1),
        "down_GBps": round(dn_b / (sum(dn_ms) * 1e-3) / 1e9, 1),
        "ffn_GBps": round((gu_b + dn_b) / ((sum(gu_ms) + sum(dn_ms)) * 1e-3) / 1e9, 1),
        "gateup_TFLOPs": round(flops_gu * steps / (sum(gu_ms) * 1e-3) / 1e12, 2),
        "down_TFLOPs": round(flops_dn * steps / (sum(dn_ms) * 1e-3) / 1e12, 2),
    }
    if alloc:
        rec["allocation"] = alloc
    if indep:
        rec["prefix_bytes_avg"] = int(np.mean([g + dd for g, dd in zip(gu_bytes, dn_bytes)]))
        rec["independent_objects_bytes_avg"] = int(np.mean(indep))
    rec["ffn_mfma_util_pct"] = round(100 * (flops_gu + flops_dn) * steps /
                                     ((sum(gu_ms) + sum(dn_ms)) * 1e-3) / 1e12 /
                                     MFMA_BF16_PEAK_TFS, 2)
    del copies, layer, xs
    torch.cuda.empty_cache()
    return rec


def _omp_threads(n):
    """Set the OpenMP thread count of the oracle library (libgomp)."""
    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))


def cpu_baseline(np, synth, oracle, cid=4, T=64, sample_1t=32):
    """The oracle as it stands on the host cores, on the headline batch: the
    whole layer (route, grouping, per-expert dequantization and SwiGLU FFN in
    fp64, combine), timed twice -- on one thread over the first `sample_1t`
    tokens of the batch, and on every host core over the whole batch.
    Expert quantization is offline on both sides and excluded (done up front
    by a thread pool)."""
    from concurrent.futures import ThreadPoolExecutor
    cfg = synth.CONFIGS[cid]
    x = synth.host_x(cfg, T, step=0)
    wr, bias = synth.host_router(cfg), synth.host_bias(cfg)
    _, idx, _ = oracle.route(x, wr, bias, cfg.k)
    cores = len(os.sched_getaffinity(0))
    cache = {}

    def pack(e):
        _omp_threads(1)  # this pool thread's own OpenMP setting
        return (oracle.quantize_w4(synth.host_expert(cfg, synth.T_W_GATE_UP, e)),
                oracle.quantize_w4(synth.host_expert(cfg, synth.T_W_DOWN, e)))

    experts = [int(e) for e in np.unique(idx)]
    t0 = time.perf_counter()
    _omp_threads(1)
    with ThreadPoolExecutor(cores) as pool:
        for e, q in zip(experts, pool.map(pack, experts)):
            cache[e] = q
    prep = time.perf_counter() - t0
    runs = []
    for n, threads in ((sample_1t, 1), (T, cores)):
        _omp_threads(threads)
        t0 = time.perf_counter()
        oracle.layer(x[:n], wr, bias, cfg.k, cfg.f, cache.__getitem__)
        el = time.perf_counter() - t0
        runs.append({"value": round(n / el, 3), "unit": "tokens/s", "cores": threads,
                     "kind": "oracle",
                     "sample": f"{n} of the {T} tokens of one headline batch ({cfg.name}, "
                               f"{n * cfg.k} pairs): the whole layer in the fp64 oracle "
                               f"(route, grouping, per-expert dequantization and SwiGLU "
                               f"FFN, combine), {threads} OpenMP thread(s), {el:.2f} s; "
                               f"measured on the sample itself, no extrapolation; "
                               f"expert quantization excluded ({len(experts)} experts "
                               f"packed up front in {prep:.1f} s)"})
    _omp_threads(cores)
    best = runs[1]
    return dict(best, single_thread=runs[0])


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gateup_w4_decode_e256_T64.txt")
DECODE_SRC = os.path.join(ROOT, "quantized_mixture_experts_fp32_amd", "csrc", "ffn_decode.hip")


def load_traffic():
    """HBM bytes per launch of the dominant kernel, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary; None once the kernel source
    differs from the one the counters were taken on."""
    import hashlib
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = {}
    for ln in open(TRAFFIC_FILE):
        if "=" in ln and not ln.lstrip().startswith("#"):
            key, val = ln.split("=", 1)
            rec[key.strip()] = val.strip()
    h = hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest()[:16]
    if rec.get("kernel_source_sha256_16") != h:
        return None
    return int(float(rec["traffic_bytes_per_launch"]))


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this layer benchmark runs on exactly one GPU (--gpus 1); "
              "no multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    import quantized_mixture_experts_fp32_amd as moe

    moe.load_library()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    hip = Hip()
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    head = Workload("e256-w4 T=64", 4, 64, args.steps)
    secondary = [
        Workload("e256-w4 T=8192", 4, 8192, max(3, args.steps // 40)),
        Workload("e256-w4 T=1", 4, 1, args.steps),
        Workload("olmoe-decode-w4 T=16", 1, 16, args.steps),
        Workload("olmoe-decode-w4 T=1", 1, 1, args.steps),
        Workload("olmoe-decode-w4 T=4", 1, 4, args.steps),
        Workload("olmoe-decode-w4 T=8", 1, 8, args.steps),
        Workload("olmoe-sequential-w4 T=16", 1, 16, max(10, args.steps // 4),
                 mode="seq-active"),
        Workload("olmoe-sequential-all-w4 T=16", 1, 16, max(10, args.steps // 4),
                 mode="seq-all"),
        Workload("olmoe-bitplane-decode T=16", 3, 16, args.steps),
        Workload("olmoe-bitplane-budget4.5 T=16", 3, 16, args.steps, budget_bits=4.5),
        Workload("olmoe-bitplane-prefill T=4096", 3, 4096, max(5, args.steps // 10), path=2),
        Workload("olmoe-cache64-w4 T=16", 1, 16, max(20, args.steps // 4), mode="cache",
                 slots=64),
        Workload("olmoe-cache32-w4 T=16", 1, 16, max(20, args.steps // 4), mode="cache",
                 slots=32),
        Workload("olmoe-cache16-w4 T=16", 1, 16, max(20, args.steps // 4), mode="cache",
                 slots=16),
        Workload("olmoe-bitplane-cache64 T=16", 3, 16, max(20, args.steps // 4), mode="cache",
                 slots=64),
        Workload("olmoe-bitplane-cache16 T=16", 3, 16, max(20, args.steps // 4), mode="cache",
                 slots=16),
        Workload("olmoe-prefill-w4 T=4096", 2, 4096, max(5, args.steps // 10)),
    ]
    if args.workloads:
        keys = args.workloads.split(",")
        secondary = [w for w in secondary
                     if any(k in w.name.replace(" ", "_") for k in keys)]
    if args.no_headline:
        for wl in secondary:
            run = run_cache_workload if wl.mode == "cache" else run_workload
            print(json.dumps(run(wl, max(2, args.warmup // 4), hip, torch, np, synth, moe)),
                  flush=True)
        return
    head_rec = run_workload(head, args.warmup, hip, torch, np, synth, moe)
    others = []
    if not args.only_headline:
        for wl in secondary:
            run = run_cache_workload if wl.mode == "cache" else run_workload
            others.append(run(wl, max(2, args.warmup // 4), hip, torch, np, synth, moe))
    fused = {(r["config"], r["T"]): r for r in [head_rec] + others
             if r.get("mode", "fused") == "fused" and "gateup_us" in r}
    for r in others:
        f_rec = fused.get((r["config"], r["T"]))
        if r.get("mode", "fused") in ("seq-active", "seq-all") and f_rec:
            r["fused_ms_per_step"] = f_rec["ms_per_step"]
            r["fused_speedup"] = round(r["ms_per_step"] / f_rec["ms_per_step"], 3)
            fk = f_rec["gateup_us"] + f_rec["down_us"]
            r["fused_ffn_kernel_us_per_step"] = round(fk, 2)
            r["fused_kernel_speedup"] = round(r["ffn_kernel_us_per_step"] / fk, 3)
    base = None
    if not args.no_cpu_baseline:
        import oracle
        base = cpu_baseline(np, synth, oracle, sample_1t=args.cpu_sample_tokens)

    achieved = head_rec["gateup_GBps"]
    ffn_bytes = head_rec["gateup_bytes_avg"] + head_rec["down_bytes_avg"]
    line = {
        "metric": METRIC, "value": head_rec["tokens_per_s"], "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head_rec["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "e256-w4: one MoE layer, d=4096, E=256 experts, top-8, "
                               "f=2048, SwiGLU, symmetric int4 group-128 experts (3.3 GB "
                               "packed), router bias N(0,1), T=64 decode tokens per step",
                   "T": 64, "d": 4096, "E": 256, "k": 8, "f": 2048,
                   "weights": "int4-g128 codes + fp16 scales",
                   "weight_copies_rotated": head_rec["weight_copies"],
                   "token_batches_rotated": 16,
                   "active_experts_avg": head_rec["active_experts_avg"]},
        "roofline": {"bound": "hbm",
                     "kernel": "expert gate/up, decode (gateup_w4_decode_lds)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(),
                     "algorithmic_bytes_per_launch": head_rec["gateup_bytes_avg"],
                     "avg_launch_us": head_rec["gateup_us"],
                     "ffn": {"kernels": "gate/up + down",
                             "algorithmic_bytes_per_step": ffn_bytes,
                             "us_per_step": round(head_rec["gateup_us"] + head_rec["down_us"], 3),
                             "achieved": head_rec["ffn_GBps"],
                             "frac": round(head_rec["ffn_GBps"] / HBM_PEAK_GBS, 4)}},
        "cpu_baseline": base,
        "headline_detail": head_rec,
        "workloads": others,
    }
    pf = fused.get(("e256-w4", 8192))
    if pf:
        line["roofline_prefill"] = {
            "bound": "mfma", "workload": "e256-w4 T=8192 (65,536 pairs)",
            "kernel": "expert gate/up, prefill (pf_w4_kernel<true>)",
            "achieved": pf["gateup_TFLOPs"], "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
            "frac": round(pf["gateup_TFLOPs"] / MFMA_BF16_PEAK_TFS, 4),
            "algorithmic_flops_per_launch": 4.0 * 8192 * 8 * 4096 * 2048,
            "avg_launch_us": pf["gateup_us"],
            "ffn_mfma_util_pct": pf["ffn_mfma_util_pct"]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
