"""Oracle: the plain, slow CPU definition of the routed-expert W4A16 MoE layer.

TEST INFRASTRUCTURE ONLY.  Only `tests/`, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` may import this package.  The GPU library
never loads it and shares no code with it; its inputs come from the seeded
generator in `synth/`, never from the GPU path.

`liboracle.so` (oracle.c) holds every arithmetic step; this module marshals
numpy arrays and sequences the steps of one layer:
route -> group pairs by expert -> per expert SwiGLU FFN -> weighted combine.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")

BITS_NONE, BITS_PER_PAIR, BITS_PER_EXPERT, BITS_RANK_RULE = 0, 1, 2, 3

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} missing: run oracle.build.build()")
        lib = ctypes.CDLL(LIB)
        i32, i64, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
        sig = {
            "oracle_router_logits": [vp, vp, vp, i32, i32, i32, vp],
            "oracle_topk": [vp, i32, i32, i32, vp, vp],
            "oracle_permute": [vp, i32, i32, i32, vp, vp, vp],
            "oracle_quantize_w4": [vp, i64, i32, vp, vp],
            "oracle_quantize_bp8": [vp, i64, i32, vp, vp],
            "oracle_dequant_w4": [vp, vp, i64, i32, vp],
            "oracle_dequant_bp": [vp, vp, i64, i32, i32, vp],
            "oracle_pair_bits": [i32, i32, i32, vp, i32, vp, vp],
            "oracle_expert_ffn": [vp, i32, i32, i32, vp, vp, vp, vp],
            "oracle_combine": [vp, vp, vp, i32, i32, i32, vp, vp],
            "oracle_bp_distortion": [vp, vp, vp, vp, i32, i32, vp],
            "oracle_allocate_bits": [vp, vp, i32, i32, i32, i32, i32, i64, vp, vp, vp],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
        lib.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_f16.restype = ctypes.c_uint16
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        _lib = lib
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "need C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _ok(rc, what):
    if rc != 0:
        raise ValueError(f"oracle: invalid argument to {what}")


# ------------------------------------------------------------- single steps
def f64_to_bf16(v: float) -> int:
    return int(_load().oracle_f64_to_bf16(float(v)))


def f64_to_f16(v: float) -> int:
    return int(_load().oracle_f64_to_f16(float(v)))


def f16_to_f64(h: int) -> float:
    return float(_load().oracle_f16_to_f64(int(h)))


def router_logits(x, wr, bias):
    T, d = x.shape
    E = wr.shape[0]
    x = np.ascontiguousarray(x, np.uint16)
    wr = np.ascontiguousarray(wr, np.uint16)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    out = np.zeros((T, E), np.float32)
    _ok(_load().oracle_router_logits(_p(x), _p(wr), _p(b), T, d, E, _p(out)),
        "router_logits")
    return out


def topk(logits, k):
    T, E = logits.shape
    logits = np.ascontiguousarray(logits, np.float32)
    idx = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float64)
    _ok(_load().oracle_topk(_p(logits), T, E, k, _p(idx), _p(w)), "topk")
    return idx, w


def route(x, wr, bias, k):
    logits = router_logits(x, wr, bias)
    idx, w = topk(logits, k)
    return logits, idx, w


def permute(topk_idx, E):
    T, k = topk_idx.shape
    idx = np.ascontiguousarray(topk_idx, np.int32)
    off = np.zeros(E + 1, np.int32)
    sp = np.zeros(T * k, np.int32)
    pp = np.zeros(T * k, np.int32)
    _ok(_load().oracle_permute(_p(idx), T, k, E, _p(off), _p(sp), _p(pp)),
        "permute")
    return off, sp, pp


def quantize_w4(w):
    w = np.ascontiguousarray(w, np.float32)
    R, K = w.shape
    codes = np.zeros((R, K // 2), np.uint8)
    scales = np.zeros((R, K // 128), np.uint16)
    _ok(_load().oracle_quantize_w4(_p(w), R, K, _p(codes), _p(scales)),
        "quantize_w4")
    return codes, scales


def quantize_bp8(w):
    w = np.ascontiguousarray(w, np.float32)
    R, K = w.shape
    planes = np.zeros((8, R, K // 8), np.uint8)
    scales = np.zeros((R, K // 128), np.uint16)
    _ok(_load().oracle_quantize_bp8(_p(w), R, K, _p(planes), _p(scales)),
        "quantize_bp8")
    return planes, scales


def dequant_w4(codes, scales):
    R, K2 = codes.shape
    out = np.zeros((R, 2 * K2), np.float64)
    _ok(_load().oracle_dequant_w4(_p(np.ascontiguousarray(codes)),
                                  _p(np.ascontiguousarray(scales)), R, 2 * K2,
                                  _p(out)), "dequant_w4")
    return out


def dequant_bp(planes, scales, bits):
    _, R, K8 = planes.shape
    out = np.zeros((R, 8 * K8), np.float64)
    _ok(_load().oracle_dequant_bp(_p(np.ascontiguousarray(planes)),
                                  _p(np.ascontiguousarray(scales)), R, 8 * K8,
                                  int(bits), _p(out)), "dequant_bp")
    return out


def pair_bits(topk_idx, E, bits_mode, bits=None):
    T, k = topk_idx.shape
    out = np.zeros(T * k, np.uint8)
    b = None if bits is None else np.ascontiguousarray(bits, np.uint8)
    _ok(_load().oracle_pair_bits(T, k, E, _p(np.ascontiguousarray(topk_idx, np.int32)),
                                 bits_mode, _p(b), _p(out)), "pair_bits")
    return out


def expert_ffn(x_rows, w_gate_up, w_down):
    n, d = x_rows.shape
    f = w_down.shape[1]
    x_rows = np.ascontiguousarray(x_rows, np.uint16)
    h = np.zeros((n, f), np.float64)
    y = np.zeros((n, d), np.float64)
    _ok(_load().oracle_expert_ffn(_p(x_rows), n, d, f,
                                  _p(np.ascontiguousarray(w_gate_up, np.float64)),
                                  _p(np.ascontiguousarray(w_down, np.float64)),
                                  _p(h), _p(y)), "expert_ffn")
    return h, y


def combine(y_pairs, pair_pos, topk_w):
    T, k = topk_w.shape
    d = y_pairs.shape[1]
    o = np.zeros((T, d), np.float64)
    out = np.zeros((T, d), np.uint16)
    _ok(_load().oracle_combine(_p(np.ascontiguousarray(y_pairs, np.float64)),
                               _p(np.ascontiguousarray(pair_pos, np.int32)),
                               _p(np.ascontiguousarray(topk_w, np.float64)),
                               T, k, d, _p(o), _p(out)), "combine")
    return o, out


# ---------------------------------------------------------------- one layer
def expert_outputs(x, topk_idx, offsets, sorted_pair, get_expert, fmt, f,
                   pbits=None, experts=None, want_h=False):
    """Per-pair FFN outputs y [P][d] in grouped order (fp64).

    get_expert(e) returns the oracle-quantized expert:
      fmt "w4":  ((gu_codes, gu_scales), (dn_codes, dn_scales))
      fmt "bp8": ((gu_planes, gu_scales), (dn_planes, dn_scales))
    pbits [P]: bit-width per pair (bitplane format only).
    experts: optional subset of experts to evaluate (others left as NaN).
    """
    T, k = topk_idx.shape
    d = x.shape[1]
    P = T * k
    y = np.full((P, d), np.nan, np.float64)
    h = np.full((P, f), np.nan, np.float64) if want_h else None
    E = len(offsets) - 1
    for e in range(E) if experts is None else experts:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        slots = np.arange(lo, hi)
        pairs = sorted_pair[lo:hi]
        (gu_q, gu_s), (dn_q, dn_s) = get_expert(e)
        if fmt == "w4":
            classes = {8: slots}
        else:
            b = pbits[pairs]
            classes = {int(v): slots[b == v] for v in np.unique(b)}
        for bits, cls in classes.items():
            if fmt == "w4":
                wgu, wdn = dequant_w4(gu_q, gu_s), dequant_w4(dn_q, dn_s)
            else:
                wgu, wdn = dequant_bp(gu_q, gu_s, bits), dequant_bp(dn_q, dn_s, bits)
            toks = sorted_pair[cls] // k
            hh, yy = expert_ffn(x[toks], wgu, wdn)
            y[cls] = yy
            if want_h:
                h[cls] = hh
    return (y, h) if want_h else y


def layer(x, wr, bias, k, f, get_expert, fmt="w4", bits_mode=BITS_NONE,
          bits=None):
    """The whole layer on T token rows; returns a dict of every step."""
    E = wr.shape[0]
    logits, idx, w = route(x, wr, bias, k)
    off, sp, pp = permute(idx, E)
    pb = pair_bits(idx, E, bits_mode, bits) if fmt == "bp8" else None
    y = expert_outputs(x, idx, off, sp, get_expert, fmt, f, pb)
    o, out = combine(y, pp, w)
    return dict(logits=logits, topk_idx=idx, topk_w=w, expert_offsets=off,
                sorted_pair=sp, pair_pos=pp, pair_bits=pb, y_pairs=y, o=o,
                out=out)


# ------------------------------------------------------- read-budget allocator
def bp_distortion(gu_planes, gu_scales, dn_planes, dn_scales, d, f):
    """Weight-space distortion [8] of one expert at prefix widths 1..8 (planes
    in the oracle's slab layout [8][R][K/8])."""
    out = np.zeros(8, np.float64)
    args = [np.ascontiguousarray(a) for a in (gu_planes, gu_scales, dn_planes, dn_scales)]
    _ok(_load().oracle_bp_distortion(*[_p(a) for a in args], d, f, _p(out)),
        "bp_distortion")
    return out


def bp_read_bytes(d, f, b):
    """Bytes one expert reads at prefix width b (planes plus fp16 scales)."""
    return b * 3 * d * f // 8 + 3 * d * f // 64


def allocate_bits(dist, counts, d, f, bmin, bmax, budget):
    """-> (bits [E] u8, lambda, read) of the read-budget bisection."""
    dist = np.ascontiguousarray(dist, np.float64)
    counts = np.ascontiguousarray(counts, np.int32)
    E = dist.shape[0]
    bits = np.zeros(E, np.uint8)
    lam = ctypes.c_double()
    rd = ctypes.c_int64()
    _ok(_load().oracle_allocate_bits(_p(dist), _p(counts), E, d, f, bmin, bmax,
                                     int(budget), _p(bits),
                                     ctypes.cast(ctypes.pointer(lam), ctypes.c_void_p),
                                     ctypes.cast(ctypes.pointer(rd), ctypes.c_void_p)),
        "allocate_bits")
    return bits, lam.value, rd.value

