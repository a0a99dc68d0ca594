"""Seeded synthetic inputs of the routed-expert MoE layer.

Input generation only: this module holds none of the layer's arithmetic.  It
is the one piece shared by the oracle side and the GPU side of every test and
benchmark.  `synth_gen.h` defines each element; `libsynth_host.so` evaluates
it on the CPU and `libsynth_dev.so` on the GPU, bit for bit the same.

Workloads (shapes and distributions of the layer configurations measured by
the benchmarks and parity tests):
  x ~ N(0,1) bf16 [T][d]; router W_r ~ N(0,1/d) bf16, stored expert-major
  [E][d]; optional router logit bias ~ N(0, sb^2) fp32 [E]; expert weights
  ~ N(0, 0.02) fp32 (variance 0.02), each entry x10 with probability 1e-3,
  gate|up stacked as [E][2f][d] and down as [E][d][f].
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(HERE, "libsynth_host.so")
DEV_LIB = os.path.join(HERE, "libsynth_dev.so")

SEED = 42
T_X, T_WR, T_BIAS, T_W_GATE_UP, T_W_DOWN = 1, 2, 3, 4, 6
MASK_OFFSET = 100
W_SIGMA = math.sqrt(0.02)


@dataclass(frozen=True)
class LayerConfig:
    cid: int
    name: str
    d: int
    E: int
    k: int
    f: int
    Ts: tuple
    fmt: str  # "w4" (symmetric int4, group 128) or "bp8" (bitplane prefixes)
    bias_sigma: float | None = None
    bits_rule: str | None = None  # "rank" for the rank -> bit-width rule
    note: str = ""

    @property
    def router_sigma(self) -> float:
        return 1.0 / math.sqrt(self.d)


CONFIGS = {
    0: LayerConfig(0, "tiny-w4", 256, 8, 2, 512, (16,), "w4",
                   note="tiny correctness layer"),
    1: LayerConfig(1, "olmoe-decode-w4", 2048, 64, 8, 1024, (1, 4, 8, 16), "w4",
                   note="OLMoE-shaped decode"),
    2: LayerConfig(2, "olmoe-prefill-w4", 2048, 64, 8, 1024, (4096,), "w4",
                   bias_sigma=1.5, note="OLMoE-shaped prefill, skewed routing"),
    3: LayerConfig(3, "olmoe-bitplane-decode", 2048, 64, 8, 1024, (16,), "bp8",
                   bits_rule="rank", note="per-pair bit-width from routing rank"),
    4: LayerConfig(4, "e256-w4", 4096, 256, 8, 2048, (1, 64, 8192), "w4",
                   bias_sigma=1.0, note="large expert count, skewed routing"),
}


_host = None
_dev = None


def _load_host():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} missing: run synth.build.build_host()")
        lib = ctypes.CDLL(HOST_LIB)
        u64, dbl, vp = ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        lib.synth_stream_key.restype = u64
        lib.synth_stream_key.argtypes = [u64, u64, u64, u64]
        lib.synth_fill_bf16.argtypes = [u64, u64, u64, u64, u64, u64, dbl, vp]
        lib.synth_fill_f32.argtypes = [u64, u64, u64, u64, u64, u64, dbl, vp]
        lib.synth_fill_weight_f32.argtypes = [u64, u64, u64, u64, u64, dbl, vp]
        lib.synth_fill_outlier_mask.argtypes = [u64, u64, u64, u64, u64, vp]
        lib.synth_fill_std_normal.argtypes = [u64, u64, u64, vp]
        _host = lib
    return _host


def _load_dev():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} missing: run synth.build.build_dev()")
        lib = ctypes.CDLL(DEV_LIB)
        u64, dbl, vp = ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        lib.synth_dev_fill_bf16.argtypes = [u64, u64, u64, u64, u64, u64, dbl, vp, vp]
        lib.synth_dev_fill_f32.argtypes = [u64, u64, u64, u64, u64, u64, dbl, vp, vp]
        lib.synth_dev_fill_weight_f32.argtypes = [u64, u64, u64, u64, u64, dbl, vp, vp]
        for fn in (lib.synth_dev_fill_bf16, lib.synth_dev_fill_f32,
                   lib.synth_dev_fill_weight_f32):
            fn.restype = ctypes.c_int
        _dev = lib
    return _dev


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------- host side
def stream_key(cid, tensor, step=0, seed=SEED) -> int:
    return int(_load_host().synth_stream_key(seed, cid, tensor, step))


def std_normal(key: int, start: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float64)
    _load_host().synth_fill_std_normal(key, start, n, _ptr(out))
    return out


def host_x(cfg: LayerConfig, T: int, step: int = 0, seed: int = SEED,
           first_token: int = 0) -> np.ndarray:
    """x rows [first_token, first_token+T) as bf16 bits, uint16 [T][d]."""
    out = np.empty((T, cfg.d), np.uint16)
    if T:
        _load_host().synth_fill_bf16(seed, cfg.cid, T_X, step,
                                     first_token * cfg.d, T * cfg.d, 1.0,
                                     _ptr(out))
    return out


def host_router(cfg: LayerConfig, seed: int = SEED) -> np.ndarray:
    """Router weights as bf16 bits, expert-major uint16 [E][d]."""
    out = np.empty((cfg.E, cfg.d), np.uint16)
    _load_host().synth_fill_bf16(seed, cfg.cid, T_WR, 0, 0, cfg.E * cfg.d,
                                 cfg.router_sigma, _ptr(out))
    return out


def host_bias(cfg: LayerConfig, seed: int = SEED):
    if cfg.bias_sigma is None:
        return None
    out = np.empty(cfg.E, np.float32)
    _load_host().synth_fill_f32(seed, cfg.cid, T_BIAS, 0, 0, cfg.E,
                                cfg.bias_sigma, _ptr(out))
    return out


def weight_shape(cfg: LayerConfig, tensor: int):
    if tensor == T_W_GATE_UP:
        return (cfg.E, 2 * cfg.f, cfg.d)
    if tensor == T_W_DOWN:
        return (cfg.E, cfg.d, cfg.f)
    raise ValueError(tensor)


def host_weight_rows(cfg: LayerConfig, tensor: int, expert: int, row0: int,
                     nrows: int, seed: int = SEED) -> np.ndarray:
    """fp32 rows [row0, row0+nrows) of one expert's weight matrix."""
    _, R, K = weight_shape(cfg, tensor)
    out = np.empty((nrows, K), np.float32)
    start = (expert * R + row0) * K
    _load_host().synth_fill_weight_f32(seed, cfg.cid, tensor, start,
                                       nrows * K, W_SIGMA, _ptr(out))
    return out


def host_expert(cfg: LayerConfig, tensor: int, expert: int,
                seed: int = SEED) -> np.ndarray:
    _, R, _ = weight_shape(cfg, tensor)
    return host_weight_rows(cfg, tensor, expert, 0, R, seed)


def host_outlier_mask(cfg: LayerConfig, tensor: int, start: int, n: int,
                      seed: int = SEED) -> np.ndarray:
    out = np.empty(n, np.uint8)
    _load_host().synth_fill_outlier_mask(seed, cfg.cid, tensor, start, n,
                                         _ptr(out))
    return out


# ------------------------------------------------------------------ GPU side
def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"synth device fill failed: {what}")


def dev_fill_x(cfg: LayerConfig, out_ptr: int, T: int, stream: int,
               step: int = 0, seed: int = SEED):
    _check(_load_dev().synth_dev_fill_bf16(seed, cfg.cid, T_X, step, 0,
                                           T * cfg.d, 1.0, out_ptr, stream), "x")


def dev_fill_router(cfg: LayerConfig, out_ptr: int, stream: int,
                    seed: int = SEED):
    _check(_load_dev().synth_dev_fill_bf16(seed, cfg.cid, T_WR, 0, 0,
                                           cfg.E * cfg.d, cfg.router_sigma,
                                           out_ptr, stream), "router")


def dev_fill_bias(cfg: LayerConfig, out_ptr: int, stream: int,
                  seed: int = SEED):
    _check(_load_dev().synth_dev_fill_f32(seed, cfg.cid, T_BIAS, 0, 0, cfg.E,
                                          cfg.bias_sigma, out_ptr, stream),
           "bias")


def dev_fill_weight(cfg: LayerConfig, tensor: int, out_ptr: int, stream: int,
                    start: int = 0, n: int | None = None, seed: int = SEED):
    if n is None:
        E, R, K = weight_shape(cfg, tensor)
        n = E * R * K - start
    _check(_load_dev().synth_dev_fill_weight_f32(seed, cfg.cid, tensor, start,
                                                 n, W_SIGMA, out_ptr, stream),
           "weights")
