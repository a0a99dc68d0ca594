"""MI355X (gfx950) routed-expert MoE FFN with low-bit weight-only experts.

Thin Python binding of the C ABI in `include/moe_wq.h` (libmoe_wq.so).  The
functions below only marshal torch tensors into pointers and sizes; every
step of the layer runs in the library's HIP kernels.  PyTorch provides
device memory and the current HIP stream.  There is no CPU fallback: the
library must be built (`build.build()`) and a GPU present, or calls raise.

Layer = moe_route -> moe_permute -> moe_expert_ffn_wq -> moe_combine (the
first two also as one call, moe_route_permute).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_wq.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_FMT_W4_SYM, MOE_FMT_BITPLANE8 = 0, 1
MOE_BITS_NONE, MOE_BITS_PER_PAIR, MOE_BITS_PER_EXPERT, MOE_BITS_RANK_RULE = 0, 1, 2, 3
MOE_OUT_BF16, MOE_OUT_F32 = 0, 1
MOE_PATH_AUTO, MOE_PATH_DECODE, MOE_PATH_PREFILL = 0, 1, 2
MOE_GROUP = 128

# Every symbol the header declares (checked by the CPU tests).
EXPORTS = ("moe_status_str", "moe_last_error", "moe_route_ws_bytes", "moe_route",
           "moe_permute_ws_bytes",
           "moe_permute", "moe_route_permute_ws_bytes", "moe_route_permute",
           "moe_ffn_ws_bytes", "moe_expert_ffn_wq", "moe_combine",
           "moe_quantize_w4", "moe_quantize_bitplane8", "moe_set_ffn_events",
           "moe_layer_ws_bytes", "moe_layer_forward_wq", "moe_layer_forward_wq_noalloc",
           "moe_bp_distortion_ws_bytes",
           "moe_bp_distortion", "moe_allocate_bits", "moe_cache_create", "moe_cache_destroy",
           "moe_cache_ws_bytes", "moe_cache_forward", "moe_cache_stats", "moe_cache_slots",
           "moe_cache_reset", "moe_cache_plan", "moe_retile_w4", "moe_retile_bitplane8")


class MoeError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__(f"{fn} failed: {status_str(status)} ({detail})")
        self.status = status


_lib = None


def load_library():
    """Load libmoe_wq.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} not built: run "
                           "quantized_mixture_experts_fp32_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    i32, vp, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    lib.moe_status_str.argtypes, lib.moe_status_str.restype = [i32], ctypes.c_char_p
    lib.moe_last_error.argtypes, lib.moe_last_error.restype = [], ctypes.c_char_p
    lib.moe_route_ws_bytes.argtypes, lib.moe_route_ws_bytes.restype = [i32, i32], sz
    lib.moe_route.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.moe_permute_ws_bytes.argtypes, lib.moe_permute_ws_bytes.restype = [i32, i32, i32], sz
    lib.moe_permute.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.moe_route_permute_ws_bytes.argtypes = [i32, i32, i32]
    lib.moe_route_permute_ws_bytes.restype = sz
    lib.moe_route_permute.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                      vp, sz, vp]
    lib.moe_ffn_ws_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.moe_ffn_ws_bytes.restype = sz
    lib.moe_expert_ffn_wq.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                      vp, vp, vp, vp, vp, i32, vp, vp, sz, i32, vp]
    lib.moe_combine.argtypes = [vp, vp, vp, i32, i32, i32, vp, i32, vp]
    lib.moe_quantize_w4.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
    lib.moe_quantize_bitplane8.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
    lib.moe_set_ffn_events.argtypes = [vp, vp, vp, vp]
    lib.moe_layer_ws_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.moe_layer_ws_bytes.restype = sz
    lib.moe_layer_forward_wq.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                         vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp,
                                         vp, i32, vp, sz, i32, vp]
    lib.moe_layer_forward_wq_noalloc.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                                 i32, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                                 vp, vp, vp, vp, i32, i32, vp]
    lib.moe_retile_w4.argtypes = [vp, i32, i32, i32, vp, vp]
    lib.moe_retile_bitplane8.argtypes = [vp, i32, i32, i32, vp, vp]
    lib.moe_bp_distortion_ws_bytes.argtypes = [i32, i32, i32]
    lib.moe_bp_distortion_ws_bytes.restype = sz
    lib.moe_bp_distortion.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp, sz, vp]
    lib.moe_allocate_bits.argtypes = [vp, vp, i32, i32, i32, i32, i32, ctypes.c_int64, vp,
                                      vp, vp, vp]
    lib.moe_cache_create.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                     vp]
    lib.moe_cache_destroy.argtypes, lib.moe_cache_destroy.restype = [vp], None
    lib.moe_cache_ws_bytes.argtypes, lib.moe_cache_ws_bytes.restype = [vp, i32, i32], sz
    lib.moe_cache_forward.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, vp, vp, vp, vp, vp,
                                      i32, vp, sz, vp]
    lib.moe_cache_stats.argtypes = [vp, vp]
    lib.moe_cache_slots.argtypes = [vp, vp, vp]
    lib.moe_cache_reset.argtypes = [vp]
    lib.moe_cache_plan.argtypes = [i32, i32, i32, vp, vp, vp, ctypes.c_int64, vp, vp, vp, i32,
                                   vp, vp, i32, vp, vp]
    for name in ("moe_route", "moe_permute", "moe_route_permute", "moe_expert_ffn_wq",
                 "moe_combine", "moe_layer_forward_wq", "moe_layer_forward_wq_noalloc",
                 "moe_bp_distortion",
                 "moe_allocate_bits", "moe_cache_create", "moe_cache_forward",
                 "moe_cache_stats", "moe_cache_slots", "moe_cache_reset", "moe_cache_plan",
                 "moe_quantize_w4", "moe_quantize_bitplane8", "moe_set_ffn_events",
                 "moe_retile_w4", "moe_retile_bitplane8"):
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load_library().moe_status_str(int(status)).decode()


def _check(fn, rc):
    if rc != MOE_OK:
        raise MoeError(fn, rc, load_library().moe_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _empty(shape, dtype, like):
    import torch
    return torch.empty(shape, dtype=dtype, device=like.device)


# ----------------------------------------------------------------- the ABI
def moe_route_ws_bytes(T, E):
    return int(load_library().moe_route_ws_bytes(T, E))


def moe_route(x, wr, bias, k, topk_idx=None, topk_w=None, ws=None, stream=None):
    """x bf16 [T][d], wr bf16 [E][d], bias fp32 [E] or None -> (idx, w)."""
    import torch
    T, d = x.shape
    E = wr.shape[0]
    if topk_idx is None:
        topk_idx = _empty((T, k), torch.int32, x)
    if topk_w is None:
        topk_w = _empty((T, k), torch.float32, x)
    if ws is None:
        ws = _empty((max(moe_route_ws_bytes(T, E), 16),), torch.uint8, x)
    _check("moe_route", load_library().moe_route(
        _ptr(x), _ptr(wr), _ptr(bias), T, d, E, k, _ptr(topk_idx), _ptr(topk_w),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return topk_idx, topk_w


def moe_permute_ws_bytes(T, k, E):
    return int(load_library().moe_permute_ws_bytes(T, k, E))


def moe_permute(topk_idx, E, ws=None, offsets=None, sorted_pair=None,
                pair_pos=None, stream=None):
    """topk_idx int32 [T][k] -> (expert_offsets [E+1], sorted_pair, pair_pos)."""
    import torch
    T, k = topk_idx.shape
    P = T * k
    if offsets is None:
        offsets = _empty((E + 1,), torch.int32, topk_idx)
    if sorted_pair is None:
        sorted_pair = _empty((P,), torch.int32, topk_idx)
    if pair_pos is None:
        pair_pos = _empty((P,), torch.int32, topk_idx)
    need = moe_permute_ws_bytes(T, k, E)
    if ws is None:
        ws = _empty((max(need, 16),), torch.uint8, topk_idx)
    _check("moe_permute", load_library().moe_permute(
        _ptr(topk_idx), T, k, E, _ptr(offsets), _ptr(sorted_pair), _ptr(pair_pos),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return offsets, sorted_pair, pair_pos


def moe_route_permute_ws_bytes(T, k, E):
    return int(load_library().moe_route_permute_ws_bytes(T, k, E))


def moe_route_permute(x, wr, bias, k, ws=None, topk_idx=None, topk_w=None, offsets=None,
                      sorted_pair=None, pair_pos=None, stream=None):
    """moe_route then moe_permute in one call -> (idx, w, offsets, sorted_pair,
    pair_pos)."""
    import torch
    T, d = x.shape
    E = wr.shape[0]
    P = T * k
    if topk_idx is None:
        topk_idx = _empty((T, k), torch.int32, x)
    if topk_w is None:
        topk_w = _empty((T, k), torch.float32, x)
    if offsets is None:
        offsets = _empty((E + 1,), torch.int32, x)
    if sorted_pair is None:
        sorted_pair = _empty((P,), torch.int32, x)
    if pair_pos is None:
        pair_pos = _empty((P,), torch.int32, x)
    if ws is None:
        ws = _empty((max(moe_route_permute_ws_bytes(T, k, E), 16),), torch.uint8, x)
    _check("moe_route_permute", load_library().moe_route_permute(
        _ptr(x), _ptr(wr), _ptr(bias), T, d, E, k, _ptr(topk_idx), _ptr(topk_w),
        _ptr(offsets), _ptr(sorted_pair), _ptr(pair_pos), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))
    return topk_idx, topk_w, offsets, sorted_pair, pair_pos


def moe_ffn_ws_bytes(T, k, E, d, f, fmt=MOE_FMT_W4_SYM):
    return int(load_library().moe_ffn_ws_bytes(T, k, E, d, f, fmt))


def moe_expert_ffn_wq(x, expert_offsets, sorted_pair, k, f, gate_up_codes,
                      gate_up_scales, down_codes, down_scales,
                      fmt=MOE_FMT_W4_SYM, bits=None, bits_mode=MOE_BITS_NONE,
                      y_pairs=None, ws=None, path=MOE_PATH_AUTO, stream=None):
    """Per-pair SwiGLU outputs y_pairs fp32 [T*k][d] in grouped order."""
    import torch
    T, d = x.shape
    E = expert_offsets.numel() - 1
    if y_pairs is None:
        y_pairs = _empty((T * k, d), torch.float32, x)
    need = moe_ffn_ws_bytes(T, k, E, d, f, fmt)
    if ws is None:
        ws = _empty((max(need, 256),), torch.uint8, x)
    _check("moe_expert_ffn_wq", load_library().moe_expert_ffn_wq(
        _ptr(x), _ptr(expert_offsets), _ptr(sorted_pair), T, k, E, d, f, fmt,
        MOE_GROUP, _ptr(gate_up_codes), _ptr(gate_up_scales), _ptr(down_codes),
        _ptr(down_scales), _ptr(bits), bits_mode, _ptr(y_pairs), _ptr(ws),
        ws.numel() * ws.element_size(), path, _stream(stream)))
    return y_pairs


def expert_ffn_per_expert(x, expert_offsets, sorted_pair, k, f, gate_up_codes,
                          gate_up_scales, down_codes, down_scales, y_pairs, ws,
                          fmt=MOE_FMT_W4_SYM, bits=None, bits_mode=MOE_BITS_NONE,
                          path=MOE_PATH_DECODE, stream=None, experts=None, events=None):
    """The sequential baseline of ExactMoE's ablation ("Every Expert Counts
    ...", Abstract: fused grouped execution against one launch per expert):
    the same expert FFN computed by one moe_expert_ffn_wq call per expert.
    Call e sees a one-expert problem whose expert_offsets are the pointer
    expert_offsets + e (so its slot range is [offsets[e], offsets[e+1]) of
    the shared sorted_pair / y_pairs) and whose weights are expert e's
    slices.  experts: the expert ids to launch (the activated ones, which
    the caller reads from the routing); None launches every expert, and
    those without pairs exit at once.  Writes the y_pairs rows of the
    launched experts like the grouped call.  ws must hold
    moe_ffn_ws_bytes(T, k, 1, d, f, fmt) bytes.  events: optional list with
    one 4-tuple of hipEvent_t handles per launched expert, armed with
    moe_set_ffn_events before that expert's call."""
    T, d = x.shape
    E = expert_offsets.numel() - 1
    lib = load_library()
    vp = ctypes.c_void_p
    esz = lambda t: (t.numel() // t.shape[0]) * t.element_size()
    gu_b, gus_b, dn_b, dns_b = (esz(gate_up_codes), esz(gate_up_scales),
                                esz(down_codes), esz(down_scales))
    wsb, st = ws.numel() * ws.element_size(), _stream(stream)
    for i, e in enumerate(range(E) if experts is None else experts):
        e = int(e)
        if events is not None:
            moe_set_ffn_events(*events[i])
        if not 0 <= e < E:
            raise ValueError(f"expert id {e} outside [0, {E})")
        # a per-expert bit-width array is indexed by the (one) local expert
        b = None if bits is None else vp(
            bits.data_ptr() + (e if bits_mode == MOE_BITS_PER_EXPERT else 0))
        _check("moe_expert_ffn_wq", lib.moe_expert_ffn_wq(
            _ptr(x), vp(expert_offsets.data_ptr() + 4 * e), _ptr(sorted_pair), T, k, 1, d,
            f, fmt, MOE_GROUP, vp(gate_up_codes.data_ptr() + e * gu_b),
            vp(gate_up_scales.data_ptr() + e * gus_b), vp(down_codes.data_ptr() + e * dn_b),
            vp(down_scales.data_ptr() + e * dns_b), b, bits_mode, _ptr(y_pairs),
            _ptr(ws), wsb, path, st))
    return y_pairs


def moe_layer_ws_bytes(T, k, E, d, f, fmt=MOE_FMT_W4_SYM):
    return int(load_library().moe_layer_ws_bytes(T, k, E, d, f, fmt))


def moe_layer_forward(x, wr, bias, k, f, gate_up_codes, gate_up_scales, down_codes,
                      down_scales, topk_idx, topk_w, offsets, sorted_pair, pair_pos,
                      y_pairs, out, ws, fmt=MOE_FMT_W4_SYM, bits=None,
                      bits_mode=MOE_BITS_NONE, out_dtype=MOE_OUT_BF16,
                      path=MOE_PATH_AUTO, stream=None):
    """moe_route_permute -> moe_expert_ffn_wq -> moe_combine in one ABI call
    (same outputs); every output buffer is caller-provided."""
    T, d = x.shape
    E = wr.shape[0]
    _check("moe_layer_forward_wq", load_library().moe_layer_forward_wq(
        _ptr(x), _ptr(wr), _ptr(bias), T, d, E, k, f, fmt, MOE_GROUP, _ptr(gate_up_codes),
        _ptr(gate_up_scales), _ptr(down_codes), _ptr(down_scales), _ptr(bits), bits_mode,
        _ptr(topk_idx), _ptr(topk_w), _ptr(offsets), _ptr(sorted_pair), _ptr(pair_pos),
        _ptr(y_pairs), _ptr(out), out_dtype, _ptr(ws), ws.numel() * ws.element_size(),
        path, _stream(stream)))
    return out


MOE_NOALLOC_SCRATCH_BYTES = 32 << 20


def moe_layer_forward_noalloc(x, wr, bias, k, f, gate_up_codes, gate_up_scales, down_codes,
                              down_scales, topk_idx, topk_w, offsets, sorted_pair, pair_pos,
                              y_pairs, out, fmt=MOE_FMT_W4_SYM, bits=None,
                              bits_mode=MOE_BITS_NONE, out_dtype=MOE_OUT_F32,
                              path=MOE_PATH_AUTO, stream=None):
    """moe_layer_forward_wq_noalloc: the layer step with the library's fixed
    device scratch in place of a workspace (nothing is allocated)."""
    T, d = x.shape
    E = wr.shape[0]
    _check("moe_layer_forward_wq_noalloc", load_library().moe_layer_forward_wq_noalloc(
        _ptr(x), _ptr(wr), _ptr(bias), T, d, E, k, f, fmt, MOE_GROUP, _ptr(gate_up_codes),
        _ptr(gate_up_scales), _ptr(down_codes), _ptr(down_scales), _ptr(bits), bits_mode,
        _ptr(topk_idx), _ptr(topk_w), _ptr(offsets), _ptr(sorted_pair), _ptr(pair_pos),
        _ptr(y_pairs), _ptr(out), out_dtype, path, _stream(stream)))
    return out


def moe_bp_distortion(gate_up_planes, gate_up_scales, down_planes, down_scales, d, f,
                      dist=None, ws=None, stream=None):
    """Weight-space distortion [E][8] (fp64) of bitplane experts at prefix
    widths 1..8 (the offline table of the read-budget allocator)."""
    import torch
    E = gate_up_planes.shape[0]
    if dist is None:
        dist = torch.empty((E, 8), dtype=torch.float64, device=gate_up_planes.device)
    if ws is None:
        ws = torch.empty((int(load_library().moe_bp_distortion_ws_bytes(E, d, f)),),
                         dtype=torch.uint8, device=gate_up_planes.device)
    _check("moe_bp_distortion", load_library().moe_bp_distortion(
        _ptr(gate_up_planes), _ptr(gate_up_scales), _ptr(down_planes), _ptr(down_scales),
        E, d, f, _ptr(dist), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return dist


def moe_allocate_bits(dist, counts, d, f, b_min, b_max, budget_bytes, bits=None,
                      lam=None, read=None, stream=None):
    """Per-expert prefix widths [E] (u8) under a routing-weighted read
    budget -> (bits, lambda [1] fp64, read [1] int64), all on the device."""
    import torch
    E = dist.shape[0]
    dev = dist.device
    if bits is None:
        bits = torch.empty((E,), dtype=torch.uint8, device=dev)
    if lam is None:
        lam = torch.empty((1,), dtype=torch.float64, device=dev)
    if read is None:
        read = torch.empty((1,), dtype=torch.int64, device=dev)
    _check("moe_allocate_bits", load_library().moe_allocate_bits(
        _ptr(dist), _ptr(counts), E, d, f, b_min, b_max, int(budget_bytes), _ptr(bits),
        _ptr(lam), _ptr(read), _stream(stream)))
    return bits, lam, read


def moe_combine(y_pairs, pair_pos, topk_w, out=None, out_dtype=MOE_OUT_BF16,
                stream=None):
    """Layer output [T][d] (bf16 bits in an int16 tensor, or fp32)."""
    import torch
    T, k = topk_w.shape
    d = y_pairs.shape[1]
    if out is None:
        out = _empty((T, d), torch.bfloat16 if out_dtype == MOE_OUT_BF16
                     else torch.float32, y_pairs)
    _check("moe_combine", load_library().moe_combine(
        _ptr(y_pairs), _ptr(pair_pos), _ptr(topk_w), T, k, d, _ptr(out), out_dtype,
        _stream(stream)))
    return out


def moe_quantize_w4(w, codes=None, scales=None, stream=None):
    """fp32 [E][N][K] -> (codes, scales fp16-bits [E][N][K/128]).

    codes is a u8 tensor of shape [E][N][K/2] holding the tiled int4 layout
    of include/moe_wq.h (per expert [N/16][K/128][16][64] bytes); N % 16 == 0.
    """
    import torch
    E, N, K = w.shape
    if codes is None:
        codes = _empty((E, N, K // 2), torch.uint8, w)
    if scales is None:
        scales = _empty((E, N, K // 128), torch.int16, w)
    _check("moe_quantize_w4", load_library().moe_quantize_w4(
        _ptr(w), E, N, K, MOE_GROUP, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def moe_retile_w4(codes_canonical, N, K, codes=None, stream=None):
    """Canonical row-major int4 codes u8 [E][N][K/2] -> the tiled layout
    (a u8 tensor [E][N][K/2] as moe_quantize_w4 returns)."""
    import torch
    E = codes_canonical.shape[0]
    if codes is None:
        codes = _empty((E, N, K // 2), torch.uint8, codes_canonical)
    _check("moe_retile_w4", load_library().moe_retile_w4(
        _ptr(codes_canonical), E, N, K, _ptr(codes), _stream(stream)))
    return codes


def moe_retile_bitplane8(planes_canonical, N, K, planes=None, stream=None):
    """Canonical plane slabs u8 [E][8][N][K/8] -> the bitplane streaming
    layout (a u8 tensor [E][8][N][K/8] as moe_quantize_bitplane8 returns)."""
    import torch
    E = planes_canonical.shape[0]
    if planes is None:
        planes = _empty((E, 8, N, K // 8), torch.uint8, planes_canonical)
    _check("moe_retile_bitplane8", load_library().moe_retile_bitplane8(
        _ptr(planes_canonical), E, N, K, _ptr(planes), _stream(stream)))
    return planes


def moe_quantize_bitplane8(w, planes=None, scales=None, stream=None):
    """fp32 [E][N][K] -> (planes, scales fp16-bits [E][N][K/128]).

    planes is a u8 tensor of shape [E][8][N][K/8] holding the bitplane layout
    of include/moe_wq.h (per expert [N/16][K/128][8][16][16] bytes);
    N % 16 == 0.
    """
    import torch
    E, N, K = w.shape
    if planes is None:
        planes = _empty((E, 8, N, K // 8), torch.uint8, w)
    if scales is None:
        scales = _empty((E, N, K // 128), torch.int16, w)
    _check("moe_quantize_bitplane8", load_library().moe_quantize_bitplane8(
        _ptr(w), E, N, K, MOE_GROUP, _ptr(planes), _ptr(scales), _stream(stream)))
    return planes, scales


def moe_set_ffn_events(gateup_begin=None, gateup_end=None, down_begin=None,
                       down_end=None):
    """Arm raw hipEvent_t handles (ints) for the next moe_expert_ffn_wq call."""
    def h(e):
        return None if e is None else ctypes.c_void_p(e)
    _check("moe_set_ffn_events", load_library().moe_set_ffn_events(
        h(gateup_begin), h(gateup_end), h(down_begin), h(down_end)))


# ------------------------------------------------------ expert slot cache
def _np_ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def moe_cache_plan(E, slots, fmt, slot_expert, slot_bits, slot_last, step, need):
    """One step's slot assignment on host state (no device work).  The slot
    arrays (numpy int32/int32/int64 [slots]) are updated in place; returns
    dict(vmap [E], chunks [n][4], loads [n][6], V)."""
    import numpy as np
    for a, dt in ((slot_expert, np.int32), (slot_bits, np.int32), (slot_last, np.int64)):
        if a.dtype != dt or not a.flags.c_contiguous or a.shape != (slots,):
            raise ValueError("slot arrays: contiguous int32, int32, int64 of length slots")
    need = np.ascontiguousarray(need, np.int32)
    vmap = np.zeros(E, np.int32)
    max_chunks = 2 + 2 * E // max(slots // 2, 1)
    chunks = np.zeros((max_chunks, 4), np.int32)
    loads = np.zeros((2 * E + 1, 6), np.int32)
    nc, nl, V = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    ref = lambda v: ctypes.cast(ctypes.pointer(v), ctypes.c_void_p)  # noqa: E731
    _check("moe_cache_plan", load_library().moe_cache_plan(
        E, slots, fmt, _np_ptr(slot_expert), _np_ptr(slot_bits), _np_ptr(slot_last),
        int(step), _np_ptr(need), _np_ptr(vmap), _np_ptr(chunks), max_chunks, ref(nc),
        _np_ptr(loads), loads.shape[0], ref(nl), ref(V)))
    return dict(vmap=vmap, chunks=chunks[:nc.value].copy(), loads=loads[:nl.value].copy(),
                V=V.value)


class ExpertCache:
    """Expert bank in pinned host memory behind `slots` device slots
    (moe_cache_*): forward(x) runs one layer step, copying the experts (or
    bitplanes) it is missing into the slots first."""

    def __init__(self, wr, bias, k, f, gate_up_codes, gate_up_scales, down_codes,
                 down_scales, fmt, slots):
        import torch
        self.wr, self.bias, self.k, self.f, self.fmt, self.slots = wr, bias, k, f, fmt, slots
        self.E, self.d = wr.shape
        dev = wr.device
        # the whole bank, pinned host memory (the cache's backing store)
        self.host = [t.detach().to("cpu").contiguous().pin_memory()
                     for t in (gate_up_codes, gate_up_scales, down_codes, down_scales)]
        self.dev = [torch.empty((slots,) + tuple(t.shape[1:]), dtype=t.dtype, device=dev)
                    for t in self.host]
        h = ctypes.c_void_p()
        _check("moe_cache_create", load_library().moe_cache_create(
            self.E, self.d, f, fmt, slots, *[_ptr(t) for t in self.host],
            *[_ptr(t) for t in self.dev], ctypes.cast(ctypes.pointer(h), ctypes.c_void_p)))
        self.handle = h
        self._T = None

    def _alloc(self, T, like):
        import torch
        k, d = self.k, self.d
        dev = like.device
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.pair_pos = torch.empty((T * k,), dtype=torch.int32, device=dev)
        self.y_pairs = torch.empty((T * k, d), dtype=torch.float32, device=dev)
        nb = int(load_library().moe_cache_ws_bytes(self.handle, T, k))
        self.ws = torch.empty((max(nb, 256),), dtype=torch.uint8, device=dev)
        self._T = T

    def forward(self, x, out=None, out_dtype=MOE_OUT_BF16, bits=None,
                bits_mode=MOE_BITS_NONE, stream=None):
        import torch
        T = x.shape[0]
        if self._T != T:
            self._alloc(T, x)
        if out is None:
            out = _empty((T, self.d), torch.bfloat16 if out_dtype == MOE_OUT_BF16
                         else torch.float32, x)
        _check("moe_cache_forward", load_library().moe_cache_forward(
            self.handle, _ptr(x), _ptr(self.wr), _ptr(self.bias), T, self.k, _ptr(bits),
            bits_mode, _ptr(self.topk_idx), _ptr(self.topk_w), _ptr(self.pair_pos),
            _ptr(self.y_pairs), _ptr(out), out_dtype, _ptr(self.ws),
            self.ws.numel(), _stream(stream)))
        return out

    def stats(self):
        import numpy as np
        a = np.zeros(6, np.int64)
        _check("moe_cache_stats", load_library().moe_cache_stats(self.handle, _np_ptr(a)))
        keys = ("steps", "hits", "loads_full", "loads_partial", "bytes", "chunks")
        return {k: int(v) for k, v in zip(keys, a)}

    def resident(self):
        """(expert [slots], planes [slots]) of each slot; -1 = empty."""
        import numpy as np
        e = np.zeros(self.slots, np.int32)
        b = np.zeros(self.slots, np.int32)
        _check("moe_cache_slots", load_library().moe_cache_slots(self.handle, _np_ptr(e),
                                                                _np_ptr(b)))
        return e, b

    def reset(self):
        _check("moe_cache_reset", load_library().moe_cache_reset(self.handle))

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            load_library().moe_cache_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# --------------------------------------------------------- one whole layer
class MoeLayer:
    """Resident quantized expert weights plus preallocated buffers for one
    batch size; `forward(x)` enqueues route+permute, the expert FFN and the
    combine on one stream."""

    def __init__(self, wr, bias, k, f, gate_up_codes, gate_up_scales,
                 down_codes, down_scales, fmt=MOE_FMT_W4_SYM,
                 bits_mode=MOE_BITS_NONE, bits=None):
        self.wr, self.bias, self.k, self.f = wr, bias, k, f
        self.E, self.d = wr.shape
        self.gu, self.gus, self.dn, self.dns = (gate_up_codes, gate_up_scales,
                                                down_codes, down_scales)
        self.fmt, self.bits_mode, self.bits = fmt, bits_mode, bits
        self._T = None

    def _alloc(self, T, like):
        import torch
        E, k, d, f = self.E, self.k, self.d, self.f
        P = T * k
        dev = like.device
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        self.sorted_pair = torch.empty((P,), dtype=torch.int32, device=dev)
        self.pair_pos = torch.empty((P,), dtype=torch.int32, device=dev)
        self.ws_rp = torch.empty((max(moe_route_permute_ws_bytes(T, k, E), 16),),
                                 dtype=torch.uint8, device=dev)
        self.ws_ffn = torch.empty((max(moe_ffn_ws_bytes(T, k, E, d, f, self.fmt), 256),),
                                  dtype=torch.uint8, device=dev)
        self.ws_layer = torch.empty((max(moe_layer_ws_bytes(T, k, E, d, f, self.fmt), 256),),
                                    dtype=torch.uint8, device=dev)
        self.y_pairs = torch.empty((P, d), dtype=torch.float32, device=dev)
        self._T = T

    def forward(self, x, out=None, out_dtype=MOE_OUT_BF16, path=MOE_PATH_AUTO,
                stream=None, weights=None):
        """One layer step through moe_layer_forward_wq."""
        import torch
        T = x.shape[0]
        if self._T != T:
            self._alloc(T, x)
        gu, gus, dn, dns = weights if weights is not None else (
            self.gu, self.gus, self.dn, self.dns)
        if out is None:
            out = _empty((T, self.d), torch.bfloat16 if out_dtype == MOE_OUT_BF16
                         else torch.float32, x)
        return moe_layer_forward(x, self.wr, self.bias, self.k, self.f, gu, gus, dn, dns,
                                 self.topk_idx, self.topk_w, self.offsets, self.sorted_pair,
                                 self.pair_pos, self.y_pairs, out, self.ws_layer, self.fmt,
                                 self.bits, self.bits_mode, out_dtype, path, stream)

    def forward_steps(self, x, out=None, out_dtype=MOE_OUT_BF16, path=MOE_PATH_AUTO,
                      stream=None, weights=None):
        """The same step as moe_route_permute, moe_expert_ffn_wq and
        moe_combine calls (the composition the layer entry point equals)."""
        T = x.shape[0]
        if self._T != T:
            self._alloc(T, x)
        gu, gus, dn, dns = weights if weights is not None else (
            self.gu, self.gus, self.dn, self.dns)
        moe_route_permute(x, self.wr, self.bias, self.k, self.ws_rp, self.topk_idx,
                          self.topk_w, self.offsets, self.sorted_pair, self.pair_pos,
                          stream)
        moe_expert_ffn_wq(x, self.offsets, self.sorted_pair, self.k, self.f, gu, gus,
                          dn, dns, self.fmt, self.bits, self.bits_mode,
                          self.y_pairs, self.ws_ffn, path, stream)
        return moe_combine(self.y_pairs, self.pair_pos, self.topk_w, out, out_dtype,
                           stream)

    def bind(self, x, out, weights=None, path=MOE_PATH_AUTO, out_dtype=MOE_OUT_BF16,
             stream=None):
        """A step with every argument marshalled once: returns a callable that
        enqueues the same ABI call as forward(x, out, ...) for these fixed
        buffers (x, out and the weights must stay alive and in place).
        For decode loops, where converting arguments on every call would cost
        as much host time as the kernels take on the GPU."""
        T = x.shape[0]
        if self._T != T:
            self._alloc(T, x)
        gu, gus, dn, dns = weights if weights is not None else (
            self.gu, self.gus, self.dn, self.dns)
        E, k, d, f = self.E, self.k, self.d, self.f
        args = (_ptr(x), _ptr(self.wr), _ptr(self.bias), T, d, E, k, f, self.fmt, MOE_GROUP,
                _ptr(gu), _ptr(gus), _ptr(dn), _ptr(dns), _ptr(self.bits), self.bits_mode,
                _ptr(self.topk_idx), _ptr(self.topk_w), _ptr(self.offsets),
                _ptr(self.sorted_pair), _ptr(self.pair_pos), _ptr(self.y_pairs), _ptr(out),
                out_dtype, _ptr(self.ws_layer),
                self.ws_layer.numel() * self.ws_layer.element_size(), path, _stream(stream))
        fn = load_library().moe_layer_forward_wq

        def step():
            rc = fn(*args)
            if rc:
                _check("moe_layer_forward_wq", rc)
            return out

        return step

    def capture(self, x, out, weights=None, path=MOE_PATH_AUTO, out_dtype=MOE_OUT_BF16):
        """One step for these fixed buffers recorded as a HIP graph (torch's
        CUDAGraph object; replay() re-runs the five kernels with one host
        call).  The library records only kernel launches (no memset or
        copy nodes) and allocates nothing, so replays are self-contained."""
        import torch
        T = x.shape[0]
        if self._T != T:
            self._alloc(T, x)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):  # binds to the capture stream
            self.bind(x, out, weights, path, out_dtype)()
        return g
