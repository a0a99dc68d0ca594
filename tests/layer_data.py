"""Shared setup of the GPU parity tests: device-resident layer inputs drawn by
the seeded generator (synth/), and the oracle's view of the same inputs."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
import quantized_mixture_experts_fp32_amd as moe

DEV = torch.device("cuda:0")


def stream():
    return torch.cuda.current_stream().cuda_stream


def custom_cfg(cid, d, E, k, f, fmt="w4", bias_sigma=None):
    return synth.LayerConfig(cid, f"custom{cid}", d, E, k, f, (), fmt,
                             bias_sigma=bias_sigma)


def apply_zeros(w, tid, e, zero):
    """Zero the blocks of zero = [(tensor id, expert, r0, r1, c0, c1)] that
    fall on matrix tid of expert e (w is that expert's [rows][K] weights, a
    numpy array or a torch view); the same spec serves device and host."""
    for (zt, ze, r0, r1, c0, c1) in (zero or ()):
        if zt == tid and ze == e:
            w[r0:r1, c0:c1] = 0


class DevLayer:
    """Device inputs of one layer configuration for a batch of T tokens.
    zero: optional blocks of the fp32 expert weights set to 0 before
    quantization (see apply_zeros)."""

    def __init__(self, cfg, T, step=0, zero=None):
        self.cfg, self.T = cfg, T
        d, E, f = cfg.d, cfg.E, cfg.f
        s = stream()
        self.x = torch.empty((T, d), dtype=torch.int16, device=DEV)
        if T:
            synth.dev_fill_x(cfg, self.x.data_ptr(), T, s, step=step)
        self.wr = torch.empty((E, d), dtype=torch.int16, device=DEV)
        synth.dev_fill_router(cfg, self.wr.data_ptr(), s)
        self.bias = None
        if cfg.bias_sigma is not None:
            self.bias = torch.empty((E,), dtype=torch.float32, device=DEV)
            synth.dev_fill_bias(cfg, self.bias.data_ptr(), s)
        q = moe.moe_quantize_w4 if cfg.fmt == "w4" else moe.moe_quantize_bitplane8
        w = torch.empty((E, 2 * f, d), dtype=torch.float32, device=DEV)
        synth.dev_fill_weight(cfg, synth.T_W_GATE_UP, w.data_ptr(), s)
        for e in {z[1] for z in (zero or ())}:
            apply_zeros(w[e], synth.T_W_GATE_UP, e, zero)
        self.guc, self.gus = q(w)
        del w
        w = torch.empty((E, d, f), dtype=torch.float32, device=DEV)
        synth.dev_fill_weight(cfg, synth.T_W_DOWN, w.data_ptr(), s)
        for e in {z[1] for z in (zero or ())}:
            apply_zeros(w[e], synth.T_W_DOWN, e, zero)
        self.dnc, self.dns = q(w)
        del w
        torch.cuda.synchronize()

    @staticmethod
    def x_only(cfg, T, step):
        """The activations of step `step` alone (weights unchanged)."""
        x = torch.empty((T, cfg.d), dtype=torch.int16, device=DEV)
        if T:
            synth.dev_fill_x(cfg, x.data_ptr(), T, stream(), step=step)
        return x

    def layer(self, bits_mode=moe.MOE_BITS_NONE, bits=None):
        fmt = moe.MOE_FMT_W4_SYM if self.cfg.fmt == "w4" else moe.MOE_FMT_BITPLANE8
        return moe.MoeLayer(self.wr, self.bias, self.cfg.k, self.cfg.f, self.guc,
                            self.gus, self.dnc, self.dns, fmt, bits_mode, bits)

    def expert_codes(self, e):
        return ((self.guc[e].cpu().numpy(), self.gus[e].cpu().numpy().view(np.uint16)),
                (self.dnc[e].cpu().numpy(), self.dns[e].cpu().numpy().view(np.uint16)))


class HostLayer:
    """The oracle's copy of the same inputs (host generator + oracle quantizer)."""

    def __init__(self, cfg, T, step=0, zero=None):
        self.cfg, self.T = cfg, T
        self.x = synth.host_x(cfg, T, step=step)
        self.wr = synth.host_router(cfg)
        self.bias = synth.host_bias(cfg)
        self.zero = zero
        self._cache = {}

    def expert(self, e):
        if e not in self._cache:
            c = self.cfg
            q = oracle.quantize_w4 if c.fmt == "w4" else oracle.quantize_bp8
            m = []
            for tid in (synth.T_W_GATE_UP, synth.T_W_DOWN):
                w = synth.host_expert(c, tid, e)
                apply_zeros(w, tid, e, self.zero)
                m.append(q(w))
            self._cache[e] = tuple(m)
        return self._cache[e]

    def y_rows(self, e, tokens, bits=None):
        """The oracle's y rows of expert e for the listed tokens (bitplane:
        at the per-row widths `bits`), dequantizing the expert once."""
        (gq, gs), (dq, ds) = self.expert(int(e))
        tokens = np.asarray(tokens, np.int64)
        if bits is None:
            wg, wd = oracle.dequant_w4(gq, gs), oracle.dequant_w4(dq, ds)
            return oracle.expert_ffn(self.x[tokens], wg, wd)[1]
        bits = np.asarray(bits)
        y = np.zeros((len(tokens), self.cfg.d))
        for b in np.unique(bits):
            sel = np.nonzero(bits == b)[0]
            wg, wd = oracle.dequant_bp(gq, gs, int(b)), oracle.dequant_bp(dq, ds, int(b))
            y[sel] = oracle.expert_ffn(self.x[tokens[sel]], wg, wd)[1]
        return y


# nibble i of a code word holds element W4_NIBBLE_ELEMENT[i] of its 8
W4_NIBBLE_ELEMENT = np.array([0, 2, 4, 6, 1, 3, 5, 7])


def w4_untile(codes, N, K):
    """The library's int4 codes of one N x K matrix (include/moe_wq.h: 16-row
    tiles [N/16][K/128][16][64] bytes; 32-bit word j of a row's group holds
    elements 8j..8j+7, even ones in nibbles 0-3, odd ones in nibbles 4-7)
    -> the oracle's row-major packing [N][K/2] (byte b: element 2b in the low
    nibble, 2b+1 in the high nibble).  A pure rearrangement of nibbles."""
    t = np.asarray(codes, np.uint8).reshape(N // 16, K // 128, 16, 64)
    t = t.transpose(0, 2, 1, 3).reshape(N, K // 8, 4).astype(np.uint32)
    words = t[..., 0] | (t[..., 1] << 8) | (t[..., 2] << 16) | (t[..., 3] << 24)
    elems = np.empty((N, K // 8, 8), np.uint8)
    for i in range(8):
        elems[:, :, W4_NIBBLE_ELEMENT[i]] = (words >> (4 * i)) & 0xF
    elems = elems.reshape(N, K)
    return (elems[:, 0::2] | (elems[:, 1::2] << 4)).astype(np.uint8)


def bp_untile(planes, N, K):
    """The library's bitplanes of one N x K matrix (include/moe_wq.h: per
    16-row tile and 128-group a 2 KiB block [pair c][row r][quarter q]
    [plane 2c + s][4 bytes]) -> the oracle's plane-major layout [8][N][K/8].
    A pure byte permutation."""
    t = np.asarray(planes, np.uint8).reshape(N // 16, K // 128, 4, 16, 4, 2, 4)
    # axes: tile, g, c, r, q, s, b  ->  [c, s][tile, r][g, q, b]
    return t.transpose(2, 5, 0, 3, 1, 4, 6).reshape(8, N, K // 8)


def untile(codes, fmt, N, K):
    return w4_untile(codes, N, K) if fmt == "w4" else bp_untile(codes, N, K)


def assert_codes_equal(dev_layer, host_layer, experts):
    """Packed codes and fp16 scales of the listed experts are bit-identical."""
    fmt = dev_layer.cfg.fmt
    for e in experts:
        g, h = dev_layer.expert_codes(int(e)), host_layer.expert(int(e))
        for (dq, ds), (hq, hs) in zip(g, h):
            N, K = hs.shape[0], 128 * hs.shape[1]
            dq = untile(dq, fmt, N, K)
            assert np.array_equal(dq, hq.reshape(dq.shape)), f"codes of expert {e}"
            assert np.array_equal(ds, hs.reshape(ds.shape)), f"scales of expert {e}"


def errors(a, ref):
    """(relative L2 error, max abs error / rms(ref)) in fp64."""
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    rel = np.linalg.norm(a - ref) / max(np.linalg.norm(ref), 1e-300)
    return rel, np.abs(a - ref).max() / max(rms, 1e-300)


REL_L2_TOL = 2e-3      # floating-point bar of the layer outputs
MAX_ABS_TOL = 3e-2     # max |a - ref| <= 3e-2 * rms(ref)


def record(line):
    """Append a measured error line to $MOE_PARITY_LOG (if set)."""
    import os
    path = os.environ.get("MOE_PARITY_LOG")
    if path:
        with open(path, "a") as fh:
            fh.write(line + "\n")


def assert_close(a, ref, what):
    rel, mx = errors(a, ref)
    import os
    line = f"{os.environ.get('PYTEST_CURRENT_TEST', '?').split(' ')[0]} {what}: " \
           f"rel_l2={rel:.3e} max_abs/rms={mx:.3e}"
    print("  " + line, flush=True)
    record(line)
    assert rel <= REL_L2_TOL and mx <= MAX_ABS_TOL, (what, rel, mx)
    return rel, mx


def bf16_rne_bits(a32):
    u = np.asarray(a32, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
