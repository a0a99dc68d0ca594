"""GPU parity of every step of the layer against the CPU oracle, through the
C ABI.  Integer results (top-k ids, grouping, codes, scales) must be
bit-identical; floating-point outputs must be within rel-L2 <= 2e-3 and
max|err| <= 3e-2 * rms(ref) of the oracle (fp64 accumulation, same
dequantized weights)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import quantized_mixture_experts_fp32_amd as moe
from layer_data import (DEV, DevLayer, HostLayer, assert_close, assert_codes_equal,
                        bf16_rne_bits, custom_cfg, record, untile,
                        stream)

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)


def t_i16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


# ----------------------------------------------------------------- inputs
def test_generator_device_equals_host():
    cfg = synth.CONFIGS[4]
    note("generator: cfg4 x/router/bias/weight slices")
    x = torch.empty((64, cfg.d), dtype=torch.int16, device=DEV)
    synth.dev_fill_x(cfg, x.data_ptr(), 64, stream())
    wr = torch.empty((cfg.E, cfg.d), dtype=torch.int16, device=DEV)
    synth.dev_fill_router(cfg, wr.data_ptr(), stream())
    b = torch.empty((cfg.E,), dtype=torch.float32, device=DEV)
    synth.dev_fill_bias(cfg, b.data_ptr(), stream())
    n = 1 << 20
    start = 3 * 2 * cfg.f * cfg.d + 12345
    w = torch.empty((n,), dtype=torch.float32, device=DEV)
    synth.dev_fill_weight(cfg, synth.T_W_GATE_UP, w.data_ptr(), stream(), start=start, n=n)
    torch.cuda.synchronize()
    assert np.array_equal(x.cpu().numpy().view(np.uint16), synth.host_x(cfg, 64))
    assert np.array_equal(wr.cpu().numpy().view(np.uint16), synth.host_router(cfg))
    assert np.array_equal(b.cpu().numpy(), synth.host_bias(cfg))
    host = np.empty(n, np.float32)
    synth._load_host().synth_fill_weight_f32(42, cfg.cid, synth.T_W_GATE_UP, start, n,
                                             synth.W_SIGMA, synth._ptr(host))
    assert np.array_equal(w.cpu().numpy().view(np.uint32), host.view(np.uint32))


# ------------------------------------------------------------- quantizers
def _edge_weights(rng, R, K):
    w = (rng.normal(0, 0.14, (R, K)) * np.where(rng.random((R, K)) < 0.01, 10, 1))
    w = w.astype(np.float32)
    w[0, :128] = 0.0                                   # all-zero group: s = 0
    w[1, :128] = 0.0
    w[1, 5] = 1e-30                                    # scale below fp16 range
    w[2, :128] = np.float32(0.4375) * np.arange(-64, 64) / 64  # exact ties at .5
    w[3, 128:256] = -np.abs(w[3, 128:256])             # negative group maximum
    w[4, :128] = 7 * 65000.0 * rng.uniform(-1, 1, 128).astype(np.float32)  # near fp16 max
    return w


@pytest.mark.parametrize("fmt", ["w4", "bp8"])
def test_quantize_bit_exact(fmt):
    rng = np.random.default_rng(7)
    # rows are tiled by 16
    for (E, N, K) in [(2, 16, 256), (3, 48, 384), (1, 32, 2048)]:
        note(f"quantize {fmt} E={E} N={N} K={K}")
        w = np.stack([_edge_weights(rng, N, K) for _ in range(E)])
        wd = torch.from_numpy(w).to(DEV)
        if fmt == "w4":
            codes, scales = moe.moe_quantize_w4(wd)
            ref = [oracle.quantize_w4(w[e]) for e in range(E)]
        else:
            codes, scales = moe.moe_quantize_bitplane8(wd)
            ref = [oracle.quantize_bp8(w[e]) for e in range(E)]
        torch.cuda.synchronize()
        c, s = codes.cpu().numpy(), scales.cpu().numpy().view(np.uint16)
        for e in range(E):
            ce = untile(c[e], fmt, N, K)
            assert np.array_equal(ce, ref[e][0]), (fmt, e)
            assert np.array_equal(s[e], ref[e][1]), (fmt, e)


@pytest.mark.parametrize("fmt", ["w4", "bp8"])
def test_retile_canonical_bit_exact(fmt):
    """Canonical code layouts -> streaming layouts: untiling the output gives
    back the input bytes, and the oracle's canonical codes of fp32 weights,
    retiled, equal the library's own quantizer output bit for bit."""
    rng = np.random.default_rng(21)
    for (E, N, K) in [(1, 16, 128), (2, 48, 384), (3, 32, 2048)]:
        note(f"retile {fmt} E={E} N={N} K={K}")
        if fmt == "w4":
            canon = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
            out = moe.moe_retile_w4(torch.from_numpy(canon).to(DEV), N, K)
        else:
            canon = rng.integers(0, 256, (E, 8, N, K // 8), dtype=np.uint8)
            out = moe.moe_retile_bitplane8(torch.from_numpy(canon).to(DEV), N, K)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        for e in range(E):
            assert np.array_equal(untile(o[e], fmt, N, K), canon[e].reshape(
                untile(o[e], fmt, N, K).shape)), (fmt, e)
        # oracle canonical codes of real weights, retiled == library quantizer
        w = np.stack([_edge_weights(rng, N, K) for _ in range(E)])
        if fmt == "w4":
            ref = np.stack([oracle.quantize_w4(w[e])[0] for e in range(E)])
            mine = moe.moe_retile_w4(torch.from_numpy(ref).to(DEV), N, K)
            lib = moe.moe_quantize_w4(torch.from_numpy(w).to(DEV))[0]
        else:
            ref = np.stack([oracle.quantize_bp8(w[e])[0] for e in range(E)])
            mine = moe.moe_retile_bitplane8(torch.from_numpy(ref).to(DEV), N, K)
            lib = moe.moe_quantize_bitplane8(torch.from_numpy(w).to(DEV))[0]
        torch.cuda.synchronize()
        assert torch.equal(mine, lib), (fmt, E, N, K)


# ----------------------------------------------------------------- router
ROUTE_CASES = [(0, 16), (1, 16), (2, 4096), (3, 16), (4, 1), (4, 64), (4, 8192)]


@pytest.mark.parametrize("cid,T", ROUTE_CASES)
def test_route_bit_exact(cid, T):
    cfg = synth.CONFIGS[cid]
    note(f"route cfg{cid} T={T}")
    x, wr, bias = synth.host_x(cfg, T), synth.host_router(cfg), synth.host_bias(cfg)
    idx, w = moe.moe_route(t_i16(x), t_i16(wr),
                           None if bias is None else torch.from_numpy(bias).to(DEV), cfg.k)
    torch.cuda.synchronize()
    _, ridx, rw = oracle.route(x, wr, bias, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("cid,T", ROUTE_CASES + [(1, 17), (1, 201), (0, 255), (1, 512),
                                                  (1, 513)])
def test_route_permute_bit_exact(cid, T):
    """The fused call equals the oracle's routing and grouping bit for bit
    (every launch shape: one block selecting and grouping at few pairs,
    logits of one or two tokens per block then top-k then grouping up to 512
    tokens (T = 201: an odd count, the last block holds one token), eight
    tokens per block beyond)."""
    cfg = synth.CONFIGS[cid]
    note(f"route+permute cfg{cid} T={T}")
    x, wr, bias = synth.host_x(cfg, T), synth.host_router(cfg), synth.host_bias(cfg)
    idx, w, off, sp, pp = moe.moe_route_permute(
        t_i16(x), t_i16(wr), None if bias is None else torch.from_numpy(bias).to(DEV), cfg.k)
    torch.cuda.synchronize()
    _, ridx, rw = oracle.route(x, wr, bias, cfg.k)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=2e-6, atol=1e-7)
    roff, rsp, rpp = oracle.permute(ridx, cfg.E)
    assert np.array_equal(off.cpu().numpy(), roff)
    assert np.array_equal(sp.cpu().numpy(), rsp)
    assert np.array_equal(pp.cpu().numpy(), rpp)


def test_route_ties_and_shapes():
    rng = np.random.default_rng(3)
    cases = []
    # duplicated router rows -> exactly equal logits, ties to the lower index
    d, E = 256, 12
    wr = (rng.normal(0, 1 / 16, (E, d)) * 256).round() / 256
    wr[7] = wr[2]
    wr[9] = wr[2]
    wr[11] = wr[4]
    cases.append(("dup-rows", d, E, 5, wr, None))
    # zero router: logits are the bias; equal biases tie
    cases.append(("zero-router", 128, 33, 6, np.zeros((33, 128)),
                  np.repeat(np.array([0.5, -1.0, 0.5], np.float32), 11)))
    cases.append(("E=1", 128, 1, 1, rng.normal(0, 0.1, (1, 128)), None))
    cases.append(("k=E", 384, 6, 6, rng.normal(0, 0.1, (6, 384)), None))
    cases.append(("E=500", 128, 500, 16, rng.normal(0, 0.1, (500, 128)), None))
    for name, d, E, k, wrf, bias in cases:
        note(f"route {name}")
        T = 37
        x = np.round(rng.normal(0, 1, (T, d)) * 64) / 64
        xb = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        wb = (np.asarray(wrf, np.float32).view(np.uint32) >> 16).astype(np.uint16)
        bt = None if bias is None else torch.from_numpy(bias).to(DEV)
        idx, w = moe.moe_route(t_i16(xb), t_i16(wb), bt, k)
        torch.cuda.synchronize()
        _, ridx, rw = oracle.route(xb, wb, bias, k)
        assert np.array_equal(idx.cpu().numpy(), ridx), name
        np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("E,k", [(65, 8), (128, 1), (200, 3), (256, 8), (300, 8),
                                 (512, 8), (256, 16)])
@pytest.mark.parametrize("T", [17, 64, 333])
def test_route_many_experts_ties(E, k, T):
    """More than 64 experts and 17..512 tokens (one wave per token selects
    over all E logits, then the pairs are grouped): exact logit ties from
    duplicated router rows and tied biases, and a token whose logits are the
    biases alone, must resolve to the lower index; routing and grouping
    bit-exact."""
    note(f"route many experts E={E} k={k} T={T}")
    rng = np.random.default_rng(E * 7 + k + T)
    d = 256
    wr = (rng.normal(0, 1 / 16, (E, d)) * 256).round() / 256
    for dst, src in ((E - 1, 0), (64 % E, 0), (E // 2, 3), (min(E - 1, 130), 3), (5, 4)):
        wr[dst] = wr[src]
    bias = np.zeros(E, np.float32)
    bias[::7] = 0.25                                     # tied biases in every group
    x = np.round(rng.normal(0, 1, (T, d)) * 64) / 64
    x[T // 2] = 0.0                                     # this token: logits = bias
    xb = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    wb = (np.asarray(wr, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bt = torch.from_numpy(bias).to(DEV)
    _, ridx, rw = oracle.route(xb, wb, bias, k)
    idx, w = moe.moe_route(t_i16(xb), t_i16(wb), bt, k)
    idx2, w2, off, sp, pp = moe.moe_route_permute(t_i16(xb), t_i16(wb), bt, k)
    torch.cuda.synchronize()
    for a, b in ((idx, w), (idx2, w2)):
        assert np.array_equal(a.cpu().numpy(), ridx)
        np.testing.assert_allclose(b.cpu().numpy(), rw, rtol=2e-6, atol=1e-7)
    roff, rsp, rpp = oracle.permute(ridx, E)
    assert np.array_equal(off.cpu().numpy(), roff)
    assert np.array_equal(sp.cpu().numpy(), rsp)
    assert np.array_equal(pp.cpu().numpy(), rpp)
    # the all-tied token picks the lowest-index experts of bias 0.25
    assert list(ridx[T // 2]) == list(np.nonzero(bias == 0.25)[0][:k]) or k > (bias > 0).sum()


# ---------------------------------------------------------------- permute
@pytest.mark.parametrize("T,k,E,mode", [(0, 8, 16, "rand"), (1, 1, 1, "rand"),
                                        (33, 3, 5, "rand"), (1000, 8, 64, "one"),
                                        (4096, 8, 64, "skew"), (8192, 8, 256, "skew"),
                                        (777, 16, 512, "rand"), (2100, 8, 64, "skew")])
def test_permute_bit_exact(T, k, E, mode):
    note(f"permute T={T} k={k} E={E} {mode}")
    rng = np.random.default_rng(T + k + E)
    if mode == "one":
        idx = np.full((T, k), 3 % E, np.int32)
    elif mode == "skew":
        p = rng.dirichlet(np.full(E, 0.3))
        idx = rng.choice(E, size=(T, k), p=p).astype(np.int32)
    else:
        idx = rng.integers(0, E, (T, k)).astype(np.int32)
    off, sp, pp = moe.moe_permute(torch.from_numpy(idx).to(DEV), E)
    torch.cuda.synchronize()
    roff, rsp, rpp = oracle.permute(idx, E)
    assert np.array_equal(off.cpu().numpy(), roff)
    assert np.array_equal(sp.cpu().numpy(), rsp)
    assert np.array_equal(pp.cpu().numpy(), rpp)


# ---------------------------------------------------------------- combine
def test_combine_fp32_and_bf16():
    rng = np.random.default_rng(5)
    for T, k, d in [(1, 8, 2048), (37, 3, 256), (513, 8, 4096)]:
        note(f"combine T={T} k={k} d={d}")
        y = rng.normal(0, 1, (T * k, d)).astype(np.float32)
        pp = rng.permutation(T * k).astype(np.int32)
        w = rng.dirichlet(np.ones(k), T).astype(np.float32)
        yd, pd, wd = (torch.from_numpy(a).to(DEV) for a in (y, pp, w))
        o32 = moe.moe_combine(yd, pd, wd, out_dtype=moe.MOE_OUT_F32)
        o16 = moe.moe_combine(yd, pd, wd, out_dtype=moe.MOE_OUT_BF16)
        torch.cuda.synchronize()
        ref, _ = oracle.combine(y.astype(np.float64), pp, w.astype(np.float64))
        a = o32.cpu().numpy()
        assert np.all(np.abs(a - ref) <= 1e-5 * (np.abs(ref) + 1))
        assert np.array_equal(o16.cpu().view(torch.int16).numpy().view(np.uint16),
                              bf16_rne_bits(a))


# ------------------------------------------------------------ whole layer
def run_layer(dl, path, bits_mode=moe.MOE_BITS_NONE, bits=None):
    lay = dl.layer(bits_mode, bits)
    o32 = lay.forward(dl.x, out_dtype=moe.MOE_OUT_F32, path=path).clone()
    o16 = moe.moe_combine(lay.y_pairs, lay.pair_pos, lay.topk_w, out_dtype=moe.MOE_OUT_BF16)
    torch.cuda.synchronize()
    return lay, o32.cpu().numpy(), o16.cpu().view(torch.int16).numpy().view(np.uint16)


def check_layer(dl, hl, path, bits_mode=moe.MOE_BITS_NONE, bits_np=None):
    bits = None if bits_np is None else torch.from_numpy(bits_np).to(DEV)
    lay, o32, o16 = run_layer(dl, path, bits_mode, bits)
    cfg = dl.cfg
    ref = oracle.layer(hl.x, hl.wr, hl.bias, cfg.k, cfg.f, hl.expert, cfg.fmt,
                       bits_mode, bits_np)
    assert np.array_equal(lay.topk_idx.cpu().numpy(), ref["topk_idx"])
    np.testing.assert_allclose(lay.topk_w.cpu().numpy(), ref["topk_w"], rtol=2e-6, atol=1e-7)
    assert np.array_equal(lay.offsets.cpu().numpy(), ref["expert_offsets"])
    assert np.array_equal(lay.sorted_pair.cpu().numpy(), ref["sorted_pair"])
    assert np.array_equal(lay.pair_pos.cpu().numpy(), ref["pair_pos"])
    active = np.nonzero(np.diff(ref["expert_offsets"]))[0]
    assert_codes_equal(dl, hl, active)
    assert_close(lay.y_pairs.cpu().numpy(), ref["y_pairs"], "y_pairs")
    assert_close(o32, ref["o"], "out fp32")
    # bf16 output: exactly the rounding of the fp32 output (whose max-abs and
    # rel-L2 errors are checked above).  Against the fp64 oracle the bf16
    # output is held to the rel-L2 bar only: its own rounding (2^-9
    # relative) alone exceeds the max-abs bar wherever |o| > 15 rms(o).
    assert np.array_equal(o16, bf16_rne_bits(o32))
    o16f = (o16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rel = np.linalg.norm(o16f - ref["o"]) / np.linalg.norm(ref["o"])
    ndiff = int((o16 != ref["out"]).sum())
    record(f"{cfg.name} bf16 out: rel_l2={rel:.3e}; {ndiff} of {o16.size} differ "
           f"from the oracle's bf16 rounding")
    assert rel <= 2e-3
    return lay, o32


PATHS = [moe.MOE_PATH_DECODE, moe.MOE_PATH_PREFILL]


@pytest.mark.parametrize("path", PATHS)
def test_layer_cfg0(path):
    note(f"layer cfg0 path={path}")
    cfg = synth.CONFIGS[0]
    check_layer(DevLayer(cfg, 16), HostLayer(cfg, 16), path)


@pytest.mark.parametrize("path", PATHS)
def test_layer_ragged_tiles(path):
    # several token tiles per expert and a ragged tail, f not a power of two
    cfg = custom_cfg(11, d=256, E=5, k=3, f=384, bias_sigma=1.0)
    note(f"layer custom ragged T=100 path={path}")
    check_layer(DevLayer(cfg, 100), HostLayer(cfg, 100), path)


def test_layer_decode_single_slice_ragged():
    # the decode kernels that stage activations in LDS (one K slice per wave,
    # tiles of up to 16 pairs): group counts 3 (gate/up) and 13 (down) that
    # are not multiples of the code prefetch depth, skewed routing so that
    # some experts span several tiles with a ragged last tile
    cfg = custom_cfg(14, d=384, E=128, k=4, f=1664, bias_sigma=2.0)
    note("layer custom single-slice decode T=32")
    dl, hl = DevLayer(cfg, 32), HostLayer(cfg, 32)
    lay, _ = check_layer(dl, hl, moe.MOE_PATH_DECODE)
    cnt = np.diff(lay.offsets.cpu().numpy())
    assert cnt.max() > 16 and (cnt % 16 != 0).any()


def test_layer_all_pairs_one_expert_and_empty_experts():
    cfg = custom_cfg(12, d=128, E=16, k=2, f=128, bias_sigma=30.0)
    note("layer skew: bias 30 sigma -> nearly all pairs on two experts")
    dl, hl = DevLayer(cfg, 70), HostLayer(cfg, 70)
    lay, _ = check_layer(dl, hl, moe.MOE_PATH_AUTO)
    cnt = np.diff(lay.offsets.cpu().numpy())
    assert (cnt == 0).sum() >= 8


@pytest.mark.parametrize("T", [1, 4, 8, 16])
def test_layer_cfg1_decode(T):
    note(f"layer cfg1 T={T}")
    cfg = synth.CONFIGS[1]
    check_layer(DevLayer(cfg, T), HostLayer(cfg, T), moe.MOE_PATH_AUTO)


@pytest.mark.parametrize("case", ["dup-rows", "zero-router"])
@pytest.mark.parametrize("T", [1, 2, 3, 16])
def test_layer_decode_router_ties(case, T):
    """Whole layer with exactly equal logits (ties to the lower index) at a
    few tokens, where the decode kernels take the routing from the logits
    (T = 1, 2: the K-split gate/up selects and groups; T = 3, 16: the
    expert-major kernels): duplicated router rows, and a zero router whose
    logits are tied biases."""
    note(f"layer decode ties {case} T={T}")
    cfg = custom_cfg(22, d=256, E=16, k=4, f=256, bias_sigma=1.0)
    dl, hl = DevLayer(cfg, T), HostLayer(cfg, T)
    wr = hl.wr.copy()
    if case == "dup-rows":
        wr[7] = wr[2]
        wr[9] = wr[2]
        wr[11] = wr[4]
        wr[15] = wr[0]
        bias = None
    else:
        wr[:] = 0
        bias = np.repeat(np.array([0.5, -1.0, 0.5, 2.0], np.float32), 4)
    hl.wr, hl.bias = wr, bias
    dl.wr = torch.from_numpy(wr.view(np.int16)).to(DEV)
    dl.bias = None if bias is None else torch.from_numpy(bias).to(DEV)
    lay, _ = check_layer(dl, hl, moe.MOE_PATH_AUTO)
    if case == "zero-router":
        # every token picks the four experts of bias 2.0 (12..15)
        assert np.array_equal(lay.topk_idx.cpu().numpy(), np.tile([12, 13, 14, 15], (T, 1)))


@pytest.mark.parametrize("E,k,T", [(16, 1, 16), (16, 1, 2), (32, 16, 1), (64, 8, 3), (48, 5, 7)])
def test_layer_decode_topk_shapes(E, k, T):
    """Routing from the logits inside the decode kernels at the extremes of k
    (1 and 16), a single token choosing half the experts, and E not a
    multiple of 64: ids, weights and grouping bit-exact or in tolerance as
    for every layer."""
    note(f"layer decode top-k shapes E={E} k={k} T={T}")
    cfg = custom_cfg(23, d=256, E=E, k=k, f=256, bias_sigma=0.5)
    check_layer(DevLayer(cfg, T), HostLayer(cfg, T), moe.MOE_PATH_AUTO)


@pytest.mark.parametrize("T", [1, 16])
def test_layer_cfg1_sequential_per_expert(T):
    """One launch per expert over the same routed pairs gives the fused result."""
    note(f"layer cfg1 sequential per-expert T={T}")
    cfg = synth.CONFIGS[1]
    dl, hl = DevLayer(cfg, T), HostLayer(cfg, T)
    lay, _, _ = run_layer(dl, moe.MOE_PATH_DECODE)
    E, d = lay.E, lay.d
    fmt = moe.MOE_FMT_W4_SYM
    ws = torch.empty((max(moe.moe_ffn_ws_bytes(T, cfg.k, 1, d, cfg.f, fmt), 256),),
                     dtype=torch.uint8, device=DEV)
    ref = oracle.layer(hl.x, hl.wr, hl.bias, cfg.k, cfg.f, hl.expert, cfg.fmt,
                       moe.MOE_BITS_NONE, None)
    active = np.nonzero(np.diff(lay.offsets.cpu().numpy()))[0]
    for experts in (None, active):      # every expert, then the activated ones
        y = torch.full_like(lay.y_pairs, float("nan"))
        moe.expert_ffn_per_expert(dl.x, lay.offsets, lay.sorted_pair, cfg.k, cfg.f,
                                  dl.guc, dl.gus, dl.dnc, dl.dns, y, ws, fmt,
                                  path=moe.MOE_PATH_DECODE, experts=experts)
        o = moe.moe_combine(y, lay.pair_pos, lay.topk_w, out_dtype=moe.MOE_OUT_F32)
        torch.cuda.synchronize()
        assert_close(y.cpu().numpy(), ref["y_pairs"], "y_pairs sequential")
        assert_close(o.cpu().numpy(), ref["o"], "out sequential")


# (config, T, whether the three-call composition runs the same decode kernel
# arithmetic, so that y_pairs and out must agree bit for bit)
LAYER_ENTRY_CASES = [
    (synth.CONFIGS[1], 16, True),
    (synth.CONFIGS[1], 1, False),
    (synth.CONFIGS[1], 4, False),
    (custom_cfg(20, 256, 8, 2, 256), 16, False),            # up to 16 pairs per expert
    (custom_cfg(21, 384, 20, 3, 640, bias_sigma=1.0), 13, False),  # G = 3, ragged
    (synth.CONFIGS[1], 17, True),                            # composition path
]


@pytest.mark.parametrize("case", range(len(LAYER_ENTRY_CASES)))
def test_layer_entry_matches_composition(case):
    """moe_layer_forward_wq equals moe_route_permute -> moe_expert_ffn_wq ->
    moe_combine: routing outputs bit for bit, y_pairs / out within the
    oracle's bar (bit for bit where the same kernels run)."""
    cfg, T, same_kernels = LAYER_ENTRY_CASES[case]
    note(f"layer entry {cfg.name} d={cfg.d} E={cfg.E} k={cfg.k} f={cfg.f} T={T}")
    dl, hl = DevLayer(cfg, T), HostLayer(cfg, T)
    lay = dl.layer()
    outs = []
    for fwd in (lay.forward, lay.forward_steps):
        o = fwd(dl.x, out_dtype=moe.MOE_OUT_F32).clone()
        torch.cuda.synchronize()
        outs.append(dict(o=o, y=lay.y_pairs.clone(), idx=lay.topk_idx.clone(),
                         w=lay.topk_w.clone(), off=lay.offsets.clone(),
                         sp=lay.sorted_pair.clone(), pp=lay.pair_pos.clone()))
        lay.y_pairs.fill_(float("nan"))
        lay.offsets.fill_(-1)
        lay.sorted_pair.fill_(-1)
        lay.pair_pos.fill_(-1)
    a, b = outs
    for key in ("idx", "w", "off", "sp", "pp"):
        assert torch.equal(a[key], b[key]), key
    ref = oracle.layer(hl.x, hl.wr, hl.bias, cfg.k, cfg.f, hl.expert, cfg.fmt,
                       moe.MOE_BITS_NONE, None)
    assert np.array_equal(a["off"].cpu().numpy(), ref["expert_offsets"])
    assert np.array_equal(a["sp"].cpu().numpy(), ref["sorted_pair"])
    assert_close(a["y"].cpu().numpy(), ref["y_pairs"], "y_pairs layer entry")
    assert_close(a["o"].cpu().numpy(), ref["o"], "out layer entry")
    if same_kernels:
        assert torch.equal(a["y"], b["y"])
        assert torch.equal(a["o"], b["o"])


def test_layer_graph_replay_matches_eager():
    """Graph-replayed steps equal eager steps bit for bit, replay after
    replay, with eager work and synchronizations between the replays."""
    note("layer cfg1 T=16 graph replay")
    cfg = synth.CONFIGS[1]
    dl_a, dl_b = DevLayer(cfg, 16, step=0), DevLayer(cfg, 16, step=1)
    lay = dl_a.layer()
    out_g = torch.empty((16, cfg.d), dtype=torch.bfloat16, device=DEV)
    g = lay.capture(dl_a.x, out_g)
    torch.cuda.synchronize()
    ref_a = lay.forward(dl_a.x, out_dtype=moe.MOE_OUT_BF16).clone()
    torch.cuda.synchronize()
    for rep in range(4):
        out_g.fill_(0)
        eager_b = lay.forward(dl_b.x, out_dtype=moe.MOE_OUT_BF16).clone()  # eager work between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref_a), f"replay {rep}"
        assert not torch.equal(eager_b, ref_a)
    del g  # the eager result itself is checked against the oracle elsewhere


def test_layer_cfg3_bitplane_rank_rule():
    note("layer cfg3 T=16 bitplane rank rule")
    cfg = synth.CONFIGS[3]
    check_layer(DevLayer(cfg, 16), HostLayer(cfg, 16), moe.MOE_PATH_AUTO,
                moe.MOE_BITS_RANK_RULE)


@pytest.mark.parametrize("mode", ["pair", "expert"])
def test_layer_bitplane_bit_modes(mode):
    cfg = custom_cfg(13, d=256, E=6, k=4, f=256, fmt="bp8", bias_sigma=0.5)
    T = 40
    rng = np.random.default_rng(11)
    if mode == "pair":
        bits, bm = rng.integers(1, 9, T * cfg.k).astype(np.uint8), moe.MOE_BITS_PER_PAIR
    else:
        bits, bm = np.array([1, 8, 3, 5, 2, 7], np.uint8), moe.MOE_BITS_PER_EXPERT
    for path in PATHS:
        note(f"layer bitplane bits={mode} path={path}")
        check_layer(DevLayer(cfg, T), HostLayer(cfg, T), path, bm, bits)


@pytest.mark.parametrize("mode", ["pair", "expert"])
def test_layer_bitplane_single_slice_ragged(mode):
    # the bitplane decode kernels with one K slice per wave: group counts 3
    # (gate/up) and 13 (down) that are not multiples of the plane prefetch
    # depth, experts spanning several tiles, every bit-width 1..8 in a tile
    cfg = custom_cfg(15, d=384, E=128, k=4, f=1664, fmt="bp8", bias_sigma=2.0)
    T = 32
    rng = np.random.default_rng(12)
    if mode == "pair":
        bits, bm = rng.integers(1, 9, T * cfg.k).astype(np.uint8), moe.MOE_BITS_PER_PAIR
    else:
        bits, bm = rng.integers(1, 9, cfg.E).astype(np.uint8), moe.MOE_BITS_PER_EXPERT
    note(f"layer bitplane single-slice T={T} bits={mode}")
    lay, _ = check_layer(DevLayer(cfg, T), HostLayer(cfg, T), moe.MOE_PATH_DECODE, bm, bits)
    cnt = np.diff(lay.offsets.cpu().numpy())
    assert cnt.max() > 16


@pytest.mark.parametrize("mode", ["pair", "expert", "rank"])
def test_layer_bitplane_prefill_width_tiles(mode):
    # the bitplane prefill kernels: an expert's pairs regrouped by width,
    # several 128-pair tiles per (expert, width) with ragged tails, widths
    # 1..8 (one and two 4-bit passes), f not a power of two
    cfg = custom_cfg(17, d=256, E=4, k=2, f=384, fmt="bp8", bias_sigma=0.3)
    rng = np.random.default_rng(17)
    if mode == "pair":
        T = 2048
        bits, bm = rng.integers(1, 9, T * cfg.k).astype(np.uint8), moe.MOE_BITS_PER_PAIR
    elif mode == "expert":
        T = 700
        bits, bm = np.array([8, 5, 4, 1], np.uint8), moe.MOE_BITS_PER_EXPERT
    else:  # the rank rule is defined for k = 8
        cfg = custom_cfg(18, d=256, E=10, k=8, f=384, fmt="bp8", bias_sigma=0.3)
        T, bits, bm = 400, None, moe.MOE_BITS_RANK_RULE
    note(f"layer bitplane prefill T={T} bits={mode}")
    hl = HostLayer(cfg, T)
    lay, _ = check_layer(DevLayer(cfg, T), hl, moe.MOE_PATH_PREFILL, bm, bits)
    _, ridx, _ = oracle.route(hl.x, hl.wr, hl.bias, cfg.k)
    pb = oracle.pair_bits(ridx, cfg.E, bm, bits)
    off = lay.offsets.cpu().numpy()
    sp = lay.sorted_pair.cpu().numpy()
    per = [np.bincount(pb[sp[off[e]:off[e + 1]]], minlength=9) for e in range(cfg.E)]
    assert max(int(c.max()) for c in per) > 128  # some (expert, width) spans 2+ tiles


def test_layer_zero_tokens():
    cfg = synth.CONFIGS[0]
    dl = DevLayer(cfg, 0)
    lay = dl.layer()
    out = lay.forward(dl.x, out_dtype=moe.MOE_OUT_F32)
    torch.cuda.synchronize()
    assert out.shape == (0, cfg.d)
    assert np.array_equal(lay.offsets.cpu().numpy(), np.zeros(cfg.E + 1, np.int32))


def test_layer_deterministic():
    cfg = synth.CONFIGS[1]
    dl = DevLayer(cfg, 16)
    lay = dl.layer()
    a = lay.forward(dl.x, out_dtype=moe.MOE_OUT_F32).clone()
    ya = lay.y_pairs.clone()
    b = lay.forward(dl.x, out_dtype=moe.MOE_OUT_F32).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(ya.view(torch.int32), lay.y_pairs.view(torch.int32))


# ----------------------------------------- full-size configs, sampled outputs
FULL = [(2, 4096, moe.MOE_PATH_AUTO, moe.MOE_BITS_NONE),
        (3, 4096, moe.MOE_PATH_AUTO, moe.MOE_BITS_RANK_RULE),
        (4, 1, moe.MOE_PATH_AUTO, moe.MOE_BITS_NONE),
        (4, 64, moe.MOE_PATH_AUTO, moe.MOE_BITS_NONE),
        (4, 8192, moe.MOE_PATH_AUTO, moe.MOE_BITS_NONE)]


@pytest.mark.parametrize("cid,T,path,bits_mode", FULL)
def test_layer_full_size_sampled(cid, T, path, bits_mode):
    """Full-size layer in the benchmark's launch configuration: routing and
    grouping bit-exact over every token; codes of every touched expert
    bit-exact; outputs of sampled tokens against the oracle."""
    cfg = synth.CONFIGS[cid]
    note(f"full-size cfg{cid} T={T} bits_mode={bits_mode}: device setup")
    dl = DevLayer(cfg, T)
    hl = HostLayer(cfg, T)
    lay, o32, o16 = run_layer(dl, path, bits_mode)
    note("  routing + grouping vs oracle")
    _, ridx, rw = oracle.route(hl.x, hl.wr, hl.bias, cfg.k)
    idx = lay.topk_idx.cpu().numpy()
    assert np.array_equal(idx, ridx)
    np.testing.assert_allclose(lay.topk_w.cpu().numpy(), rw, rtol=2e-6, atol=1e-7)
    roff, rsp, rpp = oracle.permute(ridx, cfg.E)
    assert np.array_equal(lay.offsets.cpu().numpy(), roff)
    assert np.array_equal(lay.sorted_pair.cpu().numpy(), rsp)
    assert np.array_equal(lay.pair_pos.cpu().numpy(), rpp)
    cnt = np.diff(roff)
    hot = int(np.argmax(cnt))
    toks = sorted({0, T - 1, T // 2, int(rsp[roff[hot]]) // cfg.k})[:4]
    note(f"  sampled tokens {toks} (hottest expert {hot} has {cnt[hot]} pairs)")
    y = lay.y_pairs.cpu().numpy()
    pb = oracle.pair_bits(ridx, cfg.E, bits_mode) if cfg.fmt == "bp8" else None
    for t in toks:
        experts = ridx[t]
        assert_codes_equal(dl, hl, experts)
        o = np.zeros(cfg.d)
        for j, e in enumerate(experts):
            (gq, gs), (dq, ds) = hl.expert(int(e))
            if pb is None:
                wg, wd = oracle.dequant_w4(gq, gs), oracle.dequant_w4(dq, ds)
            else:
                b = int(pb[t * cfg.k + j])
                wg, wd = oracle.dequant_bp(gq, gs, b), oracle.dequant_bp(dq, ds, b)
            _, yy = oracle.expert_ffn(hl.x[t:t + 1], wg, wd)
            assert_close(y[rpp[t * cfg.k + j]], yy[0], f"y t={t} e={e}")
            o += rw[t, j] * yy[0]
        assert_close(o32[t], o, f"out t={t}")
        assert np.array_equal(o16[t], bf16_rne_bits(o32[t]))
    if T <= 64:
        # every pair and every token, the oracle dequantizing each expert once
        note(f"  all {T} tokens: {int((cnt > 0).sum())} experts")
        yref = np.zeros_like(y, dtype=np.float64)
        for e in np.nonzero(cnt)[0]:
            slots = np.arange(roff[e], roff[e + 1])
            bits = None if pb is None else pb[rsp[slots]]
            yref[slots] = hl.y_rows(e, rsp[slots] // cfg.k, bits)
        assert_close(y, yref, "y_pairs all pairs")
        oref = np.einsum("tj,tjd->td", rw, yref[rpp.reshape(T, cfg.k)])
        assert_close(o32, oref, "out all tokens")
        assert np.array_equal(o16, bf16_rne_bits(o32))
    elif pb is None:
        # whole 128-pair tiles of the prefill grouping: the hottest expert's
        # first and last tile, and the last (ragged) tile of 8 more experts
        # spread over the expert range
        tile = 128
        ragged = [e for e in np.nonzero(cnt % tile)[0] if e != hot]
        pick = [ragged[i] for i in np.linspace(0, len(ragged) - 1, 8).astype(int)]
        cases = [(hot, 0), (hot, (cnt[hot] - 1) // tile)] + [
            (e, (cnt[e] - 1) // tile) for e in pick]
        for e, c in cases:
            lo = roff[e] + tile * c
            hi = min(lo + tile, roff[e + 1])
            slots = np.arange(lo, hi)
            note(f"  expert {e} tile {c}: slots {lo}..{hi - 1}")
            assert_close(y[slots], hl.y_rows(e, rsp[slots] // cfg.k),
                         f"y tile e={e} c={c} ({hi - lo} pairs)")


# ------------------------------------------------------ read-budget allocator
def _host_bp_expert(hl, e):
    """The oracle's bitplane matrices (planes, scales) of expert e."""
    (gp, gs), (dp, ds) = hl.expert(e)
    return gp, gs, dp, ds


@pytest.mark.parametrize("cid", [13, 3])
def test_bp_distortion_bit_exact(cid):
    """The distortion table equals the oracle's bit for bit (same fp64 order)."""
    cfg = (custom_cfg(13, d=256, E=6, k=4, f=256, fmt="bp8", bias_sigma=0.5) if cid == 13
           else synth.CONFIGS[3])
    note(f"bp distortion {cfg.name}")
    dl, hl = DevLayer(cfg, 1), HostLayer(cfg, 1)
    dist = moe.moe_bp_distortion(dl.guc, dl.gus, dl.dnc, dl.dns, cfg.d, cfg.f)
    torch.cuda.synchronize()
    got = dist.cpu().numpy()
    for e in ([0, cfg.E // 2, cfg.E - 1] if cfg.E > 8 else range(cfg.E)):
        ref = oracle.bp_distortion(*_host_bp_expert(hl, e), cfg.d, cfg.f)
        assert np.array_equal(got[e], ref), e


def test_allocate_bits_bit_exact():
    """Bits, multiplier and read equal the oracle's, over budgets from
    infeasible to unconstrained, with zero counts and narrowed ranges."""
    rng = np.random.default_rng(11)
    d, f = 2048, 1024
    for E in (1, 7, 64, 300):
        base = rng.uniform(0.5, 2.0, (E, 1)) * 4.0 ** (8 - np.arange(1, 9))[None, :]
        dist = np.sort(base * rng.uniform(0.7, 1.3, (E, 8)), axis=1)[:, ::-1].copy()
        dist[:, 7] = 0.0
        counts = rng.integers(0, 40, E).astype(np.int32)
        dd, cd = torch.from_numpy(dist).to(DEV), torch.from_numpy(counts).to(DEV)
        tot = int(counts.sum())
        for bmin, bmax in ((1, 8), (2, 6)):
            R = [oracle.bp_read_bytes(d, f, b) for b in (bmin, bmax)]
            for budget in (tot * R[0] - 1, tot * R[0], (tot * (R[0] + R[1])) // 2,
                           int(0.8 * tot * R[1]), tot * R[1]):
                note(f"allocate E={E} b=[{bmin},{bmax}] budget={budget}")
                bits, lam, read = moe.moe_allocate_bits(dd, cd, d, f, bmin, bmax, budget)
                torch.cuda.synchronize()
                rb, rl, rr = oracle.allocate_bits(dist, counts, d, f, bmin, bmax, budget)
                assert np.array_equal(bits.cpu().numpy(), rb)
                gl = float(lam.cpu()[0])
                assert gl == rl or (np.isinf(gl) and np.isinf(rl))
                assert int(read.cpu()[0]) == rr


def test_layer_with_allocated_bits():
    """Distortion and allocation on the GPU from the routing counts of a
    profiling batch, then a decode step at those per-expert widths, against
    the oracle's layer at the same widths."""
    cfg = synth.CONFIGS[3]
    note("layer with allocated bits cfg3")
    prof = DevLayer(cfg, 64, step=7)
    lay = prof.layer(moe.MOE_BITS_RANK_RULE)
    lay.forward(prof.x)
    counts = torch.diff(lay.offsets).to(torch.int32)
    dist = moe.moe_bp_distortion(prof.guc, prof.gus, prof.dnc, prof.dns, cfg.d, cfg.f)
    # halfway between 4 and 5 bits per weight on average: the synthetic experts
    # have similar distortion curves, so they split between widths 4 and 5 by
    # their marginal gain
    tot = int(counts.sum().item())
    budget = tot * (oracle.bp_read_bytes(cfg.d, cfg.f, 4) + oracle.bp_read_bytes(cfg.d, cfg.f, 5)) // 2
    bits, lam, read = moe.moe_allocate_bits(dist, counts, cfg.d, cfg.f, 2, 8, budget)
    torch.cuda.synchronize()
    assert int(read.cpu()[0]) <= budget
    b_np = bits.cpu().numpy()
    assert set(b_np.tolist()) == {4, 5}
    dl, hl = DevLayer(cfg, 16), HostLayer(cfg, 16)
    check_layer(dl, hl, moe.MOE_PATH_AUTO, moe.MOE_BITS_PER_EXPERT, b_np)

