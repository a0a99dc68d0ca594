"""GPU tests of the HBM expert slot cache (moe_cache_forward): a layer step
with the expert bank in pinned host memory and S device slots, over several
steps with fresh tokens (hits, LRU replacement, bitplanes added to resident
experts, steps routed to more experts than there are slots).  Every step is
checked against the CPU oracle to the same bar as the resident layer."""
import numpy as np
import pytest
import torch

import oracle
import synth
import quantized_mixture_experts_fp32_amd as moe
from layer_data import DEV, DevLayer, HostLayer, assert_close, custom_cfg

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)


def make_cache(dl, slots):
    fmt = moe.MOE_FMT_W4_SYM if dl.cfg.fmt == "w4" else moe.MOE_FMT_BITPLANE8
    return moe.ExpertCache(dl.wr, dl.bias, dl.cfg.k, dl.cfg.f, dl.guc, dl.gus, dl.dnc, dl.dns,
                           fmt, slots)


def check_step(cache, cfg, T, step, bits_mode=moe.MOE_BITS_NONE, bits_np=None, hl_w=None):
    x = DevLayer.x_only(cfg, T, step)
    hl = HostLayer(cfg, T, step=step)
    if hl_w is not None:
        hl._cache = hl_w._cache  # the same experts: reuse the oracle's quantized copies
    bits = None if bits_np is None else torch.from_numpy(bits_np).to(DEV)
    out = cache.forward(x, out_dtype=moe.MOE_OUT_F32, bits=bits, bits_mode=bits_mode)
    torch.cuda.synchronize()
    ref = oracle.layer(hl.x, hl.wr, hl.bias, cfg.k, cfg.f, hl.expert, cfg.fmt, bits_mode,
                       bits_np)
    assert np.array_equal(cache.topk_idx.cpu().numpy(), ref["topk_idx"])
    np.testing.assert_allclose(cache.topk_w.cpu().numpy(), ref["topk_w"], rtol=2e-6, atol=1e-7)
    pp = cache.pair_pos.cpu().numpy()
    y = cache.y_pairs.cpu().numpy()[pp]  # pair order
    assert_close(y, ref["y_pairs"][ref["pair_pos"]], f"cache y step {step}")
    assert_close(out.cpu().numpy(), ref["o"], f"cache out step {step}")
    return hl


@pytest.mark.parametrize("slots", [8, 3])
def test_cache_int4_steps(slots):
    # 8 slots hold every expert (hits after the first steps); 3 slots make
    # each step stream experts through the slot halves
    cfg = custom_cfg(21, d=256, E=8, k=2, f=512, bias_sigma=0.5)
    dl = DevLayer(cfg, 16)
    cache = make_cache(dl, slots)
    hl = None
    for step in range(4):
        note(f"cache int4 slots={slots} step={step}")
        hl = check_step(cache, cfg, 16, step, hl_w=hl)
    st = cache.stats()
    note(f"  stats {st}")
    assert st["steps"] == 4
    if slots == 8:
        assert st["loads_full"] <= 8 and st["hits"] > 0 and st["chunks"] == 4
    else:
        assert st["chunks"] > 4
    cache.close()


def test_cache_few_tokens():
    # one or two tokens per step: the small-batch decode kernels over the
    # slots, with replacements between steps
    cfg = custom_cfg(24, d=256, E=16, k=4, f=256, bias_sigma=0.5)
    dl = DevLayer(cfg, 2)
    cache = make_cache(dl, 6)
    for step, T in enumerate([1, 2, 1, 2, 1]):
        note(f"cache few tokens T={T} step={step}")
        check_step(cache, cfg, T, step)
    st = cache.stats()
    note(f"  stats {st}")
    assert st["steps"] == 5 and st["loads_full"] >= 4
    cache.close()


@pytest.mark.parametrize("slots", [6, 2])
def test_cache_bitplane_widths_grow(slots):
    # per-pair widths drawn per step: resident experts gain missing planes
    cfg = custom_cfg(22, d=256, E=6, k=2, f=256, fmt="bp8", bias_sigma=0.5)
    T = 12
    dl = DevLayer(cfg, T)
    cache = make_cache(dl, slots)
    rng = np.random.default_rng(22)
    hl = None
    for step in range(5):
        hi = 2 + 2 * step if step < 3 else 8
        bits = rng.integers(1, hi + 1, T * cfg.k).astype(np.uint8)
        note(f"cache bitplane slots={slots} step={step} widths<={hi}")
        hl = check_step(cache, cfg, T, step, moe.MOE_BITS_PER_PAIR, bits, hl_w=hl)
    st = cache.stats()
    note(f"  stats {st}")
    if slots == 6:
        assert st["loads_partial"] > 0
    e, b = cache.resident()
    assert ((e >= -1) & (e < cfg.E)).all() and (b <= 8).all()
    cache.close()


def test_cache_per_expert_widths_and_rank_rule():
    cfg = custom_cfg(23, d=256, E=10, k=8, f=256, fmt="bp8", bias_sigma=0.5)
    T = 6
    dl = DevLayer(cfg, T)
    cache = make_cache(dl, 4)
    hl = check_step(cache, cfg, T, 0, moe.MOE_BITS_PER_EXPERT,
                    np.array([1, 8, 3, 5, 2, 7, 4, 6, 8, 1], np.uint8))
    check_step(cache, cfg, T, 1, moe.MOE_BITS_RANK_RULE, None, hl_w=hl)
    cache.close()


@pytest.mark.parametrize("slots", [64, 16])
def test_cache_full_size_decode_matches_resident_layer(slots):
    """cfg1 T=16 (64 experts, top-8) through 64 and 16 slots.  With every
    expert in a slot the step runs the resident layer's kernels on the slots
    and its outputs are bit-identical to the resident layer's; with 16 slots
    the chunked step is checked against the resident layer to the oracle's
    bar (different kernels, same definition)."""
    cfg = synth.CONFIGS[1]
    T = 16
    dl = DevLayer(cfg, T)
    lay = dl.layer()
    cache = make_cache(dl, slots)
    for step in range(3):
        x = DevLayer.x_only(cfg, T, step)
        note(f"cache cfg1 slots={slots} step={step}")
        a = lay.forward(x, out_dtype=moe.MOE_OUT_F32).clone()
        ya = lay.y_pairs[lay.pair_pos.long()].clone()
        b = cache.forward(x, out_dtype=moe.MOE_OUT_F32).clone()
        yb = cache.y_pairs[cache.pair_pos.long()].clone()
        torch.cuda.synchronize()
        assert torch.equal(lay.topk_idx, cache.topk_idx)
        if slots == cfg.E:
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))
            assert torch.equal(ya.view(torch.int32), yb.view(torch.int32))
        else:
            assert_close(yb.cpu().numpy(), ya.cpu().numpy().astype(np.float64),
                         f"cache16 y step {step}")
            assert_close(b.cpu().numpy(), a.cpu().numpy().astype(np.float64),
                         f"cache16 out step {step}")
    st = cache.stats()
    note(f"  stats {st}")
    cache.close()


@pytest.mark.parametrize("fmt", ["w4", "bp8"])
def test_cache_prefill_chunks(fmt):
    # a batch large enough for the prefill kernels, routed to more experts
    # than there are slots: every chunk runs the grouped MFMA path on its
    # slice of the slots
    cfg = custom_cfg(25, d=256, E=8, k=2, f=256, fmt=fmt, bias_sigma=0.5)
    T = 300
    dl = DevLayer(cfg, T)
    cache = make_cache(dl, 4)
    rng = np.random.default_rng(25)
    hl = None
    for step in range(2):
        note(f"cache prefill {fmt} step={step}")
        if fmt == "w4":
            hl = check_step(cache, cfg, T, step, hl_w=hl)
        else:
            bits = rng.integers(1, 9, T * cfg.k).astype(np.uint8)
            hl = check_step(cache, cfg, T, step, moe.MOE_BITS_PER_PAIR, bits, hl_w=hl)
    st = cache.stats()
    note(f"  stats {st}")
    assert st["chunks"] >= 2 * 3  # chunk 0 and at least two streamed chunks per step
    cache.close()


def test_cache_rejects_unpinned_bank():
    cfg = custom_cfg(24, d=256, E=4, k=2, f=256)
    dl = DevLayer(cfg, 1)
    h = ctypes_void()
    rc = moe.load_library().moe_cache_create(
        cfg.E, cfg.d, cfg.f, moe.MOE_FMT_W4_SYM, 2,
        *[moe._ptr(t) for t in (dl.guc, dl.gus, dl.dnc, dl.dns)],  # device, not pinned host
        *[moe._ptr(t) for t in (dl.guc, dl.gus, dl.dnc, dl.dns)], h)
    assert rc == moe.MOE_ERR_INVALID_ARG


def ctypes_void():
    import ctypes
    v = ctypes.c_void_p()
    return ctypes.cast(ctypes.pointer(v), ctypes.c_void_p)
