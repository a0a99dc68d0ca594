"""The allocation-free layer entry (moe_layer_forward_wq_noalloc, for callers
that cannot allocate device memory) against moe_layer_forward_wq with a
caller workspace, through the C ABI: two calls in a row on one stream, the
second with a smaller batch (the fixed scratch then holds the first call's
contents), every output compared bit for bit."""
import numpy as np
import pytest
import torch

import synth
import quantized_mixture_experts_fp32_amd as moe
from layer_data import DEV, DevLayer, custom_cfg

pytestmark = pytest.mark.gpu

OUTS = ("topk_idx", "topk_w", "offsets", "sorted_pair", "pair_pos", "y_pairs")


def _noalloc_step(lay, x, out_dtype, path):
    """The same step through the allocation-free entry, into fresh buffers."""
    T, k, E, d = x.shape[0], lay.k, lay.E, lay.d
    P = T * k
    b = dict(topk_idx=torch.full((T, k), -1, dtype=torch.int32, device=DEV),
             topk_w=torch.full((T, k), float("nan"), device=DEV),
             offsets=torch.full((E + 1,), -1, dtype=torch.int32, device=DEV),
             sorted_pair=torch.full((P,), -1, dtype=torch.int32, device=DEV),
             pair_pos=torch.full((P,), -1, dtype=torch.int32, device=DEV),
             y_pairs=torch.full((P, d), float("nan"), device=DEV))
    out = torch.full((T, d), float("nan"), device=DEV,
                     dtype=torch.float32 if out_dtype == moe.MOE_OUT_F32 else torch.bfloat16)
    moe.moe_layer_forward_noalloc(x, lay.wr, lay.bias, k, lay.f, lay.gu, lay.gus, lay.dn,
                                  lay.dns, b["topk_idx"], b["topk_w"], b["offsets"],
                                  b["sorted_pair"], b["pair_pos"], b["y_pairs"], out,
                                  lay.fmt, lay.bits, lay.bits_mode, out_dtype, path)
    return b, out


def _bits_equal(a, b):
    if a.dtype.is_floating_point:
        a = a.view(torch.int32) if a.element_size() == 4 else a.view(torch.int16)
        b = b.view(torch.int32) if b.element_size() == 4 else b.view(torch.int16)
    return torch.equal(a, b)


# (name, config, batch sizes in call order, path, bits mode)
CASES = [
    ("OLMoE-shaped decode (expert-major)", synth.CONFIGS[1], (16, 4), moe.MOE_PATH_AUTO,
     moe.MOE_BITS_NONE),
    ("E = 256 layer decode", synth.CONFIGS[4], (64, 1), moe.MOE_PATH_AUTO, moe.MOE_BITS_NONE),
    ("bitplane rank rule", synth.CONFIGS[3], (16, 8), moe.MOE_PATH_AUTO,
     moe.MOE_BITS_RANK_RULE),
    ("small prefill then decode", custom_cfg(80, d=256, E=8, k=2, f=512, bias_sigma=1.0),
     (600, 16), moe.MOE_PATH_AUTO, moe.MOE_BITS_NONE),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_matches_workspace_entry(case):
    name, cfg, batches, path, bm = CASES[case]
    dl = DevLayer(cfg, max(batches))
    lay = dl.layer(bm)
    for i, T in enumerate(batches):
        print(f"no-alloc {name}: call {i + 1}, T={T}", flush=True)
        x = DevLayer.x_only(cfg, T, step=10 + i)
        for out_dtype in (moe.MOE_OUT_F32, moe.MOE_OUT_BF16):
            ref_out = lay.forward(x, out_dtype=out_dtype, path=path).clone()
            ref = {n: getattr(lay, n).clone() for n in OUTS}
            got, out = _noalloc_step(lay, x, out_dtype, path)
            torch.cuda.synchronize()
            for n in OUTS:
                assert _bits_equal(got[n], ref[n]), (name, T, n)
            assert _bits_equal(out, ref_out), (name, T, "out")
            assert np.isfinite(out.float().cpu().numpy()).all()


def test_noalloc_rejects_oversize_step():
    """A step whose workspace exceeds the fixed scratch is refused before
    anything is enqueued (the OLMoE-shaped 4096-token prefill needs 67 MiB)."""
    cfg = synth.CONFIGS[2]
    T, k, E, d, f = 4096, cfg.k, cfg.E, cfg.d, cfg.f
    assert moe.moe_layer_ws_bytes(T, k, E, d, f, moe.MOE_FMT_W4_SYM) > \
        moe.MOE_NOALLOC_SCRATCH_BYTES
    with pytest.raises(moe.MoeError, match="MOE_ERR_WORKSPACE"):
        moe.moe_layer_forward_noalloc(
            torch.empty((T, d), dtype=torch.int16, device=DEV),
            torch.empty((E, d), dtype=torch.int16, device=DEV), None, k, f,
            *(torch.empty(16, dtype=torch.uint8, device=DEV) for _ in range(4)),
            *(torch.empty(16, dtype=torch.int32, device=DEV) for _ in range(5)),
            torch.empty(16, device=DEV), torch.empty(16, device=DEV))
