"""GPU parity of the whole layer on inputs that exercise the degenerate cases
of every FFN kernel: all-zero weight groups (scale 0) at the start, in the
middle and over a whole expert, on each decode and prefill path; layers
with one, two or three experts at batch sizes from 2 to 1000; the
interface's largest d, E, k and a wide f; and one-token layers on the
K-split gate/up that streams its codes through LDS, including a token whose
top-k ids repeat an expert.  Every case
goes through the C ABI and is compared with the CPU oracle as in the other
layer tests (integers bit-exact, floating point within rel-L2 2e-3 and
max-abs 3e-2 rms)."""
import numpy as np
import pytest
import torch

import synth
import quantized_mixture_experts_fp32_amd as moe
import oracle
from layer_data import DEV, DevLayer, HostLayer, assert_close, custom_cfg
from test_gpu_parity import check_layer, note

pytestmark = pytest.mark.gpu

GU, DN = synth.T_W_GATE_UP, synth.T_W_DOWN


def zero_spec(d, f):
    """Zeroed weight blocks (tensor, expert, rows, input columns):
    expert 0: the first 128-group of every row of all three matrices (the
      leading group of a row has scale 0);
    expert 1: the second 128-group of every row (a middle group when the
      input dimension is at least 384);
    expert 2: every weight (the expert's output is exactly 0);
    expert 3: the first group of gate/up rows 16..47 (two whole 16-row tiles
      of the gate matrix) and all of down rows 0..15."""
    return [(GU, 0, 0, 2 * f, 0, 128), (DN, 0, 0, d, 0, 128),
            (GU, 1, 0, 2 * f, 128, 256), (DN, 1, 0, d, 128, 256),
            (GU, 2, 0, 2 * f, 0, d), (DN, 2, 0, d, 0, f),
            (GU, 3, 16, 48, 0, 128), (DN, 3, 0, 16, 0, f)]


# (name, format, d, E, k, f, T, path, bits mode)
ZERO_CASES = [
    ("expert-major decode", "w4", 384, 16, 4, 384, 16, moe.MOE_PATH_AUTO, None),
    ("K-split decode", "w4", 384, 16, 4, 384, 1, moe.MOE_PATH_AUTO, None),
    ("single-slice decode", "w4", 384, 128, 4, 1664, 32, moe.MOE_PATH_DECODE, None),
    ("int4 prefill", "w4", 384, 16, 4, 384, 300, moe.MOE_PATH_PREFILL, None),
    ("bitplane single-slice decode", "bp8", 384, 128, 4, 1664, 32, moe.MOE_PATH_DECODE,
     "pair"),
    ("bitplane decode, few experts", "bp8", 384, 16, 4, 384, 1, moe.MOE_PATH_DECODE, "pair"),
    ("bitplane prefill", "bp8", 384, 16, 4, 384, 300, moe.MOE_PATH_PREFILL, "pair"),
    ("bitplane prefill, rank rule", "bp8", 384, 16, 8, 384, 300, moe.MOE_PATH_PREFILL,
     "rank"),
    ("one-token K-split decode, LDS-streamed codes", "w4", 1024, 16, 6, 384, 1,
     moe.MOE_PATH_AUTO, None),
]


@pytest.mark.parametrize("case", range(len(ZERO_CASES)))
def test_layer_zero_weight_groups(case):
    name, fmt, d, E, k, f, T, path, mode = ZERO_CASES[case]
    note(f"zero weight groups: {name} d={d} E={E} k={k} f={f} T={T}")
    cfg = custom_cfg(40 + case, d=d, E=E, k=k, f=f, fmt=fmt, bias_sigma=1.0)
    zero = zero_spec(d, f)
    dl, hl = DevLayer(cfg, T, zero=zero), HostLayer(cfg, T, zero=zero)
    # experts 0..3 get a logit bias of +4 so that nearly every token picks
    # them; the others keep a small random bias
    bias = (np.random.default_rng(case).normal(0, 0.3, E)).astype(np.float32)
    bias[:4] += 4.0
    hl.bias = bias
    dl.bias = torch.from_numpy(bias).to(DEV)
    bm, bits = moe.MOE_BITS_NONE, None
    if mode == "pair":
        bm = moe.MOE_BITS_PER_PAIR
        bits = np.random.default_rng(100 + case).integers(1, 9, T * k).astype(np.uint8)
    elif mode == "rank":
        bm = moe.MOE_BITS_RANK_RULE
    lay, _ = check_layer(dl, hl, path, bm, bits)
    off = lay.offsets.cpu().numpy()
    cnt = np.diff(off)
    assert (cnt[:4] > 0).all(), cnt[:4]
    # the all-zero expert's rows are exactly zero
    y = lay.y_pairs.cpu().numpy()
    assert np.all(y[off[2]:off[3]] == 0.0)
    # the zeroed groups really have scale 0 in the packed layer
    gus = dl.gus.cpu().numpy().view(np.uint16)
    assert np.all(gus[0][:, 0] == 0) and np.all(gus[1][:, 1] == 0) and np.all(gus[2] == 0)
    # a weight whose scale is 0 is 0 whatever its code: random codes in the
    # zero-scale groups of experts 0 and 1 leave every output bit unchanged
    y0 = lay.y_pairs.clone()
    o0 = lay.forward(dl.x, out_dtype=moe.MOE_OUT_F32, path=path).clone()
    gen = torch.Generator(device="cpu").manual_seed(case)
    blk = 1024 if fmt == "w4" else 2048            # bytes per 16-row tile and group
    for codes, rows, K in ((dl.guc, 2 * f, d), (dl.dnc, d, f)):
        for e, g in ((0, 0), (1, 1)):
            v = codes[e].view(-1).view(rows // 16, K // 128, blk)
            v[:, g, :] = torch.randint(0, 256, (rows // 16, blk), generator=gen,
                                       dtype=torch.uint8).to(DEV)
    o1 = lay.forward(dl.x, out_dtype=moe.MOE_OUT_F32, path=path).clone()
    torch.cuda.synchronize()
    assert torch.equal(lay.y_pairs, y0), "codes under a zero scale changed y_pairs"
    assert torch.equal(o1, o0)


# (E, k) x T: layers with very few experts, every path
SMALL_E = [(1, 1), (2, 2), (3, 2)]
SMALL_T = [2, 5, 33, 1000]
PATHS3 = [moe.MOE_PATH_AUTO, moe.MOE_PATH_DECODE, moe.MOE_PATH_PREFILL]


@pytest.mark.parametrize("path", PATHS3)
@pytest.mark.parametrize("T", SMALL_T)
@pytest.mark.parametrize("E,k", SMALL_E)
def test_layer_few_experts(E, k, T, path):
    note(f"few experts: E={E} k={k} T={T} path={path}")
    cfg = custom_cfg(60 + E, d=256, E=E, k=k, f=256, bias_sigma=0.5)
    check_layer(DevLayer(cfg, T), HostLayer(cfg, T), path)


@pytest.mark.parametrize("T", [2, 16])
@pytest.mark.parametrize("E,k", [(1, 1), (2, 2), (4, 2)])
def test_layer_entry_fewer_blocks_than_tokens(E, k, T):
    """The layer entry's expert-major decode at f = 128: with E * f / 128
    gate/up blocks below T there is no block per token to select the top-k
    from the logits, so the layer routes first; results as for any layer."""
    note(f"layer entry, E * f / 128 = {E} blocks, T={T}")
    cfg = custom_cfg(70 + E, d=256, E=E, k=k, f=128, bias_sigma=0.5)
    check_layer(DevLayer(cfg, T), HostLayer(cfg, T), moe.MOE_PATH_AUTO)


# (name, format, d, E, k, f, T, bits mode): the interface's largest model
# width (d = 8192), expert count (E = 512) and top-k (k = 16), and a wide
# FFN (f = 8192), through the whole layer on both paths
EXTREME_CASES = [
    ("d=8192", "w4", 8192, 8, 2, 256, 3, None),
    ("E=512, k=16", "w4", 256, 512, 16, 128, 40, None),
    ("f=8192", "w4", 256, 4, 2, 8192, 20, None),
    ("bitplane d=8192, rank rule", "bp8", 8192, 16, 8, 128, 5, "rank"),
]


@pytest.mark.parametrize("path", [moe.MOE_PATH_DECODE, moe.MOE_PATH_PREFILL])
@pytest.mark.parametrize("case", range(len(EXTREME_CASES)))
def test_layer_extreme_shapes(case, path):
    name, fmt, d, E, k, f, T, mode = EXTREME_CASES[case]
    note(f"extreme shape: {name} d={d} E={E} k={k} f={f} T={T} path={path}")
    cfg = custom_cfg(80 + case, d=d, E=E, k=k, f=f, fmt=fmt, bias_sigma=0.5)
    bm = moe.MOE_BITS_RANK_RULE if mode == "rank" else moe.MOE_BITS_NONE
    check_layer(DevLayer(cfg, T), HostLayer(cfg, T), path, bm)


@pytest.mark.parametrize("path", [moe.MOE_PATH_DECODE, moe.MOE_PATH_PREFILL])
def test_bitplane_reads_stay_in_prefix(path):
    """A b-bit read of a bitplane expert touches only the plane pairs that
    hold its top b planes, the first 512 ceil(b / 2) bytes of every 2 KiB
    block (include/moe_wq.h): random bytes written past them, in both
    matrices of every expert, leave every output bit unchanged.  Per-expert
    widths 1..8 cover the odd widths whose last pair is read half."""
    cfg = custom_cfg(19, d=256, E=8, k=2, f=384, fmt="bp8", bias_sigma=0.3)
    T = 40 if path == moe.MOE_PATH_DECODE else 700
    widths = np.array([1, 2, 3, 4, 5, 6, 7, 8], np.uint8)
    dl = DevLayer(cfg, T)
    hl = HostLayer(cfg, T)
    note(f"bitplane prefix reads path={path} T={T}")
    lay, _ = check_layer(dl, hl, path, moe.MOE_BITS_PER_EXPERT, widths)
    assert (np.diff(lay.offsets.cpu().numpy()) > 0).all()
    bits = torch.from_numpy(widths).to(DEV)
    lay = dl.layer(moe.MOE_BITS_PER_EXPERT, bits)
    o0 = lay.forward(dl.x, out_dtype=moe.MOE_OUT_F32, path=path).clone()
    y0 = lay.y_pairs.clone()
    gen = torch.Generator(device="cpu").manual_seed(19)
    for codes, rows, K in ((dl.guc, 2 * cfg.f, cfg.d), (dl.dnc, cfg.d, cfg.f)):
        for e, b in enumerate(widths):
            keep = 512 * ((int(b) + 1) // 2)
            if keep == 2048:
                continue
            v = codes[e].view(-1).view(rows // 16, K // 128, 2048)
            v[:, :, keep:] = torch.randint(0, 256, (rows // 16, K // 128, 2048 - keep),
                                           generator=gen, dtype=torch.uint8).to(DEV)
    o1 = lay.forward(dl.x, out_dtype=moe.MOE_OUT_F32, path=path).clone()
    torch.cuda.synchronize()
    assert torch.equal(lay.y_pairs, y0), "bytes past the prefix pairs changed y_pairs"
    assert torch.equal(o1, o0)


# (d, E, k, f): one-token layers on the K-split gate/up that streams its
# codes through LDS, with K slices of 1, 3, 5, 7 and 8 groups (three slots
# in flight: slices shorter than, equal to and past one round of slots),
# four and two K slices per item, and the routing taken inside the kernel
# (E <= 64) or staged from the routing launch (E > 64); E > 2 k keeps the
# layer entry off the expert-major kernels
ONE_TOKEN = [(512, 8, 2, 256), (1536, 32, 8, 256), (2560, 32, 8, 512), (3584, 32, 8, 512),
             (2048, 32, 8, 4096), (1024, 128, 8, 256)]


@pytest.mark.parametrize("d,E,k,f", ONE_TOKEN)
def test_layer_one_token_ksplit(d, E, k, f):
    note(f"one-token K-split decode d={d} E={E} k={k} f={f}")
    cfg = custom_cfg(90 + ONE_TOKEN.index((d, E, k, f)), d=d, E=E, k=k, f=f,
                     bias_sigma=0.5)
    check_layer(DevLayer(cfg, 1), HostLayer(cfg, 1), moe.MOE_PATH_AUTO)


def test_one_token_repeated_expert_ids():
    """One token whose top-k ids (given by the caller) name an expert three
    times: that expert's tile holds three pairs, which the one-token K-split
    gate/up computes from activations read from global memory instead of its
    staged row; every pair row against the oracle."""
    cfg = custom_cfg(98, d=1024, E=16, k=4, f=384)
    note("one token, repeated expert ids [3, 3, 7, 3]")
    dl, hl = DevLayer(cfg, 1), HostLayer(cfg, 1)
    ids = np.array([[3, 3, 7, 3]], np.int32)
    off, sp, _ = moe.moe_permute(torch.from_numpy(ids).to(DEV), cfg.E)
    y = moe.moe_expert_ffn_wq(dl.x, off, sp, cfg.k, cfg.f, dl.guc, dl.gus, dl.dnc, dl.dns,
                              path=moe.MOE_PATH_DECODE)
    torch.cuda.synchronize()
    roff, rsp, _ = oracle.permute(ids, cfg.E)
    assert np.array_equal(off.cpu().numpy(), roff)
    assert np.array_equal(sp.cpu().numpy(), rsp)
    ref = oracle.expert_outputs(hl.x, ids, roff, rsp, hl.expert, "w4", cfg.f)
    assert_close(y.cpu().numpy(), ref, "y_pairs")
