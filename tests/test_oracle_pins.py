"""Pins of the CPU oracle against facts that do not come from the oracle.

Every oracle function is checked here against something independent of its
own code: hand-derived worked examples (tests/golden), numpy's own IEEE
conversions, brute-force sorts and nearest-code searches, closed forms and
invariants.  A plausible mistake (dropped term, wrong sign, wrong index,
transposed operand, wrong rounding) fails at least one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_to_bf16_bits(a):
    """Exact for values representable in bf16 (used to build inputs)."""
    a = np.asarray(a, np.float32)
    bits = a.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "value not representable in bf16"
    return (bits >> 16).astype(np.uint16)


def bf16_bits_to_f64(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32).astype(np.float64)


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ------------------------------------------------------------ rounding pins
def test_f16_rounding_matches_numpy(rng):
    # numpy's double -> half conversion is an independent IEEE RNE routine
    vals = np.concatenate([
        rng.normal(0, 1, 4000), rng.normal(0, 1e-5, 2000),  # subnormal range
        rng.uniform(60000, 70000, 500),                      # overflow edge
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 2.0**-24, 2.0**-25,
                  3 * 2.0**-26, 1.0 + 2.0**-11, 1.0 + 3 * 2.0**-11]),
    ])
    for v in vals:
        got = oracle.f64_to_f16(v)
        want = int(np.array([v], np.float64).astype(np.float16).view(np.uint16)[0])
        assert got == want, (v, hex(got), hex(want))
        if (want & 0x7C00) != 0x7C00:
            assert oracle.f16_to_f64(want) == float(np.uint16(want).view(np.float16))


def _bf16_nearest_exact(v):
    """Brute force: nearest bf16 to v (ties to even) by exact rationals."""
    f = np.float32(v)
    b = int(np.array([f], np.float32).view(np.uint32)[0] >> 16)
    cands = {(b + dlt) & 0xFFFF for dlt in (-2, -1, 0, 1, 2)}
    best = None
    for c in cands:
        cv = float(bf16_bits_to_f64(np.array([c], np.uint16))[0])
        if not math.isfinite(cv):
            continue
        dist = abs(Fraction(cv) - Fraction(v))
        key = (dist, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_bf16_rounding_exact(rng):
    vals = np.concatenate([rng.normal(0, 3, 3000),
                           (rng.integers(-2**20, 2**20, 500) + 0.5) / 2**12])
    for v in vals:
        assert oracle.f64_to_bf16(v) == _bf16_nearest_exact(float(v)), v
    # ties: 1 + 2^-8 is halfway between 1 and 1+2^-7 -> even (1.0)
    assert oracle.f64_to_bf16(1.0 + 2.0**-8) == 0x3F80
    assert oracle.f64_to_bf16(1.0 + 3 * 2.0**-8) == 0x3F82


# --------------------------------------------------------------- router pins
def test_router_fixed_order_worked_examples():
    for name, d, big, want, *ones in read_golden("router_order.txt"):
        d, big, want = int(d), int(big), int(want)
        x = np.full((1, d), 0x3F80, np.uint16)             # 1.0
        if ones:                                           # sparse weights
            w = np.zeros((1, d), np.uint16)
            w[0, [int(i) for i in ones]] = 0x3F80
        else:
            w = np.full((1, d), 0x3F80, np.uint16)
        w[0, big] = f32_to_bf16_bits([2.0**24])[0]
        got = oracle.router_logits(x, w, None)[0, 0]
        assert got == np.float32(want), (name, got, want)


def test_router_within_higham_bound(rng):
    T, d, E = 6, 512, 16
    x = f32_to_bf16_bits(np.round(rng.normal(0, 1, (T, d)) * 64) / 64)
    w = f32_to_bf16_bits(np.round(rng.normal(0, 1, (E, d)) * 64) / 64)
    bias = rng.normal(0, 1, E).astype(np.float32)
    lg = oracle.router_logits(x, w, bias)
    xf, wf = bf16_bits_to_f64(x), bf16_bits_to_f64(w)
    exact = xf @ wf.T                       # exact: 13-bit products, small sums
    absum = np.abs(xf) @ np.abs(wf).T
    n = d // 16 + 4                         # longest chain of fp32 additions
    u = 2.0**-24
    gamma = n * u / (1 - n * u)
    nobias = oracle.router_logits(x, w, None)
    assert np.all(np.abs(nobias - exact) <= gamma * absum + 1e-30)
    # the bias enters as one fp32 addition after the sum
    assert np.array_equal(lg, (nobias + bias[None, :]).astype(np.float32))


def test_router_integer_inputs_exact(rng):
    # small-integer inputs: every partial sum is an exact fp32 integer
    T, d, E = 3, 384, 5
    xi = rng.integers(-3, 4, (T, d))
    wi = rng.integers(-3, 4, (E, d))
    lg = oracle.router_logits(f32_to_bf16_bits(xi), f32_to_bf16_bits(wi), None)
    assert np.array_equal(lg.astype(np.int64), xi @ wi.T)


# ----------------------------------------------------------------- top-k pins
def test_topk_brute_force_sort(rng):
    T, E, k = 200, 37, 6
    logits = (rng.integers(-8, 8, (T, E)) / 4).astype(np.float32)  # many ties
    idx, w = oracle.topk(logits, k)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))
        assert np.array_equal(idx[t], order[:k])
        sel = logits[t, order[:k]].astype(np.float64)
        ref = np.exp(sel - sel.max())
        ref /= ref.sum()                       # softmax over the selected only
        np.testing.assert_allclose(w[t], ref, rtol=1e-14, atol=0)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-14)


def test_topk_special_cases():
    idx, w = oracle.topk(np.zeros((2, 8), np.float32), 3)
    assert np.array_equal(idx, [[0, 1, 2]] * 2)
    assert np.all(w == 1.0 / 3.0) or np.allclose(w, 1 / 3, rtol=1e-15)
    # two experts, k = 2: weights are the logistic of the logit difference
    lg = np.array([[0.5, -1.25]], np.float32)
    idx, w = oracle.topk(lg, 2)
    assert list(idx[0]) == [0, 1]
    assert math.isclose(w[0, 0], 1 / (1 + math.exp(-1.75)), rel_tol=1e-14)
    # k = E returns every expert
    idx, _ = oracle.topk(np.array([[3, 1, 2, 3]], np.float32), 4)
    assert list(idx[0]) == [0, 3, 2, 1]


def test_route_zero_router_orders_by_bias():
    d, E = 256, 9
    x = np.full((1, d), 0x3F80, np.uint16)
    wr = np.zeros((E, d), np.uint16)
    bias = np.array([0.1, 0.9, -1, 0.5, 0.9, 0.2, 3, -2, 0.0], np.float32)
    _, idx, _ = oracle.route(x, wr, bias, 4)
    assert list(idx[0]) == [6, 1, 4, 3]


# --------------------------------------------------------------- permute pins
def test_permute_stable_sort(rng):
    for T, k, E in [(50, 4, 7), (1, 8, 64), (33, 2, 3), (0, 8, 16)]:
        idx = rng.integers(0, E, (T, k)).astype(np.int32)
        off, sp, pp = oracle.permute(idx, E)
        flat = idx.reshape(-1)
        assert np.array_equal(sp, np.argsort(flat, kind="stable"))
        cnt = np.bincount(flat, minlength=E)
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(cnt)]))
        assert np.array_equal(pp[sp], np.arange(T * k))   # inverse permutation
    idx = np.full((10, 3), 5, np.int32)                     # all on one expert
    off, sp, pp = oracle.permute(idx, 6)
    assert list(off) == [0, 0, 0, 0, 0, 0, 30] and np.array_equal(sp, np.arange(30))


# -------------------------------------------------------------- quantize pins
def _unpack_w4(codes):
    lo = (codes & 0xF).astype(np.int64)
    hi = (codes >> 4).astype(np.int64)
    q = np.stack([lo, hi], -1).reshape(codes.shape[0], -1)
    return np.where(q >= 8, q - 16, q)


def test_w4_worked_example():
    rows = {(r[0], r[1]): r[2:] for r in read_golden("quant_worked.txt")}
    s16 = int(rows[("int4", "scale_f16")][0], 16)
    s = oracle.f16_to_f64(s16)
    w = np.zeros((1, 128), np.float32)
    w[0, :6] = np.array([float(v) for v in rows[("int4", "w_over_s")]]) * s
    codes, scales = oracle.quantize_w4(w)
    assert scales[0, 0] == s16
    assert list(_unpack_w4(codes)[0, :6]) == [int(v) for v in rows[("int4", "q")]]
    assert list(codes[0, :3]) == [int(v, 16) for v in rows[("int4", "bytes")]]


def test_w4_nearest_code_brute_force(rng):
    R, K = 24, 512
    w = (rng.normal(0, 0.14, (R, K)) * np.where(rng.random((R, K)) < 0.01, 10, 1)
         ).astype(np.float32)
    w[3, 128:256] = 0.0                                   # an all-zero group
    codes, scales = oracle.quantize_w4(w)
    q = _unpack_w4(codes)
    s = scales.astype(np.uint16).view(np.float16).astype(np.float64)
    amax = np.abs(w.reshape(R, -1, 128)).max(-1).astype(np.float64)
    assert np.array_equal(scales, (amax / 7).astype(np.float16).view(np.uint16))
    assert np.all(s[3, 1] == 0) and np.all(q[3, 128:256] == 0)
    sfull = np.repeat(s, 128, axis=1)
    cand = np.arange(-7, 8)
    for r in range(R):
        for i in range(K):
            if sfull[r, i] == 0:
                continue
            dist = [abs(Fraction(float(w[r, i])) - Fraction(float(sfull[r, i])) * c)
                    for c in cand]
            m = min(dist)
            best = [c for c, dd in zip(cand, dist) if dd == m]
            want = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
            assert q[r, i] == want, (r, i)
    # round trip within s/2 unless clamped, group max maps to +-7
    ok = np.abs(w / np.where(sfull == 0, 1, sfull)) <= 7.5
    assert np.all(np.abs(w - sfull * q)[ok] <= sfull[ok] / 2)
    gmax = np.abs(w.reshape(R, -1, 128)).argmax(-1)
    for r in range(R):
        for g in range(K // 128):
            if s[r, g] > 0:
                assert abs(q[r, 128 * g + gmax[r, g]]) == 7


def test_w4_dequant_is_s_times_q(rng):
    w = rng.normal(0, 0.1, (8, 256)).astype(np.float32)
    codes, scales = oracle.quantize_w4(w)
    deq = oracle.dequant_w4(codes, scales)
    s = np.repeat(scales.view(np.float16).astype(np.float64), 128, axis=1)
    assert np.array_equal(deq, s * _unpack_w4(codes))


def _planes_to_u(planes):
    """Independent reassembly of u from the plane slabs (numpy unpackbits)."""
    P, R, K8 = planes.shape
    bits = np.unpackbits(planes, axis=-1, bitorder="little").astype(np.int64)
    return sum(bits[p] << (7 - p) for p in range(8))       # [R][K]


def test_bitplane_worked_example():
    rows = read_golden("quant_worked.txt")
    u = int([r for r in rows if r[:2] == ["bp", "u"]][0][2])
    s = 2.0**-7                        # max|w| = 127 * 2^-7 -> s exact in fp16
    w = np.zeros((1, 128), np.float32)
    w[0, 0] = (u - 128) * s
    w[0, 1] = 127 * s
    planes, scales = oracle.quantize_bp8(w)
    assert oracle.f16_to_f64(int(scales[0, 0])) == s
    assert _planes_to_u(planes)[0, 0] == u
    for r in rows:
        if r[:2] == ["bp", "v"]:
            b, v = int(r[2]), int(r[3])
            assert oracle.dequant_bp(planes, scales, b)[0, 0] == v * s, b


def test_bitplane_tie_worked_example():
    """Exact half quotients round to the even code (round-half-even, as the
    quantizer of the tiny int4 workload; PagedMoE's 8-bit code)."""
    rows = {(r[0], r[1]): r[2:] for r in read_golden("quant_worked.txt")}
    s16 = int(rows[("bp", "tie_scale_f16")][0], 16)
    s = oracle.f16_to_f64(s16)
    assert s == 2.0**-7
    ws = [float(v) for v in rows[("bp", "tie_w_over_s")]]
    w = np.zeros((1, 128), np.float32)
    w[0, :len(ws)] = np.array(ws) * s
    planes, scales = oracle.quantize_bp8(w)
    assert scales[0, 0] == s16
    assert list(_planes_to_u(planes)[0, :len(ws)]) == [
        int(v) for v in rows[("bp", "tie_u")]]


def test_bitplane_nearest_code_brute_force(rng):
    """Every stored code is the nearest of all 256 codes u to w (distance
    |w - s(u - 128)| in exact rationals), ties to the even code; a quarter of
    the inputs are placed on exact half steps."""
    R, K = 8, 256
    w = rng.normal(0, 0.14, (R, K)).astype(np.float32)
    # exact halves: the group's max is 127 * 2^-6 (s = 2^-6) and the rest are
    # (n + 1/2) * 2^-6 for random n, all exactly representable in fp32
    for r in range(0, R, 2):
        n = rng.integers(-126, 126, 128)
        w[r, :128] = ((n + 0.5) * 2.0**-6).astype(np.float32)
        w[r, 0] = np.float32(127 * 2.0**-6)
    planes, scales = oracle.quantize_bp8(w)
    u = _planes_to_u(planes)
    s = np.repeat(scales.view(np.float16).astype(np.float64), 128, axis=1)
    codes = np.arange(256)
    ties = 0
    for r in range(R):
        for i in range(K):
            fw, fs = Fraction(float(w[r, i])), Fraction(float(s[r, i]))
            dist = [abs(fw - fs * (c - 128)) for c in codes]
            m = min(dist)
            best = [c for c, dd in zip(codes, dist) if dd == m]
            ties += len(best) > 1
            want = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
            assert u[r, i] == want, (r, i, float(w[r, i] / s[r, i]))
    assert ties >= 4 * 127


def test_bitplane_prefix_properties(rng):
    R, K = 16, 256
    w = rng.normal(0, 0.14, (R, K)).astype(np.float32)
    w[5, :128] = 0
    planes, scales = oracle.quantize_bp8(w)
    u = _planes_to_u(planes)
    s = np.repeat(scales.view(np.float16).astype(np.float64), 128, axis=1)
    amax = np.abs(w.reshape(R, -1, 128)).max(-1).astype(np.float64)
    assert np.array_equal(scales, (amax / 127).astype(np.float16).view(np.uint16))
    assert np.all(u[5, :128] == 128)
    # the 8-plane prefix dequantizes exactly like the plain 8-bit code
    assert np.array_equal(oracle.dequant_bp(planes, scales, 8), s * (u - 128))
    assert np.all(np.abs(w - s * (u - 128)) <= s / 2 + 0.0)
    for b in range(1, 8):
        deq = oracle.dequant_bp(planes, scales, b)
        # only the top b slabs are read
        cut = planes.copy()
        cut[b:] = rng.integers(0, 256, cut[b:].shape, dtype=np.uint8)
        assert np.array_equal(oracle.dequant_bp(cut, scales, b), deq)
        # floor-and-compensation: midpoint of the dropped range
        ub = (u >> (8 - b)) << (8 - b)
        assert np.array_equal(deq, s * (ub + 2 ** (7 - b) - 128))
        assert np.all(np.abs(w - deq) <= s * (2 ** (7 - b) + 0.5))


# ---------------------------------------------------- read-budget allocator
def _bp_expert(rng, d, f):
    gu = rng.normal(0, 0.14, (2 * f, d)).astype(np.float32)
    dn = rng.normal(0, 0.14, (d, f)).astype(np.float32)
    return oracle.quantize_bp8(gu) + oracle.quantize_bp8(dn)


def test_bp_distortion_is_prefix_error_energy(rng):
    """D(b) equals the summed squared difference between the b-bit and the
    8-bit dequantized weights (brute force through dequant_bp, another sum
    order), and D(8) = 0."""
    d, f = 256, 128
    gp, gs, dp, ds = _bp_expert(rng, d, f)
    dist = oracle.bp_distortion(gp, gs, dp, ds, d, f)
    assert dist[7] == 0.0
    for b in range(1, 8):
        ref = 0.0
        for planes, scales in ((gp, gs), (dp, ds)):
            diff = oracle.dequant_bp(planes, scales, b) - oracle.dequant_bp(planes, scales, 8)
            ref += float(np.sum(diff * diff))
        assert abs(dist[b - 1] - ref) <= 1e-12 * ref, b
    assert np.all(np.diff(dist) < 0)  # each extra plane halves the step


def test_bp_distortion_closed_form_zero_codes():
    """All codes u = 0: every element's prefix error is 2^(7-b), so
    D(b) = sum over groups of s^2 * 128 * 4^(7-b), exactly."""
    d, f = 128, 128
    gp = np.zeros((8, 2 * f, d // 8), np.uint8)
    dp = np.zeros((8, d, f // 8), np.uint8)
    gs = np.full((2 * f, 1), oracle.f64_to_f16(0.5), np.uint16)
    ds = np.full((d, 1), oracle.f64_to_f16(0.25), np.uint16)
    dist = oracle.bp_distortion(gp, gs, dp, ds, d, f)
    for b in range(1, 9):
        e = 4.0 ** (7 - b) if b < 8 else 0.0
        assert dist[b - 1] == 128 * e * (2 * f * 0.25 + d * 0.0625), b


def _rand_dist(rng, E):
    # decreasing in b, roughly halving per plane, with per-expert spread
    base = rng.uniform(0.5, 2.0, (E, 1)) * 4.0 ** (8 - np.arange(1, 9))[None, :]
    dist = base * rng.uniform(0.7, 1.3, (E, 8))
    dist[:, 7] = 0.0
    return np.sort(dist, axis=1)[:, ::-1].copy()


def test_allocate_bits_is_budget_optimal_brute_force(rng):
    """Everett: the Lagrangian choice is optimal for its own read level; no
    assignment reading no more has a lower routing-weighted distortion
    (exhaustive over 3 experts x widths 1..8)."""
    import itertools
    d, f, E = 128, 128, 3
    R = np.array([oracle.bp_read_bytes(d, f, b) for b in range(1, 9)], np.int64)
    for trial in range(6):
        dist = _rand_dist(rng, E)
        counts = rng.integers(0, 5, E).astype(np.int32)
        counts[0] = max(counts[0], 1)
        full = int(np.sum(counts * R[7]))
        budget = int(rng.uniform(0.3, 1.0) * full)
        bits, lam, read = oracle.allocate_bits(dist, counts, d, f, 1, 8, budget)
        assert read == int(np.sum(counts * R[bits.astype(int) - 1]))
        if read <= budget:
            obj = float(np.sum(counts * dist[np.arange(E), bits.astype(int) - 1]))
            for a in itertools.product(range(8), repeat=E):
                a = np.array(a)
                if np.sum(counts * R[a]) <= read:
                    assert np.sum(counts * dist[np.arange(E), a]) >= obj * (1 - 1e-12), (trial, a)
        else:
            assert np.all(bits == 1)


def test_allocate_bits_budget_extremes(rng):
    d, f, E = 256, 256, 5
    dist = _rand_dist(rng, E)
    counts = np.array([3, 0, 1, 7, 2], np.int32)
    R = [oracle.bp_read_bytes(d, f, b) for b in range(1, 9)]
    hi = int(np.sum(counts)) * R[6]
    bits, lam, read = oracle.allocate_bits(dist, counts, d, f, 2, 7, hi)
    assert np.all(bits == 7) and lam == 0.0 and read == hi
    lo = int(np.sum(counts)) * R[1]
    bits, lam, read = oracle.allocate_bits(dist, counts, d, f, 2, 7, lo)
    assert np.all(bits == 2) and read == lo
    bits, lam, read = oracle.allocate_bits(dist, counts, d, f, 2, 7, lo - 1)
    assert np.all(bits == 2) and math.isinf(lam) and read == lo


def test_allocate_bits_frequency_cancels_and_monotone(rng):
    """Scaling every routing count and the budget by one factor leaves every
    decision unchanged (the frequency cancels from the per-expert choice),
    and a larger budget never narrows any expert."""
    d, f, E = 256, 128, 16
    dist = _rand_dist(rng, E)
    counts = rng.integers(1, 9, E).astype(np.int32)
    R8 = oracle.bp_read_bytes(d, f, 8)
    prev = None
    for frac in np.linspace(0.3, 1.0, 8):
        budget = int(frac * int(np.sum(counts)) * R8)
        bits, _, _ = oracle.allocate_bits(dist, counts, d, f, 1, 8, budget)
        bits3, _, _ = oracle.allocate_bits(dist, 3 * counts, d, f, 1, 8, 3 * budget)
        assert np.array_equal(bits, bits3)
        if prev is not None:
            assert np.all(bits >= prev)
        prev = bits


def test_pair_bits_modes():
    idx = np.tile(np.arange(8, dtype=np.int32), (3, 1))
    pb = oracle.pair_bits(idx, 8, oracle.BITS_RANK_RULE)
    assert list(pb[:8]) == [8, 4, 4, 4, 2, 2, 2, 2] and list(pb[8:16]) == list(pb[:8])
    per_e = np.arange(1, 9, dtype=np.uint8)
    pb = oracle.pair_bits(idx[:, ::-1].copy(), 8, oracle.BITS_PER_EXPERT, per_e)
    assert list(pb[:8]) == [8, 7, 6, 5, 4, 3, 2, 1]
    with pytest.raises(ValueError):
        oracle.pair_bits(idx[:, :4].copy(), 8, oracle.BITS_RANK_RULE)


# ------------------------------------------------------------------ FFN pins
def test_ffn_zero_gate_gives_zero():
    d, f = 128, 128
    x = f32_to_bf16_bits(np.linspace(-2, 2, 2 * d).reshape(2, d).astype(np.float32)
                         .round(2).astype(np.float32).view(np.uint32)
                         .__and__(0xFFFF0000).view(np.float32))
    wgu = np.zeros((2 * f, d))
    wgu[f:] = 0.5
    h, y = oracle.expert_ffn(x, wgu, np.ones((d, f)))
    assert np.all(h == 0) and np.all(y == 0)


def test_ffn_closed_form_large_gate(rng):
    # x = e_0, gate column 0 = 128 -> g = 128 and silu(g) = 128 in fp64;
    # up column 0 = small integers u -> h = 128 u exactly (bf16-representable)
    d, f = 256, 128
    x = np.zeros((1, d), np.uint16)
    x[0, 0] = 0x3F80
    wgu = rng.normal(0, 1, (2 * f, d))
    wgu[:f, 0] = 128.0
    ui = rng.integers(-3, 4, f)
    wgu[f:, 0] = ui
    wd = rng.integers(-5, 6, (d, f)).astype(np.float64)
    h, y = oracle.expert_ffn(x, wgu, wd)
    assert np.array_equal(h[0], 128.0 * ui)
    assert np.array_equal(y[0], wd.astype(np.int64) @ (128 * ui))
    # gate and up swapped gives something else (gate rows come first)
    h2, _ = oracle.expert_ffn(x, np.concatenate([wgu[f:], wgu[:f]]), wd)
    assert not np.array_equal(h2, h)
    # silu(-128) * u is far below bf16 resolution of the sums -> ~0
    wgu[:f, 0] = -128.0
    h3, _ = oracle.expert_ffn(x, wgu, wd)
    assert np.all(np.abs(h3) < 1e-50)


def test_ffn_silu_moderate_gates():
    """h = bf16(silu(g) u) with silu(g) = g / (1 + e^-g) at gates where the
    SiLU is far from its asymptotes, computed here with Python's math.exp and
    rounded to bf16 by an exact-rational nearest search."""
    d, f = 128, 128
    gates = [0.5, -0.5, 1.0, -1.0, 2.0, -2.0, 4.0, -4.0]
    ups = [1.0, 3.0, -2.0, 0.75, 5.0, -1.5, 0.25, 7.0]
    x = np.zeros((1, d), np.uint16)
    x[0, 0] = 0x3F80                                # x = e_0 (bf16 1.0)
    wgu = np.zeros((2 * f, d))
    wgu[:f, 0] = np.resize(gates, f)
    wgu[f:, 0] = np.resize(ups, f)
    wd = np.zeros((d, f))
    wd[np.arange(d), np.arange(f) % f] = 1.0        # y_m = h_m
    wd[1, :] = 0.0
    wd[1, 0], wd[1, 2] = 2.0, -1.0                  # y_1 = 2 h_0 - h_2
    h, y = oracle.expert_ffn(x, wgu, wd)
    for n in range(f):
        g, uu = wgu[n, 0], wgu[f + n, 0]
        silu = g / (1.0 + math.exp(-g))
        want = float(bf16_bits_to_f64(np.array([_bf16_nearest_exact(silu * uu)],
                                               np.uint16))[0])
        assert h[0, n] == want, (g, uu, h[0, n], want)
    assert y[0, 0] == h[0, 0] and y[0, 5] == h[0, 5]
    assert y[0, 1] == 2 * h[0, 0] - h[0, 2]


def test_ffn_h_is_bf16_and_scales_exactly(rng):
    d, f = 256, 256
    x = f32_to_bf16_bits((rng.normal(0, 1, (3, d)) * 16).round() / 16)
    wgu = rng.normal(0, 0.1, (2 * f, d))
    wd = rng.normal(0, 0.1, (d, f))
    h, y = oracle.expert_ffn(x, wgu, wd)
    hb = np.array([oracle.f64_to_bf16(v) for v in h.reshape(-1)], np.uint16)
    assert np.array_equal(bf16_bits_to_f64(hb).reshape(h.shape), h)
    # doubling the up rows doubles h exactly (power-of-two scaling commutes
    # with rounding) and hence y
    w2 = wgu.copy()
    w2[f:] *= 2
    h2, y2 = oracle.expert_ffn(x, w2, wd)
    assert np.array_equal(h2, 2 * h)
    np.testing.assert_allclose(y2, 2 * y, rtol=1e-13, atol=1e-12)


# -------------------------------------------------------------- layer pins
def _tiny_layer(rng, T=9, d=256, E=6, k=3, f=128, fmt="w4"):
    x = f32_to_bf16_bits((rng.normal(0, 1, (T, d)) * 32).round() / 32)
    wr = f32_to_bf16_bits((rng.normal(0, 1 / 16, (E, d)) * 256).round() / 256)
    bias = rng.normal(0, 1, E).astype(np.float32)
    wts = {}
    for e in range(E):
        gu = rng.normal(0, 0.14, (2 * f, d)).astype(np.float32)
        dn = rng.normal(0, 0.14, (d, f)).astype(np.float32)
        q = oracle.quantize_w4 if fmt == "w4" else oracle.quantize_bp8
        wts[e] = (q(gu), q(dn))
    return x, wr, bias, wts


def test_layer_equals_dense_all_expert_sum(rng):
    """No expert is pruned or substituted: the sparse grouped layer equals a
    dense sum over all experts with zero gate weight for unselected ones."""
    x, wr, bias, wts = _tiny_layer(rng)
    T, d = x.shape
    E, k, f = wr.shape[0], 3, 128
    res = oracle.layer(x, wr, bias, k, f, wts.__getitem__)
    assert np.array_equal(np.sort(res["sorted_pair"]), np.arange(T * k))
    G = np.zeros((T, E))
    for t in range(T):
        G[t, res["topk_idx"][t]] = res["topk_w"][t]
    dense = np.zeros((T, d))
    for e in range(E):
        (gq, gs), (dq, ds) = wts[e]
        _, ye = oracle.expert_ffn(x, oracle.dequant_w4(gq, gs), oracle.dequant_w4(dq, ds))
        dense += G[:, e:e + 1] * ye
    np.testing.assert_allclose(res["o"], dense, rtol=1e-12, atol=1e-12)
    ob = np.array([oracle.f64_to_bf16(v) for v in res["o"].reshape(-1)], np.uint16)
    assert np.array_equal(ob.reshape(T, d), res["out"])


def test_layer_bitplane_rank_rule_dense_sum(rng):
    x, wr, bias, wts = _tiny_layer(rng, T=5, E=10, k=8, fmt="bp8")
    T, d = x.shape
    E, k, f = 10, 8, 128
    res = oracle.layer(x, wr, bias, k, f, wts.__getitem__, fmt="bp8",
                       bits_mode=oracle.BITS_RANK_RULE)
    dense = np.zeros((T, d))
    rank_bits = [8, 4, 4, 4, 2, 2, 2, 2]
    for t in range(T):
        for j in range(k):
            e = res["topk_idx"][t, j]
            (gq, gs), (dq, ds) = wts[e]
            b = rank_bits[j]
            _, ye = oracle.expert_ffn(x[t:t + 1], oracle.dequant_bp(gq, gs, b),
                                      oracle.dequant_bp(dq, ds, b))
            dense[t] += res["topk_w"][t, j] * ye[0]
    np.testing.assert_allclose(res["o"], dense, rtol=1e-12, atol=1e-12)


def test_combine_single_rank_identity(rng):
    y = rng.normal(0, 1, (4, 8))
    o, _ = oracle.combine(y, np.array([2, 0, 3, 1], np.int32), np.ones((4, 1)))
    assert np.array_equal(o, y[[2, 0, 3, 1]])


# -------------------------------------------------------------- input pins
def test_synth_distribution_and_determinism():
    key = synth.stream_key(1, synth.T_X)
    z = synth.std_normal(key, 0, 400_000)
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1) < 0.01
    assert z.min() >= -6 and z.max() <= 6
    assert np.array_equal(z[1000:2000], synth.std_normal(key, 1000, 1000))
    c = synth.CONFIGS[1]
    assert np.array_equal(synth.host_x(c, 16)[:1], synth.host_x(c, 1))
    m = synth.host_outlier_mask(c, synth.T_W_GATE_UP, 0, 2_000_000)
    assert 0.0008 < m.mean() < 0.0012
    w = synth.host_weight_rows(c, synth.T_W_GATE_UP, 0, 0, 4)
    assert abs(np.std(w) - math.sqrt(0.02)) < 0.03
