"""CPU tests of the expert slot cache's slot assignment (moe_cache_plan: the
host policy moe_cache_forward applies each step, no device work): resident
experts are hits, new ones take empty slots then the least recently used,
bitplane experts grow by their missing planes only, and steps with more
experts than slots stream through the two slot halves."""
import numpy as np
import pytest

import quantized_mixture_experts_fp32_amd as moe

W4, BP = moe.MOE_FMT_W4_SYM, moe.MOE_FMT_BITPLANE8


class Slots:
    def __init__(self, S):
        self.e = np.full(S, -1, np.int32)
        self.b = np.zeros(S, np.int32)
        self.last = np.full(S, -1, np.int64)
        self.S = S

    def plan(self, E, fmt, step, need):
        return moe.moe_cache_plan(E, self.S, fmt, self.e, self.b, self.last, step, need)


def need_of(E, experts, width=8):
    n = np.zeros(E, np.int32)
    for e in experts:
        n[e] = width
    return n


def test_fresh_cache_with_a_streaming_chunk():
    s = Slots(4)
    p = s.plan(8, W4, 0, need_of(8, [0, 2, 3, 6, 7]))
    assert p["V"] == 5
    assert p["vmap"].tolist() == [0, -1, 1, 2, -1, -1, 3, 4]
    assert p["chunks"].tolist() == [[0, 4, 0, -1], [4, 1, 0, 0]]
    assert p["loads"].tolist() == [[0, 0, 0, 8, 0, 1], [2, 1, 0, 8, 0, 1], [3, 2, 0, 8, 0, 1],
                                   [6, 3, 0, 8, 0, 1], [7, 0, 0, 8, 1, 1]]
    assert s.e.tolist() == [7, 2, 3, 6]


def test_resident_experts_are_hits():
    s = Slots(4)
    s.plan(8, W4, 0, need_of(8, [0, 1, 2, 3]))
    p = s.plan(8, W4, 1, need_of(8, [2, 3]))
    assert len(p["loads"]) == 0
    assert p["vmap"][2] == 2 and p["vmap"][3] == 3
    assert s.last.tolist() == [0, 0, 1, 1]


def test_least_recently_used_slot_is_replaced():
    s = Slots(4)
    s.plan(8, W4, 0, need_of(8, [0, 1, 2, 3]))
    s.plan(8, W4, 1, need_of(8, [0, 1]))
    p = s.plan(8, W4, 2, need_of(8, [0, 4]))
    # experts 2 and 3 were last used at step 0; the lower slot goes first
    assert p["loads"].tolist() == [[4, 2, 0, 8, 0, 1]]
    assert s.e.tolist() == [0, 1, 4, 3]
    p = s.plan(8, W4, 3, need_of(8, [5]))
    assert p["loads"][0, 1] == 3  # expert 3's slot (step 0) before 1 (step 1)


def test_empty_slots_fill_before_eviction():
    s = Slots(4)
    s.plan(8, W4, 0, need_of(8, [5]))
    s.plan(8, W4, 1, need_of(8, [6]))
    assert s.e.tolist() == [5, 6, -1, -1]


def test_bitplane_prefix_grows_by_missing_planes():
    s = Slots(2)
    n = np.zeros(4, np.int32)
    n[1] = 2
    p = s.plan(4, BP, 0, n)
    assert p["loads"].tolist() == [[1, 0, 0, 2, 0, 1]]
    n[1] = 4
    p = s.plan(4, BP, 1, n)
    assert p["loads"].tolist() == [[1, 0, 2, 4, 0, 0]]  # planes 2, 3 only, no scales
    n[1] = 3
    p = s.plan(4, BP, 2, n)
    assert len(p["loads"]) == 0 and s.b[0] == 4
    n[1] = 8
    p = s.plan(4, BP, 3, n)
    assert p["loads"].tolist() == [[1, 0, 4, 8, 0, 0]]


def test_all_experts_stream_through_slot_halves():
    s = Slots(4)
    p = s.plan(16, W4, 0, need_of(16, range(16)))
    assert p["V"] == 16
    ch = p["chunks"].tolist()
    assert ch[0] == [0, 4, 0, -1]
    assert ch[1:] == [[4, 2, 0, 0], [6, 2, 2, 0], [8, 2, 0, 1], [10, 2, 2, 2], [12, 2, 0, 3],
                      [14, 2, 2, 4]]
    assert sorted(p["vmap"].tolist()) == list(range(16))


def replay_and_check(E, S, fmt, state_before, need, p):
    """Apply the loads chunk by chunk to a copy of the slot contents and check
    that every routed expert sits in its slot, with enough planes, when its
    chunk's FFN runs."""
    se, sb = state_before[0].copy(), state_before[1].copy()
    vmap, chunks, loads = p["vmap"], p["chunks"], p["loads"]
    routed = np.nonzero(need > 0)[0]
    assert (vmap[need == 0] == -1).all()
    assert len(set(vmap[routed].tolist())) == len(routed)
    assert (vmap[routed] >= 0).all() and (vmap[routed] < p["V"]).all()
    H = S // 2
    for c, (v0, n, slot0, wait) in enumerate(chunks):
        if c == 0:
            assert (v0, n, slot0, wait) == (0, S, 0, -1)
        else:
            assert slot0 == ((c - 1) % 2) * H and 1 <= n <= H
            assert wait == (c - 2 if c >= 3 else 0)
        for e, slot, p0, p1, lc, sc in loads:
            if lc != c:
                continue
            assert slot0 <= slot < slot0 + n or c == 0
            if sc:  # a new expert in the slot: whole prefix
                assert p0 == 0
            else:  # a longer prefix of the resident expert
                assert se[slot] == e and sb[slot] == p0 and fmt == BP
            se[slot], sb[slot] = e, p1
        for e in routed:
            v = vmap[e]
            if v0 <= v < v0 + n:
                slot = slot0 + (v - v0)
                assert se[slot] == e
                assert sb[slot] >= (8 if fmt == W4 else need[e])
    return se, sb


@pytest.mark.parametrize("fmt", [W4, BP])
@pytest.mark.parametrize("S", [2, 5, 8])
def test_random_steps_keep_every_routed_expert_resident_for_its_chunk(fmt, S):
    E = 12
    rng = np.random.default_rng(S * 10 + fmt)
    s = Slots(S)
    for step in range(40):
        k = int(rng.integers(1, E + 1))
        experts = rng.choice(E, k, replace=False)
        need = np.zeros(E, np.int32)
        need[experts] = rng.integers(1, 9, k) if fmt == BP else 8
        before = (s.e.copy(), s.b.copy())
        was = {int(e): int(b) for e, b in zip(*before) if e >= 0}
        p = s.plan(E, fmt, step, need)
        se, sb = replay_and_check(E, S, fmt, before, need, p)
        assert s.e.tolist() == se.tolist() and s.b.tolist() == sb.tolist()
        # whole loads only for experts not resident before the step; a
        # resident expert with enough planes is never copied again
        for e, slot, p0, p1, c, sc in p["loads"]:
            if sc:
                assert int(e) not in was
        for e in experts:
            if was.get(int(e), 0) >= need[e]:
                assert not any(ld[0] == e for ld in p["loads"])


def test_plan_rejects_bad_state():
    s = Slots(2)
    s.e[:] = [1, 1]
    with pytest.raises(moe.MoeError):
        s.plan(4, W4, 0, need_of(4, [0]))
    with pytest.raises(moe.MoeError):
        moe.moe_cache_plan(4, 8, W4, np.full(8, -1, np.int32), np.zeros(8, np.int32),
                           np.zeros(8, np.int64), 0, need_of(4, [0]))
