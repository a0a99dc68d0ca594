"""CPU tests of the C ABI: the library loads, exports every declared symbol,
and rejects invalid arguments before anything is enqueued (no GPU needed:
every call here fails validation, so no HIP call is made)."""
import ctypes
import os
import re

import pytest

import quantized_mixture_experts_fp32_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_wq.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        from quantized_mixture_experts_fp32_amd import build
        build.build()
    return moe.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10
    assert sorted(moe.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert moe.status_str(0) == "MOE_OK"
    assert moe.status_str(3) == "MOE_ERR_WORKSPACE"
    assert moe.status_str(99) == "MOE_ERR_UNKNOWN"


FAKE = ctypes.c_void_p(0x10000)      # 16-byte-aligned non-null pointer
ODD = ctypes.c_void_p(0x10002)       # misaligned
NULL = None


def err(lib):
    return lib.moe_last_error().decode()


def test_route_validation(lib):
    def r(x, w, b, T, d, E, k, i, tw, ws=FAKE, wsb=1 << 20):
        return lib.moe_route(x, w, b, T, d, E, k, i, tw, ws, wsb, NULL)
    assert r(FAKE, FAKE, NULL, 4, 200, 8, 2, FAKE, FAKE) == moe.MOE_ERR_UNSUPPORTED
    assert "128" in err(lib)
    assert r(FAKE, FAKE, NULL, 4, 256, 8, 9, FAKE, FAKE) == moe.MOE_ERR_INVALID_ARG
    assert r(FAKE, FAKE, NULL, 4, 256, 600, 2, FAKE, FAKE) == moe.MOE_ERR_UNSUPPORTED
    assert r(FAKE, FAKE, NULL, 4, 256, 64, 17, FAKE, FAKE) == moe.MOE_ERR_UNSUPPORTED
    assert r(FAKE, FAKE, NULL, 4, 256 * 33, 64, 8, FAKE, FAKE) == moe.MOE_ERR_UNSUPPORTED
    assert r(NULL, FAKE, NULL, 4, 256, 8, 2, FAKE, FAKE) == moe.MOE_ERR_INVALID_ARG
    assert r(ODD, FAKE, NULL, 4, 256, 8, 2, FAKE, FAKE) == moe.MOE_ERR_INVALID_ARG
    assert r(FAKE, FAKE, NULL, -1, 256, 8, 2, FAKE, FAKE) == moe.MOE_ERR_INVALID_ARG
    need = lib.moe_route_ws_bytes(4, 8)
    assert need >= 4 * 8 * 4
    assert r(FAKE, FAKE, NULL, 4, 256, 8, 2, FAKE, FAKE, FAKE, need - 1) == moe.MOE_ERR_WORKSPACE
    assert r(FAKE, FAKE, NULL, 4, 256, 8, 2, FAKE, FAKE, NULL, need) == moe.MOE_ERR_WORKSPACE
    # T = 0 is a valid no-op, even with null pointers
    assert r(NULL, NULL, NULL, 0, 256, 8, 2, NULL, NULL, NULL, 0) == moe.MOE_OK


def test_permute_validation(lib):
    need = lib.moe_permute_ws_bytes(100, 8, 64)
    assert need >= 64 * 4
    p = lib.moe_permute
    assert p(FAKE, 100, 8, 64, FAKE, FAKE, FAKE, FAKE, need - 4, NULL) == moe.MOE_ERR_WORKSPACE
    assert p(FAKE, 100, 8, 64, FAKE, FAKE, FAKE, NULL, need, NULL) == moe.MOE_ERR_WORKSPACE
    assert p(FAKE, 100, 8, 64, NULL, FAKE, FAKE, FAKE, need, NULL) == moe.MOE_ERR_INVALID_ARG
    assert p(FAKE, 100, 9, 8, FAKE, FAKE, FAKE, FAKE, need, NULL) == moe.MOE_ERR_INVALID_ARG


def test_route_permute_validation(lib):
    rp = lib.moe_route_permute
    need = lib.moe_route_permute_ws_bytes(4, 2, 8)
    assert need >= max(lib.moe_route_ws_bytes(4, 8), lib.moe_permute_ws_bytes(4, 2, 8))
    args = lambda **kw: [kw.get("x", FAKE), FAKE, NULL, kw.get("T", 4), kw.get("d", 256), 8,
                         kw.get("k", 2), FAKE, FAKE, kw.get("off", FAKE), FAKE, FAKE,
                         kw.get("ws", FAKE), kw.get("wsb", need), NULL]
    assert rp(*args(d=200)) == moe.MOE_ERR_UNSUPPORTED
    assert rp(*args(k=9)) == moe.MOE_ERR_INVALID_ARG
    assert rp(*args(x=NULL)) == moe.MOE_ERR_INVALID_ARG
    assert rp(*args(off=NULL)) == moe.MOE_ERR_INVALID_ARG
    assert rp(*args(wsb=need - 1)) == moe.MOE_ERR_WORKSPACE
    assert rp(*args(ws=NULL)) == moe.MOE_ERR_WORKSPACE
    assert rp(*args(x=ODD)) == moe.MOE_ERR_INVALID_ARG


def _ffn(lib, **kw):
    a = dict(x=FAKE, off=FAKE, sp=FAKE, T=4, k=2, E=8, d=256, f=512, fmt=0, group=128,
             guc=FAKE, gus=FAKE, dnc=FAKE, dns=FAKE, bits=NULL, mode=0, y=FAKE,
             ws=FAKE, wsb=1 << 30, path=0)
    a.update(kw)
    return lib.moe_expert_ffn_wq(a["x"], a["off"], a["sp"], a["T"], a["k"], a["E"],
                                 a["d"], a["f"], a["fmt"], a["group"], a["guc"],
                                 a["gus"], a["dnc"], a["dns"], a["bits"], a["mode"],
                                 a["y"], a["ws"], a["wsb"], a["path"], NULL)


def test_ffn_validation(lib):
    U, I, W = moe.MOE_ERR_UNSUPPORTED, moe.MOE_ERR_INVALID_ARG, moe.MOE_ERR_WORKSPACE
    assert _ffn(lib, group=64) == U
    assert _ffn(lib, f=500) == U
    assert _ffn(lib, d=200) == U
    assert _ffn(lib, fmt=7) == I
    assert _ffn(lib, path=5) == I
    assert _ffn(lib, mode=1) == I                      # int4 takes no bits
    assert _ffn(lib, fmt=1, mode=0) == I               # bitplane needs a mode
    assert _ffn(lib, fmt=1, mode=1, bits=NULL) == I
    assert _ffn(lib, fmt=1, mode=3, k=2) == U          # rank rule needs k = 8
    assert _ffn(lib, guc=ODD) == I
    assert _ffn(lib, y=NULL) == I
    need = lib.moe_ffn_ws_bytes(4, 2, 8, 256, 512, 0)
    assert _ffn(lib, wsb=need - 1) == W
    assert _ffn(lib, ws=ctypes.c_void_p(0x10010)) == I  # ws needs 256-byte alignment
    assert _ffn(lib, T=0, x=NULL, off=NULL, sp=NULL, y=NULL, ws=NULL, wsb=0) == moe.MOE_OK
    # the prefill kernels' 32-bit row offsets: T * max(d, f) * 2 < 2^32
    big = dict(T=262144, k=1, E=64, d=8192, f=1024, wsb=1 << 62)
    assert _ffn(lib, path=2, **big) == U                       # explicit prefill
    assert _ffn(lib, path=0, **big) == U                       # AUTO picks prefill
    assert "2^32" in err(lib)
    assert _ffn(lib, path=2, **dict(big, d=1024, f=8192)) == U  # down: K = f


def test_combine_and_quantize_validation(lib):
    c = lib.moe_combine
    assert c(FAKE, FAKE, FAKE, 4, 2, 256, FAKE, 5, NULL) == moe.MOE_ERR_INVALID_ARG
    assert c(FAKE, FAKE, FAKE, 4, 17, 256, FAKE, 0, NULL) == moe.MOE_ERR_UNSUPPORTED
    assert c(FAKE, FAKE, FAKE, 4, 2, 256, ODD, 0, NULL) == moe.MOE_ERR_INVALID_ARG
    assert c(NULL, NULL, NULL, 0, 2, 256, NULL, 0, NULL) == moe.MOE_OK
    q = lib.moe_quantize_w4
    assert q(FAKE, 2, 4, 256, 64, FAKE, FAKE, NULL) == moe.MOE_ERR_UNSUPPORTED
    assert q(FAKE, 2, 4, 100, 128, FAKE, FAKE, NULL) == moe.MOE_ERR_UNSUPPORTED
    assert q(FAKE, 2, 4, 256, 128, FAKE, FAKE, NULL) == moe.MOE_ERR_UNSUPPORTED  # rows tiled by 16
    assert lib.moe_quantize_bitplane8(FAKE, 2, 8, 256, 128, FAKE, FAKE, NULL) == moe.MOE_ERR_UNSUPPORTED
    assert "16" in err(lib)
    assert q(NULL, 2, 16, 256, 128, FAKE, FAKE, NULL) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_bitplane8(FAKE, 0, 16, 256, 128, NULL, NULL, NULL) == moe.MOE_OK


def test_allocator_validation(lib):
    ws = lib.moe_bp_distortion_ws_bytes(4, 256, 128)
    assert ws == 8 * 8 * 4 * (2 * 128 + 256)
    dz = lib.moe_bp_distortion
    assert dz(FAKE, FAKE, FAKE, FAKE, 4, 200, 128, FAKE, FAKE, ws, NULL) == moe.MOE_ERR_UNSUPPORTED
    assert dz(FAKE, FAKE, FAKE, FAKE, 0, 256, 128, FAKE, FAKE, ws, NULL) == moe.MOE_ERR_INVALID_ARG
    assert dz(FAKE, FAKE, NULL, FAKE, 4, 256, 128, FAKE, FAKE, ws, NULL) == moe.MOE_ERR_INVALID_ARG
    assert dz(FAKE, FAKE, FAKE, FAKE, 4, 256, 128, FAKE, FAKE, ws - 1, NULL) == moe.MOE_ERR_WORKSPACE
    assert dz(ODD, FAKE, FAKE, FAKE, 4, 256, 128, FAKE, FAKE, ws, NULL) == moe.MOE_ERR_INVALID_ARG
    al = lib.moe_allocate_bits
    assert al(FAKE, FAKE, 4, 256, 128, 0, 8, 10, FAKE, NULL, NULL, NULL) == moe.MOE_ERR_INVALID_ARG
    assert al(FAKE, FAKE, 4, 256, 128, 5, 4, 10, FAKE, NULL, NULL, NULL) == moe.MOE_ERR_INVALID_ARG
    assert al(FAKE, FAKE, 4, 256, 128, 1, 9, 10, FAKE, NULL, NULL, NULL) == moe.MOE_ERR_INVALID_ARG
    assert al(FAKE, FAKE, 513, 256, 128, 1, 8, 10, FAKE, NULL, NULL, NULL) == moe.MOE_ERR_UNSUPPORTED
    assert al(FAKE, NULL, 4, 256, 128, 1, 8, 10, FAKE, NULL, NULL, NULL) == moe.MOE_ERR_INVALID_ARG
    assert al(FAKE, FAKE, 4, 256, 128, 1, 8, 10, FAKE, ODD, NULL, NULL) == moe.MOE_ERR_INVALID_ARG


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(moe, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        moe.load_library()


def test_w4_untile_matches_header_formula():
    """The tests' untiling of int4 codes follows the layout the ABI header
    states: row n, element k lives in the 32-bit word at byte offset
    (((n/16)*(K/128) + k/128)*16 + n%16)*64 + 4*((k%128)/8), in nibble
    e/2 for even e = k%8 and 4 + e/2 for odd e."""
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from layer_data import w4_untile
    import numpy as np
    N, K = 48, 384
    tiled = np.random.default_rng(5).integers(0, 256, N * K // 2, dtype=np.uint8)
    rm = w4_untile(tiled, N, K)
    for n in range(N):
        for k in range(K):
            g, w = divmod(k, 128)
            off = (((n // 16) * (K // 128) + g) * 16 + n % 16) * 64 + 4 * (w // 8)
            word = int.from_bytes(bytes(tiled[off:off + 4]), "little")
            e = k % 8
            nib = e // 2 if e % 2 == 0 else 4 + e // 2
            want = (word >> (4 * nib)) & 0xF
            got = (rm[n, k // 2] >> (4 * (k % 2))) & 0xF
            assert got == want, (n, k)


def test_bp_untile_matches_header_formula():
    """The tests' untiling of bitplanes follows the ABI header: plane p of
    row n, byte j of group g lives at ((n/16)*(K/128) + g)*2048 +
    512 (p/2) + 32 (n%16) + 8 (j/4) + 4 (p%2) + j%4."""
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from layer_data import bp_untile
    import numpy as np
    N, K = 32, 256
    tiled = np.random.default_rng(6).integers(0, 256, N * K, dtype=np.uint8)
    pm = bp_untile(tiled, N, K)
    for p in range(8):
        for n in range(N):
            for jj in range(K // 8):
                g, j = divmod(jj, 16)
                off = (((n // 16) * (K // 128) + g) * 2048 + 512 * (p // 2) + 32 * (n % 16)
                       + 8 * (j // 4) + 4 * (p % 2) + j % 4)
                assert pm[p, n, jj] == tiled[off], (p, n, jj)


def test_noalloc_entry_refuses_oversize_on_host(lib):
    """The allocation-free layer entry refuses a step whose workspace
    exceeds its fixed scratch before touching the device (no GPU here)."""
    T, k, E, d, f = 4096, 8, 64, 2048, 1024
    assert lib.moe_layer_ws_bytes(T, k, E, d, f, 0) > moe.MOE_NOALLOC_SCRATCH_BYTES
    rc = lib.moe_layer_forward_wq_noalloc(FAKE, FAKE, NULL, T, d, E, k, f, 0, 128, FAKE,
                                          FAKE, FAKE, FAKE, NULL, 0, FAKE, FAKE, FAKE,
                                          FAKE, FAKE, FAKE, FAKE, 1, 0, NULL)
    assert rc == moe.MOE_ERR_WORKSPACE
    assert "scratch" in err(lib)


def test_retile_validation(lib):
    """Shape and pointer checks of the canonical-layout conversions (no GPU)."""
    U, I = moe.MOE_ERR_UNSUPPORTED, moe.MOE_ERR_INVALID_ARG
    far = ctypes.c_void_p(0x4000000)
    for fn in (lib.moe_retile_w4, lib.moe_retile_bitplane8):
        assert fn(FAKE, 2, 16, 100, far, NULL) == U      # K not a multiple of 128
        assert fn(FAKE, 2, 24, 256, far, NULL) == U      # N not a multiple of 16
        assert fn(FAKE, -1, 16, 256, far, NULL) == I
        assert fn(NULL, 2, 16, 256, far, NULL) == I
        assert fn(ODD, 2, 16, 256, far, NULL) == I
        assert fn(FAKE, 2, 16, 256, FAKE, NULL) == I     # in place
        assert "overlap" in err(lib)
        assert fn(NULL, 0, 16, 256, NULL, NULL) == moe.MOE_OK
