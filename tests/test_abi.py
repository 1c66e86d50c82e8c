"""CPU-only checks of the C ABI library: it loads, exports every symbol that
include/moe.h declares, and its host-side logic (shape checks, workspace
sizing, status strings, argument errors found before any launch) behaves."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if not h.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^\s*[\w\s\*]+?\b(moe_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def moe():
    import combine_dispatch_amd as m
    if not os.path.exists(m.LIB_PATH):
        from combine_dispatch_amd import build
        build.build()
    m.lib()
    return m


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("moe_fused_forward", "moe_dispatch", "moe_combine", "moe_workspace_bytes",
              "moe_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(moe):
    L = moe.lib()
    for n in _declared_functions():
        assert hasattr(L, n), n
    assert set(moe.EXPORTED) <= set(_declared_functions())


def test_status_strings(moe):
    for st in (0, -1, -2, -3, -4, -5, 17):
        assert isinstance(moe.moe_status_string(st), str) and moe.moe_status_string(st)


def test_default_options(moe):
    o = moe.moe_default_options()
    assert o.fast_math == 1 and o.debug_validate == 0 and o.activation_clamp != o.activation_clamp
    assert o.gemm_tiles == moe.MOE_TILES_AUTO


def test_workspace_sizing(moe):
    T, H, I, E, K = 8192, 7168, 2048, 32, 8
    b = moe.moe_workspace_bytes(T, H, I, E, K)
    cap = T * K + 256
    # token rows e4m3 + scales, act e4m3 + scales, L2 bf16 rows: the bulk of it
    bulk = T * (H + H // 32) + cap * (I + I // 32 + 2 * H)
    assert bulk <= b <= bulk + 64 * 1024 * 1024
    v = moe.moe_workspace_views(T, H, I, E, K)
    assert v["capacity_rows"] == cap
    offs = sorted(v[k] for k in v if k != "capacity_rows")
    assert len(set(offs)) == len(offs) and all(o % 256 == 0 for o in offs)
    assert v["l2_out"] + 2 * H * cap <= b
    assert moe.moe_workspace_bytes(-1, H, I, E, K) == 0
    assert moe.moe_workspace_bytes(T, H, I, 0, K) == 0
    assert moe.moe_workspace_bytes(T, H, I, 2000, K) == 0
    assert moe.moe_workspace_bytes(T, H, I, E, 65) == 0
    assert 0 < moe.moe_dispatch_workspace_bytes(T, H, E, K) < b
    # shapes the fused layer refuses get no workspace size and no views, so a
    # caller cannot size a buffer for a call that would fail
    for bad in ((T, 7168 - 32, I, E, K), (T, H, I - 32, E, K), (1 << 20, 7168, I, E, 1)):
        assert moe.moe_workspace_bytes(*bad) == 0, bad
        with pytest.raises(moe.MoeError):
            moe.moe_workspace_views(*bad)
    # the standalone dispatch still takes any H % 32 == 0
    assert moe.moe_dispatch_workspace_bytes(T, 7168 - 32, E, K) > 0


def test_host_side_errors_need_no_device(moe):
    L = moe.lib()
    s = moe.MoeShape(16, 256, 128, 4, 2)
    null = ctypes.c_void_p(0)
    # T == 0 returns at once, nothing to launch
    assert L.moe_fused_forward(ctypes.byref(moe.MoeShape(0, 256, 128, 4, 2)), None, *[null] * 8,
                               null, 0, null) == moe.MOE_OK
    # null tensors -> invalid argument, found before any launch
    assert L.moe_fused_forward(ctypes.byref(s), None, *[null] * 8, null, 0,
                               null) == moe.MOE_ERR_INVALID_ARG
    # shape outside the tiling
    bad = moe.MoeShape(16, 200, 128, 4, 2)
    assert L.moe_fused_forward(ctypes.byref(bad), None, *[null] * 8, null, 0,
                               null) == moe.MOE_ERR_UNSUPPORTED
    # activation clamp is not implemented
    o = moe.options(activation_clamp=3.0)
    assert L.moe_fused_forward(ctypes.byref(s), ctypes.byref(o), *[null] * 8, null, 0,
                               null) == moe.MOE_ERR_UNSUPPORTED
    # unknown GEMM tiling
    o = moe.options(gemm_tiles=7)
    assert L.moe_fused_forward(ctypes.byref(s), ctypes.byref(o), *[null] * 8, null, 0,
                               null) == moe.MOE_ERR_INVALID_ARG
    # forced tile-per-workgroup GEMMs on a shape whose routing takes two
    # launches (ceil(T*K / 1024) * E > 65536): refused before any launch or
    # dereference (the pointers below are never touched)
    big = moe.MoeShape(8192, 256, 128, 1024, 16)
    fake = ctypes.c_void_p(1 << 20)
    for tiles in (moe.MOE_TILES_64, moe.MOE_TILES_128, moe.MOE_TILES_FUSED):
        o = moe.options(gemm_tiles=tiles)
        assert L.moe_fused_forward(ctypes.byref(big), ctypes.byref(o), *[fake] * 8, fake, 1 << 40,
                                   null) == moe.MOE_ERR_UNSUPPORTED
    # L1 and L2 in one launch keeps a 128 x I activation tile in LDS: I <= 768
    o = moe.options(gemm_tiles=moe.MOE_TILES_FUSED)
    wide = moe.MoeShape(64, 256, 896, 8, 2)
    assert L.moe_fused_forward(ctypes.byref(wide), ctypes.byref(o), *[fake] * 8, fake, 1 << 40,
                               null) == moe.MOE_ERR_UNSUPPORTED
    # unknown payload
    assert L.moe_dispatch(ctypes.byref(s), null, null, null, 7, *[null] * 7, null, 0,
                          null) == moe.MOE_ERR_INVALID_ARG
    # combine with T == 0 is a no-op, with nulls an error
    assert L.moe_combine(ctypes.byref(moe.MoeShape(0, 256, 32, 1, 2)), null, null, null, null,
                         null) == moe.MOE_OK
    assert L.moe_combine(ctypes.byref(s), null, null, null, null, null) == moe.MOE_ERR_INVALID_ARG


def test_prepacked_weight_entry_points_host_side(moe):
    L = moe.lib()
    null = ctypes.c_void_p(0)
    H, I, E = 7168, 2048, 32
    w1, w2 = E * 2 * I * (H // 2), E * H * (I // 2)
    up = lambda n: (n + 255) // 256 * 256
    assert moe.moe_packed_weights_bytes(H, I, E) == up(w1) + up(w2) + moe.moe_packed_scales_bytes(H, I, E)
    assert moe.moe_packed_weights_bytes(200, I, E) == 0
    s = moe.MoeShape(16, 256, 128, 4, 2)
    fake = ctypes.c_void_p(1 << 20)
    # null or misaligned pointers, a short buffer: found before any device call
    assert L.moe_pack_weights(ctypes.byref(s), null, fake, fake, fake, fake, 1 << 30, null) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights(ctypes.byref(s), ctypes.c_void_p((1 << 20) + 8), fake, fake, fake, fake, 1 << 30,
                              null) == moe.MOE_ERR_INVALID_ARG
    need = moe.moe_packed_weights_bytes(256, 128, 4)
    assert L.moe_pack_weights(ctypes.byref(s), fake, fake, fake, fake, fake, need - 1, null) == moe.MOE_ERR_WORKSPACE
    assert L.moe_pack_weights(ctypes.byref(moe.MoeShape(16, 200, 128, 4, 2)), fake, fake, fake, fake, fake,
                              1 << 30, null) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_fused_forward_prepacked(ctypes.byref(s), None, fake, fake, fake, null, fake, fake, 1 << 30,
                                         null) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_fused_forward_prepacked(ctypes.byref(s), None, fake, fake, fake, ctypes.c_void_p((1 << 20) + 16),
                                         fake, fake, 1 << 30, null) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_fused_forward_prepacked(ctypes.byref(moe.MoeShape(16, 200, 128, 4, 2)), None, fake, fake, fake,
                                         fake, fake, fake, 1 << 30, null) == moe.MOE_ERR_UNSUPPORTED


def test_packed_scale_entry_points_host_side(moe):
    L = moe.lib()
    null = ctypes.c_void_p(0)
    H, I, E = 7168, 2048, 32
    # S1's words, then S2's from the next 256-byte boundary: the same bytes as S1, S2
    s1 = E * 2 * I * (H // 32)
    assert moe.moe_packed_scales_bytes(H, I, E) == (s1 + 255) // 256 * 256 + E * H * (I // 32)
    assert moe.moe_packed_scales_bytes(200, I, E) == 0
    s = moe.MoeShape(16, 256, 128, 4, 2)
    assert L.moe_pack_weight_scales(ctypes.byref(s), null, null, null, 0,
                                    null) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weight_scales(ctypes.byref(moe.MoeShape(16, 200, 128, 4, 2)), null, null,
                                    null, 0, null) == moe.MOE_ERR_UNSUPPORTED
    # a missing packed buffer, null tensors -> invalid argument before any launch
    assert L.moe_fused_forward_packed(ctypes.byref(s), None, *[null] * 7, null, 0,
                                      null) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_fused_forward_packed(ctypes.byref(moe.MoeShape(0, 256, 128, 4, 2)), None,
                                      *[null] * 5, ctypes.c_void_p(256), null, null, 0,
                                      null) == moe.MOE_OK


def test_noalloc_entry_host_side(moe):
    """The allocation-free entry refuses shapes whose workspace exceeds its
    device scratch before touching the device, and takes T == 0 as a no-op."""
    L = moe.lib()
    null = ctypes.c_void_p(0)
    one = ctypes.c_void_p(256)
    big = moe.MoeShape(8192, 7168, 2048, 32, 8)
    assert moe.moe_workspace_bytes(8192, 7168, 2048, 32, 8) > moe.MOE_NOALLOC_SCRATCH_BYTES
    assert L.moe_fused_forward_packed_noalloc(ctypes.byref(big), None, *[one] * 6, one,
                                              null) == moe.MOE_ERR_TOO_LARGE
    assert "scratch" in moe.moe_status_string(moe.MOE_ERR_TOO_LARGE)
    assert L.moe_fused_forward_packed_noalloc(ctypes.byref(moe.MoeShape(0, 256, 128, 4, 2)), None,
                                              *[null] * 5, one, null, null) == moe.MOE_OK
    assert L.moe_fused_forward_packed_noalloc(ctypes.byref(big), None, *[one] * 5, null, one,
                                              null) == moe.MOE_ERR_INVALID_ARG
    # decode-sized shapes fit
    assert moe.moe_workspace_bytes(128, 7168, 2048, 32, 8) <= moe.MOE_NOALLOC_SCRATCH_BYTES
