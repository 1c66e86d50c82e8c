"""Python binding of libmoe_hip.so -- argument marshalling only.

Every step of the MoE layer runs in the HIP kernels behind the C ABI in
``include/moe.h``; this module passes torch device tensors' pointers and the
current HIP stream through ctypes.  There is no fallback: if the library is
missing or the device is not gfx950 the calls raise.

Names match the C entry points: ``moe_fused_forward``,
``moe_fused_forward_packed``, ``moe_fused_forward_packed_noalloc``, ``moe_dispatch``,
``moe_combine``, ``moe_workspace_bytes``, ``moe_dispatch_workspace_bytes``,
``moe_workspace_views``, ``moe_status_string``.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_hip.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_DEVICE = -4
MOE_ERR_BAD_ROUTING = -5
MOE_ERR_TOO_LARGE = -6
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
MOE_PAYLOAD_FP8_E4M3 = 0
MOE_PAYLOAD_BF16 = 1
MOE_TILES_AUTO = 0
MOE_TILES_PERSISTENT = 1
MOE_TILES_64 = 2
MOE_TILES_128 = 3
MOE_TILES_FUSED = 4

EXPORTED = ("moe_default_options", "moe_workspace_bytes", "moe_dispatch_workspace_bytes",
            "moe_fused_forward", "moe_dispatch", "moe_combine", "moe_workspace_views",
            "moe_status_string", "moe_profile_start", "moe_profile_stop",
            "moe_profile_stage_name", "moe_packed_scales_bytes", "moe_pack_weight_scales",
            "moe_packed_weights_bytes", "moe_pack_weights", "moe_fused_forward_prepacked",
            "moe_fused_forward_packed", "moe_fused_forward_packed_noalloc")
PROFILE_STAGES = 8


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("K", ctypes.c_int32)]


class MoeOptions(ctypes.Structure):
    _fields_ = [("fast_math", ctypes.c_int32), ("activation_clamp", ctypes.c_float),
                ("debug_validate", ctypes.c_int32), ("gemm_tiles", ctypes.c_int32)]


class MoeWorkspaceViews(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("counts", "offsets", "pool_src", "slot_to_pool", "pool_w", "pool_tok", "x_q",
                 "x_s", "pool_s", "act_q", "act_s", "l2_out", "capacity_rows")]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {moe_status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib():
    """Load libmoe_hip.so (built by combine_dispatch_amd/build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with combine_dispatch_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        shp = ctypes.POINTER(MoeShape)
        L.moe_default_options.restype = MoeOptions
        L.moe_workspace_bytes.argtypes = [shp]
        L.moe_workspace_bytes.restype = sz
        L.moe_dispatch_workspace_bytes.argtypes = [shp]
        L.moe_dispatch_workspace_bytes.restype = sz
        L.moe_fused_forward.argtypes = [shp, ctypes.POINTER(MoeOptions), vp, vp, vp, vp, vp, vp,
                                        vp, vp, vp, sz, vp]
        L.moe_fused_forward.restype = i32
        L.moe_packed_scales_bytes.argtypes = [shp]
        L.moe_packed_scales_bytes.restype = sz
        L.moe_pack_weight_scales.argtypes = [shp, vp, vp, vp, sz, vp]
        L.moe_pack_weight_scales.restype = i32
        L.moe_fused_forward_packed.argtypes = [shp, ctypes.POINTER(MoeOptions), vp, vp, vp, vp,
                                               vp, vp, vp, vp, sz, vp]
        L.moe_fused_forward_packed.restype = i32
        L.moe_packed_weights_bytes.argtypes = [shp]
        L.moe_packed_weights_bytes.restype = sz
        L.moe_pack_weights.argtypes = [shp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_pack_weights.restype = i32
        L.moe_fused_forward_prepacked.argtypes = [shp, ctypes.POINTER(MoeOptions), vp, vp, vp, vp, vp,
                                                  vp, sz, vp]
        L.moe_fused_forward_prepacked.restype = i32
        L.moe_fused_forward_packed_noalloc.argtypes = [shp, ctypes.POINTER(MoeOptions), vp, vp, vp,
                                                       vp, vp, vp, vp, vp]
        L.moe_fused_forward_packed_noalloc.restype = i32
        L.moe_dispatch.argtypes = [shp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_dispatch.restype = i32
        L.moe_combine.argtypes = [shp, vp, vp, vp, vp, vp]
        L.moe_combine.restype = i32
        L.moe_workspace_views.argtypes = [shp, ctypes.POINTER(MoeWorkspaceViews)]
        L.moe_workspace_views.restype = i32
        L.moe_status_string.argtypes = [i32]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_profile_start.argtypes = [i32]
        L.moe_profile_start.restype = i32
        L.moe_profile_stop.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]
        L.moe_profile_stop.restype = i32
        L.moe_profile_stage_name.argtypes = [i32]
        L.moe_profile_stage_name.restype = ctypes.c_char_p
        _lib = L
    return _lib


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc: int, what: str):
    if rc != MOE_OK:
        raise MoeError(rc, what)


def moe_default_options() -> MoeOptions:
    return lib().moe_default_options()


def options(fast_math: bool = True, activation_clamp: float | None = None,
            debug_validate: bool = False, gemm_tiles: int = MOE_TILES_AUTO) -> MoeOptions:
    return MoeOptions(1 if fast_math else 0,
                      math.nan if activation_clamp is None else float(activation_clamp),
                      1 if debug_validate else 0, int(gemm_tiles))


def moe_workspace_bytes(T: int, H: int, I: int, E: int, K: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(MoeShape(T, H, I, E, K))))


def moe_dispatch_workspace_bytes(T: int, H: int, E: int, K: int, I: int = 32) -> int:
    return int(lib().moe_dispatch_workspace_bytes(ctypes.byref(MoeShape(T, H, I, E, K))))


def moe_workspace_views(T: int, H: int, I: int, E: int, K: int) -> dict:
    v = MoeWorkspaceViews()
    _check(lib().moe_workspace_views(ctypes.byref(MoeShape(T, H, I, E, K)), ctypes.byref(v)),
           "moe_workspace_views")
    return {n: int(getattr(v, n)) for n, _ in MoeWorkspaceViews._fields_}


def moe_fused_forward(x, topk_idx, topk_w, W1q, S1, W2q, S2, y, workspace, opts=None,
                      stream=None, E: int | None = None, I: int | None = None) -> None:
    """y[T][H] (bf16) <- the layer on device tensors.  ``workspace`` is a
    uint8 device tensor of at least moe_workspace_bytes(...) bytes."""
    T, H = x.shape
    K = topk_idx.shape[1]
    E = W1q.shape[0] if E is None else E
    I = W2q.shape[2] * 2 if I is None else I
    shape = MoeShape(T, H, I, E, K)
    o = ctypes.byref(opts) if opts is not None else None
    _check(lib().moe_fused_forward(ctypes.byref(shape), o, _ptr(x), _ptr(topk_idx), _ptr(topk_w),
                                   _ptr(W1q), _ptr(S1), _ptr(W2q), _ptr(S2), _ptr(y),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)), "moe_fused_forward")


def moe_packed_scales_bytes(H: int, I: int, E: int) -> int:
    """Bytes of the buffer moe_pack_weight_scales fills (0 on a bad shape)."""
    return int(lib().moe_packed_scales_bytes(ctypes.byref(MoeShape(1, H, I, E, 1))))


def moe_pack_weight_scales(S1, S2, packed, E: int, H: int, I: int, stream=None) -> None:
    """Lay the weight scales out once for moe_fused_forward_packed; ``packed``
    is a uint8 device tensor of at least moe_packed_scales_bytes(H, I, E) bytes."""
    shape = MoeShape(1, H, I, E, 1)
    _check(lib().moe_pack_weight_scales(ctypes.byref(shape), _ptr(S1), _ptr(S2), _ptr(packed),
                                        packed.numel() * packed.element_size(), _stream(stream)),
           "moe_pack_weight_scales")


def moe_fused_forward_packed(x, topk_idx, topk_w, W1q, W2q, packed, y, workspace, opts=None,
                             stream=None, E: int | None = None, I: int | None = None) -> None:
    """moe_fused_forward with weight scales from moe_pack_weight_scales."""
    T, H = x.shape
    K = topk_idx.shape[1]
    E = W1q.shape[0] if E is None else E
    I = W2q.shape[2] * 2 if I is None else I
    shape = MoeShape(T, H, I, E, K)
    o = ctypes.byref(opts) if opts is not None else None
    _check(lib().moe_fused_forward_packed(ctypes.byref(shape), o, _ptr(x), _ptr(topk_idx),
                                          _ptr(topk_w), _ptr(W1q), _ptr(W2q), _ptr(packed),
                                          _ptr(y), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          _stream(stream)), "moe_fused_forward_packed")


def moe_packed_weights_bytes(H: int, I: int, E: int) -> int:
    """Bytes of the buffer moe_pack_weights fills (0 on a bad shape)."""
    return int(lib().moe_packed_weights_bytes(ctypes.byref(MoeShape(1, H, I, E, 1))))


def moe_pack_weights(W1q, S1, W2q, S2, packed, E: int, H: int, I: int, stream=None) -> None:
    """Lay every weight (FP4 codes tile-blocked, scales packed) out once for
    moe_fused_forward_prepacked; ``packed`` is a uint8 device tensor of at
    least moe_packed_weights_bytes(H, I, E) bytes."""
    shape = MoeShape(1, H, I, E, 1)
    _check(lib().moe_pack_weights(ctypes.byref(shape), _ptr(W1q), _ptr(S1), _ptr(W2q), _ptr(S2),
                                  _ptr(packed), packed.numel() * packed.element_size(), _stream(stream)),
           "moe_pack_weights")


def moe_fused_forward_prepacked(x, topk_idx, topk_w, packed, y, workspace, E: int, I: int, opts=None,
                                stream=None) -> None:
    """moe_fused_forward with every weight read from the buffer moe_pack_weights filled."""
    T, H = x.shape
    K = topk_idx.shape[1]
    shape = MoeShape(T, H, I, E, K)
    o = ctypes.byref(opts) if opts is not None else None
    _check(lib().moe_fused_forward_prepacked(ctypes.byref(shape), o, _ptr(x), _ptr(topk_idx),
                                             _ptr(topk_w), _ptr(packed), _ptr(y), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(),
                                             _stream(stream)), "moe_fused_forward_prepacked")


def moe_fused_forward_packed_noalloc(x, topk_idx, topk_w, W1q, W2q, packed, y, opts=None,
                                     stream=None, E: int | None = None,
                                     I: int | None = None) -> None:
    """moe_fused_forward_packed with the library's own device scratch as the
    workspace (no allocation in the call; shapes whose moe_workspace_bytes
    exceeds MOE_NOALLOC_SCRATCH_BYTES raise MoeError MOE_ERR_TOO_LARGE)."""
    T, H = x.shape
    K = topk_idx.shape[1]
    E = W1q.shape[0] if E is None else E
    I = W2q.shape[2] * 2 if I is None else I
    shape = MoeShape(T, H, I, E, K)
    o = ctypes.byref(opts) if opts is not None else None
    _check(lib().moe_fused_forward_packed_noalloc(ctypes.byref(shape), o, _ptr(x), _ptr(topk_idx),
                                                  _ptr(topk_w), _ptr(W1q), _ptr(W2q), _ptr(packed),
                                                  _ptr(y), _stream(stream)),
           "moe_fused_forward_packed_noalloc")


def moe_dispatch(x, topk_idx, topk_w, E: int, payload: int, counts, offsets, pool_src,
                 slot_to_pool, pool_w, pool, pool_scales, workspace, stream=None) -> None:
    T, H = x.shape
    K = topk_idx.shape[1]
    shape = MoeShape(T, H, 32, E, K)
    _check(lib().moe_dispatch(ctypes.byref(shape), _ptr(x), _ptr(topk_idx), _ptr(topk_w),
                              int(payload), _ptr(counts), _ptr(offsets), _ptr(pool_src),
                              _ptr(slot_to_pool), _ptr(pool_w), _ptr(pool), _ptr(pool_scales),
                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream)), "moe_dispatch")


def moe_combine(pool_out, slot_to_pool, T: int, K: int, y, topk_w=None, stream=None) -> None:
    H = pool_out.shape[1]
    shape = MoeShape(T, H, 32, 1, K)
    _check(lib().moe_combine(ctypes.byref(shape), _ptr(pool_out), _ptr(slot_to_pool),
                             _ptr(topk_w), _ptr(y), _stream(stream)), "moe_combine")


def moe_profile_start(max_calls: int) -> None:
    _check(lib().moe_profile_start(int(max_calls)), "moe_profile_start")


def moe_profile_stop() -> tuple[dict, int]:
    """-> ({stage name: summed ms}, number of recorded calls)."""
    ms = (ctypes.c_double * PROFILE_STAGES)()
    n = ctypes.c_int(0)
    _check(lib().moe_profile_stop(ms, ctypes.byref(n)), "moe_profile_stop")
    names = [lib().moe_profile_stage_name(i).decode() for i in range(PROFILE_STAGES)]
    return dict(zip(names, list(ms))), int(n.value)
