"""CPU oracle for the MoE layer hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never loads it, and the
oracle never loads the HIP library: the two share no code.

The arithmetic lives in ``moe_oracle.c`` (plain C11); this module only builds
it and marshals numpy arrays through ctypes.  Page citations are in the C
file's header comments.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libmoe_oracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-shared", "-fPIC", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("K", ctypes.c_int32)]


class _Mid(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("pool_q", "pool_s", "h1", "act_q", "act_s", "o", "counts", "offsets",
                 "pool_src", "slot_to_pool", "pool_w")]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_to_f32.restype = ctypes.c_float
        L.oracle_e4m3_from_f64.argtypes = [ctypes.c_double]
        L.oracle_e4m3_from_f64.restype = ctypes.c_uint8
        L.oracle_e2m1_to_f32.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_to_f32.restype = ctypes.c_float
        L.oracle_ue8m0_for_e4m3.argtypes = [ctypes.c_float]
        L.oracle_ue8m0_for_e4m3.restype = ctypes.c_uint8
        L.oracle_ue8m0_value.argtypes = [ctypes.c_uint8]
        L.oracle_ue8m0_value.restype = ctypes.c_double
        L.oracle_e4m3_from_f64_array.argtypes = [vp, vp, ctypes.c_size_t]
        L.oracle_ue8m0_for_e4m3_array.argtypes = [vp, vp, ctypes.c_size_t]
        L.oracle_quant_e4m3_row.argtypes = [vp, i32, vp, vp]
        L.oracle_route.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_dispatch.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, i32, vp, vp, vp, vp, vp,
                                      vp, vp]
        L.oracle_combine.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.oracle_forward.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, vp, vp, vp, vp,
                                     ctypes.POINTER(_Mid)]
        L.oracle_forward_tokens.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, vp, vp, vp, vp,
                                            i32, vp, vp, vp, vp]
        L.oracle_l1_act_rows.argtypes = [ctypes.POINTER(Shape), vp, vp, vp, i32, vp, vp, vp, vp,
                                         vp, vp]
        L.oracle_l2_rows.argtypes = [ctypes.POINTER(Shape), vp, vp, i32, vp, vp, vp, vp]
        L.oracle_num_threads.restype = i32
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


# ---- codecs -----------------------------------------------------------------
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(v: np.ndarray) -> np.ndarray:
    L = lib()
    return np.array([L.oracle_f32_to_bf16(float(a)) for a in np.ravel(v)],
                    dtype=np.uint16).reshape(np.shape(v))


def e4m3_to_f32(codes: np.ndarray) -> np.ndarray:
    L = lib()
    table = np.array([L.oracle_e4m3_to_f32(c) for c in range(256)], dtype=np.float32)
    return table[np.asarray(codes, dtype=np.uint8)]


def e4m3_from_f64(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_e4m3_from_f64_array(_p(v), _p(out), v.size)
    return out


def e2m1_to_f32(nibbles: np.ndarray) -> np.ndarray:
    L = lib()
    table = np.array([L.oracle_e2m1_to_f32(c) for c in range(16)], dtype=np.float32)
    return table[np.asarray(nibbles, dtype=np.uint8) & 0xF]


def ue8m0_for_e4m3(amax: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(amax, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint8)
    lib().oracle_ue8m0_for_e4m3_array(_p(a), _p(out), a.size)
    return out


def quant_e4m3_row(v: np.ndarray):
    v = np.ascontiguousarray(v, dtype=np.float32)
    q = np.empty(v.shape, dtype=np.uint8)
    s = np.empty(v.size // 32, dtype=np.uint8)
    _check(lib().oracle_quant_e4m3_row(_p(v), v.size, _p(q), _p(s)), "quant_e4m3_row")
    return q, s


# ---- the layer --------------------------------------------------------------
def route(topk_idx: np.ndarray, topk_w: np.ndarray, E: int):
    T, K = topk_idx.shape
    idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    pool_src = np.full(T * K, -1, np.int32)
    slot_to_pool = np.full(T * K, -1, np.int32)
    pool_w = np.zeros(T * K, np.float32)
    _check(lib().oracle_route(T, K, E, _p(idx), _p(w), _p(counts), _p(offsets), _p(pool_src),
                              _p(slot_to_pool), _p(pool_w)), "route")
    return dict(counts=counts, offsets=offsets, pool_src=pool_src, slot_to_pool=slot_to_pool,
                pool_w=pool_w)


def dispatch(x_bf16: np.ndarray, topk_idx: np.ndarray, topk_w: np.ndarray, E: int,
             payload: int = 0):
    T, H = x_bf16.shape
    K = topk_idx.shape[1]
    s = Shape(T, H, 32, E, K)
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int64)
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    pool_src = np.full(T * K, -1, np.int32)
    slot_to_pool = np.full(T * K, -1, np.int32)
    pool_w = np.zeros(T * K, np.float32)
    if payload == 0:
        pool = np.zeros((T * K, H), np.uint8)
        scales = np.zeros((T * K, H // 32), np.uint8)
    else:
        pool = np.zeros((T * K, H), np.uint16)
        scales = None
    _check(lib().oracle_dispatch(ctypes.byref(s), _p(x), _p(idx), _p(w), payload, _p(counts),
                                 _p(offsets), _p(pool_src), _p(slot_to_pool), _p(pool_w),
                                 _p(pool), _p(scales)), "dispatch")
    return dict(counts=counts, offsets=offsets, pool_src=pool_src, slot_to_pool=slot_to_pool,
                pool_w=pool_w, pool=pool, pool_scales=scales)


def combine(o_bf16: np.ndarray, slot_to_pool: np.ndarray, T: int, K: int,
            topk_w: np.ndarray | None = None):
    H = o_bf16.shape[1]
    o = np.ascontiguousarray(o_bf16, dtype=np.uint16)
    s2p = np.ascontiguousarray(slot_to_pool, dtype=np.int32)
    w = None if topk_w is None else np.ascontiguousarray(topk_w, dtype=np.float32)
    y = np.zeros((T, H), np.uint16)
    _check(lib().oracle_combine(T, K, H, _p(o), _p(s2p), _p(w), _p(y)), "combine")
    return y


def forward(inp: dict, intermediates: bool = False):
    """Grouped forward.  ``inp`` holds x, topk_idx, topk_w, W1q, S1, W2q, S2 and
    the shape keys T, H, I, E, K (see moe_inputs)."""
    T, H, I, E, K = (inp[k] for k in ("T", "H", "I", "E", "K"))
    s = Shape(T, H, I, E, K)
    y = np.zeros((T, H), np.uint16)
    mid_arrays = None
    mid = None
    if intermediates:
        TK = T * K
        mid_arrays = dict(pool_q=np.zeros((TK, H), np.uint8), pool_s=np.zeros((TK, H // 32), np.uint8),
                          h1=np.zeros((TK, 2 * I), np.uint16), act_q=np.zeros((TK, I), np.uint8),
                          act_s=np.zeros((TK, I // 32), np.uint8), o=np.zeros((TK, H), np.uint16),
                          counts=np.zeros(E, np.int32), offsets=np.zeros(E + 1, np.int32),
                          pool_src=np.full(TK, -1, np.int32), slot_to_pool=np.full(TK, -1, np.int32),
                          pool_w=np.zeros(TK, np.float32))
        mid = _Mid(**{k: v.ctypes.data for k, v in mid_arrays.items()})
    args = [np.ascontiguousarray(inp[k]) for k in ("x", "topk_idx", "topk_w", "W1q", "S1", "W2q", "S2")]
    _check(lib().oracle_forward(ctypes.byref(s), *[_p(a) for a in args], _p(y),
                                ctypes.byref(mid) if mid is not None else None), "forward")
    if intermediates:
        return y, mid_arrays
    return y


def forward_tokens(inp: dict, tokens, activations: bool = False):
    """Brute-force per-token forward for the listed token indices -> bf16 rows;
    with ``activations``, also each slot's requantised activation row:
    (y, act_q [n][K][I], act_s [n][K][I/32]), zero for masked slots."""
    T, H, I, E, K = (inp[k] for k in ("T", "H", "I", "E", "K"))
    s = Shape(T, H, I, E, K)
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
    y = np.zeros((tok.size, H), np.uint16)
    aq = np.zeros((tok.size, K, I), np.uint8) if activations else None
    as_ = np.zeros((tok.size, K, I // 32), np.uint8) if activations else None
    args = [np.ascontiguousarray(inp[k]) for k in ("x", "topk_idx", "topk_w", "W1q", "S1", "W2q", "S2")]
    _check(lib().oracle_forward_tokens(ctypes.byref(s), *[_p(a) for a in args], tok.size, _p(tok),
                                       _p(y), _p(aq), _p(as_)), "forward_tokens")
    if activations:
        return y, aq, as_
    return y


def l1_act_rows(inp: dict, experts, tokens, weights, h1: bool = False):
    """Chosen routed rows through quantise -> L1 -> SwiGLU*w -> requant:
    row i is token tokens[i] through expert experts[i] with weight weights[i].
    -> (act_q [n][I], act_s [n][I/32]) or, with ``h1``, (h1 [n][2I] bf16,
    act_q, act_s)."""
    T, H, I, E, K = (inp[k] for k in ("T", "H", "I", "E", "K"))
    s = Shape(T, H, I, E, K)
    ex = np.ascontiguousarray(np.asarray(experts, dtype=np.int32))
    tk = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
    wt = np.ascontiguousarray(np.asarray(weights, dtype=np.float32))
    n = ex.size
    assert tk.size == n and wt.size == n
    aq = np.zeros((n, I), np.uint8)
    as_ = np.zeros((n, I // 32), np.uint8)
    h1_rows = np.zeros((n, 2 * I), np.uint16) if h1 else None
    x, W1q, S1 = (np.ascontiguousarray(inp[k]) for k in ("x", "W1q", "S1"))
    _check(lib().oracle_l1_act_rows(ctypes.byref(s), _p(x), _p(W1q), _p(S1), n, _p(ex), _p(tk),
                                    _p(wt), _p(h1_rows), _p(aq), _p(as_)), "l1_act_rows")
    return (h1_rows, aq, as_) if h1 else (aq, as_)


def l2_rows(inp: dict, experts, act_q: np.ndarray, act_s: np.ndarray) -> np.ndarray:
    """L2 alone on given activation rows (codes [n][I], scale bytes [n][I/32])
    through experts[i] -> bf16 bits [n][H]."""
    T, H, I, E, K = (inp[k] for k in ("T", "H", "I", "E", "K"))
    s = Shape(T, H, I, E, K)
    ex = np.ascontiguousarray(np.asarray(experts, dtype=np.int32))
    aq = np.ascontiguousarray(act_q, dtype=np.uint8)
    as_ = np.ascontiguousarray(act_s, dtype=np.uint8)
    n = ex.size
    assert aq.shape == (n, I) and as_.shape == (n, I // 32)
    o = np.zeros((n, H), np.uint16)
    W2q, S2 = (np.ascontiguousarray(inp[k]) for k in ("W2q", "S2"))
    _check(lib().oracle_l2_rows(ctypes.byref(s), _p(W2q), _p(S2), n, _p(ex), _p(aq), _p(as_),
                                _p(o)), "l2_rows")
    return o


def num_threads() -> int:
    return int(lib().oracle_num_threads())
