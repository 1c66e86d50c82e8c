"""Seeded synthetic inputs for the MoE layer.

This module prepares inputs only and holds none of the layer's arithmetic.
The HIP library's tests and benchmark and the CPU oracle both consume what it
returns, so the two sides always see identical bytes.

Workloads (one MoE layer's share on one GPU):

=====  ======  =====  =====  ====  ==  ===========================================
name   T       H      I      E     K   routing
=====  ======  =====  =====  ====  ==  ===========================================
tiny   64      256    512    8     2   softmax of N(0,1) router logits, top-2,
                                       weights renormalised to sum 1
small  128     7168   2048   32    8   K distinct experts uniformly at random
prefill 8192   7168   2048   32    8   same as small (~2048 rows per expert)
skewed 8192    7168   2048   32    8   Zipf(1.2) popularity, drawn without
                                       replacement; 5% of slots masked to -1
many   16384   2048   768    128   8   uniform, ~1024 rows per expert
=====  ======  =====  =====  ====  ==  ===========================================

Values: x ~ N(0,1) as bf16; W1 [E][2I][H] and W2 [E][H][I] ~ N(0, 0.02) as FP4
e2m1 with one UE8M0 scale per 32 along K (W1 rows 0..I-1 are the gate
projection, rows I..2I-1 the up projection).  Where the routing recipe leaves
the weights open (uniform and Zipf routing), ``topk_w`` is the softmax of K
iid N(0,1) logits in draw order.

Bulk tensors come from ``gen.c`` (Philox4x32-10 + Box-Muller, OpenMP);
routing uses numpy's Philox bit generator.  Everything is a pure function of
(shape, routing recipe, seed).
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libmoe_inputs.so")
_lib = None

# stream ids inside one seed
_STREAM_X, _STREAM_W1, _STREAM_W2 = 1, 2, 3
WEIGHT_STD = 0.02

CONFIGS = [
    dict(name="tiny", T=64, H=256, I=512, E=8, K=2, routing="softmax_topk", seed=0),
    dict(name="small", T=128, H=7168, I=2048, E=32, K=8, routing="uniform", seed=1),
    dict(name="prefill", T=8192, H=7168, I=2048, E=32, K=8, routing="uniform", seed=2),
    dict(name="skewed", T=8192, H=7168, I=2048, E=32, K=8, routing="zipf", zipf_s=1.2,
         mask_p=0.05, seed=3),
    dict(name="many", T=16384, H=2048, I=768, E=128, K=8, routing="uniform", seed=4),
]
CONFIG_BY_NAME = {c["name"]: c for c in CONFIGS}


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-Wall", "-o",
                        tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _gen():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        u64, u32, vp, i64 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int64
        L.gen_normal_f32.argtypes = [u64, u32, ctypes.c_double, ctypes.c_double, vp, i64]
        L.gen_normal_bf16.argtypes = [u64, u32, vp, i64]
        L.gen_fp4_weights.argtypes = [u64, u32, ctypes.c_double, i64, ctypes.c_int32, vp, vp]
        L.gen_philox4x32_10.argtypes = [vp, vp, vp]
        _lib = L
    return _lib


def philox4x32_10(ctr, key) -> np.ndarray:
    """One block of the generator: four uint32 words from counter ctr[4], key key[2]."""
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.empty(4, np.uint32)
    _gen().gen_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def normal_f32(seed: int, stream: int, n: int, mean=0.0, std=1.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    _gen().gen_normal_f32(seed, stream, mean, std, out.ctypes.data, n)
    return out


def bf16_normal(seed: int, stream: int, shape) -> np.ndarray:
    out = np.empty(shape, np.uint16)
    _gen().gen_normal_bf16(seed, stream, out.ctypes.data, out.size)
    return out


def fp4_weights(seed: int, stream: int, rows: int, kdim: int, std: float = WEIGHT_STD):
    assert kdim % 32 == 0
    q = np.empty((rows, kdim // 2), np.uint8)
    s = np.empty((rows, kdim // 32), np.uint8)
    _gen().gen_fp4_weights(seed, stream, std, rows, kdim, q.ctypes.data, s.ctypes.data)
    return q, s


def _softmax(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def make_routing(T: int, E: int, K: int, routing: str, seed: int, zipf_s: float = 1.2,
                 mask_p: float = 0.0):
    """topk_idx int64 [T][K] (-1 = masked) and topk_w float32 [T][K]."""
    rng = np.random.Generator(np.random.Philox(key=seed))
    if routing == "softmax_topk":
        p = _softmax(rng.standard_normal((T, E)))
        order = np.argsort(-p, axis=1, kind="stable")[:, :K]  # descending, ties -> lower index
        top = np.take_along_axis(p, order, axis=1)
        idx = order.astype(np.int64)
        w = (top / top.sum(axis=1, keepdims=True)).astype(np.float32)
    elif routing in ("uniform", "zipf"):
        if K > E:
            raise ValueError("distinct-expert routing needs K <= E")
        if routing == "uniform":
            keys = rng.random((T, E))
        else:
            # sequential sampling without replacement from p_e ~ (e+1)^-s is the
            # descending order of log p_e + Gumbel noise (Plackett-Luce)
            logp = -zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
            u = rng.random((T, E))
            keys = logp[None, :] - np.log(-np.log(np.clip(u, 1e-300, 1.0)))
        idx = np.argsort(-keys, axis=1, kind="stable")[:, :K].astype(np.int64)
        w = _softmax(rng.standard_normal((T, K))).astype(np.float32)
    elif routing == "all_to_zero":
        idx = np.zeros((T, K), np.int64)
        w = np.full((T, K), 1.0 / K, np.float32)
    else:
        raise ValueError(f"unknown routing {routing!r}")
    if mask_p > 0.0:
        idx = np.where(rng.random((T, K)) < mask_p, np.int64(-1), idx)
    return np.ascontiguousarray(idx), np.ascontiguousarray(w)


def make_inputs(T: int, H: int, I: int, E: int, K: int, routing: str = "uniform", seed: int = 0,
                name: str = "custom", weights: bool = True, **routing_kw) -> dict:
    """All layer inputs as numpy arrays (host memory)."""
    if H % 32 or I % 32:
        raise ValueError("H and I must be multiples of 32")
    idx, w = make_routing(T, E, K, routing, seed, **routing_kw)
    d = dict(name=name, seed=seed, T=T, H=H, I=I, E=E, K=K, topk_idx=idx, topk_w=w,
             x=bf16_normal(seed, _STREAM_X, (T, H)))
    if weights:
        W1q, S1 = fp4_weights(seed, _STREAM_W1, E * 2 * I, H)
        W2q, S2 = fp4_weights(seed, _STREAM_W2, E * H, I)
        d.update(W1q=W1q.reshape(E, 2 * I, H // 2), S1=S1.reshape(E, 2 * I, H // 32),
                 W2q=W2q.reshape(E, H, I // 2), S2=S2.reshape(E, H, I // 32))
    return d


def config_inputs(name_or_index, **overrides) -> dict:
    c = dict(CONFIGS[name_or_index] if isinstance(name_or_index, int) else CONFIG_BY_NAME[name_or_index])
    c.update(overrides)
    return make_inputs(**c)


def sha256_manifest(inp: dict) -> dict:
    return {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()
            for k, v in inp.items() if isinstance(v, np.ndarray)}
