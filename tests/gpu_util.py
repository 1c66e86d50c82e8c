"""Helpers for the GPU parity tests: upload seeded inputs, call the C ABI
through the thin binding, read intermediates back out of the workspace."""
from __future__ import annotations

import numpy as np
import torch

import combine_dispatch_amd as moe

DEV = "cuda:0"


def to_dev(inp: dict) -> dict:
    d = {}
    for k in ("x", "topk_idx", "topk_w", "W1q", "S1", "W2q", "S2"):
        if k not in inp:
            continue
        a = np.ascontiguousarray(inp[k])
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        d[k] = torch.from_numpy(a).to(DEV)
    return d


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def run_forward(inp: dict, dev: dict | None = None, opts=None, workspace=None):
    """Returns (y bits [T][H], workspace tensor)."""
    dev = dev or to_dev(inp)
    T, H, I, E, K = (inp[k] for k in ("T", "H", "I", "E", "K"))
    if workspace is None:
        workspace = torch.empty(moe.moe_workspace_bytes(T, H, I, E, K), dtype=torch.uint8, device=DEV)
    y = torch.empty((T, H), dtype=torch.int16, device=DEV)
    moe.moe_fused_forward(dev["x"], dev["topk_idx"], dev["topk_w"], dev["W1q"], dev["S1"],
                          dev["W2q"], dev["S2"], y, workspace, opts=opts, E=E, I=I)
    torch.cuda.synchronize()
    return bf16_bits(y), workspace


def view(workspace: torch.Tensor, inp: dict, name: str, rows: int | None = None) -> np.ndarray:
    """Read an intermediate of a fused forward out of its workspace."""
    T, H, I, E, K = (inp[k] for k in ("T", "H", "I", "E", "K"))
    v = moe.moe_workspace_views(T, H, I, E, K)
    TK = T * K
    spec = {
        "counts": (np.int32, (E,)), "offsets": (np.int32, (E + 1,)),
        "pool_src": (np.int32, (TK,)), "slot_to_pool": (np.int32, (TK,)),
        "pool_w": (np.float32, (TK,)), "pool_tok": (np.int32, (TK,)),
        "x_q": (np.uint8, (T, H)), "x_s": (np.uint8, (T, H // 32)),
        "pool_s": (np.uint8, (TK, H // 32)), "act_q": (np.uint8, (TK, I)),
        "act_s": (np.uint8, (TK, I // 32)), "l2_out": (np.uint16, (TK, H)),
    }
    dt, shape = spec[name]
    off = v[name]
    if name == "x_s":
        # token-major words, bytes = groups 4w, 4w+2, 4w+1, 4w+3
        raw = workspace[off:off + T * (H // 32)].cpu().numpy()
        return np.ascontiguousarray(raw.reshape(T, H // 128, 4)[:, :, [0, 2, 1, 3]].reshape(T, H // 32))
    if name in ("pool_s", "act_s"):
        # packed k-major words: word (w, r) at 4 * (w * cap + r), bytes = groups
        # 4w, 4w+2, 4w+1, 4w+3
        cap, groups = v["capacity_rows"], shape[1]
        raw = workspace[off:off + cap * groups].cpu().numpy()
        rm = raw.reshape(groups // 4, cap, 4)[:, :, [0, 2, 1, 3]].transpose(1, 0, 2).reshape(cap, groups)
        return np.ascontiguousarray(rm[:(rows if rows is not None else shape[0])])
    if rows is not None:
        shape = (rows,) + shape[1:]
    nbytes = int(np.prod(shape)) * np.dtype(dt).itemsize
    return workspace[off:off + nbytes].cpu().numpy().view(dt).reshape(shape)


def uses_decode_path(inp: dict) -> bool:
    """Whether the fused layer leaves the workspace's pool_s unwritten: its
    decode-shaped GEMMs (at most 64 routed rows per expert on average) read
    the A-scale words by token when there are at most 1024 routed slots."""
    TK = inp["T"] * inp["K"]
    return TK <= 64 * inp["E"] and TK <= 1024
