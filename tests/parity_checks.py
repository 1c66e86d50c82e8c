"""Element-wise bars the GPU parity tests apply (no GPU needed here).

What the hardware does (measured, tests/test_gpu_mfma_block.py): the scaled
MFMA sums each run of 8 consecutive k of a block with every product aligned
to the run's largest one and truncated toward zero below 2^(e_max - 13);
the runs' sums are then added at fp32 precision, and each MFMA adds its
block to the fp32 accumulator.  A run of 8 therefore loses at most
7 * 2^-13 < 2^-10.19 of its sum of |products|, and a whole GEMM output at
most MFMA_SUM_BOUND * sum_i |a_i * w_i| (the fp32 accumulates add about
2^-19 of it at K = 2048).  The oracle sums exactly.

routing and byte work: bit-exact.

L2 rows (check_l2_rows): compared with the oracle's L2 applied to the GPU's
own activation rows, so that L1's rounding does not enter.  Both sides round
to bf16 at the end, which adds at most one bf16 ulp.  Bar per element:
|o_gpu - o_ref| <= ulp_bf16(max(|o_gpu|, |o_ref|)) + MFMA_SUM_BOUND *
sum_i |a_i * w_i|.

FP8 activations after the L1 epilogue (check_act): codes and scale bytes
identical except at most CODE_FRAC of them; a scale byte moves by at most
one step.  An element whose code differs must satisfy |a_gpu - a_ref| <=
one e4m3 step at its magnitude under the coarser of the two scales (the two
sides' roundings) + the error that the GEMM bound above can carry through
SwiGLU: with gate g and up u each off by at most ulp_bf16 +
MFMA_SUM_BOUND * sum|x_h * w_h|, a = silu(g) * u * w moves by at most
|w| (1.1 |u| dg + |silu(g)| du + 1.1 dg du) (1.1 bounds |silu'|), plus a few
fp32 ulps of a for the fast exp and reciprocal.  Most differing codes are
one step apart; the GEMM term only matters for values near zero, where the
truncated runs can move a value by several steps of the fine grid.

y: per-token relative L2 error <= Y_TOL; all-masked tokens exactly +0; and
y equals the oracle's combine of the GPU's own L2 rows bit for bit.
"""
from __future__ import annotations

import numpy as np

import oracle

Y_TOL = 2e-2
CODE_FRAC = 1e-3
MFMA_SUM_BOUND = 2.0 ** -10


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3_step_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|index difference| of two e4m3 codes on the ordered value line."""
    def ordinal(c):
        c = c.astype(np.int32)
        mag = c & 0x7F
        return np.where(c & 0x80, -mag, mag)
    return np.abs(ordinal(a) - ordinal(b))


def e4m3_step_at(q: np.ndarray) -> np.ndarray:
    """Spacing of the e4m3 grid at magnitude q (q in units of the scale):
    2^-9 below 2^-6 (subnormals), else 2^(floor(log2 q) - 3)."""
    q = np.abs(q)
    e = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
    return np.where(q < 2.0 ** -6, 2.0 ** -9, np.exp2(e - 3))


def check_act(gq, gs, rq, rs, gemm_slack=None):
    """FP8 activation rows: codes [n][I] and scale bytes [n][I/32], GPU (g)
    against oracle (r).  gemm_slack(rows, cols) -> the propagated GEMM error
    bound (absolute) for those elements; None means no slack (the elements
    must then be within one step).  Returns (codes that differ, groups whose
    scale moved, largest |difference| in units of one step)."""
    sdiff = np.abs(gs.astype(np.int32) - rs.astype(np.int32))
    assert sdiff.max(initial=0) <= 1, "a scale byte moved by more than one step"
    assert (sdiff != 0).mean() <= CODE_FRAC, (sdiff != 0).mean()
    gsr = np.repeat(gs, 32, axis=1).astype(np.float64)
    rsr = np.repeat(rs, 32, axis=1).astype(np.float64)
    diff = (gq != rq) | (gsr != rsr)
    assert (gq != rq).mean() <= CODE_FRAC, (gq != rq).mean()
    if not diff.any():
        return 0, 0, 0.0
    i, j = np.nonzero(diff)
    gv = oracle.e4m3_to_f32(gq[i, j]).astype(np.float64) * np.exp2(gsr[i, j] - 127)
    rv = oracle.e4m3_to_f32(rq[i, j]).astype(np.float64) * np.exp2(rsr[i, j] - 127)
    coarse = np.exp2(np.maximum(gsr[i, j], rsr[i, j]) - 127)
    step = e4m3_step_at(np.maximum(np.abs(gv), np.abs(rv)) / coarse) * coarse
    over = np.abs(gv - rv) > step
    if over.any():
        assert gemm_slack is not None, ("codes more than one step apart", int(over.sum()))
        slack = gemm_slack(i[over], j[over])
        bad = np.abs(gv - rv)[over] > step[over] + slack
        assert not bad.any(), (f"{int(bad.sum())} activations beyond one step + the GEMM bound; first: "
                               f"row {i[over][bad][0]} col {j[over][bad][0]} gpu {gv[over][bad][0]} "
                               f"ref {rv[over][bad][0]} step {step[over][bad][0]} slack {slack[bad][0]}")
    return int((gq != rq).sum()), int((sdiff != 0).sum()), float((np.abs(gv - rv) / step).max())


def l1_slack(inp, experts, tokens, weights, h1):
    """gemm_slack for check_act: the bound on |a_gpu - a_ref| that the GEMM
    error bound carries through SwiGLU, for (row, column) pairs of the
    checked rows (experts/tokens/weights/h1 per row; h1 = the oracle's bf16
    gate|up)."""
    I, H = inp["I"], inp["H"]
    xf = oracle.bf16_to_f32(inp["x"])
    cache = {}

    def xdeq(t):
        if t not in cache:
            q, s = oracle.quant_e4m3_row(xf[t])
            cache[t] = act_dequant(q[None], s[None])[0]
        return cache[t]

    def slack(rows, cols):
        out = np.empty(len(rows))
        for n, (r, c) in enumerate(zip(rows, cols)):
            e, t, w = int(experts[r]), int(tokens[r]), float(weights[r])
            xa = np.abs(xdeq(t))
            Wg = fp4_dequant(inp["W1q"][e][[c]], inp["S1"][e][[c]])[0]
            Wu = fp4_dequant(inp["W1q"][e][[I + c]], inp["S1"][e][[I + c]])[0]
            g = float(bf16_f64(h1[r, c:c + 1])[0])
            u = float(bf16_f64(h1[r, I + c:I + c + 1])[0])
            ulp = lambda v: 2.0 ** (np.floor(np.log2(max(abs(v), 2.0 ** -126))) - 7)
            dg = ulp(g) + MFMA_SUM_BOUND * float(xa @ np.abs(Wg))
            du = ulp(u) + MFMA_SUM_BOUND * float(xa @ np.abs(Wu))
            silu = g / (1.0 + np.exp(-g))
            a = silu * u * w
            out[n] = abs(w) * (1.1 * abs(u) * dg + abs(silu) * du + 1.1 * dg * du) + 2.0 ** -20 * abs(a)
        return out

    return slack


def fp4_dequant(Wq: np.ndarray, S: np.ndarray) -> np.ndarray:
    """[N][K/2] packed e2m1 + [N][K/32] scale bytes -> float64 [N][K]
    (OCP FP4 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; sign in bit 3)."""
    mag = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    table = np.concatenate([mag, -mag])
    codes = np.stack([Wq & 0xF, Wq >> 4], axis=-1).reshape(Wq.shape[0], -1)
    return table[codes] * np.repeat(np.exp2(S.astype(np.float64) - 127), 32, axis=1)


def act_dequant(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    return oracle.e4m3_to_f32(q).astype(np.float64) * np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)


def check_l2_rows(inp, experts, gpu_o, ref_o, act_q, act_s):
    """GPU L2 rows (bf16 bits [n][H]) against the oracle's L2 of the same
    activation rows (act_q/act_s: the GPU's), with the bar in the module
    docstring.  Returns (elements not bit-identical, rows checked)."""
    experts = np.asarray(experts)
    g, r = bf16_f64(gpu_o), bf16_f64(ref_o)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.maximum(np.abs(g), np.abs(r)), 2.0 ** -126))) - 7)
    bound = np.empty_like(g)
    ad = np.abs(act_dequant(act_q, act_s))
    for e in np.unique(experts):
        sel = np.nonzero(experts == e)[0]
        W = np.abs(fp4_dequant(inp["W2q"][e], inp["S2"][e]))
        bound[sel] = ad[sel] @ W.T
    lim = ulp + MFMA_SUM_BOUND * bound
    bad = np.abs(g - r) > lim
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(f"L2 row {i} col {j}: gpu {g[i, j]} ref {r[i, j]} limit {lim[i, j]}; "
                             f"{int(bad.sum())} elements over the bar")
    return int((gpu_o != ref_o).sum()), len(experts)


def rel_l2_rows(y: np.ndarray, ref: np.ndarray) -> np.ndarray:
    yf, rf = bf16_f64(y), bf16_f64(ref)
    num = np.linalg.norm(yf - rf, axis=1)
    den = np.linalg.norm(rf, axis=1)
    return np.where(den > 0, num / np.maximum(den, 1e-300), num)


def check_y(y, ref, idx):
    rel = rel_l2_rows(y, ref)
    masked = (idx < 0).all(axis=1)
    assert (y[masked] == 0).all()
    assert rel[~masked].max(initial=0) <= Y_TOL, rel.max()
    return float(rel.max(initial=0))


def mtile_sample_rows(offsets: np.ndarray, bm: int = 256, rng=None) -> np.ndarray:
    """The first and last valid pool row of every bm-row m-tile of every
    expert (the GEMMs' tiling), plus one row in between when rng is given."""
    rows = []
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        for r0 in range(lo, hi, bm):
            r1 = min(r0 + bm, hi) - 1
            rows += [r0, r1]
            if rng is not None and r1 > r0 + 1:
                rows.append(int(rng.integers(r0 + 1, r1)))
    return np.unique(np.asarray(rows, np.int64))
