"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

Bars (routing and dispatch are integer/byte work, the rest floating point):
  - counts, offsets, pool_src, slot_to_pool, pool_w, the token of each pool
    row, and the quantised token rows (codes and scale bytes) the L1 GEMM
    gathers its pool rows from: bit-exact;
  - combine fed identical bf16 rows: bit-exact (same summation order);
  - intermediate FP8 activations after L1: scale bytes and codes identical
    except at most 0.1% of elements, which may be one code step apart (one
    scale step for scale bytes);
  - y: per-token relative L2 error <= 2e-2, all-masked tokens exactly +0.
"""
import os

import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from tests.gpu_util import (DEV, bf16_bits, e4m3_step_distance, rel_l2_rows, run_forward, to_dev,
                            view)

pytestmark = pytest.mark.gpu

Y_TOL = 2e-2
CODE_FRAC = 1e-3


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_dispatch_amd as moe
    moe.lib()  # fails loudly if the HIP library is missing


def check_routing(inp, ws):
    r = oracle.route(inp["topk_idx"], inp["topk_w"], inp["E"])
    R = int(r["offsets"][-1])
    np.testing.assert_array_equal(view(ws, inp, "counts"), r["counts"])
    np.testing.assert_array_equal(view(ws, inp, "offsets"), r["offsets"])
    np.testing.assert_array_equal(view(ws, inp, "pool_src")[:R], r["pool_src"][:R])
    np.testing.assert_array_equal(view(ws, inp, "slot_to_pool"), r["slot_to_pool"])
    np.testing.assert_array_equal(view(ws, inp, "pool_w")[:R].view(np.uint32),
                                  r["pool_w"][:R].view(np.uint32))
    return r, R


def check_act(gq, gs, rq, rs):
    """FP8 intermediate: codes [n][I], scale bytes [n][I/32].

    At most CODE_FRAC of the codes may differ, each by one e4m3 step; near
    zero (both codes subnormal) by two subnormal steps, i.e. 2^-8 of the
    group scale.  The scaled MFMA does not accumulate a 64-wide K block
    exactly in fp32 (measured: a block whose exact sum has 22 significant
    bits comes out 2^-18 off), so an activation whose exact value is 0 can
    come out a step or two of the subnormal grid away from 0."""
    sdiff = np.abs(gs.astype(np.int32) - rs.astype(np.int32))
    assert sdiff.max(initial=0) <= 1
    assert (sdiff != 0).mean() <= CODE_FRAC
    same = np.repeat(sdiff == 0, 32, axis=1)
    dist = e4m3_step_distance(gq, rq)
    subnormal = ((gq & 0x78) == 0) & ((rq & 0x78) == 0)
    allowed = np.where(subnormal, 2, 1)
    assert (dist[same] <= allowed[same]).all(), dist[same].max(initial=0)
    assert (dist[same] != 0).mean() <= CODE_FRAC, (dist[same] != 0).mean()
    if (~same).any():  # scale moved by one step: values within one step of the coarser scale
        gv = oracle.e4m3_to_f32(gq) * np.exp2(np.repeat(gs, 32, axis=1).astype(np.float64) - 127)
        rv = oracle.e4m3_to_f32(rq) * np.exp2(np.repeat(rs, 32, axis=1).astype(np.float64) - 127)
        coarse = np.exp2(np.maximum(np.repeat(gs, 32, 1), np.repeat(rs, 32, 1)).astype(np.float64) - 127)
        assert (np.abs(gv - rv)[~same] <= 32 * coarse[~same]).all()


def check_y(y, ref, idx):
    rel = rel_l2_rows(y, ref)
    masked = (idx < 0).all(axis=1)
    assert (y[masked] == 0).all()
    assert rel[~masked].max(initial=0) <= Y_TOL, rel.max()
    return float(rel.max(initial=0))


# ----------------------------------------------------------------------------
# small shapes: every intermediate against the grouped oracle
# ----------------------------------------------------------------------------
SMALL = [
    dict(name="tiny"),
    # several M tiles, ragged tails, masked slots, skewed routing, K-steps 4
    dict(T=300, H=512, I=256, E=6, K=3, routing="zipf", seed=41, mask_p=0.1),
    # one expert, one slot: a dense FFN
    dict(T=97, H=256, I=128, E=1, K=1, routing="uniform", seed=42),
    # many experts, several empty, T not a multiple of anything
    dict(T=71, H=768, I=384, E=40, K=4, routing="zipf", seed=43, zipf_s=2.0, mask_p=0.05),
    # every slot of some tokens masked
    dict(T=64, H=256, I=128, E=4, K=2, routing="uniform", seed=44, mask_p=0.6),
    # the largest expert count (one scan thread per expert), most experts empty
    dict(T=200, H=256, I=128, E=1000, K=8, routing="zipf", seed=45, mask_p=0.02),
    # an expert count that is not a power of two (two scan threads per expert)
    dict(T=150, H=512, I=256, E=257, K=6, routing="uniform", seed=46),
    # the same expert twice in a token (each slot is its own route)
    dict(T=120, H=256, I=128, E=8, K=4, routing="uniform", seed=47, dup=True),
    # the largest top-k
    dict(T=40, H=256, I=128, E=96, K=64, routing="uniform", seed=48),
    # one token
    dict(T=1, H=512, I=256, E=4, K=2, routing="uniform", seed=49),
    # experts with 32, 33, 64, 65, 256 and 257 rows: narrow tiles with one
    # and two row tiles, the first full-mode short tile, one whole tile and
    # one row past it
    dict(T=707, H=256, I=128, E=6, K=1, routing="uniform", seed=50,
         counts=(32, 33, 64, 65, 256, 257)),
]
SMALL_IDS = ["tiny", "ragged", "dense", "sparse", "masked", "e1000", "e257", "dup", "k64", "t1",
             "tile_edges"]


def small_inputs(case):
    if "name" in case:
        return moe_inputs.config_inputs(case["name"])
    kw = {k: v for k, v in case.items() if k not in ("dup", "counts")}
    inp = moe_inputs.make_inputs(**kw)
    rng = np.random.default_rng(case["seed"])
    idx = inp["topk_idx"]
    if case.get("dup"):
        # every third token repeats its first expert in slot 1
        idx[::3, 1] = idx[::3, 0]
    if "counts" in case:
        # token t goes to the expert given by a seeded shuffle of the counts
        assert case["K"] == 1 and sum(case["counts"]) == case["T"]
        e = np.repeat(np.arange(len(case["counts"]), dtype=np.int64), case["counts"])
        idx[:, 0] = rng.permutation(e)
    return inp


@pytest.mark.parametrize("case", SMALL, ids=SMALL_IDS)
def test_forward_matches_oracle_small(case):
    inp = small_inputs(case)
    say("case", case)
    y_ref, mid = oracle.forward(inp, intermediates=True)
    y, ws = run_forward(inp)
    r, R = check_routing(inp, ws)
    # pool row r is token row pool_tok[r] of the quantised input
    ptok = view(ws, inp, "pool_tok", R)
    np.testing.assert_array_equal(ptok, r["pool_src"][:R] // inp["K"])
    np.testing.assert_array_equal(view(ws, inp, "x_q")[ptok], mid["pool_q"][:R])
    np.testing.assert_array_equal(view(ws, inp, "x_s")[ptok], mid["pool_s"][:R])
    np.testing.assert_array_equal(view(ws, inp, "pool_s", R), mid["pool_s"][:R])
    check_act(view(ws, inp, "act_q", R), view(ws, inp, "act_s", R), mid["act_q"][:R],
              mid["act_s"][:R])
    worst = check_y(y, y_ref, inp["topk_idx"])
    say("max rel l2", worst, "exact y fraction", float((y == y_ref).mean()))


def test_forward_is_deterministic():
    inp = small_inputs(SMALL[1])
    dev = to_dev(inp)
    y1, ws1 = run_forward(inp, dev)
    y2, ws2 = run_forward(inp, dev)
    np.testing.assert_array_equal(y1, y2)
    R = int(view(ws1, inp, "offsets")[-1])
    for name in ("pool_src", "pool_tok", "act_q", "act_s", "l2_out"):  # rows past R are scratch
        np.testing.assert_array_equal(view(ws1, inp, name, R), view(ws2, inp, name, R))
    np.testing.assert_array_equal(view(ws1, inp, "x_q"), view(ws2, inp, "x_q"))


# ----------------------------------------------------------------------------
# dispatch and combine entry points on their own
# ----------------------------------------------------------------------------
# blocks of 23 tokens (H = 352) and of 4 (H = 2048), one token over several
# chunks (H = 7168), the largest top-k, one token
DISPATCH_CASES = [dict(T=513, H=352, E=13, K=5, routing="zipf", mask_p=0.1),
                  dict(T=300, H=2048, E=16, K=8, routing="uniform"),
                  dict(T=40, H=7168, E=32, K=8, routing="uniform"),
                  dict(T=9, H=256, E=96, K=64, routing="uniform"),
                  dict(T=1, H=512, E=4, K=2, routing="uniform")]


@pytest.mark.parametrize("case", DISPATCH_CASES,
                         ids=["h352", "h2048", "h7168", "k64", "t1"])
@pytest.mark.parametrize("payload", [0, 1], ids=["fp8", "bf16"])
def test_dispatch_entry_matches_oracle(payload, case):
    import combine_dispatch_amd as moe
    inp = moe_inputs.make_inputs(I=32, seed=51, weights=False, **case)
    T, H, E, K = inp["T"], inp["H"], inp["E"], inp["K"]
    ref = oracle.dispatch(inp["x"], inp["topk_idx"], inp["topk_w"], E, payload)
    dev = to_dev(inp)
    i32 = dict(dtype=torch.int32, device=DEV)
    counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    pool_src, s2p = torch.full((T * K,), -7, **i32), torch.empty(T * K, **i32)
    pool_w = torch.empty(T * K, dtype=torch.float32, device=DEV)
    pool = torch.empty((T * K, H), dtype=torch.uint8 if payload == 0 else torch.int16, device=DEV)
    scales = torch.empty((T * K, H // 32), dtype=torch.uint8, device=DEV) if payload == 0 else None
    ws = torch.empty(moe.moe_dispatch_workspace_bytes(T, H, E, K), dtype=torch.uint8, device=DEV)
    moe.moe_dispatch(dev["x"], dev["topk_idx"], dev["topk_w"], E, payload, counts, offsets,
                     pool_src, s2p, pool_w, pool, scales, ws)
    torch.cuda.synchronize()
    R = int(ref["offsets"][-1])
    np.testing.assert_array_equal(counts.cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(offsets.cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(pool_src.cpu().numpy()[:R], ref["pool_src"][:R])
    np.testing.assert_array_equal(s2p.cpu().numpy(), ref["slot_to_pool"])
    np.testing.assert_array_equal(pool_w.cpu().numpy()[:R], ref["pool_w"][:R])
    got = pool.cpu().numpy()[:R]
    if payload == 1:
        got = got.view(np.uint16)
    np.testing.assert_array_equal(got, ref["pool"][:R])
    if payload == 0:
        np.testing.assert_array_equal(scales.cpu().numpy()[:R], ref["pool_scales"][:R])


@pytest.mark.parametrize("name", ["tiny", "small", "prefill", "skewed", "many"])
def test_dispatch_entry_on_workloads(name):
    """moe_dispatch (FP8 payload) on the five workloads at full size: routing
    arrays, pool codes and pool scale bytes bit-exact against the oracle."""
    import combine_dispatch_amd as moe
    say("dispatch", name)
    inp = moe_inputs.config_inputs(name)
    T, H, E, K = inp["T"], inp["H"], inp["E"], inp["K"]
    ref = oracle.dispatch(inp["x"], inp["topk_idx"], inp["topk_w"], E, 0)
    dev = to_dev({k: inp[k] for k in ("x", "topk_idx", "topk_w")})
    i32 = dict(dtype=torch.int32, device=DEV)
    counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    pool_src, s2p = torch.empty(T * K, **i32), torch.empty(T * K, **i32)
    pool_w = torch.empty(T * K, dtype=torch.float32, device=DEV)
    pool = torch.empty((T * K, H), dtype=torch.uint8, device=DEV)
    scales = torch.empty((T * K, H // 32), dtype=torch.uint8, device=DEV)
    ws = torch.empty(moe.moe_dispatch_workspace_bytes(T, H, E, K), dtype=torch.uint8, device=DEV)
    moe.moe_dispatch(dev["x"], dev["topk_idx"], dev["topk_w"], E, 0, counts, offsets, pool_src,
                     s2p, pool_w, pool, scales, ws)
    torch.cuda.synchronize()
    R = int(ref["offsets"][-1])
    np.testing.assert_array_equal(counts.cpu().numpy(), ref["counts"])
    np.testing.assert_array_equal(offsets.cpu().numpy(), ref["offsets"])
    np.testing.assert_array_equal(pool_src.cpu().numpy()[:R], ref["pool_src"][:R])
    np.testing.assert_array_equal(s2p.cpu().numpy(), ref["slot_to_pool"])
    np.testing.assert_array_equal(pool_w.cpu().numpy()[:R], ref["pool_w"][:R])
    np.testing.assert_array_equal(pool.cpu().numpy()[:R], ref["pool"][:R])
    np.testing.assert_array_equal(scales.cpu().numpy()[:R], ref["pool_scales"][:R])
    say(name, "dispatch bit-exact, R =", R)


# (T, H, K): blocks of 8, 4, 2, 1 and 32 tokens with a ragged last block, a
# partly used chunk (H = 3072), and a row longer than one pass (H = 16384).
COMBINE_SHAPES = [(777, 1024, 8), (1001, 2048, 8), (333, 3072, 6), (65, 7168, 8), (130, 40, 64),
                  (17, 16384, 3)]


@pytest.mark.parametrize("shape", COMBINE_SHAPES, ids=lambda s: "T%d_H%d_K%d" % s)
@pytest.mark.parametrize("weighted", [False, True])
def test_combine_entry_bit_exact(weighted, shape):
    import combine_dispatch_amd as moe
    T, H, K = shape
    rng = np.random.default_rng(61 + H)
    R = T * K
    o = (rng.standard_normal((R, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    s2p = rng.permutation(R).astype(np.int32)
    s2p[rng.random(R) < 0.2] = -1
    s2p[:K] = -1  # token 0 fully masked
    w = rng.random((T, K)).astype(np.float32)
    ref = oracle.combine(o, s2p, T, K, w if weighted else None)
    y = torch.empty((T, H), dtype=torch.int16, device=DEV)
    moe.moe_combine(torch.from_numpy(o.view(np.int16)).to(DEV), torch.from_numpy(s2p).to(DEV), T,
                    K, y, torch.from_numpy(w).to(DEV) if weighted else None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_bits(y), ref)


def test_dispatch_then_combine_identity_k1():
    """K = 1, bf16 payload, no expert in between: combine returns x exactly."""
    import combine_dispatch_amd as moe
    inp = moe_inputs.make_inputs(T=1000, H=2048, I=32, E=16, K=1, routing="uniform", seed=62,
                                 weights=False)
    T, H, E, K = 1000, 2048, 16, 1
    dev = to_dev(inp)
    i32 = dict(dtype=torch.int32, device=DEV)
    counts, offsets = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    pool_src, s2p = torch.empty(T * K, **i32), torch.empty(T * K, **i32)
    pool_w = torch.empty(T * K, dtype=torch.float32, device=DEV)
    pool = torch.empty((T * K, H), dtype=torch.int16, device=DEV)
    ws = torch.empty(moe.moe_dispatch_workspace_bytes(T, H, E, K), dtype=torch.uint8, device=DEV)
    moe.moe_dispatch(dev["x"], dev["topk_idx"], dev["topk_w"], E, 1, counts, offsets, pool_src,
                     s2p, pool_w, pool, None, ws)
    y = torch.empty((T, H), dtype=torch.int16, device=DEV)
    moe.moe_combine(pool, s2p, T, K, y)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_bits(y), inp["x"])


# ----------------------------------------------------------------------------
# edge cases and error conventions
# ----------------------------------------------------------------------------
def test_edge_empty_and_all_masked():
    inp = moe_inputs.make_inputs(T=0, H=256, I=128, E=4, K=2, routing="uniform", seed=1)
    y, _ = run_forward(inp)
    assert y.shape == (0, 256)
    inp = moe_inputs.make_inputs(T=37, H=256, I=128, E=4, K=2, routing="uniform", seed=1,
                                 mask_p=1.0)
    y, ws = run_forward(inp)
    assert (y == 0).all()
    assert (view(ws, inp, "counts") == 0).all()


def test_errors_are_reported():
    import combine_dispatch_amd as moe
    inp = moe_inputs.make_inputs(T=16, H=256, I=128, E=4, K=2, routing="uniform", seed=2)
    bad = dict(inp)
    bad["topk_idx"] = inp["topk_idx"].copy()
    bad["topk_idx"][3, 1] = 4  # == E
    with pytest.raises(moe.MoeError) as ei:
        run_forward(bad, opts=moe.options(debug_validate=True))
    assert ei.value.status == moe.MOE_ERR_BAD_ROUTING
    # the same call without validation treats the slot as masked and does not fault
    y, ws = run_forward(bad)
    assert view(ws, bad, "slot_to_pool")[3 * 2 + 1] == -1
    small = torch.empty(1024, dtype=torch.uint8, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        run_forward(inp, workspace=small)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
    with pytest.raises(moe.MoeError) as ei:
        run_forward(inp, opts=moe.options(activation_clamp=7.0))
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED
    odd = moe_inputs.make_inputs(T=8, H=128, I=128, E=2, K=1, routing="uniform", seed=3)
    with pytest.raises(moe.MoeError) as ei:
        run_forward(odd)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("case", [SMALL[1], SMALL[6]], ids=["ragged", "e257"])
def test_packed_weight_scales(case):
    """moe_pack_weight_scales writes the documented layout (S1's words then,
    from the next 256-byte boundary, S2's; per expert and 128-wide K step one
    word per weight row with the k-blocks in byte order 0, 2, 1, 3), and the
    packed forward equals the canonical one bit for bit."""
    import combine_dispatch_amd as moe
    inp = small_inputs(case)
    T, H, I, E, K = (inp[k] for k in ("T", "H", "I", "E", "K"))
    dev = to_dev(inp)
    nbytes = moe.moe_packed_scales_bytes(H, I, E)
    packed = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    moe.moe_pack_weight_scales(dev["S1"], dev["S2"], packed, E=E, H=H, I=I)
    raw = packed.cpu().numpy()

    def unpack(words, N, kdim):
        nw = kdim // 128
        w = words.reshape(E, nw, N, 4)[:, :, :, [0, 2, 1, 3]]
        return np.ascontiguousarray(w.transpose(0, 2, 1, 3).reshape(E, N, kdim // 32))

    s1 = E * 2 * I * (H // 32)
    off2 = (s1 + 255) // 256 * 256
    np.testing.assert_array_equal(unpack(raw[:s1], 2 * I, H), inp["S1"])
    np.testing.assert_array_equal(unpack(raw[off2:off2 + E * H * (I // 32)], H, I), inp["S2"])

    y_ref, ws_ref = run_forward(inp, dev)
    ws = torch.empty(moe.moe_workspace_bytes(T, H, I, E, K), dtype=torch.uint8, device=DEV)
    y = torch.empty((T, H), dtype=torch.int16, device=DEV)
    moe.moe_fused_forward_packed(dev["x"], dev["topk_idx"], dev["topk_w"], dev["W1q"],
                                 dev["W2q"], packed, y, ws, E=E, I=I)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_bits(y), y_ref)
    R = int(view(ws_ref, inp, "offsets")[-1])
    for name in ("act_q", "act_s", "l2_out"):
        np.testing.assert_array_equal(view(ws, inp, name, R), view(ws_ref, inp, name, R))
    short = torch.empty(nbytes - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_pack_weight_scales(dev["S1"], dev["S2"], short, E=E, H=H, I=I)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE


def test_exact_math_option_also_within_tolerance():
    import combine_dispatch_amd as moe
    inp = small_inputs(SMALL[1])
    y_ref = oracle.forward(inp)
    y, _ = run_forward(inp, opts=moe.options(fast_math=False))
    check_y(y, y_ref, inp["topk_idx"])


# ----------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark times
# ----------------------------------------------------------------------------
FULL = ["small", "prefill", "skewed", "many"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(name):
    say("generating", name)
    inp = moe_inputs.config_inputs(name)
    say("running", name, {k: inp[k] for k in "THIEK"})
    y, ws = run_forward(inp)
    r, R = check_routing(inp, ws)
    say("routing bit-exact, R =", R)
    # the quantised token rows behind sampled pool rows against the oracle
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([rng.integers(0, R, 256), [0, R - 1]]))
    K, H = inp["K"], inp["H"]
    ptok = view(ws, inp, "pool_tok", R)
    np.testing.assert_array_equal(ptok, r["pool_src"][:R] // K)
    xq, xs = view(ws, inp, "x_q"), view(ws, inp, "x_s")
    for rr in rows:
        t = r["pool_src"][rr] // K
        q, s = oracle.quant_e4m3_row(oracle.bf16_to_f32(inp["x"][t]))
        np.testing.assert_array_equal(xq[t], q)
        np.testing.assert_array_equal(xs[t], s)
    # y on sampled tokens (including any fully masked one) against brute force
    masked = np.nonzero((inp["topk_idx"] < 0).all(axis=1))[0][:2]
    toks = np.unique(np.concatenate([rng.integers(0, inp["T"], 6), [0, inp["T"] - 1], masked]))
    ref, aq, as_ = oracle.forward_tokens(inp, toks.astype(np.int32), activations=True)
    worst = check_y(y[toks], ref, inp["topk_idx"][toks])
    say(name, "sampled tokens", len(toks), "max rel l2", worst)
    # the L1 epilogue's e4m3 activations of those tokens' routes, at their pool rows
    s2p = view(ws, inp, "slot_to_pool").reshape(inp["T"], K)[toks]
    valid = s2p >= 0
    check_act(view(ws, inp, "act_q", R)[s2p[valid]], view(ws, inp, "act_s", R)[s2p[valid]],
              aq[valid], as_[valid])
    say(name, "sampled routes' activations within the FP8 rule:", int(valid.sum()))
    # the benchmark times the packed-scale entry: same y, bit for bit
    import combine_dispatch_amd as moe
    T, I, E = inp["T"], inp["I"], inp["E"]
    dev = to_dev(inp)
    packed = torch.empty(moe.moe_packed_scales_bytes(H, I, E), dtype=torch.uint8, device=DEV)
    moe.moe_pack_weight_scales(dev["S1"], dev["S2"], packed, E=E, H=H, I=I)
    yp = torch.empty((T, H), dtype=torch.int16, device=DEV)
    moe.moe_fused_forward_packed(dev["x"], dev["topk_idx"], dev["topk_w"], dev["W1q"],
                                 dev["W2q"], packed, yp, ws, E=E, I=I)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_bits(yp), y)
    say(name, "packed-scale entry bit-identical")
