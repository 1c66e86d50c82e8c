"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

Bars (routing and dispatch are integer/byte work, the rest floating point):
  - counts, offsets, pool_src, slot_to_pool, pool_w, the token of each pool
    row, and the quantised token rows (codes and scale bytes) the L1 GEMM
    gathers its pool rows from: bit-exact;
  - combine fed identical bf16 rows: bit-exact (same summation order);
  - intermediate FP8 activations after L1, the L2 rows (against the oracle's
    L2 of the GPU's own activations) and y: the bars in
    tests/parity_checks.py; y also equals the oracle's combine of the GPU's
    L2 rows bit for bit.
"""
import os

import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from tests.gpu_util import DEV, bf16_bits, run_forward, to_dev, uses_decode_path, view
from tests.parity_checks import check_act, check_l2_rows, check_y, l1_slack, rel_l2_rows

pytestmark = pytest.mark.gpu


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
    # few rows per expert (the decode-shaped GEMMs, 64-row tiles): experts of
    # 1, 2, 20, 40, 64, 65 and 128 rows and an empty one, K loops of 6 and 3
    dict(T=320, H=768, I=384, E=8, K=1, routing="uniform", seed=51,
         counts=(64, 65, 1, 128, 2, 0, 40, 20)),
]
SMALL_IDS = ["tiny", "ragged", "dense", "sparse", "masked", "e1000", "e257", "dup", "k64", "t1",
             "tile_edges", "decode_edges"]


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
    T, K = inp["T"], inp["K"]
    y_ref, mid = oracle.forward(inp, intermediates=True)
    y, ws = run_forward(inp)
    r, R = check_routing(inp, ws)
    # pool row r is token row pool_tok[r] of the quantised input
    ptok = view(ws, inp, "pool_tok", R)
    np.testing.assert_array_equal(ptok, r["pool_src"][:R] // inp["K"])
    np.testing.assert_array_equal(view(ws, inp, "x_q")[ptok], mid["pool_q"][:R])
    np.testing.assert_array_equal(view(ws, inp, "x_s")[ptok], mid["pool_s"][:R])
    if not uses_decode_path(inp):
        np.testing.assert_array_equal(view(ws, inp, "pool_s", R), mid["pool_s"][:R])
    gq, gs = view(ws, inp, "act_q", R), view(ws, inp, "act_s", R)
    experts = np.searchsorted(r["offsets"], np.arange(R), side="right") - 1
    slack = l1_slack(inp, experts, ptok, r["pool_w"][:R], mid["h1"][:R])
    ncode, nscale, worst_steps = check_act(gq, gs, mid["act_q"][:R], mid["act_s"][:R], gemm_slack=slack)
    # L2 rows against the oracle's L2 of the GPU's own activations
    l2 = view(ws, inp, "l2_out", R)
    nl2, _ = check_l2_rows(inp, experts, l2, oracle.l2_rows(inp, experts, gq, gs), gq, gs)
    # combine of the GPU's L2 rows: bit-exact
    np.testing.assert_array_equal(y, oracle.combine(l2, r["slot_to_pool"], T, K))
    worst = check_y(y, y_ref, inp["topk_idx"])
    # the worst token, explained: how many of its routes' activation codes
    # moved (one e4m3 step in a row of I values moves that route's L2 row by
    # about 2^-4 / sqrt(I) of its norm; with K = 1 nothing averages it out)
    rel = rel_l2_rows(y, y_ref)
    t = int(np.argmax(rel))
    slots = r["slot_to_pool"].reshape(T, K)[t]
    moved = [int((gq[s] != mid["act_q"][s]).sum() + (gs[s] != mid["act_s"][s]).sum())
             for s in slots if s >= 0]
    say(f"max rel l2 {worst:.2e} (token {t}: codes or scales moved per route {moved}); "
        f"act codes off {ncode} (largest move {worst_steps:.2f} steps), scales moved {nscale}, "
        f"L2 elements not identical {nl2}; "
        f"exact y fraction {float((y == y_ref).mean()):.4f}")


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


# Every GEMM kernel family (gemm_tiles: persistent 256-row tiles, 64- and
# 128-row tiles with one workgroup each) accumulates each output in the same
# K order with the same MFMA blocks, so all give the same bits.  The cases:
# several tiles per expert with ragged tails and masked slots, the narrow
# tile edges (32/33/64/65/256/257 rows), the decode edges (1..128 rows, an
# empty expert), many experts mostly empty, one token, the largest top-k.
TILE_CASES = [SMALL[1], SMALL[10], SMALL[11], SMALL[3], SMALL[9], SMALL[8],
              dict(T=1000, H=1024, I=512, E=5, K=2, routing="zipf", seed=52, mask_p=0.05)]
TILE_IDS = ["ragged", "tile_edges", "decode_edges", "sparse", "t1", "k64", "multi"]


@pytest.mark.parametrize("case", TILE_CASES, ids=TILE_IDS)
def test_gemm_tile_kernels_agree(case):
    import combine_dispatch_amd as moe
    inp = small_inputs(case)
    say("case", case)
    dev = to_dev(inp)
    outs = {}
    for tiles in (moe.MOE_TILES_PERSISTENT, moe.MOE_TILES_64, moe.MOE_TILES_128, moe.MOE_TILES_AUTO):
        say("gemm_tiles", tiles)
        y, ws = run_forward(inp, dev, opts=moe.options(gemm_tiles=tiles))
        R = int(view(ws, inp, "offsets")[-1])
        outs[tiles] = (y, {n: view(ws, inp, n, R) for n in ("act_q", "act_s", "l2_out")})
    y0, m0 = outs[moe.MOE_TILES_PERSISTENT]
    for tiles, (y, m) in outs.items():
        for n in m0:
            np.testing.assert_array_equal(m[n], m0[n], err_msg=f"{n}, gemm_tiles {tiles}")
        np.testing.assert_array_equal(y, y0, err_msg=f"y, gemm_tiles {tiles}")
    # L1 and L2 in one launch (activations kept in LDS, so the workspace's
    # act_q / act_s are not written): the same L2 rows and y
    if inp["I"] <= 768:
        say("gemm_tiles fused")
        y, ws = run_forward(inp, dev, opts=moe.options(gemm_tiles=moe.MOE_TILES_FUSED))
        R = int(view(ws, inp, "offsets")[-1])
        np.testing.assert_array_equal(view(ws, inp, "l2_out", R), m0["l2_out"], err_msg="l2_out, fused")
        np.testing.assert_array_equal(y, y0, err_msg="y, fused")
    # and the common result is the oracle's, to the layer's bars
    y_ref = oracle.forward(inp)
    check_y(y0, y_ref, inp["topk_idx"])


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


def tile_blocked(W, l1: bool, I: int) -> np.ndarray:
    """The documented tile-blocked layout of weight codes W [E][N][K/2]: per
    expert, 256-row n-tile (L1: 128 gate rows then the 128 matching up rows)
    and 128-wide K step, one block of 256 rows x 64 bytes."""
    E, N, kb = W.shape
    nk, nt = kb // 64, N // 256
    if l1:
        rows = np.concatenate([np.concatenate([np.arange(128 * t, 128 * t + 128),
                                               I + np.arange(128 * t, 128 * t + 128)]) for t in range(nt)])
    else:
        rows = np.arange(N)
    Wr = W[:, rows, :].reshape(E, nt, 256, nk, 64)
    return np.ascontiguousarray(Wr.transpose(0, 1, 3, 2, 4)).reshape(-1)


PREPACK_CASES = [SMALL[1], SMALL[10], SMALL[11], SMALL[6], TILE_CASES[6]]


@pytest.mark.parametrize("case", PREPACK_CASES, ids=["ragged", "tile_edges", "decode_edges", "e257", "multi"])
def test_prepacked_weights(case):
    """moe_pack_weights writes the documented layout (W1's blocks, W2's from
    the next 256-byte boundary, then the packed scales), and the prepacked
    forward equals the canonical one bit for bit with every GEMM kernel."""
    import combine_dispatch_amd as moe
    inp = small_inputs(case)
    say("case", case)
    T, H, I, E, K = (inp[k] for k in ("T", "H", "I", "E", "K"))
    dev = to_dev(inp)
    nbytes = moe.moe_packed_weights_bytes(H, I, E)
    packed = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    moe.moe_pack_weights(dev["W1q"], dev["S1"], dev["W2q"], dev["S2"], packed, E=E, H=H, I=I)
    raw = packed.cpu().numpy()
    w1 = E * 2 * I * (H // 2)
    off2 = (w1 + 255) // 256 * 256
    w2 = E * H * (I // 2)
    offs = off2 + (w2 + 255) // 256 * 256
    np.testing.assert_array_equal(raw[:w1], tile_blocked(inp["W1q"], True, I))
    np.testing.assert_array_equal(raw[off2:off2 + w2], tile_blocked(inp["W2q"], False, I))
    sc = torch.empty(moe.moe_packed_scales_bytes(H, I, E), dtype=torch.uint8, device=DEV)
    moe.moe_pack_weight_scales(dev["S1"], dev["S2"], sc, E=E, H=H, I=I)
    np.testing.assert_array_equal(raw[offs:offs + sc.numel()], sc.cpu().numpy())
    y_ref, ws_ref = run_forward(inp, dev)
    R = int(view(ws_ref, inp, "offsets")[-1])
    for tiles in (moe.MOE_TILES_AUTO, moe.MOE_TILES_PERSISTENT, moe.MOE_TILES_64):
        say("gemm_tiles", tiles)
        ws = torch.empty(moe.moe_workspace_bytes(T, H, I, E, K), dtype=torch.uint8, device=DEV)
        y = torch.empty((T, H), dtype=torch.int16, device=DEV)
        moe.moe_fused_forward_prepacked(dev["x"], dev["topk_idx"], dev["topk_w"], packed, y, ws, E=E, I=I,
                                        opts=moe.options(gemm_tiles=tiles))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bf16_bits(y), y_ref)
        for name in ("act_q", "act_s", "l2_out"):
            np.testing.assert_array_equal(view(ws, inp, name, R), view(ws_ref, inp, name, R))
    if I <= 768:
        say("gemm_tiles fused")
        ws = torch.empty(moe.moe_workspace_bytes(T, H, I, E, K), dtype=torch.uint8, device=DEV)
        y = torch.empty((T, H), dtype=torch.int16, device=DEV)
        moe.moe_fused_forward_prepacked(dev["x"], dev["topk_idx"], dev["topk_w"], packed, y, ws, E=E, I=I,
                                        opts=moe.options(gemm_tiles=moe.MOE_TILES_FUSED))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bf16_bits(y), y_ref)
        np.testing.assert_array_equal(view(ws, inp, "l2_out", R), view(ws_ref, inp, "l2_out", R))
    short = torch.empty(nbytes - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_pack_weights(dev["W1q"], dev["S1"], dev["W2q"], dev["S2"], short, E=E, H=H, I=I)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE


def test_exact_math_option_also_within_tolerance():
    import combine_dispatch_amd as moe
    inp = small_inputs(SMALL[1])
    y_ref = oracle.forward(inp)
    y, ws = run_forward(inp, opts=moe.options(fast_math=False))
    check_y(y, y_ref, inp["topk_idx"])
    # every GEMM kernel family takes the same exact-math epilogue: the same bits
    R = int(view(ws, inp, "offsets")[-1])
    l2 = view(ws, inp, "l2_out", R).copy()
    dev = to_dev(inp)
    for tiles in (moe.MOE_TILES_PERSISTENT, moe.MOE_TILES_64, moe.MOE_TILES_128, moe.MOE_TILES_FUSED):
        say("gemm_tiles", tiles)
        yt, wt = run_forward(inp, dev, opts=moe.options(fast_math=False, gemm_tiles=tiles))
        np.testing.assert_array_equal(yt, y, err_msg=f"y, exact math, gemm_tiles {tiles}")
        np.testing.assert_array_equal(view(wt, inp, "l2_out", R), l2, err_msg=f"l2_out, gemm_tiles {tiles}")
