"""Pins of the oracle's routing, dispatch, combine and whole layer.

Each check compares the oracle with something other than itself: numpy's
stable sort and bincount, closed forms of dispatch->combine, an independent
implementation of the layer built from torch CPU library routines (float8
casts, bf16 casts, fp64 matmul), brute force per token, and the pages'
worked example of a token's output as the weighted sum of two experts'
outputs (page "Dispatch/Combine in Mega MoE", section 4.2)."""
import numpy as np
import pytest
import torch

import moe_inputs
import oracle

from tests.golden_util import e2m1_table


# ----------------------------------------------------------------------------
# routing (a1-a3)
# ----------------------------------------------------------------------------
ROUTING_CASES = [
    dict(T=64, E=8, K=2, routing="softmax_topk", seed=0),
    dict(T=300, E=32, K=8, routing="uniform", seed=1),
    dict(T=257, E=16, K=4, routing="zipf", seed=3, mask_p=0.2),
    dict(T=50, E=5, K=3, routing="all_to_zero", seed=4, mask_p=0.5),
    dict(T=33, E=7, K=1, routing="uniform", seed=6, mask_p=1.0),  # everything masked
]


@pytest.mark.parametrize("case", ROUTING_CASES, ids=lambda c: f"{c['routing']}-T{c['T']}")
def test_route_matches_stable_sort(case):
    c = dict(case)
    T, E, K = c.pop("T"), c.pop("E"), c.pop("K")
    idx, w = moe_inputs.make_routing(T, E, K, c.pop("routing"), c.pop("seed"), **c)
    r = oracle.route(idx, w, E)
    flat = idx.ravel()
    valid = flat >= 0
    R = int(valid.sum())
    # counts and offsets
    np.testing.assert_array_equal(r["counts"], np.bincount(flat[valid], minlength=E))
    assert r["counts"].sum() == R and r["offsets"][0] == 0 and r["offsets"][E] == R
    assert (np.diff(r["offsets"]) == r["counts"]).all()
    # pool order = stable sort of valid slots by expert
    order = np.nonzero(valid)[0][np.argsort(flat[valid], kind="stable")]
    np.testing.assert_array_equal(r["pool_src"][:R], order)
    np.testing.assert_array_equal(r["pool_w"][:R], w.ravel()[order])
    # slot_to_pool is the inverse permutation, -1 on masked slots
    s2p = r["slot_to_pool"]
    assert (s2p[~valid] == -1).all()
    np.testing.assert_array_equal(s2p[order], np.arange(R))


def test_route_rejects_out_of_range_expert():
    idx = np.array([[0, 3]], np.int64)
    with pytest.raises(ValueError):
        oracle.route(idx, np.ones((1, 2), np.float32), 3)


# ----------------------------------------------------------------------------
# dispatch -> combine closed forms (a4, a9)
# ----------------------------------------------------------------------------
def _bf16_from_torch(t):
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_to_torch(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def test_dispatch_bf16_then_combine_k1_is_identity():
    inp = moe_inputs.make_inputs(T=70, H=64, I=32, E=6, K=1, routing="uniform", seed=8, weights=False)
    d = oracle.dispatch(inp["x"], inp["topk_idx"], inp["topk_w"], 6, payload=1)
    y = oracle.combine(d["pool"], d["slot_to_pool"], 70, 1)
    np.testing.assert_array_equal(y, inp["x"])


def test_dispatch_bf16_then_combine_counts_copies():
    """Unweighted combine of m identical bf16 rows is bf16(m * x): the fp32
    sums are exact, so only the final rounding matters."""
    T, H, E, K = 90, 96, 16, 8
    inp = moe_inputs.make_inputs(T=T, H=H, I=32, E=E, K=K, routing="uniform", seed=9,
                                 weights=False, mask_p=0.3)
    d = oracle.dispatch(inp["x"], inp["topk_idx"], inp["topk_w"], E, payload=1)
    y = oracle.combine(d["pool"], d["slot_to_pool"], T, K)
    m = (inp["topk_idx"] >= 0).sum(axis=1).astype(np.float32)
    ref = _bf16_from_torch(_bf16_to_torch(inp["x"]).float() * torch.from_numpy(m)[:, None])
    np.testing.assert_array_equal(y, ref)
    zero_rows = m == 0
    assert (y[zero_rows] == 0).all()  # all-masked token -> +0


def test_combine_weighted_sums_in_slot_order():
    T, H, K = 40, 64, 4
    rng = np.random.default_rng(2)
    o = _bf16_from_torch(torch.from_numpy(rng.standard_normal((T * K, H)).astype(np.float32)))
    s2p = rng.permutation(T * K).astype(np.int32)
    s2p[rng.random(T * K) < 0.25] = -1
    w = rng.random((T, K)).astype(np.float32)
    y = oracle.combine(o, s2p, T, K, w)
    of = _bf16_to_torch(o).float()
    acc = torch.zeros((T, H), dtype=torch.float32)
    for k in range(K):
        rows = torch.from_numpy(s2p.reshape(T, K)[:, k].astype(np.int64))
        ok = rows >= 0
        term = of[rows.clamp(min=0)] * torch.from_numpy(w[:, k])[:, None]
        acc = torch.where(ok[:, None], acc + term, acc)
    np.testing.assert_array_equal(y, _bf16_from_torch(acc))


def test_dispatch_fp8_pool_rows_are_quantised_token_rows():
    T, H, E, K = 48, 128, 8, 3
    inp = moe_inputs.make_inputs(T=T, H=H, I=32, E=E, K=K, routing="uniform", seed=10, weights=False)
    d = oracle.dispatch(inp["x"], inp["topk_idx"], inp["topk_w"], E, payload=0)
    xt = _bf16_to_torch(inp["x"]).float()
    codes, b, _ = torch_quant_e4m3(xt)
    R = d["offsets"][E]
    tok = d["pool_src"][:R] // K
    np.testing.assert_array_equal(d["pool"][:R], codes.numpy()[tok])
    np.testing.assert_array_equal(d["pool_scales"][:R], b.numpy().astype(np.uint8)[tok])


# ----------------------------------------------------------------------------
# the layer, rebuilt from torch library routines
# ----------------------------------------------------------------------------
def torch_quant_e4m3(v: torch.Tensor):
    """Groups of 32 along the last dim: scale byte from the fp32 fields of the
    group amax (smallest power of two with amax <= 448 * scale), codes by
    torch's float8_e4m3fn cast of v / scale.  Returns codes (uint8), scale
    bytes (int64) and the dequantised values (float64)."""
    g = v.float().reshape(*v.shape[:-1], -1, 32)
    amax = g.abs().amax(-1)
    bits = amax.view(torch.int32).long()
    ef, mf = (bits >> 23) & 0xFF, bits & 0x7FFFFF
    b = (ef - 8 + (mf > 0x600000).long()).clamp(0, 254)
    scaled = (g.double() * torch.exp2((127 - b).double()).unsqueeze(-1)).float()
    f8 = scaled.to(torch.float8_e4m3fn)
    deq = f8.float().double() * torch.exp2((b - 127).double()).unsqueeze(-1)
    return (f8.view(torch.uint8).reshape(v.shape), b, deq.reshape(v.shape))


def torch_dequant_fp4(Wq: np.ndarray, S: np.ndarray) -> torch.Tensor:
    """[N][K/2] packed e2m1 + [N][K/32] scale bytes -> float64 [N][K]."""
    table = torch.tensor([e2m1_table()[c] for c in range(16)], dtype=torch.float64)
    q = torch.from_numpy(Wq.astype(np.int64))
    codes = torch.stack([q & 0xF, q >> 4], dim=-1).reshape(Wq.shape[0], -1)
    scale = torch.exp2(torch.from_numpy(S.astype(np.float64)) - 127)
    return table[codes] * scale.repeat_interleave(32, dim=1)


def torch_layer(inp):
    T, H, I, E, K = (inp[k] for k in ("T", "H", "I", "E", "K"))
    x = _bf16_to_torch(inp["x"]).float()
    _, _, xd = torch_quant_e4m3(x)
    idx = torch.from_numpy(inp["topk_idx"])
    w = torch.from_numpy(inp["topk_w"])
    y_acc = torch.zeros((T, H), dtype=torch.float32)
    h1_rows, act_rows = {}, {}
    for k in range(K):  # slot order, as the combine sums
        o_k = torch.zeros((T, H), dtype=torch.float32)
        for e in range(E):
            rows = torch.nonzero(idx[:, k] == e).flatten()
            if rows.numel() == 0:
                continue
            W1 = torch_dequant_fp4(inp["W1q"][e], inp["S1"][e])
            W2 = torch_dequant_fp4(inp["W2q"][e], inp["S2"][e])
            h = (xd[rows] @ W1.T).float().to(torch.bfloat16).float()
            g, u = h[:, :I], h[:, I:]
            a = (g / (1.0 + torch.exp(-g)) * u) * w[rows, k][:, None]
            codes, _, ad = torch_quant_e4m3(a)
            o = (ad @ W2.T).float().to(torch.bfloat16).float()
            o_k[rows] = o
            for j, t in enumerate(rows.tolist()):
                h1_rows[(t, k)] = h[j]
                act_rows[(t, k)] = codes[j]
        valid = (idx[:, k] >= 0)[:, None]
        y_acc = torch.where(valid, y_acc + o_k, y_acc)
    return _bf16_from_torch(y_acc), h1_rows, act_rows


LAYER_CASES = [
    dict(name="tiny"),
    dict(T=40, H=128, I=96, E=4, K=3, routing="zipf", seed=12, mask_p=0.15),
    dict(T=16, H=64, I=64, E=1, K=1, routing="uniform", seed=13),  # a dense FFN
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=["tiny", "masked", "dense"])
def test_layer_matches_torch_library_rebuild(case):
    inp = (moe_inputs.config_inputs(case["name"]) if "name" in case
           else moe_inputs.make_inputs(**case))
    T, K, I = inp["T"], inp["K"], inp["I"]
    if case.get("E") == 1:
        inp["topk_w"][:] = 1.0
    y, mid = oracle.forward(inp, intermediates=True)
    y_ref, h1_ref, act_ref = torch_layer(inp)
    s2p = mid["slot_to_pool"]
    n_code_diff = n_codes = 0
    for (t, k), h in h1_ref.items():
        r = s2p[t * K + k]
        # L1 is an exact dot product rounded fp64 -> fp32 -> bf16 on both sides
        np.testing.assert_array_equal(oracle.bf16_to_f32(mid["h1"][r]), h.numpy())
        n_codes += I
        n_code_diff += int((mid["act_q"][r] != act_ref[(t, k)].numpy()).sum())
    # exp() may differ by an ulp between libm and torch: only rare codes may move
    assert n_code_diff <= max(2, n_codes // 10000), (n_code_diff, n_codes)
    yf, rf = oracle.bf16_to_f32(y).astype(np.float64), oracle.bf16_to_f32(y_ref).astype(np.float64)
    rel = np.linalg.norm(yf - rf, axis=1) / np.maximum(np.linalg.norm(rf, axis=1), 1e-30)
    assert rel.max() < 1e-2
    assert (y == y_ref).mean() > 0.99


def test_grouped_equals_per_token_brute_force():
    for inp in (moe_inputs.config_inputs("tiny"),
                moe_inputs.make_inputs(T=37, H=96, I=64, E=6, K=4, routing="zipf", seed=21,
                                       mask_p=0.3)):
        y, mid = oracle.forward(inp, intermediates=True)
        toks = np.arange(inp["T"], dtype=np.int32)
        yb, aq, as_ = oracle.forward_tokens(inp, toks, activations=True)
        np.testing.assert_array_equal(y, yb)
        # each slot's activation row equals the grouped path's at its pool row
        s2p = mid["slot_to_pool"].reshape(inp["T"], inp["K"])
        valid = s2p >= 0
        np.testing.assert_array_equal(aq[valid], mid["act_q"][s2p[valid]])
        np.testing.assert_array_equal(as_[valid], mid["act_s"][s2p[valid]])
        assert (aq[~valid] == 0).all()


def test_worked_example_two_experts_weighted_sum():
    """One token routed to experts 2 and 7 with weights 0.73 and 0.27: the
    layer output is the weighted sum of those two experts' outputs.  Checked
    against a float64 torch evaluation with no intermediate quantisation
    (input and weights quantised as given); the gap is the FP8/bf16
    rounding of the intermediates."""
    inp = moe_inputs.make_inputs(T=1, H=256, I=128, E=8, K=2, routing="uniform", seed=31)
    inp["topk_idx"][:] = np.array([[2, 7]])
    inp["topk_w"][:] = np.array([[0.73, 0.27]], np.float32)
    y = oracle.bf16_to_f32(oracle.forward(inp)[0]).astype(np.float64)
    x = _bf16_to_torch(inp["x"]).float()
    _, _, xd = torch_quant_e4m3(x)
    ref = torch.zeros(inp["H"], dtype=torch.float64)
    for e, wt in ((2, 0.73), (7, 0.27)):
        W1 = torch_dequant_fp4(inp["W1q"][e], inp["S1"][e])
        W2 = torch_dequant_fp4(inp["W2q"][e], inp["S2"][e])
        h = xd[0] @ W1.T
        g, u = h[:128], h[128:]
        ref += wt * ((g * torch.sigmoid(g) * u) @ W2.T)
    ref = ref.numpy()
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel < 0.05, rel
    # swapping the weights must move the output well beyond that rounding gap
    inp["topk_w"][:] = np.array([[0.27, 0.73]], np.float32)
    y2 = oracle.bf16_to_f32(oracle.forward(inp)[0]).astype(np.float64)
    assert np.linalg.norm(y2 - ref) / np.linalg.norm(ref) > 4 * rel


def test_forward_empty_and_fully_masked():
    inp = moe_inputs.make_inputs(T=0, H=64, I=32, E=4, K=2, routing="uniform", seed=1)
    assert oracle.forward(inp).shape == (0, 64)
    inp = moe_inputs.make_inputs(T=5, H=64, I=32, E=4, K=2, routing="uniform", seed=1, mask_p=1.0)
    assert (oracle.forward(inp) == 0).all()


# ----------------------------------------------------------------------------
# single-row entries (used to check chosen rows of full-size GPU runs)
# ----------------------------------------------------------------------------
def test_row_entries_equal_grouped_path():
    """oracle.l1_act_rows on each pool row's (token, expert, weight) and
    oracle.l2_rows on the grouped path's activation rows reproduce the
    grouped path's h1, act_q, act_s and L2 rows bit for bit."""
    inp = moe_inputs.make_inputs(T=45, H=160, I=96, E=5, K=3, routing="zipf", seed=23, mask_p=0.2)
    K, E = inp["K"], inp["E"]
    _, mid = oracle.forward(inp, intermediates=True)
    R = int(mid["offsets"][-1])
    experts = np.searchsorted(mid["offsets"], np.arange(R), side="right") - 1
    tokens = mid["pool_src"][:R] // K
    h1, aq, as_ = oracle.l1_act_rows(inp, experts, tokens, mid["pool_w"][:R], h1=True)
    np.testing.assert_array_equal(h1, mid["h1"][:R])
    np.testing.assert_array_equal(aq, mid["act_q"][:R])
    np.testing.assert_array_equal(as_, mid["act_s"][:R])
    o = oracle.l2_rows(inp, experts, mid["act_q"][:R], mid["act_s"][:R])
    np.testing.assert_array_equal(o, mid["o"][:R])
    assert 0 <= experts.min() and experts.max() < E


def test_row_entries_at_production_width_match_torch_fp64():
    """At the production widths (H = 7168 along L1's K, I = 2048 along L2's
    K), where the products' exponents spread furthest, the oracle's L1 rows
    equal torch's fp64 matmul of the dequantised operands rounded fp32 ->
    bf16, and its L2 rows on the oracle's own activations equal the same for
    L2: the exact-sum reading holds at these sizes too."""
    H, I = 7168, 2048
    inp = moe_inputs.make_inputs(T=6, H=H, I=I, E=2, K=2, routing="uniform", seed=24)
    experts = np.array([0, 1, 1, 0], np.int32)
    tokens = np.array([0, 3, 5, 2], np.int32)
    weights = np.array([0.61, 0.39, 1.0, 0.125], np.float32)
    h1, aq, as_ = oracle.l1_act_rows(inp, experts, tokens, weights, h1=True)
    o = oracle.l2_rows(inp, experts, aq, as_)
    x = _bf16_to_torch(inp["x"]).float()
    _, _, xd = torch_quant_e4m3(x)
    for e in (0, 1):
        sel = np.nonzero(experts == e)[0]
        W1 = torch_dequant_fp4(inp["W1q"][e], inp["S1"][e])
        h = (xd[torch.from_numpy(tokens[sel].astype(np.int64))] @ W1.T).float()
        np.testing.assert_array_equal(h1[sel], _bf16_from_torch(h))
        del W1
        W2 = torch_dequant_fp4(inp["W2q"][e], inp["S2"][e])
        ad = (torch.from_numpy(oracle.e4m3_to_f32(aq[sel]).astype(np.float64))
              * torch.exp2(torch.from_numpy(as_[sel].astype(np.float64)) - 127).repeat_interleave(32, dim=1))
        np.testing.assert_array_equal(o[sel], _bf16_from_torch((ad @ W2.T).float()))
        del W2
