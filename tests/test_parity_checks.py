"""The parity bars themselves (CPU): they accept the oracle's own rows and
reject plausible GPU mistakes, planted here in oracle-computed rows."""
import numpy as np
import pytest

import moe_inputs
import oracle
from tests.parity_checks import check_act, check_l2_rows, e4m3_step_at, l1_slack, mtile_sample_rows


@pytest.fixture(scope="module")
def rows():
    inp = moe_inputs.make_inputs(T=40, H=256, I=2048, E=3, K=2, routing="uniform", seed=81)
    r = oracle.route(inp["topk_idx"], inp["topk_w"], inp["E"])
    R = int(r["offsets"][-1])
    experts = np.searchsorted(r["offsets"], np.arange(R), side="right") - 1
    tokens = r["pool_src"][:R] // inp["K"]
    h1, aq, as_ = oracle.l1_act_rows(inp, experts, tokens, r["pool_w"][:R], h1=True)
    o = oracle.l2_rows(inp, experts, aq, as_)
    inp["_rows"] = (experts, tokens, r["pool_w"][:R], h1)
    return inp, experts, aq, as_, o


def test_l2_bar_accepts_identical_rows(rows):
    inp, experts, aq, as_, o = rows
    assert check_l2_rows(inp, experts, o, o, aq, as_)[0] == 0


def test_l2_bar_accepts_one_ulp(rows):
    inp, experts, aq, as_, o = rows
    g = o.copy()
    g[:, ::7] = np.where(g[:, ::7] & 0x7F80, g[:, ::7] + 1, g[:, ::7])  # one bf16 ulp up (normal values)
    check_l2_rows(inp, experts, g, o, aq, as_)


def test_l2_bar_rejects_a_wrong_kblock_scale(rows):
    """One of the 64 k-blocks of a row (I = 2048) summed with its scale one
    step off moves that row's outputs far beyond the bar."""
    inp, experts, aq, as_, o = rows
    bad_s = as_.copy()
    bad_s[0, 17] += 1
    wrong = oracle.l2_rows(inp, experts[:1], aq[:1], bad_s[:1])
    g = o.copy()
    g[0] = wrong[0]
    with pytest.raises(AssertionError):
        check_l2_rows(inp, experts, g, o, aq, as_)


def test_l2_bar_rejects_a_dropped_kblock(rows):
    inp, experts, aq, as_, o = rows
    bad_q = aq.copy()
    bad_q[3, 64:96] = 0
    g = o.copy()
    g[3] = oracle.l2_rows(inp, experts[3:4], bad_q[3:4], as_[3:4])[0]
    with pytest.raises(AssertionError):
        check_l2_rows(inp, experts, g, o, aq, as_)


def test_act_bar(rows):
    inp, _, aq, as_, _ = rows
    slack = l1_slack(inp, *inp["_rows"])
    check_act(aq, as_, aq, as_)
    g = aq.copy()
    # one code one step up (within the 0.1 % budget): accepted
    c = int(g[0, 5])
    g[0, 5] = c + 1 if (c & 0x7F) < 0x7E else c - 1
    check_act(g, as_, aq, as_)
    # two steps on an element whose propagated GEMM bound is well below one
    # step (no heavy cancellation in its gate or up sum): rejected, with or
    # without the GEMM slack
    g2 = aq.copy()
    cols = np.nonzero(((aq[1] & 0x7F) > 0x40) & ((aq[1] & 0x7F) < 0x70))[0][:64]
    steps = e4m3_step_at(oracle.e4m3_to_f32(aq[1, cols]).astype(np.float64)) * np.exp2(
        as_[1, cols // 32].astype(np.float64) - 127)
    ratio = slack(np.full(len(cols), 1), cols) / steps
    i = int(cols[np.argmin(ratio)])
    assert ratio.min() < 0.5
    g2[1, i] = aq[1, i] + 2
    with pytest.raises(AssertionError):
        check_act(g2, as_, aq, as_)
    with pytest.raises(AssertionError):
        check_act(g2, as_, aq, as_, gemm_slack=slack)
    # a scale byte two steps off: rejected
    s2 = as_.copy()
    s2[2, 3] += 2
    with pytest.raises(AssertionError):
        check_act(aq, s2, aq, as_, gemm_slack=slack)
    # one group's scale up by one with codes left as they were (values
    # doubled): rejected
    s1 = as_.copy()
    s1[4, 1] += 1
    with pytest.raises(AssertionError):
        check_act(aq, s1, aq, as_, gemm_slack=slack)


def test_act_slack_is_small_against_the_group_scale(rows):
    """The propagated GEMM bound stays a small fraction of the group's
    largest step: it can excuse moves of near-zero values, not of the
    values that set the group's scale."""
    inp, _, aq, as_, _ = rows
    slack = l1_slack(inp, *inp["_rows"])
    r = np.arange(8)
    c = np.arange(8) * 37
    top_step = 32.0 * np.exp2(as_[r, c // 32].astype(np.float64) - 127)
    assert (slack(r, c) < 0.25 * top_step).all()


def test_mtile_sample_rows():
    off = np.array([0, 300, 300, 301, 812])
    rows = mtile_sample_rows(off, 256)
    assert list(rows) == [0, 255, 256, 299, 300, 301, 556, 557, 811]
