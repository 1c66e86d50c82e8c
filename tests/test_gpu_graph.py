"""The fused layer captured into a HIP graph and replayed.

The layer's launches take every size from the device (the m-tile table, the
routed-row count) and the library allocates nothing, issues no memset and
never synchronises, so one captured call serves every later batch of the same
shape.  Each replay here runs after the output and the whole workspace have
been overwritten with junk and after eager work on the same stream, and is
compared bit for bit with an eager call on the same inputs; between replays
the inputs change in place, so a replay that reused anything from an earlier
one would show.
"""
import numpy as np
import pytest
import torch

import moe_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bits(t):
    return t.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("case", [dict(T=300, H=512, I=256, E=6, K=3, routing="zipf", seed=41,
                                       mask_p=0.1),
                                  dict(T=128, H=1024, I=512, E=16, K=8, routing="uniform",
                                       seed=52)],
                         ids=["ragged", "uniform"])
def test_graph_replay_matches_eager(case):
    import combine_dispatch_amd as moe
    from tests.gpu_util import to_dev

    seeds = [case["seed"], case["seed"] + 100, case["seed"] + 200]
    inputs = [moe_inputs.make_inputs(**dict(case, seed=s)) for s in seeds]
    T, H, I, E, K = (inputs[0][k] for k in ("T", "H", "I", "E", "K"))
    # the weights stay those of the first draw; x and the routing change
    dev = to_dev(inputs[0])
    packed = torch.empty(moe.moe_packed_scales_bytes(H, I, E), dtype=torch.uint8, device=DEV)
    moe.moe_pack_weight_scales(dev["S1"], dev["S2"], packed, E=E, H=H, I=I)
    ws = torch.empty(moe.moe_workspace_bytes(T, H, I, E, K), dtype=torch.uint8, device=DEV)
    y = torch.empty((T, H), dtype=torch.int16, device=DEV)

    def call(out, stream=None):
        moe.moe_fused_forward_packed(dev["x"], dev["topk_idx"], dev["topk_w"], dev["W1q"],
                                     dev["W2q"], packed, out, ws, E=E, I=I, stream=stream)

    def load(inp):
        dev["x"].copy_(torch.from_numpy(inp["x"].view(np.int16)))
        dev["topk_idx"].copy_(torch.from_numpy(inp["topk_idx"]))
        dev["topk_w"].copy_(torch.from_numpy(inp["topk_w"]))

    # eager reference for every input draw
    refs = []
    for inp in inputs:
        load(inp)
        y_e = torch.empty_like(y)
        call(y_e)
        torch.cuda.synchronize()
        refs.append(_bits(y_e))
    assert not np.array_equal(refs[0], refs[1])

    load(inputs[0])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(y, stream=s)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call(y)
    torch.cuda.synchronize()

    for rep in range(6):
        inp = inputs[rep % 3]
        load(inp)
        y.fill_(0x7FC0)  # a bf16 NaN in every element
        ws.fill_(0xA5)
        # eager work on the same stream between replays
        y_other = torch.empty_like(y)
        call(y_other)
        ws.fill_(0x5A)
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(y), refs[rep % 3], err_msg=f"replay {rep}")
        np.testing.assert_array_equal(_bits(y_other), refs[rep % 3])
