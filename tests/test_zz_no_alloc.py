"""The allocation-free entry (moe_fused_forward_packed_noalloc, its
workspace a device array inside the library) through the C ABI: two calls in
a row -- the small-batch workload, then a smaller ragged input, so the
second call runs on scratch the first one left full -- each bit-identical to
moe_fused_forward_packed with a caller workspace, and within the layer's bar
of the oracle."""
import numpy as np
import pytest
import torch

import moe_inputs
import oracle
from tests.gpu_util import DEV, bf16_bits, to_dev
from tests.parity_checks import check_y

pytestmark = pytest.mark.gpu


def _packed_pair(inp):
    import combine_dispatch_amd as moe
    T, H, I, E, K = (inp[k] for k in ("T", "H", "I", "E", "K"))
    dev = to_dev(inp)
    packed = torch.empty(moe.moe_packed_scales_bytes(H, I, E), dtype=torch.uint8, device=DEV)
    moe.moe_pack_weight_scales(dev["S1"], dev["S2"], packed, E=E, H=H, I=I)
    ws = torch.empty(moe.moe_workspace_bytes(T, H, I, E, K), dtype=torch.uint8, device=DEV)
    y_ref = torch.empty((T, H), dtype=torch.int16, device=DEV)
    moe.moe_fused_forward_packed(dev["x"], dev["topk_idx"], dev["topk_w"], dev["W1q"], dev["W2q"],
                                 packed, y_ref, ws, E=E, I=I)
    y = torch.full((T, H), 0x7FC0, dtype=torch.int16, device=DEV)  # poisoned
    moe.moe_fused_forward_packed_noalloc(dev["x"], dev["topk_idx"], dev["topk_w"], dev["W1q"],
                                         dev["W2q"], packed, y, E=E, I=I)
    torch.cuda.synchronize()
    return bf16_bits(y), bf16_bits(y_ref)


def test_noalloc_two_calls_match_the_workspace_entry():
    import combine_dispatch_amd as moe
    moe.lib()
    first = moe_inputs.config_inputs("small")
    second = moe_inputs.make_inputs(T=300, H=512, I=256, E=6, K=3, routing="zipf", seed=41,
                                    mask_p=0.1)
    for inp in (first, second):
        print("noalloc call", {k: inp[k] for k in "THIEK"}, flush=True)
        y, y_ref = _packed_pair(inp)
        np.testing.assert_array_equal(y, y_ref)
        if inp is second:
            check_y(y, oracle.forward(inp), inp["topk_idx"])


def test_noalloc_refuses_a_shape_beyond_its_scratch():
    import combine_dispatch_amd as moe
    T, H, I, E, K = 4096, 7168, 2048, 32, 8
    assert moe.moe_workspace_bytes(T, H, I, E, K) > moe.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.empty((T, H), dtype=torch.int16, device=DEV)
    idx = torch.zeros((T, K), dtype=torch.int64, device=DEV)
    w = torch.zeros((T, K), dtype=torch.float32, device=DEV)
    W1q = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=DEV)
    W2q = torch.empty((E, H, I // 2), dtype=torch.uint8, device=DEV)
    packed = torch.empty(moe.moe_packed_scales_bytes(H, I, E), dtype=torch.uint8, device=DEV)
    y = torch.empty((T, H), dtype=torch.int16, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_fused_forward_packed_noalloc(x, idx, w, W1q, W2q, packed, y, E=E, I=I)
    assert ei.value.status == moe.MOE_ERR_TOO_LARGE
