"""A plain C11 program (tests/abi_consumer.c, built by the build step) drives
moe_fused_forward through include/moe.h with device memory from the HIP
runtime alone; its y must equal the Python binding's bit for bit, and the
oracle's within the layer's tolerance."""
import os
import subprocess

import numpy as np
import pytest

import moe_inputs
import oracle

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "abi_consumer")


@pytest.mark.parametrize("case", [dict(name="tiny"),
                                  dict(T=300, H=512, I=256, E=6, K=3, routing="zipf", seed=41,
                                       mask_p=0.1)],
                         ids=["tiny", "ragged"])
def test_plain_c_caller(case, tmp_path):
    from tests.gpu_util import run_forward
    from tests.test_gpu_parity import check_y
    assert os.path.exists(EXE), "tests/abi_consumer is missing: run __graft_entry__.build()"
    inp = (moe_inputs.config_inputs(case["name"]) if "name" in case
           else moe_inputs.make_inputs(**case))
    for k in ("x", "topk_idx", "topk_w", "W1q", "S1", "W2q", "S2"):
        np.ascontiguousarray(inp[k]).tofile(str(tmp_path / f"{k}.bin"))
    args = [EXE, str(tmp_path)] + [str(int(inp[k])) for k in ("T", "H", "I", "E", "K")]
    print("running", " ".join(args), flush=True)
    r = subprocess.run(args, capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    T, H = inp["T"], inp["H"]
    y_c = np.fromfile(str(tmp_path / "y.bin"), dtype=np.uint16).reshape(T, H)
    y_py, _ = run_forward(inp)
    np.testing.assert_array_equal(y_c, y_py)
    check_y(y_c, oracle.forward(inp), inp["topk_idx"])
