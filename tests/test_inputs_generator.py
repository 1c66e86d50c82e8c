"""The seeded input generator (moe_inputs) is the published counter-based
generator: Philox4x32-10 against its known-answer vectors, and its normals
have the moments of N(0, 1) and N(0, 0.02)."""
import os

import numpy as np

import moe_inputs
from tests.golden_util import GOLDEN


def test_philox4x32_10_known_answers():
    rows = [line.split() for line in open(os.path.join(GOLDEN, "philox4x32_10_kat.txt"))
            if line.strip() and not line.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        ctr = [int(w, 16) for w in r[0:4]]
        key = [int(w, 16) for w in r[4:6]]
        want = np.array([int(w, 16) for w in r[6:10]], dtype=np.uint32)
        np.testing.assert_array_equal(moe_inputs.philox4x32_10(ctr, key), want)


def test_normals_have_the_right_moments():
    n = 1 << 20
    for mean, std in ((0.0, 1.0), (0.0, 0.02)):
        v = moe_inputs.normal_f32(seed=3, stream=11, n=n, mean=mean, std=std).astype(np.float64)
        z = (v - mean) / std
        # sample moments of 2^20 N(0,1) draws: standard errors 1e-3 (mean),
        # 1.4e-3 (variance), 2.4e-3 (skewness), 4.8e-3 (excess kurtosis)
        assert abs(z.mean()) < 5e-3
        assert abs(z.var() - 1.0) < 7e-3
        assert abs((z ** 3).mean()) < 1.2e-2
        assert abs((z ** 4).mean() - 3.0) < 2.4e-2
    # different streams and seeds give different draws
    a = moe_inputs.normal_f32(seed=3, stream=11, n=64)
    b = moe_inputs.normal_f32(seed=3, stream=12, n=64)
    c = moe_inputs.normal_f32(seed=4, stream=11, n=64)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)
