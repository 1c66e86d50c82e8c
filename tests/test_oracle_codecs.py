"""Pins of the oracle's element codecs against things other than itself:
torch's CPU casts (library routines), the OCP e2m1 table (golden fixture), a
closed-form bit formula for the scale rule, and brute force."""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_decode_is_top_half_of_f32():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    L = oracle.lib()
    sel = bits[::97][np.isfinite(ref[::97])]  # a float return through ctypes quiets NaNs
    got = np.array([L.oracle_bf16_to_f32(int(b)) for b in sel], np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), ref[::97][np.isfinite(ref[::97])].view(np.uint32))


def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(11)
    u = rng.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    # add exact ties (low 16 bits 0x8000) with both parities of the kept bit
    ties = (rng.integers(0, 1 << 16, size=2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    f = np.concatenate([f, ties]).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16(f)
    np.testing.assert_array_equal(got, ref)


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    got = oracle.e4m3_to_f32(codes)
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.isnan(got[nan]).all()
    np.testing.assert_array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9


def test_e4m3_encode_all_bf16_in_range_match_torch():
    """Every finite bf16 value with |v| <= 448 (the range the scale rule
    guarantees), rounded to e4m3: oracle vs torch's RNE cast."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    v = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()
    keep = torch.isfinite(v) & (v.abs() <= 448)
    v = v[keep]
    ref = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_from_f64(v.double().numpy())
    np.testing.assert_array_equal(got, ref)


def test_e4m3_encode_random_f32_and_ties_match_torch():
    rng = np.random.default_rng(5)
    mag = np.exp2(rng.uniform(-14, np.log2(448), size=200000))
    v = (mag * rng.choice([-1.0, 1.0], size=mag.size)).astype(np.float32)
    # exact midpoints between neighbouring e4m3 values (ties)
    vals = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids, np.float32([0.0, -0.0, 448.0, -448.0])])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_from_f64(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_e4m3_saturates_above_448():
    got = oracle.e4m3_from_f64(np.array([448.0, 460.0, 1e6, -1e6]))
    assert list(got) == [0x7E, 0x7E, 0x7E, 0xFE]


def _golden_e2m1():
    rows = [line.split() for line in open(os.path.join(GOLDEN, "e2m1_values.txt"))
            if line.strip() and not line.startswith("#")]
    return {int(c): float(v) for c, v in rows}


def test_e2m1_decode_matches_ocp_table():
    table = _golden_e2m1()
    got = oracle.e2m1_to_f32(np.arange(16, dtype=np.uint8))
    for c in range(16):
        assert got[c] == table[c], c
        assert np.signbit(got[c]) == (c >= 8)


def test_e2m1_table_is_the_e2m1_minifloat():
    """Closed form of a 1-2-1 minifloat with bias 1 (subnormal when the
    exponent field is 0), independent of the table."""
    got = oracle.e2m1_to_f32(np.arange(16, dtype=np.uint8))
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = (m / 2.0) * 2.0 ** (1 - 1) if e == 0 else (1 + m / 2.0) * 2.0 ** (e - 1)
        assert got[c] == (-mag if s else mag)


def _rule_q_bits(amax: np.ndarray) -> np.ndarray:
    """Closed form of the scale rule on the fp32 fields of amax: exponent
    field minus 8, plus one when the mantissa exceeds 0.75 (448 = 1.75 * 2^8),
    clamped to [0, 254]."""
    bits = amax.astype(np.float32).view(np.uint32)
    ef = ((bits >> 23) & 0xFF).astype(np.int64)
    mf = (bits & 0x7FFFFF).astype(np.int64)
    return np.clip(ef - 8 + (mf > 0x600000), 0, 254).astype(np.uint8)


def test_scale_rule_matches_closed_form_and_is_minimal():
    rng = np.random.default_rng(3)
    a = np.exp2(rng.uniform(-30, 30, size=200000)).astype(np.float32)
    edges = np.float32([1.0, 1.75, 1.7500001, 448.0, 448.00003, 2.0 ** -20, 3.5, 7.0, 7.0000005])
    a = np.concatenate([a, edges])
    b = oracle.ue8m0_for_e4m3(a)
    np.testing.assert_array_equal(b, _rule_q_bits(a))
    s = np.exp2(b.astype(np.float64) - 127)
    assert (a.astype(np.float64) <= 448 * s).all()
    assert (a.astype(np.float64) > 448 * s / 2).all()  # one step smaller would not fit


def test_scale_rule_examples():
    b = oracle.ue8m0_for_e4m3(np.float32([1.0, 448.0, 0.0, 1.75, 1.76]))
    assert list(b) == [119, 127, 0, 119, 120]


def test_quant_row_uses_power_of_two_division():
    rng = np.random.default_rng(9)
    v = rng.standard_normal(256).astype(np.float32) * 3
    v[32:64] = 0.0  # an all-zero group: scale byte 0, codes 0
    q, s = oracle.quant_e4m3_row(v)
    assert s[1] == 0 and (q[32:64] == 0).all()
    for g in range(8):
        grp = v[32 * g:32 * g + 32]
        ref = torch.from_numpy((grp.astype(np.float64) * 2.0 ** (127 - int(s[g]))).astype(np.float32))
        np.testing.assert_array_equal(q[32 * g:32 * g + 32],
                                      ref.to(torch.float8_e4m3fn).view(torch.uint8).numpy())
        if g != 1:
            assert np.abs(oracle.e4m3_to_f32(q[32 * g:32 * g + 32])).max() >= 224  # amax/scale lies in (224, 448]
