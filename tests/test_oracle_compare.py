"""Pins for the comparison metrics and the bf16 rounding helper (no GPU)."""
import numpy as np
import torch

import oracle
from oracle.compare import compare_bf16, bf16_rne


def _to_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-5, 5, 100000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(bf16_rne(x.astype(np.float64)), ref)


def test_exact_result_passes_with_zero_error():
    r = np.array([[1.0, -2.0], [0.5, 4.0]])
    m = compare_bf16(_to_bits(r), r)
    assert m["normwise"] == 0.0 and m["elem_floored"] == 0.0 and m["ok"]


def test_rounded_result_within_rne_bound():
    rng = np.random.default_rng(1)
    r = rng.standard_normal((64, 64)) * 100
    m = compare_bf16(_to_bits(r), r)
    assert m["ok"]
    assert m["elem_floored"] <= 2.0 ** -8
    assert m["normwise"] <= 2.0 ** -8


def test_single_wrong_element_detected():
    rng = np.random.default_rng(2)
    r = rng.standard_normal((32, 32))
    c = r.copy()
    c[5, 7] *= 1.05
    m = compare_bf16(_to_bits(c), r)
    assert not m["ok"] and m["elem_floored"] > 0.04


def test_elementwise_bound_fails_alone():
    """One element 5% off in a large bf16-exact result: the normwise error
    stays far inside its bound, so only the elementwise bound can reject it."""
    rng = np.random.default_rng(3)
    r = rng.integers(-64, 65, size=(256, 256)).astype(np.float64)   # exact in bf16
    r[r == 0] = 1.0
    r[100, 200] = 80.0
    c = r.copy()
    c[100, 200] = 84.0                          # 5 % off, exact in bf16
    m = compare_bf16(_to_bits(c), r)
    assert m["normwise"] < 1e-3 and abs(m["elem_floored"] - 0.05) < 1e-12
    assert not m["ok"]


def test_normwise_value():
    r = np.ones((16, 16))
    c = np.ones((16, 16)) * 1.0078125         # every element off by one bf16 ulp, 2^-7
    m = compare_bf16(_to_bits(c), r)
    assert abs(m["normwise"] - 2.0 ** -7) < 1e-12
    assert not m["ok"]                         # 7.8e-3 > 2e-3


def test_floor_only_affects_tiny_references():
    r = np.ones((10, 10))
    r[0, 0] = 1e-6
    c = r.copy()
    c[0, 0] = 2e-6                             # literal 100 % off, but tiny
    m = compare_bf16(_to_bits(c), r)
    assert m["elem_literal"] > 0.5
    assert m["elem_floored"] < 1e-3


def test_nonfinite_fails():
    r = np.ones((4, 4))
    bits = _to_bits(r)
    bits[0, 0] = 0x7FC0
    assert not compare_bf16(bits, r)["ok"]


def test_tolerances():
    assert oracle.NORMWISE_TOL == 2e-3 and oracle.ELEM_TOL == 1e-2


# ---------------------------------------------------------------- fp16 / bf16 rounding helpers
def _f16_normals():
    """Every finite positive normal binary16 value, ascending, as float64."""
    bits = np.arange(0x0400, 0x7C00, dtype=np.uint16)
    return bits.view(np.float16).astype(np.float64)


def test_f16_rne_matches_numpy_on_every_normal_value():
    v = _f16_normals()
    for s in (1.0, -1.0):
        assert np.array_equal(oracle.f16_rne(s * v), s * v)


def test_f16_rne_ties_and_neighbours_match_numpy():
    """Exact midpoints between consecutive normal binary16 values (ties go to
    the even significand), and the float64 values one ulp either side of
    each midpoint (they round down / up): numpy's binary64 -> binary16 cast
    rounds once, to nearest even."""
    v = _f16_normals()
    mid = (v[:-1] + v[1:]) / 2.0                 # exact in float64
    for x in (mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf)):
        for s in (1.0, -1.0):
            ref = (s * x).astype(np.float16).astype(np.float64)
            assert np.array_equal(oracle.f16_rne(s * x), ref)
    # ties to even: the midpoint goes to the neighbour whose last significand bit is 0
    lo_bits = np.arange(0x0400, 0x7BFF, dtype=np.uint16)
    even_lo = (lo_bits & 1) == 0
    got = oracle.f16_rne(mid)
    assert np.array_equal(got[even_lo], v[:-1][even_lo]) and np.array_equal(got[~even_lo], v[1:][~even_lo])


def test_f16_rne_random_values_match_numpy():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-13, 15, 200000))
    x = x[(np.abs(x) >= 2.0 ** -14) & (np.abs(x) < 65504.0)]
    assert np.array_equal(oracle.f16_rne(x), x.astype(np.float16).astype(np.float64))
    assert oracle.f16_rne(np.array([0.0]))[0] == 0.0


def test_bf16_rne_ties_go_to_even():
    """Midpoints of consecutive bf16 values are exact in fp32; torch's
    fp32 -> bf16 cast rounds them to the even neighbour."""
    bits = np.arange(0x0080, 0x7F80, dtype=np.uint32)           # positive normal bf16
    v = (bits << 16).view(np.float32).astype(np.float64)
    mid = ((v[:-1] + v[1:]) / 2.0).astype(np.float32)
    ref = torch.from_numpy(mid).to(torch.bfloat16).double().numpy()
    assert np.array_equal(bf16_rne(mid.astype(np.float64)), ref)
