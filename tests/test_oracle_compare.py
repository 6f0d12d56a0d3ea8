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
