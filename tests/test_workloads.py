"""Checks of the seeded input generators (no GPU)."""
import numpy as np
import pytest

import oracle
import workloads


def test_deterministic():
    a = workloads.make_inputs("fp8", 16, 64, 128, 7)
    b = workloads.make_inputs("fp8", 16, 64, 128, 7)
    for k in a:
        assert np.array_equal(a[k], b[k])


def test_int8_range_and_shape():
    x = workloads.make_inputs("int8", 32, 48, 64, 1)
    assert x["a"].shape == (32, 64) and x["b"].shape == (48, 64)
    assert x["a"].dtype == np.int8
    assert x["a"].min() == -8 and x["a"].max() == 8


def test_fp8_rows_reach_448():
    x = workloads.make_inputs("fp8", 8, 32, 256, 2)
    va = oracle.decode_e4m3(x["a"])
    assert np.all(np.isfinite(va))
    assert np.all(np.abs(va).max(1) == 448.0)
    assert x["scale_a"].dtype == np.float32 and x["scale_a"].shape == (8,)
    assert x["scale_b"].shape == (32,)


def test_bf16_is_rounded_normal():
    x = workloads.make_inputs("bf16", 16, 16, 512, 4)
    v = oracle.decode_bf16(x["a"])
    assert 0.9 < v.std() < 1.1 and abs(v.mean()) < 0.1


def test_mxfp4_shapes_and_reconstruction():
    x = workloads.make_inputs("mxfp4", 8, 16, 256, 5)
    assert x["a"].shape == (8, 128) and x["scale_a"].shape == (8, 8)
    assert x["b"].shape == (16, 128) and x["scale_b"].shape == (16, 8)
    # the block-scaled values approximate the N(0,1) draw: values span ~[-6, 6]*scale
    vals = oracle.decode_e2m1(oracle.unpack_fp4(x["a"]))
    assert np.abs(vals).max() == 6.0
    assert np.all(x["scale_a"] < 255)


@pytest.mark.parametrize("name", sorted(workloads.CONFIGS))
def test_config_table(name):
    dtype, M, N, K, seed, tile = workloads.CONFIGS[name]
    assert M % 16 == 0 and N % 16 == 0
    assert (K * workloads.elem_bytes(dtype)) % 64 == 0


def test_w4a8_ranges():
    x = workloads.make_inputs("w4a8", 16, 32, 256, 6)
    assert x["a"].dtype == np.int8 and x["a"].shape == (16, 256)
    assert np.all(np.abs(x["a"].astype(int)).max(1) == 127) and x["a"].min() >= -127
    vb = oracle.decode_int4(oracle.unpack_nibbles(x["b"]))
    assert x["b"].shape == (32, 128) and vb.shape == (32, 256)
    assert np.all(np.abs(vb).max(1) >= 7) and vb.min() >= -8 and vb.max() <= 7
    assert x["scale_a"].dtype == np.float32 and x["scale_b"].shape == (32,)


def test_fp16_is_rounded_normal():
    x = workloads.make_inputs("fp16", 16, 16, 512, 4)
    v = oracle.decode_f16(x["a"])
    assert 0.9 < v.std() < 1.1 and abs(v.mean()) < 0.1
    assert np.array_equal(v, v.astype(np.float16).astype(np.float64))


def test_bias_scale():
    x = workloads.make_inputs("bf16", 16, 4096, 1024, 4, bias=True)
    assert x["bias"].dtype == np.float32 and x["bias"].shape == (4096,)
    assert 0.9 * 32 < x["bias"].std() < 1.1 * 32
