"""Pins for the oracle's element decoders (no GPU).

Each decoder evaluates bit fields; it is checked here against independent
sources: torch's own float8_e4m3fn / float8_e8m0fnu / bfloat16 conversions
(library routines), the OCP MX E2M1 value table, and spot values of the
formats' definitions.
"""
import numpy as np
import pytest
import torch

import oracle


def test_e4m3_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])


def test_e4m3_spot_values_and_structure():
    d = oracle.decode_e4m3
    assert d(np.uint8(0x38)) == 1.0
    assert d(np.uint8(0x7E)) == 448.0
    assert d(np.uint8(0xFE)) == -448.0
    assert d(np.uint8(0x01)) == 2.0 ** -9          # smallest subnormal
    assert d(np.uint8(0x07)) == 7 * 2.0 ** -9      # largest subnormal
    assert d(np.uint8(0x08)) == 2.0 ** -6          # smallest normal
    assert d(np.uint8(0x80)) == 0.0
    v = d(np.arange(256, dtype=np.uint8))
    assert np.sum(np.isnan(v)) == 2                  # 0x7F and 0xFF only
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                  # positive codes monotone
    assert np.array_equal(v[0x80:0xFF], -v[0x00:0x7F])


# OCP MX v1.0, E2M1 element encodings: codes 0..7 and their negatives.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
              -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e2m1_table():
    v = oracle.decode_e2m1(np.arange(16))
    assert np.array_equal(v, np.array(E2M1_TABLE))


def test_e8m0_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode_e8m0(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    assert np.isnan(mine[255]) and np.isnan(ref[255])
    assert np.array_equal(mine[:255], ref[:255])
    assert mine[127] == 1.0 and mine[0] == 2.0 ** -127 and mine[254] == 2.0 ** 127


def test_bf16_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 16, size=20000, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    mine = oracle.decode_bf16(bits)
    ok = ~np.isnan(ref)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.array_equal(mine[ok], ref[ok])
    assert oracle.decode_bf16(np.uint16(0x3F80)) == 1.0


def test_unpack_fp4_low_nibble_first():
    packed = np.array([[0x21, 0xF7]], dtype=np.uint8)
    assert oracle.unpack_fp4(packed).tolist() == [[0x1, 0x2, 0x7, 0xF]]


def test_int8_twos_complement():
    x = np.array([0x00, 0x7F, 0x80, 0xFF], dtype=np.uint8)
    assert oracle.decode_int8(x).tolist() == [0, 127, -128, -1]


@pytest.mark.parametrize("name", ["fp8", "bf16"])
def test_decoder_rejects_nothing_silently(name):
    # decoders are total on their code space and return float64
    if name == "fp8":
        assert oracle.decode_e4m3(np.arange(256, dtype=np.uint8)).dtype == np.float64
    else:
        assert oracle.decode_bf16(np.arange(16, dtype=np.uint16)).dtype == np.float64


def test_f16_matches_numpy_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.decode_f16(codes)
    ref = codes.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])


def test_f16_spot_values():
    d = oracle.decode_f16
    assert d(np.uint16(0x3C00)) == 1.0
    assert d(np.uint16(0xC000)) == -2.0
    assert d(np.uint16(0x7BFF)) == 65504.0            # largest finite
    assert d(np.uint16(0x0001)) == 2.0 ** -24         # smallest subnormal
    assert d(np.uint16(0x0400)) == 2.0 ** -14         # smallest normal
    assert d(np.uint16(0x7C00)) == np.inf
    assert np.isnan(d(np.uint16(0x7E00)))


def test_int4_codes_are_twos_complement():
    codes = np.arange(16, dtype=np.uint8)
    # sign extension by an arithmetic shift of the nibble placed in the top of a byte
    ref = (codes << 4).astype(np.uint8).view(np.int8).astype(np.int64) >> 4
    assert np.array_equal(oracle.decode_int4(codes), ref)
    assert oracle.decode_int4(codes).tolist() == [0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1]


def test_unpack_nibbles_order():
    packed = np.array([[0x21, 0x43, 0xF5]], np.uint8)
    assert oracle.unpack_nibbles(packed).tolist() == [[1, 2, 3, 4, 5, 15]]
