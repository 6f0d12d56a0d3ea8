"""Pins for the oracle GEMM (no GPU).

The oracle (decode then float64 / int64 matmul) is checked against:
  * brute force with exact rationals (fractions.Fraction) on tiny inputs;
  * closed forms: all-ones, B = ones (row sums), identity B, permutation B,
    power-of-two scales;
  * subset selection (rows / cols) agreeing with the full result.
A dropped term, a wrong sign or index, or a transposed operand fails one of
these.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.formats import decode_e4m3, decode_e2m1, decode_e8m0, decode_bf16


def _frac_e4m3(c):
    c = int(c)
    s = -1 if c & 0x80 else 1
    e = (c >> 3) & 0xF
    m = c & 7
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 2 ** 6)
    return s * (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))


def _frac_bf16(bits):
    # exact value of an IEEE binary32 whose low 16 bits are zero
    bits = int(bits)
    s = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0:
        return s * Fraction(m, 128) * Fraction(2) ** (-126)
    return s * (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)


def _frac_e2m1(c):
    return Fraction([0, 1, 2, 3, 4, 6, 8, 12][c & 7], 2) * (-1 if c & 8 else 1)


def _brute(A, B, f):
    M, K = A.shape
    N = B.shape[0]
    return [[sum(f(A[m, k]) * f(B[n, k]) for k in range(K)) for n in range(N)] for m in range(M)]


def test_int8_bruteforce():
    rng = np.random.default_rng(1)
    A = rng.integers(-128, 128, size=(5, 7), dtype=np.int8)
    B = rng.integers(-128, 128, size=(6, 7), dtype=np.int8)
    ref = [[sum(int(A[m, k]) * int(B[n, k]) for k in range(7)) for n in range(6)] for m in range(5)]
    out = oracle.gemm_int8(A, B)
    assert out.dtype == np.int32
    assert out.tolist() == ref


def test_int8_overflow_detected():
    A = np.full((1, 2 ** 17 + 2), -128, dtype=np.int8)
    with pytest.raises(OverflowError):
        oracle.gemm_int8(A, A)


def test_fp8_bruteforce_exact_including_subnormals():
    rng = np.random.default_rng(2)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    A = rng.choice(finite, size=(4, 9))
    B = rng.choice(finite, size=(3, 9))
    A[0, :] = np.arange(1, 10)   # subnormals and small normals
    ref = _brute(A, B, _frac_e4m3)
    out = oracle.gemm_fp8(A, B, np.ones(4, np.float32), np.ones(3, np.float32))
    assert [[Fraction(x) for x in row] for row in out.tolist()] == ref


def test_fp8_scales_applied_per_row_and_col():
    rng = np.random.default_rng(3)
    A = rng.integers(0, 0x7E, size=(3, 8)).astype(np.uint8)
    B = rng.integers(0, 0x7E, size=(5, 8)).astype(np.uint8)
    sa = np.array([0.5, 2.0, 0.25], np.float32)
    sb = np.array([1.0, 4.0, 0.125, 8.0, 2.0], np.float32)
    ref = _brute(A, B, _frac_e4m3)
    out = oracle.gemm_fp8(A, B, sa, sb)
    for m in range(3):
        for n in range(5):
            assert Fraction(out[m, n]) == ref[m][n] * Fraction(float(sa[m])) * Fraction(float(sb[n]))


def test_bf16_bruteforce():
    rng = np.random.default_rng(4)
    A = (rng.integers(0, 2 ** 16, size=(3, 6)).astype(np.uint16) & 0xBFFF) | 0x3000
    B = (rng.integers(0, 2 ** 16, size=(4, 6)).astype(np.uint16) & 0xBFFF) | 0x3000
    ref = _brute(A, B, _frac_bf16)
    out = oracle.gemm_bf16(A, B)
    for m in range(3):
        for n in range(4):
            assert abs(Fraction(out[m, n]) - ref[m][n]) <= abs(ref[m][n]) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_mxfp4_bruteforce():
    rng = np.random.default_rng(5)
    M, N, K = 3, 2, 64
    ca = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    cb = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    sa = rng.integers(120, 135, size=(M, K // 32)).astype(np.uint8)
    sb = rng.integers(120, 135, size=(N, K // 32)).astype(np.uint8)
    pa = ca[:, 0::2] | (ca[:, 1::2] << 4)
    pb = cb[:, 0::2] | (cb[:, 1::2] << 4)
    out = oracle.gemm_mxfp4(pa, sa, pb, sb)
    for m in range(M):
        for n in range(N):
            ref = sum(_frac_e2m1(ca[m, k]) * Fraction(2) ** (int(sa[m, k // 32]) - 127)
                      * _frac_e2m1(cb[n, k]) * Fraction(2) ** (int(sb[n, k // 32]) - 127)
                      for k in range(K))
            assert Fraction(out[m, n]) == ref


@pytest.mark.parametrize("K", [64, 512, 2048])
def test_all_ones_closed_form(K):
    M, N = 16, 32
    one_i8 = np.ones((M, K), np.int8)
    assert np.all(oracle.gemm_int8(one_i8, np.ones((N, K), np.int8)) == K)
    one_fp8 = np.full((M, K), 0x38, np.uint8)
    r = oracle.gemm_fp8(one_fp8, np.full((N, K), 0x38, np.uint8), np.ones(M, np.float32), np.ones(N, np.float32))
    assert np.all(r == K)
    one_bf = np.full((M, K), 0x3F80, np.uint16)
    assert np.all(oracle.gemm_bf16(one_bf, np.full((N, K), 0x3F80, np.uint16)) == K)
    # E2M1 code 2 is 1.0; scale 127 is 2^0
    p = np.full((M, K // 2), 0x22, np.uint8)
    s = np.full((M, K // 32), 127, np.uint8)
    assert np.all(oracle.gemm_mxfp4(p, s, np.full((N, K // 2), 0x22, np.uint8),
                                    np.full((N, K // 32), 127, np.uint8)) == K)


def test_power_of_two_scales_closed_form():
    K = 256
    a = np.full((4, K), 0x38, np.uint8)
    b = np.full((8, K), 0x38, np.uint8)
    sa = np.array([1, 2, 0.5, 4], np.float32)
    sb = np.array([1, 0.25, 8, 2, 1, 1, 0.5, 16], np.float32)
    r = oracle.gemm_fp8(a, b, sa, sb)
    assert np.array_equal(r, K * np.outer(sa.astype(np.float64), sb.astype(np.float64)))


def test_b_ones_gives_row_sums():
    rng = np.random.default_rng(6)
    a = rng.integers(-8, 9, size=(8, 128), dtype=np.int8)
    r = oracle.gemm_int8(a, np.ones((16, 128), np.int8))
    assert np.array_equal(r, np.repeat(a.astype(np.int64).sum(1, keepdims=True), 16, 1))
    af = rng.integers(0, 0x7E, size=(8, 128)).astype(np.uint8)
    rf = oracle.gemm_fp8(af, np.full((16, 128), 0x38, np.uint8), np.ones(8, np.float32), np.ones(16, np.float32))
    assert np.array_equal(rf[:, 3], decode_e4m3(af).sum(1))


def test_constant_rows_of_a_give_scaled_col_sums():
    rng = np.random.default_rng(7)
    b = rng.integers(-8, 9, size=(16, 64), dtype=np.int8)
    c = np.arange(-4, 4, dtype=np.int8)
    a = np.repeat(c[:, None], 64, 1)
    r = oracle.gemm_int8(a, b)
    assert np.array_equal(r, np.outer(c.astype(np.int64), b.astype(np.int64).sum(1)))


def test_identity_b_returns_a():
    rng = np.random.default_rng(8)
    K = 64
    a = rng.integers(0, 0x7E, size=(5, K)).astype(np.uint8)
    eye = np.where(np.eye(K, dtype=bool), 0x38, 0x00).astype(np.uint8)
    r = oracle.gemm_fp8(a, eye, np.ones(5, np.float32), np.ones(K, np.float32))
    assert np.array_equal(r, decode_e4m3(a))
    ab = (rng.integers(0, 2 ** 16, size=(5, K)).astype(np.uint16) & 0xBFFF)
    eyeb = np.where(np.eye(K, dtype=bool), 0x3F80, 0).astype(np.uint16)
    assert np.array_equal(oracle.gemm_bf16(ab, eyeb), decode_bf16(ab))


def test_permutation_b_selects_columns_of_a():
    rng = np.random.default_rng(9)
    K, N = 64, 48
    perm = rng.integers(0, K, size=N)
    a = rng.integers(-8, 9, size=(7, K), dtype=np.int8)
    b = np.zeros((N, K), np.int8)
    b[np.arange(N), perm] = 1
    assert np.array_equal(oracle.gemm_int8(a, b), a[:, perm].astype(np.int32))


def test_row_col_subset_matches_full():
    rng = np.random.default_rng(10)
    a = rng.integers(0, 0x7E, size=(20, 64)).astype(np.uint8)
    b = rng.integers(0, 0x7E, size=(30, 64)).astype(np.uint8)
    sa = rng.random(20).astype(np.float32)
    sb = rng.random(30).astype(np.float32)
    full = oracle.gemm_fp8(a, b, sa, sb)
    rows, cols = [3, 0, 19], [29, 5, 5, 1]
    assert np.array_equal(oracle.gemm_fp8(a, b, sa, sb, rows, cols), full[np.ix_(rows, cols)])


def test_mxfp4_scale_blocks_are_32_wide():
    # a scale change in block 1 must affect exactly elements 32..63
    K = 128
    codes = np.full((1, K), 2, np.uint8)                 # all 1.0
    p = codes[:, 0::2] | (codes[:, 1::2] << 4)
    sa = np.array([[127, 130, 127, 127]], np.uint8)      # block 1 scaled by 8
    sb = np.full((1, 4), 127, np.uint8)
    r = oracle.gemm_mxfp4(p, sa, p, sb)
    assert r[0, 0] == 32 + 32 * 8 + 32 + 32
    assert decode_e8m0(np.uint8(130)) == 8.0 and decode_e2m1(2) == 1.0


def _frac_f16(bits):
    bits = int(bits)
    s = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 0x1F
    m = bits & 0x3FF
    if e == 0:
        return s * Fraction(m, 1024) * Fraction(2) ** (-14)
    return s * (1 + Fraction(m, 1024)) * Fraction(2) ** (e - 15)


def test_f16_bruteforce_including_subnormals():
    rng = np.random.default_rng(11)
    A = (rng.integers(0, 2 ** 16, size=(3, 7)).astype(np.uint16) & 0xBBFF)   # finite, |x| < 2^15
    B = (rng.integers(0, 2 ** 16, size=(4, 7)).astype(np.uint16) & 0xBBFF)
    A[0, :4] = [1, 2, 0x3FF, 0x8001]                                          # subnormals
    ref = _brute(A, B, _frac_f16)
    out = oracle.gemm_f16(A, B)
    for m in range(3):
        for n in range(4):
            # every product is a multiple of 2^-48 below 2^31: the float64 sum of 7 is exact
            assert Fraction(out[m, n]) == ref[m][n]


def _int4_val(c):
    c = int(c) & 0xF
    return c - 16 if c >= 8 else c


def test_w4a8_bruteforce():
    rng = np.random.default_rng(12)
    M, N, K = 3, 5, 12
    A = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    codes = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    sa = np.array([0.5, 0.25, 3.0], np.float32)
    sb = np.array([1.0, 2.0, 0.125, 0.75, 4.0], np.float32)
    out = oracle.gemm_w4a8(A, packed, sa, sb)
    for m in range(M):
        for n in range(N):
            acc = sum(int(A[m, k]) * _int4_val(codes[n, k]) for k in range(K))
            assert Fraction(out[m, n]) == acc * Fraction(float(sa[m])) * Fraction(float(sb[n]))


def test_w4a8_closed_forms():
    rng = np.random.default_rng(13)
    K = 256
    a = rng.integers(-127, 128, size=(6, K), dtype=np.int8)
    ones = np.full((8, K // 2), 0x11, np.uint8)                    # every int4 = 1
    r = oracle.gemm_w4a8(a, ones, np.ones(6, np.float32), np.ones(8, np.float32))
    assert np.array_equal(r, np.repeat(a.astype(np.float64).sum(1, keepdims=True), 8, 1))
    minus8 = np.full((2, K // 2), 0x88, np.uint8)                  # every int4 = -8
    r = oracle.gemm_w4a8(np.ones((1, K), np.int8), minus8, np.ones(1, np.float32), np.ones(2, np.float32))
    assert np.all(r == -8 * K)
    # one-hot B at odd / even k selects the matching column of A
    perm = rng.integers(0, K, size=16)
    codes = np.zeros((16, K), np.uint8)
    codes[np.arange(16), perm] = 1
    b = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    r = oracle.gemm_w4a8(a, b, np.ones(6, np.float32), np.ones(16, np.float32))
    assert np.array_equal(r, a[:, perm].astype(np.float64))


def test_fp16_identity_b_returns_a():
    rng = np.random.default_rng(14)
    K = 64
    a = rng.integers(0, 2 ** 16, size=(5, K)).astype(np.uint16) & 0xBBFF
    eye = np.where(np.eye(K, dtype=bool), 0x3C00, 0).astype(np.uint16)
    assert np.array_equal(oracle.gemm_f16(a, eye), oracle.decode_f16(a))


def test_dispatch_new_types():
    import workloads

    h = workloads.make_inputs("w4a8", 16, 32, 128, 1)
    assert np.array_equal(oracle.gemm("w4a8", h), oracle.gemm_w4a8(h["a"], h["b"], h["scale_a"], h["scale_b"]))
    h = workloads.make_inputs("fp16", 16, 32, 128, 1)
    assert np.array_equal(oracle.gemm("fp16", h), oracle.gemm_f16(h["a"], h["b"]))


@pytest.mark.parametrize("dtype", ["int8", "fp8", "bf16", "mxfp4", "fp16", "w4a8"])
@pytest.mark.parametrize("M,N", [(32, 32), (16, 48)])
def test_dispatch_routes_every_type(dtype, M, N):
    """oracle.gemm(dtype, inputs) is the type's own function on the same
    arrays, with the operands and their scales in their places (M == N too,
    where swapped row / column scales would keep every shape)."""
    import workloads

    K = 256
    h = workloads.make_inputs(dtype, M, N, K, seed=M + N)
    direct = {
        "int8": lambda r, c: oracle.gemm_int8(h["a"], h["b"], r, c),
        "fp8": lambda r, c: oracle.gemm_fp8(h["a"], h["b"], h["scale_a"], h["scale_b"], r, c),
        "bf16": lambda r, c: oracle.gemm_bf16(h["a"], h["b"], r, c),
        "mxfp4": lambda r, c: oracle.gemm_mxfp4(h["a"], h["scale_a"], h["b"], h["scale_b"], r, c),
        "fp16": lambda r, c: oracle.gemm_f16(h["a"], h["b"], r, c),
        "w4a8": lambda r, c: oracle.gemm_w4a8(h["a"], h["b"], h["scale_a"], h["scale_b"], r, c),
    }[dtype]
    assert np.array_equal(oracle.gemm(dtype, h), direct(None, None))
    rows, cols = np.array([0, 3, M - 1]), np.array([1, N - 2])
    assert np.array_equal(oracle.gemm(dtype, h, rows, cols), direct(rows, cols))
    if "scale_a" in h:
        # the row scales really are per row and the column scales per column:
        # doubling scale_a of row 0 doubles row 0 only
        h2 = dict(h)
        sa = np.array(h["scale_a"], copy=True)
        if dtype == "mxfp4":
            sa[0] = sa[0] + 1                    # E8M0: one more in the exponent doubles
        else:
            sa[0] = sa[0] * 2
        h2["scale_a"] = sa
        r1, r2 = oracle.gemm(dtype, h), oracle.gemm(dtype, h2)
        assert np.array_equal(r2[0], 2 * r1[0]) and np.array_equal(r2[1:], r1[1:])
