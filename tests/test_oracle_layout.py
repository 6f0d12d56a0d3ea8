"""Pins for the oracle's B preshuffle layout (no GPU).

The layout (GEMM Optimization Guide §1.4 and §12.1) must put, for every 16-row
block n0 and 64-byte K block k0, one contiguous 1 KiB chunk in which lane
l = 16*g + j of a wave finds the 16 bytes of row 16*n0 + j at K bytes
[64*k0 + 16*g, +16): the 16-axis is the lanes of one MFMA column block, the
4-axis the lane group that takes one dwordx4.
"""
import numpy as np
import pytest

import oracle


def _rand_b(N, Kb, seed=0):
    return np.random.default_rng(seed).integers(0, 256, size=(N, Kb), dtype=np.uint8)


def test_golden_single_block():
    # N = 16, Kb = 64: byte (n, kb) lands at (kb // 16) * 256 + n * 16 + kb % 16
    b = np.arange(16 * 64, dtype=np.int64).reshape(16, 64)
    tag = (b % 251).astype(np.uint8)
    s = oracle.preshuffle(tag)
    for n in range(16):
        for kb in range(64):
            assert s[(kb // 16) * 256 + n * 16 + kb % 16] == tag[n, kb]


@pytest.mark.parametrize("N,Kb", [(16, 64), (32, 128), (48, 256), (64, 512)])
def test_lane_view_of_each_1k_chunk(N, Kb):
    b = _rand_b(N, Kb)
    s = oracle.preshuffle(b)
    for n0 in range(N // 16):
        for k0 in range(Kb // 64):
            chunk = s[(n0 * (Kb // 64) + k0) * 1024:][:1024].reshape(64, 16)
            for lane in range(64):
                g, j = divmod(lane, 16)
                assert np.array_equal(chunk[lane], b[16 * n0 + j, 64 * k0 + 16 * g: 64 * k0 + 16 * g + 16])


@pytest.mark.parametrize("N,Kb", [(16, 64), (32, 192), (128, 1024)])
def test_round_trip_and_bijection(N, Kb):
    b = _rand_b(N, Kb, 1)
    s = oracle.preshuffle(b)
    assert s.size == N * Kb
    assert np.array_equal(oracle.unshuffle(s, N, Kb), b)
    # destination indices form a permutation
    idx = np.array([oracle.preshuffle_index(n, kb, Kb) for n in range(N) for kb in range(Kb)])
    assert np.array_equal(np.sort(idx), np.arange(N * Kb))
    # and agree with the array permutation
    flat = b.reshape(-1)
    out = np.empty_like(flat)
    out[idx] = flat
    assert np.array_equal(out, s)


def test_shape_rules():
    with pytest.raises(ValueError):
        oracle.preshuffle(np.zeros((15, 64), np.uint8))
    with pytest.raises(ValueError):
        oracle.preshuffle(np.zeros((16, 96), np.uint8))


def test_bytes_not_elements():
    # a bf16 B of N x K elements is shuffled as N x 2K bytes
    b = np.random.default_rng(2).integers(0, 2 ** 16, size=(16, 32), dtype=np.uint16)
    s = oracle.preshuffle(b.view(np.uint8))
    assert np.array_equal(oracle.unshuffle(s, 16, 64).view(np.uint16), b)


def test_int4_piece_repack_positions():
    """Element t of a 16-byte piece (32 INT4 values) lands in byte t % 16,
    low nibble for t < 16, high nibble otherwise."""
    rng = np.random.default_rng(5)
    N, Kb = 16, 128
    vals = rng.integers(0, 16, size=(N, 2 * Kb)).astype(np.uint8)     # element order
    packed = (vals[:, 0::2] | (vals[:, 1::2] << 4)).astype(np.uint8)
    r = oracle.repack_int4_pieces(packed)
    for n in (0, 7, 15):
        for k in (0, 1, 15, 16, 17, 31, 32, 100, 255):
            piece, t = divmod(k, 32)
            byte = r[n, piece * 16 + t % 16]
            nib = (byte & 0xF) if t < 16 else (byte >> 4)
            assert nib == vals[n, k], (n, k)


def test_int4_layout_lane_view():
    """In the INT4 preshuffled layout, lane (g, j) of the KiB block (n0, k0)
    holds column 16 n0 + j: its low nibbles are K elements
    128 k0 + 32 g + 0..15 and its high nibbles 128 k0 + 32 g + 16..31."""
    rng = np.random.default_rng(6)
    N, K = 32, 512
    Kb = K // 2
    vals = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    packed = (vals[:, 0::2] | (vals[:, 1::2] << 4)).astype(np.uint8)
    bs = oracle.preshuffle_int4(packed)
    for n0 in range(N // 16):
        for k0 in range(Kb // 64):
            blk = bs[(n0 * (Kb // 64) + k0) * 1024:][:1024].reshape(4, 16, 16)
            for g in range(4):
                for j in range(16):
                    lane = blk[g, j]
                    k = 128 * k0 + 32 * g
                    assert np.array_equal(lane & 0xF, vals[16 * n0 + j, k:k + 16])
                    assert np.array_equal(lane >> 4, vals[16 * n0 + j, k + 16:k + 32])


def test_int4_layout_round_trip():
    rng = np.random.default_rng(7)
    b = rng.integers(0, 256, size=(48, 192), dtype=np.uint8)
    assert np.array_equal(oracle.unpack_int4_pieces(oracle.repack_int4_pieces(b)), b)
    assert np.array_equal(oracle.unshuffle_int4(oracle.preshuffle_int4(b), 48, 192), b)
