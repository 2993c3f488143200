"""Pins of the oracle's 3-bit weights: the 2 + 1 bit-plane layout of MNN's
3-bit path (code 0..7, offset -4) in the operator's per-block blob, LSB first.

Checked against hand-derived bytes (tests/golden/codec3_bytes.txt), an
independent decoder built on numpy.unpackbits over the two planes, pack /
unpack round trips, the default zero point 4 (MNN's -4 offset: signed codes
-4..3), codes equal to the zero point dequantizing to zero, and the float
matmul against a dense numpy formulation.
"""
import numpy as np
import pytest

import oracle
from tests.test_oracle_codec import np_decode_fields


def parse(golden, tag):
    for row in golden("codec3_bytes.txt"):
        if row[0] == tag:
            i = row.index(":")
            return (np.array([int(b, 16) for b in row[1:i]], np.uint8),
                    [int(v) for v in row[i + 1:]])
    raise KeyError(tag)


def test_golden_blob_and_zero_points(golden):
    blob, codes = parse(golden, "codes")
    got = oracle.unpack_codes(blob.reshape(1, 1, 6), 1, 16, 16, 3)[0]
    assert list(got) == codes
    assert np.array_equal(oracle.pack_codes(np.array([codes], np.uint8), 16, 3).ravel(), blob)
    zb, zps = parse(golden, "zps")
    assert list(oracle.unpack_zero_points(zb.reshape(1, 2), 1, 3, 3)[0]) == zps
    assert np.array_equal(oracle.pack_zero_points(np.array([zps], np.uint8), 3).ravel(), zb)


def np_codes3(B, K):
    """Independent decoder: per block, unpackbits of the main plane into
    2-bit fields and of the aux plane into 1-bit fields."""
    N, kb, blob = B.shape
    bs = blob * 8 // 3
    lo = np_decode_fields(B[:, :, :bs // 4], 2)          # [N, kb, bs]
    hi = np_decode_fields(B[:, :, bs // 4:], 1)
    return (lo | (hi << 2)).reshape(N, kb * bs)[:, :K]


@pytest.mark.parametrize("bs", [16, 32, 64, 128])
def test_independent_decoder_and_round_trip(bs):
    rng = np.random.default_rng(bs)
    N, K = 7, 5 * bs - 3
    kb = -(-K // bs)
    B = rng.integers(0, 256, (N, kb, 3 * bs // 8), dtype=np.uint8)
    codes = oracle.unpack_codes(B, N, K, bs, 3)
    assert np.array_equal(codes, np_codes3(B, K))
    assert codes.max() <= 7
    # Round trip (bits of the tail past K are cleared by the packer).
    assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(codes, bs, 3), N, K, bs, 3), codes)
    zps = rng.integers(0, 8, (N, kb)).astype(np.uint8)
    zb = oracle.pack_zero_points(zps, 3)
    assert zb.shape == (N, -(-kb * 3 // 8))
    assert np.array_equal(oracle.unpack_zero_points(zb, N, kb, 3), zps)
    # Independent zero-point decoder: one LSB-first bit stream per row.
    bits = np.unpackbits(zb, axis=1, bitorder="little")[:, :3 * kb].reshape(N, kb, 3)
    assert np.array_equal((bits * (1 << np.arange(3))).sum(-1), zps)


def test_default_zero_point_is_mnn_offset():
    assert (oracle.unpack_zero_points(None, 2, 5, 3) == 4).all()
    # codes 0..7 dequantize to (code - 4) * scale: the signed range -4..3.
    codes = np.arange(16).reshape(1, 16) % 8
    B = oracle.pack_codes(codes.astype(np.uint8), 16, 3)
    W = oracle.dequantize(B, np.ones((1, 1)), None, 1, 16, 16, 3)
    assert list(W[0]) == [float(c - 4) for c in codes[0]]


def test_codes_equal_zero_point_give_zero_weight_and_dense_matmul():
    rng = np.random.default_rng(1)
    N, K, bs = 5, 200, 32
    kb = -(-K // bs)
    zps = rng.integers(0, 8, (N, kb)).astype(np.uint8)
    codes = np.repeat(zps, bs, 1)[:, :K]
    B = oracle.pack_codes(codes, bs, 3)
    zb = oracle.pack_zero_points(zps, 3)
    assert (oracle.dequantize(B, rng.uniform(0.1, 1, (N, kb)), zb, N, K, bs, 3) == 0).all()
    B = rng.integers(0, 256, (N, kb, 3 * bs // 8), dtype=np.uint8)
    s = rng.uniform(0.01, 0.02, (N, kb))
    A = rng.standard_normal((3, K))
    Y, S = oracle.matmul_nbits(A, B, s, zb, None, N, K, bs, 3)
    z = np.repeat(zps.astype(np.int64), bs, 1)[:, :K]
    Wd = (np_codes3(B, K) - z) * np.repeat(s, bs, 1)[:, :K]
    assert np.all(np.abs(Y - A @ Wd.T) <= 1e-12 * S)
