"""Pins of the oracle's float matmul (Y = A W_deq^T + bias, and S).

Checked against hand-derived worked examples (tests/golden/matmul_worked.txt),
an independent dense formulation (numpy bit decoding + float64 matmul),
exact integer matmuls, and the scaling / permutation invariants.
"""
import numpy as np
import pytest

import oracle
from tests.test_oracle_codec import np_codes, np_zero_points


def test_golden_worked_examples(golden):
    B = np.array([[[0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]]], np.uint8)
    scales = np.array([[0.5]])
    for zp_byte, pattern, expect in golden("matmul_worked.txt"):
        zp = None if zp_byte == "none" else np.array([[int(zp_byte, 16)]], np.uint8)
        x = np.ones(16) if pattern == "ones" else np.arange(16, dtype=np.float64)
        y, s = oracle.matmul_nbits(x[None], B, scales, zp, None, 1, 16, 16, 4)
        assert y[0, 0] == float(expect), (zp_byte, pattern)


def dense_reference(A, B, scales, zp, bias, K, bits):
    """Independent formulation: decode fields with numpy, build the dense
    float64 weight, multiply with numpy's matmul."""
    N, kb, blob = B.shape
    bs = blob * 8 // bits
    z = np.repeat(np_zero_points(zp, N, kb, bits), bs, 1)[:, :K]
    W = (np_codes(B, K, bits) - z) * np.repeat(scales, bs, 1)[:, :K]
    Y = A @ W.T
    S = np.abs(A) @ np.abs(W).T
    if bias is not None:
        Y = Y + bias
        S = S + np.abs(bias)
    return Y, S


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("K", [16, 33, 100, 256])
@pytest.mark.parametrize("N", [1, 7, 64])
def test_matches_dense_formulation(bits, K, N):
    bs = 16 if K < 64 else 32
    rng = np.random.default_rng(bits * 10000 + K * 100 + N)
    M = 3
    kb = -(-K // bs)
    A = rng.standard_normal((M, K))
    B = rng.integers(0, 256, size=(N, kb, bs * bits // 8), dtype=np.uint8)
    zp = rng.integers(0, 256, size=(N, -(-kb * bits // 8)), dtype=np.uint8)
    s = rng.uniform(0.002, 0.02, size=(N, kb))
    bias = rng.standard_normal(N)
    for z, b in [(zp, bias), (None, None)]:
        Y, S = oracle.matmul_nbits(A, B, s, z, b, N, K, bs, bits)
        Yr, Sr = dense_reference(A, B, s, z, b, K, bits)
        assert np.all(np.abs(Y - Yr) <= 1e-12 * Sr)
        assert np.allclose(S, Sr, rtol=1e-12, atol=0)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_integer_matmul_when_block_is_whole_row(bits):
    """block_size = K and scale 1 reduce the method to sum_k x_k (q - z):
    an exact integer matmul."""
    rng = np.random.default_rng(40 + bits)
    M, N, K = 4, 9, 64
    codes = rng.integers(0, 1 << bits, size=(N, K)).astype(np.uint8)
    zps = rng.integers(0, 1 << bits, size=(N, 1)).astype(np.uint8)
    x = rng.integers(-3, 4, size=(M, K))
    B = oracle.pack_codes(codes, K, bits)
    zp = oracle.pack_zero_points(zps, bits)
    Y, _ = oracle.matmul_nbits(x.astype(np.float64), B, np.ones((N, 1)), zp, None, N, K, K, bits)
    expect = x.astype(np.int64) @ (codes.astype(np.int64) - zps.astype(np.int64)).T
    assert np.array_equal(Y, expect.astype(np.float64))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_codes_equal_zero_point_give_bias(bits):
    rng = np.random.default_rng(50 + bits)
    M, N, K, bs = 2, 5, 64, 16
    kb = K // bs
    zps = rng.integers(0, 1 << bits, size=(N, kb)).astype(np.uint8)
    B = oracle.pack_codes(np.repeat(zps, bs, 1), bs, bits)
    zp = oracle.pack_zero_points(zps, bits)
    bias = rng.standard_normal(N)
    Y, S = oracle.matmul_nbits(rng.standard_normal((M, K)), B, rng.uniform(0.1, 1, (N, kb)),
                               zp, bias, N, K, bs, bits)
    assert np.array_equal(Y, np.broadcast_to(bias, (M, N)))
    assert np.array_equal(S, np.broadcast_to(np.abs(bias), (M, N)))


def test_doubling_scales_doubles_output():
    rng = np.random.default_rng(60)
    M, N, K, bs, bits = 3, 11, 96, 32, 4
    kb = 3
    A = rng.standard_normal((M, K))
    B = rng.integers(0, 256, size=(N, kb, 16), dtype=np.uint8)
    s = rng.uniform(0.002, 0.02, size=(N, kb))
    zp = rng.integers(0, 256, size=(N, 2), dtype=np.uint8)
    Y1, _ = oracle.matmul_nbits(A, B, s, zp, None, N, K, bs, bits)
    Y2, _ = oracle.matmul_nbits(A, B, 2 * s, zp, None, N, K, bs, bits)
    assert np.array_equal(Y2, 2 * Y1)


def test_permuting_rows_permutes_output():
    rng = np.random.default_rng(61)
    M, N, K, bs, bits = 2, 13, 64, 16, 4
    kb = 4
    A = rng.standard_normal((M, K))
    B = rng.integers(0, 256, size=(N, kb, 8), dtype=np.uint8)
    s = rng.uniform(0.002, 0.02, size=(N, kb))
    zp = rng.integers(0, 256, size=(N, 2), dtype=np.uint8)
    perm = rng.permutation(N)
    Y, _ = oracle.matmul_nbits(A, B, s, zp, None, N, K, bs, bits)
    Yp, _ = oracle.matmul_nbits(A, B[perm], s[perm], zp[perm], None, N, K, bs, bits)
    assert np.array_equal(Yp, Y[:, perm])


def test_mutating_one_code_moves_one_output():
    """A change of one code by +1 moves exactly output n by x_k * scale."""
    rng = np.random.default_rng(62)
    M, N, K, bs, bits = 2, 4, 32, 16, 4
    codes = rng.integers(0, 15, size=(N, K)).astype(np.uint8)
    s = np.full((N, 2), 0.25)
    A = rng.integers(-4, 5, size=(M, K)).astype(np.float64)
    Y0, _ = oracle.matmul_nbits(A, oracle.pack_codes(codes, bs, bits), s, None, None, N, K, bs, bits)
    codes[2, 19] += 1
    Y1, _ = oracle.matmul_nbits(A, oracle.pack_codes(codes, bs, bits), s, None, None, N, K, bs, bits)
    d = Y1 - Y0
    assert np.array_equal(d[:, [0, 1, 3]], np.zeros((M, 3)))
    assert np.array_equal(d[:, 2], A[:, 19] * 0.25)
