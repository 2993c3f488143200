"""Pins of the oracle's group-index (g_idx, act-order) branch.

MatMulNBits input 4 (onnx-runtime-ep-cpu matmul_nbits.rs, dequantize_weight
and execute): element k keeps its code from block k / bs, but its scale and
zero point come from group g_idx[k]; g_idx has shape [K] or [kb * bs] and
every entry must lie in 0..kb.  Checked against hand-derived values
(tests/golden/gidx_worked.txt), the plain operator (g_idx = k / bs must
reproduce it bit for bit), an independent numpy formulation (numpy bit
decoding + fancy indexing of the scales and zero points), the permutation
invariance of K, and the range / shape checks.
"""
import numpy as np
import pytest

import oracle
from tests.test_oracle_codec import np_codes, np_zero_points

ROW = np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE], np.uint8)


def test_golden_worked_examples(golden):
    B = np.stack([ROW, ROW])[None]                  # [1, 2, 8]: codes k % 16
    scales = np.array([[0.5, 2.0]])
    zp = np.array([[0x31]], np.uint8)
    k = np.arange(32)
    g_of = {"blocks": k // 16, "swapped": 1 - k // 16, "alternate": k % 2,
            "all1": np.ones(32, np.int64)}
    x_of = {"ones": np.ones(32), "first16": (k < 16).astype(np.float64)}
    for gp, xp, expect in golden("gidx_worked.txt"):
        y, _ = oracle.matmul_nbits(x_of[xp][None], B, scales, zp, None, 1, 32, 16, 4,
                                   g_idx=g_of[gp].astype(np.int32))
        assert y[0, 0] == float(expect), (gp, xp)
        W = oracle.dequantize(B, scales, zp, 1, 32, 16, 4, g_idx=g_of[gp].astype(np.int32))
        assert float(W[0] @ x_of[xp]) == float(expect), (gp, xp)


def case(M, K, N, bs, bits, seed, has_zp=True):
    rng = np.random.default_rng(seed)
    kb = -(-K // bs)
    A = rng.standard_normal((M, K))
    B = rng.integers(0, 256, (N, kb, bs * bits // 8), dtype=np.uint8)
    s = rng.uniform(0.002, 0.02, (N, kb))
    zp = rng.integers(0, 256, (N, -(-kb * bits // 8)), dtype=np.uint8) if has_zp else None
    return rng, A, B, s, zp, kb


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("K,bs", [(64, 16), (100, 32), (256, 64)])
def test_block_indices_reproduce_the_plain_operator(bits, K, bs):
    _, A, B, s, zp, kb = case(3, K, 9, bs, bits, K + bits)
    bias = np.linspace(-1, 1, 9)
    Y0, S0 = oracle.matmul_nbits(A, B, s, zp, bias, 9, K, bs, bits)
    g = (np.arange(K) // bs).astype(np.int32)
    Y1, S1 = oracle.matmul_nbits(A, B, s, zp, bias, 9, K, bs, bits, g_idx=g)
    assert np.array_equal(Y0, Y1) and np.array_equal(S0, S1)
    # The padded shape [kb * bs] is accepted too; its tail is not used.
    gp = (np.arange(kb * bs) // bs).astype(np.int32)
    Y2, _ = oracle.matmul_nbits(A, B, s, zp, bias, 9, K, bs, bits, g_idx=gp)
    assert np.array_equal(Y0, Y2)


def dense_gidx(A, B, s, zp, g, K, bits):
    """Independent formulation: numpy-decoded codes, per-element scale and
    zero point gathered with fancy indexing, float64 matmul."""
    N, kb, blob = B.shape
    q = np_codes(B, K, bits)
    z = np_zero_points(zp, N, kb, bits)[:, g[:K]]
    W = (q - z) * s[:, g[:K]]
    return A @ W.T, np.abs(A) @ np.abs(W).T


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("has_zp", [True, False])
def test_matches_an_independent_formulation(bits, has_zp):
    for i, (K, bs) in enumerate([(33, 16), (128, 32), (300, 64)]):
        rng, A, B, s, zp, kb = case(4, K, 7, bs, bits, 10 * bits + i, has_zp)
        g = rng.integers(0, kb, K).astype(np.int32)
        Y, S = oracle.matmul_nbits(A, B, s, zp, None, 7, K, bs, bits, g_idx=g)
        Yr, Sr = dense_gidx(A, B, s, zp, g, K, bits)
        assert np.all(np.abs(Y - Yr) <= 1e-12 * Sr)
        assert np.allclose(S, Sr, rtol=1e-12, atol=0)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_permuting_k_together_leaves_y_unchanged(bits):
    """Permute the columns of A, the codes and g_idx by the same permutation
    (the codes repacked at their new positions, scales and zero points
    untouched): y is unchanged up to the order of the sum."""
    K, bs, N = 256, 32, 11
    rng, A, B, s, zp, kb = case(2, K, N, bs, bits, 77 + bits)
    g = rng.integers(0, kb, K).astype(np.int32)
    perm = rng.permutation(K)
    codes = oracle.unpack_codes(B, N, K, bs, bits)
    Bp = oracle.pack_codes(codes[:, perm], bs, bits)
    Y, S = oracle.matmul_nbits(A, B, s, zp, None, N, K, bs, bits, g_idx=g)
    Yp, Sp = oracle.matmul_nbits(A[:, perm], Bp, s, zp, None, N, K, bs, bits, g_idx=g[perm])
    assert np.all(np.abs(Y - Yp) <= 1e-12 * S)
    assert np.allclose(S, Sp, rtol=1e-12, atol=0)


def test_act_order_groups_equal_a_permuted_plain_operator():
    """The act-order pattern: g_idx[k] = rank(k) // bs for a permutation of K.
    Gathering the codes and activations into rank order turns it into the
    plain operator (blocks = groups) on the permuted problem."""
    K, bs, N, bits = 128, 32, 5, 4
    rng, A, B, s, zp, kb = case(3, K, N, bs, bits, 5)
    order = rng.permutation(K)               # order[j] = k placed at rank j
    rank = np.empty(K, np.int64)
    rank[order] = np.arange(K)
    g = (rank // bs).astype(np.int32)
    Y, S = oracle.matmul_nbits(A, B, s, zp, None, N, K, bs, bits, g_idx=g)
    codes = oracle.unpack_codes(B, N, K, bs, bits)
    Bp = oracle.pack_codes(codes[:, order], bs, bits)
    Yp, _ = oracle.matmul_nbits(A[:, order], Bp, s, zp, None, N, K, bs, bits)
    assert np.all(np.abs(Y - Yp) <= 1e-12 * S)


def test_range_and_shape_checks():
    K, bs = 100, 32                          # kb = 4, padded K = 128
    ok = np.zeros(K, np.int32)
    oracle.check_g_idx(ok, K, bs)
    oracle.check_g_idx(np.zeros(128, np.int32), K, bs)
    for bad, where in [(4, 7), (-1, 0), (1 << 30, 99)]:
        g = ok.copy()
        g[where] = bad
        with pytest.raises(oracle.GroupIndexError, match=rf"g_idx\[{where}\]={bad} is outside 0\.\.4"):
            oracle.check_g_idx(g, K, bs)
        with pytest.raises(oracle.GroupIndexError):
            oracle.matmul_nbits(np.ones((1, K)), np.zeros((1, 4, 16), np.uint8), np.ones((1, 4)),
                                None, None, 1, K, bs, 4, g_idx=g)
    # The padding entries of a [kb * bs] index are checked as well.
    gp = np.zeros(128, np.int32)
    gp[120] = 9
    with pytest.raises(oracle.GroupIndexError, match=r"g_idx\[120\]=9"):
        oracle.check_g_idx(gp, K, bs)
    for n in (K - 1, K + 1, 127, 129):
        with pytest.raises(oracle.GroupIndexError, match="must have shape"):
            oracle.check_g_idx(np.zeros(n, np.int32), K, bs)
