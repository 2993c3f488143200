"""Pins of the oracle's CompInt8 steps: activation quantization, exact int32
block dots and the scaled float output.

Checked against hand-derived rounding ties (tests/golden/quantize_a_ties.txt),
an independent numpy float32 formulation of the quantizer, the integer
identities the CompInt8 kernels rely on (zero-point split, u8 offset), brute
force block dots, and independence from how N is split.
"""
import numpy as np
import pytest

import oracle
from tests.test_oracle_codec import np_codes, np_zero_points


def test_golden_ties(golden):
    rows = golden("quantize_a_ties.txt")
    x = np.array([float(r[0]) for r in rows], np.float32)
    expect = np.array([int(r[1]) for r in rows], np.int8)
    qa, sa = oracle.quantize_a(x[None], len(x), 16)
    assert sa[0, 0] == np.float32(1.0)
    assert np.array_equal(qa[0, :len(x)], expect)
    assert (qa[0, len(x):] == 0).all()          # padding past K is zero


def np_quantize(x, bs):
    """Independent float32 formulation of the per-block quantizer."""
    M, K = x.shape
    kb = -(-K // bs)
    xp = np.zeros((M, kb * bs), np.float32)
    xp[:, :K] = x
    blocks = xp.reshape(M, kb, bs)
    amax = np.abs(blocks).max(-1)
    sa = (amax / np.float32(127)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(blocks / sa[..., None])
    q = np.where(sa[..., None] == 0, 0, np.clip(q, -127, 127))
    return q.reshape(M, kb * bs).astype(np.int8), sa


@pytest.mark.parametrize("K,bs", [(16, 16), (100, 32), (256, 64), (300, 128), (4096, 128)])
def test_quantize_matches_numpy_float32(K, bs):
    rng = np.random.default_rng(K + bs)
    x = rng.standard_normal((5, K)).astype(np.float32) * rng.uniform(0.01, 100, (5, 1)).astype(np.float32)
    x[1, :bs] = 0                                            # an all-zero block
    qa, sa = oracle.quantize_a(x, K, bs)
    qn, sn = np_quantize(x, bs)
    assert np.array_equal(sa, sn)
    assert np.array_equal(qa, qn)


def test_quantize_invariants():
    rng = np.random.default_rng(3)
    K, bs = 512, 64
    x = (rng.standard_normal((4, K)) * 3).astype(np.float32)
    qa, sa = oracle.quantize_a(x, K, bs)
    assert np.abs(qa.astype(np.int32)).max() <= 127
    blocks = x.reshape(4, K // bs, bs)
    idx = np.abs(blocks).argmax(-1)
    q = qa.reshape(4, K // bs, bs)
    for m in range(4):
        for b in range(K // bs):
            v = blocks[m, b, idx[m, b]]
            assert q[m, b, idx[m, b]] == (127 if v > 0 else -127)
    z = np.zeros((1, K), np.float32)
    qz, sz = oracle.quantize_a(z, K, bs)
    assert (qz == 0).all() and (sz == 0).all()


def np_block_dots(qa, B, zp, K, bits):
    N, kb, blob = B.shape
    bs = blob * 8 // bits
    M = qa.shape[0]
    w = np.zeros((N, kb * bs), np.int64)
    w[:, :K] = np_codes(B, K, bits) - np.repeat(np_zero_points(zp, N, kb, bits), bs, 1)[:, :K]
    return np.einsum("mbk,nbk->mnb", qa.astype(np.int64).reshape(M, kb, bs), w.reshape(N, kb, bs))


@pytest.mark.parametrize("bits,bs,asym", [(4, 128, False), (8, 64, True), (2, 64, True),
                                          (4, 32, True), (4, 16, False)])
@pytest.mark.parametrize("K", [128, 200])
def test_block_dots_brute_force_and_identities(bits, bs, asym, K):
    rng = np.random.default_rng(bits * 100 + bs + K)
    M, N = 3, 10
    kb = -(-K // bs)
    x = rng.standard_normal((M, K)).astype(np.float32)
    qa, sa = oracle.quantize_a(x, K, bs)
    B = rng.integers(0, 256, size=(N, kb, bs * bits // 8), dtype=np.uint8)
    zp = rng.integers(0, 256, size=(N, -(-kb * bits // 8)), dtype=np.uint8) if asym else None
    dots = oracle.compint8_block_dots(qa, B, zp, N, K, bs, bits)
    assert np.array_equal(dots, np_block_dots(qa, B, zp, K, bits))
    # Zero-point split: sum qa (q - z) = sum qa q - z sum qa.
    q = np.zeros((N, kb * bs), np.int64)
    q[:, :K] = np_codes(B, K, bits)
    z = np_zero_points(zp, N, kb, bits)
    qa3 = qa.astype(np.int64).reshape(M, kb, bs)
    split = np.einsum("mbk,nbk->mnb", qa3, q.reshape(N, kb, bs)) - z[None] * qa3.sum(-1)[:, None]
    assert np.array_equal(dots, split)
    # u8 offset: sum (qa + 128)(q - z) - 128 sum (q - z) = sum qa (q - z).
    wz = q.reshape(N, kb, bs) - z[..., None]
    wz[:, :, :][np.broadcast_to(np.arange(kb * bs).reshape(kb, bs) >= K, wz.shape)] = 0
    off = np.einsum("mbk,nbk->mnb", qa3 + 128, wz) - 128 * wz.sum(-1)[None]
    assert np.array_equal(dots, off)


def test_block_dots_do_not_depend_on_column_split():
    rng = np.random.default_rng(77)
    M, N, K, bs, bits = 2, 16, 256, 64, 4
    qa, _ = oracle.quantize_a(rng.standard_normal((M, K)).astype(np.float32), K, bs)
    B = rng.integers(0, 256, size=(N, K // bs, bs // 2), dtype=np.uint8)
    zp = rng.integers(0, 256, size=(N, 2), dtype=np.uint8)
    full = oracle.compint8_block_dots(qa, B, zp, N, K, bs, bits)
    a = oracle.compint8_block_dots(qa, B[:5], zp[:5], 5, K, bs, bits)
    b = oracle.compint8_block_dots(qa, B[5:], zp[5:], N - 5, K, bs, bits)
    assert np.array_equal(full, np.concatenate([a, b], axis=1))


def test_compint8_output_matches_block_formula():
    rng = np.random.default_rng(78)
    M, N, K, bs, bits = 3, 12, 320, 64, 8
    kb = K // bs
    qa, sa = oracle.quantize_a(rng.standard_normal((M, K)).astype(np.float32), K, bs)
    B = rng.integers(0, 256, size=(N, kb, bs), dtype=np.uint8)
    zp = rng.integers(0, 256, size=(N, kb), dtype=np.uint8)
    s = rng.uniform(0.002, 0.02, size=(N, kb))
    bias = rng.standard_normal(N)
    Y, S = oracle.compint8_matmul(qa, sa, B, s, zp, bias, N, K, bs, bits)
    dots = np_block_dots(qa, B, zp, K, bits).astype(np.float64)
    f = sa.astype(np.float64)[:, None, :] * s[None]
    assert np.allclose(Y, (dots * f).sum(-1) + bias, rtol=1e-13, atol=1e-13)
    # S bounds |Y - bias| and is the sum of per-element magnitudes.
    assert np.all(np.abs(Y - bias) <= S - np.abs(bias) + 1e-12)


def test_compint8_close_to_float_matmul():
    """CompInt8 approximates the float product: per block the activation
    error is at most half a quantization step, sa/2 per element."""
    rng = np.random.default_rng(79)
    M, N, K, bs, bits = 2, 8, 256, 32, 4
    kb = K // bs
    x = rng.standard_normal((M, K)).astype(np.float32)
    qa, sa = oracle.quantize_a(x, K, bs)
    B = rng.integers(0, 256, size=(N, kb, bs // 2), dtype=np.uint8)
    s = rng.uniform(0.002, 0.02, size=(N, kb))
    Yc, _ = oracle.compint8_matmul(qa, sa, B, s, None, None, N, K, bs, bits)
    Yf, _ = oracle.matmul_nbits(x.astype(np.float64), B, s, None, None, N, K, bs, bits)
    W = np.abs(oracle.dequantize(B, s, None, N, K, bs, bits))
    bound = (np.repeat(sa.astype(np.float64), bs, 1)[:, :K] / 2) @ W.T
    assert np.all(np.abs(Yc - Yf) <= bound * (1 + 1e-6) + 1e-12)
