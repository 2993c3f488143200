"""Pins of the oracle's int16-activation route (the 8-bit path of
onnx-runtime-ep-cpu matmul_nbits.rs execute: activations quantized to int16
per K-block, an integer dot against the codes).  Reading: the int8
quantizer with 32767 (sa = max|x| / 32767, round half to even).

Checked against exact ties, an independent numpy float32 quantizer, the
invariants of the quantizer, an int64 brute-force block dot, and the page's
claim that int16 keeps the fp32 result (the error is bounded by half a
quantization step per element).
"""
import numpy as np
import pytest

import oracle


def test_ties_round_half_to_even():
    x = np.zeros((1, 16), np.float32)
    x[0, :6] = [32767.0, 2.5, 3.5, -2.5, -0.5, 1.5]
    qa, sa = oracle.quantize_a16(x, 16, 16)
    assert sa[0, 0] == 1.0
    assert list(qa[0, :6]) == [32767, 2, 4, -2, 0, 2]


@pytest.mark.parametrize("bs", [16, 64, 128])
def test_matches_numpy_float32_quantizer(bs):
    rng = np.random.default_rng(bs)
    M, K = 3, 5 * bs - 7
    A = (rng.standard_normal((M, K)) * rng.uniform(0.01, 100, (M, 1))).astype(np.float32)
    A[1, :bs] = 0.0                                   # an all-zero block
    qa, sa = oracle.quantize_a16(A, K, bs)
    kb = -(-K // bs)
    Ap = np.zeros((M, kb * bs), np.float32)
    Ap[:, :K] = A
    amax = np.abs(Ap).reshape(M, kb, bs).max(-1)
    s = (amax / np.float32(32767.0)).astype(np.float32)
    assert np.array_equal(s, sa)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(Ap.reshape(M, kb, bs) / s[..., None].astype(np.float32))
    q = np.where(s[..., None] == 0, 0, np.clip(q, -32767, 32767)).reshape(M, kb * bs)
    assert np.array_equal(q.astype(np.int16), qa)
    assert np.abs(qa).max() == 32767 and (qa[1, :bs] == 0).all() and (sa[1, 0] == 0)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_block_dot_brute_force_and_fp32_closeness(bits):
    rng = np.random.default_rng(bits)
    M, K, N, bs = 2, 300, 9, 64
    kb = -(-K // bs)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.integers(0, 256, (N, kb, bs * bits // 8), dtype=np.uint8)
    s = rng.uniform(0.002, 0.02, (N, kb))
    zp = rng.integers(0, 256, (N, -(-kb * bits // 8)), dtype=np.uint8)
    qa, sa = oracle.quantize_a16(A, K, bs)
    Y, S = oracle.int16_matmul(qa, sa, B, s, zp, None, N, K, bs, bits)
    codes = oracle.unpack_codes(B, N, K, bs, bits).astype(np.int64)
    z = np.repeat(oracle.unpack_zero_points(zp, N, kb, bits).astype(np.int64), bs, 1)[:, :K]
    q = qa[:, :K].astype(np.int64)
    Yb = np.zeros((M, N))
    for b in range(kb):
        sl = slice(b * bs, min(K, (b + 1) * bs))
        dot = q[:, sl] @ (codes[:, sl] - z[:, sl]).T            # exact int64
        Yb += dot * (sa[:, b:b + 1].astype(np.float64) * s[:, b][None, :])
    assert np.all(np.abs(Y - Yb) <= 1e-12 * S)
    # Within half a quantization step per element of the float result.
    Yf, _ = oracle.matmul_nbits(A.astype(np.float64), B, s, zp, None, N, K, bs, bits)
    W = np.abs(oracle.dequantize(B, s, zp, N, K, bs, bits))
    step = np.repeat(sa.astype(np.float64), bs, 1)[:, :K]
    assert np.all(np.abs(Y - Yf) <= 0.5 * (step @ W.T) * (1 + 1e-9))
