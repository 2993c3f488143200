"""Pins of the oracle's int8 convolution with requantization.

Checked against hand-derived rounding ties (tests/golden/conv_requant_ties.txt),
an independent numpy formulation (explicit zero-point padding, one int64
tensordot per tap, numpy float32 requantization), the 1x1 case reducing to an
int8 matmul with requantization, and saturation.
"""
import numpy as np
import pytest

import oracle


def test_golden_requant_ties(golden):
    rows = golden("conv_requant_ties.txt")
    acc = np.array([int(r[0]) for r in rows], np.int8)
    expect = np.array([int(r[1]) for r in rows], np.int8)
    X = acc.reshape(1, 1, len(acc), 1)
    W = np.ones((1, 1, 1, 1), np.int8)
    Y, A = oracle.conv_int8(X, W, np.zeros(1, np.int32), np.array([0.25], np.float32),
                            0.5, 0.25)
    assert np.array_equal(A.ravel(), acc.astype(np.int32))
    assert np.array_equal(Y.ravel(), expect)


def np_conv(X, W, bias, w_scale, in_scale, out_scale, in_zp, out_zp, lo, hi, stride, pad):
    Nb, H, Wd, C = X.shape
    Co, KH, KW, _ = W.shape
    sh, sw = stride
    ph, pw = pad
    OH = (H + 2 * ph - KH) // sh + 1
    OW = (Wd + 2 * pw - KW) // sw + 1
    Xp = np.pad(X.astype(np.int64), ((0, 0), (ph, ph), (pw, pw), (0, 0)), constant_values=in_zp)
    Xp = Xp - in_zp
    acc = np.broadcast_to(bias.astype(np.int64), (Nb, OH, OW, Co)).copy()
    for kh in range(KH):
        for kw in range(KW):
            patch = Xp[:, kh:kh + sh * (OH - 1) + 1:sh, kw:kw + sw * (OW - 1) + 1:sw, :]
            acc += np.tensordot(patch, W[:, kh, kw, :].astype(np.int64), axes=([3], [1]))
    mult = (np.float32(in_scale) * w_scale.astype(np.float32)) / np.float32(out_scale)
    r = np.rint(acc.astype(np.float32) * mult.astype(np.float32))
    y = np.clip(r.astype(np.float64) + out_zp, lo, hi).astype(np.int8)
    return y, acc.astype(np.int32)


@pytest.mark.parametrize("shape,k,stride,pad", [
    ((1, 5, 5, 3), (2, 3, 3), (1, 1), (1, 1)),
    ((1, 5, 5, 3), (2, 3, 3), (2, 2), (0, 0)),
    ((2, 7, 6, 4), (5, 3, 3), (2, 1), (1, 0)),
    ((1, 9, 9, 8), (3, 5, 5), (1, 1), (2, 2)),
    ((1, 6, 6, 16), (8, 1, 1), (1, 1), (0, 0)),
])
@pytest.mark.parametrize("in_zp,out_zp", [(0, 0), (3, -5), (-7, 10)])
def test_matches_numpy_formulation(shape, k, stride, pad, in_zp, out_zp):
    rng = np.random.default_rng(sum(shape) * 31 + sum(k) + in_zp * 7 + out_zp)
    Nb, H, Wd, C = shape
    Co, KH, KW = k
    X = rng.integers(-128, 128, size=shape, dtype=np.int8)
    W = rng.integers(-127, 128, size=(Co, KH, KW, C), dtype=np.int8)
    bias = rng.integers(-1000, 1001, size=Co).astype(np.int32)
    ws = rng.uniform(0.001, 0.01, size=Co).astype(np.float32)
    args = (bias, ws, 0.02, 0.05, in_zp, out_zp, -128, 127, stride, pad)
    Y, A = oracle.conv_int8(X, W, bias, ws, 0.02, 0.05, in_zp, out_zp, -128, 127, stride, pad)
    Yn, An = np_conv(X, W, *args)
    assert np.array_equal(A, An)
    assert np.array_equal(Y, Yn)


def test_pointwise_conv_is_requantized_int8_matmul():
    """A 1x1, stride-1, unpadded conv is the int8 QMatMul of rlx-cpu
    quant.rs (exec_q_mat_mul) with a per-channel multiplier."""
    rng = np.random.default_rng(5)
    P, C, Co = 30, 16, 6
    x = rng.integers(-128, 128, size=(P, C), dtype=np.int8)
    w = rng.integers(-127, 128, size=(Co, C), dtype=np.int8)
    bias = rng.integers(-1000, 1001, size=Co).astype(np.int32)
    ws = rng.uniform(0.001, 0.01, size=Co).astype(np.float32)
    x_zp, out_zp = 4, -3
    Y, A = oracle.conv_int8(x.reshape(1, 1, P, C), w.reshape(Co, 1, 1, C), bias, ws, 0.02, 0.05,
                            x_zp, out_zp)
    acc = bias.astype(np.int64) + (x.astype(np.int64) - x_zp) @ w.astype(np.int64).T
    assert np.array_equal(A.reshape(P, Co), acc)
    mult = (np.float32(0.02) * ws) / np.float32(0.05)
    y = np.clip(np.rint(acc.astype(np.float32) * mult) + out_zp, -128, 127)
    assert np.array_equal(Y.reshape(P, Co), y.astype(np.int8))


def test_saturation_and_relu_clamp():
    X = np.full((1, 3, 3, 4), 127, np.int8)
    W = np.full((2, 3, 3, 4), 127, np.int8)
    W[1] = -127
    ws = np.array([1.0, 1.0], np.float32)
    Y, _ = oracle.conv_int8(X, W, np.zeros(2, np.int32), ws, 1.0, 1.0, pad=(1, 1))
    assert (Y[..., 0] == 127).all() and (Y[..., 1] == -128).all()
    # ReLU-style clamp: the lower bound equals the output zero point.
    Y, _ = oracle.conv_int8(X, W, np.zeros(2, np.int32), ws, 1.0, 1.0, out_zp=5, clamp_min=5,
                            pad=(1, 1))
    assert (Y[..., 1] == 5).all()


def test_padding_reads_input_zero_point():
    """With every input equal to in_zp, all taps (padded or not) contribute 0."""
    X = np.full((1, 4, 4, 2), 9, np.int8)
    W = np.ones((1, 3, 3, 2), np.int8)
    Y, A = oracle.conv_int8(X, W, np.array([17], np.int32), np.array([1.0], np.float32), 1.0, 1.0,
                            in_zp=9, pad=(1, 1))
    assert (A == 17).all() and (Y == 17).all()
