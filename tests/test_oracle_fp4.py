"""Pins of the oracle's block-scaled FP4 weights (MXFP4 / NVFP4).

rlx-cpu quant.rs (dequant_matmul_nvfp4; lowp_dequantize, lowp_scaled_matmul):
w(n, k) = e2m1(code) * scale(block) (* global scale for NVFP4).  Checked
against the E2M1 value table (tests/golden/e2m1_values.txt), PyTorch's own
float8_e4m3fn / float8_e8m0fnu decoders for every scale byte, hand-derived
worked examples, an independent dense formulation on PyTorch-decoded scales,
the page's own [K, N] flat packing (the same weights re-laid out), and the
scaling invariants.
"""
import numpy as np
import pytest
import torch

import oracle

E2M1 = None


def e2m1_table(golden):
    return np.array([float(v) for _, v in golden("e2m1_values.txt")])


def test_e2m1_values(golden):
    rows = golden("e2m1_values.txt")
    assert len(rows) == 16
    for code, v in rows:
        got = oracle.e2m1(int(code))
        assert got == float(v) and np.signbit(got) == np.signbit(float(v)), code


def test_scale_bytes_match_torch_decoders():
    b = torch.arange(256, dtype=torch.uint8)
    e4 = b.view(torch.float8_e4m3fn).double().numpy()
    e8 = b.view(torch.float8_e8m0fnu).double().numpy()
    for i in range(256):
        for got, want in ((oracle.e4m3(i), e4[i]), (oracle.e8m0(i), e8[i])):
            assert (np.isnan(got) and np.isnan(want)) or got == want, (i, got, want)


def test_worked_examples():
    # One row, codes k % 16 (bytes 0x10 0x32 ... 0xFE), activations 1 for the
    # first 8 elements (codes 0..7: sum of e2m1 = 0+0.5+1+1.5+2+3+4+6 = 18).
    row = np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE], np.uint8)
    x = np.zeros((1, 32))
    x[0, :8] = 1
    # MXFP4: one block of 32, E8M0 byte 128 = 2.0: y = 2 * 18 = 36.
    W = np.concatenate([row, row])[None]
    y, _ = oracle.fp4_matmul(x, W, np.array([[128]], np.uint8), "mxfp4", 1.0, None, 1, 32)
    assert y[0, 0] == 36.0
    # NVFP4: two blocks of 16, E4M3 bytes 0x38 (1.0) and 0x40 (2.0), global
    # 0.5: the first block gives 0.5 * 18 = 9; activations on codes 8..15 of
    # the second block (sum -18) add 0.5 * 2 * -18 = -18.
    x2 = x.copy()
    x2[0, 24:32] = 1
    y, _ = oracle.fp4_matmul(x2, W, np.array([[0x38, 0x40]], np.uint8), "nvfp4", 0.5, None, 1,
                             32)
    assert y[0, 0] == 9.0 - 18.0


def case(fmt, M, K, N, seed, global_scale=1.0):
    rng = np.random.default_rng(seed)
    bs = oracle.FP4_BLOCK[fmt]
    kb = -(-K // bs)
    A = rng.standard_normal((M, K))
    W = rng.integers(0, 256, (N, kb * bs // 2), dtype=np.uint8)
    if fmt == "mxfp4":
        sc = rng.integers(120, 135, (N, kb), dtype=np.uint8)
    else:
        sc = rng.integers(0x20, 0x58, (N, kb), dtype=np.uint8)   # finite E4M3, both signs off
    return A, W, sc, global_scale


def dense_reference(A, W, sc, fmt, g, K, golden):
    """Codes split with numpy, values from the golden table, scales decoded
    by PyTorch's float8 types, then a float64 matmul."""
    tab = e2m1_table(golden)
    N = W.shape[0]
    codes = np.stack([W & 0x0F, W >> 4], axis=-1).reshape(N, -1)[:, :K]
    dt = torch.float8_e8m0fnu if fmt == "mxfp4" else torch.float8_e4m3fn
    s = torch.from_numpy(sc).view(dt).double().numpy()
    bs = oracle.FP4_BLOCK[fmt]
    Wd = tab[codes] * np.repeat(s, bs, axis=1)[:, :K] * g
    return A @ Wd.T, np.abs(A) @ np.abs(Wd).T


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_matches_an_independent_formulation(fmt, golden):
    for i, (M, K, N) in enumerate([(1, 32, 5), (3, 100, 7), (2, 512, 33)]):
        A, W, sc, g = case(fmt, M, K, N, 10 + i, 0.75 if fmt == "nvfp4" else 1.0)
        Y, S = oracle.fp4_matmul(A, W, sc, fmt, g, None, N, K)
        Yr, Sr = dense_reference(A, W, sc, fmt, g, K, golden)
        assert np.all(np.abs(Y - Yr) <= 1e-12 * Sr)
        assert np.allclose(S, Sr, rtol=1e-12, atol=0)


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_the_pages_k_by_n_packing_is_the_same_weight(fmt):
    """dequant_matmul_nvfp4 packs a flat [K, N] index (nibble of p*n + j,
    low nibble first) with scales [K / gs, N]; the same weights re-laid out
    as [N, K] rows (this library's reading) give the same product."""
    K, N, M = 64, 6, 2
    A, W, sc, g = case(fmt, M, K, N, 3, 0.5 if fmt == "nvfp4" else 1.0)
    bs = oracle.FP4_BLOCK[fmt]
    codes = np.stack([W & 0x0F, W >> 4], axis=-1).reshape(N, K)      # [N, K]
    flat = codes.T.reshape(-1)                                        # index p * N + j
    kn = (flat[0::2] | (flat[1::2] << 4)).astype(np.uint8)
    dec = oracle.e8m0 if fmt == "mxfp4" else oracle.e4m3
    Y = np.zeros((M, N))
    for i in range(M):
        for j in range(N):
            acc = 0.0
            for p in range(K):
                idx = p * N + j
                nib = kn[idx // 2] & 0x0F if idx % 2 == 0 else kn[idx // 2] >> 4
                acc += A[i, p] * oracle.e2m1(nib) * dec(sc.T[p // bs, j]) * g
            Y[i, j] = acc
    Yo, S = oracle.fp4_matmul(A, W, sc, fmt, g, None, N, K)
    assert np.all(np.abs(Y - Yo) <= 1e-12 * S)


def test_scaling_invariants():
    A, W, sc, g = case("mxfp4", 2, 256, 9, 5)
    Y, _ = oracle.fp4_matmul(A, W, sc, "mxfp4", 1.0, None, 9, 256)
    Y2, _ = oracle.fp4_matmul(A, W, sc + 1, "mxfp4", 1.0, None, 9, 256)   # every scale x2
    assert np.array_equal(Y2, 2 * Y)
    A, W, sc, g = case("nvfp4", 2, 256, 9, 6, 1.0)
    Y, _ = oracle.fp4_matmul(A, W, sc, "nvfp4", 1.0, None, 9, 256)
    Y4, _ = oracle.fp4_matmul(A, W, sc, "nvfp4", 0.25, None, 9, 256)
    assert np.array_equal(Y4, Y * 0.25)
    # A nan scale (E8M0 255) makes its row's outputs nan.
    A, W, sc, g = case("mxfp4", 1, 64, 3, 7)
    sc[1, 1] = 255
    Y, _ = oracle.fp4_matmul(A, W, sc, "mxfp4", 1.0, None, 3, 64)
    assert np.isnan(Y[0, 1]) and not np.isnan(Y[0, 0]) and not np.isnan(Y[0, 2])
