"""Pins of the oracle's low-precision scaled GEMM (rlx-cpu quant.rs: the
FP8 / FP6 / FP4 scaled-GEMM reference lowp_compute_scales, lowp_quantize,
lowp_dequantize, lowp_scaled_matmul, lowp_snap_scale, lowp_read_scales).

The element codec is not printed on the pages; the oracle decodes from the
published format definitions and encodes by its stated reading (nearest
finite value, ties to even, saturating).  Pinned against: PyTorch's own
float8_e4m3fn / float8_e5m2 decoders and encoders (in range), the formats'
published limits (tests/golden/lowp_format_limits.txt), the E2M1 table
already pinned for FP4 weights, monotonicity and round trips of every code,
brute-force tie cases, the defining property of each scale snap, and an
independent dense formulation of the matmul on PyTorch-decoded values.
"""
import numpy as np
import pytest
import torch

import oracle

FMTS = ["e4m3", "e5m2", "e2m3", "e3m2", "e2m1"]
BITS = {"e4m3": 8, "e5m2": 8, "e2m3": 6, "e3m2": 6, "e2m1": 4}


def finite_codes(fmt):
    """Non-negative finite codes in code order."""
    n = 1 << (BITS[fmt] - 1)
    return [c for c in range(n) if np.isfinite(oracle.lowp_decode(fmt, c))]


def test_fp8_decode_matches_torch():
    b = torch.arange(256, dtype=torch.uint8)
    for fmt, dt in (("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)):
        ref = b.view(dt).double().numpy()
        for i in range(256):
            got = oracle.lowp_decode(fmt, i)
            assert (np.isnan(got) and np.isnan(ref[i])) or got == ref[i], (fmt, i, got, ref[i])


def test_e2m1_matches_the_pinned_table(golden):
    for code, v in golden("e2m1_values.txt"):
        got = oracle.lowp_decode("e2m1", int(code))
        assert got == float(v) and np.signbit(got) == np.signbit(float(v))


def test_published_limits(golden):
    for fmt, mx, mn_norm, mx_sub, mn_sub in golden("lowp_format_limits.txt"):
        vals = [oracle.lowp_decode(fmt, c) for c in finite_codes(fmt)]
        pos = [v for v in vals if v > 0]
        assert max(vals) == float(mx) == oracle.lowp_max_finite(fmt), fmt
        assert min(pos) == float(mn_sub), fmt
        mb = {"e4m3": 3, "e5m2": 2, "e2m3": 3, "e3m2": 2, "e2m1": 1}[fmt]
        sub = [oracle.lowp_decode(fmt, c) for c in range(1, 1 << mb)]
        assert max(sub) == float(mx_sub) and oracle.lowp_decode(fmt, 1 << mb) == float(mn_norm)


@pytest.mark.parametrize("fmt", FMTS)
def test_codes_are_monotone_and_signed(fmt):
    codes = finite_codes(fmt)
    vals = [oracle.lowp_decode(fmt, c) for c in codes]
    assert all(a < b for a, b in zip(vals[1:], vals[2:])) and vals[0] == 0.0
    sb = 1 << (BITS[fmt] - 1)
    for c in codes:
        v, n = oracle.lowp_decode(fmt, c), oracle.lowp_decode(fmt, c | sb)
        assert n == -v and np.signbit(n)
        # Bits above the format's width are ignored.
        assert oracle.lowp_decode(fmt, c | (1 << BITS[fmt])) == v if BITS[fmt] < 8 else True


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_round_trips_and_ties(fmt):
    codes = finite_codes(fmt)
    sb = 1 << (BITS[fmt] - 1)
    for c in codes:
        v = oracle.lowp_decode(fmt, c)
        assert oracle.lowp_encode(fmt, v) == c
        assert oracle.lowp_encode(fmt, -v) == c | sb
    for a, b in zip(codes, codes[1:]):
        va, vb = oracle.lowp_decode(fmt, a), oracle.lowp_decode(fmt, b)
        mid = (va + vb) / 2
        assert oracle.lowp_encode(fmt, mid) == (a if a % 2 == 0 else b), (fmt, va, vb)
        assert oracle.lowp_encode(fmt, np.nextafter(mid, va)) == a
        assert oracle.lowp_encode(fmt, np.nextafter(mid, vb)) == b
    mx = oracle.lowp_max_finite(fmt)
    top = codes[-1]
    for v in (mx * 1.01, mx * 4, 1e30, float("inf")):
        assert oracle.lowp_encode(fmt, v) == top and oracle.lowp_encode(fmt, -v) == top | sb


def test_fp8_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    for fmt, dt, mx in (("e4m3", torch.float8_e4m3fn, 448.0), ("e5m2", torch.float8_e5m2, 57344.0)):
        x = np.concatenate([rng.uniform(-mx, mx, 4000),
                            rng.standard_normal(4000) * np.exp2(rng.integers(-20, 8, 4000))])
        x = x[np.abs(x) <= mx].astype(np.float32)
        ref = torch.from_numpy(x).to(dt).view(torch.uint8).numpy()
        got = np.array([oracle.lowp_encode(fmt, float(v)) for v in x])
        assert np.array_equal(got, ref), fmt


def test_e8m0_snap_is_the_power_of_two_at_or_below():
    assert [oracle.f32_to_e8m0(v) for v in (1.0, 2.0, 3.0, 0.75, 0.0, float("inf"))] == \
        [127, 128, 128, 126, 0, 255]
    rng = np.random.default_rng(1)
    for s in np.exp2(rng.uniform(-120, 120, 500)).astype(np.float32):
        v = oracle.lowp_snap_scale("mx", s)
        assert v <= s < 2 * v and v == 2.0 ** round(np.log2(v))


def test_nvfp4_snap_is_the_nearest_e4m3():
    rng = np.random.default_rng(2)
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    vals = np.sort(vals[np.isfinite(vals) & (vals >= 0)])
    for s in np.exp2(rng.uniform(-9, 8.8, 500)).astype(np.float32):
        v = oracle.lowp_snap_scale("nvfp4", s)
        assert abs(v - s) == np.min(np.abs(vals - float(s))), s


@pytest.mark.parametrize("layout", ["tensor", "mx", "nvfp4"])
@pytest.mark.parametrize("fmt", FMTS)
def test_compute_scales_and_quantize(layout, fmt):
    rng = np.random.default_rng(hash((layout, fmt)) % 2**32)
    rows, cols = 5, 77                      # a ragged last block
    x = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-6, 6, (rows, 1)))).astype(np.float32)
    x[1, 32:64] = 0.0                       # an all-zero block: scale 1
    sc = oracle.lowp_compute_scales(x, fmt, layout)
    mx = np.float32(oracle.lowp_max_finite(fmt))
    if layout == "tensor":
        assert sc[0] == np.float32(np.max(np.abs(x))) / mx
    else:
        bs = 32 if layout == "mx" else 16
        for r in range(rows):
            for b in range(-(-cols // bs)):
                amax = np.float32(np.max(np.abs(x[r, b * bs:(b + 1) * bs])))
                raw = amax / mx if amax > 0 else np.float32(1.0)
                assert sc[r, b] == oracle.lowp_snap_scale(layout, raw)
        if layout == "mx":
            assert sc[1, 1] == 1.0
    q = oracle.lowp_quantize(x, sc, fmt, layout)
    # Every code is the encoding of its quotient; a stored-then-read scale is
    # the same scale.
    st = oracle.lowp_store_scales(sc, layout)
    assert np.array_equal(oracle.lowp_read_scales(st, layout), sc)
    bs = 32 if layout == "mx" else 16
    for r in range(rows):
        for c in range(cols):
            s = sc[0] if layout == "tensor" else sc[r, c // bs]
            v = np.float32(x[r, c]) / s if s != 0 else np.float32(0)
            assert q[r, c] == oracle.lowp_encode(fmt, float(v))
    d = oracle.lowp_dequantize(q, sc, fmt, layout)
    dec = np.vectorize(lambda c: oracle.lowp_decode(fmt, c))(q)
    scale_full = np.broadcast_to(sc, (rows, 1)) if layout == "tensor" else \
        np.repeat(sc, 32 if layout == "mx" else 16, axis=1)[:, :cols]
    assert np.array_equal(d, dec * scale_full.astype(np.float64))


def test_scaled_matmul_worked_example():
    # lhs row: e2m1 codes 2 (1.0), 5 (3.0), 9 (-0.5); rhs rows with e4m3.
    # MX scales: lhs 2^1 (byte 128) for its one block, rhs 2^-1 (byte 126) and
    # 2^0 (byte 127).  out[0, 0] = (1*2)(1*0.5) + (3*2)(2*0.5) + (-0.5*2)(-1.5*0.5)
    #                            = 1 + 6 + 0.75 = 7.75, plus bias 0.25.
    e4 = lambda v: oracle.lowp_encode("e4m3", v)
    lhs = np.array([[2, 5, 9]], np.uint8)
    rhs = np.array([[e4(1.0), e4(2.0), e4(-1.5)], [e4(0.5), e4(0.0), e4(4.0)]], np.uint8)
    ls = oracle.lowp_read_scales(np.array([[128]], np.uint8), "mx")
    rs = oracle.lowp_read_scales(np.array([[126], [127]], np.uint8), "mx")
    y, S = oracle.lowp_scaled_matmul(lhs, rhs, ls, rs, np.array([0.25, -1.0]), "mx", "e2m1",
                                     "e4m3")
    # out[0, 1] = (1*2)(0.5) + (3*2)(0) + (-1)(4) - 1 = 1 - 4 - 1 = -4.
    assert y[0, 0] == 8.0 and y[0, 1] == -4.0
    assert S[0, 0] == 1 + 6 + 0.75 + 0.25


@pytest.mark.parametrize("layout", ["tensor", "mx", "nvfp4"])
def test_scaled_matmul_equals_dense_torch_formulation(layout):
    rng = np.random.default_rng(7)
    m, n, k = 6, 9, 100
    lhs = rng.integers(0, 256, (m, k)).astype(np.uint8)
    lhs[(lhs & 0x7F) == 0x7F] = 0                   # no e4m3 nan
    rhs = rng.integers(0, 16, (n, k)).astype(np.uint8)
    nb = 1 if layout == "tensor" else -(-k // (32 if layout == "mx" else 16))
    if layout == "tensor":
        ls, rs = np.array([0.37], np.float32), np.array([1.9], np.float32)
    elif layout == "mx":
        ls = oracle.lowp_read_scales(rng.integers(120, 135, (m, nb)).astype(np.uint8), "mx")
        rs = oracle.lowp_read_scales(rng.integers(120, 135, (n, nb)).astype(np.uint8), "mx")
    else:
        ls = oracle.lowp_read_scales(rng.integers(0x20, 0x60, (m, nb)).astype(np.uint8), "nvfp4")
        rs = oracle.lowp_read_scales(rng.integers(0x20, 0x60, (n, nb)).astype(np.uint8), "nvfp4")
    bias = rng.standard_normal(n)
    y, _ = oracle.lowp_scaled_matmul(lhs, rhs, ls, rs, bias, layout, "e4m3", "e2m1")
    a = torch.from_numpy(lhs).view(torch.float8_e4m3fn).double().numpy()
    e2 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
    b = e2[rhs]
    if layout == "tensor":
        a, b = a * float(ls[0]), b * float(rs[0])
    else:
        bs = 32 if layout == "mx" else 16
        a = a * np.repeat(ls.astype(np.float64), bs, axis=1)[:, :k]
        b = b * np.repeat(rs.astype(np.float64), bs, axis=1)[:, :k]
    ref = a @ b.T + bias
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-13)
