"""GPU parity of the low-precision scaled GEMM (qmm_lowp_matmul) against the
oracle (rlx-cpu quant.rs: lowp_scaled_matmul, lowp_read_scales).

* Exact data: element values from {0, 0.5, 1, 1.5, 2, 3, 4, 6} (in every
  format), scales 2^-1..2^1 (and 1.5 for NVFP4), so every product and partial
  sum is exact in fp32: the output equals the oracle's value, for all 25
  format pairs, the three scale layouts, ragged m / n and k (a partial last
  block, k not a multiple of 16, k below one step).
* Random codes of every format (nan and inf codes excluded) with random
  scales, within the bound of the instruction's arithmetic: the
  block-scaled matrix-core instruction adds the products of each aligned
  group of 8 elements of K in a fixed-point sum aligned to the group's
  largest product, cut 2^-14 below it (measured on gfx950: with 448 * 448
  at k = 0, a product of 4 at k = 1..7 is dropped, at k = 8 it is kept), and
  the group sums in fp32.  Bound, with a factor 2 on the cut (its position
  relative to a product's own exponent) and one more cut unit for the group
  sum: |gpu - oracle| <= 8 * 2^-12 * sum_g max_g |a b| + (k / 8 + 16) *
  2^-24 * S, S = sum |a b| + |bias|.
* The MXFP4 x MXFP4 prefill shape (m 2048, k 4096, n 14336) on sampled rows
  and columns; rows are independent of the batch.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"
FMTS = ["e4m3", "e5m2", "e2m3", "e3m2", "e2m1"]
LAYOUTS = ["tensor", "mx", "nvfp4"]
VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def qmm():
    from block_quantized_weight_matmulnbits_amd import qmm as q
    return q


def codes_of(values, fmt):
    table = {v: oracle.lowp_encode(fmt, v) for v in set(np.ravel(values).tolist())}
    return np.vectorize(lambda v: table[v])(values).astype(np.uint8)


def stored_scales(rng, rows, nb, layout, exact):
    """Stored scales and their raw float32 values."""
    if layout == "tensor":
        st = np.array([rng.choice([0.5, 1.0, 2.0]) if exact else rng.uniform(0.01, 3.0)],
                      np.float32)
    elif layout == "mx":
        st = rng.integers(126, 129, (rows, nb)) if exact else rng.integers(110, 140, (rows, nb))
        st = st.astype(np.uint8)
    else:
        pool = [0.5, 1.0, 1.5, 2.0] if exact else None
        if exact:
            st = codes_of(rng.choice(pool, (rows, nb)), "e4m3")
        else:
            st = rng.integers(0x18, 0x60, (rows, nb)).astype(np.uint8)
    return st, oracle.lowp_read_scales(st, layout)


def run(lhs, rhs, ls, rs, bias, m, n, k, layout, lf, rf):
    out = torch.empty(m, n, dtype=torch.float32, device=DEV)
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    qmm().qmm_lowp_matmul(t(lhs), t(rhs), t(ls), t(rs), t(bias), out, m, n, k, layout, lf, rf)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def nblocks(k, layout):
    return 1 if layout == "tensor" else -(-k // (32 if layout == "mx" else 16))


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("lf", FMTS)
def test_exact_data_every_format_pair(layout, lf):
    for rf in FMTS:
        for i, (m, n, k) in enumerate([(37, 45, 200), (130, 129, 256), (5, 200, 40), (3, 7, 5)]):
            rng = np.random.default_rng(1000 * FMTS.index(lf) + 10 * FMTS.index(rf) + i)
            sign = lambda shape: np.where(rng.random(shape) < 0.5, -1.0, 1.0)
            lv = rng.choice(VALUES, (m, k)) * sign((m, k))
            rv = rng.choice(VALUES, (n, k)) * sign((n, k))
            lhs, rhs = codes_of(lv, lf), codes_of(rv, rf)
            nb = nblocks(k, layout)
            lst, lsr = stored_scales(rng, m, nb, layout, True)
            rst, rsr = stored_scales(rng, n, nb, layout, True)
            bias = rng.integers(-4, 5, n).astype(np.float32) if i % 2 == 0 else None
            print(f"[lowp exact] {layout} {lf} x {rf} m={m} n={n} k={k}", flush=True)
            want, _ = oracle.lowp_scaled_matmul(lhs, rhs, lsr, rsr, bias, layout, lf, rf)
            got = run(lhs, rhs, lst, rst, bias, m, n, k, layout, lf, rf)
            assert np.array_equal(got, want.astype(np.float32)), (layout, lf, rf, m, n, k)


def hw_bound(lhs, rhs, lsr, rsr, layout, lf, rf, S):
    """Per-output error bound of the instruction's arithmetic (module doc)."""
    a = np.abs(oracle.lowp_dequantize(lhs, lsr, lf, layout))
    b = np.abs(oracle.lowp_dequantize(rhs, rsr, rf, layout))
    k = a.shape[1]
    kp = -(-k // 8) * 8
    a = np.pad(a, ((0, 0), (0, kp - k))).reshape(a.shape[0], 1, kp // 8, 8)
    b = np.pad(b, ((0, 0), (0, kp - k))).reshape(1, b.shape[0], kp // 8, 8)
    gmax = (a * b).max(axis=3).sum(axis=2)
    return 8 * 2.0 ** -12 * gmax + (k / 8 + 16) * 2.0 ** -24 * S


def finite_random_codes(rng, shape, fmt):
    bits = {"e4m3": 8, "e5m2": 8, "e2m3": 6, "e3m2": 6, "e2m1": 4}[fmt]
    c = rng.integers(0, 1 << bits, shape).astype(np.uint8)
    if fmt == "e4m3":
        c[(c & 0x7F) == 0x7F] = 0x7E
    if fmt == "e5m2":
        c[(c & 0x7C) == 0x7C] = 0x7B
    return c


@pytest.mark.parametrize("layout", LAYOUTS)
def test_random_codes_within_tolerance(layout):
    for i, (lf, rf) in enumerate([(a, b) for a in FMTS for b in FMTS]):
        rng = np.random.default_rng(7 + i)
        m, n, k = [(64, 96, 1024), (33, 17, 300), (128, 256, 512)][i % 3]
        lhs, rhs = finite_random_codes(rng, (m, k), lf), finite_random_codes(rng, (n, k), rf)
        nb = nblocks(k, layout)
        lst, lsr = stored_scales(rng, m, nb, layout, False)
        rst, rsr = stored_scales(rng, n, nb, layout, False)
        bias = rng.standard_normal(n).astype(np.float32)
        want, S = oracle.lowp_scaled_matmul(lhs, rhs, lsr, rsr, bias, layout, lf, rf)
        got = run(lhs, rhs, lst, rst, bias, m, n, k, layout, lf, rf)
        err = np.abs(got - want)
        bound = hw_bound(lhs, rhs, lsr, rsr, layout, lf, rf, S)
        print(f"[lowp random] {layout} {lf} x {rf} m={m} n={n} k={k}: max err/S "
              f"{float(np.max(err / S)):.2e}, max err/bound {float(np.max(err / bound)):.3f}",
              flush=True)
        assert np.all(err <= bound), (layout, lf, rf)


def test_prefill_shape_mxfp4_sampled():
    """m 2048, k 4096, n 14336, E2M1 x E2M1 with MX scales: 8 sampled rows (the
    first and last included) against the oracle on 1024 sampled columns."""
    rng = np.random.default_rng(3)
    m, n, k = 2048, 14336, 4096
    lhs = rng.integers(0, 16, (m, k)).astype(np.uint8)
    rhs = rng.integers(0, 16, (n, k)).astype(np.uint8)
    lst = rng.integers(118, 124, (m, k // 32)).astype(np.uint8)
    rst = rng.integers(118, 124, (n, k // 32)).astype(np.uint8)
    got = run(lhs, rhs, lst, rst, None, m, n, k, "mx", "e2m1", "e2m1")
    rows = np.array([0, 1, 517, 1024, 1500, 2000, 2046, 2047])
    cols = np.sort(rng.choice(n, 1024, replace=False))
    cols[0], cols[-1] = 0, n - 1
    want, S = oracle.lowp_scaled_matmul(lhs[rows], rhs[cols], oracle.lowp_read_scales(lst[rows], "mx"),
                                        oracle.lowp_read_scales(rst[cols], "mx"), None, "mx",
                                        "e2m1", "e2m1")
    bound = hw_bound(lhs[rows], rhs[cols], oracle.lowp_read_scales(lst[rows], "mx"),
                     oracle.lowp_read_scales(rst[cols], "mx"), "mx", "e2m1", "e2m1", S)
    assert np.all(np.abs(got[np.ix_(rows, cols)] - want) <= bound)


def test_rows_are_independent_and_m_zero_is_a_no_op():
    rng = np.random.default_rng(5)
    m, n, k = 300, 200, 512
    lhs, rhs = finite_random_codes(rng, (m, k), "e4m3"), finite_random_codes(rng, (n, k), "e2m1")
    lst = rng.integers(120, 130, (m, k // 32)).astype(np.uint8)
    rst = rng.integers(120, 130, (n, k // 32)).astype(np.uint8)
    full = run(lhs, rhs, lst, rst, None, m, n, k, "mx", "e4m3", "e2m1")
    part = run(lhs[140:150], rhs, lst[140:150], rst, None, 10, n, k, "mx", "e4m3", "e2m1")
    assert np.array_equal(full[140:150], part)
    out = torch.full((1, n), 7.0, device=DEV)
    t = lambda a: torch.from_numpy(a).to(DEV)
    qmm().qmm_lowp_matmul(t(lhs[:1]), t(rhs), t(lst[:1]), t(rst), None, out, 0, n, k, "mx",
                          "e4m3", "e2m1")
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def run_quantize(x, fmt, layout):
    rows, cols = x.shape
    nb = nblocks(cols, layout)
    codes = torch.empty(rows, cols, dtype=torch.uint8, device=DEV)
    scales = (torch.empty(1, dtype=torch.float32, device=DEV) if layout == "tensor"
              else torch.empty(rows, nb, dtype=torch.uint8, device=DEV))
    qmm().qmm_lowp_quantize(x.to(DEV), codes, scales, rows, cols, fmt, layout)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("xdt", [torch.float32, torch.bfloat16, torch.float16])
def test_quantize_bit_exact(layout, xdt):
    """Codes and stored scales equal the oracle's (lowp_compute_scales,
    lowp_snap_scale, lowp_quantize) bit for bit, for every format, ragged
    cols, an all-zero block, signed zeros, values past the format's range
    and a nan."""
    for fmt in FMTS:
        rng = np.random.default_rng(FMTS.index(fmt) + 10 * LAYOUTS.index(layout))
        for rows, cols in [(5, 77), (3, 100), (130, 64), (2, 5)]:
            x = (rng.standard_normal((rows, cols)) *
                 np.exp2(rng.integers(-12, 12, (rows, 1)))).astype(np.float32)
            if cols >= 64:
                x[0, 32:64] = 0.0
                x[1, 3] = -0.0
                x[1, 40] = 1e30 if xdt != torch.float16 else 6e4
                x[rows - 1, 0] = np.nan
            xt = torch.from_numpy(x).to(xdt)
            xf = xt.float().numpy()
            print(f"[lowp quantize] {layout} {fmt} {xdt} rows={rows} cols={cols}", flush=True)
            codes, st = run_quantize(xt, fmt, layout)
            want_sc = oracle.lowp_compute_scales(xf, fmt, layout)
            want_codes = oracle.lowp_quantize(xf, want_sc, fmt, layout)
            want_st = oracle.lowp_store_scales(want_sc, layout)
            assert np.array_equal(codes, want_codes), (fmt, rows, cols)
            if layout == "tensor":
                assert st.view(np.uint32)[0] == want_st.view(np.uint32)[0]
            else:
                assert np.array_equal(st, want_st), (fmt, rows, cols)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_quantize_then_matmul(layout):
    """Activations quantized on the GPU feed the GPU matmul: equal to the
    oracle's matmul of the oracle's quantization, within the bound."""
    rng = np.random.default_rng(11)
    m, n, k = 96, 80, 512
    x = rng.standard_normal((m, k)).astype(np.float32)
    w = rng.standard_normal((n, k)).astype(np.float32)
    lc, ls = run_quantize(torch.from_numpy(x), "e4m3", layout)
    rc, rs = run_quantize(torch.from_numpy(w), "e2m1", layout)
    got = run(lc, rc, ls, rs, None, m, n, k, layout, "e4m3", "e2m1")
    lsr, rsr = oracle.lowp_read_scales(ls, layout), oracle.lowp_read_scales(rs, layout)
    want, S = oracle.lowp_scaled_matmul(lc, rc, lsr, rsr, None, layout, "e4m3", "e2m1")
    assert np.all(np.abs(got - want) <= hw_bound(lc, rc, lsr, rsr, layout, "e4m3", "e2m1", S))
    # The quantized product approximates the float one (a sanity check of the
    # pipeline, not a bound of the method).
    rel = np.abs(got - x @ w.T).max() / np.abs(x @ w.T).max()
    assert rel < 0.5, rel


@pytest.mark.parametrize("lf,rf", [("e2m1", "e2m1"), ("e4m3", "e2m1"), ("e5m2", "e3m2")])
def test_tile_and_scale_routes_exact_sampled(lf, rf):
    """Exact data on each route of the block-scaled kernel: 256-row tiles
    (grid of at least 256 workgroups) and 128-row tiles, MX scale words staged
    in LDS (k % 128 == 0) or loaded per lane, per-tensor scales; 12 sampled
    rows (first and last included) against the oracle on all columns."""
    for i, (m, n, k, layout) in enumerate([(1100, 8000, 200, "mx"), (1100, 8000, 256, "mx"),
                                           (1100, 8000, 256, "tensor"), (300, 500, 384, "mx")]):
        rng = np.random.default_rng(40 + i)
        sign = lambda shape: np.where(rng.random(shape) < 0.5, -1.0, 1.0)
        lhs = codes_of(rng.choice(VALUES, (m, k)) * sign((m, k)), lf)
        rhs = codes_of(rng.choice(VALUES, (n, k)) * sign((n, k)), rf)
        nb = nblocks(k, layout)
        lst, lsr = stored_scales(rng, m, nb, layout, True)
        rst, rsr = stored_scales(rng, n, nb, layout, True)
        print(f"[lowp route] {lf} x {rf} {layout} m={m} n={n} k={k}", flush=True)
        got = run(lhs, rhs, lst, rst, None, m, n, k, layout, lf, rf)
        rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, 10, replace=False)]))
        want, _ = oracle.lowp_scaled_matmul(lhs[rows], rhs, lsr if layout == "tensor" else lsr[rows],
                                            rsr, None, layout, lf, rf)
        assert np.array_equal(got[rows], want.astype(np.float32)), (m, n, k, layout)
