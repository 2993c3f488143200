"""GPU checks of the one-time repack into the tiled layout (qmm_repack) and of
the matmuls that read it.

* qmm_repack followed by qmm_unrepack returns B and the scales bit for bit,
  and the zero points with the unused bits of each row's last byte cleared.
* The repacked buffer itself matches a host-side permutation of the inputs
  written in numpy from the layout's definition (codes, scales, zero points
  and zero padding).
* qmm_gemm and qmm_gemv on the repacked buffer give bit-identical outputs to
  the same calls on the operator's layout (the kernels only read the bytes
  from other addresses), and agree with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.util import TOL, assert_within, f64, oracle_matmul, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"
TG, TKC = 32, 64


def case_of(M, K, N, bs, bits, a_dtype="bf16", s_dtype="bf16", has_zp=True, seed=0):
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    return make_matmul_case(M, K, N, bs, bits, a_dtype=a_dtype, s_dtype=s_dtype, has_zp=has_zp,
                            has_bias=True, seed=seed)


def expected_tiled(case):
    """The tiled buffer, built on the host from the layout's definition."""
    K, N, bs, bits = case.K, case.N, case.block_size, case.bits
    kb = case.k_blocks
    groups = -(-N // TG)
    chunks = -(-(kb * bs) // TKC)
    cb = TKC * bits // 8
    r256 = lambda v: -(-v // 256) * 256
    B = case.B.numpy().reshape(N, kb * bs * bits // 8)
    rowpad = np.zeros((groups * TG, chunks * cb), np.uint8)
    rowpad[:N, :B.shape[1]] = B
    codes = rowpad.reshape(groups, TG, chunks, cb).transpose(0, 2, 1, 3).reshape(-1)
    S = case.scales.view(torch.int16 if case.scales.element_size() == 2 else torch.int32).numpy()
    spad = np.zeros((groups * TG, kb), S.dtype)
    spad[:N] = S.reshape(N, kb)
    scales = spad.reshape(groups, TG, kb).transpose(0, 2, 1).reshape(-1).view(np.uint8)
    out = np.zeros(r256(codes.size) + r256(scales.size) + (
        r256(groups * kb * TG * bits // 8) if case.zero_points is not None else 0), np.uint8)
    out[:codes.size] = codes
    so = r256(codes.size)
    out[so:so + scales.size] = scales
    if case.zero_points is not None:
        zo = so + r256(scales.size)
        zb = case.zero_points.numpy().reshape(N, -1)
        per = 8 // bits
        mask = (1 << bits) - 1
        zvals = np.zeros((groups * TG, kb), np.uint32)
        for b in range(kb):
            zvals[:N, b] = (zb[:, (b * bits) // 8] >> ((b * bits) % 8)) & mask
        z = zvals.reshape(groups, TG, kb).transpose(0, 2, 1).reshape(groups, kb, TG // per, per)
        packed = np.zeros(z.shape[:3], np.uint32)
        for e in range(per):
            packed |= z[..., e] << (e * bits)
        out[zo:zo + packed.size] = packed.reshape(-1).astype(np.uint8)
    return out


SHAPES = [(64, 64, 32), (100, 33, 32), (1000, 300, 64), (4096, 97, 128), (96, 520, 16)]


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("s_dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("has_zp", [True, False])
def test_repack_layout_and_round_trip(bits, s_dtype, has_zp):
    from block_quantized_weight_matmulnbits_amd import qmm
    for i, (K, N, bs) in enumerate(SHAPES):
        print(f"[repack] K={K} N={N} bs={bs} bits={bits} s={s_dtype} zp={has_zp}", flush=True)
        case = case_of(1, K, N, bs, bits, s_dtype=s_dtype, has_zp=has_zp, seed=7 * i + bits)
        c = case.to(DEV)
        t = qmm.qmm_repack(c.B, c.scales, c.zero_points, K, N, bs, bits)
        torch.cuda.synchronize()
        want = expected_tiled(case)
        got = t.buf.cpu().numpy()
        assert got.size == want.size
        assert np.array_equal(got, want)
        B2 = torch.full_like(c.B, 0xAA)
        S2 = torch.full_like(c.scales, 7.0)
        Z2 = torch.full_like(c.zero_points, 0xFF) if has_zp else None
        qmm.qmm_unrepack(t, K, N, bs, bits, B2, S2, Z2)
        torch.cuda.synchronize()
        assert torch.equal(B2.cpu(), case.B)
        assert torch.equal(S2.cpu().view(torch.uint8), case.scales.view(torch.uint8))
        if has_zp:
            kb = case.k_blocks
            used = kb * bits
            zw = case.zero_points.numpy().reshape(N, -1).copy()
            if used % 8:
                zw[:, -1] &= (1 << (used % 8)) - 1
            assert np.array_equal(Z2.cpu().numpy().reshape(N, -1), zw)


def run(case, tiled):
    from block_quantized_weight_matmulnbits_amd import qmm
    c = case.to(DEV)
    Y = torch.empty(case.M, case.N, dtype=c.A.dtype, device=DEV)
    if tiled:
        t = qmm.qmm_repack(c.B, c.scales, c.zero_points, case.K, case.N, case.block_size, case.bits)
        B, S = t, None
    else:
        B, S = c.B, c.scales
    Z = None if tiled else c.zero_points
    if case.M == 1:
        qmm.qmm_gemv(c.A.reshape(-1), B, S, Z, c.bias, Y.reshape(-1), case.K, case.N,
                     case.block_size, case.bits)
    else:
        qmm.qmm_gemm(c.A, B, S, Z, c.bias, Y, case.M, case.K, case.N, case.block_size, case.bits)
    torch.cuda.synchronize()
    return Y.cpu()


@pytest.mark.parametrize("a_dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("has_zp", [True, False])
def test_tiled_matmul_equals_operator_layout(a_dtype, bits, has_zp):
    # (M, K, N, bs): MFMA tiles with ragged M / N / K, the fp32 row kernel
    # (M <= 16, f32) and the M = 1 route.
    for i, (M, K, N, bs) in enumerate([(1, 1000, 300, 32), (1, 4096, 64, 128), (5, 512, 100, 64),
                                       (40, 520, 257, 16), (300, 1024, 520, 128),
                                       (257, 4096, 448, 32)]):
        print(f"[tiled] M={M} K={K} N={N} bs={bs} bits={bits} a={a_dtype} zp={has_zp}",
              flush=True)
        case = case_of(M, K, N, bs, bits, a_dtype=a_dtype, has_zp=has_zp, seed=100 + i)
        y_ort = run(case, False)
        y_t = run(case, True)
        # Both layouts against the oracle; for M > 1 the same kernel runs on
        # both layouts, so the results must also agree bit for bit.
        Y, S = oracle_matmul(case)
        assert_within(y_t, Y, S, TOL[y_t.dtype], "tiled")
        assert_within(y_ort, Y, S, TOL[y_t.dtype], "operator layout")
        if M > 1:
            assert torch.equal(y_t.view(torch.uint8), y_ort.view(torch.uint8)), (M, K, N, bs)


def test_tiled_prefill_sampled_rows():
    """M = 2048, K = 4096, N = 14336 (4-bit, block 32, bf16) on the repacked
    weights: every output of sampled rows against the oracle."""
    from block_quantized_weight_matmulnbits_amd.workloads import prefill_gemm
    case = prefill_gemm()
    print(f"[tiled prefill] M={case.M} K={case.K} N={case.N}", flush=True)
    y = run(case, True)
    rows = np.random.default_rng(1).choice(case.M, 32, replace=False)
    rows[:2] = [0, case.M - 1]
    Y, S = oracle.matmul_nbits(f64(case.A)[rows], u8(case.B), f64(case.scales),
                               u8(case.zero_points), f64(case.bias), case.N, case.K,
                               case.block_size, case.bits)
    r = assert_within(y[rows], Y, S, TOL[torch.bfloat16], "tiled prefill", strict=True)
    print(f"  max |err|/S = {r:.3e}")
