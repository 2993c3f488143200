"""GPU parity of 3-bit weights (the 2 + 1 bit-plane blob of MNN
ConvInt8TiledExecutor.cpp's 3-bit reorder; LSB-first 3-bit zero points,
default 4) against the oracle, on the operator's layout.

Bit-exact: the decoded codes and zero points (qmm_debug_unpack, including
zero points that continue into the next byte); CompInt8's int8 activations,
their scales and its int32 block dots (qmm_debug_compint8_block_dots).
Within tol * S of the oracle: qmm_gemv (M = 1) and qmm_gemm for every
activation dtype, small and large blocks, ragged K and N, with and without
zero points and bias; CompInt8's output against the oracle's CompInt8 value;
the decode projection 4096 x 14336 (block 32) and sampled rows of the
M = 2048 prefill shape strictly.  The matrix-core kernels (few-row and
256-row, 16-bit activations) on exact data bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.util import TOL, assert_within, f64, oracle_matmul, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def qmm():
    from block_quantized_weight_matmulnbits_amd import qmm as q
    return q


def case_of(M, K, N, bs, **kw):
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    return make_matmul_case(M, K, N, bs, 3, **kw)


def gpu_float(case):
    c = case.to(DEV)
    Y = torch.empty(case.M, case.N, dtype=c.A.dtype, device=DEV)
    if case.M == 1:
        qmm().qmm_gemv(c.A.reshape(-1), c.B, c.scales, c.zero_points, c.bias, Y.reshape(-1),
                       case.K, case.N, case.block_size, 3)
    else:
        qmm().qmm_gemm(c.A, c.B, c.scales, c.zero_points, c.bias, Y, case.M, case.K, case.N,
                       case.block_size, 3)
    torch.cuda.synchronize()
    return Y


@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
def test_unpack_matches_oracle(bs):
    for has_zp in (True, False):
        for K, N in [(333, 37), (bs * 11, 5)]:      # kb = 11: zero points straddle bytes
            case = case_of(1, K, N, bs, s_dtype="bf16", has_zp=has_zp, seed=bs + K)
            print(f"[bits3 codec] K={K} N={N} bs={bs} zp={has_zp}", flush=True)
            c = case.to(DEV)
            kb = case.k_blocks
            codes = torch.empty(N, K, dtype=torch.uint8, device=DEV)
            zps = torch.empty(N, kb, dtype=torch.uint8, device=DEV)
            w = torch.empty(N, K, dtype=torch.float32, device=DEV)
            qmm().qmm_debug_unpack(c.B, c.scales, c.zero_points, K, N, bs, 3, codes, zps, w)
            torch.cuda.synchronize()
            assert np.array_equal(codes.cpu().numpy(), oracle.unpack_codes(u8(case.B), N, K, bs, 3))
            assert np.array_equal(zps.cpu().numpy(),
                                  oracle.unpack_zero_points(u8(case.zero_points), N, kb, 3))
            W = oracle.dequantize(u8(case.B), f64(case.scales), u8(case.zero_points), N, K, bs, 3)
            assert np.array_equal(w.cpu().numpy(), W.astype(np.float32))


@pytest.mark.parametrize("a_dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("bs", [16, 32, 128, 1024])
def test_float_activations_within_tolerance(a_dtype, bs):
    for i, (M, K, N) in enumerate([(1, 1000, 129), (1, 4096, 64), (3, 520, 70), (9, 777, 33),
                                   (40, 300, 257)]):
        case = case_of(M, K, N, bs, a_dtype=a_dtype, has_zp=(i % 2 == 0), has_bias=(i % 3 == 0),
                       seed=4000 + bs + i)
        print(f"[bits3 float] M={M} K={K} N={N} bs={bs} a={a_dtype}", flush=True)
        Y, S = oracle_matmul(case)
        r = assert_within(gpu_float(case), Y, S, TOL[case.A.dtype], "bits3 float")
        print(f"  max |err|/S = {r:.3e}")


@pytest.mark.parametrize("a_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("bs", [16, 32, 64, 128, 1024])
def test_matrix_core_gemm_exact_data(a_dtype, bs):
    """16-bit activations run the matrix-core kernels, which decode the two
    planes themselves: the few-row kernel for the first two shapes, the
    256-row kernel for the last (35 x 32 workgroups of 32 x 32 outputs, past
    the few-row limit of 1024).  Small-integer activations and scale 0.25 make
    every dequantized weight exact in bf16 / f16 and every sum exact in fp32,
    so the result is the oracle's rounded once (ragged M, N, K % 64 != 0)."""
    rng = np.random.default_rng(bs)
    for i, (M, K, N) in enumerate([(17, 1032, 33), (300, 2056, 224), (1100, 264, 1000)]):
        K = max(K, bs)
        case = case_of(M, K, N, bs, a_dtype=a_dtype, has_zp=(i != 1), has_bias=True, seed=70 + i)
        case.A = torch.from_numpy(rng.integers(-3, 4, (M, K)).astype(np.float32)).to(case.A.dtype)
        case.scales = torch.full_like(case.scales, 0.25)
        case.bias = torch.from_numpy(rng.integers(-8, 9, N).astype(np.float32)).to(case.A.dtype)
        print(f"[bits3 gemm exact] M={M} K={K} N={N} bs={bs} a={a_dtype}", flush=True)
        Y, _ = oracle_matmul(case)
        assert torch.equal(gpu_float(case).cpu(), torch.from_numpy(Y).to(case.A.dtype)), (M, K, N)


def test_prefill_shape_sampled_rows():
    """M = 2048, K = 4096, N = 14336, 3-bit block 32: every output of 32
    sampled rows against the oracle, strictly."""
    case = case_of(2048, 4096, 14336, 32, a_dtype="bf16", has_zp=True, seed=81)
    y = gpu_float(case).cpu()
    rows = np.random.default_rng(1).choice(2048, 32, replace=False)
    rows[:2] = [0, 2047]
    Y, S = oracle.matmul_nbits(f64(case.A)[rows], u8(case.B), f64(case.scales),
                               u8(case.zero_points), None, case.N, case.K, 32, 3)
    r = assert_within(y[rows], Y, S, TOL[torch.bfloat16], "bits3 prefill", strict=True)
    print(f"  max |err|/S = {r:.3e}")


def test_largest_block():
    """block_size 8192: one block per staged chunk (128 KiB of LDS for four
    fp32 rows)."""
    case = case_of(5, 8192 + 4096 + 3, 40, 8192, a_dtype="bf16", has_zp=True, has_bias=True,
                   seed=9)
    Y, S = oracle_matmul(case)
    assert_within(gpu_float(case), Y, S, TOL[torch.bfloat16], "bits3 bs8192")


def test_decode_projection_full_size():
    case = case_of(1, 4096, 14336, 32, a_dtype="bf16", has_zp=True, seed=31)
    Y, S = oracle_matmul(case)
    r = assert_within(gpu_float(case), Y, S, TOL[torch.bfloat16], "bits3 decode", strict=True)
    print(f"  max |err|/S = {r:.3e}")


def ws_compint8(M, K, bs):
    n = qmm().qmm_compint8_workspace_size(M, K, bs)
    return torch.empty(n, dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("bs", [16, 32, 64, 128])
@pytest.mark.parametrize("a_dtype", ["bf16", "f32"])
def test_compint8_dots_exact_and_output_within_tolerance(bs, a_dtype):
    for i, (M, K, N) in enumerate([(1, 1000, 129), (4, 4096, 100), (17, 300, 40)]):
        case = case_of(M, K, N, bs, a_dtype=a_dtype, has_zp=(i != 1), has_bias=(i == 0),
                       seed=5000 + bs + i)
        print(f"[bits3 compint8] M={M} K={K} N={N} bs={bs} a={a_dtype}", flush=True)
        c = case.to(DEV)
        kb = case.k_blocks
        qa, sa = oracle.quantize_a(case.A.float().numpy().reshape(M, K), K, bs)
        dots = torch.empty(M, N, kb, dtype=torch.int32, device=DEV)
        ws = ws_compint8(M, K, bs)
        ws.fill_(0x5A)
        qmm().qmm_debug_compint8_block_dots(c.A, c.B, c.zero_points, M, K, N, bs, 3, dots, ws)
        torch.cuda.synchronize()
        w = ws.cpu()
        qa_bytes = -(-(M * kb * bs) // 256) * 256
        assert np.array_equal(w[:M * kb * bs].view(torch.int8).reshape(M, kb * bs).numpy(), qa)
        assert np.array_equal(w[qa_bytes:qa_bytes + 4 * M * kb].view(torch.float32)
                              .reshape(M, kb).numpy(), sa)
        assert np.array_equal(dots.cpu().numpy(), oracle.compint8_block_dots(
            qa, u8(case.B), u8(case.zero_points), N, K, bs, 3))
        Y, S = oracle.compint8_matmul(qa, sa, u8(case.B), f64(case.scales), u8(case.zero_points),
                                      f64(case.bias), N, K, bs, 3)
        y = torch.empty(M, N, dtype=c.A.dtype, device=DEV)
        qmm().qmm_gemm_compint8(c.A, c.B, c.scales, c.zero_points, c.bias, y, M, K, N, bs, 3,
                                ws_compint8(M, K, bs))
        torch.cuda.synchronize()
        assert_within(y, Y, S, TOL[c.A.dtype], "bits3 compint8")


def test_repack_and_group_indices_are_rejected():
    q = qmm()
    case = case_of(1, 256, 64, 32, a_dtype="bf16", has_zp=True, seed=1).to(DEV)
    with pytest.raises(q.QmmError) as err:
        q.qmm_repack(case.B, case.scales, case.zero_points, 256, 64, 32, 3)
    assert err.value.status == q.QMM_ERR_UNSUPPORTED
    Y = torch.empty(64, dtype=torch.bfloat16, device=DEV)
    g = torch.zeros(256, dtype=torch.int32, device=DEV)
    with pytest.raises(q.QmmError) as err:
        q.qmm_gemv(case.A.reshape(-1), case.B, case.scales, case.zero_points, None, Y, 256, 64,
                   32, 3, g_idx=g)
    assert err.value.status == q.QMM_ERR_UNSUPPORTED


@pytest.mark.parametrize("bs", [64, 128, 256])
def test_compint8_matrix_core_route_dots_exact(bs):
    """From M = 8 (M = 6 takes the generic kernel): the int8 matrix-core
    kernel with the two planes merged; its int32 block dots equal the
    oracle's bit for bit, with and without zero points (zero points
    straddling bytes), M past one 16-row pass."""
    for i, (M, K, N) in enumerate([(16, 4096, 300), (6, 2048, 200), (33, 1024, 70)]):
        case = case_of(M, K, N, bs, a_dtype="bf16", has_zp=(i != 1), has_bias=True,
                       seed=7000 + bs + i)
        print(f"[bits3 compint8 mfma] M={M} K={K} N={N} bs={bs}", flush=True)
        c = case.to(DEV)
        kb = case.k_blocks
        qa, sa = oracle.quantize_a(case.A.float().numpy().reshape(M, K), K, bs)
        dots = torch.empty(M, N, kb, dtype=torch.int32, device=DEV)
        qmm().qmm_debug_compint8_block_dots(c.A, c.B, c.zero_points, M, K, N, bs, 3, dots,
                                            ws_compint8(M, K, bs))
        torch.cuda.synchronize()
        assert np.array_equal(dots.cpu().numpy(), oracle.compint8_block_dots(
            qa, u8(case.B), u8(case.zero_points), N, K, bs, 3))
        Y, S = oracle.compint8_matmul(qa, sa, u8(case.B), f64(case.scales), u8(case.zero_points),
                                      f64(case.bias), N, K, bs, 3)
        y = torch.empty(M, N, dtype=c.A.dtype, device=DEV)
        qmm().qmm_gemm_compint8(c.A, c.B, c.scales, c.zero_points, c.bias, y, M, K, N, bs, 3,
                                ws_compint8(M, K, bs))
        torch.cuda.synchronize()
        assert_within(y, Y, S, TOL[c.A.dtype], "bits3 compint8 mfma")
