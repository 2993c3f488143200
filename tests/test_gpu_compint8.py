"""GPU parity of CompInt8 (qmm_gemm_compint8 and its debug exports).

Bit-exact: the quantized activations and their scales of the quantization
launch (qmm_debug_quantize_a); and the int32 block dots together with the
quantized activations and scales left in the workspace by the kernels of the
route qmm_gemm_compint8 takes (qmm_debug_compint8_block_dots) -- for M = 1
on the tiled layout, the one-launch kernel's in-LDS quantization and its
per-block int32 sums.  Within tol * S: the scaled float output, against the
oracle's CompInt8 value (strictly, with no output-rounding allowance, on the
seeded full-size workload).  Shapes: small ragged ones for every
(bits, block size, dtype, zero point) and the full batched-decode workload
(M in {1, 4, 16}, K = 4096, N = 14336; bits 4 / bs 128 symmetric, bits 8 /
bs 64 and bits 2 / bs 64 asymmetric).  Every test runs on the operator's
layout and on the tiled layout of qmm_repack.  On the tiled layout M = 1
runs the fused single-launch kernel (v_dot4 block dots, activations
quantized in LDS; any block of at least one 16-byte unit of codes) and
larger M the int8 matrix-core kernel, which, like the block-dot export,
rejects blocks shorter than 64 codes.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.util import TOL, assert_within, f64, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"
LAYOUT = {"v": "ort"}


@pytest.fixture(params=["ort", "tiled"], autouse=True)
def layout(request):
    LAYOUT["v"] = request.param
    yield request.param


def weights(case, c):
    """(B, scales, zero_points) of the case on the current layout."""
    if LAYOUT["v"] == "tiled":
        t = qmm().qmm_repack(c.B, c.scales, c.zero_points, case.K, case.N, case.block_size,
                             case.bits)
        return t, None, None
    return c.B, c.scales, c.zero_points


def qmm():
    from block_quantized_weight_matmulnbits_amd import qmm as q
    return q


def workspace(M, K, bs):
    n = qmm().qmm_compint8_workspace_size(M, K, bs)
    return torch.empty(n, dtype=torch.uint8, device=DEV)


def oracle_quant(case):
    return oracle.quantize_a(case.A.float().numpy().reshape(case.M, case.K), case.K, case.block_size)


def gpu_quant(case):
    c = case.to(DEV)
    kb = case.k_blocks
    qa = torch.empty(case.M, kb * case.block_size, dtype=torch.int8, device=DEV)
    sa = torch.empty(case.M, kb, dtype=torch.float32, device=DEV)
    qmm().qmm_debug_quantize_a(c.A, case.M, case.K, case.block_size, qa, sa)
    torch.cuda.synchronize()
    return qa.cpu().numpy(), sa.cpu().numpy()


def gpu_dots(case):
    """int32 block dots [M, N, kb] and the workspace's qa [M, kb*bs] / sa
    [M, kb] as the route's kernels left them."""
    c = case.to(DEV)
    kb, bs, M = case.k_blocks, case.block_size, case.M
    dots = torch.empty(M, case.N, kb, dtype=torch.int32, device=DEV)
    B, _, Z = weights(case, c)
    ws = workspace(M, case.K, bs)
    ws.fill_(0x5A)                     # stale bytes: every exported byte must be written
    qmm().qmm_debug_compint8_block_dots(c.A, B, Z, M, case.K, case.N, bs, case.bits, dots, ws)
    torch.cuda.synchronize()
    qa_bytes = -(-(M * kb * bs) // 256) * 256
    w = ws.cpu()
    qa = w[:M * kb * bs].view(torch.int8).reshape(M, kb * bs).numpy()
    sa = w[qa_bytes:qa_bytes + 4 * M * kb].view(torch.float32).reshape(M, kb).numpy()
    return dots.cpu().numpy(), qa, sa


def gpu_matmul(case):
    c = case.to(DEV)
    Y = torch.empty(case.M, case.N, dtype=c.A.dtype, device=DEV)
    B, S, Z = weights(case, c)
    qmm().qmm_gemm_compint8(c.A, B, S, Z, c.bias, Y, case.M, case.K, case.N,
                            case.block_size, case.bits, workspace(case.M, case.K, case.block_size))
    torch.cuda.synchronize()
    return Y


def small_route(case):
    """Whether qmm_gemm_compint8 takes the one-launch M = 1 kernel: tiled
    layout, a block of at least one 16-byte unit of codes and at most 1024,
    and the quantized row within its LDS budget."""
    if LAYOUT["v"] != "tiled" or case.M != 1:
        return False
    if not 128 // case.bits <= case.block_size <= 1024:
        return False
    # LDS bytes: the permuted row + unit sums + block scales + share sums.
    chunks = -(-(case.k_blocks * case.block_size) // 64)
    rs = 64 * chunks + 64 * {2: 8, 4: 4, 8: 2}[case.bits]
    lds = -(-rs // 16) * 16 + rs // (128 // case.bits) * 4 + case.k_blocks * 4 + 16 * 8 * 4
    return lds <= 64 * 1024


def check_all(case, what, strict=False):
    print(f"[compint8 {LAYOUT['v']}] {what} M={case.M} K={case.K} N={case.N} bs={case.block_size} "
          f"bits={case.bits} a={case.a_dtype} zp={case.zero_points is not None}", flush=True)
    qa, sa = oracle_quant(case)
    gqa, gsa = gpu_quant(case)
    assert np.array_equal(gsa, sa), f"{what}: activation scales differ"
    assert np.array_equal(gqa, qa), f"{what}: int8 activations differ"
    tiled = LAYOUT["v"] == "tiled"
    mfma_ok = not tiled or case.block_size >= 32
    small_ok = small_route(case)
    if mfma_ok or small_ok:
        dots = oracle.compint8_block_dots(qa, u8(case.B), u8(case.zero_points), case.N, case.K,
                                          case.block_size, case.bits)
        gdots, wqa, wsa = gpu_dots(case)
        route = "one-launch" if small_ok else "two-launch"
        assert np.array_equal(wsa, sa), f"{what}: {route} activation scales differ"
        assert np.array_equal(wqa, qa), f"{what}: {route} int8 activations differ"
        assert np.array_equal(gdots, dots), f"{what}: {route} int32 block dots differ"
    else:
        with pytest.raises(qmm().QmmError) as err:
            gpu_dots(case)
        assert err.value.status == qmm().QMM_ERR_UNSUPPORTED
        with pytest.raises(qmm().QmmError) as err:
            gpu_matmul(case)
        assert err.value.status == qmm().QMM_ERR_UNSUPPORTED
        return 0.0
    Y, S = oracle.compint8_matmul(qa, sa, u8(case.B), f64(case.scales), u8(case.zero_points),
                                  f64(case.bias), case.N, case.K, case.block_size, case.bits)
    return assert_within(gpu_matmul(case), Y, S, TOL[case.A.dtype], what, strict=strict)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("bs", [16, 32, 64, 128])
@pytest.mark.parametrize("a_dtype", ["f32", "bf16", "f16"])
def test_small_ragged_shapes(bits, bs, a_dtype):
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    for i, (M, K, N) in enumerate([(1, 16, 1), (1, 100, 33), (3, 257, 70), (4, 1000, 129),
                                   (17, 300, 40)]):
        for has_zp, has_bias in [(True, True), (False, False)]:
            case = make_matmul_case(M, K, N, bs, bits, a_dtype=a_dtype, has_zp=has_zp,
                                    has_bias=has_bias, seed=100 * bits + bs + i)
            check_all(case, f"small b{bits} bs{bs} {a_dtype}")


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_few_rows_long_k_and_lds_limit(bits):
    """M = 2 and 3 with K long enough for several wave loads per share, an
    M = 1 row whose quantized activations nearly fill the fused kernel's LDS
    budget, and one past it (which takes the quantize-then-matrix-core route
    on the tiled layout); M > 4 with the activation rows staged in LDS (33
    rows: three launches of 16, 16 and 1 rows) and with rows too long to
    stage."""
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    for i, (M, K, N, bs) in enumerate([(2, 4096, 300, 64), (3, 4104, 96, 128),
                                       (1, 40000, 65, 64), (1, 60000, 64, 128),
                                       (33, 4096, 100, 128), (20, 10000, 64, 64)]):
        case = make_matmul_case(M, K, N, bs, bits, a_dtype="bf16", has_zp=True, has_bias=True,
                                seed=500 + 10 * bits + i)
        r = check_all(case, f"rows/long K b{bits}")
        print(f"  max |err|/S = {r:.3e}")


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("variant", [(4, 128, False), (8, 64, True), (2, 64, True)])
def test_batched_decode_workload_full_size(M, variant):
    from block_quantized_weight_matmulnbits_amd.workloads import compint8_case
    bits, bs, asym = variant
    case = compint8_case(M, bits, bs, asym)
    r = check_all(case, case.meta["name"], strict=True)
    print(f"  max |err|/S = {r:.3e}")


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_one_row_every_block_size(bits):
    """M = 1 (the one-launch kernel on the tiled layout) for every block size
    it takes, from one 16-byte unit of codes to 1024: blocks within one wave
    load (units combined across lanes) and blocks over several loads (int32
    sums carried between loads), with ragged K so the last block is partial
    and shares of K that must stay whole blocks."""
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    sizes = [bs for bs in (16, 32, 64, 128, 256, 512, 1024) if bs >= 128 // bits]
    for i, bs in enumerate(sizes):
        for j, (K, N) in enumerate([(4096, 300), (4096 + 64 * 3 + 5, 96), (bs * 9 - 17, 40)]):
            case = make_matmul_case(1, K, N, bs, bits, a_dtype="bf16", has_zp=(j != 1),
                                    has_bias=(j == 0), seed=7000 + 100 * bits + 10 * i + j)
            check_all(case, f"one row b{bits} bs{bs}")


def test_quantize_a_ties_and_zero_blocks():
    """Exact ties round half to even on the device too; an all-zero block has
    scale 0 and zero codes."""
    rows = [float(x) for x in (127.0, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -1.5, -127.0, 0.0, 64.49,
                               -64.51)]
    A = torch.zeros(2, 32, dtype=torch.float32)
    A[0, :len(rows)] = torch.tensor(rows)
    from block_quantized_weight_matmulnbits_amd.workloads import MatmulCase
    case = MatmulCase(2, 32, 1, 16, 4, "f32", A, None, None, None, None)
    qa, sa = oracle_quant(case)
    gqa, gsa = gpu_quant(case)
    assert np.array_equal(gqa, qa) and np.array_equal(gsa, sa)
    assert list(gqa[0, :12]) == [127, 2, 4, -2, 0, 0, 2, -2, -127, 0, 64, -65]
    assert (gqa[1] == 0).all() and (gsa[1] == 0).all()


def test_deterministic():
    from block_quantized_weight_matmulnbits_amd.workloads import compint8_case
    case = compint8_case(4, 4, 128, False)
    assert torch.equal(gpu_matmul(case), gpu_matmul(case))


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_block32_matrix_core_route_dots_exact(bits):
    """Blocks of 32 codes: the int8 matrix-core kernel closes two blocks per
    64-code chunk (on the operator's layout from M = 8, on the tiled layout
    from M = 2; M = 5 on the operator's layout takes the other kernels); the
    int32 block dots equal the oracle's bit for bit (odd kb included) and the
    output is within tolerance."""
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    for i, (M, K, N) in enumerate([(16, 4096, 300), (5, 1056, 130), (20, 352, 64)]):
        case = make_matmul_case(M, K, N, 32, bits, a_dtype="bf16", has_zp=(i != 1),
                                has_bias=True, seed=900 + 10 * bits + i)
        print(f"[compint8 bs32] bits={bits} M={M} K={K} N={N}", flush=True)
        c = case.to(DEV)
        kb = case.k_blocks
        qa, sa = oracle.quantize_a(case.A.float().numpy().reshape(M, K), K, 32)
        ws = torch.empty(qmm().qmm_compint8_workspace_size(M, K, 32), dtype=torch.uint8,
                         device=DEV)
        dots = torch.empty(M, N, kb, dtype=torch.int32, device=DEV)
        qmm().qmm_debug_compint8_block_dots(c.A, c.B, c.zero_points, M, K, N, 32, bits, dots, ws)
        torch.cuda.synchronize()
        want = oracle.compint8_block_dots(qa, u8(case.B), u8(case.zero_points), N, K, 32, bits)
        assert np.array_equal(dots.cpu().numpy(), want), (M, K, N)
        Y, S = oracle.compint8_matmul(qa, sa, u8(case.B), f64(case.scales), u8(case.zero_points),
                                      f64(case.bias), N, K, 32, bits)
        y = torch.empty(M, N, dtype=c.A.dtype, device=DEV)
        qmm().qmm_gemm_compint8(c.A, c.B, c.scales, c.zero_points, c.bias, y, M, K, N, 32, bits,
                                ws)
        torch.cuda.synchronize()
        assert_within(y, Y, S, TOL[c.A.dtype], "compint8 bs32")
        if bits != 3:
            t = qmm().qmm_repack(c.B, c.scales, c.zero_points, K, N, 32, bits)
            yt = torch.empty_like(y)
            qmm().qmm_gemm_compint8(c.A, t, None, None, c.bias, yt, M, K, N, 32, bits, ws)
            torch.cuda.synchronize()
            assert_within(yt, Y, S, TOL[c.A.dtype], "compint8 bs32 tiled")
