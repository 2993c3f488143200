"""qmm_gemm_compint8_noalloc (the CompInt8 entry point that allocates
nothing: its workspace is the library's fixed device array) against
qmm_gemm_compint8 with a caller workspace, called through the C ABI.  Both
run the same kernels, so the outputs must agree bit for bit; each output is
also checked against the oracle.  Every case makes two calls in a row, the
second with a smaller input, so the second reads only what it wrote itself
over the first call's leftovers in the shared array."""
import numpy as np
import pytest
import torch

import oracle
from tests.util import TOL, assert_within, f64, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def qmm():
    from block_quantized_weight_matmulnbits_amd import qmm as q
    return q


def both(case, tiled):
    q = qmm()
    c = case.to(DEV)
    if tiled:
        B, S, Z = q.qmm_repack(c.B, c.scales, c.zero_points, case.K, case.N, case.block_size,
                               case.bits), None, None
    else:
        B, S, Z = c.B, c.scales, c.zero_points
    y_ws = torch.empty(case.M, case.N, dtype=c.A.dtype, device=DEV)
    ws = torch.empty(q.qmm_compint8_workspace_size(case.M, case.K, case.block_size),
                     dtype=torch.uint8, device=DEV)
    q.qmm_gemm_compint8(c.A, B, S, Z, c.bias, y_ws, case.M, case.K, case.N, case.block_size,
                        case.bits, ws)
    y_na = torch.full((case.M, case.N), float("nan"), dtype=c.A.dtype, device=DEV)
    q.qmm_gemm_compint8_noalloc(c.A, B, S, Z, c.bias, y_na, case.M, case.K, case.N,
                                case.block_size, case.bits)
    torch.cuda.synchronize()
    return y_ws, y_na


def check(case, tiled, what):
    print(f"[noalloc] {what} tiled={tiled} M={case.M} K={case.K} N={case.N} "
          f"bs={case.block_size} bits={case.bits}", flush=True)
    y_ws, y_na = both(case, tiled)
    assert torch.equal(y_na.view(torch.uint8), y_ws.view(torch.uint8)), what
    qa, sa = oracle.quantize_a(case.A.float().numpy().reshape(case.M, case.K), case.K,
                               case.block_size)
    Y, S = oracle.compint8_matmul(qa, sa, u8(case.B), f64(case.scales), u8(case.zero_points),
                                  f64(case.bias), case.N, case.K, case.block_size, case.bits)
    assert_within(y_na, Y, S, TOL[case.A.dtype], what)


@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("bits,bs", [(4, 128), (8, 64), (2, 64)])
def test_noalloc_matches_workspace_entry_point(tiled, bits, bs):
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    # Two calls in a row: the second smaller (fewer rows, shorter K).
    for i, (M, K, N) in enumerate([(16, 4096, 1000), (3, 1000, 300), (1, 640, 77)]):
        case = make_matmul_case(M, K, N, bs, bits, a_dtype="bf16", has_zp=(bits != 4),
                                has_bias=(i == 1), seed=900 + 10 * bits + i)
        check(case, tiled, f"call {i + 1} b{bits} bs{bs}")


def test_noalloc_near_its_limit_then_small():
    """A call whose workspace nearly fills the array, then a small one."""
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    q = qmm()
    M, K, bs = 240, 16384, 128
    assert q.qmm_compint8_workspace_size(M, K, bs) <= q.QMM_NOALLOC_SCRATCH_BYTES
    assert q.qmm_compint8_workspace_size(M, K, bs) > q.QMM_NOALLOC_SCRATCH_BYTES * 0.9
    for i, (m, k, n) in enumerate([(M, K, 64), (2, 256, 40)]):
        case = make_matmul_case(m, k, n, bs, 4, a_dtype="bf16", has_zp=False, seed=950 + i)
        check(case, False, f"limit call {i + 1}")


def test_noalloc_rejects_a_workspace_beyond_its_array():
    q = qmm()
    M, K, bs = 300, 16384, 128
    assert q.qmm_compint8_workspace_size(M, K, bs) > q.QMM_NOALLOC_SCRATCH_BYTES
    A = torch.zeros(M, K, dtype=torch.bfloat16, device=DEV)
    B = torch.zeros(64, K // bs, bs // 2, dtype=torch.uint8, device=DEV)
    S = torch.ones(64, K // bs, dtype=torch.bfloat16, device=DEV)
    Y = torch.empty(M, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(q.QmmError) as err:
        q.qmm_gemm_compint8_noalloc(A, B, S, None, None, Y, M, K, 64, bs, 4)
    assert err.value.status == q.QMM_ERR_WORKSPACE
    assert "row batches" in str(err.value)
