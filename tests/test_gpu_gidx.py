"""GPU parity of group indices (g_idx, act-order) against the oracle.

MatMulNBits input 4 (onnx-runtime-ep-cpu matmul_nbits.rs, dequantize_weight):
element k takes the scale and zero point of group g_idx[k].  qmm_gemv and
qmm_gemm on the operator's layout, for every (bits, block size, activation
dtype), M from 1 through the tabled GEMV (M <= 4, or 8 on a short grid), the
fp32 row kernel and the matrix-core GEMM, ragged K and N, random and
act-order index patterns, the padded [kb * bs] index shape; element-wise
within tol * S of the oracle (exact data: equal to the oracle's value
rounded once).  CompInt8 with group indices takes the float path, as the
operator routes it: its output equals qmm_gemm's bit for bit.
"""
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


def gidx_pattern(kind, K, bs, kb, rng, padded=False):
    n = kb * bs if padded else K
    if kind == "random":
        g = rng.integers(0, kb, n)
    elif kind == "act_order":
        # g_idx[k] = rank(k) // bs for a random order of K (each group has bs
        # members, the last possibly fewer).
        order = rng.permutation(K)
        rank = np.empty(K, np.int64)
        rank[order] = np.arange(K)
        g = rank // bs
        if padded:
            g = np.concatenate([g, np.full(n - K, kb - 1)])
    else:
        g = np.arange(n) // bs
    return g.astype(np.int32)


def run(case, g, entry="gemm"):
    q = qmm()
    c = case.to(DEV)
    gd = torch.from_numpy(g).to(DEV)
    Y = torch.empty(case.M, case.N, dtype=c.A.dtype, device=DEV)
    if entry == "gemv":
        q.qmm_gemv(c.A.reshape(-1), c.B, c.scales, c.zero_points, c.bias, Y.reshape(-1), case.K,
                   case.N, case.block_size, case.bits, g_idx=gd)
    elif entry == "compint8":
        ws = torch.empty(q.qmm_compint8_workspace_size(case.M, case.K, case.block_size),
                         dtype=torch.uint8, device=DEV)
        q.qmm_gemm_compint8(c.A, c.B, c.scales, c.zero_points, c.bias, Y, case.M, case.K,
                            case.N, case.block_size, case.bits, ws, g_idx=gd)
    else:
        q.qmm_gemm(c.A, c.B, c.scales, c.zero_points, c.bias, Y, case.M, case.K, case.N,
                   case.block_size, case.bits, g_idx=gd)
    torch.cuda.synchronize()
    return Y


def oracle_y(case, g):
    return oracle.matmul_nbits(f64(case.A).reshape(case.M, case.K), u8(case.B), f64(case.scales),
                               u8(case.zero_points), f64(case.bias), case.N, case.K,
                               case.block_size, case.bits, g_idx=g)


@pytest.mark.parametrize("a_dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("bs", [16, 32, 64, 128])
def test_random_data_within_tolerance(a_dtype, bits, bs):
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    rng = np.random.default_rng(bits * 100 + bs)
    for i, (M, K, N, kind, padded) in enumerate([
            (1, 1000, 129, "random", False), (1, 4096, 300, "act_order", True),
            (5, 520, 70, "act_order", False), (40, 1000, 257, "random", True),
            (300, 512, 300, "act_order", False)]):
        case = make_matmul_case(M, K, N, bs, bits, a_dtype=a_dtype, has_zp=(i % 2 == 0),
                                has_bias=(i % 3 == 0), seed=3000 + 10 * bits + bs + i)
        g = gidx_pattern(kind, K, bs, case.k_blocks, rng, padded)
        print(f"[gidx] M={M} K={K} N={N} bs={bs} bits={bits} a={a_dtype} {kind} "
              f"padded={padded}", flush=True)
        Y, S = oracle_y(case, g)
        y = run(case, g, "gemv" if M == 1 else "gemm")
        r = assert_within(y, Y, S, TOL[case.A.dtype], "gidx")
        print(f"  max |err|/S = {r:.3e}")


@pytest.mark.parametrize("a_dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_exact_data_matches_bit_for_bit(a_dtype, bits):
    """Small-integer activations and power-of-two scales: every product and
    partial sum is exact on the row kernel and the matrix-core path, so the
    result equals the oracle's rounded once to the output dtype."""
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    rng = np.random.default_rng(bits)
    for i, (M, K, N, bs) in enumerate([(1, 256, 33, 32), (7, 200, 65, 16), (48, 512, 300, 64),
                                       (260, 128, 40, 32)]):
        case = make_matmul_case(M, K, N, bs, bits, a_dtype=a_dtype, has_zp=True, has_bias=True,
                                seed=i)
        case.A = torch.from_numpy(rng.integers(-3, 4, (M, K)).astype(np.float32)).to(case.A.dtype)
        kb = case.k_blocks
        case.scales = torch.from_numpy(
            2.0 ** rng.integers(-4, 0, (N, kb)).astype(np.float32)).to(case.scales.dtype)
        case.bias = torch.from_numpy(rng.integers(-8, 9, N).astype(np.float32)).to(case.A.dtype)
        g = gidx_pattern("random", K, bs, kb, rng)
        print(f"[gidx exact] M={M} K={K} N={N} bs={bs} bits={bits} a={a_dtype}", flush=True)
        Y, _ = oracle_y(case, g)
        y = run(case, g, "gemv" if M == 1 else "gemm")
        assert torch.equal(y.cpu(), torch.from_numpy(Y).to(case.A.dtype)), (M, K, N, bs)


def test_decode_and_prefill_shapes_with_act_order():
    """A 4096 x 14336 decode projection (M = 1) and a prefill slice (M = 512)
    with act-order group indices, bf16, 4-bit asymmetric block 32."""
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    rng = np.random.default_rng(11)
    for M, N in [(1, 14336), (512, 2048)]:
        case = make_matmul_case(M, 4096, N, 32, 4, a_dtype="bf16", has_zp=True, seed=21 + M)
        g = gidx_pattern("act_order", 4096, 32, case.k_blocks, rng)
        print(f"[gidx full] M={M} K=4096 N={N}", flush=True)
        Y, S = oracle_y(case, g)
        r = assert_within(run(case, g, "gemv" if M == 1 else "gemm"), Y, S, TOL[torch.bfloat16],
                          "gidx full", strict=True)
        print(f"  max |err|/S = {r:.3e}")


@pytest.mark.parametrize("M", [1, 4, 40])
def test_compint8_with_group_indices_takes_the_float_path(M):
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    rng = np.random.default_rng(M)
    case = make_matmul_case(M, 1024, 200, 64, 4, a_dtype="bf16", has_zp=True, has_bias=True,
                            seed=M)
    g = gidx_pattern("act_order", 1024, 64, case.k_blocks, rng)
    y8 = run(case, g, "compint8")
    yf = run(case, g, "gemm")
    assert torch.equal(y8, yf)
    Y, S = oracle_y(case, g)
    assert_within(y8, Y, S, TOL[torch.bfloat16], "compint8 g_idx")


def test_tiled_layout_rejects_group_indices():
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    q = qmm()
    case = make_matmul_case(1, 256, 64, 32, 4, a_dtype="bf16", has_zp=True, seed=1).to(DEV)
    t = q.qmm_repack(case.B, case.scales, case.zero_points, 256, 64, 32, 4)
    g = torch.zeros(256, dtype=torch.int32, device=DEV)
    Y = torch.empty(64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(q.QmmError) as err:
        q.qmm_gemv(case.A.reshape(-1), t, None, None, None, Y, 256, 64, 32, 4, g_idx=g)
    assert err.value.status == q.QMM_ERR_UNSUPPORTED


def test_out_of_range_entries_are_clamped_not_faulting():
    """An unchecked out-of-range entry reads in bounds: it acts as the nearest
    valid group (the documented contract; qmm_check_g_idx rejects it on the
    host)."""
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    rng = np.random.default_rng(5)
    for M in (1, 3, 40):
        case = make_matmul_case(M, 512, 96, 32, 4, a_dtype="bf16", has_zp=True, seed=M)
        kb = case.k_blocks
        g = gidx_pattern("random", 512, 32, kb, rng)
        bad = g.copy()
        bad[::7] = 1000
        bad[3::11] = -5
        with pytest.raises(qmm().QmmError):
            qmm().qmm_check_g_idx(torch.from_numpy(bad), 512, 32)
        clamped = np.clip(bad, 0, kb - 1).astype(np.int32)
        entry = "gemv" if M == 1 else "gemm"
        assert torch.equal(run(case, bad, entry), run(case, clamped, entry))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_every_route_exact(bits):
    """Exact data on each route of qmm_gemm with group indices and 16-bit
    activations: the tabled matrix-core kernel with 128-column tiles (grid of
    at least 256 workgroups, table of at most 63 groups) and with 64-column
    tiles (M = 6 on a grid of 257 workgroups, M = 16, ragged N), the
    256-column kernel with lookups in memory (M > 16, a table of 160 groups
    does not fit in LDS), the row kernel (M = 12 on a grid of 129
    workgroups, same table), and a group-index
    array that is not 16-byte aligned (the tabled kernel reads it 16 bytes
    at a time)."""
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    rng = np.random.default_rng(77 + bits)
    cases = [("table128", 520, 264, 11000, 32, "bf16", "f32"),
             ("table64 M6", 6, 1032, 16400, 64, "f16", "f16"),
             ("table64 M16", 16, 776, 97, 16, "bf16", "bf16"),
             ("memory", 40, 2560, 130, 16, "bf16", "f16"),
             ("rows", 12, 2560, 8200, 16, "f16", "bf16"),
             ("unaligned", 24, 512, 200, 32, "bf16", "bf16")]
    for i, (name, M, K, N, bs, a_dtype, s_dtype) in enumerate(cases):
        case = make_matmul_case(M, K, N, bs, bits, a_dtype=a_dtype, s_dtype=s_dtype,
                                has_zp=i % 2 == 0, has_bias=True, seed=500 + i)
        case.A = torch.from_numpy(rng.integers(-3, 4, (M, K)).astype(np.float32)).to(case.A.dtype)
        kb = case.k_blocks
        case.scales = torch.from_numpy(
            2.0 ** rng.integers(-4, 0, (N, kb)).astype(np.float32)).to(case.scales.dtype)
        case.bias = torch.from_numpy(rng.integers(-8, 9, N).astype(np.float32)).to(case.A.dtype)
        g = gidx_pattern("act_order", K, bs, kb, rng)
        print(f"[gidx route] {name}: M={M} K={K} N={N} bs={bs} bits={bits} a={a_dtype} "
              f"s={s_dtype}", flush=True)
        Y, _ = oracle_y(case, g)
        expect = torch.from_numpy(Y).to(case.A.dtype)
        if name == "unaligned":
            c = case.to(DEV)
            gd = torch.from_numpy(np.concatenate([[0], g]).astype(np.int32)).to(DEV)[1:]
            y = torch.empty(M, N, dtype=c.A.dtype, device=DEV)
            qmm().qmm_gemm(c.A, c.B, c.scales, c.zero_points, c.bias, y, M, K, N, bs, bits,
                           g_idx=gd)
            torch.cuda.synchronize()
        else:
            y = run(case, g)
        assert torch.equal(y.cpu(), expect), name


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_gemv_routes_exact(bits):
    """Exact data through the tabled GEMV with group indices on each of its
    shapes: 8 waves (fewer than 512 workgroups; ragged N and K, f32 and f16
    activations), 4 waves (N 16400), LDS past 64 KiB (K 8192 at block 16: a
    table of 512 groups, 4 waves since 8 do not fit), 2 rows, 3 rows (one
    idle row slot), 8 rows and 12 rows (two launches of 8, the second with 4
    rows) on a short matrix-core grid, the row kernel when no table fits
    (1024 groups), and the smallest shapes (one block, one column; N = 5)."""
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    rng = np.random.default_rng(301 + bits)
    cases = [("eight waves f32", 1, 1000, 77, 32, "f32", "f16"),
             ("eight waves f16", 1, 4100, 300, 64, "f16", "bf16"),
             ("four waves", 1, 512, 16400, 32, "bf16", "bf16"),
             ("large table", 1, 8192, 100, 16, "bf16", "f16"),
             ("two rows", 2, 1000, 300, 32, "bf16", "bf16"),
             ("three rows", 3, 2100, 100, 64, "f16", "f16"),
             ("eight rows", 8, 4096, 200, 32, "bf16", "f32"),
             ("twelve rows", 12, 1000, 150, 32, "f16", "bf16"),
             ("rows", 1, 16384, 40, 16, "bf16", "bf16"),
             ("one block one column", 1, 16, 1, 16, "bf16", "bf16"),
             ("four rows five columns", 4, 40, 5, 16, "f32", "f32")]
    for i, (name, M, K, N, bs, a_dtype, s_dtype) in enumerate(cases):
        case = make_matmul_case(M, K, N, bs, bits, a_dtype=a_dtype, s_dtype=s_dtype,
                                has_zp=i % 2 == 0, has_bias=i % 2 == 1, seed=700 + i)
        case.A = torch.from_numpy(rng.integers(-3, 4, (M, K)).astype(np.float32)).to(case.A.dtype)
        kb = case.k_blocks
        case.scales = torch.from_numpy(
            2.0 ** rng.integers(-4, 0, (N, kb)).astype(np.float32)).to(case.scales.dtype)
        if case.bias is not None:
            case.bias = torch.from_numpy(rng.integers(-8, 9, N).astype(np.float32)).to(case.A.dtype)
        g = gidx_pattern("act_order", K, bs, kb, rng)
        print(f"[gidx gemv] {name}: M={M} K={K} N={N} bs={bs} bits={bits} a={a_dtype} "
              f"s={s_dtype}", flush=True)
        Y, _ = oracle_y(case, g)
        y = run(case, g, "gemv" if M == 1 else "gemm")
        assert torch.equal(y.cpu(), torch.from_numpy(Y).to(case.A.dtype)), name
