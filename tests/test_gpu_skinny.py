"""GPU parity of the few-row matrix-core matmul (qmm_gemm with bf16 / f16
activations, K % 8 == 0, and M <= 16 or at most 1024 workgroups of 32 x 32
outputs: the path for batched decode).

* Exact data (small-integer activations, power-of-two scales): the result
  equals the oracle's value rounded once to the output dtype, for every
  code width (3-bit: the 2 + 1 bit planes, zero points that straddle
  bytes), block size 16..256, with and without zero points and bias, every
  scale dtype, ragged M, N and K (K not a multiple of the 256-code wave
  step, K < 256, blocks past K), on the operator's layout and (2, 4, 8 bits)
  on the repacked one.
* Random data within tol * S; the decode projections (K, N) = (4096, 14336)
  and (14336, 4096) at M = 16 and M = 64 strictly.
* The edges of the route: M = 64 against M = 65 at N = 14336 (the 256-row
  kernel) on the same rows; many rows of a narrow matrix; row m of a batch
  equals the same row computed in another batch.
"""
import numpy as np
import pytest
import torch

from tests.util import TOL, assert_within, oracle_matmul

pytestmark = pytest.mark.gpu
DEV = "cuda"


def qmm():
    from block_quantized_weight_matmulnbits_amd import qmm as q
    return q


def run(case, tiled=False):
    c = case.to(DEV)
    Y = torch.empty(case.M, case.N, dtype=c.A.dtype, device=DEV)
    if tiled:
        t = qmm().qmm_repack(c.B, c.scales, c.zero_points, case.K, case.N, case.block_size,
                             case.bits)
        qmm().qmm_gemm(c.A, t, None, None, c.bias, Y, case.M, case.K, case.N, case.block_size,
                       case.bits)
    else:
        qmm().qmm_gemm(c.A, c.B, c.scales, c.zero_points, c.bias, Y, case.M, case.K, case.N,
                       case.block_size, case.bits)
    torch.cuda.synchronize()
    return Y


def exact_case(M, K, N, bs, bits, a_dtype, s_dtype, has_zp, has_bias, seed):
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    case = make_matmul_case(M, K, N, bs, bits, a_dtype=a_dtype, s_dtype=s_dtype, has_zp=has_zp,
                            has_bias=has_bias, seed=seed)
    rng = np.random.default_rng(seed + 1)
    case.A = torch.from_numpy(rng.integers(-3, 4, (M, K)).astype(np.float32)).to(case.A.dtype)
    sc = rng.choice([0.125, 0.25, 0.5], size=tuple(case.scales.shape)).astype(np.float32)
    case.scales = torch.from_numpy(sc).to(case.scales.dtype)
    if has_bias:
        case.bias = torch.from_numpy(rng.integers(-8, 9, N).astype(np.float32)).to(case.A.dtype)
    return case


SHAPES = [(2, 64, 7), (3, 256, 33), (5, 264, 100), (16, 1000, 130), (17, 520, 31),
          (33, 1032, 64), (64, 776, 50)]


@pytest.mark.parametrize("a_dtype", ["bf16", "f16"])
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
def test_exact_data_ragged(a_dtype, bits, bs):
    for i, (M, K, N) in enumerate(SHAPES):
        s_dtype = ["f32", "f16", "bf16"][i % 3]
        has_zp, has_bias = i % 2 == 0, i % 3 != 1
        case = exact_case(M, K, N, bs, bits, a_dtype, s_dtype, has_zp, has_bias,
                          seed=100 * bits + bs + i)
        print(f"[skinny exact] M={M} K={K} N={N} bs={bs} bits={bits} a={a_dtype} "
              f"s={s_dtype} zp={has_zp} bias={has_bias}", flush=True)
        Y, _ = oracle_matmul(case)
        expect = torch.from_numpy(Y).to(case.A.dtype)
        assert torch.equal(run(case).cpu(), expect), (M, K, N)
        if bits != 3:                              # 3-bit weights have no repacked layout
            assert torch.equal(run(case, tiled=True).cpu(), expect), ("tiled", M, K, N)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_random_data_within_tolerance(bits):
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    for i, (M, K, N, bs, a) in enumerate([(4, 2048, 300, 32, "bf16"), (16, 1024, 257, 64, "f16"),
                                          (40, 4096, 96, 128, "bf16"), (64, 512, 520, 16, "f16")]):
        case = make_matmul_case(M, K, N, bs, bits, a_dtype=a, has_zp=i % 2 == 0, has_bias=True,
                                seed=50 * bits + i)
        print(f"[skinny random] M={M} K={K} N={N} bs={bs} bits={bits} a={a}", flush=True)
        Y, S = oracle_matmul(case)
        r = assert_within(run(case), Y, S, TOL[case.A.dtype], "skinny random")
        print(f"  max |err|/S = {r:.3e}")


@pytest.mark.parametrize("M", [16, 64])
@pytest.mark.parametrize("K,N", [(4096, 14336), (14336, 4096)])
def test_decode_projection_strict(M, K, N):
    """Full batched-decode projection shapes, 4-bit asymmetric block 32, bf16
    scales in [0.002, 0.02]: every output strictly within 2e-3 * S; the oracle
    runs on a sample of 512 columns (all rows, full K)."""
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    case = make_matmul_case(M, K, N, 32, 4, a_dtype="bf16", has_zp=True, seed=M + K)
    print(f"[skinny decode] M={M} K={K} N={N}", flush=True)
    y = run(case).cpu()
    cols = np.sort(np.random.default_rng(M).choice(N, 512, replace=False))
    cols[0], cols[-1] = 0, N - 1
    sub = make_matmul_case(M, K, 512, 32, 4, a_dtype="bf16", has_zp=True, seed=0)
    sub.A, sub.B, sub.scales = case.A, case.B[cols], case.scales[cols]
    sub.zero_points = case.zero_points[cols]      # packed rows are per column
    Y, S = oracle_matmul(sub)
    r = assert_within(y[:, cols], Y, S, TOL[torch.bfloat16], "skinny decode", strict=True)
    print(f"  max |err|/S = {r:.3e}")


def test_route_edge_m64_vs_m65():
    """N = 14336: M = 64 takes the few-row kernel (2 x 448 workgroups), M = 65
    the 256-row kernel (3 x 448 would pass the limit of 1024); on exact data
    rows 0..63 agree bit for bit."""
    case = exact_case(65, 256, 14336, 32, 4, "bf16", "bf16", True, True, seed=9)
    y65 = run(case).cpu()
    case.M, case.A = 64, case.A[:64].contiguous()
    assert torch.equal(run(case).cpu(), y65[:64])


def test_many_rows_narrow_matrix():
    """M = 200 on N = 100 stays on the few-row kernel (7 x 4 workgroups):
    exact data on both layouts."""
    case = exact_case(200, 520, 100, 64, 4, "f16", "f32", True, True, seed=21)
    Y, _ = oracle_matmul(case)
    expect = torch.from_numpy(Y).to(case.A.dtype)
    assert torch.equal(run(case).cpu(), expect)
    assert torch.equal(run(case, tiled=True).cpu(), expect)


def test_rows_are_independent():
    """Row m of a 64-row batch equals the same row computed in a batch of 2."""
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    case = make_matmul_case(64, 2048, 300, 32, 4, a_dtype="bf16", has_zp=True, has_bias=True,
                            seed=11)
    y = run(case).cpu()
    for m0 in (0, 30, 62):
        sub = make_matmul_case(2, 2048, 300, 32, 4, a_dtype="bf16", seed=0)
        sub.A, sub.B, sub.scales, sub.zero_points, sub.bias = (
            case.A[m0:m0 + 2].contiguous(), case.B, case.scales, case.zero_points, case.bias)
        assert torch.equal(run(sub).cpu(), y[m0:m0 + 2]), m0


def test_deterministic():
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    case = make_matmul_case(16, 4096, 1024, 32, 4, a_dtype="bf16", has_zp=True, seed=3)
    assert torch.equal(run(case), run(case))
