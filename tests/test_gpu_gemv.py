"""GPU parity of the M = 1 GEMV (qmm_gemv) against the oracle.

Element-wise within tol * S (strictly, with no output-rounding allowance,
on the seeded workloads: the tiny configuration and the full layer) at small
ragged shapes for every (bits, block
size, dtype, zero point, bias) combination, at the full Llama-3-8B layer
shapes of the decode workload, and on the degenerate cases.  Every test runs
on the operator's layout and on the tiled layout written by qmm_repack (the
weights repacked on the device before the call).
"""
import numpy as np
import pytest
import torch

from tests.util import TOL, assert_within, oracle_matmul

pytestmark = pytest.mark.gpu

DEV = "cuda"
LAYOUT = {"v": "ort"}


@pytest.fixture(params=["ort", "tiled"], autouse=True)
def layout(request):
    LAYOUT["v"] = request.param
    yield request.param


def run_gemv(case):
    from block_quantized_weight_matmulnbits_amd import qmm
    c = case.to(DEV)
    Y = torch.empty(case.N, dtype=c.A.dtype, device=DEV)
    B, S, Z = c.B, c.scales, c.zero_points
    if LAYOUT["v"] == "tiled":
        B = qmm.qmm_repack(c.B, c.scales, c.zero_points, case.K, case.N, case.block_size,
                           case.bits)
        S = Z = None
    qmm.qmm_gemv(c.A.reshape(-1), B, S, Z, c.bias, Y, case.K, case.N, case.block_size,
                 case.bits)
    torch.cuda.synchronize()
    return Y


def check(case, what="", strict=False):
    print(f"[gemv {LAYOUT['v']}] {what} M=1 K={case.K} N={case.N} bs={case.block_size} bits={case.bits} "
          f"a={case.a_dtype} s={case.s_dtype} zp={case.zero_points is not None} "
          f"bias={case.bias is not None}", flush=True)
    Y, S = oracle_matmul(case)
    y = run_gemv(case)
    return assert_within(y, Y[0], S[0], TOL[case.A.dtype], what, strict=strict)


@pytest.mark.parametrize("a_dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("bs", [16, 32, 64, 128])
def test_small_ragged_shapes(a_dtype, bits, bs):
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    for i, (K, N) in enumerate([(16, 1), (33, 7), (100, 64), (257, 300), (1000, 129)]):
        for has_zp, has_bias in [(True, True), (False, False)]:
            case = make_matmul_case(1, K, N, bs, bits, a_dtype=a_dtype, has_zp=has_zp,
                                    has_bias=has_bias, seed=1000 * bits + 10 * bs + i)
            check(case, f"small {a_dtype} b{bits} bs{bs}")


@pytest.mark.parametrize("s_dtype", ["f32", "f16", "bf16"])
def test_scale_dtypes(s_dtype):
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    case = make_matmul_case(1, 512, 77, 32, 4, a_dtype="bf16", s_dtype=s_dtype, seed=5)
    check(case, f"scales {s_dtype}")


def test_tiny_matmulnbits_config():
    from block_quantized_weight_matmulnbits_amd.workloads import tiny_matmulnbits
    check(tiny_matmulnbits(), "tiny f32", strict=True)


def test_decode_layer_full_shapes():
    """Every projection of the Llama-3-8B layer at full size, all outputs."""
    from block_quantized_weight_matmulnbits_amd.workloads import decode_layer
    for case in decode_layer():
        r = check(case, f"decode {case.meta['name']}", strict=True)
        print(f"  max |err|/S = {r:.3e}")


def test_decode_layer_fused_shapes():
    """The layer with q|k|v and gate|up stacked along N (N = 6144 and 28672),
    as the benchmark runs it: all outputs."""
    from block_quantized_weight_matmulnbits_amd.workloads import decode_layer_fused
    for case in decode_layer_fused():
        r = check(case, f"decode fused {case.meta['name']}", strict=True)
        print(f"  max |err|/S = {r:.3e}")


def test_long_k_spans_several_lds_chunks():
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    for bits in (2, 4, 8):
        case = make_matmul_case(1, 40000 + 7, 65, 64, bits, a_dtype="bf16", has_zp=True, seed=bits)
        check(case, f"long K b{bits}")


def test_codes_equal_zero_point_give_bias_exactly():
    import oracle
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    for a_dtype in ("f32", "bf16", "f16"):
        for bits in (2, 4, 8):
            case = make_matmul_case(1, 200, 33, 32, bits, a_dtype=a_dtype, has_zp=True,
                                    has_bias=True, seed=bits)
            kb = case.k_blocks
            zps = np.random.default_rng(bits).integers(0, 1 << bits, (case.N, kb)).astype(np.uint8)
            codes = np.repeat(zps, 32, 1)[:, :case.K]
            case.B = torch.from_numpy(oracle.pack_codes(codes, 32, bits))
            case.zero_points = torch.from_numpy(oracle.pack_zero_points(zps, bits))
            y = run_gemv(case)
            assert torch.equal(y.cpu(), case.bias), (a_dtype, bits)


def test_wide_dynamic_range_takes_exact_path():
    """A 16-byte unit whose bf16 activations span more than fp16 normals can
    carry (a large value meeting a zero weight, tiny values meeting nonzero
    weights) must still be exact to the tolerance: an fp16 shortcut would
    lose the tiny values, which are all of S here."""
    import oracle
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    for a_dtype in ("bf16", "f16"):
        case = make_matmul_case(1, 64, 8, 32, 4, a_dtype=a_dtype, has_zp=False, seed=9)
        rng = np.random.default_rng(9)
        codes = rng.integers(0, 16, (8, 64)).astype(np.uint8)
        codes[:, 0] = 8                      # w = 0 where the large value sits
        case.B = torch.from_numpy(oracle.pack_codes(codes, 32, 4))
        A = torch.from_numpy(rng.standard_normal((1, 64)).astype(np.float32)) * 1e-6
        A[0, 0] = 1.0e4
        A[0, 40] = 1.0                       # a second, ordinary unit
        case.A = A.to(case.A.dtype)
        check(case, f"wide range {a_dtype}")


def test_integer_data_is_exact():
    """Small-integer activations and power-of-two scales make every product
    and partial sum exact, so the GPU must match the oracle bit for bit."""
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    for a_dtype in ("f32", "f16", "bf16"):
        case = make_matmul_case(1, 1024, 96, 32, 4, a_dtype=a_dtype, has_zp=True, seed=3)
        rng = np.random.default_rng(4)
        case.A = torch.from_numpy(rng.integers(-3, 4, (1, 1024)).astype(np.float32)).to(case.A.dtype)
        case.scales = torch.full_like(case.scales, 0.25)
        Y, _ = oracle_matmul(case)
        y = run_gemv(case)
        # The exact value, rounded once to the output dtype.
        expect = torch.from_numpy(Y[0]).to(case.A.dtype)
        assert torch.equal(y.cpu(), expect), a_dtype


def test_deterministic():
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    case = make_matmul_case(1, 4096, 4096, 32, 4, a_dtype="bf16", has_zp=True, seed=12)
    assert torch.equal(run_gemv(case), run_gemv(case))
