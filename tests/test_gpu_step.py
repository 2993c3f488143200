"""GPU parity of a recorded step (qmm_step_*: calls captured once into a HIP
graph and replayed).  The decode layer's four stacked projections on the
tiled layout, plus an operator-layout GEMV and a CompInt8 call, recorded in
one step; the step is replayed several times with fresh activations written
in place before each replay and the program's own eager work (direct calls,
torch ops, synchronizations) between replays.  Every replay is checked
against the oracle and bit for bit against the same calls made directly."""
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


def test_decode_step_graph_replays_match_direct_calls_and_oracle():
    from block_quantized_weight_matmulnbits_amd.workloads import (compint8_case,
                                                                   decode_layer_fused,
                                                                   make_matmul_case)
    q = qmm()
    fcases = decode_layer_fused()
    extra = make_matmul_case(1, 1000, 300, 32, 4, a_dtype="bf16", has_zp=True, has_bias=True,
                             seed=31)
    ci8 = compint8_case(4, 4, 128, False, K=1024, N=512)
    dev = [c.to(DEV) for c in fcases]
    tiled = [q.qmm_repack(d.B, d.scales, d.zero_points, c.K, c.N, c.block_size, c.bits)
             for c, d in zip(fcases, dev)]
    xs = [torch.empty(c.K, dtype=torch.bfloat16, device=DEV) for c in fcases]
    ys = [torch.empty(c.N, dtype=torch.bfloat16, device=DEV) for c in fcases]
    de = extra.to(DEV)
    xe = torch.empty(extra.K, dtype=torch.bfloat16, device=DEV)
    ye = torch.empty(extra.N, dtype=torch.bfloat16, device=DEV)
    dc = ci8.to(DEV)
    xc = torch.empty(4, ci8.K, dtype=torch.bfloat16, device=DEV)
    yc = torch.empty(4, ci8.N, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(q.qmm_compint8_workspace_size(4, ci8.K, 128), dtype=torch.uint8, device=DEV)

    step = q.Step()
    for c, t, x, y in zip(fcases, tiled, xs, ys):
        step.add_gemv(x, t, None, None, None, y, c.K, c.N, c.block_size, c.bits)
    step.add_gemv(xe, de.B, de.scales, de.zero_points, de.bias, ye, extra.K, extra.N, 32, 4)
    step.add_gemm_compint8(xc, dc.B, dc.scales, None, None, yc, 4, ci8.K, ci8.N, 128, 4, ws)
    assert len(step) == 6
    step.finalize()

    rng = np.random.default_rng(0)
    for replay in range(4):
        # Fresh activations, written in place (the graph holds these buffers).
        new = [torch.from_numpy(rng.standard_normal(c.K).astype(np.float32)).to(torch.bfloat16)
               for c in fcases]
        for x, v in zip(xs, new):
            x.copy_(v)
        ve = torch.from_numpy(rng.standard_normal(extra.K).astype(np.float32)).to(torch.bfloat16)
        xe.copy_(ve)
        vc = torch.from_numpy(rng.standard_normal((4, ci8.K)).astype(np.float32)).to(
            torch.bfloat16)
        xc.copy_(vc)
        for y in ys + [ye, yc]:
            y.fill_(float("nan"))
        print(f"[step] replay {replay}", flush=True)
        step.launch()
        torch.cuda.synchronize()
        got = [y.clone() for y in ys + [ye, yc]]
        # The same calls made directly, with the program's eager work between.
        direct = [torch.empty_like(y) for y in ys + [ye, yc]]
        for c, t, x, y in zip(fcases, tiled, xs, direct[:4]):
            q.qmm_gemv(x, t, None, None, None, y, c.K, c.N, c.block_size, c.bits)
        q.qmm_gemv(xe, de.B, de.scales, de.zero_points, de.bias, direct[4], extra.K, extra.N, 32, 4)
        q.qmm_gemm_compint8(xc, dc.B, dc.scales, None, None, direct[5], 4, ci8.K, ci8.N, 128, 4,
                            ws)
        _ = (torch.ones(1 << 20, device=DEV) * 2).sum()
        torch.cuda.synchronize()
        for a, b in zip(got, direct):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), replay
        for c, v, y in zip(fcases, new, got[:4]):
            Y, S = oracle.matmul_nbits(f64(v)[None], u8(c.B), f64(c.scales), u8(c.zero_points),
                                       None, c.N, c.K, c.block_size, c.bits)
            assert_within(y, Y[0], S[0], TOL[torch.bfloat16], f"step {c.meta['name']}",
                          strict=True)
        Y, S = oracle.matmul_nbits(f64(ve)[None], u8(extra.B), f64(extra.scales),
                                   u8(extra.zero_points), f64(extra.bias), extra.N, extra.K, 32, 4)
        assert_within(got[4], Y[0], S[0], TOL[torch.bfloat16], "step operator-layout gemv")
        qa, sa = oracle.quantize_a(vc.float().numpy(), ci8.K, 128)
        Y, S = oracle.compint8_matmul(qa, sa, u8(ci8.B), f64(ci8.scales), None, None, ci8.N,
                                      ci8.K, 128, 4)
        assert_within(got[5], Y, S, TOL[torch.bfloat16], "step compint8")
    step.close()


def test_finalize_reports_the_failing_call():
    q = qmm()
    x = torch.zeros(256, dtype=torch.bfloat16, device=DEV)
    B = torch.zeros(64, 8, 16, dtype=torch.uint8, device=DEV)
    s = torch.ones(64, 8, dtype=torch.bfloat16, device=DEV)
    y = torch.empty(64, dtype=torch.bfloat16, device=DEV)
    step = q.Step()
    step.add_gemv(x, B, s, None, None, y, 256, 64, 32, 4)
    step.add_gemv(x, B, s, None, None, y, 256, 64, 48, 4)     # block_size 48: invalid
    with pytest.raises(q.QmmError) as err:
        step.finalize()
    assert err.value.status == q.QMM_ERR_INVALID_ARG
    assert "recorded call 1" in str(err.value) and "power of two" in str(err.value)
    with pytest.raises(q.QmmError):
        step.launch()
    step.close()
