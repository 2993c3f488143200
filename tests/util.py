"""Helpers shared by the GPU parity tests: run the oracle on a case and
compare a device result with it under the tolerance of the method."""
from __future__ import annotations

import numpy as np
import torch

import oracle

# |gpu - oracle| <= TOL[dtype] * S, S = sum_k |x_k w_k| (+ |bias|), plus the
# rounding of the result to the output dtype: a correctly rounded output can
# sit up to unit roundoff * |Y| away from the exact value (bf16: 2^-8 = 3.9e-3,
# which alone exceeds 2e-3 * S whenever |Y| > 0.51 S).
TOL = {torch.float32: 1e-5, torch.float16: 2e-3, torch.bfloat16: 2e-3}
# Below the normal range the rounding error is absolute: half the smallest
# subnormal of the output dtype.
OUT_ROUNDOFF = {torch.float32: 2.0 ** -24, torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}
OUT_HALF_SUBNORMAL = {torch.float32: 2.0 ** -150, torch.float16: 2.0 ** -25,
                      torch.bfloat16: 2.0 ** -134}


def f64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def u8(t):
    return None if t is None else t.detach().cpu().numpy().astype(np.uint8)


def oracle_matmul(case):
    """Oracle Y, S (float64 [M, N]) of a MatmulCase (host or device tensors)."""
    return oracle.matmul_nbits(f64(case.A).reshape(case.M, case.K), u8(case.B), f64(case.scales),
                               u8(case.zero_points), f64(case.bias), case.N, case.K,
                               case.block_size, case.bits)


def assert_within(y_dev, Y, S, tol, what="", strict=False):
    """Element-wise |y - Y| <= tol * S + u_out * (|Y| + tol * S) + h_out, u_out
    the unit roundoff and h_out half the smallest subnormal of y's dtype;
    reports the worst |y - Y| / S.

    strict=True asserts the plain bound |y - Y| <= tol * S with no allowance
    for rounding the result to the output dtype.  That is attainable when
    |Y| is small next to S, as on the seeded workloads (random signs keep
    |Y| / S near 1 / sqrt(K)); exact-data and edge cases, where |Y| can
    approach S, need the output-rounding term."""
    u = OUT_ROUNDOFF[y_dev.dtype]
    y = f64(y_dev).reshape(Y.shape)
    err = np.abs(y - Y)
    if strict:
        bound = tol * S
    else:
        bound = tol * S + u * (np.abs(Y) + tol * S) + OUT_HALF_SUBNORMAL[y_dev.dtype]
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = np.max(np.where(S > 0, err / S, np.inf))
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{bad.size} elements outside tol={tol}*S"
            f"{' (strict)' if strict else ''}; "
            f"max |err|/S = {ratio:.3e}; first at {idx.tolist()}: "
            f"gpu={[y[tuple(i)] for i in idx]} oracle={[Y[tuple(i)] for i in idx]} "
            f"S={[S[tuple(i)] for i in idx]}")
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(S > 0, err / np.where(S > 0, S, 1), 0.0)
    return float(r.max()) if r.size else 0.0
