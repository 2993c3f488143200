"""Seeded synthetic inputs for block-quantized-weight matmuls.

This module only draws random numbers and lays them out in the operator's
input format; it holds none of the method's arithmetic (no unpacking,
dequantization or matmul).  Both the HIP path and the CPU oracle consume what
it produces.

Recipes follow the MatMulNBits problem statement (onnx-runtime-ep-cpu
matmul_nbits.rs, module documentation): packed weights ``B`` are
``[N, ceil(K/bs), bs*bits/8]`` bytes, scales ``[N, kb]``, packed zero points
``[N, ceil(kb*bits/8)]`` bytes.  Codes uniform over ``0 .. 2^bits-1`` are drawn
as uniform random *bytes*: every bit field of a uniform byte is itself uniform
and independent, so no packing step is needed.  Zero points are drawn the same
way.  Half-precision values are produced by one round-to-nearest-even cast of
float32 draws; consumers read the rounded values.

Generation order within a case: activations, codes, scales, zero points, bias.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def n_blocks(K: int, bs: int) -> int:
    return -(-K // bs)


@dataclass
class MatmulCase:
    """One MatMulNBits problem, all tensors on the host (torch CPU)."""
    M: int
    K: int
    N: int
    block_size: int
    bits: int
    a_dtype: str
    A: torch.Tensor                 # [M, K] a_dtype
    B: torch.Tensor                 # [N, kb, blob] uint8
    scales: torch.Tensor            # [N, kb] s_dtype
    zero_points: torch.Tensor | None  # [N, ceil(kb*bits/8)] uint8 or None
    bias: torch.Tensor | None       # [N] a_dtype or None
    s_dtype: str = "f32"
    meta: dict = field(default_factory=dict)

    @property
    def k_blocks(self) -> int:
        return n_blocks(self.K, self.block_size)

    def weight_bytes(self) -> int:
        """Bytes of packed codes + scales + zero points."""
        n = self.B.numel() + self.scales.numel() * self.scales.element_size()
        if self.zero_points is not None:
            n += self.zero_points.numel()
        return n

    def to(self, device) -> "MatmulCase":
        mv = lambda t: None if t is None else t.to(device)
        return MatmulCase(self.M, self.K, self.N, self.block_size, self.bits, self.a_dtype,
                          mv(self.A), mv(self.B), mv(self.scales), mv(self.zero_points),
                          mv(self.bias), self.s_dtype, dict(self.meta))


def _half(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DTYPES[dtype])


def make_matmul_case(M: int, K: int, N: int, block_size: int, bits: int, *,
                     a_dtype: str = "bf16", s_dtype: str | None = None,
                     has_zp: bool = True, has_bias: bool = False, seed: int = 0,
                     scale_range=(0.002, 0.02), a_std: float = 1.0) -> MatmulCase:
    """Random MatMulNBits inputs with the recipe of the module docstring."""
    s_dtype = s_dtype or a_dtype
    rng = np.random.default_rng(seed)
    kb = n_blocks(K, block_size)
    blob = block_size * bits // 8
    A = _half(rng.standard_normal((M, K), dtype=np.float32) * a_std, a_dtype)
    B = torch.from_numpy(rng.integers(0, 256, size=(N, kb, blob), dtype=np.uint8))
    scales = _half(rng.uniform(scale_range[0], scale_range[1], size=(N, kb)), s_dtype)
    zp = None
    if has_zp:
        zp = torch.from_numpy(rng.integers(0, 256, size=(N, -(-(kb * bits) // 8)),
                                           dtype=np.uint8))
    bias = None
    if has_bias:
        bias = _half(rng.standard_normal(N, dtype=np.float32), a_dtype)
    return MatmulCase(M, K, N, block_size, bits, a_dtype, A, B, scales, zp, bias, s_dtype)


# -- The five named workloads -----------------------------------------------

def tiny_matmulnbits(seed: int = 1) -> MatmulCase:
    """M=1, K=N=256, f32 activations, 4-bit symmetric bs=32, f32 scales in
    [0.005, 0.02], implicit zero point 8, f32 output."""
    return make_matmul_case(1, 256, 256, 32, 4, a_dtype="f32", s_dtype="f32", has_zp=False,
                            seed=seed, scale_range=(0.005, 0.02))


# Llama-3-8B-shaped decoder layer projections: (name, K, N).
LLAMA3_8B_LAYER = [
    ("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024), ("o", 4096, 4096),
    ("gate", 4096, 14336), ("up", 4096, 14336), ("down", 14336, 4096),
]


def decode_layer(seed: int = 2) -> list[MatmulCase]:
    """M=1 decode GEMV over one Llama-3-8B-shaped layer: bf16 activations,
    4-bit asymmetric bs=32, bf16 scales in [0.002, 0.02], packed zero points."""
    out = []
    for i, (name, K, N) in enumerate(LLAMA3_8B_LAYER):
        c = make_matmul_case(1, K, N, 32, 4, a_dtype="bf16", has_zp=True, seed=seed * 100 + i)
        c.meta["name"] = name
        out.append(c)
    return out


# Projections of the layer that read the same activations, stored as one
# weight matrix (their rows of B, scales and zero points stacked along N).
FUSED_GROUPS = [("qkv", ("q", "k", "v")), ("o", ("o",)), ("gate_up", ("gate", "up")),
                ("down", ("down",))]


def concat_along_n(cases: list[MatmulCase], name: str) -> MatmulCase:
    """One MatMulNBits problem whose weights are the given problems' weights
    stacked along N (same K, block size, bits and dtypes); the activations are
    the first problem's.  Output column n of the result is output column n' of
    the problem that row came from, so the layer's projections that share an
    input run as one launch.  Pure concatenation of the operator's layout."""
    c0 = cases[0]
    for c in cases[1:]:
        assert (c.M, c.K, c.block_size, c.bits, c.a_dtype, c.s_dtype) == \
            (c0.M, c0.K, c0.block_size, c0.bits, c0.a_dtype, c0.s_dtype)
        assert (c.zero_points is None) == (c0.zero_points is None)
        assert (c.bias is None) == (c0.bias is None)
    cat = lambda ts: None if ts[0] is None else torch.cat(ts, dim=0)
    out = MatmulCase(c0.M, c0.K, sum(c.N for c in cases), c0.block_size, c0.bits, c0.a_dtype,
                     c0.A, cat([c.B for c in cases]), cat([c.scales for c in cases]),
                     cat([c.zero_points for c in cases]), cat([c.bias for c in cases]),
                     c0.s_dtype)
    out.meta["name"] = name
    out.meta["parts"] = [(c.meta.get("name"), c.N) for c in cases]
    return out


def decode_layer_fused(seed: int = 2) -> list[MatmulCase]:
    """The decode layer as it runs with fused projections: q|k|v and gate|up
    each as one matrix (stacked along N), o and down alone -- four launches
    in the order the layer's data dependencies allow (qkv, o, gate_up, down).
    The weights are those of decode_layer(seed)."""
    by_name = {c.meta["name"]: c for c in decode_layer(seed)}
    return [concat_along_n([by_name[p] for p in parts], name) for name, parts in FUSED_GROUPS]


# (bits, block_size, asymmetric) of the batched-decode CompInt8 workload.
COMPINT8_VARIANTS = [(4, 128, False), (8, 64, True), (2, 64, True)]


def compint8_case(M: int, bits: int, block_size: int, asym: bool, seed: int = 3,
                  K: int = 4096, N: int = 14336) -> MatmulCase:
    """Batched-decode CompInt8: bf16 activations, K=4096, N=14336."""
    c = make_matmul_case(M, K, N, block_size, bits, a_dtype="bf16", has_zp=asym,
                         seed=seed * 1000 + M * 10 + bits)
    c.meta["name"] = f"compint8_b{bits}_bs{block_size}_M{M}"
    return c


def prefill_gemm(seed: int = 4, M: int = 2048, K: int = 4096, N: int = 14336) -> MatmulCase:
    """Prefill GEMM: bf16 activations, 4-bit asymmetric bs=32, bf16 output."""
    c = make_matmul_case(M, K, N, 32, 4, a_dtype="bf16", has_zp=True, seed=seed)
    c.meta["name"] = "prefill"
    return c


@dataclass
class Fp4Case:
    """Block-scaled FP4 weights (MXFP4 / NVFP4) with float activations."""
    M: int
    K: int
    N: int
    fmt: str                        # "mxfp4" (E8M0 / 32) or "nvfp4" (E4M3 / 16)
    A: torch.Tensor                 # [M, K] a_dtype
    W: torch.Tensor                 # [N, kb, bs/2] uint8 E2M1 codes
    scales: torch.Tensor            # [N, kb] uint8 scale bytes
    global_scale: float
    bias: torch.Tensor | None

    @property
    def block_size(self) -> int:
        return 32 if self.fmt == "mxfp4" else 16

    def weight_bytes(self) -> int:
        return self.W.numel() + self.scales.numel()

    def to(self, device) -> "Fp4Case":
        mv = lambda t: None if t is None else t.to(device)
        return Fp4Case(self.M, self.K, self.N, self.fmt, mv(self.A), mv(self.W),
                       mv(self.scales), self.global_scale, mv(self.bias))


def make_fp4_case(M: int, K: int, N: int, fmt: str, *, a_dtype: str = "bf16",
                  has_bias: bool = False, seed: int = 0) -> Fp4Case:
    """Random block-scaled FP4 inputs: activations N(0,1), codes uniform random
    bytes (every nibble uniform over the 16 E2M1 codes), scale bytes uniform
    over a range of ordinary magnitudes -- E8M0 118..125 (2^-9 .. 2^-2) for
    MXFP4; E4M3 0x18..0x37 (2^-4 .. 2^-1 * 1.875) and a global scale 0.25 for
    NVFP4 -- so that weights are of the size of the integer workloads'."""
    rng = np.random.default_rng(seed)
    bs = 32 if fmt == "mxfp4" else 16
    kb = n_blocks(K, bs)
    A = _half(rng.standard_normal((M, K), dtype=np.float32), a_dtype)
    W = torch.from_numpy(rng.integers(0, 256, size=(N, kb, bs // 2), dtype=np.uint8))
    if fmt == "mxfp4":
        sc = rng.integers(118, 126, size=(N, kb), dtype=np.uint8)
        g = 1.0
    else:
        sc = rng.integers(0x18, 0x38, size=(N, kb), dtype=np.uint8)
        g = 0.25
    bias = _half(rng.standard_normal(N, dtype=np.float32), a_dtype) if has_bias else None
    return Fp4Case(M, K, N, fmt, A, W, torch.from_numpy(sc), g, bias)


@dataclass
class ConvCase:
    X: torch.Tensor         # NHWC int8
    W: torch.Tensor         # OHWI int8
    bias: torch.Tensor      # [Co] int32
    w_scale: torch.Tensor   # [Co] float32
    in_scale: float
    out_scale: float
    in_zp: int
    out_zp: int
    clamp_min: int
    clamp_max: int
    stride: tuple
    pad: tuple

    def to(self, device) -> "ConvCase":
        return ConvCase(self.X.to(device), self.W.to(device), self.bias.to(device),
                        self.w_scale.to(device), self.in_scale, self.out_scale, self.in_zp,
                        self.out_zp, self.clamp_min, self.clamp_max, self.stride, self.pad)


def make_conv_case(Nb=1, H=56, W=56, C=64, Co=64, KH=3, KW=3, stride=(1, 1), pad=(1, 1),
                   in_scale=0.02, out_scale=0.05, in_zp=0, out_zp=0, clamp=(-128, 127),
                   seed=5, w_scale_range=(0.001, 0.01), bias_range=(-1000, 1000)) -> ConvCase:
    """int8 NHWC conv: input uniform over [-128, 127], OHWI weights uniform over
    [-127, 127], per-channel float32 weight scales, int32 bias."""
    rng = np.random.default_rng(seed)
    X = torch.from_numpy(rng.integers(-128, 128, size=(Nb, H, W, C), dtype=np.int8))
    Wt = torch.from_numpy(rng.integers(-127, 128, size=(Co, KH, KW, C), dtype=np.int8))
    ws = torch.from_numpy(rng.uniform(*w_scale_range, size=Co).astype(np.float32))
    bias = torch.from_numpy(rng.integers(bias_range[0], bias_range[1] + 1, size=Co,
                                         dtype=np.int32))
    return ConvCase(X, Wt, bias, ws, in_scale, out_scale, in_zp, out_zp, clamp[0], clamp[1],
                    stride, pad)
