"""CPU oracle for block-quantized-weight matmuls (test infrastructure only).

This package is the independent checker.  Only the test-suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the product path
(the HIP library and its Python binding) never does, and shares no code with
it.  The arithmetic lives in ``qmm_oracle.c`` (plain C, natural loop order,
double accumulation, exact integers); this module only marshals numpy arrays.

Every function cites the passage of the web pages it follows:

* "onnx-runtime-ep-cpu matmul_nbits.rs" -- MatMulNBits: the module
  documentation (layout ``[N, ceil(K/bs), bs*bits/8]``, LSB first), the
  ``dequantize_nbits_value`` formula, the group-index branch of
  ``dequantize_weight`` and the ``g_idx`` checks of ``execute``,
  ``quantize_activation_signed`` and the CompInt8 block dot of
  ``int4_dot_row_scalar`` / ``int8_row``.
* "rlx-cpu quant.rs" -- ``exec_q_mat_mul`` (int32 accumulate, requantize,
  clamp), the ``QConv2d`` attribute set, ``dequant_matmul_nvfp4`` and the
  low-precision scaled-GEMM reference (``lowp_compute_scales``,
  ``lowp_quantize``, ``lowp_dequantize``, ``lowp_scaled_matmul``): FP8 / FP6 /
  FP4 codes with per-tensor, MX (E8M0 per 32) or NVFP4 (E4M3 per 16) scales.
* "MNN ConvInt8TiledExecutor.cpp" -- zero-point padding of the im2col and the
  clamp defaults.

Parity is pinned (see ``tests/test_oracle_*.py``) against hand-decoded bytes,
closed-form invariants, rounding-tie cases and independent brute-force numpy
formulations.  The float matmul on the large seeded configurations has no
printed values on the pages; there only the tolerance applies.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# -O2 without fast-math and without FMA contraction: the binary32 decisions
# (activation quantization, conv requantization) must be the plain IEEE ops.
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
          "-shared", "-std=c99", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile ``qmm_oracle.c`` with gcc into ``liboracle.so`` (in-tree)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        _lib = ctypes.CDLL(_LIB_PATH)
        i64, i32, f32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p
        sig = {
            "oracle_unpack_codes": [vp, i64, i64, i64, i32, vp],
            "oracle_unpack_zero_points": [vp, i64, i64, i32, vp],
            "oracle_pack_codes": [vp, i64, i64, i64, i32, vp],
            "oracle_pack_zero_points": [vp, i64, i64, i32, vp],
            "oracle_dequantize": [vp, vp, vp, vp, i64, i64, i64, i32, vp],
            "oracle_matmul_nbits": [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp, vp],
            "oracle_check_g_idx": [vp, i64, i64, i64],
            "oracle_quantize_a16": [vp, i64, i64, i64, vp, vp],
            "oracle_int16_matmul": [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp, vp],
            "oracle_fp4_dequantize": [vp, vp, i32, ctypes.c_double, i64, i64, vp],
            "oracle_fp4_matmul": [vp, vp, vp, i32, ctypes.c_double, vp, i64, i64, i64, vp, vp],
            "oracle_e2m1": [ctypes.c_uint],
            "oracle_e8m0": [ctypes.c_uint],
            "oracle_e4m3": [ctypes.c_uint],
            "oracle_quantize_a": [vp, i64, i64, i64, vp, vp],
            "oracle_compint8_block_dots": [vp, vp, vp, i64, i64, i64, i64, i32, vp],
            "oracle_compint8_matmul": [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp, vp],
            "oracle_conv_int8": [vp, vp, vp, vp, f32, f32, i32, i32, i32, i32, i32, i32,
                                 i32, i32, i32, i32, i32, i32, i32, i32, i32, vp, vp],
            "oracle_lowp_decode": [i32, ctypes.c_uint],
            "oracle_lowp_max_finite": [i32],
            "oracle_lowp_encode": [i32, ctypes.c_double],
            "oracle_f32_to_e8m0": [f32],
            "oracle_lowp_snap_scale": [i32, f32],
            "oracle_lowp_compute_scales": [vp, i32, i32, i64, i64, vp],
            "oracle_lowp_store_scales": [vp, i32, i64, vp],
            "oracle_lowp_read_scales": [vp, i32, i64, vp],
            "oracle_lowp_quantize": [vp, vp, i32, i32, i64, i64, vp],
            "oracle_lowp_dequantize": [vp, vp, i32, i32, i64, i64, vp],
            "oracle_lowp_scaled_matmul": [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, vp,
                                          vp],
        }
        for name, argtypes in sig.items():
            fn = getattr(_lib, name)
            fn.argtypes = argtypes
            fn.restype = None
        _lib.oracle_check_g_idx.restype = i64
        for name in ("oracle_e2m1", "oracle_e8m0", "oracle_e4m3", "oracle_lowp_decode",
                     "oracle_lowp_max_finite"):
            getattr(_lib, name).restype = ctypes.c_double
        _lib.oracle_lowp_encode.restype = ctypes.c_uint
        _lib.oracle_f32_to_e8m0.restype = ctypes.c_uint
        _lib.oracle_lowp_snap_scale.restype = f32
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def n_blocks(K: int, block_size: int) -> int:
    """ceil(K / block_size) (MatMulNBits module documentation)."""
    return -(-K // block_size)


def blob_bytes(block_size: int, bits: int) -> int:
    return block_size * bits // 8


def zp_row_bytes(k_blocks: int, bits: int) -> int:
    return -(-(k_blocks * bits) // 8)


# -- O1 codec ---------------------------------------------------------------

def unpack_codes(B, N, K, block_size, bits):
    """Codes ``[N, K]`` (uint8) from packed ``B`` (dequantize_nbits_value)."""
    B = _c(B, np.uint8)
    out = np.empty((N, K), np.uint8)
    _load().oracle_unpack_codes(_ptr(B), N, K, block_size, bits, _ptr(out))
    return out


def unpack_zero_points(zp, N, k_blocks, bits):
    """Zero points ``[N, kb]``; ``zp=None`` gives the default 2^(bits-1)."""
    zp = _c(zp, np.uint8)
    out = np.empty((N, k_blocks), np.uint8)
    _load().oracle_unpack_zero_points(_ptr(zp), N, k_blocks, bits, _ptr(out))
    return out


def pack_codes(codes, block_size, bits):
    """Inverse of :func:`unpack_codes`; ``codes`` is ``[N, K]``."""
    codes = _c(codes, np.uint8)
    N, K = codes.shape
    kb = n_blocks(K, block_size)
    out = np.empty((N, kb, blob_bytes(block_size, bits)), np.uint8)
    _load().oracle_pack_codes(_ptr(codes), N, K, block_size, bits, _ptr(out))
    return out


def pack_zero_points(zps, bits):
    """Inverse of :func:`unpack_zero_points`; ``zps`` is ``[N, kb]``."""
    zps = _c(zps, np.uint8)
    N, kb = zps.shape
    out = np.empty((N, zp_row_bytes(kb, bits)), np.uint8)
    _load().oracle_pack_zero_points(_ptr(zps), N, kb, bits, _ptr(out))
    return out


class GroupIndexError(ValueError):
    """g_idx has the wrong length or an entry outside 0..kb."""


def check_g_idx(g_idx, K, block_size):
    """Range and shape check of group indices (MatMulNBits ``execute``: shape
    ``[K]`` or ``[kb * block_size]``; ``dequantize_weight``: every entry in
    ``0..kb``).  Returns the int32 array or raises :class:`GroupIndexError`."""
    g = _c(np.ravel(g_idx), np.int32)
    r = _load().oracle_check_g_idx(_ptr(g), g.size, K, block_size)
    kb = n_blocks(K, block_size)
    if r == -1:
        raise GroupIndexError(f"g_idx must have shape [{K}] or [{kb * block_size}], got "
                              f"[{g.size}]")
    if r < g.size:
        raise GroupIndexError(f"g_idx[{r}]={int(g[r])} is outside 0..{kb}")
    return g


def dequantize(B, scales, zp, N, K, block_size, bits, g_idx=None):
    """Dense float64 ``[N, K]`` weight (code - zp) * scale; with ``g_idx`` the
    scale and zero point of element k are those of group ``g_idx[k]``."""
    B = _c(B, np.uint8)
    s = _c(scales, np.float64)
    zp = _c(zp, np.uint8)
    g = None if g_idx is None else check_g_idx(g_idx, K, block_size)
    out = np.empty((N, K), np.float64)
    _load().oracle_dequantize(_ptr(B), _ptr(s), _ptr(zp), _ptr(g), N, K, block_size, bits,
                              _ptr(out))
    return out


# -- O2 float matmul ---------------------------------------------------------

def matmul_nbits(A, B, scales, zp, bias, N, K, block_size, bits, g_idx=None):
    """Y = A @ W_deq^T (+ bias) in float64, plus the tolerance base S.

    ``A`` is ``[M, K]`` (any float dtype, widened exactly to float64).
    ``g_idx`` (optional, ``[K]`` or ``[kb * block_size]`` int32) selects the
    scale and zero point of element k (group ``g_idx[k]`` instead of its
    block); it is range-checked first.
    Returns ``(Y, S)`` with ``S[m, n] = sum_k |A[m,k] w(n,k)| + |bias[n]|``.
    """
    A = _c(np.atleast_2d(A), np.float64)
    M = A.shape[0]
    B = _c(B, np.uint8)
    s = _c(scales, np.float64)
    zp = _c(zp, np.uint8)
    bias = _c(bias, np.float64)
    g = None if g_idx is None else check_g_idx(g_idx, K, block_size)
    Y = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64)
    _load().oracle_matmul_nbits(_ptr(A), _ptr(B), _ptr(s), _ptr(zp), _ptr(g), _ptr(bias), M, N,
                                K, block_size, bits, _ptr(Y), _ptr(S))
    return Y, S


# -- O3/O4 CompInt8 ------------------------------------------------------------

def quantize_a(A, K, block_size):
    """Per-row, per-block symmetric int8 quantization of float32 activations.

    Returns ``qa`` ``[M, kb*bs]`` int8 (zero past K) and ``sa`` ``[M, kb]``
    float32 (quantize_activation_signed).
    """
    A = _c(np.atleast_2d(A), np.float32)
    M = A.shape[0]
    kb = n_blocks(K, block_size)
    qa = np.empty((M, kb * block_size), np.int8)
    sa = np.empty((M, kb), np.float32)
    _load().oracle_quantize_a(_ptr(A), M, K, block_size, _ptr(qa), _ptr(sa))
    return qa, sa


def quantize_a16(A, K, block_size):
    """Per-row, per-block symmetric int16 quantization (the int16-activation
    route of MatMulNBits ``execute``): ``qa`` ``[M, kb*bs]`` int16 (zero past
    K), ``sa`` ``[M, kb]`` float32 = max|x| / 32767."""
    A = _c(np.atleast_2d(A), np.float32)
    M = A.shape[0]
    kb = n_blocks(K, block_size)
    qa = np.empty((M, kb * block_size), np.int16)
    sa = np.empty((M, kb), np.float32)
    _load().oracle_quantize_a16(_ptr(A), M, K, block_size, _ptr(qa), _ptr(sa))
    return qa, sa


def int16_matmul(qa, sa, B, scales, zp, bias, N, K, block_size, bits):
    """int16-activation output in float64 and its tolerance base ``S``."""
    qa = _c(qa, np.int16)
    sa = _c(sa, np.float32)
    M = qa.shape[0]
    Y = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64)
    _load().oracle_int16_matmul(_ptr(qa), _ptr(sa), _ptr(_c(B, np.uint8)),
                                _ptr(_c(scales, np.float64)), _ptr(_c(zp, np.uint8)),
                                _ptr(_c(bias, np.float64)), M, N, K, block_size, bits, _ptr(Y),
                                _ptr(S))
    return Y, S


def compint8_block_dots(qa, B, zp, N, K, block_size, bits):
    """Exact int32 block dots ``[M, N, kb]``."""
    qa = _c(qa, np.int8)
    M = qa.shape[0]
    kb = n_blocks(K, block_size)
    out = np.empty((M, N, kb), np.int32)
    _load().oracle_compint8_block_dots(_ptr(qa), _ptr(_c(B, np.uint8)), _ptr(_c(zp, np.uint8)),
                                       M, N, K, block_size, bits, _ptr(out))
    return out


def compint8_matmul(qa, sa, B, scales, zp, bias, N, K, block_size, bits):
    """CompInt8 output in float64 and its tolerance base ``S``."""
    qa = _c(qa, np.int8)
    sa = _c(sa, np.float32)
    M = qa.shape[0]
    Y = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64)
    _load().oracle_compint8_matmul(_ptr(qa), _ptr(sa), _ptr(_c(B, np.uint8)),
                                   _ptr(_c(scales, np.float64)), _ptr(_c(zp, np.uint8)),
                                   _ptr(_c(bias, np.float64)), M, N, K, block_size, bits,
                                   _ptr(Y), _ptr(S))
    return Y, S


# -- Block-scaled FP4 weights ([RLX] dequant_matmul_nvfp4, lowp_*) ------------

FP4_FORMATS = {"mxfp4": 0, "nvfp4": 1}
FP4_BLOCK = {"mxfp4": 32, "nvfp4": 16}


def e2m1(code):
    """Value of an FP4 E2M1 code (OCP Microscaling element format)."""
    return _load().oracle_e2m1(int(code))


def e8m0(byte):
    """Value of an E8M0 scale byte: 2^(e - 127), nan for 255."""
    return _load().oracle_e8m0(int(byte))


def e4m3(byte):
    """Value of an FP8 E4M3 byte (bias 7, subnormals, nan = S.1111.111)."""
    return _load().oracle_e4m3(int(byte))


def fp4_dequantize(W, scales, fmt, global_scale, N, K):
    """Dense float64 ``[N, K]`` weight e2m1(code) * scale * global_scale."""
    W = _c(W, np.uint8)
    s = _c(scales, np.uint8)
    out = np.empty((N, K), np.float64)
    _load().oracle_fp4_dequantize(_ptr(W), _ptr(s), FP4_FORMATS[fmt], float(global_scale), N, K,
                                  _ptr(out))
    return out


def fp4_matmul(A, W, scales, fmt, global_scale, bias, N, K):
    """Y = A @ W_fp4^T (+ bias) in float64 and the tolerance base S, for
    ``fmt`` "mxfp4" (E8M0 scales per 32) or "nvfp4" (E4M3 per 16, times
    ``global_scale``)."""
    A = _c(np.atleast_2d(A), np.float64)
    M = A.shape[0]
    Y = np.empty((M, N), np.float64)
    S = np.empty((M, N), np.float64)
    _load().oracle_fp4_matmul(_ptr(A), _ptr(_c(W, np.uint8)), _ptr(_c(scales, np.uint8)),
                              FP4_FORMATS[fmt], float(global_scale), _ptr(_c(bias, np.float64)),
                              M, N, K, _ptr(Y), _ptr(S))
    return Y, S


# -- Low-precision scaled GEMM ([RLX] quant.rs: lowp_* reference) -------------

LOWP_FORMATS = {"e4m3": 0, "e5m2": 1, "e2m3": 2, "e3m2": 3, "e2m1": 4}
LOWP_LAYOUTS = {"tensor": 0, "mx": 1, "nvfp4": 2}
LOWP_BLOCK = {"mx": 32, "nvfp4": 16}


def _fmt(f):
    return LOWP_FORMATS[f] if isinstance(f, str) else int(f)


def _lay(l):
    return LOWP_LAYOUTS[l] if isinstance(l, str) else int(l)


def lowp_decode(fmt, code):
    """Value of one code of an element format (e4m3, e5m2, e2m3, e3m2, e2m1)."""
    return _load().oracle_lowp_decode(_fmt(fmt), int(code))


def lowp_encode(fmt, v):
    """Code of the finite value nearest to v (ties to even, saturating)."""
    return int(_load().oracle_lowp_encode(_fmt(fmt), float(v)))


def lowp_max_finite(fmt):
    return _load().oracle_lowp_max_finite(_fmt(fmt))


def f32_to_e8m0(s):
    return int(_load().oracle_f32_to_e8m0(float(np.float32(s))))


def lowp_snap_scale(layout, s):
    return float(_load().oracle_lowp_snap_scale(_lay(layout), float(np.float32(s))))


def lowp_nblk(cols, layout):
    return 1 if _lay(layout) == 0 else -(-cols // LOWP_BLOCK[["tensor", "mx", "nvfp4"][_lay(layout)]])


def lowp_compute_scales(x, fmt, layout):
    """Raw float32 scales of x [rows, cols] (lowp_compute_scales)."""
    x = _c(np.atleast_2d(x), np.float32)
    rows, cols = x.shape
    out = np.empty(1 if _lay(layout) == 0 else rows * lowp_nblk(cols, layout), np.float32)
    _load().oracle_lowp_compute_scales(_ptr(x), _fmt(fmt), _lay(layout), rows, cols, _ptr(out))
    return out if _lay(layout) == 0 else out.reshape(rows, -1)


def lowp_store_scales(scales, layout):
    """Stored form of raw scales: float32 (per tensor) or one byte each."""
    s = _c(np.ravel(scales), np.float32)
    out = np.empty(1, np.float32) if _lay(layout) == 0 else np.empty(s.size, np.uint8)
    _load().oracle_lowp_store_scales(_ptr(s), _lay(layout), s.size, _ptr(out))
    return out if _lay(layout) == 0 else out.reshape(np.shape(scales))


def lowp_read_scales(stored, layout):
    """Raw float32 scales from their stored form (lowp_read_scales)."""
    st = np.ascontiguousarray(stored)
    n = 1 if _lay(layout) == 0 else st.size
    out = np.empty(n, np.float32)
    _load().oracle_lowp_read_scales(_ptr(st), _lay(layout), n, _ptr(out))
    return out if _lay(layout) == 0 else out.reshape(np.shape(stored))


def lowp_quantize(x, scales, fmt, layout):
    """Codes [rows, cols] (one per byte) of x with raw scales (lowp_quantize)."""
    x = _c(np.atleast_2d(x), np.float32)
    rows, cols = x.shape
    out = np.empty((rows, cols), np.uint8)
    _load().oracle_lowp_quantize(_ptr(x), _ptr(_c(scales, np.float32)), _fmt(fmt), _lay(layout),
                                 rows, cols, _ptr(out))
    return out


def lowp_dequantize(codes, scales, fmt, layout):
    codes = _c(np.atleast_2d(codes), np.uint8)
    rows, cols = codes.shape
    out = np.empty((rows, cols), np.float64)
    _load().oracle_lowp_dequantize(_ptr(codes), _ptr(_c(scales, np.float32)), _fmt(fmt),
                                   _lay(layout), rows, cols, _ptr(out))
    return out


def lowp_scaled_matmul(lhs, rhs, lhs_scales, rhs_scales, bias, layout, lhs_fmt, rhs_fmt):
    """out = dequant(lhs) . dequant(rhs)^T (+ bias) in float64 and S = sum |a b|
    (lowp_scaled_matmul; lhs [m, k], rhs [n, k] codes, raw float32 scales)."""
    lhs = _c(np.atleast_2d(lhs), np.uint8)
    rhs = _c(np.atleast_2d(rhs), np.uint8)
    m, k = lhs.shape
    n = rhs.shape[0]
    out = np.empty((m, n), np.float64)
    S = np.empty((m, n), np.float64)
    _load().oracle_lowp_scaled_matmul(_ptr(lhs), _ptr(rhs), _ptr(_c(lhs_scales, np.float32)),
                                      _ptr(_c(rhs_scales, np.float32)), _ptr(_c(bias, np.float64)),
                                      m, n, k, _lay(layout), _fmt(lhs_fmt), _fmt(rhs_fmt),
                                      _ptr(out), _ptr(S))
    return out, S


# -- O5 int8 conv --------------------------------------------------------------

def conv_int8(X, W, bias, w_scale, in_scale, out_scale, in_zp=0, out_zp=0,
              clamp_min=-128, clamp_max=127, stride=(1, 1), pad=(0, 0)):
    """int8 NHWC conv (OHWI weights) with int32 bias and binary32 requant.

    Returns ``(Y int8 [Nb, OH, OW, Co], acc int32 [Nb, OH, OW, Co])``.
    """
    X = _c(X, np.int8)
    W = _c(W, np.int8)
    Nb, H, Wd, C = X.shape
    Co, KH, KW, C2 = W.shape
    assert C2 == C
    sh, sw = stride
    ph, pw = pad
    OH = (H + 2 * ph - KH) // sh + 1
    OW = (Wd + 2 * pw - KW) // sw + 1
    Y = np.empty((Nb, OH, OW, Co), np.int8)
    acc = np.empty((Nb, OH, OW, Co), np.int32)
    _load().oracle_conv_int8(_ptr(X), _ptr(W), _ptr(_c(bias, np.int32)),
                             _ptr(_c(w_scale, np.float32)), float(in_scale), float(out_scale),
                             int(in_zp), int(out_zp), int(clamp_min), int(clamp_max),
                             Nb, H, Wd, C, Co, KH, KW, sh, sw, ph, pw, _ptr(Y), _ptr(acc))
    return Y, acc
