"""CPU-side checks of the C ABI: the library loads, exports every function
include/qmm.h declares, and rejects bad arguments on the host (before any
device work) with a status code and a what / why / how-to-fix message."""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "qmm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(qmm\w+|qconv\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def qmm():
    from block_quantized_weight_matmulnbits_amd import qmm as q
    return q


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["qmm_gemv", "qmm_gemm", "qmm_gemm_compint8", "qconv_int8",
              "qmm_compint8_workspace_size", "qmm_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol(qmm):
    for name in declared_functions():
        assert hasattr(qmm.lib, name), name
    assert set(declared_functions()) <= set(qmm.EXPORTED)


FAKE = 0x10000   # never dereferenced: validation fails before any device work


def gemv(qmm, **kw):
    a = dict(A=FAKE, a_dtype=2, B=FAKE, b_layout=0, scales=FAKE, s_dtype=2, zp=None, bias=None,
             Y=FAKE, K=4096, N=4096, bs=32, bits=4, acc=0)
    a.update(kw)
    return qmm.lib.qmm_gemv(a["A"], a["a_dtype"], a["B"], a["b_layout"], a["scales"],
                            a["s_dtype"], a["zp"], a.get("g", None), a.get("glen", 0), a["bias"],
                            a["Y"], a["K"], a["N"], a["bs"], a["bits"], a["acc"], None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(bits=5), -1, "bits must be 2, 3, 4 or 8"),
    (dict(bits=3, b_layout=1, scales=None), -2, "3-bit weights run on the operator's layout"),
    (dict(bits=16), -1, "bits must be 2, 3, 4 or 8"),
    (dict(bs=8), -1, "power of two and at least 16"),
    (dict(bs=48), -1, "power of two and at least 16"),
    (dict(K=0), -1, "K and N must be positive"),
    (dict(N=-3), -1, "K and N must be positive"),
    (dict(a_dtype=7), -1, "not a qmm_dtype"),
    (dict(b_layout=5), -1, "not a qmm_layout"),
    (dict(b_layout=1), -1, "must be NULL"),
    (dict(b_layout=2, scales=None, B=FAKE + 16), -1, "256-byte aligned"),
    (dict(acc=4), -1, "qmm_gemm_compint8"),
    (dict(acc=9), -1, "accuracy_level must be in 0..4"),
    (dict(B=None), -1, "non-null"),
    (dict(Y=None), -1, "non-null"),
    (dict(B=FAKE + 8), -1, "16-byte aligned"),
    (dict(A=FAKE + 1), -1, "aligned to their element size"),
    (dict(K=1 << 31), -2, "below 2^30"),
    (dict(g=None, glen=5), -1, "g_idx is NULL"),
    (dict(g=FAKE, glen=100), -1, "g_idx must have shape [4096] or [4096]"),
    (dict(g=FAKE + 2, glen=4096), -1, "g_idx must be 4-byte aligned"),
    (dict(g=FAKE, glen=4096, b_layout=2, scales=None), -2, "operator's layout only"),
    (dict(bits=3, g=FAKE, glen=4096), -2, "not supported with 3-bit weights"),
    (dict(bits=3, bs=16384, K=16384), -2, "block_size <= 8192"),
])
def test_gemv_rejects_bad_arguments(qmm, kw, code, needle):
    assert gemv(qmm, **kw) == code
    msg = qmm.qmm_last_error()
    assert needle in msg, msg
    if code == -1 and "bits" in needle:
        assert "Why" in msg and "How to fix" in msg


def test_compint8_requires_level_4_and_workspace_size(qmm):
    st = qmm.lib.qmm_gemm_compint8(FAKE, 2, FAKE, 0, FAKE, 2, None, None, 0, None, FAKE, 4, 4096, 4096, 128,
                                   4, 0, FAKE, 1 << 20, None)
    assert st == -1 and "accuracy_level must be 4" in qmm.qmm_last_error()
    # int8 activations [M, kb*bs] + float scales [M, kb], regions 256-byte aligned.
    ws = qmm.qmm_compint8_workspace_size(16, 4096, 128)
    assert ws >= 16 * 4096 + 4 * 16 * 32 and ws % 256 == 0
    assert qmm.qmm_compint8_workspace_size(1, 100, 64) >= 128 + 4 * 2
    st = qmm.lib.qmm_gemm_compint8(FAKE, 2, FAKE, 0, FAKE, 2, None, None, 0, None, FAKE, 4, 4096, 4096, 128,
                                   4, 4, FAKE, 100, None)
    assert st == -3 and "workspace" in qmm.qmm_last_error()


def test_gemm_with_m_zero_is_a_noop(qmm):
    st = qmm.lib.qmm_gemm(None, 2, FAKE, 0, FAKE, 2, None, None, 0, None, None, 0, 64, 64, 32, 4, 0, None)
    assert st == 0


def conv(qmm, **kw):
    a = dict(X=FAKE, W=FAKE, bias=None, ws=FAKE, in_scale=0.02, out_scale=0.05, in_zp=0, out_zp=0,
             lo=-128, hi=127, Nb=1, H=56, Wd=56, C=64, Co=64, KH=3, KW=3, sh=1, sw=1, ph=1, pw=1,
             Y=FAKE)
    a.update(kw)
    return qmm.lib.qconv_int8(a["X"], a["W"], a["bias"], a["ws"], a["in_scale"], a["out_scale"],
                              a["in_zp"], a["out_zp"], a["lo"], a["hi"], a["Nb"], a["H"], a["Wd"],
                              a["C"], a["Co"], a["KH"], a["KW"], a["sh"], a["sw"], a["ph"], a["pw"],
                              a["Y"], None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(X=None), -1, "non-null"),
    (dict(sh=0), -1, "strides must be >= 1"),
    (dict(KH=9, ph=0, H=4), -1, "smaller than the kernel"),
    (dict(lo=10, hi=5), -1, "clamp_min"),
    (dict(in_zp=300), -1, "in_zp"),
    (dict(out_scale=0.0), -1, "out_scale"),
    (dict(C=1 << 20), -2, "too large"),
])
def test_conv_rejects_bad_arguments(qmm, kw, code, needle):
    assert conv(qmm, **kw) == code
    assert needle in qmm.qmm_last_error(), qmm.qmm_last_error()


def test_repacked_bytes_geometry(qmm):
    # 4-bit, K=4096, N=4096, bs=32, bf16 scales, zero points: 128 groups of 32
    # columns, 64 chunks of 64 codes (32 bytes per column chunk), 128 blocks.
    codes = 128 * 64 * 32 * 32
    scales = 128 * 128 * 32 * 2
    zps = 128 * 128 * 32 * 4 // 8
    assert qmm.qmm_repacked_bytes(4096, 4096, 32, 4, 2, True) == codes + scales + zps
    assert qmm.qmm_repacked_bytes(4096, 4096, 32, 4, 2, False) == codes + scales
    # Ragged: K=100 (kb=4 blocks of 32 -> 128 codes -> 2 chunks), N=33 (2 groups),
    # each region rounded up to 256 bytes.
    r = lambda v: (v + 255) // 256 * 256
    assert qmm.qmm_repacked_bytes(100, 33, 32, 8, 0, True) == (
        r(2 * 2 * 32 * 64) + r(2 * 4 * 32 * 4) + r(2 * 4 * 32))
    assert qmm.qmm_repacked_bytes(100, 33, 24, 4, 2, True) == 0      # bad block size
    assert qmm.qmm_repacked_bytes(100, 33, 32, 3, 2, True) == 0      # bad bits


def test_repack_rejects_bad_arguments(qmm):
    st = qmm.lib.qmm_repack(FAKE, FAKE, 2, None, 4096, 4096, 32, 4, FAKE, 100, None)
    assert st == -1 and "at least" in qmm.qmm_last_error()
    st = qmm.lib.qmm_repack(FAKE, FAKE, 2, None, 4096, 4096, 32, 4, FAKE + 64, 1 << 30, None)
    assert st == -1 and "256-byte aligned" in qmm.qmm_last_error()
    st = qmm.lib.qmm_repack(FAKE, FAKE, 2, None, 4096, 4096, 32, 5, FAKE, 1 << 30, None)
    assert st == -1 and "bits" in qmm.qmm_last_error()
    st = qmm.lib.qmm_unrepack(FAKE, 1, 4096, 4096, 32, 4, 2, FAKE, FAKE, None, None)
    assert st == -1 and "zero_points" in qmm.qmm_last_error()


def test_compint8_tiled_layout_needs_whole_chunks_per_block(qmm):
    st = qmm.lib.qmm_gemm_compint8(FAKE, 2, FAKE, 1, None, 2, None, None, 0, None, FAKE, 4, 4096, 4096, 16,
                                   4, 4, FAKE, 1 << 30, None)
    assert st == -2 and "block_size >= 32" in qmm.qmm_last_error()
    # M = 1 takes blocks down to one 16-byte unit of codes (32 codes at 4
    # bits); 16 is shorter, so it is rejected on the host as well.
    st = qmm.lib.qmm_gemm_compint8(FAKE, 2, FAKE, 1, None, 2, None, None, 0, None, FAKE, 1, 4096, 4096, 16,
                                   4, 4, FAKE, 1 << 30, None)
    assert st == -2 and "M = 1" in qmm.qmm_last_error()


def test_benchmark_probe_library_exports_its_read_kernel():
    """bench.py's reference read (bench_probe/libqmm_probe.so, not part of
    libqmm.so and not built by the library's build) loads and rejects bad
    arguments on the host."""
    path = os.path.join(ROOT, "bench_probe", "libqmm_probe.so")
    lib = ctypes.CDLL(path)
    fn = lib.qmm_probe_stream_read
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p]
    big = 1 << 20
    assert fn(None, 16, None, 256, 1, 256, 4, 1, 0, None) != 0        # null pointers
    assert fn(big, 15, big, 256, 1, 256, 4, 1, 0, None) != 0          # not whole 16-byte words
    assert fn(big, 16, big, 256, 0, 256, 4, 1, 0, None) != 0          # empty grid
    assert fn(big, 16, big, 256, 2, 256, 4, 1, 0, None) != 0          # out too small for the grid
    assert fn(big, 16, big, 4096, 1, 96, 4, 1, 0, None) != 0          # block not whole waves
    assert fn(big, 16, big, 4096, 1, 256, 3, 1, 0, None) != 0         # unroll not offered
    assert "qmm_probe_stream_read" not in open(
        os.path.join(ROOT, "include", "qmm.h")).read()   # not part of the matmul ABI
    import block_quantized_weight_matmulnbits_amd.build as libbuild
    assert "stream_read" not in open(libbuild.__file__).read()


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus 2 exits with status 2 and says so,
    before touching any device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_repacked_geometry_is_checked_by_the_binding(qmm):
    """A Repacked buffer remembers the (K, N, block_size, bits) it was
    repacked with; the binding rejects a call that passes other values
    before anything reaches the library."""
    import torch
    nbytes = qmm.qmm_repacked_bytes(4096, 1024, 32, 4, torch.bfloat16, True)
    r = qmm.Repacked(torch.empty(nbytes, dtype=torch.uint8), qmm.QMM_BF16, True, 4096, 1024, 32, 4)
    r.check(4096, 1024, 32, 4)
    for bad in [(4096, 2048, 32, 4), (4097, 1024, 32, 4), (4096, 1024, 64, 4),
                (4096, 1024, 32, 8)]:
        with pytest.raises(ValueError, match="geometry mismatch"):
            r.check(*bad)
    short = qmm.Repacked(torch.empty(nbytes - 256, dtype=torch.uint8), qmm.QMM_BF16, True, 4096,
                         1024, 32, 4)
    with pytest.raises(ValueError, match="holds"):
        short.check(4096, 1024, 32, 4)
    with pytest.raises(ValueError, match="geometry mismatch"):
        qmm.qmm_gemv(None, r, None, None, None, None, 4096, 2048, 32, 4)


def test_noalloc_compint8_rejects_on_the_host(qmm):
    """The CompInt8 entry point without a workspace refuses, before any
    device work, a problem whose workspace exceeds its fixed device array,
    and validates its other arguments like qmm_gemm_compint8."""
    lim = qmm.QMM_NOALLOC_SCRATCH_BYTES
    assert qmm.qmm_compint8_workspace_size(300, 16384, 128) > lim
    st = qmm.lib.qmm_gemm_compint8_noalloc(FAKE, 2, FAKE, 0, FAKE, 2, None, None, 0, None, FAKE, 300,
                                           16384, 64, 128, 4, 4, None)
    assert st == -3 and "row batches" in qmm.qmm_last_error()
    st = qmm.lib.qmm_gemm_compint8_noalloc(FAKE, 2, FAKE, 0, FAKE, 2, None, None, 0, None, FAKE, 4, 4096,
                                           64, 128, 5, 4, None)
    assert st == -1 and "bits must be 2, 3, 4 or 8" in qmm.qmm_last_error()
    st = qmm.lib.qmm_gemm_compint8_noalloc(FAKE, 2, FAKE, 0, FAKE, 2, None, None, 0, None, FAKE, 4, 4096,
                                           64, 128, 4, 0, None)
    assert st == -1 and "accuracy_level must be 4" in qmm.qmm_last_error()


def test_int16_activations_reject_on_the_host(qmm):
    """qmm_gemm_int16 and its block-dot export: operator layout, block_size
    <= 128 and a workspace of qmm_int16_workspace_size bytes, checked before
    any device work."""
    ws = qmm.qmm_int16_workspace_size(4, 4096, 64)
    kb = 4096 // 64
    assert ws == -(-4 * 4096 * 2 // 256) * 256 + -(-4 * kb * 4 // 256) * 256
    assert qmm.qmm_int16_workspace_size(-1, 4096, 64) == 0

    def call(bs=64, layout=0, scales=FAKE, w=FAKE, wbytes=1 << 30, bits=4):
        return qmm.lib.qmm_gemm_int16(FAKE, 2, FAKE, layout, scales, 2, None, None, FAKE, 4, 4096,
                                      64, bs, bits, w, wbytes, None)
    assert call(bs=256) == -2 and "block_size <= 128" in qmm.qmm_last_error()
    assert call(layout=1, scales=None) == -2 and "operator's layout" in qmm.qmm_last_error()
    assert call(w=None) == -3 and "qmm_int16_workspace_size" in qmm.qmm_last_error()
    assert call(wbytes=ws - 1) == -3
    assert call(w=FAKE + 16) == -3
    assert call(bits=5) == -1
    st = qmm.lib.qmm_debug_int16_block_dots(FAKE, 2, FAKE, None, 4, 4096, 64, 64, 4, None, FAKE,
                                            1 << 30, None)
    assert st == -1 and "dots must be non-null" in qmm.qmm_last_error()


def test_three_bit_weights_have_no_tiled_layout(qmm):
    assert qmm.lib.qmm_repack(FAKE, FAKE, 2, None, 4096, 64, 32, 3, FAKE, 1 << 30, None) == -2
    assert "no tiled layout" in qmm.qmm_last_error()


def test_check_g_idx_on_host_arrays(qmm):
    """qmm_check_g_idx: shape [K] or [kb * bs], every entry in 0..kb-1, the
    first bad entry named (matmul_nbits.rs execute / dequantize_weight)."""
    import numpy as np
    import torch
    K, bs = 100, 32                                 # kb = 4, padded 128
    qmm.qmm_check_g_idx(torch.zeros(K, dtype=torch.int32), K, bs)
    qmm.qmm_check_g_idx(torch.arange(128, dtype=torch.int32) // 32, K, bs)
    g = torch.zeros(K, dtype=torch.int32)
    g[37] = 4
    with pytest.raises(qmm.QmmError, match=r"g_idx\[37\]=4 is outside 0..4"):
        qmm.qmm_check_g_idx(g, K, bs)
    g[37] = -1
    with pytest.raises(qmm.QmmError, match=r"g_idx\[37\]=-1"):
        qmm.qmm_check_g_idx(g, K, bs)
    gp = torch.zeros(128, dtype=torch.int32)
    gp[127] = 7                                    # padding entries are checked too
    with pytest.raises(qmm.QmmError, match=r"g_idx\[127\]=7"):
        qmm.qmm_check_g_idx(gp, K, bs)
    with pytest.raises(qmm.QmmError, match="must have shape"):
        qmm.qmm_check_g_idx(torch.zeros(101, dtype=torch.int32), K, bs)
    # Agrees with the oracle's check on random indices.
    import oracle
    rng = np.random.default_rng(0)
    for t in range(20):
        a = rng.integers(-2, 6, K).astype(np.int32)
        try:
            oracle.check_g_idx(a, K, bs)
            ok = True
        except oracle.GroupIndexError:
            ok = False
        st = qmm.lib.qmm_check_g_idx(a.ctypes.data, K, K, bs)
        assert (st == 0) == ok


def test_step_object_host_checks(qmm):
    """qmm_step_*: create / record / destroy on the host; finalizing an empty
    step and launching an unfinalized one are rejected before any device
    work."""
    import ctypes as c
    h = c.c_void_p()
    assert qmm.lib.qmm_step_create(c.byref(h)) == 0 and h.value
    assert qmm.lib.qmm_step_size(h) == 0
    assert qmm.lib.qmm_step_finalize(h) == -1
    assert "no call was recorded" in qmm.qmm_last_error()
    assert qmm.lib.qmm_step_add_gemv(h, FAKE, 2, FAKE, 0, FAKE, 2, None, None, 0, None, FAKE,
                                     4096, 4096, 32, 4, 0) == 0
    assert qmm.lib.qmm_step_size(h) == 1
    assert qmm.lib.qmm_step_launch(h, None) == -1
    assert "not finalized" in qmm.qmm_last_error()
    qmm.lib.qmm_step_destroy(h)
    qmm.lib.qmm_step_destroy(None)
    assert qmm.lib.qmm_step_create(None) == -1
