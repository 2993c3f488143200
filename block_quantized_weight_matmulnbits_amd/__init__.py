"""Block-quantized-weight matmuls (MatMulNBits) for AMD Instinct MI355X.

The compute lives in ``libqmm.so`` (hand-written HIP kernels for gfx950
behind the C ABI of ``include/qmm.h``); :mod:`.qmm` is its ctypes binding and
:mod:`.workloads` generates seeded synthetic inputs.
"""
