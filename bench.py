#!/usr/bin/env python3
"""Benchmark of the block-quantized-weight matmul hot path on one MI355X.

A step is one M = 1 decode pass over a Llama-3-8B-shaped layer (4-bit
asymmetric, block 32, bf16 activations and scales).  The projections that
read the same activations are stored stacked along N, as one weight matrix
each, so a step is four ``qmm_gemv`` launches in dependency order: q|k|v
(K 4096, N 6144), o, gate|up (K 4096, N 28672), down.  ``value`` is the
step's algorithmic bytes (packed codes + scales + zero points + activations
+ outputs) divided by the measured time per step, in GB/s.  Weights rotate
through enough copies (> 512 MB) that each step streams them from HBM
instead of the 256 MB Infinity Cache.  The same layer as seven separate
launches is reported beside it (``unfused``).

The JSON line also carries the roofline of the dominant kernel (the GEMV on
the gate|up matrix, timed by HIP events around a run of its own
back-to-back launches on the same stream), the same for one 4096 x 14336
projection, the prefill GEMM, CompInt8 and conv figures, and the CPU oracle
timed on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5033.2       # MI355X dense fp8 MFMA
FP4_PEAK_TFLOPS = 10066.3      # MI355X dense fp4 / fp6 MFMA
POOL_BYTES = 640 << 20         # rotating weight pool, > 2x the Infinity Cache
COPY_CAL_BYTES = 256 << 20     # plain copy used to scale the HBM byte counters
PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
KERNEL_SOURCE = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                             "block_quantized_weight_matmulnbits_amd", "csrc", "gemv_tiled.hip")


def measured_traffic(name):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary profiles/<name>, or None when it is missing or the kernel source
    has changed since it was taken."""
    import hashlib
    try:
        fields = dict(line.split(":", 1) for line in open(os.path.join(PROFILES, name))
                      if ":" in line and not line.startswith("#"))
        src_hash = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
        if fields.get("kernel_source_sha256", "").strip() != src_hash:
            return None
        return int(float(fields["hbm_bytes_per_launch"].strip()))
    except (OSError, KeyError, ValueError):
        return None

METRIC = "int4 GEMV weight GB/s (% HBM peak) at M=1; GEMM TFLOPS (% MFMA) at M=2048"


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip timing the CPU oracle (profiling runs)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run a plain 256 MiB device copy (the reference kernel for "
                        "scaling the FETCH_SIZE / WRITE_SIZE counters of profiling runs)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target wall time of the CPU-oracle sample")
    p.add_argument("--only", choices=["compint8", "prefill", "conv", "tiny", "fp4", "lowbit", "batched",
                                      "lowp", "gidx"],
                   default=None,
                   help="time only this workload and print its object (profiling runs)")
    p.add_argument("--read-sweep", action="store_true",
                   help="only sweep the plain streaming read (bench_probe/) over launch shapes "
                        "and sizes and print a markdown table")
    return p.parse_args()


def layer_bytes(case) -> int:
    """Algorithmic bytes of one GEMV: codes + scales + zero points + x + y."""
    return case.weight_bytes() + case.A.numel() * case.A.element_size() \
        + case.N * case.A.element_size()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the decode GEMV shards by output column with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)
    from block_quantized_weight_matmulnbits_amd import qmm
    from block_quantized_weight_matmulnbits_amd.workloads import decode_layer, decode_layer_fused

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.read_sweep:
        read_sweep(dev, torch.cuda.current_stream(dev))
        return
    if args.only:
        from block_quantized_weight_matmulnbits_amd import qmm
        stream = torch.cuda.current_stream(dev)
        if args.copy_calibration:
            src = torch.ones(COPY_CAL_BYTES, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
        fn = {"compint8": bench_compint8, "prefill": bench_prefill, "conv": bench_conv,
              "tiny": bench_tiny, "fp4": bench_fp4, "lowbit": bench_lowbit,
              "batched": bench_batched, "lowp": bench_lowp, "gidx": bench_gidx}[args.only]
        print(json.dumps({args.only: fn(qmm, dev, stream, args)}), flush=True)
        return
    if args.copy_calibration:
        src = torch.ones(COPY_CAL_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cases = decode_layer()                 # the seven projections
    fcases = decode_layer_fused()          # q|k|v and gate|up stacked: four launches
    step_bytes = sum(layer_bytes(c) for c in cases)
    fstep_bytes = sum(layer_bytes(c) for c in fcases)
    n_copies = max(2, -(-POOL_BYTES // step_bytes))

    def pool_of(clist):
        """Per case: n_copies (B, scales, zero points) on the device. Copy 0 is
        the seeded weights; the others are byte-identical copies at other
        addresses (only the addresses matter for cache behaviour)."""
        pools = []
        for c in clist:
            d = c.to(dev)
            pools.append([(d.B, d.scales, d.zero_points)] +
                         [(d.B.clone(), d.scales.clone(), d.zero_points.clone())
                          for _ in range(n_copies - 1)])
        return pools

    def repacked(clist, pools):
        """The same weights repacked once into the tiled layout (qmm_repack), as
        an inference session does when it loads constant weights; not timed."""
        return [[(qmm.qmm_repack(B, sc, zp, c.K, c.N, c.block_size, c.bits), None, None)
                 for (B, sc, zp) in pool] for c, pool in zip(clist, pools)]

    pools = pool_of(cases)
    tiled = repacked(cases, pools)
    fpools = pool_of(fcases)
    ftiled = repacked(fcases, fpools)
    del fpools
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()

    def series(clist, weights):
        xs = [c.to(dev).A.reshape(-1) for c in clist]
        ys = [torch.empty(c.N, dtype=torch.bfloat16, device=dev) for c in clist]

        def launch(i, j):
            c = clist[i]
            B, sc, zp = weights[i][j]
            qmm.qmm_gemv(xs[i], B, sc, zp, None, ys[i], c.K, c.N, c.block_size, c.bits, 0,
                         stream)
        return launch

    def time_steps(clist, weights):
        """ms per layer step: every launch of clist in order, weight copy s."""
        launch = series(clist, weights)

        def step(s):
            for i in range(len(clist)):
                launch(i, s % n_copies)

        for s in range(args.warmup):
            step(s)
        torch.cuda.synchronize()
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        _queue_ahead(len(clist) * args.steps)
        t_start.record(stream)
        for s in range(args.steps):
            step(s)
        t_end.record(stream)
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_end) / args.steps

    def time_steps_host(clist, weights):
        """ms per layer step as a host issues it: the launches of each step
        in order, no device-side spin ahead of them, so the host's work per
        call counts wherever it is longer than the kernels."""
        launch = series(clist, weights)

        def step(s):
            for i in range(len(clist)):
                launch(i, s % n_copies)

        for s in range(args.warmup):
            step(s)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for s in range(args.steps):
            step(s)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps

    def time_graph_steps(clist, weights):
        """The same step recorded once per weight copy (qmm_step: its launches
        captured into one HIP graph) and replayed: (host-issued ms, device-only
        ms) per step."""
        xs = [c.to(dev).A.reshape(-1) for c in clist]
        ys = [torch.empty(c.N, dtype=torch.bfloat16, device=dev) for c in clist]
        steps = []
        for j in range(n_copies):
            st = qmm.Step()
            for i, c in enumerate(clist):
                B, sc, zp = weights[i][j]
                st.add_gemv(xs[i], B, sc, zp, None, ys[i], c.K, c.N, c.block_size, c.bits)
            steps.append(st.finalize())
        for s in range(args.warmup):
            steps[s % n_copies].launch(stream)
        torch.cuda.synchronize()
        res = []
        for spin in (False, True):
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            if spin:
                _queue_ahead(args.steps)
            t0.record(stream)
            for s in range(args.steps):
                steps[s % n_copies].launch(stream)
            t1.record(stream)
            torch.cuda.synchronize()
            res.append(t0.elapsed_time(t1) / args.steps)
        for st in steps:
            st.close()
        return res[0], res[1]

    def time_kernel(clist, weights, idx):
        """ms per launch of the GEMVs clist[i], i in idx, launched back to back
        (rotating weight copies) between one pair of HIP events on the launch
        stream; per-launch events would add their own overhead."""
        launch = series(clist, weights)
        n = max(20, args.steps)
        for s in range(n):
            launch(idx[s % len(idx)], s % n_copies)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        _queue_ahead(n)
        e0.record(stream)
        for s in range(n):
            launch(idx[s % len(idx)], s % n_copies)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms_f = time_steps(fcases, ftiled)
    ms_f_host = time_steps_host(fcases, ftiled)
    ms_g_host, ms_g_dev = time_graph_steps(fcases, ftiled)
    ms_t = time_steps(cases, tiled)
    ms_o = time_steps(cases, pools)
    # Dominant kernel of the step: the gate|up launch (K = 4096, N = 28672).
    fdom = [i for i, c in enumerate(fcases) if c.meta["name"] == "gate_up"]
    fdom_bytes = layer_bytes(fcases[fdom[0]])
    fdom_ms = time_kernel(fcases, ftiled, fdom)
    # The single 4096 x 14336 projection (gate or up alone).
    dom = [i for i, c in enumerate(cases) if (c.K, c.N) == (4096, 14336)]
    dom_bytes = layer_bytes(cases[dom[0]])
    dom_t = time_kernel(cases, tiled, dom)
    dom_o = time_kernel(cases, pools, dom)
    value = fstep_bytes / (ms_f * 1e-3) / 1e9
    achieved = fdom_bytes / (fdom_ms * 1e-3) / 1e9
    achieved_1 = dom_bytes / (dom_t * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_f, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 activations x int4 weights, fp32 accumulate",
        "data": "synthetic",
        "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "config": {
            "workload": "decode GEMV, one Llama-3-8B-shaped layer (q,k,v,o,gate,up,down), M=1, "
                        "bf16 activations, 4-bit asymmetric block 32, bf16 scales, packed zero points",
            "projections": "q|k|v stacked along N (K=4096, N=6144), o, gate|up stacked "
                           "(K=4096, N=28672), down: four launches per step",
            "weight_layout": "tiled (qmm_repack once at load, not timed)",
            "M": 1,
            "shapes_KxN": [[c.K, c.N] for c in fcases],
            "bytes_per_step": fstep_bytes,
            "weight_copies_rotated": n_copies,
        },
        "roofline": {
            "kernel": "gemv_tiled_kernel (4-bit, bf16, zero points) on K=4096 N=28672 (gate|up)",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("gemv_tiled_K4096_N28672_traffic.txt"),
            "avg_launch_us": round(fdom_ms * 1e3, 3),
            "bytes_per_launch": fdom_bytes,
        },
        "step_launch": {
            "what": "the same four-launch step: device-only (launches queued behind a "
                    "device-side spin) and as a host issues it (no spin: the binding's work "
                    "per call counts where it is longer than the kernels), with direct "
                    "qmm_gemv calls and with the calls recorded once as one HIP graph "
                    "(qmm_step) and replayed",
            "direct_device_ms": round(ms_f, 5),
            "direct_host_issued_ms": round(ms_f_host, 5),
            "graph_device_ms": round(ms_g_dev, 5),
            "graph_host_issued_ms": round(ms_g_host, 5),
            "graph_host_issued_GBps": round(fstep_bytes / (ms_g_host * 1e-3) / 1e9, 2),
        },
        "unfused": {
            "what": "the seven projections as seven launches, tiled layout",
            "value": round(step_bytes / (ms_t * 1e-3) / 1e9, 2),
            "ms_per_step": round(ms_t, 5),
            "bytes_per_step": step_bytes,
        },
        "roofline_K4096_N14336": {
            "kernel": "gemv_tiled_kernel on K=4096 N=14336 (gate or up alone)",
            "achieved": round(achieved_1, 2),
            "frac": round(achieved_1 / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("gemv_tiled_K4096_N14336_traffic.txt"),
            "avg_launch_us": round(dom_t * 1e3, 3),
            "bytes_per_launch": dom_bytes,
        },
        "operator_layout": {
            "kernel": "gemv_kernel on the operator's [N, kb, blob] layout, seven launches",
            "value": round(step_bytes / (ms_o * 1e-3) / 1e9, 2),
            "ms_per_step": round(ms_o, 5),
            "dominant_avg_launch_us": round(dom_o * 1e3, 3),
            "dominant_GBps": round(dom_bytes / (dom_o * 1e-3) / 1e9, 2),
        },
    }

    out["roofline"]["read_ceiling"] = read_ceiling(dev, stream, fdom_bytes, fdom_ms)
    out["tiny"] = bench_tiny(qmm, dev, stream, args)
    out["prefill_gemm"] = bench_prefill(qmm, dev, stream, args)
    out["compint8"] = bench_compint8(qmm, dev, stream, args)
    out["conv_int8"] = bench_conv(qmm, dev, stream, args)
    out["fp4"] = bench_fp4(qmm, dev, stream, args)
    out["lowbit"] = bench_lowbit(qmm, dev, stream, args)
    out["lowp"] = bench_lowp(qmm, dev, stream, args)
    out["gidx"] = bench_gidx(qmm, dev, stream, args)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cases, args.cpu_seconds)
        out["cpu_baseline_configs"] = cpu_baseline_configs(args.cpu_seconds / 4)

    print(json.dumps(out), flush=True)


_SLEEP_CYCLES_PER_MS = None


def _queue_ahead(n_launches):
    """Hold the current stream with a device-side spin long enough for the
    host to queue n_launches calls (10 us each, about twice what the Python
    binding takes per call), so that the HIP events which follow time the
    device executing the launches back to back rather than the host issuing
    them: the smallest projections run for about as long as one Python
    call takes."""
    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(1_000_000)
        e1.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = 1_000_000 / max(e0.elapsed_time(e1), 1e-3)
    torch.cuda._sleep(int(_SLEEP_CYCLES_PER_MS * max(1.0, 0.01 * n_launches)))


def _time_launches(fn, n, stream):
    """Average ms per launch of fn(i), i = 0..n-1, after one untimed pass of
    the same n launches (so clocks have ramped up and every buffer of a
    rotating pool has been touched before the timed region)."""
    for i in range(n):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    _queue_ahead(n)
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


READ_SWEEP = [(grid, block, unroll, nt, slab)
              for grid in (256, 512, 1024, 2048)
              for block in (256, 512, 1024)
              for unroll in (2, 4, 8, 16)
              for nt in (1, 0)
              for slab in (1, 0)]


class ReadProbe:
    """The plain streaming read of bench_probe/ (its own library): times one
    launch reading n bytes over rotating buffers (> 2x the Infinity Cache),
    as the matmul kernels' launches are timed."""

    def __init__(self, dev, stream):
        import ctypes
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bench_probe",
                            "libqmm_probe.so")
        if not os.path.exists(path):
            raise FileNotFoundError(path)
        self.lib = ctypes.CDLL(path)
        c = ctypes
        self.lib.qmm_probe_stream_read.argtypes = [c.c_void_p, c.c_int64, c.c_void_p, c.c_int64,
                                                   c.c_int, c.c_int, c.c_int, c.c_int, c.c_int,
                                                   c.c_void_p]
        self.dev, self.stream = dev, stream
        self.out = torch.empty(2048 * 1024, dtype=torch.int32, device=dev)
        self.nb = None

    def _buffers(self, nbytes):
        if self.nb != nbytes:
            self.bufs = None
            copies = max(2, -(-POOL_BYTES // nbytes))
            self.bufs = [torch.full((nbytes,), i, dtype=torch.uint8, device=self.dev)
                         for i in range(copies)]
            self.nb = nbytes
        return self.bufs

    def ms(self, nbytes, cfg, launches=100):
        import ctypes
        nbytes = nbytes // 16 * 16
        bufs = self._buffers(nbytes)
        grid, block, unroll, nt, slab = cfg

        def run(i):
            rc = self.lib.qmm_probe_stream_read(bufs[i % len(bufs)].data_ptr(), nbytes,
                                                self.out.data_ptr(), self.out.numel(), grid,
                                                block, unroll, nt, slab,
                                                ctypes.c_void_p(self.stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"stream read probe failed: {rc}")

        return _time_launches(run, launches, self.stream)

    def release(self):
        self.bufs, self.nb = None, None


def _cfg_name(cfg):
    grid, block, unroll, nt, slab = cfg
    return (f"{grid} x {block} threads, {unroll} 16-byte loads in flight per lane, "
            f"{'non-temporal' if nt else 'plain'} loads, "
            f"{'one contiguous slab per workgroup' if slab else 'grid-stride'}")


def read_ceiling(dev, stream, nbytes, kernel_ms):
    """The fastest plain streaming read of nbytes over READ_SWEEP (grid,
    workgroup size, loads in flight per lane, non-temporal or plain loads,
    grid-stride or slab order): what one launch needs just to read that many
    bytes here.  None if the probe library was not built."""
    try:
        probe = ReadProbe(dev, stream)
    except FileNotFoundError:
        return None
    best = None
    for cfg in READ_SWEEP:
        ms = probe.ms(nbytes, cfg, launches=50)
        if best is None or ms < best[0]:
            best = (ms, cfg)
    # Re-time the winner with as many launches as the kernel's own series.
    ms = probe.ms(nbytes, best[1], launches=100)
    probe.release()
    nb = nbytes // 16 * 16
    gbps = nb / (ms * 1e-3) / 1e9
    return {"what": "fastest plain streaming read of the same bytes over "
                    f"{len(READ_SWEEP)} launch shapes: {_cfg_name(best[1])}; one launch per "
                    "buffer, rotating buffers",
            "bytes": nb, "us": round(ms * 1e3, 3), "GBps": round(gbps, 2),
            "frac_of_peak": round(gbps / HBM_PEAK_GBS, 4),
            "kernel_frac_of_read": round(ms / kernel_ms, 4)}


def read_sweep(dev, stream):
    """--read-sweep: every READ_SWEEP shape at several read sizes; prints a
    markdown table (the summary kept under profiles/)."""
    probe = ReadProbe(dev, stream)
    sizes = [(29360128, "codes of one 4096x14336 4-bit projection"),
             (67960832, "gate|up GEMV bytes"),
             (126255104, "decode layer bytes"),
             (536870912, "512 MiB")]
    print("| bytes | what | best us | best GB/s | frac of 8 TB/s | best shape | "
          "best non-temporal | best plain | best stride | best slab |", flush=True)
    print("|---|---|---|---|---|---|---|---|---|---|", flush=True)
    for nb, what in sizes:
        res = []
        for cfg in READ_SWEEP:
            res.append((probe.ms(nb, cfg, launches=50 if nb < (256 << 20) else 10), cfg))
        gb = lambda ms: nb / (ms * 1e-3) / 1e9
        best = min(res)
        sub = lambda f: min(r for r in res if f(r[1]))
        print(f"| {nb} | {what} | {best[0] * 1e3:.2f} | {gb(best[0]):.0f} | "
              f"{gb(best[0]) / HBM_PEAK_GBS:.3f} | {_cfg_name(best[1])} | "
              f"{gb(sub(lambda c: c[3] == 1)[0]):.0f} | {gb(sub(lambda c: c[3] == 0)[0]):.0f} | "
              f"{gb(sub(lambda c: c[4] == 0)[0]):.0f} | {gb(sub(lambda c: c[4] == 1)[0]):.0f} |",
              flush=True)
        # Per loads-in-flight and per grid: the best over the other knobs.
        for key, idx in (("loads in flight per lane", 2), ("workgroups", 0),
                         ("threads per workgroup", 1)):
            vals = sorted({c[idx] for _, c in res})
            cells = ", ".join(f"{v}: {gb(min(r for r in res if r[1][idx] == v)[0]):.0f}"
                              for v in vals)
            print(f"|  | best GB/s by {key} | {cells} | | | | | | | |", flush=True)
    probe.release()


def bench_tiny(qmm, dev, stream, args):
    """The tiny configuration (M=1, K=N=256, f32, 4-bit symmetric block 32):
    a latency case (43,008 bytes, 5 ns at HBM peak).  Per launch: device-only
    (launches queued behind a spin) and host-issued (one launch after another,
    each waited for: what a caller sees for one call)."""
    from block_quantized_weight_matmulnbits_amd.workloads import tiny_matmulnbits
    c = tiny_matmulnbits().to(dev)
    y = torch.empty(c.N, dtype=torch.float32, device=dev)
    x = c.A.reshape(-1)

    def run(_):
        qmm.qmm_gemv(x, c.B, c.scales, None, None, y, c.K, c.N, c.block_size, c.bits, 0, stream)

    dev_ms = _time_launches(run, max(100, args.steps), stream)
    # One call at a time, synchronized: the latency of a lone call.
    n = 200
    t0 = time.perf_counter()
    for i in range(n):
        run(i)
        torch.cuda.synchronize()
    lone_us = (time.perf_counter() - t0) / n * 1e6
    nbytes = c.weight_bytes() + c.K * 4 + c.N * 4
    return {"workload": "tiny MatMulNBits M=1 K=256 N=256, f32 activations, 4-bit symmetric "
                        "block 32, f32 scales, f32 output (operator layout)",
            "bytes_per_launch": nbytes,
            "device_us_per_launch": round(dev_ms * 1e3, 3),
            "host_call_and_sync_us": round(lone_us, 2)}


def bench_prefill(qmm, dev, stream, args):
    """Prefill GEMM M=2048, K=4096, N=14336 (4-bit asymmetric bs 32, bf16), on
    the operator's layout and on the tiled layout (weights repacked once,
    before the timed region, as an inference session does at load time)."""
    from block_quantized_weight_matmulnbits_amd.workloads import prefill_gemm
    c = prefill_gemm().to(dev)
    Y = torch.empty(c.M, c.N, dtype=torch.bfloat16, device=dev)
    t = qmm.qmm_repack(c.B, c.scales, c.zero_points, c.K, c.N, c.block_size, c.bits,
                       stream=stream)
    flop = 2.0 * c.M * c.N * c.K
    res = {"workload": "prefill GEMM M=2048 K=4096 N=14336, bf16 activations, 4-bit asymmetric "
                       "block 32, bf16 output, fp32 accumulate",
           "bound": "mfma", "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "flop_per_launch": flop}
    for name, B, S, Z in (("tiled", t, None, None), ("operator_layout", c.B, c.scales,
                                                    c.zero_points)):
        def run(_):
            qmm.qmm_gemm(c.A, B, S, Z, None, Y, c.M, c.K, c.N, c.block_size, c.bits, 0, stream)

        for i in range(3):
            run(i)
        torch.cuda.synchronize()
        ms = _time_launches(run, max(20, args.steps // 5), stream)
        tflops = flop / (ms * 1e-3) / 1e12
        res[name] = {"ms": round(ms, 4), "tflops": round(tflops, 2),
                     "frac": round(tflops / BF16_PEAK_TFLOPS, 4)}
    return res


def bench_compint8(qmm, dev, stream, args):
    """Batched-decode CompInt8, K=4096 N=14336, M in {1,4,16} x 3 weight formats,
    on the tiled layout (int8 matrix cores; weights repacked once, not timed)
    and on the operator's layout; weights rotate through copies so each
    launch streams them from HBM.  Times include the activation quantization."""
    from block_quantized_weight_matmulnbits_amd.workloads import COMPINT8_VARIANTS, compint8_case
    res = {}
    for bits, bs, asym in COMPINT8_VARIANTS:
        base = compint8_case(1, bits, bs, asym).to(dev)
        nbytes = base.weight_bytes()
        n_copies = max(2, -(-POOL_BYTES // nbytes))
        copies = [(base.B, base.scales, base.zero_points)] + [
            (base.B.clone(), base.scales.clone(),
             None if base.zero_points is None else base.zero_points.clone())
            for _ in range(n_copies - 1)]
        tiled = [(qmm.qmm_repack(B, sc, zp, base.K, base.N, bs, bits), None, None)
                 for (B, sc, zp) in copies]
        for M in (1, 4, 16):
            c = compint8_case(M, bits, bs, asym)
            A = c.A.to(dev)
            Y = torch.empty(M, c.N, dtype=torch.bfloat16, device=dev)
            ws = torch.empty(qmm.qmm_compint8_workspace_size(M, c.K, bs), dtype=torch.uint8,
                             device=dev)
            byts = nbytes + A.numel() * 2 + M * c.N * 2
            entry = {}
            for name, pool in (("tiled", tiled), ("operator_layout", copies)):
                def run(i, pool=pool):
                    B, sc, zp = pool[i % len(pool)]
                    qmm.qmm_gemm_compint8(A, B, sc, zp, None, Y, M, c.K, c.N, bs, bits, ws, 4,
                                          stream)

                for i in range(3):
                    run(i)
                torch.cuda.synchronize()
                ms = _time_launches(run, max(10, args.steps // 4), stream)
                entry[name] = {"us": round(ms * 1e3, 2),
                               "GBps": round(byts / (ms * 1e-3) / 1e9, 1),
                               "frac_hbm": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            res[f"b{bits}_bs{bs}_M{M}"] = entry
    return res


def bench_fp4(qmm, dev, stream, args):
    """Block-scaled FP4 weights (MXFP4 / NVFP4), bf16 activations: the decode
    GEMV and batched decode at M = 16 on a 4096 x 14336 projection (weights
    rotating through copies, so they stream from HBM) and the prefill GEMM
    M=2048 K=4096 N=14336."""
    from block_quantized_weight_matmulnbits_amd.workloads import make_fp4_case
    res = {}
    for fmt in ("mxfp4", "nvfp4"):
        c = make_fp4_case(1, 4096, 14336, fmt, a_dtype="bf16", seed=41).to(dev)
        nbytes = c.weight_bytes() + c.K * 2 + c.N * 2
        copies = max(2, -(-POOL_BYTES // nbytes))
        pool = [(c.W, c.scales)] + [(c.W.clone(), c.scales.clone()) for _ in range(copies - 1)]
        y = torch.empty(1, c.N, dtype=torch.bfloat16, device=dev)

        def run(i, c=c, pool=pool, y=y):
            W, S = pool[i % len(pool)]
            qmm.qmm_gemm_fp4(c.A, W, S, c.fmt, c.global_scale, None, y, 1, c.K, c.N, stream)

        ms = _time_launches(run, max(20, args.steps), stream)
        a16 = make_fp4_case(16, 4096, 14336, fmt, a_dtype="bf16", seed=43).A.to(dev)
        y16 = torch.empty(16, c.N, dtype=torch.bfloat16, device=dev)

        def run16(i, c=c, pool=pool, a16=a16, y16=y16):
            W, S = pool[i % len(pool)]
            qmm.qmm_gemm_fp4(a16, W, S, c.fmt, c.global_scale, None, y16, 16, c.K, c.N, stream)

        for i in range(3):
            run16(i)
        torch.cuda.synchronize()
        ms16 = _time_launches(run16, max(20, args.steps // 4), stream)
        b16 = nbytes + 15 * c.K * 2 + 15 * c.N * 2
        del pool
        p = make_fp4_case(2048, 4096, 14336, fmt, a_dtype="bf16", seed=42).to(dev)
        Y = torch.empty(p.M, p.N, dtype=torch.bfloat16, device=dev)

        def runp(_, p=p, Y=Y):
            qmm.qmm_gemm_fp4(p.A, p.W, p.scales, p.fmt, p.global_scale, None, Y, p.M, p.K, p.N,
                             stream)

        for i in range(3):
            runp(i)
        torch.cuda.synchronize()
        msp = _time_launches(runp, max(20, args.steps // 5), stream)
        flop = 2.0 * p.M * p.N * p.K
        res[fmt] = {
            "gemv_K4096_N14336": {"us": round(ms * 1e3, 3), "bytes": nbytes,
                                  "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                  "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "batched_M16_K4096_N14336": {"us": round(ms16 * 1e3, 3), "bytes": b16,
                                         "GBps": round(b16 / (ms16 * 1e-3) / 1e9, 1),
                                         "frac_hbm": round(b16 / (ms16 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "prefill_M2048_K4096_N14336": {"ms": round(msp, 4),
                                           "tflops": round(flop / (msp * 1e-3) / 1e12, 2),
                                           "frac_bf16_peak": round(
                                               flop / (msp * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
        }
        del p, Y
    return res


def bench_lowp(qmm, dev, stream, args):
    """Low-precision scaled GEMM (qmm_lowp_matmul) on the prefill shape
    m=2048, k=4096, n=14336: operands produced by qmm_lowp_quantize from
    seeded normal activations and weights (the weights once, before timing;
    the activations' quantization timed on its own).  Peaks: FP4 x FP4 the
    dense FP4 matrix-core rate, a pair with an FP8 operand the FP8 rate, and
    NVFP4 scales (decoded into the bf16 matrix cores) the bf16 rate."""
    m, k, n = 2048, 4096, 14336
    g = torch.Generator(device=dev)
    g.manual_seed(61)
    x = torch.randn(m, k, generator=g, device=dev).to(torch.bfloat16)
    w = torch.randn(n, k, generator=g, device=dev).to(torch.bfloat16)
    flop = 2.0 * m * n * k
    res = {"workload": "scaled GEMM m=2048 k=4096 n=14336, codes quantized from seeded normal "
                       "bf16 activations and weights, f32 output"}

    def quantized(t, fmt, layout):
        rows, cols = t.shape
        codes = torch.empty(rows, cols, dtype=torch.uint8, device=dev)
        if layout == "tensor":
            sc = torch.empty(1, dtype=torch.float32, device=dev)
        else:
            sc = torch.empty(rows, cols // (32 if layout == "mx" else 16), dtype=torch.uint8,
                             device=dev)
        qmm.qmm_lowp_quantize(t, codes, sc, rows, cols, fmt, layout, stream)
        return codes, sc

    out = torch.empty(m, n, dtype=torch.float32, device=dev)
    for name, lf, rf, layout, peak in (("mxfp4_x_mxfp4", "e2m1", "e2m1", "mx", FP4_PEAK_TFLOPS),
                                       ("mx_e4m3_x_e2m1", "e4m3", "e2m1", "mx", FP8_PEAK_TFLOPS),
                                       ("mx_e4m3_x_e4m3", "e4m3", "e4m3", "mx", FP8_PEAK_TFLOPS),
                                       ("tensor_e4m3_x_e4m3", "e4m3", "e4m3", "tensor",
                                        FP8_PEAK_TFLOPS),
                                       ("nvfp4_x_nvfp4", "e2m1", "e2m1", "nvfp4",
                                        BF16_PEAK_TFLOPS)):
        lc, ls = quantized(x, lf, layout)
        rc, rs = quantized(w, rf, layout)

        def run(_, lc=lc, ls=ls, rc=rc, rs=rs, lf=lf, rf=rf, layout=layout):
            qmm.qmm_lowp_matmul(lc, rc, ls, rs, None, out, m, n, k, layout, lf, rf, stream)

        for i in range(2):
            run(i)
        torch.cuda.synchronize()
        ms = _time_launches(run, max(10, args.steps // 10), stream)
        tflops = flop / (ms * 1e-3) / 1e12
        res[name] = {"ms": round(ms, 4), "tflops": round(tflops, 2), "peak": peak,
                     "frac": round(tflops / peak, 4)}
        del lc, ls, rc, rs
    codes = torch.empty(m, k, dtype=torch.uint8, device=dev)
    sc = torch.empty(m, k // 32, dtype=torch.uint8, device=dev)

    def runq(_):
        qmm.qmm_lowp_quantize(x, codes, sc, m, k, "e2m1", "mx", stream)

    for i in range(2):
        runq(i)
    torch.cuda.synchronize()
    msq = _time_launches(runq, max(20, args.steps // 5), stream)
    qbytes = m * k * 2 + m * k + m * (k // 32)
    res["quantize_activations_mx_e2m1"] = {
        "us": round(msq * 1e3, 3), "bytes": qbytes, "GBps": round(qbytes / (msq * 1e-3) / 1e9, 1),
        "frac_hbm": round(qbytes / (msq * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return res


def bench_lowbit(qmm, dev, stream, args):
    """3-bit weights (bs 32, asymmetric, bf16 scales) and 8-bit weights with
    int16 activations (bs 32, asymmetric) on the decode-shaped projection
    K=4096 N=14336, operator layout, bf16 activations: the float GEMV / GEMM
    (3-bit) at M in {1, 16}, CompInt8 (3-bit) and the int16 route (8-bit) at
    M in {1, 4, 16}.  Weights rotate through copies so each launch streams them
    from HBM; times include the activation quantization.  Plus the 3-bit
    prefill M=2048 on the matrix cores (TFLOP/s)."""
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    res = {}
    for bits, route in ((3, "float"), (3, "compint8"), (8, "int16")):
        base = make_matmul_case(1, 4096, 14336, 32, bits, a_dtype="bf16", has_zp=True,
                                seed=50 + bits).to(dev)
        nbytes = base.weight_bytes()
        n_copies = max(2, -(-POOL_BYTES // nbytes))
        pool = [(base.B, base.scales, base.zero_points)] + [
            (base.B.clone(), base.scales.clone(), base.zero_points.clone())
            for _ in range(n_copies - 1)]
        for M in ((1, 16) if route == "float" else (1, 4, 16)):
            c = make_matmul_case(M, 4096, 14336, 32, bits, a_dtype="bf16", has_zp=True,
                                 seed=60 + M)
            A = c.A.to(dev)
            Y = torch.empty(M, c.N, dtype=torch.bfloat16, device=dev)
            if route == "compint8":
                ws = torch.empty(qmm.qmm_compint8_workspace_size(M, c.K, 32), dtype=torch.uint8,
                                 device=dev)
            elif route == "int16":
                ws = torch.empty(qmm.qmm_int16_workspace_size(M, c.K, 32), dtype=torch.uint8,
                                 device=dev)

            def run(i, route=route, A=A, Y=Y, M=M, c=c, bits=bits):
                B, sc, zp = pool[i % len(pool)]
                if route == "float" and M == 1:
                    qmm.qmm_gemv(A.reshape(-1), B, sc, zp, None, Y.reshape(-1), c.K, c.N, 32,
                                 bits, stream=stream)
                elif route == "float":
                    qmm.qmm_gemm(A, B, sc, zp, None, Y, M, c.K, c.N, 32, bits, stream=stream)
                elif route == "compint8":
                    qmm.qmm_gemm_compint8(A, B, sc, zp, None, Y, M, c.K, c.N, 32, bits, ws, 4,
                                          stream)
                else:
                    qmm.qmm_gemm_int16(A, B, sc, zp, None, Y, M, c.K, c.N, 32, bits, ws, stream)

            for i in range(3):
                run(i)
            torch.cuda.synchronize()
            ms = _time_launches(run, max(10, args.steps // 4), stream)
            byts = nbytes + A.numel() * 2 + M * c.N * 2
            res[f"b{bits}_{route}_M{M}"] = {
                "us": round(ms * 1e3, 2), "bytes": byts,
                "GBps": round(byts / (ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del pool
    # 3-bit prefill on the matrix cores (operator layout).
    c = make_matmul_case(2048, 4096, 14336, 32, 3, a_dtype="bf16", has_zp=True, seed=63).to(dev)
    Y = torch.empty(c.M, c.N, dtype=torch.bfloat16, device=dev)

    def runp(_):
        qmm.qmm_gemm(c.A, c.B, c.scales, c.zero_points, None, Y, c.M, c.K, c.N, 32, 3, 0, stream)

    for i in range(3):
        runp(i)
    torch.cuda.synchronize()
    ms = _time_launches(runp, max(20, args.steps // 5), stream)
    flop = 2.0 * c.M * c.N * c.K
    res["b3_prefill_M2048"] = {"ms": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
                               "frac_bf16_peak": round(flop / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    return res


def bench_gidx(qmm, dev, stream, args):
    """Group indices (act-order g_idx) on the decode-shaped projection K=4096
    N=14336, 4-bit asymmetric bs 32, bf16 scales and activations, operator
    layout: g_idx[k] = rank(k) // 32 for a seeded random order of K (every
    group has 32 members).  M = 1 (qmm_gemv), 2 and 16 (qmm_gemm; the tabled
    GEMV and the tabled MFMA kernel) with weights rotating through copies so
    each launch streams them from HBM (bytes include the index array), and
    the prefill M = 2048 (TFLOP/s)."""
    import numpy as np
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    K, N, bs = 4096, 14336, 32
    rng = np.random.default_rng(71)
    order = rng.permutation(K)
    rank = np.empty(K, np.int64)
    rank[order] = np.arange(K)
    gi = torch.from_numpy((rank // bs).astype(np.int32)).to(dev)
    base = make_matmul_case(1, K, N, bs, 4, a_dtype="bf16", has_zp=True, seed=72).to(dev)
    nbytes = base.weight_bytes() + K * 4
    n_copies = max(2, -(-POOL_BYTES // nbytes))
    pool = [(base.B, base.scales, base.zero_points)] + [
        (base.B.clone(), base.scales.clone(), base.zero_points.clone())
        for _ in range(n_copies - 1)]
    res = {"workload": "K=4096 N=14336, 4-bit asymmetric bs 32, bf16, act-order g_idx"}
    for M in (1, 2, 16):
        c = make_matmul_case(M, K, N, bs, 4, a_dtype="bf16", has_zp=True, seed=73 + M)
        A = c.A.to(dev)
        Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)

        def run(i, A=A, Y=Y, M=M):
            B, sc, zp = pool[i % len(pool)]
            if M == 1:
                qmm.qmm_gemv(A.reshape(-1), B, sc, zp, None, Y.reshape(-1), K, N, bs, 4,
                             stream=stream, g_idx=gi)
            else:
                qmm.qmm_gemm(A, B, sc, zp, None, Y, M, K, N, bs, 4, stream=stream, g_idx=gi)

        for i in range(3):
            run(i)
        torch.cuda.synchronize()
        ms = _time_launches(run, max(10, args.steps // 4), stream)
        byts = nbytes + A.numel() * 2 + M * N * 2
        res[f"M{M}"] = {"us": round(ms * 1e3, 2), "bytes": byts,
                        "GBps": round(byts / (ms * 1e-3) / 1e9, 1),
                        "frac_hbm": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del pool
    c = make_matmul_case(2048, K, N, bs, 4, a_dtype="bf16", has_zp=True, seed=74).to(dev)
    Y = torch.empty(c.M, N, dtype=torch.bfloat16, device=dev)

    def runp(_):
        qmm.qmm_gemm(c.A, c.B, c.scales, c.zero_points, None, Y, c.M, K, N, bs, 4, stream=stream,
                     g_idx=gi)

    for i in range(3):
        runp(i)
    torch.cuda.synchronize()
    ms = _time_launches(runp, max(20, args.steps // 5), stream)
    flop = 2.0 * c.M * N * K
    res["prefill_M2048"] = {"ms": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
                            "frac_bf16_peak": round(flop / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                                                    4)}
    return res


def bench_batched(qmm, dev, stream, args):
    """Float (bf16) batched decode on the decode-layer weights, 4-bit asymmetric
    bs 32 with bf16 scales, operator layout: qmm_gemv at M = 1 and qmm_gemm
    for M = 2 .. 256 on the projections (K, N) = (4096, 14336) and
    (14336, 4096).  Weights rotate through copies so each launch streams them
    from HBM; bytes = codes + scales + zero points + activations + output."""
    from block_quantized_weight_matmulnbits_amd.workloads import make_matmul_case
    res = {}
    for K, N in ((4096, 14336), (14336, 4096)):
        base = make_matmul_case(1, K, N, 32, 4, a_dtype="bf16", has_zp=True, seed=70).to(dev)
        nbytes = base.weight_bytes()
        n_copies = max(2, -(-POOL_BYTES // nbytes))
        pool = [(base.B, base.scales, base.zero_points)] + [
            (base.B.clone(), base.scales.clone(), base.zero_points.clone())
            for _ in range(n_copies - 1)]
        for M in (1, 2, 4, 8, 16, 32, 64, 128, 256):
            A = make_matmul_case(M, K, N, 32, 4, a_dtype="bf16", seed=71 + M).A.to(dev)
            Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)

            def run(i, A=A, Y=Y, M=M, K=K, N=N):
                B, sc, zp = pool[i % len(pool)]
                if M == 1:
                    qmm.qmm_gemv(A.reshape(-1), B, sc, zp, None, Y.reshape(-1), K, N, 32, 4,
                                 stream=stream)
                else:
                    qmm.qmm_gemm(A, B, sc, zp, None, Y, M, K, N, 32, 4, 0, stream)

            for i in range(3):
                run(i)
            torch.cuda.synchronize()
            ms = _time_launches(run, max(20, args.steps // 4), stream)
            byts = nbytes + A.numel() * 2 + M * N * 2
            res[f"K{K}_N{N}_M{M}"] = {
                "us": round(ms * 1e3, 2), "GBps": round(byts / (ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "tflops": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 2)}
        del pool
    return res


def bench_conv(qmm, dev, stream, args):
    """int8 conv 1x56x56x64, 3x3, stride 1, pad 1, 64 output channels."""
    from block_quantized_weight_matmulnbits_amd.workloads import make_conv_case
    c = make_conv_case().to(dev)
    Y = torch.empty(1, 56, 56, 64, dtype=torch.int8, device=dev)

    def run(_):
        qmm.qconv_int8(c.X, c.W, c.bias, c.w_scale, c.in_scale, c.out_scale, c.in_zp, c.out_zp,
                       c.clamp_min, c.clamp_max, c.stride, c.pad, Y, stream)

    for i in range(3):
        run(i)
    torch.cuda.synchronize()
    ms = _time_launches(run, max(20, args.steps), stream)
    ops = 2 * 56 * 56 * 64 * 3 * 3 * 64
    byts = c.X.numel() + c.W.numel() + 4 * 64 + 4 * 64 + Y.numel()
    return {"workload": "int8 conv NHWC 1x56x56x64, 3x3, stride 1, pad 1, Co=64, requant to int8",
            "us": round(ms * 1e3, 2), "int8_tops": round(ops / (ms * 1e-3) / 1e12, 3),
            "GBps": round(byts / (ms * 1e-3) / 1e9, 2), "int_ops_per_launch": ops,
            "bytes_per_launch": byts}


def cpu_baseline(cases, seconds):
    """The oracle (as it stands) on the same layer, on the host cores."""
    import numpy as np

    import oracle
    prepared = []
    for c in cases:
        prepared.append((c.A.double().numpy().reshape(1, -1), c.B.numpy(), c.scales.double().numpy(),
                         c.zero_points.numpy(), None, c.N, c.K, c.block_size, c.bits))
    step_bytes = sum(layer_bytes(c) for c in cases)
    oracle.matmul_nbits(*prepared[1])            # load + warm the library
    reps, t0 = 0, time.perf_counter()
    while True:
        for p in prepared:
            oracle.matmul_nbits(*p)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return {
        "value": round(step_bytes * reps / el / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"the full decode layer (all 7 projections, all outputs), {reps} passes in "
                  f"{el:.1f} s, OpenMP over output columns",
        "ms_per_step": round(el / reps * 1e3, 2),
    }


def _timed(fn, seconds):
    """Run fn() until `seconds` have passed (at least once); seconds per call."""
    fn()
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return el / reps, reps


def cpu_baseline_configs(seconds):
    """The oracle on the other configurations, each on a bounded sample,
    scaled to the configuration's own unit."""
    import numpy as np

    import oracle
    from block_quantized_weight_matmulnbits_amd.workloads import (COMPINT8_VARIANTS,
                                                                   compint8_case, make_conv_case,
                                                                   prefill_gemm, tiny_matmulnbits)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    f64 = lambda t: None if t is None else t.double().numpy()
    u8 = lambda t: None if t is None else t.numpy()
    res = {"cores": threads, "kind": "oracle"}
    # Tiny: the whole problem.
    c = tiny_matmulnbits()
    sec, reps = _timed(lambda: oracle.matmul_nbits(f64(c.A), u8(c.B), f64(c.scales), None, None,
                                                   c.N, c.K, c.block_size, c.bits), seconds / 4)
    res["tiny"] = {"us_per_call": round(sec * 1e6, 2), "sample": "the whole problem",
                   "reps": reps}
    # CompInt8: quantize the activations and the full matmul, on 512 columns.
    ci8 = {}
    for bits, bs, asym in COMPINT8_VARIANTS:
        for M in (1, 16):
            c = compint8_case(M, bits, bs, asym)
            ncol = 512
            B, S = u8(c.B[:ncol]), f64(c.scales[:ncol])
            Z = None if c.zero_points is None else u8(c.zero_points[:ncol])
            A = c.A.float().numpy()

            def run(A=A, B=B, S=S, Z=Z, c=c, ncol=ncol):
                qa, sa = oracle.quantize_a(A, c.K, c.block_size)
                oracle.compint8_matmul(qa, sa, B, S, Z, None, ncol, c.K, c.block_size, c.bits)

            sec, reps = _timed(run, seconds / 8)
            byts = (c.weight_bytes() * ncol // c.N) + A.size * 2 + M * ncol * 2
            ci8[f"b{bits}_bs{bs}_M{M}"] = {"GBps": round(byts / sec / 1e9, 4), "reps": reps}
    res["compint8"] = {"sample": "512 of the 14336 columns (all K), activations quantized "
                                 "in every call", "per_case": ci8}
    # Prefill: 4 rows of A against every column.
    c = prefill_gemm()
    A = f64(c.A[:4])
    sec, reps = _timed(lambda: oracle.matmul_nbits(A, u8(c.B), f64(c.scales), u8(c.zero_points),
                                                   None, c.N, c.K, c.block_size, c.bits),
                       seconds / 4)
    res["prefill_gemm"] = {"tflops": round(2.0 * 4 * c.N * c.K / sec / 1e12, 6),
                           "sample": "4 of the 2048 rows, every column", "reps": reps}
    # Conv: the whole problem (one thread: the oracle's conv loop is serial).
    c = make_conv_case()
    sec, reps = _timed(lambda: oracle.conv_int8(c.X.numpy(), c.W.numpy(), c.bias.numpy(),
                                                c.w_scale.numpy(), c.in_scale, c.out_scale,
                                                c.in_zp, c.out_zp, c.clamp_min, c.clamp_max,
                                                c.stride, c.pad), seconds / 4)
    res["conv_int8"] = {"us_per_call": round(sec * 1e6, 1),
                        "int8_tops": round(231211008 / sec / 1e12, 6),
                        "sample": "the whole problem (serial loop)", "reps": reps}
    return res


if __name__ == "__main__":
    main()
