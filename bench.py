#!/usr/bin/env python3
"""libgemm benchmark: GEMM TFLOP/s (2MNK / time) on MI355X and the fraction of
the dense matrix-core peak, on seeded synthetic matrices resident in HBM.

A step is one GEMM call.  The headline is bf16 C = A*B at M = N = K = 4096
(row-major A and B, fp32 accumulation, bf16 C).  The other workloads (fp16
4096^3, the ragged bf16 shapes, bf16 2048^3 and 2560^3 on the medium-grid
tiles, fp32 4096^3, fp8 block-scaled 8192^3, fp16 256^3, the 4096^3 bf16
product with a fused bias + relu epilogue and with a fused residual add, the
MFMA-only ceiling of the headline kernel, the nine rungs of the optimisation
ladder on fp16 4096^3, two 3x3 convolution layers through im2col + GEMM and the
im2col pack alone, and the FP8 block quantiser on the fp8 workload's 8192 x 8192
operand) are measured in the same run and listed under "workloads".

Each workload first runs a settle pass (about 50 ms of back-to-back launches:
the clock ramps up from idle over the first ~20 ms of work), then W warm-up
launches, then the K timed launches.  Plain GEMM workloads whose launches take
less than 40 us are also timed from a HIP graph of captured launches, since the
host's per-call launch cost bounds them otherwise.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads headline|all]
                    [--settle-ms MS] [--cold-steps N] [--no-cpu-baseline] [--no-graph]
                    [--no-loop-fit]

Prints ONE JSON line.  Only one GPU is used: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s at M=N=K=4096 bf16/fp16 + % of MI355X dense MFMA peak"
# MI355X dense peaks (TFLOP/s): 256 CUs x 2.4 GHz x (4096 bf16/fp16, 8192 fp8,
# 256 fp32 matrix) flop per clock per CU.  HBM3E 8 TB/s.
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "fp8": 5033.2, "f32": 157.3}
HBM_PEAK_GBS = 8000.0
# Best kernel of "[CUDA 优化实战] hgemm - 超越 cuBLAS" section 5 at M=N=K=4096
# (half precision, RTX 5060 Laptop GPU): 4.075860 ms = 33.72 TFLOP/s.  Context only.
PAGES_TFLOPS_4096 = 33.72
ELEM_BYTES = {"f16": 2, "bf16": 2, "f32": 4, "fp8": 1}
OUT_BYTES = {"f16": 2, "bf16": 2, "f32": 4, "fp8": 2}


def tflops(M: int, N: int, K: int, seconds: float) -> float:
    """The pages' metric: 2*M*N*K floating-point operations over the time."""
    return 2.0 * M * N * K / seconds / 1e12


def algorithmic_bytes(dtype: str, M: int, N: int, K: int) -> int:
    """Bytes a GEMM must move at least once: A and B read, C written (+ fp8 scales)."""
    b = ELEM_BYTES[dtype] * (M * K + K * N) + OUT_BYTES[dtype] * M * N
    if dtype == "fp8":
        cd = lambda a: -(-a // 64)
        b += 4 * (cd(M) * cd(K) + cd(K) * cd(N))
    return b


# Sources that define the headline kernel's machine code: the measured traffic
# below stays valid while these are unchanged.
HEADLINE_KERNEL_SOURCES = ("gemm_h16_fast.hip", "gemm_device.hpp", "gemm_lds_layout.hpp")


def kernel_source_digest(files=HEADLINE_KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        p = os.path.join(ROOT, "dense_gemm_13_amd", "csrc", f)
        h.update(f.encode())
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(name: str):
    """HBM bytes per launch from a committed counter summary, if it was taken on
    the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_digest") != kernel_source_digest():
        return None
    try:
        return int(float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


# Settle pass before each workload's timed steps: about 50 ms of back-to-back
# launches (at most 2000), so the clock has ramped up from idle.
SETTLE_SECONDS = 0.05
SETTLE_MAX_LAUNCHES = 2000

_FLUSH = {}


# Plain GEMM workloads whose launches take less than this are also timed from a
# HIP graph (the host's launch rate bounds them otherwise).
GRAPH_BELOW_S = 40e-6


def set_settle(seconds: float):
    global SETTLE_SECONDS
    SETTLE_SECONDS = seconds


def flush_buffer(device):
    """A 512 MiB device buffer, written once (twice the Infinity Cache)."""
    import torch
    if device not in _FLUSH:
        _FLUSH[device] = torch.ones((512 << 20) // 4, dtype=torch.int32, device=device)
    return _FLUSH[device]


def flush_read(buf):
    """Read every byte of `buf` (a reduction kernel; nothing is written back)."""
    return buf.sum()


class Workload:
    sustain = 0          # launches of the sustained pass (0: none)

    def __init__(self, key, name, dtype, M, N, K, wid, sustain=0):
        self.key, self.name, self.dtype = key, name, dtype
        self.M, self.N, self.K, self.wid = M, N, K, wid
        self.sustain = sustain

    def setup(self):
        import numpy as np
        import torch

        import dense_gemm_13_amd as dg
        import gemm_inputs as gi
        ops = gi.operands(self.dtype, self.M, self.N, self.K, self.wid)
        self.ops = ops
        dev = torch.device("cuda:0")
        if self.dtype in ("bf16", "f16"):
            tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float16
            self.A = torch.from_numpy(ops["A"].view(np.int16)).view(tdt).to(dev)
            self.B = torch.from_numpy(ops["B"].view(np.int16)).view(tdt).to(dev)
            self.C = torch.empty((self.M, self.N), dtype=tdt, device=dev)
        elif self.dtype == "f32":
            self.A = torch.from_numpy(ops["A"]).to(dev)
            self.B = torch.from_numpy(ops["B"]).to(dev)
            self.C = torch.empty((self.M, self.N), dtype=torch.float32, device=dev)
        else:
            self.A = torch.from_numpy(ops["A"]).to(dev)
            self.B = torch.from_numpy(ops["B"]).to(dev)
            self.sa = torch.from_numpy(ops["scale_a"]).to(dev)
            self.sb = torch.from_numpy(ops["scale_b"]).to(dev)
            self.C = torch.empty((self.M, self.N), dtype=torch.bfloat16, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        M, N, K = self.M, self.N, self.K
        a, b, c = self.A.data_ptr(), self.B.data_ptr(), self.C.data_ptr()
        if self.dtype == "fp8":
            fn, sa, sb = dg.lib.gemm_fp8_blockscaled, self.sa.data_ptr(), self.sb.data_ptr()
            self.call_on = lambda st: (lambda h=ctypes.c_void_p(st.cuda_stream):
                                       fn(a, b, c, M, N, K, K, N, N, sa, sb, h))
        else:
            fn = getattr(dg.lib, "gemm_" + self.dtype)
            self.call_on = lambda st: (lambda h=ctypes.c_void_p(st.cuda_stream):
                                       fn(a, b, c, M, N, K, K, N, N, h))
        self.call = self.call_on(self.stream)
        torch.cuda.synchronize()

    def graph(self, launches: int, replays: int = 5):
        """Mean launch time with `launches` launches captured in one HIP graph and
        the graph replayed `replays` times between two events: the kernel's own
        rate, without the host's per-call launch cost, which is longer than
        kernels of a few microseconds.  Every replay's C is checked bit for bit
        against the eager launches' C (the kernels are deterministic)."""
        import torch
        torch.cuda.synchronize()
        ref = self.C.clone()
        self.C.fill_(0)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream()
            call = self.call_on(cap)
            for _ in range(launches):
                rc = call()
                if rc != 0:
                    raise RuntimeError(f"{self.name}: libgemm returned {rc} under capture")
        for _ in range(2):
            self.C.fill_(0)
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(self.C.view(torch.uint8), ref.view(torch.uint8)):
                raise RuntimeError(f"{self.name}: graph replay differs from the eager result")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        if not torch.equal(self.C.view(torch.uint8), ref.view(torch.uint8)):
            raise RuntimeError(f"{self.name}: graph replay differs from the eager result")
        del g
        return e0.elapsed_time(e1) * 1e-3 / (replays * launches)

    def cold(self, steps: int) -> float:
        """Mean launch time with L2 and the Infinity Cache flushed before each
        launch (the operands of every workload fit in the 256 MiB Infinity Cache
        otherwise).  The flush READS a 512 MiB buffer that was written once at
        allocation: the lines it leaves in the caches are clean, and whatever the
        previous launch left dirty is written back during the flush, so the timed
        launch pays for its own HBM traffic only."""
        import torch
        flush = flush_buffer(self.C.device)
        evs = []
        for _ in range(steps):
            flush_read(flush)
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(self.stream)
            self.call()
            e.record(self.stream)
            evs.append((s, e))
        torch.cuda.synchronize()
        return sum(s.elapsed_time(e) for s, e in evs) / steps * 1e-3

    def sustained(self, launches: int) -> float:
        """Mean launch time over `launches` back-to-back launches in one region:
        long enough (hundreds of launches, tens of milliseconds) for the chip's
        power controller to settle at the clock it holds under this load."""
        import torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(launches):
            self.call()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / launches

    def settle_launches(self) -> int:
        """Launches of the settle pass: about SETTLE_SECONDS of back-to-back work
        (at least `sustain`), estimated from one timed launch."""
        import torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        self.call()
        e1.record(self.stream)
        torch.cuda.synchronize()
        t1 = max(e0.elapsed_time(e1) * 1e-3, 1e-6)
        if SETTLE_SECONDS <= 0:
            return 0
        return max(self.sustain, min(SETTLE_MAX_LAUNCHES, int(SETTLE_SECONDS / t1)))

    def run(self, steps: int, warmup: int, cold_steps: int) -> dict:
        """Settle pass, then `warmup` untimed launches, then the timed region:
        `steps` back-to-back launches on one stream between two HIP events (the
        mean launch time is the region over `steps`).  A second pass with an
        event pair around every launch gives the per-launch median, and a cold
        pass the time with flushed caches.

        The settle pass exists because the chip comes out of idle (the host
        generating the next workload's inputs) at a low clock and ramps up over
        the first ~20 ms of sustained work: the first ~200 launches of the
        4096^3 product run 10-30 % slower than the rest, for this library's
        kernels and the vendor library's alike.  Its launches are timed as one
        region and reported as the sustained figure."""
        import torch
        rc = self.call()
        if rc != 0:
            raise RuntimeError(f"{self.name}: libgemm returned {rc}")
        settle = self.settle_launches()
        sustained = self.sustained(settle) if settle > 0 else None
        for _ in range(warmup):
            rc = self.call()
            if rc != 0:
                raise RuntimeError(f"{self.name}: libgemm returned {rc}")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(self.stream)
        for _ in range(steps):
            self.call()
        e1.record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        region = e0.elapsed_time(e1) * 1e-3
        mean = region / steps
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for i in range(steps):
            starts[i].record(self.stream)
            self.call()
            ends[i].record(self.stream)
        torch.cuda.synchronize()
        per = sorted(s.elapsed_time(e) * 1e-3 for s, e in zip(starts, ends))
        median = per[len(per) // 2]
        cold = self.cold(cold_steps) if cold_steps > 0 else None
        r = self.report(region, wall, mean, median, cold)
        if type(self) is Workload and mean < GRAPH_BELOW_S:
            g = self.graph(max(steps, 50))
            r["graph_mean_launch_us"] = g * 1e6
            r["graph_tflops"] = tflops(self.M, self.N, self.K, g)
            r["graph_alg_gbs"] = algorithmic_bytes(self.dtype, self.M, self.N, self.K) / g / 1e9
        r["settle_launches"] = settle
        if sustained is not None:
            r["sustained_launches"] = settle
            r["sustained_mean_launch_us"] = sustained * 1e6
            if self.K:
                r["sustained_tflops"] = tflops(self.M, self.N, self.K, sustained)
        return r

    def report(self, region, wall, mean, median, cold) -> dict:
        M, N, K, dt = self.M, self.N, self.K, self.dtype
        return {
            "workload": self.name, "key": self.key, "dtype": dt, "M": M, "N": N, "K": K,
            "region_s": region, "wall_s": wall,
            "mean_launch_us": mean * 1e6, "median_launch_us": median * 1e6,
            "tflops": tflops(M, N, K, mean),
            "pct_peak": 100.0 * tflops(M, N, K, mean) / PEAK_TFLOPS[dt],
            "alg_gbs": algorithmic_bytes(dt, M, N, K) / mean / 1e9,
            "cold_mean_launch_us": cold * 1e6 if cold else None,
            "cold_tflops": tflops(M, N, K, cold) if cold else None,
            "cold_alg_gbs": algorithmic_bytes(dt, M, N, K) / cold / 1e9 if cold else None,
            "cold_pct_hbm_peak": 100.0 * algorithmic_bytes(dt, M, N, K) / cold / 1e9
                                 / HBM_PEAK_GBS if cold else None,
        }

    def summary(self, r) -> str:
        g = (f"; from a graph {r['graph_mean_launch_us']:.1f} us, {r['graph_tflops']:.1f} TFLOP/s"
             if "graph_mean_launch_us" in r else "")
        return (f"{r['tflops']:.1f} TFLOP/s ({r['pct_peak']:.1f}% peak), "
                f"{r['mean_launch_us']:.1f} us/launch{g}")


class QuantWorkload(Workload):
    """The block-scaled FP8 quantiser on a rows x cols fp32 matrix (the step
    that makes the fp8 GEMM's operands).  HBM-bound: reported as algorithmic
    GB/s (input read once, codes and scales written once) against 8 TB/s."""

    def __init__(self, key, name, rows, cols, block, fmt, seed):
        super().__init__(key, name, "f32", rows, cols, 0, 0)
        self.block, self.fmt, self.seed = block, fmt, seed

    def setup(self):
        import torch

        import dense_gemm_13_amd as dg
        import gemm_inputs as gi
        dev = torch.device("cuda:0")
        rows, cols, blk = self.M, self.N, self.block
        self.A = torch.from_numpy(gi.normal_f32(rows, cols, self.seed)).to(dev)
        self.C = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        self.B = torch.empty((-(-rows // blk), -(-cols // blk)), dtype=torch.float32, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        s = ctypes.c_void_p(self.stream.cuda_stream)
        fn, fmt = dg.lib.gemm_quantize_fp8, dg.FP8_FORMATS[self.fmt]
        x, q, sc = self.A.data_ptr(), self.C.data_ptr(), self.B.data_ptr()
        self.call = lambda: fn(x, 0, rows, cols, cols, blk, fmt, q, cols, sc, s)
        torch.cuda.synchronize()

    def alg_bytes(self) -> int:
        rows, cols, blk = self.M, self.N, self.block
        return rows * cols * (4 + 1) + 4 * (-(-rows // blk)) * (-(-cols // blk))

    def report(self, region, wall, mean, median, cold) -> dict:
        gbs = self.alg_bytes() / mean / 1e9
        return {
            "workload": self.name, "key": self.key, "dtype": "f32->" + self.fmt,
            "rows": self.M, "cols": self.N, "block": self.block,
            "region_s": region, "wall_s": wall,
            "mean_launch_us": mean * 1e6, "median_launch_us": median * 1e6,
            "alg_gbs": gbs, "pct_hbm_peak": 100.0 * gbs / HBM_PEAK_GBS,
            "cold_mean_launch_us": cold * 1e6 if cold else None,
            "cold_alg_gbs": self.alg_bytes() / cold / 1e9 if cold else None,
            "cold_pct_hbm_peak": 100.0 * self.alg_bytes() / cold / 1e9 / HBM_PEAK_GBS
                                 if cold else None,
        }

    def summary(self, r) -> str:
        return (f"{r['alg_gbs']:.0f} GB/s ({r['pct_hbm_peak']:.1f}% of HBM peak), "
                f"{r['mean_launch_us']:.1f} us/launch")


class LadderWorkload(Workload):
    """One rung of the optimisation ladder (gemm_h16_ladder) on the same
    operands as the plain workload; `rung` None is the MFMA-only ceiling kernel
    (the large-tile kernel's MFMA sequence with register-held operands, which
    writes (K/32) * A[:, :32] * B[:32, :], not the product)."""

    def __init__(self, key, name, dtype, M, N, K, wid, rung, max_steps=None):
        super().__init__(key, name, dtype, M, N, K, wid)
        self.rung, self.max_steps = rung, max_steps

    def setup(self):
        import torch

        import dense_gemm_13_amd as dg
        super().setup()
        s = ctypes.c_void_p(self.stream.cuda_stream)
        M, N, K = self.M, self.N, self.K
        a, b, c = self.A.data_ptr(), self.B.data_ptr(), self.C.data_ptr()
        bf = int(self.dtype == "bf16")
        if self.rung is None:
            fn = dg.lib.gemm_h16_mfma_ceiling
            self.call = lambda: fn(bf, a, b, c, M, N, K, K, N, N, s)
        else:
            fn, r = dg.lib.gemm_h16_ladder, self.rung
            self.call = lambda: fn(r, bf, a, b, c, M, N, K, K, N, N, s)
        torch.cuda.synchronize()

    def run(self, steps, warmup, cold_steps):
        if self.max_steps:
            steps, warmup, cold_steps = min(steps, self.max_steps), min(warmup, 1), 0
        return super().run(steps, warmup, cold_steps)

    def settle_launches(self) -> int:
        return 0 if self.max_steps else super().settle_launches()

    def report(self, region, wall, mean, median, cold) -> dict:
        r = super().report(region, wall, mean, median, cold)
        r["rung"] = "mfma_only_ceiling" if self.rung is None else self.rung
        return r


class ConvWorkload(Workload):
    """A 3x3 convolution layer (NHWC, HWIO weights, padding 1, bias + relu) through
    gemm_conv2d_nhwc: the im2col pack into a preallocated workspace, then the
    GEMM (n*ho*wo) x (9*c_in) x c_out.  TFLOP/s counts the convolution's
    2 * n*ho*wo * 9*c_in * c_out flops; with `pack_only` the line times the
    im2col kernel alone and reports its GB/s (input read once, matrix written)."""

    def __init__(self, key, name, n, hw, c_in, c_out, wid, pack_only=False):
        M = n * hw * hw
        super().__init__(key, name, "bf16", M, c_out, 9 * c_in, wid)
        self.n, self.hw, self.c_in, self.c_out, self.pack_only = n, hw, c_in, c_out, pack_only

    def setup(self):
        import numpy as np
        import torch

        import dense_gemm_13_amd as dg
        import gemm_inputs as gi
        dev = torch.device("cuda:0")
        n, hw, ci, co = self.n, self.hw, self.c_in, self.c_out
        as_bf16 = lambda b, shape: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16) \
            .reshape(shape).to(dev)
        self.A = as_bf16(gi.uniform_h16(n * hw * hw, ci, 1000 + self.wid, "bf16"), (n, hw, hw, ci))
        self.B = as_bf16(gi.uniform_h16(9 * ci, co, 2000 + self.wid, "bf16"), (3, 3, ci, co))
        self.bias = torch.from_numpy(gi.uniform_f32(1, co, 7000 + self.wid)[0]).to(dev)
        self.C = torch.empty((n, hw, hw, co), dtype=torch.bfloat16, device=dev)
        shape = dg.Conv2dShape(n, hw, hw, ci, co, 3, 3, 1, 1, 1, 1, 1, 1)
        self.shape = shape
        need = dg.lib.gemm_conv2d_workspace_bytes(dg.DTYPES["bf16"], ctypes.byref(shape))
        self.ws = torch.empty(need, dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream(dev)
        s = ctypes.c_void_p(self.stream.cuda_stream)
        x, w, y, ws, b = (self.A.data_ptr(), self.B.data_ptr(), self.C.data_ptr(),
                          self.ws.data_ptr(), self.bias.data_ptr())
        sp = ctypes.byref(shape)
        relu = dg.ACTIVATIONS["relu"]
        if self.pack_only:
            fn = dg.lib.gemm_im2col_nhwc
            self.call = lambda: fn(dg.DTYPES["bf16"], x, ws, 9 * ci, sp, s)
        else:
            fn = dg.lib.gemm_conv2d_nhwc
            self.call = lambda: fn(dg.DTYPES["bf16"], x, w, y, ws, need, sp, b, relu, s)
        torch.cuda.synchronize()

    def report(self, region, wall, mean, median, cold) -> dict:
        r = super().report(region, wall, mean, median, cold)
        n, hw, ci, co = self.n, self.hw, self.c_in, self.c_out
        r.update({"conv": f"{n}x{hw}x{hw}x{ci} -> {co}, 3x3, pad 1, stride 1, bias + relu",
                  "gemm": f"{self.M} x {co} x {9 * ci}"})
        pack_bytes = 2 * n * hw * hw * ci + 2 * self.M * 9 * ci
        if self.pack_only:
            r["alg_gbs"] = pack_bytes / mean / 1e9
            r["pct_hbm_peak"] = 100.0 * r["alg_gbs"] / HBM_PEAK_GBS
            if cold:
                r["cold_alg_gbs"] = pack_bytes / cold / 1e9
                r["cold_pct_hbm_peak"] = 100.0 * r["cold_alg_gbs"] / HBM_PEAK_GBS
            for k in ("tflops", "pct_peak", "cold_tflops"):
                r.pop(k, None)
        else:
            conv_bytes = 2 * n * hw * hw * (ci + co) + 2 * 9 * ci * co + 4 * co
            r["alg_gbs"] = conv_bytes / mean / 1e9
            r.pop("cold_pct_hbm_peak", None)
            r["cold_alg_gbs"] = conv_bytes / cold / 1e9 if cold else None
        return r

    def summary(self, r) -> str:
        if self.pack_only:
            return f"{r['alg_gbs']:.0f} GB/s, {r['mean_launch_us']:.1f} us/launch"
        return super().summary(r)


class EpilogueWorkload(Workload):
    """A GEMM through its fused-epilogue entry point: a fully connected layer
    C = relu(A*B + bias) (alpha 1, beta 0, one fp32 bias per column), or with
    beta != 0 a residual add of the prior C as well."""

    def __init__(self, key, name, dtype, M, N, K, wid, beta=0.0):
        super().__init__(key, name, dtype, M, N, K, wid)
        self.beta = beta

    def setup(self):
        import torch

        import dense_gemm_13_amd as dg
        import gemm_inputs as gi
        super().setup()
        dev = self.C.device
        self.bias = torch.from_numpy(gi.uniform_f32(1, self.N, 7000 + self.wid)[0]).to(dev)
        self.C.zero_()
        s = ctypes.c_void_p(self.stream.cuda_stream)
        M, N, K = self.M, self.N, self.K
        a, b, c, bias = self.A.data_ptr(), self.B.data_ptr(), self.C.data_ptr(), self.bias.data_ptr()
        fn = getattr(dg.lib, f"gemm_{self.dtype}_epilogue")
        relu = dg.ACTIVATIONS["relu"]
        beta = self.beta
        self.call = lambda: fn(a, b, c, M, N, K, K, N, N, 1.0, beta, bias, relu, s)
        torch.cuda.synchronize()

    def report(self, region, wall, mean, median, cold) -> dict:
        r = super().report(region, wall, mean, median, cold)
        # the prior C is read once more when beta != 0
        extra = OUT_BYTES[self.dtype] * self.M * self.N if self.beta != 0 else 0
        r["alg_gbs"] = (algorithmic_bytes(self.dtype, self.M, self.N, self.K) + extra
                        + 4 * self.N) / mean / 1e9
        r["epilogue"] = f"relu(A*B + {'C + ' if self.beta else ''}bias)"
        return r


WORKLOADS = [
    Workload("bf16_4096", "bf16 GEMM M=N=K=4096", "bf16", 4096, 4096, 4096, 2, sustain=300),
    Workload("f16_4096", "fp16 GEMM M=N=K=4096", "f16", 4096, 4096, 4096, 2, sustain=300),
    Workload("f16_256", "fp16 GEMM M=N=K=256", "f16", 256, 256, 256, 1),
    Workload("bf16_1000", "bf16 GEMM 1000x1000x1000", "bf16", 1000, 1000, 1000, 3),
    Workload("bf16_ragged", "bf16 GEMM 4097x4095x4100", "bf16", 4097, 4095, 4100, 3),
    Workload("bf16_skinny", "bf16 GEMM 8192x64x4096", "bf16", 8192, 64, 4096, 3),
    # medium grids: 128 x 128 tiles (two workgroups per CU) and 128 x 256 tiles
    Workload("bf16_2048", "bf16 GEMM M=N=K=2048", "bf16", 2048, 2048, 2048, 6),
    Workload("bf16_2560", "bf16 GEMM M=N=K=2560", "bf16", 2560, 2560, 2560, 7),
    Workload("f32_4096", "fp32 SGEMM M=N=K=4096", "f32", 4096, 4096, 4096, 4),
    Workload("fp8_8192", "fp8 E4M3 64x64-block-scaled GEMM M=N=K=8192, bf16 C", "fp8",
             8192, 8192, 8192, 5),
    EpilogueWorkload("bf16_4096_bias_relu", "bf16 GEMM M=N=K=4096, fused relu(A*B + bias)",
                     "bf16", 4096, 4096, 4096, 2),
    EpilogueWorkload("bf16_4096_residual", "bf16 GEMM M=N=K=4096, fused relu(A*B + C + bias)",
                     "bf16", 4096, 4096, 4096, 2, beta=1.0),
    LadderWorkload("bf16_4096_mfma_ceiling", "bf16 M=N=K=4096 MFMA-only ceiling (the "
                   "large-tile kernel's MFMAs, register-held operands, no memory traffic)",
                   "bf16", 4096, 4096, 4096, 2, None),
] + [
    LadderWorkload(f"ladder_{r}", f"fp16 GEMM M=N=K=4096, ladder rung {r} ({name})", "f16",
                   4096, 4096, 4096, 2, r, max_steps=5 if r <= 2 else None)
    for r, name in enumerate(("naive", "64x64 LDS tiles", "register tiles, conflict-free LDS",
                              "MFMA, one LDS stage", "MFMA + double buffer",
                              "MFMA + double buffer + swizzle", "library kernel",
                              "MFMA, one LDS stage, one workgroup per CU",
                              "MFMA + double buffer, one workgroup per CU"))
] + [
    ConvWorkload("conv_56x64", "bf16 3x3 conv 32x56x56x64 -> 64 (im2col + GEMM, bias + relu)",
                 32, 56, 64, 64, 8),
    ConvWorkload("conv_14x256", "bf16 3x3 conv 32x14x14x256 -> 256 (im2col + GEMM, bias + relu)",
                 32, 14, 256, 256, 9),
    ConvWorkload("im2col_56x64", "bf16 im2col pack, 32x56x56x64, 3x3, pad 1", 32, 56, 64, 64, 8,
                 pack_only=True),
    QuantWorkload("quant_8192", "FP8 E4M3 64x64 block quantiser, 8192x8192 fp32 N(0,1)",
                  8192, 8192, 64, "e4m3", 1005),
]


# Oracle timings: (key, dtype, M, N, K, workload id, rows timed (None: all),
# threads (None: the host's CPU share)).  The workloads are the five configured
# ones at their full shapes; large products are timed on their first rows (the
# oracle's rows are independent and cost the same each, so the rate carries
# over).  Two single-core runs give the per-core rate on the small shapes.
ORACLE_CASES = (
    ("f16_256", "f16", 256, 256, 256, 1, None, None),
    ("bf16_4096", "bf16", 4096, 4096, 4096, 2, 2048, None),
    ("f16_4096", "f16", 4096, 4096, 4096, 2, 2048, None),
    ("bf16_1000", "bf16", 1000, 1000, 1000, 3, None, None),
    ("bf16_ragged", "bf16", 4097, 4095, 4100, 3, 1024, None),
    ("bf16_skinny", "bf16", 8192, 64, 4096, 3, None, None),
    ("f32_4096", "f32", 4096, 4096, 4096, 4, 1024, None),
    ("fp8_8192", "fp8", 8192, 8192, 8192, 5, 256, None),
    ("f16_256_1core", "f16", 256, 256, 256, 1, None, 1),
    ("bf16_1000_1core", "bf16", 1000, 1000, 1000, 3, None, 1),
)


def loop_fit(rounds: int = 2, settle: int = 300, launches: int = 200) -> dict:
    """Launch time against K at M = N = 4096 for the headline kernel and for the
    MFMA-only ceiling: each at K = 4096 and 8192, alternated, `settle` launches
    then the mean of `launches` back-to-back ones, medians over `rounds`.  The
    line through the two points splits a launch into a fixed part (prologue,
    epilogue, launch) and a per-K loop rate, so the two kernels' loops can be
    compared without their different fixed costs."""
    import numpy as np
    import torch

    import dense_gemm_13_amd as dg
    import gemm_inputs as gi
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    s = ctypes.c_void_p(st.cuda_stream)
    M = N = 4096
    bufs, calls = [], {}
    for K in (4096, 8192):
        ops = gi.operands("bf16", M, N, K, 2)
        A = torch.from_numpy(ops["A"].view(np.int16)).view(torch.bfloat16).to(dev)
        B = torch.from_numpy(ops["B"].view(np.int16)).view(torch.bfloat16).to(dev)
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        bufs += [A, B, C]
        a, b, c = A.data_ptr(), B.data_ptr(), C.data_ptr()
        calls[("gemm", K)] = (lambda a=a, b=b, c=c, K=K:
                              dg.lib.gemm_bf16(a, b, c, M, N, K, K, N, N, s))
        calls[("ceiling", K)] = (lambda a=a, b=b, c=c, K=K:
                                 dg.lib.gemm_h16_mfma_ceiling(1, a, b, c, M, N, K, K, N, N, s))
    times = {key: [] for key in calls}
    for _ in range(rounds):
        for key, f in calls.items():
            if f() != 0:
                raise RuntimeError(f"loop fit: {key} returned an error")
            for _ in range(settle):
                f()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(launches):
                f()
            e1.record(st)
            torch.cuda.synchronize()
            times[key].append(e0.elapsed_time(e1) * 1e3 / launches)
    del bufs
    torch.cuda.empty_cache()
    out = {"method": f"K = 4096 and 8192 at M = N = 4096, {settle} launches to settle then the "
                     f"mean of {launches}, alternated, median of {rounds} rounds"}
    for kind in ("gemm", "ceiling"):
        t1 = float(np.median(times[(kind, 4096)]))
        t2 = float(np.median(times[(kind, 8192)]))
        slope = t2 - t1
        out[kind] = {"k4096_us": round(t1, 2), "k8192_us": round(t2, 2),
                     "us_per_4096_of_k": round(slope, 2), "intercept_us": round(t1 - slope, 2),
                     "loop_tflops": round(2 * M * N * 4096 / (slope * 1e-6) / 1e12, 1)}
    out["gemm_loop_frac_of_ceiling_loop"] = round(out["ceiling"]["us_per_4096_of_k"]
                                                  / out["gemm"]["us_per_4096_of_k"], 4)
    out["ceiling_loop_frac_of_peak"] = round(out["ceiling"]["loop_tflops"] / PEAK_TFLOPS["bf16"], 4)
    return out


def vs_hipblaslt(w, rounds: int = 3, settle: int = 300, launches: int = 200) -> dict:
    """The same product through torch.matmul (hipBLASLt on ROCm; TF32 and
    reduced-precision reductions off), timed in alternation with the library's
    call on the workload's own operands: `settle` launches, then the mean of
    `launches` back-to-back ones, median over `rounds`.  Context only: it does
    not enter `value`."""
    import numpy as np
    import torch
    torch.backends.cuda.matmul.allow_tf32 = False
    torch.backends.cuda.matmul.allow_bf16_reduced_precision_reduction = False
    torch.backends.cuda.matmul.allow_fp16_reduced_precision_reduction = False
    st = w.stream
    C2 = torch.empty_like(w.C)
    calls = {"libgemm": w.call, "hipblaslt": lambda: torch.matmul(w.A, w.B, out=C2)}
    times = {k: [] for k in calls}
    for _ in range(rounds):
        for k, f in calls.items():
            for _ in range(settle):
                f()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(launches):
                f()
            e1.record(st)
            torch.cuda.synchronize()
            times[k].append(e0.elapsed_time(e1) * 1e3 / launches)
    out = {k: round(float(np.median(v)), 2) for k, v in times.items()}
    out["hipblaslt_time_over_libgemm"] = round(out["hipblaslt"] / out["libgemm"], 4)
    out["method"] = (f"{settle} launches to settle, then the mean of {launches} back to back (us), "
                     f"alternated, median of {rounds} rounds")
    del C2
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cpu_share() -> int:
    """Threads the oracle may use: the CPUs this process may run on, capped by
    the share the host grants one GPU job when it states one (OMP_NUM_THREADS)."""
    n = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    return min(n, int(share)) if share.isdigit() and int(share) > 0 else n


def cpu_baseline() -> dict:
    """The CPU oracle, as it stands, timed on every configured workload (first
    rows of the large ones) with the host's CPU share, plus two single-core
    runs.  `value` is the rate on the headline workload."""
    import gemm_inputs as gi
    import oracle
    share = host_cpu_share()
    cases, total = [], 0.0
    for key, dt, M, N, K, wid, rows, threads in ORACLE_CASES:
        nt = threads or share
        ops = gi.operands(dt, M, N, K, wid)
        r = rows or M
        sa = ops.get("scale_a")
        if sa is not None:
            sa = sa[:-(-r // 64)]
        t0 = time.perf_counter()
        oracle.gemm(dt, ops["A"][:r], ops["B"], r, N, K, sa, ops.get("scale_b"), nthreads=nt)
        t = time.perf_counter() - t0
        total += t
        rate = tflops(r, N, K, t)
        cases.append({"workload": key, "dtype": dt, "M": M, "N": N, "K": K, "rows_timed": r,
                      "threads": nt, "seconds": round(t, 3), "tflops": rate,
                      "gflops": round(rate * 1e3, 2),
                      "full_product_s_est": round(2.0 * M * N * K / (rate * 1e12), 2)})
        print(f"[bench] oracle {key}: {r} of {M} rows, {nt} threads, {t:.2f} s, "
              f"{rate * 1e3:.1f} GFLOP/s", file=sys.stderr, flush=True)
    head = next(c for c in cases if c["workload"] == "bf16_4096")
    return {"value": head["tflops"], "unit": "TFLOP/s", "cores": head["threads"],
            "kind": "oracle",
            "sample": f"first {head['rows_timed']} of 4096 rows of the bf16 M=N=K=4096 product "
                      f"(fp64, bit-exact decode included), {head['seconds']:.2f} s wall; every "
                      f"configured workload timed the same way under 'per_workload' "
                      f"({total:.1f} s in all)",
            "cpu_model": cpu_model(), "host_cpus_visible": os.cpu_count(),
            "threads_used": share, "per_workload": cases}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workloads", default="all",
                    help="all | headline | comma-separated keys: "
                         + ",".join(w.key for w in WORKLOADS))
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="launches timed after a 512 MiB cache-flushing read each (0: skip)")
    ap.add_argument("--no-loop-fit", action="store_true",
                    help="skip the K = 4096 / 8192 fit of the headline kernel and the ceiling")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph timing of short workloads (counter runs use it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_SECONDS * 1e3,
                    help="back-to-back launches before each workload's warm-up, in ms of "
                         "GPU time (0: none; counter runs use 0)")
    ap.add_argument("--vs-hipblaslt", action="store_true",
                    help="also time torch.matmul (hipBLASLt) on each plain fp16/bf16/fp32 "
                         "workload, in alternation with the library (context, not the metric)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a plain elementwise copy (torch.neg) of this many MiB, "
                         "5 times: the known-size kernel that calibrates HBM byte counters")
    args = ap.parse_args()
    set_settle(args.settle_ms * 1e-3)
    if args.no_graph:
        global GRAPH_BELOW_S
        GRAPH_BELOW_S = 0.0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library "
              "has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    headline = WORKLOADS[0]
    if args.workloads == "all":
        todo = WORKLOADS
    elif args.workloads == "headline":
        todo = [headline]
    else:
        keys = args.workloads.split(",")
        unknown = set(keys) - {w.key for w in WORKLOADS}
        if unknown:
            ap.error(f"unknown workloads: {sorted(unknown)}")
        todo = [headline] + [w for w in WORKLOADS if w.key in keys and w is not headline]
    results = []
    for w in todo:
        print(f"[bench] {w.name}: setup", file=sys.stderr, flush=True)
        w.setup()
        steps = args.steps if w is headline else max(10, args.steps // 2)
        r = w.run(steps, args.warmup, args.cold_steps)
        print(f"[bench] {w.name}: {w.summary(r)}", file=sys.stderr, flush=True)
        if args.vs_hipblaslt and type(w) is Workload and w.dtype != "fp8":
            r["vs_hipblaslt"] = vs_hipblaslt(w)
            print(f"[bench] {w.name}: libgemm {r['vs_hipblaslt']['libgemm']} us, hipBLASLt "
                  f"{r['vs_hipblaslt']['hipblaslt']} us", file=sys.stderr, flush=True)
        results.append(r)
        if w is not headline:
            del w.A, w.B, w.C
            torch.cuda.empty_cache()
    if args.copy_mib > 0:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: 5 x torch.neg over {args.copy_mib} MiB "
              f"(reads {args.copy_mib} MiB, writes {args.copy_mib} MiB each)",
              file=sys.stderr, flush=True)
        del src, dst
    h = results[0]
    ceiling = next((r for r in results if r.get("rung") == "mfma_only_ceiling"), None)
    steps = args.steps
    flops = 2 * headline.M * headline.N * headline.K
    out = {
        "metric": METRIC,
        "value": round(h["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["region_s"] / steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(h["tflops"] / PAGES_TFLOPS_4096, 2),
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": headline.name + " (row-major A and B, fp32 accumulation, bf16 C; "
                   "uniform[-1,1) inputs, seeds A=1002 B=2002)",
                   "M": headline.M, "N": headline.N, "K": headline.K,
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "mfma",
            "achieved": round(flops / (h["mean_launch_us"] * 1e-6) / 1e12, 2),
            "peak": PEAK_TFLOPS["bf16"],
            "unit": "TFLOP/s",
            "frac": round(flops / (h["mean_launch_us"] * 1e-6) / 1e12 / PEAK_TFLOPS["bf16"], 4),
            "traffic": measured_traffic("bf16_4096"),
        },
        # the settle pass (>= 300 launches back to back in one region, before
        # the warm-up and the timed steps): the rate over the clock's ramp from
        # idle and after it
        "settle_launches": h.get("settle_launches"),
        "sustained": None if "sustained_tflops" not in h else {
            "launches": h["sustained_launches"],
            "mean_launch_us": round(h["sustained_mean_launch_us"], 2),
            "tflops": round(h["sustained_tflops"], 2),
            "frac_of_peak": round(h["sustained_tflops"] / PEAK_TFLOPS["bf16"], 4)},
        "kernel_source_digest": kernel_source_digest(),
        # the same MFMA instruction sequence with register-held operands and no
        # memory traffic: what the matrix cores sustain on these operand values
        "mfma_only_ceiling": None if ceiling is None else {
            "tflops": round(ceiling["tflops"], 2),
            "mean_launch_us": round(ceiling["mean_launch_us"], 2),
            "headline_frac_of_ceiling": round(h["tflops"] / ceiling["tflops"], 4)},
        "workloads": [{k: (round(v, 3) if isinstance(v, float) else v) for k, v in r.items()}
                      for r in results],
    }
    if ceiling is not None and not args.no_loop_fit:
        print("[bench] loop fit: bf16 4096 x 4096 x {4096, 8192}, GEMM and MFMA-only ceiling",
              file=sys.stderr, flush=True)
        out["loop_fit"] = loop_fit()
        lf = out["loop_fit"]
        print(f"[bench] loop fit: GEMM {lf['gemm']['intercept_us']} us + "
              f"{lf['gemm']['us_per_4096_of_k']} us per 4096 of K ({lf['gemm']['loop_tflops']} "
              f"TFLOP/s in the loop); ceiling {lf['ceiling']['intercept_us']} us + "
              f"{lf['ceiling']['us_per_4096_of_k']} us ({lf['ceiling']['loop_tflops']} TFLOP/s, "
              f"{100 * lf['ceiling_loop_frac_of_peak']:.1f}% of peak); GEMM loop at "
              f"{lf['gemm_loop_frac_of_ceiling_loop']:.3f} of the ceiling's",
              file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
