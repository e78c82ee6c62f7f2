#!/usr/bin/env python3
"""Benchmark of the block-scaled FP8 GEMM hot path on one MI355X.

One step = one library call (the whole hot path: dispatch, staging, FP8 MFMA,
promotion, BF16 epilogue) on one batch of seeded synthetic input that is
already resident in HBM.  The headline workload is the largest one: the
M-grouped contiguous GEMM of 4 experts x 8192 tokens, N = 4096, K = 7168 (the
MoE table of the DeepGEMM launch article, section 3).  Before it, one JSON line
per other workload (the three dense shapes of the same article's dense table,
the first with an added C, and the masked decode shape) goes to stdout, each
marked "per_shape"; the headline line comes last.

Metric (as the pages quote it): TFLOPS = 2 M N K / t and HBM GB/s =
(|A| + |B| + |D| [+ |C|] + scales) / t with 1-byte A/B and 2-byte D, t the
kernel time; the roofline fraction is the bound resource's share of the
MI355X peak (8 TB/s HBM, 5.0 PFLOP/s dense FP8), and also of the peaks this
part reaches with the library's probes (a streaming read, back-to-back MFMAs).

Timing.  The K timed steps are captured in one HIP graph and replayed between
one event pair on the launching stream (the average launch duration).  Before
that the W warm-up calls run and the graph is replayed once untimed; where one
replay takes a millisecond or more, further untimed replays follow until the
GPU has run at least 60 ms back to back, since the part raises its clock over
some tens of milliseconds of sustained load.  Besides,
every shape is timed launch by launch (at least 50 launches for the short
shapes, 10 for the long ones), each behind a spin kernel that keeps the GPU
busy while the host enqueues the launch, for the median and the minimum.
Inputs rotate over enough copies that each cycle touches more than 512 MB,
twice the 256 MB Infinity Cache, so every step reads its operands from HBM.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOPS + HBM GB/s per shape (FP8 block-scaled GEMM), % of roofline"
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0    # also the peak used for FP8 x FP4: each MFMA there has an FP8 operand
PEAK_BF16_TFLOPS = 2500.0   # dense BF16 MFMA peak (the unscaled BF16 GEMM)
PEAK_FP4_TFLOPS = 10100.0   # dense FP4 MFMA peak (FP4 x FP4)
RIDGE = PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # FLOP per byte
WARM_S = 0.06               # seconds of back-to-back untimed work before a timed region
# The pages' H800 numbers for the same shapes (DeepGEMM launch article,
# section 3 dense table): other hardware, context only.
PAGES_TFLOPS = {0: 206.0, 1: 535.0, 2: 1358.0}
HEADLINE = 3
PER_SHAPE = [0, 1, "1c", 2, 4]
KERNEL_SRC = os.path.join(ROOT, "moe_grouped_gemm_scales_amd", "csrc", "kernels", "fp8_gemm.hip")


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def algorithmic(p) -> tuple[float, float, int]:
    """(FLOPs, bytes, computed rows) of one call, by the pages' convention."""
    K, N = p.K, p.N
    if getattr(p, "bf16", False):
        # 2-byte A, B and D, no scales
        if p.kind == "dense":
            rows, groups_used = p.M, 1
        elif p.kind == "contiguous":
            idx = p.m_indices
            rows = int(((idx >= 0) & (idx < p.G)).sum())
            groups_used = int(idx[(idx >= 0) & (idx < p.G)].unique().numel())
        else:
            mm = p.masked_m.clamp(0, p.A.shape[1])
            rows, groups_used = int(mm.sum()), int((mm > 0).sum())
        nbytes = rows * K * 2 + groups_used * N * K * 2 + rows * N * 2 + (rows * N * 4 if p.C is not None else 0)
        return 2.0 * rows * N * K, float(nbytes), rows
    if p.kind == "k_grouped":
        # each group's D [M, N] is computed; A [K, M] and B [K, N] are read once
        M, G = p.M, p.G
        nbytes = K * M + K * N + G * M * N * 2 + (K // 128) * (M + N) * 4
        if p.C is not None:
            nbytes += G * M * N * 4
        return 2.0 * M * N * K, float(nbytes), G * M
    Kb, Nb = K // 128, (N + 127) // 128
    Kb_b = Kb                       # B scale entries along K per scale row
    if p.ue8m0:
        Kb = (Kb + 3) // 4          # one packed 4-byte word per four K blocks
        Kb_b = Kb
    if p.fp4:
        Kb_b = K // 128             # FP4 B: one word (four 1x32 scales) per row and K block
        Nb = N
    if p.kind == "dense":
        rows, groups_used = p.M, 1
    elif p.kind == "contiguous":
        idx = p.m_indices
        rows = int(((idx >= 0) & (idx < p.G)).sum())
        groups_used = int(idx[(idx >= 0) & (idx < p.G)].unique().numel())
    else:
        mm = p.masked_m.clamp(0, p.A.shape[1])
        rows = int(mm.sum())
        groups_used = int((mm > 0).sum())
    flops = 2.0 * rows * N * K
    b_row = K // 2 if p.fp4 else K  # E2M1 B: two codes per byte
    a_row = K // 2 if p.fp4a else K
    if p.fp4a:
        Kb = K // 128               # FP4 A: one word (four 1x32 scales) per row and K block
    nbytes = rows * a_row + groups_used * N * b_row + rows * N * 2
    if p.C is not None:
        nbytes += rows * N * 4
    nbytes += rows * Kb * 4 + groups_used * Nb * Kb_b * 4
    return flops, float(nbytes), rows


def kind_id(kind: str) -> int:
    return {"dense": 0, "contiguous": 1, "masked": 2, "k_grouped": 3}[kind]


def _probe_lib():
    """The probe entry points of libdg.so (include/dg_probe.h)."""
    import moe_grouped_gemm_scales_amd.dg as dgm
    lib = dgm.lib
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.dg_probe_null.argtypes = [i32, vp]
    lib.dg_probe_spin.argtypes = [i32, vp]
    lib.dg_probe_stream_read.argtypes = [vp, ctypes.c_size_t, vp, i32, vp]
    lib.dg_probe_mfma_fp8.argtypes = [i32, i32, vp, vp]
    for f in (lib.dg_probe_null, lib.dg_probe_spin, lib.dg_probe_stream_read, lib.dg_probe_mfma_fp8, lib.dg_probe_call_floor):
        f.restype = i32
    return lib


def _ok(lib, rc):
    if rc != 0:
        raise RuntimeError(f"probe failed ({rc}): {lib.dg_last_error().decode()}")


def _mode_of(mode: str) -> dict:
    return dict(ue8m0=mode == "_ue8m0", fp4=mode == "_fp4", bf16=mode == "_bf16", fp4x4=mode == "_fp4x4")


def make_problem(cfg, mode=""):
    from tests import gen
    m = _mode_of(mode)
    if cfg == "kg":
        return gen.make_k_grouped_workload()
    if m["bf16"]:
        c = gen.WORKLOADS[cfg]
        assert c["kind"] == "dense", "the BF16 bench covers the dense workloads"
        return gen.make_bf16("dense", seed=gen.workload_seed(cfg), M=c["M"], N=c["N"], K=c["K"],
                             with_c=c.get("with_c", False))
    return gen.make_workload(cfg, ue8m0=m["ue8m0"], fp4=m["fp4"], fp4x4=m["fp4x4"])


def bench_workload(p, steps: int, warmup: int, samples: int, graph: bool, mode: str = ""):
    """Time one workload: the graph-replayed timed region, then launch-by-launch samples."""
    import torch

    import moe_grouped_gemm_scales_amd as dg
    from tests.gpu_util import out_shape, to_dev

    m = _mode_of(mode)
    plib = _probe_lib()
    flops, nbytes, rows = algorithmic(p)
    oshape = (p.G, p.M, p.N) if p.kind == "k_grouped" else out_shape(p)
    ws = sum(t.numel() * t.element_size() for t in (p.A, p.sfa, p.B, p.sfb, p.C) if t is not None)
    ws += math.prod(oshape) * 2
    copies = max(1, min(64, math.ceil(512e6 / ws)))
    if p.kind == "k_grouped":
        f = lambda t: None if t is None else t.to("cuda")
        devs = [dict(A=f(p.A), sfa=f(p.sfa), B=f(p.B), sfb=f(p.sfb), C=f(p.C), ks=f(p.ks)) for _ in range(copies)]
    else:
        devs = [to_dev(p) for _ in range(copies)]
    outs = [torch.empty(oshape, dtype=torch.bfloat16, device="cuda") for _ in range(copies)]

    def call(i):
        d, D = devs[i % copies], outs[i % copies]
        if p.kind == "k_grouped":
            dg.dg_k_grouped_fp8_gemm_tn_contiguous(d["A"], d["sfa"], d["B"], d["sfb"], d["ks"], d["C"], D)
        elif m["bf16"]:
            dg.dg_bf16_gemm_nt(d["A"], d["B"], d["C"], D)
        elif m["fp4x4"]:
            if p.kind == "dense":
                dg.dg_fp4_fp4_gemm_nt(d["A"], d["sfa"], d["B"], d["sfb"], d["C"], D)
            elif p.kind == "contiguous":
                dg.dg_m_grouped_fp4_fp4_gemm_nt_contiguous(d["A"], d["sfa"], d["B"], d["sfb"], d["m_indices"],
                                                           d["C"], D)
            else:
                dg.dg_m_grouped_fp4_fp4_gemm_nt_masked(d["A"], d["sfa"], d["B"], d["sfb"], d["masked_m"], d["C"],
                                                       D)
        elif m["fp4"]:
            if p.kind == "dense":
                dg.dg_fp8_fp4_gemm_nt(d["A"], d["sfa"], d["B"], d["sfb"], d["C"], D)
            elif p.kind == "contiguous":
                dg.dg_m_grouped_fp8_fp4_gemm_nt_contiguous(d["A"], d["sfa"], d["B"], d["sfb"], d["m_indices"],
                                                           d["C"], D)
            else:
                dg.dg_m_grouped_fp8_fp4_gemm_nt_masked(d["A"], d["sfa"], d["B"], d["sfb"], d["masked_m"], d["C"],
                                                       D)
        elif p.kind == "dense":
            dg.dg_fp8_gemm_nt(d["A"], d["sfa"], d["B"], d["sfb"], d["C"], D)
        elif p.kind == "contiguous":
            dg.dg_m_grouped_fp8_gemm_nt_contiguous(d["A"], d["sfa"], d["B"], d["sfb"], d["m_indices"], d["C"], D)
        else:
            dg.dg_m_grouped_fp8_gemm_nt_masked(d["A"], d["sfa"], d["B"], d["sfb"], d["masked_m"], d["C"], D)

    rows_arg = p.A.shape[1] if p.kind == "masked" else p.M
    flag = dg.KIND_BF16 if m["bf16"] else dg.SCALE_FP4_FP4 if m["fp4x4"] else dg.SCALE_FP8_FP4 if m["fp4"] else \
        (dg.SCALE_UE8M0 if m["ue8m0"] else 0)
    kernel = dg.describe_config(kind_id(p.kind) | flag, rows_arg, p.N, p.K, p.G, p.C is not None)
    # everything runs on one non-default stream (HIP graphs cannot capture the null stream)
    stream = torch.cuda.Stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        t_jit = time.perf_counter()
        call(0)                                    # JIT compile / cache load, never timed
        torch.cuda.synchronize()
        t_jit = time.perf_counter() - t_jit
        for i in range(warmup):
            call(i)
        torch.cuda.synchronize()
        g = None
        if graph:
            # all K steps captured into one graph (one call per step, walking the
            # input copies in order); one untimed replay uploads it
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(steps):
                    call(i)
            t_up = time.perf_counter()
            g.replay()
            torch.cuda.synchronize()
            t_up = time.perf_counter() - t_up
        # The part raises its clock over some tens of milliseconds of sustained
        # load: after an idle pause, 20 steps of 4096 x 7168 x 16384 timed 472,
        # 435, 404 and 401 us per step after 0, 1, 3 and 10 untimed replays.  So
        # where one replay takes a millisecond or more, the untimed replays go on
        # until the GPU has run WARM_S back to back.  A short timed region keeps
        # the single replay: after 60-90 ms of back-to-back short kernels, 20
        # steps of 64 x 2112 x 7168 (0.2 ms) now and then landed in a clock
        # transition (10.5 us per step became 13-18 us).  Either way the timed
        # region below is exactly the K steps.
        n_warm = max(0, math.ceil(WARM_S / t_up) - 1) if graph and t_up >= 1e-3 else 0
        for _ in range(n_warm):
            g.replay()
        torch.cuda.synchronize()
        # Timed region: the K calls back to back on this stream, one HIP event pair
        # (recorded on this stream) around all of them.
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        if graph:
            g.replay()
        else:
            for i in range(steps):
                call(i)
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kernel_ms = start.elapsed_time(end) / steps
        # Launch-by-launch samples: a spin kernel holds the stream while the host
        # enqueues the start event, the call and the end event, so each pair
        # times the call alone.  Inputs keep rotating over the copies.
        spin_us = int(min(20000, max(200, 3 * kernel_ms * 1e3)))
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(samples)]
        for i, (a, b) in enumerate(ev):
            _ok(plib, plib.dg_probe_spin(spin_us, sp))
            a.record(stream)
            call(i)
            b.record(stream)
        torch.cuda.synchronize()
        per_launch = [a.elapsed_time(b) * 1e3 for a, b in ev]
    del g
    t_kernel = kernel_ms * 1e-3
    peak = PEAK_BF16_TFLOPS if m["bf16"] else PEAK_FP4_TFLOPS if m["fp4x4"] else PEAK_FP8_TFLOPS
    ai = flops / nbytes
    bound = "mfma" if ai >= peak * 1e12 / (PEAK_HBM_GBS * 1e9) else "hbm"
    tflops = flops / t_kernel / 1e12
    gbs = nbytes / t_kernel / 1e9
    frac = (tflops / peak) if bound == "mfma" else (gbs / PEAK_HBM_GBS)
    return dict(peak=peak, flops=flops, bytes=nbytes, rows=rows, kernel=kernel, copies=copies,
                kernel_ms=kernel_ms, ms_per_step=wall * 1e3 / steps, wall_s=wall, tflops=tflops, gbs=gbs,
                bound=bound, frac=frac, jit_s=t_jit, step_tflops=flops / (wall / steps) / 1e12,
                median_us=statistics.median(per_launch), min_us=min(per_launch), samples=samples,
                spin_us=spin_us, untimed_replays=(1 + n_warm) if graph else 0)


def measured_peaks():
    """The part's reachable rates, from the library's probes (include/dg_probe.h)."""
    import torch
    plib = _probe_lib()
    stream = torch.cuda.Stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    out = {}
    with torch.cuda.stream(stream):
        # streaming read of 2 GiB (8x the Infinity Cache), best of several grids and runs
        nbytes = 2 << 30
        buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(3)
        sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
        best = 0.0
        for grid in (1024, 2048, 4096, 8192):
            for _ in range(3):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                _ok(plib, plib.dg_probe_spin(500, sp))
                a.record(stream)
                _ok(plib, plib.dg_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                                    ctypes.c_void_p(sink.data_ptr()), grid, sp))
                b.record(stream)
                torch.cuda.synchronize()
                best = max(best, nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
        out["hbm_read_gbs"] = round(best, 1)
        del buf
        # back-to-back FP8 MFMAs, one 8-wave workgroup per CU
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        fs = torch.zeros(cus * 4, dtype=torch.float32, device="cuda")
        iters = 4000
        best = 0.0
        for grid in (cus, 2 * cus):
            for _ in range(3):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                _ok(plib, plib.dg_probe_mfma_fp8(grid, iters, ctypes.c_void_p(fs.data_ptr()), sp))
                b.record(stream)
                torch.cuda.synchronize()
                fl = grid * 8 * 8 * iters * 65536.0
                best = max(best, fl / (a.elapsed_time(b) * 1e-3) / 1e12)
        out["mfma_fp8_tflops"] = round(best, 1)
        # empty kernel: 200 launches captured in one graph, replayed between one event pair
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(200):
                _ok(plib, plib.dg_probe_null(1, sp))
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        out["null_kernel_us"] = round(a.elapsed_time(b) * 1e3 / 200, 3)
        # the floor of the small dense shape (64 x 2112 x 7168): one launch that does
        # nothing but read its 15.9 MB of operands once, from 32 rotating copies (512 MB,
        # twice the Infinity Cache) so that each launch reads from HBM; launches
        # back-to-back in one graph, as the GEMM is timed
        small = 15_886_048                                   # bytes of A, B, the scales and D
        bufs = [torch.empty(small, dtype=torch.uint8, device="cuda").fill_(5) for _ in range(32)]
        best = None
        for grid in (512, 1024, 2048):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for t in bufs:
                    _ok(plib, plib.dg_probe_stream_read(ctypes.c_void_p(t.data_ptr()), small,
                                                        ctypes.c_void_p(sink.data_ptr()), grid, sp))
            g.replay()
            torch.cuda.synchronize()
            for _ in range(3):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                g.replay()
                b.record(stream)
                torch.cuda.synchronize()
                us = a.elapsed_time(b) * 1e3 / len(bufs)
                best = us if best is None else min(best, us)
        out["read_15.9MB_us"] = round(best, 3)
        del bufs
    return out


def host_overhead(p):
    """Host cost of one call on a warm shape, without synchronising: the raw C ABI
    through ctypes (less the cost of a ctypes call with the same arguments to a C
    function that does nothing), the HIP runtime's own cost of launching an empty
    kernel (less a ctypes call without arguments) and the Python binding."""
    import torch

    import moe_grouped_gemm_scales_amd as dg
    import moe_grouped_gemm_scales_amd.dg as dgm
    from tests.gpu_util import out_shape, to_dev
    lib = dgm.lib
    d = to_dev(p)
    D = torch.empty(out_shape(p), dtype=torch.bfloat16, device="cuda")
    v = lambda t: ctypes.c_void_p(None if t is None else t.data_ptr())
    args = (v(d["A"]), v(d["sfa"]), v(d["B"]), v(d["sfb"]), v(d["C"]), v(D), ctypes.c_int(p.M),
            ctypes.c_int(p.N), ctypes.c_int(p.K), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    n = 200
    assert lib.dg_fp8_gemm_nt(*args) == 0
    torch.cuda.synchronize()

    def per_call(fn):
        best = float("inf")
        for _ in range(5):
            t = time.perf_counter()
            for _ in range(n):
                fn()
            best = min(best, (time.perf_counter() - t) / n)
            torch.cuda.synchronize()
        return best * 1e6

    c_abi = per_call(lambda: lib.dg_fp8_gemm_nt(*args))
    # a call with the same arguments that does nothing: ctypes' cost of passing them
    trivial = per_call(lambda: lib.dg_probe_call_floor(*args))
    binding = per_call(lambda: dg.dg_fp8_gemm_nt(d["A"], d["sfa"], d["B"], d["sfb"], d["C"], D))
    # the HIP runtime's own cost of one kernel launch: an empty kernel through the same ctypes path
    plib = _probe_lib()
    launch = per_call(lambda: plib.dg_probe_null(1, args[-1]))
    bare = per_call(lambda: lib.dg_get_mk_alignment_for_contiguous_layout())
    return dict(c_abi_us=round(c_abi - trivial, 3), ctypes_floor_us=round(trivial, 3),
                hip_launch_us=round(launch - bare, 3), python_binding_us=round(binding, 3),
                shape=f"{p.M}x{p.N}x{p.K}")


def library_reference(steps: int = 20):
    """Context for the large dense shape: torch._scaled_mm (hipBLASLt on ROCm) on
    4096 x 7168 x 16384 E4M3 operands with ONE scale per tensor, i.e. without the
    fine-grained block scales and their promotion; not the same operation."""
    import torch
    M, N, K = 4096, 7168, 16384
    g = torch.Generator(device="cpu").manual_seed(7)
    a = (torch.randn(M, K, generator=g) * 0.5).to(torch.float8_e4m3fn).to("cuda")
    b = (torch.randn(N, K, generator=g) * 0.5).to(torch.float8_e4m3fn).to("cuda")
    one = torch.ones((), dtype=torch.float32, device="cuda")
    f = lambda: torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
    for _ in range(3):
        f()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        f()
    e.record()
    torch.cuda.synchronize()
    us = s.elapsed_time(e) * 1e3 / steps
    return dict(library="torch._scaled_mm (hipBLASLt), per-tensor scales", shape=f"{M}x{N}x{K}",
                kernel_us=round(us, 3), tflops=round(2.0 * M * N * K / (us * 1e-6) / 1e12, 1))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(p, budget_s: float = 20.0):
    """The oracle, as it stands, on this host's cores: the full workload when it
    fits the budget, else evenly spaced rows of it, scaled to the whole."""
    import numpy as np

    from oracle import Oracle
    from tests.gpu_util import oracle_rows

    o = Oracle()
    total_rows = p.A.shape[0] * p.A.shape[1] if p.kind == "masked" else p.M
    # probe with a few rows per thread to size the sample
    probe = np.arange(min(total_rows, 2 * o.threads()))
    t = time.perf_counter()
    oracle_rows(o, p, rows=probe)
    per_row = (time.perf_counter() - t) / len(probe)
    n = int(min(total_rows, max(len(probe), budget_s / max(per_row, 1e-9))))
    rows = np.linspace(0, total_rows - 1, n).astype(np.int64)
    # repeat the sample until about half the budget has been spent (at least once)
    reps, dt, computed = 0, 0.0, 0
    while reps == 0 or dt < 0.5 * budget_s:
        t = time.perf_counter()
        _, comp = oracle_rows(o, p, rows=rows)
        dt += time.perf_counter() - t
        computed += int(comp.sum())
        reps += 1
    flops = 2.0 * computed * p.N * p.K
    desc = ("full problem" if n == total_rows else f"{n} of {total_rows} rows, evenly spaced") + \
        f" x {reps}, {dt:.1f} s, FP64 exact block sums"
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOPS", cores=o.threads(), kind="oracle",
                sample=desc, cpu_model=cpu_model())


def traffic_for(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source and the same plan."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash() or rec.get("kernel") != kernel:
        return None
    return rec.get("hbm_bytes_per_launch")


def workload_name(cfg, mode="") -> str:
    from tests import gen
    return {**gen.WORKLOAD_NAMES, **gen.WORKLOAD_NAMES_EXTRA}[cfg] + mode


def shape_line(cfg, mode, r, peaks):
    line = dict(per_shape=True, workload=workload_name(cfg, mode), kernel=r["kernel"],
                kernel_us=round(r["kernel_ms"] * 1e3, 3), median_us=round(r["median_us"], 3),
                min_us=round(r["min_us"], 3), samples=r["samples"], tflops=round(r["tflops"], 2),
                hbm_gbs=round(r["gbs"], 1), bound=r["bound"], roofline_frac=round(r["frac"], 4),
                step_us=round(r["ms_per_step"] * 1e3, 3), rows=r["rows"], copies=r["copies"])
    if peaks and r["peak"] == PEAK_FP8_TFLOPS:
        meas = peaks["mfma_fp8_tflops"] if r["bound"] == "mfma" else peaks["hbm_read_gbs"]
        line["frac_of_measured_peak"] = round((r["tflops"] if r["bound"] == "mfma" else r["gbs"]) / meas, 4)
    return line


def steps_for(cfg, steps):
    """Timed steps and launch samples: the long shapes get fewer of both."""
    long = cfg in (2, 3, "kg")
    return (max(5, steps // 4) if long else steps), (10 if long else 50)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=str(HEADLINE),
                    help="headline workload: 0, 1, 1c, 2, 3, 4 or kg (the K-grouped weight gradient of 3); "
                         "default 3, the largest")
    ap.add_argument("--no-per-shape", action="store_true", help="skip the per-shape lines before the headline")
    ap.add_argument("--all", action="store_true",
                    help="per-shape lines also for packed UE8M0 scales, FP8 x FP4, BF16, FP4 x FP4 and K-grouped")
    ap.add_argument("--ue8m0", action="store_true",
                    help="time the headline workload with packed UE8M0 scales instead of FP32 ones")
    ap.add_argument("--fp4", action="store_true",
                    help="time the headline workload as FP8 x FP4 (E2M1 B with 1x32 UE8M0 scales)")
    ap.add_argument("--fp4x4", action="store_true",
                    help="time the headline workload as FP4 x FP4 (E2M1 A and B, 1x32 UE8M0 scales)")
    ap.add_argument("--bf16", action="store_true",
                    help="time the chosen dense workload as an unscaled BF16 GEMM")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from Python instead of replaying a captured HIP graph")
    ap.add_argument("--copy-kernel", action="store_true",
                    help="only run a plain 256 MiB device copy (calibrates rocprofv3 byte counters)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the probe measurements (streaming read, MFMA)")
    ap.add_argument("--no-host", action="store_true", help="skip the host-overhead measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--library-reference", action="store_true",
                    help="only time torch._scaled_mm (hipBLASLt, per-tensor scales) on 4096 x 7168 x 16384")
    ap.add_argument("--out", default=None, help="also write all lines as JSON here")
    args = ap.parse_args()

    if args.copy_kernel:
        import torch
        x = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_kernel_bytes_read": 256 << 20, "copy_kernel_bytes_written": 256 << 20,
                          "launches": 3}))
        return

    if args.library_reference:
        print(json.dumps(library_reference(args.steps)), flush=True)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)

    cfg = args.workload if args.workload in ("1c", "kg") else int(args.workload)
    mode = "_fp4" if args.fp4 else "_fp4x4" if args.fp4x4 else "_ue8m0" if args.ue8m0 else \
        "_bf16" if args.bf16 else ""
    peaks = None if args.no_peaks else measured_peaks()
    if peaks:
        print(json.dumps(dict(per_shape=True, measured_peaks=peaks)), flush=True)
    lines = []
    shapes = [] if args.no_per_shape else [(c, "") for c in PER_SHAPE if (c, "") != (cfg, mode)]
    if args.all:
        shapes += [(c, "_ue8m0") for c in [0, 1, 2, 3, 4]] + [(c, "_fp4") for c in [0, 1, "1c", 2, 3, 4]] + \
            [("kg", ""), (2, "_bf16")] + [(c, "_fp4x4") for c in [1, 2, 4]]
    for c, md in shapes:
        st, ns = steps_for(c, args.steps)
        pc = make_problem(c, md)
        r = bench_workload(pc, st, min(args.warmup, st), ns, not args.eager, md)
        line = shape_line(c, md, r, peaks)
        lines.append(line)
        print(json.dumps(line), flush=True)
        del r, pc
        torch.cuda.empty_cache()

    p = make_problem(cfg, mode)
    _, nsamp = steps_for(cfg, args.steps)
    r = bench_workload(p, args.steps, args.warmup, nsamp, not args.eager, mode)
    torch.cuda.empty_cache()
    name = workload_name(cfg, mode)
    roof = dict(bound=r["bound"],
                achieved=round(r["tflops"] if r["bound"] == "mfma" else r["gbs"], 3),
                peak=r["peak"] if r["bound"] == "mfma" else PEAK_HBM_GBS,
                unit="TFLOP/s" if r["bound"] == "mfma" else "GB/s",
                frac=round(r["frac"], 4),
                traffic=traffic_for(name, r["kernel"]))
    if peaks and r["peak"] == PEAK_FP8_TFLOPS:
        meas = peaks["mfma_fp8_tflops"] if r["bound"] == "mfma" else peaks["hbm_read_gbs"]
        roof["measured_peak"] = meas
        roof["frac_of_measured_peak"] = round(roof["achieved"] / meas, 4)
    host = None
    if not args.no_host:
        from tests import gen
        host = host_overhead(gen.make_workload(0))
    alt = bool(mode) or cfg == "kg"
    cpu = None if (args.no_cpu_baseline or alt) else cpu_baseline(p)
    value = r["step_tflops"]
    pages = PAGES_TFLOPS.get(cfg) if isinstance(cfg, int) and not alt else None
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / pages, 4) if pages else None,
        "dtype": "fp8_e4m3 x fp4_e2m1" if args.fp4 else "fp4_e2m1" if args.fp4x4 else "bf16" if args.bf16
        else "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": name, "kind": p.kind, "M": p.M if p.kind == "k_grouped" else p.A.shape[-2],
                   "N": p.N, "K": p.K, "groups": p.G, "with_c": p.C is not None, "kernel": r["kernel"],
                   "input_copies": r["copies"], "hip_graph": bool(not args.eager)},
        "kernel_us": round(r["kernel_ms"] * 1e3, 3),
        "kernel_median_us": round(r["median_us"], 3),
        "kernel_min_us": round(r["min_us"], 3),
        "kernel_samples": r["samples"],
        "untimed_replays": r["untimed_replays"],
        "kernel_tflops": round(r["tflops"], 3),
        "hbm_gbs": round(r["gbs"], 1),
        "roofline": roof,
        "measured_peaks": peaks,
        "host_us": host,
        "cpu_baseline": cpu,
    }
    if args.out:
        with open(args.out, "w") as f:
            json.dump(dict(main=out, per_shape=lines, measured_peaks=peaks), f, indent=1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
