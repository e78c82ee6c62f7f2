#!/usr/bin/env python3
"""Benchmark of the block-scaled FP8 GEMM hot path on one MI355X.

One step = one library call (the whole hot path: dispatch, staging, FP8 MFMA,
promotion, BF16 epilogue) on one batch of seeded synthetic input that is
already resident in HBM.  The default workload is the dense 128 x 24576 x 1536
GEMM (a shape of the DeepGEMM launch article's section 3 table); --workload
picks another of the five, --all runs every one of them and prints one line
per shape on stderr.

Metric (as the pages quote it): TFLOPS = 2 M N K / t and HBM GB/s =
(|A| + |B| + |D| [+ |C|] + scales) / t with 1-byte A/B and 2-byte D, t the
kernel time; the roofline fraction is the bound resource's share of the
MI355X peak (8 TB/s HBM, 5.0 PFLOP/s dense FP8).

HBM honesty: inputs are rotated over enough copies that the working set of a
cycle exceeds 512 MB, twice the 256 MB Infinity Cache, so every step reads its
operands from HBM, not from the cache.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
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
# The pages' H800 numbers for the same shapes (DeepGEMM launch article,
# section 3 dense table): other hardware, context only.
PAGES_TFLOPS = {0: 206.0, 1: 535.0, 2: 1358.0}
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


def bench_workload(cfg, steps: int, warmup: int, graph: bool, ue8m0: bool = False, fp4: bool = False,
                   bf16: bool = False, fp4x4: bool = False):
    import torch

    import moe_grouped_gemm_scales_amd as dg
    from tests import gen
    from tests.gpu_util import out_shape, to_dev

    if cfg == "kg":
        p = gen.make_k_grouped_workload()
    elif bf16:
        c = gen.WORKLOADS[cfg]
        assert c["kind"] == "dense", "the BF16 bench covers the dense workloads"
        p = gen.make_bf16("dense", seed=gen.workload_seed(cfg), M=c["M"], N=c["N"], K=c["K"],
                          with_c=c.get("with_c", False))
    else:
        p = gen.make_workload(cfg, ue8m0=ue8m0, fp4=fp4, fp4x4=fp4x4)
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
        elif bf16:
            dg.dg_bf16_gemm_nt(d["A"], d["B"], d["C"], D)
        elif fp4x4:
            if p.kind == "dense":
                dg.dg_fp4_fp4_gemm_nt(d["A"], d["sfa"], d["B"], d["sfb"], d["C"], D)
            elif p.kind == "contiguous":
                dg.dg_m_grouped_fp4_fp4_gemm_nt_contiguous(d["A"], d["sfa"], d["B"], d["sfb"], d["m_indices"],
                                                           d["C"], D)
            else:
                dg.dg_m_grouped_fp4_fp4_gemm_nt_masked(d["A"], d["sfa"], d["B"], d["sfb"], d["masked_m"], d["C"],
                                                       D)
        elif fp4:
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
    flag = dg.KIND_BF16 if bf16 else dg.SCALE_FP4_FP4 if fp4x4 else dg.SCALE_FP8_FP4 if fp4 else \
        (dg.SCALE_UE8M0 if ue8m0 else 0)
    kernel = dg.describe_config(kind_id(p.kind) | flag, rows_arg, p.N, p.K, p.G,
                                p.C is not None)
    # everything runs on one non-default stream (HIP graphs cannot capture the null stream)
    stream = torch.cuda.Stream()
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
            # all K steps captured into one graph (one kernel node per step, walking
            # the input copies in order); one untimed replay uploads it
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(steps):
                    call(i)
            g.replay()
            torch.cuda.synchronize()
        n_launch = steps
        # Timed region: the K launches back to back on this stream, one HIP event
        # pair around all of them (per-launch event pairs would add the dispatch
        # cost of every event to every kernel).
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
    kernel_ms = start.elapsed_time(end) / n_launch
    ms_per_step = wall * 1e3 / n_launch
    t_kernel = kernel_ms * 1e-3
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP4_TFLOPS if fp4x4 else PEAK_FP8_TFLOPS
    ai = flops / nbytes
    bound = "mfma" if ai >= peak * 1e12 / (PEAK_HBM_GBS * 1e9) else "hbm"
    tflops = flops / t_kernel / 1e12
    gbs = nbytes / t_kernel / 1e9
    frac = (tflops / peak) if bound == "mfma" else (gbs / PEAK_HBM_GBS)
    return dict(problem=p, peak=peak, flops=flops, bytes=nbytes, rows=rows, kernel=kernel, copies=copies,
                kernel_ms=kernel_ms, ms_per_step=ms_per_step, wall_s=wall, tflops=tflops, gbs=gbs,
                bound=bound, frac=frac, jit_s=t_jit, step_tflops=flops / (ms_per_step * 1e-3) / 1e12)


def cpu_baseline(cfg, budget_s: float = 20.0):
    """The oracle, as it stands, on this host's cores: the full workload when it
    fits the budget, else a row sample scaled to the whole."""
    import numpy as np

    from oracle import Oracle
    from tests import gen
    from tests.gpu_util import oracle_rows

    o = Oracle()
    p = gen.make_workload(cfg)
    flops_total, _, rows_total = algorithmic(p)
    total_rows = p.A.shape[0] * p.A.shape[1] if p.kind == "masked" else p.M
    # probe with a few rows to size the sample
    probe = np.arange(min(8, total_rows))
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
                sample=desc)


def traffic_for(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="1",
                    help="0, 1, 1c, 2, 3, 4 or kg (the K-grouped weight gradient of 3) (default 1)")
    ap.add_argument("--all", action="store_true",
                    help="also run every workload, one stderr line each (FP32 scales, packed UE8M0 scales, "
                         "then FP8 x FP4)")
    ap.add_argument("--ue8m0", action="store_true",
                    help="time the chosen workload with packed UE8M0 scales instead of FP32 ones")
    ap.add_argument("--fp4", action="store_true",
                    help="time the chosen workload as FP8 x FP4 (E2M1 B with 1x32 UE8M0 scales)")
    ap.add_argument("--fp4x4", action="store_true",
                    help="time the chosen workload as FP4 x FP4 (E2M1 A and B, 1x32 UE8M0 scales)")
    ap.add_argument("--bf16", action="store_true",
                    help="time the chosen dense workload as an unscaled BF16 GEMM")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from Python instead of replaying a captured HIP graph")
    ap.add_argument("--copy-kernel", action="store_true",
                    help="only run a plain 256 MiB device copy (calibrates rocprofv3 byte counters)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--out", default=None, help="also write the per-shape results as JSON here")
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

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    from tests import gen

    cfg = args.workload if args.workload in ("1c", "kg") else int(args.workload)
    per_shape = []
    if args.all:
        modes = [(c, "") for c in [0, 1, "1c", 2, 3, 4]] + [(c, "_ue8m0") for c in [0, 1, 2, 3, 4]] + \
            [(c, "_fp4") for c in [0, 1, "1c", 2, 3, 4]] + [("kg", ""), (2, "_bf16")] + \
            [(c, "_fp4x4") for c in [1, 2, 4]]
        for c, mode in modes:
            steps = args.steps if c in (0, 1, "1c", 4) else max(10, args.steps // 10)
            if c == "kg":
                steps = max(5, args.steps // 20)
            r = bench_workload(c, steps, min(args.warmup, steps), not args.eager, ue8m0=mode == "_ue8m0",
                               fp4=mode == "_fp4", bf16=mode == "_bf16", fp4x4=mode == "_fp4x4")
            wl = {**gen.WORKLOAD_NAMES, **gen.WORKLOAD_NAMES_EXTRA}[c] + mode
            line = dict(workload=wl, kernel=r["kernel"], kernel_us=round(r["kernel_ms"] * 1e3, 3),
                        tflops=round(r["tflops"], 2), hbm_gbs=round(r["gbs"], 1), bound=r["bound"],
                        roofline_frac=round(r["frac"], 4), step_us=round(r["ms_per_step"] * 1e3, 3),
                        rows=r["rows"], copies=r["copies"])
            per_shape.append(line)
            print(json.dumps(line), file=sys.stderr, flush=True)
            del r
            torch.cuda.empty_cache()

    r = bench_workload(cfg, args.steps, args.warmup, not args.eager, ue8m0=args.ue8m0, fp4=args.fp4, bf16=args.bf16,
                       fp4x4=args.fp4x4)
    p = r["problem"]
    name = {**gen.WORKLOAD_NAMES, **gen.WORKLOAD_NAMES_EXTRA}[cfg] + \
        ("_fp4" if args.fp4 else "_fp4x4" if args.fp4x4 else "_ue8m0" if args.ue8m0 else "_bf16" if args.bf16 else "")
    roof = dict(bound=r["bound"],
                achieved=round(r["tflops"] if r["bound"] == "mfma" else r["gbs"], 3),
                peak=r["peak"] if r["bound"] == "mfma" else PEAK_HBM_GBS,
                unit="TFLOP/s" if r["bound"] == "mfma" else "GB/s",
                frac=round(r["frac"], 4),
                traffic=traffic_for(name))
    alt = args.ue8m0 or args.fp4 or args.bf16 or args.fp4x4
    cpu = None if (args.no_cpu_baseline or alt or cfg == "kg") else cpu_baseline(cfg)
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
        "dtype": "fp8_e4m3 x fp4_e2m1" if args.fp4 else "fp4_e2m1" if args.fp4x4 else "bf16" if args.bf16 else "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": name, "kind": p.kind, "M": p.M if p.kind == "k_grouped" else p.A.shape[-2], "N": p.N, "K": p.K, "groups": p.G,
                   "with_c": p.C is not None, "kernel": r["kernel"], "input_copies": r["copies"],
                   "hip_graph": bool(not args.eager)},
        "kernel_us": round(r["kernel_ms"] * 1e3, 3),
        "kernel_tflops": round(r["tflops"], 3),
        "hbm_gbs": round(r["gbs"], 1),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if args.out:
        with open(args.out, "w") as f:
            json.dump(dict(main=out, per_shape=per_shape), f, indent=1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
