"""Helpers for GPU tests: move a generated problem to the device, run the
library on it with D prefilled by a sentinel, and bring the result back."""
from __future__ import annotations

import numpy as np
import torch

from tests import gen


def to_dev(p: gen.Problem, device="cuda"):
    f = lambda t: None if t is None else t.to(device)
    return dict(A=f(p.A), sfa=f(p.sfa), B=f(p.B), sfb=f(p.sfb), C=f(p.C),
                m_indices=f(p.m_indices), masked_m=f(p.masked_m))


def out_shape(p: gen.Problem):
    if p.kind == "masked":
        return (p.A.shape[0], p.A.shape[1], p.N)
    return (p.A.shape[0], p.N)


def run(p: gen.Problem, sentinel_seed: int = 12345, dev=None, D=None):
    """Run the problem through the library; returns (D on the CPU, sentinel on the CPU)."""
    import moe_grouped_gemm_scales_amd as dg
    dev = dev or to_dev(p)
    sent = gen.sentinel_like(out_shape(p), sentinel_seed)
    if D is None:
        D = sent.to("cuda")
    else:
        D.copy_(sent.to("cuda"))
    if p.ue8m0_pairs:
        if p.kind == "dense":
            dg.dg_fp8_gemm_nt_ue8m0_i16(dev["A"], dev["sfa"], dev["B"], dev["sfb"], dev["C"], D)
        elif p.kind == "contiguous":
            dg.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_i16(dev["A"], dev["sfa"], dev["B"], dev["sfb"],
                                                             dev["m_indices"], dev["C"], D)
        else:
            dg.dg_m_grouped_fp8_gemm_nt_masked_ue8m0_i16(dev["A"], dev["sfa"], dev["B"], dev["sfb"],
                                                         dev["masked_m"], dev["C"], D)
    elif p.bf16:
        if p.kind == "dense":
            dg.dg_bf16_gemm_nt(dev["A"], dev["B"], dev["C"], D)
        elif p.kind == "contiguous":
            dg.dg_m_grouped_bf16_gemm_nt_contiguous(dev["A"], dev["B"], dev["m_indices"], dev["C"], D)
        else:
            dg.dg_m_grouped_bf16_gemm_nt_masked(dev["A"], dev["B"], dev["masked_m"], dev["C"], D)
    elif p.fp4a:
        if p.kind == "dense":
            dg.dg_fp4_fp4_gemm_nt(dev["A"], dev["sfa"], dev["B"], dev["sfb"], dev["C"], D)
        elif p.kind == "contiguous":
            dg.dg_m_grouped_fp4_fp4_gemm_nt_contiguous(dev["A"], dev["sfa"], dev["B"], dev["sfb"],
                                                       dev["m_indices"], dev["C"], D)
        else:
            dg.dg_m_grouped_fp4_fp4_gemm_nt_masked(dev["A"], dev["sfa"], dev["B"], dev["sfb"], dev["masked_m"],
                                                   dev["C"], D)
    elif p.fp4:
        if p.kind == "dense":
            dg.dg_fp8_fp4_gemm_nt(dev["A"], dev["sfa"], dev["B"], dev["sfb"], dev["C"], D)
        elif p.kind == "contiguous":
            dg.dg_m_grouped_fp8_fp4_gemm_nt_contiguous(dev["A"], dev["sfa"], dev["B"], dev["sfb"],
                                                       dev["m_indices"], dev["C"], D)
        else:
            dg.dg_m_grouped_fp8_fp4_gemm_nt_masked(dev["A"], dev["sfa"], dev["B"], dev["sfb"], dev["masked_m"],
                                                   dev["C"], D)
    elif p.kind == "dense":
        dg.dg_fp8_gemm_nt(dev["A"], dev["sfa"], dev["B"], dev["sfb"], dev["C"], D)
    elif p.kind == "contiguous":
        dg.dg_m_grouped_fp8_gemm_nt_contiguous(dev["A"], dev["sfa"], dev["B"], dev["sfb"], dev["m_indices"],
                                               dev["C"], D)
    else:
        dg.dg_m_grouped_fp8_gemm_nt_masked(dev["A"], dev["sfa"], dev["B"], dev["sfb"], dev["masked_m"],
                                           dev["C"], D)
    torch.cuda.synchronize()
    return D.cpu(), sent


def oracle_rows(oracle, p: gen.Problem, rows=None, threads=0):
    """(reference FP64 [rows, N], computed mask [rows]) for flat row indices."""
    d = gen.to_numpy(p)
    if p.bf16:        # unscaled BF16 GEMM
        gi = {"dense": None, "contiguous": d["m_indices"], "masked": d["masked_m"]}[p.kind]
        return oracle.bf16_gemm(p.kind, d["A"], d["B"], gi, d["C"], rows=rows, threads=threads)
    if p.fp4a:        # FP4 x FP4: both operands E2M1 with 1x32 UE8M0 scales per row
        gi = {"dense": None, "contiguous": d["m_indices"], "masked": d["masked_m"]}[p.kind]
        return oracle.fp4_fp4_gemm(p.kind, d["A"], d["sfa"], d["B"], d["sfb"], gi, d["C"], rows=rows,
                                   threads=threads)
    if p.fp4:         # FP8 x FP4: E2M1 B with 1x32 UE8M0 scales
        gi = {"dense": None, "contiguous": d["m_indices"], "masked": d["masked_m"]}[p.kind]
        ref, comp = oracle.fp8_fp4_gemm(p.kind, d["A"], d["sfa"], d["B"], d["sfb"], gi, d["C"], rows=rows,
                                        threads=threads)
        return ref, comp
    if p.ue8m0:       # packed UE8M0 scales: the oracle unpacks them to the FP32 scales they stand for
        Kb = p.K // 128
        d["sfa"] = oracle.unpack_sfa_ue8m0(d["sfa"], Kb)
        d["sfb"] = oracle.unpack_sfb_ue8m0(d["sfb"], Kb)
    if p.ue8m0_pairs:  # UE8M0 pairs in int16, MN-major: the same, from the pair packing
        Kb = p.K // 128
        d["sfa"] = oracle.unpack_sfa_ue8m0_pairs(d["sfa"], Kb)
        d["sfb"] = oracle.unpack_sfb_ue8m0_pairs(d["sfb"], Kb)
    if p.kind == "dense":
        ref = oracle.fp8_gemm_nt(d["A"], d["sfa"], d["B"], d["sfb"], d["C"], rows=rows, threads=threads)
        return ref, np.ones(ref.shape[0], dtype=bool)
    if p.kind == "contiguous":
        return oracle.m_grouped_contiguous(d["A"], d["sfa"], d["B"], d["sfb"], d["m_indices"], d["C"],
                                           rows=rows, threads=threads)
    return oracle.m_grouped_masked(d["A"], d["sfa"], d["B"], d["sfb"], d["masked_m"], d["C"],
                                   rows=rows, threads=threads)


def flat_rows(D: torch.Tensor) -> torch.Tensor:
    return D.reshape(-1, D.shape[-1])


def sample_rows(total: int, count: int, block: int = 128, seed: int = 0) -> np.ndarray:
    """Rows spread over the whole range, always including both ends and tile edges."""
    rng = np.random.default_rng(seed)
    must = {0, total - 1}
    for b in range(block, total, block * max(1, total // (block * 8))):
        must.update({b - 1, b})
    rows = set(int(r) for r in must if 0 <= r < total)
    while len(rows) < min(count, total):
        rows.add(int(rng.integers(0, total)))
    return np.array(sorted(rows), dtype=np.int64)
