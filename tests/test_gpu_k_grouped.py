"""GPU parity of the K-grouped TN GEMM (MoE weight backward) against the CPU oracle,
through the C ABI.

Bar as for the other forms: |D - ref| <= 2^-7 |ref| + 1e-3 rms(ref) per element,
with every (group, row) computed; bitwise where the exact result is a BF16
number (integer data with power-of-two scales).
"""
import numpy as np
import pytest
import torch

from tests import check, gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def run_kg(p: gen.KGroupedProblem, sentinel_seed: int = 321):
    import moe_grouped_gemm_scales_amd as dg
    f = lambda t: None if t is None else t.to("cuda")
    D = gen.sentinel_like((p.G, p.M, p.N), sentinel_seed).to("cuda")
    dg.dg_k_grouped_fp8_gemm_tn_contiguous(f(p.A), f(p.sfa), f(p.B), f(p.sfb), f(p.ks), f(p.C), D)
    torch.cuda.synchronize()
    return D.cpu()


def compare(oracle, p, D, rows=None, what=""):
    ref, comp = oracle.k_grouped_tn(p.A, p.sfa, p.B, p.sfb, p.ks, p.C, rows=rows)
    assert comp.all()
    Df = D.reshape(-1, p.N)
    idx = np.arange(Df.shape[0]) if rows is None else rows
    got = check.bf16_to_f64(Df[torch.as_tensor(idx)])
    check.assert_close(got, ref, what)
    return ref


KG_SHAPES = [([128, 256, 0, 384], 37, 129, True), ([512], 1, 5, False), ([0, 128], 130, 64, False),
             ([128] * 8, 256, 256, True), ([1024, 2048, 512], 300, 520, True), ([256, 0, 0], 64, 2112, False)]


@pytest.mark.parametrize("ks,M,N,with_c", KG_SHAPES)
def test_k_grouped_small(oracle, ks, M, N, with_c):
    p = gen.make_k_grouped(ks, M, N, seed=sum(ks) + M + N + 3, with_c=with_c)
    D = run_kg(p)
    compare(oracle, p, D, what=f"k-grouped {ks} {M}x{N}")


def test_k_grouped_empty_groups_write_c(oracle):
    """A group with no K rows still owns its output: D[g] = bf16(C[g]) (zeros without C)."""
    p = gen.make_k_grouped([0, 256, 0], 70, 96, seed=7, with_c=True)
    D = run_kg(p)
    ref = compare(oracle, p, D, what="k-grouped empty groups")
    for g in (0, 2):
        got = check.bf16_bits(D[g])
        assert np.array_equal(got, oracle.bf16_rne(ref.reshape(3, 70, 96)[g]).reshape(70, 96))


def test_k_grouped_integer_data_bitwise(oracle):
    g = torch.Generator().manual_seed(17)
    ks, M, N = [384, 128, 512], 96, 200
    K = sum(ks)
    A = gen.integer_codes((K, M), g, max_abs=8)
    B = gen.integer_codes((K, N), g, max_abs=8)
    sfa = gen.pow2_scales((K // 128, M), g, lo=-2, hi=2)
    sfb = gen.pow2_scales((K // 128, N), g, lo=-2, hi=2)
    p = gen.KGroupedProblem(A, sfa, B, sfb, torch.tensor(ks, dtype=torch.int32))
    D = run_kg(p)
    ref, _ = oracle.k_grouped_tn(p.A, p.sfa, p.B, p.sfb, p.ks)
    assert np.array_equal(check.bf16_bits(D.reshape(-1, N)), oracle.bf16_rne(ref).reshape(-1, N))


@pytest.mark.parametrize("forced", ["128,128,4,2,2,1,1,0", "64,96,2,2,4,1,1,0", "256,256,4,2,2,1,1,0",
                                    "32,64,1,2,3,1,1,0", "192,256,4,2,2,1,1,0", "128,256,4,2,3,1,1,0",
                                    "192,256,4,2,2,1,1,6", "128,256,4,2,2,1,1,6"])     # split refill
def test_k_grouped_forced_tile_configs(oracle, monkeypatch, forced):
    monkeypatch.setenv("DG_FORCE_CONFIG", forced)
    p = gen.make_k_grouped([256, 0, 640], 300, 520, seed=19, with_c=True)
    D = run_kg(p)
    compare(oracle, p, D, what=f"k-grouped forced {forced}")


def test_k_grouped_unaligned_count_leaves_earlier_groups_exact(oracle):
    """A count that is not a multiple of 128 makes that group and the later ones
    undefined; the call still succeeds and the groups before it are exact."""
    p = gen.make_k_grouped([128, 128, 128], 40, 72, seed=23)
    bad = gen.KGroupedProblem(p.A, p.sfa, p.B, p.sfb, torch.tensor([128, 100, 156], dtype=torch.int32))
    D = run_kg(bad)
    ref, _ = oracle.k_grouped_tn(p.A, p.sfa, p.B, p.sfb, torch.tensor([128, 0, 0], dtype=torch.int32))
    check.assert_close(check.bf16_to_f64(D[0]), ref[:40], "group before the bad count")


def test_k_grouped_workload_full_size(oracle):
    """The weight gradient of the contiguous workload: 4 experts x 8192 tokens,
    M = 4096, N = 7168 (every element of every group)."""
    p = gen.make_k_grouped([8192] * 4, 4096, 7168, seed=1005)
    D = run_kg(p)
    compare(oracle, p, D, what="k-grouped 4x8192 x 4096x7168")


def test_graph_replays_of_newer_forms_match_eager():
    """K-grouped (its rewrite pass included), FP8 x FP4 masked and BF16 contiguous calls
    captured into one HIP graph give the eager bits on every replay, with eager work
    (which reuses the same rewrite buffer) between replays."""
    import moe_grouped_gemm_scales_amd as dg
    from tests.gpu_util import to_dev
    pk = gen.make_k_grouped([256, 0, 384], 200, 136, seed=31, with_c=True)
    pf = gen.make_masked(2, 128, 200, 512, seed=32, masked_m=[100, 7], fp4=True)
    pb = gen.make_bf16("contiguous", seed=33, N=96, K=256, group_rows=[128, 50])
    c = lambda t: None if t is None else t.to("cuda")
    k = dict(A=c(pk.A), sfa=c(pk.sfa), B=c(pk.B), sfb=c(pk.sfb), ks=c(pk.ks), C=c(pk.C))
    f, b = to_dev(pf), to_dev(pb)

    def calls(Dk, Df, Db):
        dg.dg_k_grouped_fp8_gemm_tn_contiguous(k["A"], k["sfa"], k["B"], k["sfb"], k["ks"], k["C"], Dk)
        dg.dg_m_grouped_fp8_fp4_gemm_nt_masked(f["A"], f["sfa"], f["B"], f["sfb"], f["masked_m"], None, Df)
        dg.dg_m_grouped_bf16_gemm_nt_contiguous(b["A"], b["B"], b["m_indices"], None, Db)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        outs_e = (torch.empty(3, 200, 136, dtype=torch.bfloat16, device="cuda"),
                  gen.sentinel_like((2, 128, 200), 5).to("cuda"),
                  gen.sentinel_like((pb.M, 96), 6).to("cuda"))
        calls(*outs_e)
        torch.cuda.synchronize()
        outs_g = (torch.empty_like(outs_e[0]), gen.sentinel_like((2, 128, 200), 5).to("cuda"),
                  gen.sentinel_like((pb.M, 96), 6).to("cuda"))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            calls(*outs_g)
        for rep in range(3):
            outs_g[0].zero_()
            g.replay()
            torch.cuda.synchronize()
            for i, (x, y) in enumerate(zip(outs_g, outs_e)):
                assert torch.equal(x.view(torch.int16), y.view(torch.int16)), f"output {i}, replay {rep}"
            calls(*outs_e)       # eager work between replays
            torch.cuda.synchronize()


def test_graph_survives_workspace_growth(monkeypatch):
    """A graph captures a K-grouped call (rewrite buffer) and a split-K call (partials);
    larger eager calls on the same stream then grow both workspaces; every replay of
    the graph still gives the eager bits (outgrown buffers stay allocated)."""
    import os
    import moe_grouped_gemm_scales_amd as dg
    from tests.gpu_util import to_dev
    c = lambda t: None if t is None else t.to("cuda")
    small = gen.make_k_grouped([128, 256], 64, 80, seed=51)
    large = gen.make_k_grouped([2048, 2048], 512, 640, seed=52)
    ps = gen.make_dense(64, 2112, 7168, seed=53)          # split-K 7: 3.8 MB of partials
    pl = gen.make_dense(1024, 2112, 8192, seed=54)        # split-K 8 forced below: 71 MB
    ds, dl = to_dev(ps), to_dev(pl)
    ks = {k: c(getattr(small, k)) for k in ("A", "sfa", "B", "sfb", "ks")}
    kl = {k: c(getattr(large, k)) for k in ("A", "sfa", "B", "sfb", "ks")}
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Ke = torch.empty(2, 64, 80, dtype=torch.bfloat16, device="cuda")
        De = torch.empty(64, 2112, dtype=torch.bfloat16, device="cuda")
        dg.dg_k_grouped_fp8_gemm_tn_contiguous(ks["A"], ks["sfa"], ks["B"], ks["sfb"], ks["ks"], None, Ke)
        dg.dg_fp8_gemm_nt(ds["A"], ds["sfa"], ds["B"], ds["sfb"], None, De)
        torch.cuda.synchronize()
        Kg, Dg = torch.empty_like(Ke), torch.empty_like(De)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            dg.dg_k_grouped_fp8_gemm_tn_contiguous(ks["A"], ks["sfa"], ks["B"], ks["sfb"], ks["ks"], None, Kg)
            dg.dg_fp8_gemm_nt(ds["A"], ds["sfa"], ds["B"], ds["sfb"], None, Dg)
        KL = torch.empty(2, 512, 640, dtype=torch.bfloat16, device="cuda")
        DL = torch.empty(1024, 2112, dtype=torch.bfloat16, device="cuda")
        for rep in range(2):
            # larger calls on the same stream: the rewrite buffer and the partials grow
            dg.dg_k_grouped_fp8_gemm_tn_contiguous(kl["A"], kl["sfa"], kl["B"], kl["sfb"], kl["ks"], None, KL)
            monkeypatch.setenv("DG_FORCE_CONFIG", "128,128,4,2,2,8,1,0")
            dg.dg_fp8_gemm_nt(dl["A"], dl["sfa"], dl["B"], dl["sfb"], None, DL)
            monkeypatch.delenv("DG_FORCE_CONFIG")
            Kg.zero_(); Dg.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(Kg.view(torch.int16), Ke.view(torch.int16)), f"k-grouped replay {rep}"
            assert torch.equal(Dg.view(torch.int16), De.view(torch.int16)), f"split-K replay {rep}"
            assert os.environ.get("DG_FORCE_CONFIG") is None
