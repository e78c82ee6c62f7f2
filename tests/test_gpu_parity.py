"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Bar: every computed element within |D - ref| <= 2^-7 |ref| + 1e-3 rms(ref)
(tests/check.py); bitwise equality where the exact result is representable
(integer data with power-of-two scales, one-hot rows); rows the method does
not compute keep the sentinel bits they were prefilled with.
"""
import numpy as np
import pytest
import torch

from tests import check, gen
from tests.gpu_util import flat_rows, oracle_rows, run, sample_rows, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _compare(p, D, sent, ref, comp, rows=None, what=""):
    Df = flat_rows(D)
    Sf = flat_rows(sent)
    idx = np.arange(Df.shape[0]) if rows is None else rows
    if comp.any():
        # only the computed rows are widened (the sentinel rows are compared as bits)
        got = check.bf16_to_f64(Df[torch.as_tensor(idx[comp])])
        check.assert_close(got, ref[comp], what)
    if (~comp).any():
        untouched = idx[~comp]
        assert np.array_equal(check.bf16_bits(Df[torch.as_tensor(untouched)]),
                              check.bf16_bits(Sf[torch.as_tensor(untouched)])), f"{what}: a skipped row was written"


# ------------------------------------------------------------------ dense, small and ragged
DENSE_SHAPES = [
    (1, 16, 128, False),
    (5, 129, 384, True),
    (16, 64, 256, False),
    (64, 2112, 1024, False),
    (100, 300, 512, True),
    (128, 256, 1536, False),
    (257, 515, 640, True),
    (300, 1000, 2048, False),
]


@pytest.mark.parametrize("M,N,K,with_c", DENSE_SHAPES)
def test_dense_small(oracle, M, N, K, with_c):
    p = gen.make_dense(M, N, K, seed=M * 7 + N + K, with_c=with_c)
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    _compare(p, D, sent, ref, comp, what=f"dense {M}x{N}x{K}")


def test_dense_integer_data_bitwise(oracle):
    g = torch.Generator().manual_seed(77)
    M, N, K = 96, 400, 1024
    A = gen.integer_codes((M, K), g, max_abs=8)
    B = gen.integer_codes((N, K), g, max_abs=8)
    sfa = gen.pow2_scales((K // 128, M), g, -2, 2)
    sfb = gen.pow2_scales(((N + 127) // 128, K // 128), g, -2, 2)
    p = gen.Problem("dense", A, sfa, B, sfb)
    D, _ = run(p)
    ref, _ = oracle_rows(oracle, p)
    # every partial sum is an integer multiple of 2^-9 below 2^24 ulps: exact in FP32
    want = oracle.bf16_rne(ref).reshape(M, N)
    assert np.array_equal(check.bf16_bits(D), want)


def test_dense_one_hot_maps_lanes(oracle):
    """A[m, pi(m)] = 1 picks one column of B per row: checks row/column/lane mapping bitwise."""
    g = torch.Generator().manual_seed(5)
    M, N, K = 80, 272, 768
    pi = torch.randint(0, K, (M,), generator=g)
    A = torch.zeros(M, K, dtype=torch.uint8)
    A[torch.arange(M), pi] = gen.E4M3_ONE
    q = gen.make_dense(1, N, K, seed=99)
    sfa = gen.pow2_scales((K // 128, M), g)
    p = gen.Problem("dense", A, sfa, q.B, q.sfb)
    D, _ = run(p)
    ref, _ = oracle_rows(oracle, p)
    assert np.array_equal(check.bf16_bits(D), oracle.bf16_rne(ref).reshape(M, N))


def test_dense_repeatable_and_stream(oracle):
    p = gen.make_dense(64, 2112, 7168, seed=1000)
    dev = to_dev(p)
    D1, _ = run(p, dev=dev)
    D2, _ = run(p, dev=dev, sentinel_seed=1)
    assert torch.equal(D1.view(torch.int16), D2.view(torch.int16))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        D3, _ = run(p, dev=dev, sentinel_seed=2)
    assert torch.equal(D1.view(torch.int16), D3.view(torch.int16))


# ------------------------------------------------------------------ the five workloads at full size
@pytest.mark.parametrize("cfg", [0, 1, "1c", 2])
def test_workload_dense(oracle, cfg):
    """Every element of D at full size (4096 x 7168 x 16384: ~1 TFLOP of FP64 oracle work)."""
    p = gen.make_workload(cfg)
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    assert comp.all()
    _compare(p, D, sent, ref, comp, what=gen.WORKLOAD_NAMES[cfg])


def test_workload_contiguous(oracle):
    """Every element of the 4 x 8192 x 4096 x 7168 contiguous result (~1.9 TFLOP of oracle work)."""
    p = gen.make_workload(3)
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    assert comp.all()
    _compare(p, D, sent, ref, comp, what=gen.WORKLOAD_NAMES[3])


def test_workload_masked(oracle):
    p = gen.make_workload(4)
    D, sent = run(p)
    G, M_max = p.A.shape[0], p.A.shape[1]
    mm = p.masked_m.numpy().clip(0, M_max)
    rows = np.arange(G * M_max)          # all rows: cheap enough at K = 2048
    ref, comp = oracle_rows(oracle, p, rows=rows)
    assert comp.sum() == mm.sum()
    _compare(p, D, sent, ref, comp, rows=rows, what=gen.WORKLOAD_NAMES[4])


# ------------------------------------------------------------------ contiguous, 256-row blocks
@pytest.mark.parametrize("forced", ["256,256,4,2,2,1,1,0", "256,256,4,2,2,1,1,6", "256,128,4,2,3,1,1,6",
                                    "256,224,4,2,2,1,1,4"])
@pytest.mark.parametrize("group_rows,N,K,pad", [
    ([128, 384, 0, 256, 100], 300, 512, 128),    # blocks of 256 rows that hold two experts
    ([256, 256, 512], 520, 384, 0),              # every block one expert
    ([100, 1, 129], 96, 256, 128),               # padding and an odd tail (M = 512)
])
def test_contiguous_256_row_blocks(oracle, monkeypatch, forced, group_rows, N, K, pad):
    """Row blocks of 256 rows in the contiguous form: a block whose two 128-row halves
    name different experts is computed once for each, so every row gets its own
    expert's result; padding rows stay untouched."""
    monkeypatch.setenv("DG_FORCE_CONFIG", forced)
    for e8 in (False, True):
        p = gen.make_contiguous(group_rows, N, K, seed=sum(group_rows) + N + K, with_c=True, pad_rows=pad, ue8m0=e8)
        D, sent = run(p)
        ref, comp = oracle_rows(oracle, p)
        _compare(p, D, sent, ref, comp, what=f"contiguous {group_rows} {forced} ue8m0={e8}")


# ------------------------------------------------------------------ contiguous, edge cases
@pytest.mark.parametrize("group_rows,N,K,pad,with_c", [
    ([128, 0, 256, 100], 200, 256, 128, True),
    ([1, 127, 128, 129], 129, 384, 0, False),
    ([512], 512, 1024, 0, False),
    ([0, 0, 300], 96, 128, 256, True),
])
def test_contiguous_edges(oracle, group_rows, N, K, pad, with_c):
    p = gen.make_contiguous(group_rows, N, K, seed=sum(group_rows) + N, with_c=with_c, pad_rows=pad)
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    _compare(p, D, sent, ref, comp, what=f"contiguous {group_rows}")


def test_contiguous_groups_independent(oracle):
    p = gen.make_contiguous([256, 128, 128], 300, 512, seed=8)
    dev = to_dev(p)
    D1, _ = run(p, dev=dev)
    B2 = dev["B"].clone()
    B2[1] = torch.where(B2[1] != 0, B2[1] ^ 0x80, B2[1])
    dev2 = dict(dev, B=B2)
    D2, _ = run(p, dev=dev2)
    idx = p.m_indices
    assert torch.equal(D1.view(torch.int16)[idx != 1], D2.view(torch.int16)[idx != 1])
    # flipping the sign of every code of B[1] negates its rows exactly (RNE is sign-symmetric)
    assert torch.equal(D1.view(torch.int16)[idx == 1] ^ torch.tensor(-32768, dtype=torch.int16),
                       D2.view(torch.int16)[idx == 1]) or torch.equal(
        (-D1.float())[idx == 1], D2.float()[idx == 1])


@pytest.mark.parametrize("forced", [None, "128,128,4,2,2,1,1,0", "64,96,2,2,4,1,1,0", "32,64,1,2,3,1,1,0",
                                    "256,256,4,2,2,1,1,0", "256,128,4,2,3,1,1,6"])
def test_contiguous_mixed_blocks_never_use_another_experts_weights(oracle, monkeypatch, forced):
    """Aligned blocks that break the layout (rows naming another expert inside a
    block, a block that starts with a padding row): whatever the tile size, every
    row is either left untouched or holds its result for its own expert, padding
    rows are untouched, and the blocks that keep the layout are computed in full."""
    if forced:
        monkeypatch.setenv("DG_FORCE_CONFIG", forced)
    p = gen.make_contiguous([128, 128, 128], 160, 256, seed=61)
    idx = p.m_indices.clone()
    idx[40:60] = 2           # block 0 (expert 0) holds rows naming expert 2
    idx[128] = -1            # block 1 starts with a padding row; rows 129.. still name expert 1
    q = gen.Problem("contiguous", p.A, p.sfa, p.B, p.sfb, m_indices=idx)
    D, sent = run(q)
    ref, comp = oracle_rows(oracle, q)            # every row with a valid index, for its own expert
    got, bits, sbits = check.bf16_to_f64(D), check.bf16_bits(D), check.bf16_bits(sent)
    untouched = (bits == sbits).all(axis=1)
    assert untouched[~comp].all(), "a padding row was written"
    written = comp & ~untouched
    check.assert_close(got[written], ref[written], f"contiguous, mixed blocks ({forced or 'default plan'})")
    assert written[256:].all(), "the block that keeps the layout was not computed in full"


# ------------------------------------------------------------------ masked, edge cases
@pytest.mark.parametrize("masked_m", [[0, 0, 0], [96, 96, 96], [-3, 200, 17], [1, 95, 48]])
def test_masked_edges(oracle, masked_m):
    p = gen.make_masked(3, 96, 333, 512, seed=len(masked_m) + sum(masked_m), with_c=True, masked_m=masked_m)
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    _compare(p, D, sent, ref, comp, what=f"masked {masked_m}")


def test_masked_full_equals_dense(oracle):
    p = gen.make_masked(2, 128, 256, 384, seed=9, masked_m=[128, 128])
    D, _ = run(p)
    for g in range(2):
        q = gen.Problem("dense", p.A[g], p.sfa[g], p.B[g], p.sfb[g])
        Dg, _ = run(q)
        assert torch.equal(D[g].view(torch.int16), Dg.view(torch.int16))


# ------------------------------------------------------------------ tile configurations
FORCED = [
    "16,16,1,1,2,1",
    "32,64,1,2,3,2",
    "64,96,2,2,4,1",
    "64,112,1,1,2,4",
    "128,128,2,2,2,1",
    "128,256,2,4,2,1",
    "256,224,4,2,2,1",
    "256,256,4,2,2,1",
    "128,96,2,2,2,1,2",
    "64,64,2,2,3,2,2",
    "32,128,1,4,2,4,2",
    # variant 1: B straight into VGPRs (fields 7-8: kstep 1, variant 1)
    "128,128,1,8,9,1,1,1",
    "128,128,1,4,3,1,1,1",
    "64,96,1,2,4,2,1,1",
    "256,64,1,4,2,1,1,1",
    "32,64,1,1,3,4,1,1",
    "16,48,1,1,2,8,1,1",
    # variant 2: B straight into VGPRs, A of the K range resident in LDS
    "64,128,1,4,4,1,1,2",
    "64,192,1,4,4,2,1,2",
    "128,64,1,4,4,1,1,2",
    "32,48,1,1,3,4,1,2",
    # variant 6: both operands through LDS, each slot refilled in two parts
    "256,256,4,2,2,1,1,6",
    "128,128,2,2,3,1,1,6",
    "64,128,1,2,4,2,1,6",
    "128,256,4,2,3,1,1,6",
    # variant 3: B straight into VGPRs, a producer wave streams A through LDS
    "128,96,1,6,3,1,1,3",
    "64,64,1,4,3,1,1,3",
    "32,48,1,1,2,1,1,3",
    "64,64,1,4,3,2,1,3",
    "32,48,1,1,2,4,1,3",
]


@pytest.mark.parametrize("forced", FORCED)
def test_forced_tile_configs(oracle, monkeypatch, forced):
    monkeypatch.setenv("DG_FORCE_CONFIG", forced)
    p = gen.make_dense(300, 520, 1024, seed=11, with_c=True)
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    _compare(p, D, sent, ref, comp, what=f"forced {forced}")


# ------------------------------------------------------------------ HIP graph capture
def test_graph_replays_match_eager(oracle):
    """Calls captured into a HIP graph (split-K dense, masked) give the eager bits
    on every replay, with eager work and synchronisations between replays."""
    import moe_grouped_gemm_scales_amd as dg
    pd = gen.make_dense(64, 2112, 7168, seed=1000)          # selects split-K
    pm = gen.make_workload(4)
    dd, dm = to_dev(pd), to_dev(pm)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        De = torch.empty(64, 2112, dtype=torch.bfloat16, device="cuda")
        Me = gen.sentinel_like((4, 256, 7168), 3).to("cuda")
        dg.dg_fp8_gemm_nt(dd["A"], dd["sfa"], dd["B"], dd["sfb"], None, De)
        dg.dg_m_grouped_fp8_gemm_nt_masked(dm["A"], dm["sfa"], dm["B"], dm["sfb"], dm["masked_m"], None, Me)
        torch.cuda.synchronize()
        Dg = torch.empty_like(De)
        Mg = gen.sentinel_like((4, 256, 7168), 3).to("cuda")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            dg.dg_fp8_gemm_nt(dd["A"], dd["sfa"], dd["B"], dd["sfb"], None, Dg)
            dg.dg_m_grouped_fp8_gemm_nt_masked(dm["A"], dm["sfa"], dm["B"], dm["sfb"], dm["masked_m"], None, Mg)
        for rep in range(3):
            Dg.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(Dg.view(torch.int16), De.view(torch.int16)), f"dense replay {rep}"
            assert torch.equal(Mg.view(torch.int16), Me.view(torch.int16)), f"masked replay {rep}"
            # eager work between replays, on the same stream and workspace
            dg.dg_fp8_gemm_nt(dd["A"], dd["sfa"], dd["B"], dd["sfb"], None, De)
            torch.cuda.synchronize()


# ------------------------------------------------------------------ variants 1 and 2 on the grouped forms
@pytest.mark.parametrize("forced", ["128,128,4,2,2,1,1,4", "64,96,2,2,2,1,1,4", "256,224,4,2,2,1,1,4",
                                    "128,128,4,2,2,2,1,4"])
def test_a_ahead_variant(oracle, monkeypatch, forced):
    """Variant 4 (A requested one K block further ahead than B, separate LDS rings) on
    ragged dense (split-K included), masked and contiguous problems, FP32 and UE8M0 scales."""
    monkeypatch.setenv("DG_FORCE_CONFIG", forced)
    for e8 in (False, True):
        p = gen.make_dense(300, 520, 1024, seed=41, with_c=True, ue8m0=e8)
        D, sent = run(p)
        ref, comp = oracle_rows(oracle, p)
        _compare(p, D, sent, ref, comp, what=f"dense {forced} ue8m0={e8}")
        if forced.split(",")[5] != "1":
            continue                      # split-K is dense only
        pm = gen.make_masked(3, 200, 333, 512, seed=42, with_c=True, masked_m=[200, 0, 77], ue8m0=e8)
        D, sent = run(pm)
        ref, comp = oracle_rows(oracle, pm)
        _compare(pm, D, sent, ref, comp, what=f"masked {forced} ue8m0={e8}")
        if int(forced.split(",")[0]) <= 128:
            pc = gen.make_contiguous([128, 0, 256, 100], 200, 384, seed=43, with_c=True, pad_rows=128, ue8m0=e8)
            D, sent = run(pc)
            ref, comp = oracle_rows(oracle, pc)
            _compare(pc, D, sent, ref, comp, what=f"contiguous {forced} ue8m0={e8}")


@pytest.mark.parametrize("forced", ["256,256,4,2,2,1,1,6", "128,256,4,2,3,1,1,6", "128,128,2,2,3,1,1,6",
                                    "64,128,1,2,4,2,1,6", "128,128,4,2,2,1,1,6"])
def test_split_refill_variant(oracle, monkeypatch, forced):
    """Variant 6 (each LDS slot refilled in two parts, after a barrier in the middle of the
    K block and after its end) on ragged dense (split-K included), masked and contiguous
    problems, FP32, UE8M0 and UE8M0-pair scales."""
    monkeypatch.setenv("DG_FORCE_CONFIG", forced)
    for e8 in (False, True):
        p = gen.make_dense(300, 520, 1024, seed=141, with_c=True, ue8m0=e8)
        D, sent = run(p)
        ref, comp = oracle_rows(oracle, p)
        _compare(p, D, sent, ref, comp, what=f"dense {forced} ue8m0={e8}")
        if e8:
            pp = gen.to_ue8m0_pairs(p)
            D, sent = run(pp)
            _compare(pp, D, sent, ref, comp, what=f"dense {forced} ue8m0 pairs")
        if forced.split(",")[5] != "1":
            continue                      # split-K is dense only
        pm = gen.make_masked(3, 200, 333, 512, seed=142, with_c=True, masked_m=[200, 0, 77], ue8m0=e8)
        D, sent = run(pm)
        ref, comp = oracle_rows(oracle, pm)
        _compare(pm, D, sent, ref, comp, what=f"masked {forced} ue8m0={e8}")
        if int(forced.split(",")[0]) <= 128:
            pc = gen.make_contiguous([128, 0, 256, 100], 200, 384, seed=143, with_c=True, pad_rows=128, ue8m0=e8)
            D, sent = run(pc)
            ref, comp = oracle_rows(oracle, pc)
            _compare(pc, D, sent, ref, comp, what=f"contiguous {forced} ue8m0={e8}")


@pytest.mark.parametrize("K", [128, 256, 384, 640])
def test_split_refill_short_k(oracle, monkeypatch, K):
    """Variant 6 with one to five K blocks per tile and two or three slots: the prologue's
    later groups and the loop's refills are placeholders there."""
    for forced in ("256,256,4,2,2,1,1,6", "128,128,2,2,3,1,1,6"):
        monkeypatch.setenv("DG_FORCE_CONFIG", forced)
        p = gen.make_dense(260, 300, K, seed=150 + K, with_c=True)
        D, sent = run(p)
        ref, comp = oracle_rows(oracle, p)
        _compare(p, D, sent, ref, comp, what=f"{forced} K={K}")


@pytest.mark.parametrize("K", [128, 256, 384])
def test_a_ahead_short_k(oracle, monkeypatch, K):
    """Variant 4 with one, two and three K blocks per tile: the prologue's second A block
    and the loop's refills are placeholders there."""
    monkeypatch.setenv("DG_FORCE_CONFIG", "64,96,2,2,2,1,1,4")
    p = gen.make_dense(130, 200, K, seed=44 + K, with_c=True)
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    _compare(p, D, sent, ref, comp, what=f"a-ahead K={K}")


@pytest.mark.parametrize("forced", ["128,128,1,8,5,1,1,1", "64,64,1,4,3,1,1,1", "64,128,1,4,4,1,1,2",
                                    "64,64,1,4,3,1,1,3"])
def test_bdirect_grouped(oracle, monkeypatch, forced):
    monkeypatch.setenv("DG_FORCE_CONFIG", forced)
    pm = gen.make_masked(3, 200, 333, 512, seed=21, with_c=True, masked_m=[200, 0, 77])
    D, sent = run(pm)
    ref, comp = oracle_rows(oracle, pm)
    _compare(pm, D, sent, ref, comp, what=f"masked {forced}")
    pc = gen.make_contiguous([128, 0, 256, 100], 200, 384, seed=22, with_c=True, pad_rows=128)
    D, sent = run(pc)
    ref, comp = oracle_rows(oracle, pc)
    _compare(pc, D, sent, ref, comp, what=f"contiguous {forced}")


# ------------------------------------------------------------------ variant 5: B in VGPRs, A through a deep ring
V5_FORCED = ["192,256,1,8,4,1,1,5", "128,256,1,8,6,1,1,5", "64,128,1,4,3,1,1,5", "128,128,1,4,4,1,1,5"]


@pytest.mark.parametrize("forced", V5_FORCED)
def test_b_in_registers_large_tile(oracle, monkeypatch, forced):
    """Variant 5 on ragged dense problems (K of 1, 2, 3 and 9 blocks: the prologue's and the
    tail's loads past the last block), and on masked and contiguous problems."""
    monkeypatch.setenv("DG_FORCE_CONFIG", forced)
    for M, N, K in ((300, 520, 1152), (77, 333, 128), (257, 260, 256), (130, 515, 384)):
        p = gen.make_dense(M, N, K, seed=61 + M + K, with_c=(K != 256))
        D, sent = run(p)
        ref, comp = oracle_rows(oracle, p)
        _compare(p, D, sent, ref, comp, what=f"dense {M}x{N}x{K} {forced}")
    pm = gen.make_masked(3, 200, 333, 640, seed=62, with_c=True, masked_m=[200, 0, 77])
    D, sent = run(pm)
    ref, comp = oracle_rows(oracle, pm)
    _compare(pm, D, sent, ref, comp, what=f"masked {forced}")
    if int(forced.split(",")[0]) <= 128:
        pc = gen.make_contiguous([128, 0, 256, 100], 200, 384, seed=63, with_c=True, pad_rows=128)
        D, sent = run(pc)
        ref, comp = oracle_rows(oracle, pc)
        _compare(pc, D, sent, ref, comp, what=f"contiguous {forced}")


def test_b_in_registers_integer_data_bitwise(oracle, monkeypatch):
    """Variant 5 with integer data and power-of-two scales: D equals the oracle's BF16 bitwise
    (maps the B-register lanes and the permuted A-scale layout)."""
    monkeypatch.setenv("DG_FORCE_CONFIG", "192,256,1,8,4,1,1,5")
    g = torch.Generator().manual_seed(97)
    M, N, K = 200, 520, 1280
    A = gen.integer_codes((M, K), g, max_abs=8)
    B = gen.integer_codes((N, K), g, max_abs=8)
    sfa = gen.pow2_scales((K // 128, M), g, -2, 2)
    sfb = gen.pow2_scales(((N + 127) // 128, K // 128), g, -2, 2)
    p = gen.Problem("dense", A, sfa, B, sfb)
    D, _ = run(p)
    ref, _ = oracle_rows(oracle, p)
    assert np.array_equal(check.bf16_bits(D), oracle.bf16_rne(ref).reshape(M, N))


# ------------------------------------------------------------------ two launches over column ranges
# (fields 9-10 of a launch: first and end column; launches separated by ';')
SEGMENTS = [   # (launches, kinds they are valid for)
    ("128,128,4,2,2,1,1,0,0,256;64,96,2,2,3,1,1,0,256,520", "dense masked contiguous"),
    ("256,256,4,2,2,1,1,0,0,256;256,192,4,2,2,1,1,0,256,520", "dense masked"),
    ("64,64,1,4,3,2,1,2,0,128;64,96,1,2,3,1,1,1,128,520", "dense"),
    ("128,96,1,6,3,1,1,3,0,96;64,112,1,1,2,1,1,0,96,520", "dense masked contiguous"),
    ("64,64,1,4,3,4,1,3,0,192;64,64,1,4,3,2,1,3,192,520", "dense"),
]


@pytest.mark.parametrize("forced,kinds", SEGMENTS)
def test_column_range_plans(oracle, monkeypatch, forced, kinds):
    import moe_grouped_gemm_scales_amd as dg
    monkeypatch.setenv("DG_FORCE_CONFIG", forced)
    problems = {
        "dense": gen.make_dense(300, 520, 1024, seed=12, with_c=True),
        "masked": gen.make_masked(3, 200, 520, 512, seed=23, with_c=True, masked_m=[200, 0, 77]),
        "contiguous": gen.make_contiguous([128, 0, 256, 100], 520, 384, seed=24, with_c=True, pad_rows=128),
    }
    for kind in kinds.split():
        p = problems[kind]
        # the forced launches are the ones used (two column ranges)
        key = dg.describe_config({"dense": 0, "contiguous": 1, "masked": 2}[kind], p.M, p.N, p.K, p.G, True)
        assert key.count("_cols") == 2, key
        D, sent = run(p)
        ref, comp = oracle_rows(oracle, p)
        _compare(p, D, sent, ref, comp, what=f"{kind} {forced}")


# ------------------------------------------------------------------ packed UE8M0 scales
UE8M0_DENSE = [(1, 16, 128, False), (5, 129, 640, True), (100, 300, 512, True), (257, 515, 1152, False),
               (300, 1000, 2048, True)]


@pytest.mark.parametrize("M,N,K,with_c", UE8M0_DENSE)
def test_ue8m0_dense(oracle, M, N, K, with_c):
    p = gen.make_dense(M, N, K, seed=M + N + K + 5, with_c=with_c, ue8m0=True)
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    _compare(p, D, sent, ref, comp, what=f"ue8m0 dense {M}x{N}x{K}")


def test_ue8m0_integer_data_bitwise(oracle):
    """Integer codes and power-of-two scales: every sum is exact, so D is the oracle's BF16 bit for bit."""
    g = torch.Generator().manual_seed(78)
    M, N, K = 96, 400, 1664          # 13 K blocks: the last word is partly unused
    A = gen.integer_codes((M, K), g, max_abs=8)
    B = gen.integer_codes((N, K), g, max_abs=8)
    ea = torch.randint(125, 130, (K // 128, M), generator=g)
    eb = torch.randint(125, 130, ((N + 127) // 128, K // 128), generator=g)
    p = gen.Problem("dense", A, gen.pack_ue8m0(ea.T).T.contiguous(), B, gen.pack_ue8m0(eb), ue8m0=True)
    D, _ = run(p)
    ref, _ = oracle_rows(oracle, p)
    assert np.array_equal(check.bf16_bits(D), oracle.bf16_rne(ref).reshape(M, N))


def test_ue8m0_grouped(oracle):
    pm = gen.make_masked(3, 200, 333, 640, seed=31, with_c=True, masked_m=[200, 0, 77], ue8m0=True)
    D, sent = run(pm)
    ref, comp = oracle_rows(oracle, pm)
    _compare(pm, D, sent, ref, comp, what="ue8m0 masked")
    pc = gen.make_contiguous([128, 0, 256, 100], 333, 640, seed=32, with_c=True, pad_rows=128, ue8m0=True)
    D, sent = run(pc)
    ref, comp = oracle_rows(oracle, pc)
    _compare(pc, D, sent, ref, comp, what="ue8m0 contiguous")


UE8M0_FORCED = ["128,128,4,2,2,1,1,0", "256,256,4,2,2,1,1,0", "64,96,2,2,4,2,1,0", "256,224,4,2,2,1,1,0",
                "32,64,1,2,3,4,1,0", "128,128,4,2,2,1,1,0,0,256;64,96,2,2,3,1,1,0,256,520",
                "256,192,2,2,2,1,1,0"]   # the last: 4 waves of 128 x 96, accumulators in AGPRs


@pytest.mark.parametrize("forced", UE8M0_FORCED)
def test_ue8m0_forced_tile_configs(oracle, monkeypatch, forced):
    monkeypatch.setenv("DG_FORCE_CONFIG", forced)
    p = gen.make_dense(300, 520, 1024, seed=13, with_c=True, ue8m0=True)
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    _compare(p, D, sent, ref, comp, what=f"ue8m0 forced {forced}")


@pytest.mark.parametrize("cfg", [0, 1, "1c", 2, 3, 4])
def test_ue8m0_workloads(oracle, cfg):
    p = gen.make_workload(cfg, ue8m0=True)
    D, sent = run(p)
    # the masked and the large dense result are compared whole, the contiguous one on sampled rows
    rows = sample_rows(p.M, 48, seed=5, block=128) if p.kind == "contiguous" else None
    ref, comp = oracle_rows(oracle, p, rows=rows)
    _compare(p, D, sent, ref, comp, rows=rows, what="ue8m0 " + gen.WORKLOAD_NAMES[cfg])
