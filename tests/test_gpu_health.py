"""GPU checks of what parity on one call cannot show.

* The producer/consumer variant's bounded LDS-flag waits never give up on the
  shapes that use it (the library's give-up counter stays 0), and a wait that
  does run out is counted (forced from the host with a one-iteration spin
  limit compiled into the kernel: the waits end at once, the grid drains, and
  only the values of that call are wrong).
* Guard bands: D sits inside one larger allocation whose bytes just before and
  just after it hold sentinel bits; the ragged-N, N % 4 != 0, split-K and
  masked paths must leave them untouched.
* Split-K hand-off under reuse: two different input sets alternate through the
  same stream workspace, eagerly and through one captured graph, 500 replays,
  every result compared bitwise with that set's eager result (which is checked
  against the oracle), so a partial left over from the other set would show.
"""
import ctypes

import numpy as np
import pytest
import torch

from tests import check, gen
from tests.gpu_util import oracle_rows, run, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _giveups() -> int:
    import moe_grouped_gemm_scales_amd as dg
    return dg.get_wait_giveups()


# ------------------------------------------------------------------ bounded waits
def test_variant3_waits_never_give_up(oracle, monkeypatch):
    import moe_grouped_gemm_scales_amd as dg
    dg.reset_wait_giveups()
    assert _giveups() == 0
    # the dense 128-row workload's plan uses the producer wave; the masked decode
    # workload runs it with the producer variant forced
    for cfg, forced in ((1, None), (4, "128,112,1,7,3,1,1,3")):
        if forced:
            monkeypatch.setenv("DG_FORCE_CONFIG", forced)
        p = gen.make_workload(cfg)
        kind = 0 if p.kind == "dense" else 2
        rows = p.A.shape[1] if p.kind == "masked" else p.M
        assert "v3" in dg.describe_config(kind, rows, p.N, p.K, p.G, False), "expected the producer variant"
        D, sent = run(p)
        ref, comp = oracle_rows(oracle, p)
        Df = D.reshape(-1, p.N)
        check.assert_close(check.bf16_to_f64(Df[torch.as_tensor(np.nonzero(comp)[0])]), ref[comp],
                           gen.WORKLOAD_NAMES[cfg])
    assert _giveups() == 0


def test_tiny_spin_limit_is_counted(monkeypatch):
    """A one-iteration spin limit makes the waits run out at once (all accesses stay
    inside LDS and the buffers, so only D is wrong); each is counted."""
    import moe_grouped_gemm_scales_amd as dg
    monkeypatch.setenv("DG_JIT_EXTRA_OPTION", "-DDG_SPIN_LIMIT=1")
    monkeypatch.setenv("DG_FORCE_CONFIG", "128,96,1,6,3,1,1,3")
    dg.reset_wait_giveups()
    p = gen.make_dense(128, 960, 1536, seed=71)
    run(p)
    n = _giveups()
    dg.reset_wait_giveups()
    assert n > 0, "a wait with a one-iteration limit should have run out"
    assert _giveups() == 0


# ------------------------------------------------------------------ guard bands around D
GUARD = 4096   # bf16 elements before and after D


def _run_guarded(p, forced=None, monkeypatch=None):
    """D placed in the middle of one allocation; returns (D, sentinel, guard ok)."""
    import moe_grouped_gemm_scales_amd as dg
    if forced:
        monkeypatch.setenv("DG_FORCE_CONFIG", forced)
    shape = (p.A.shape[0], p.A.shape[1], p.N) if p.kind == "masked" else (p.A.shape[0], p.N)
    n = int(np.prod(shape))
    whole = gen.sentinel_like((GUARD + n + GUARD,), 99).to("cuda")
    before = whole.clone()
    D = whole[GUARD:GUARD + n].view(shape)
    sent = D.cpu().clone()
    d = to_dev(p)
    if p.kind == "dense":
        dg.dg_fp8_gemm_nt(d["A"], d["sfa"], d["B"], d["sfb"], d["C"], D)
    elif p.kind == "contiguous":
        dg.dg_m_grouped_fp8_gemm_nt_contiguous(d["A"], d["sfa"], d["B"], d["sfb"], d["m_indices"], d["C"], D)
    else:
        dg.dg_m_grouped_fp8_gemm_nt_masked(d["A"], d["sfa"], d["B"], d["sfb"], d["masked_m"], d["C"], D)
    torch.cuda.synchronize()
    w, b = whole.view(torch.int16), before.view(torch.int16)
    guards_ok = torch.equal(w[:GUARD], b[:GUARD]) and torch.equal(w[GUARD + n:], b[GUARD + n:])
    return D.cpu(), sent, guards_ok


@pytest.mark.parametrize("name,make,forced", [
    ("ragged N, N % 4 = 3", lambda: gen.make_dense(100, 515, 640, seed=81, with_c=True), None),
    ("N % 4 = 2, M = 1", lambda: gen.make_dense(1, 130, 256, seed=82), None),
    ("split-K 7 (64 x 2112 x 7168)", lambda: gen.make_dense(64, 2112, 7168, seed=83), None),
    ("split-K 4, ragged", lambda: gen.make_dense(77, 333, 2048, seed=84, with_c=True), "64,64,2,2,2,4,1,0"),
    ("split-K 2, producer variant", lambda: gen.make_dense(50, 243, 1024, seed=85), "64,64,1,4,3,2,1,3"),
    ("masked, ragged N", lambda: gen.make_masked(3, 96, 203, 512, seed=86, masked_m=[96, 0, 33]), None),
    ("contiguous with padding", lambda: gen.make_contiguous([128, 0, 100], 131, 384, seed=87, pad_rows=128),
     None),
])
def test_guard_bands_around_d(oracle, monkeypatch, name, make, forced):
    p = make()
    D, sent, guards_ok = _run_guarded(p, forced, monkeypatch)
    assert guards_ok, f"{name}: a byte just outside D was written"
    ref, comp = oracle_rows(oracle, p)
    Df, Sf = D.reshape(-1, p.N), sent.reshape(-1, p.N)
    if comp.any():
        check.assert_close(check.bf16_to_f64(Df[torch.as_tensor(np.nonzero(comp)[0])]), ref[comp], name)
    if (~comp).any():
        un = torch.as_tensor(np.nonzero(~comp)[0])
        assert np.array_equal(check.bf16_bits(Df[un]), check.bf16_bits(Sf[un])), f"{name}: a skipped row was written"


# ------------------------------------------------------------------ split-K hand-off under reuse
def test_split_k_alternating_inputs_soak(oracle):
    """64 x 2112 x 7168 (7 K splits): two input sets alternate through one stream's
    workspace, eagerly (100 calls) and through one captured graph (500 replays)."""
    import moe_grouped_gemm_scales_amd as dg
    assert "sk7" in dg.describe_config(0, 64, 2112, 7168), "expected a split-K plan"
    px, py = gen.make_dense(64, 2112, 7168, seed=91), gen.make_dense(64, 2112, 7168, seed=92)
    dx, dy = to_dev(px), to_dev(py)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        refs = []
        for name, p, d in (("set 0", px, dx), ("set 1", py, dy)):
            D = torch.empty(64, 2112, dtype=torch.bfloat16, device="cuda")
            dg.dg_fp8_gemm_nt(d["A"], d["sfa"], d["B"], d["sfb"], None, D)
            torch.cuda.synchronize()
            ref, _ = oracle_rows(oracle, p)
            check.assert_close(check.bf16_to_f64(D), ref, name)
            refs.append(D.view(torch.int16).clone())
        # eager alternation through the same workspace
        D = torch.empty(64, 2112, dtype=torch.bfloat16, device="cuda")
        for i in range(100):
            d = (dx, dy)[i % 2]
            dg.dg_fp8_gemm_nt(d["A"], d["sfa"], d["B"], d["sfb"], None, D)
            torch.cuda.synchronize()
            assert torch.equal(D.view(torch.int16), refs[i % 2]), f"eager call {i}"
        # one captured call on fixed input buffers; the sets are copied in between replays
        inp = {k: dx[k].clone() for k in ("A", "sfa", "B", "sfb")}
        Dg = torch.empty(64, 2112, dtype=torch.bfloat16, device="cuda")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            dg.dg_fp8_gemm_nt(inp["A"], inp["sfa"], inp["B"], inp["sfb"], None, Dg)
        order = np.random.default_rng(7).integers(0, 2, 500)
        for i, which in enumerate(order):
            src = (dx, dy)[which]
            for k in inp:
                inp[k].copy_(src[k])
            Dg.fill_(0)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(Dg.view(torch.int16), refs[which]), f"replay {i} (set {which})"


def test_wait_giveup_counter_abi():
    """The counter's C entry points through ctypes: NULL is rejected, reset clears."""
    import moe_grouped_gemm_scales_amd.dg as dgm
    lib = dgm.lib
    assert lib.dg_get_wait_giveups(None) == -1
    assert lib.dg_reset_wait_giveups() == 0
    c = ctypes.c_uint(123)
    assert lib.dg_get_wait_giveups(ctypes.byref(c)) == 0
    assert c.value == 0
