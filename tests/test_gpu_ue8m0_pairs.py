"""GPU parity of the FP8 GEMM with UE8M0 scale pairs in 16-bit words, stored
MN-major (the Ascend packing: sfa int16 [ceil(Kb/2)][M], sfb int16
[ceil(Kb/2)][Nb]), against the CPU oracle, through the C ABI, in all three
forms.

Bar as for the other forms: |D - ref| <= 2^-7 |ref| + 1e-3 rms(ref) per computed
element; bitwise where the exact result is a BF16 number (integer data with
power-of-two scales); rows not computed keep their sentinel bits.
"""
import numpy as np
import pytest
import torch

from tests import check, gen
from tests.gpu_util import flat_rows, oracle_rows, run, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _compare(p, D, sent, ref, comp, rows=None, what=""):
    Df, Sf = flat_rows(D), flat_rows(sent)
    idx = np.arange(Df.shape[0]) if rows is None else rows
    if comp.any():
        got = check.bf16_to_f64(Df[torch.as_tensor(idx[comp])])
        check.assert_close(got, ref[comp], what)
    if (~comp).any():
        un = torch.as_tensor(idx[~comp])
        assert np.array_equal(check.bf16_bits(Df[un]), check.bf16_bits(Sf[un])), f"{what}: a skipped row was written"


def _pairs(p):
    return gen.to_ue8m0_pairs(p)


# odd and even K-block counts (a trailing half-used pair word), ragged M and N
SHAPES = [(1, 16, 128, False), (5, 129, 640, True), (100, 300, 384, True), (257, 515, 1152, False),
          (300, 1000, 2048, True), (64, 2112, 7168, False)]


@pytest.mark.parametrize("M,N,K,with_c", SHAPES)
def test_pairs_dense(oracle, M, N, K, with_c):
    p = _pairs(gen.make_dense(M, N, K, seed=M + N + K + 9, with_c=with_c, ue8m0=True))
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    _compare(p, D, sent, ref, comp, what=f"pairs dense {M}x{N}x{K}")


def test_pairs_integer_data_bitwise(oracle):
    """Integer codes and power-of-two scales: every sum is exact, so D is the oracle's BF16
    bit for bit; 13 K blocks, so the last pair word's high byte is unused (set to 0xFF)."""
    g = torch.Generator().manual_seed(79)
    M, N, K = 96, 400, 1664
    A = gen.integer_codes((M, K), g, max_abs=8)
    B = gen.integer_codes((N, K), g, max_abs=8)
    Kb, Nb = K // 128, (N + 127) // 128
    ea = torch.randint(124, 131, (Kb, M), generator=g)
    eb = torch.randint(124, 131, (Kb, Nb), generator=g)
    sfa, sfb = gen.pack_ue8m0_pairs(ea), gen.pack_ue8m0_pairs(eb)
    sfa[-1] = (sfa[-1].to(torch.int32) | 0xFF00).to(torch.int16)    # unused trailing bytes: NaN code, ignored
    sfb[-1] = (sfb[-1].to(torch.int32) | 0xFF00).to(torch.int16)
    p = gen.Problem("dense", A, sfa.contiguous(), B, sfb.contiguous(), ue8m0_pairs=True)
    D, _ = run(p)
    ref, _ = oracle_rows(oracle, p)
    assert np.all(np.isfinite(ref))
    assert np.array_equal(check.bf16_bits(D), oracle.bf16_rne(ref).reshape(M, N))


def test_pairs_grouped(oracle):
    pm = _pairs(gen.make_masked(3, 200, 333, 640, seed=33, with_c=True, masked_m=[200, 0, 77], ue8m0=True))
    D, sent = run(pm)
    ref, comp = oracle_rows(oracle, pm)
    _compare(pm, D, sent, ref, comp, what="pairs masked")
    pc = _pairs(gen.make_contiguous([128, 0, 256, 100], 333, 640, seed=34, with_c=True, pad_rows=128, ue8m0=True))
    D, sent = run(pc)
    ref, comp = oracle_rows(oracle, pc)
    _compare(pc, D, sent, ref, comp, what="pairs contiguous")


FORCED = ["128,128,4,2,2,1,1,0", "256,256,4,2,2,1,1,0", "64,96,2,2,4,2,1,0", "256,224,4,2,2,1,1,4",
          "128,128,4,2,2,1,1,4", "32,64,1,2,3,4,1,0", "256,192,2,2,2,1,1,0"]


@pytest.mark.parametrize("forced", FORCED)
def test_pairs_forced_tile_configs(oracle, monkeypatch, forced):
    monkeypatch.setenv("DG_FORCE_CONFIG", forced)
    p = _pairs(gen.make_dense(300, 520, 1152, seed=15, with_c=True, ue8m0=True))
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    _compare(p, D, sent, ref, comp, what=f"pairs forced {forced}")


@pytest.mark.parametrize("cfg", [0, 2, 3, 4])
def test_pairs_workloads(oracle, cfg):
    """The workloads at full size with pair-packed scales: the dense and masked results
    compared whole, the contiguous one on sampled rows."""
    p = gen.make_workload(cfg, ue8m0_pairs=True)
    D, sent = run(p)
    rows = sample_rows(p.M, 48, seed=21, block=128) if p.kind == "contiguous" else None
    ref, comp = oracle_rows(oracle, p, rows=rows)
    _compare(p, D, sent, ref, comp, rows=rows, what="pairs " + gen.WORKLOAD_NAMES[cfg])


def test_pairs_equal_quads_on_the_gpu():
    """The same exponents packed two to an int16 and four to an int32 give bitwise the same D."""
    p = gen.make_workload(4, ue8m0=True)
    q = gen.to_ue8m0_pairs(p)
    Dq, _ = run(p)
    Dp, _ = run(q)
    assert torch.equal(Dq.view(torch.int16), Dp.view(torch.int16))
