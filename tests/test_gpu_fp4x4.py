"""GPU parity of the FP4 x FP4 GEMM (E2M1 A and B, one UE8M0 scale per 1x32 block of
every row of both) against the CPU oracle, through the C ABI.  Same bar as the
other forms; bitwise where the exact result is a BF16 number."""
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


def _compare(D, sent, ref, comp, rows=None, what=""):
    Df, Sf = flat_rows(D), flat_rows(sent)
    idx = np.arange(Df.shape[0]) if rows is None else rows
    got = check.bf16_to_f64(Df[torch.as_tensor(idx)])
    if comp.any():
        check.assert_close(got[comp], ref[comp], what)
    if (~comp).any():
        un = torch.as_tensor(idx[~comp])
        assert np.array_equal(check.bf16_bits(Df[un]), check.bf16_bits(Sf[un])), f"{what}: a skipped row was written"


def _pack(q):
    return (q[..., 0::2] | (q[..., 1::2] << 4)).to(torch.uint8).contiguous()


def _words(e, rows, K):
    return gen.pack_ue8m0(e.reshape(rows * (K // 128), 4)).reshape(rows, K // 128).contiguous()


@pytest.mark.parametrize("M,N,K,with_c", [(1, 16, 128, False), (5, 129, 640, True), (100, 300, 512, True),
                                          (257, 515, 1152, False)])
def test_fp4x4_dense(oracle, M, N, K, with_c):
    p = gen.make_dense(M, N, K, seed=M + N + K + 21, with_c=with_c, fp4x4=True)
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    _compare(D, sent, ref, comp, what=f"fp4x4 dense {M}x{N}x{K}")


def test_fp4x4_one_hot_bitwise(oracle):
    """Row m of A is E2M1 1.0 at column pi(m), scale 1: D[m, n] = 2^(eb-127) e2m1(B[n, pi(m)])
    exactly, which fixes A's nibble order and K map against B's."""
    g = torch.Generator().manual_seed(23)
    M, N, K = 256, 192, 512
    pi = torch.randperm(K, generator=g)[:M]
    qa = torch.zeros(M, K, dtype=torch.uint8)
    qa[torch.arange(M), pi] = 0x2                          # E2M1 1.0
    qb = torch.randint(0, 16, (N, K), generator=g, dtype=torch.uint8)
    ea = torch.full((M, K // 32), 127)
    eb = torch.randint(120, 135, (N, K // 32), generator=g)
    p = gen.Problem("dense", _pack(qa), _words(ea, M, K), _pack(qb), _words(eb, N, K), ue8m0=True, fp4=True,
                    fp4a=True)
    D, _ = run(p)
    ref, _ = oracle_rows(oracle, p)
    assert np.array_equal(check.bf16_bits(D), oracle.bf16_rne(ref).reshape(M, N))


def test_fp4x4_grouped(oracle):
    pm = gen.make_masked(3, 200, 333, 640, seed=24, with_c=True, masked_m=[200, 0, 77], fp4x4=True)
    D, sent = run(pm)
    ref, comp = oracle_rows(oracle, pm)
    _compare(D, sent, ref, comp, what="fp4x4 masked")
    pc = gen.make_contiguous([128, 0, 256, 100], 333, 640, seed=25, with_c=True, pad_rows=128, fp4x4=True)
    D, sent = run(pc)
    ref, comp = oracle_rows(oracle, pc)
    _compare(D, sent, ref, comp, what="fp4x4 contiguous")


@pytest.mark.parametrize("forced", ["128,128,4,2,2,1,1,0", "256,256,4,2,2,1,1,0", "64,96,2,2,4,2,1,0",
                                    "32,64,1,2,3,4,1,0", "128,224,4,2,4,1,1,0"])
def test_fp4x4_forced_tile_configs(oracle, monkeypatch, forced):
    monkeypatch.setenv("DG_FORCE_CONFIG", forced)
    p = gen.make_dense(300, 520, 1024, seed=26, with_c=True, fp4x4=True)
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    _compare(D, sent, ref, comp, what=f"fp4x4 forced {forced}")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_fp4x4_workloads(oracle, cfg):
    p = gen.make_workload(cfg, fp4x4=True)
    D, sent = run(p)
    if p.kind == "masked":
        rows = np.arange(p.A.shape[0] * p.A.shape[1])
    elif p.M <= 256:
        rows = None
    else:
        rows = sample_rows(p.M, 32, seed=7, block=128)
    ref, comp = oracle_rows(oracle, p, rows=rows)
    _compare(D, sent, ref, comp, rows=rows, what="fp4x4 " + gen.WORKLOAD_NAMES[cfg])
