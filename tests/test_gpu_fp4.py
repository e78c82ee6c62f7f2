"""GPU parity of the FP8 x FP4 GEMM (E4M3 A with 1x128 UE8M0 scales, E2M1 B with
1x32 UE8M0 scales per row) against the CPU oracle, through the C ABI.

Bar as for the FP8 forms: |D - ref| <= 2^-7 |ref| + 1e-3 rms(ref) per computed
element; bitwise where the exact result is a BF16 number (one-hot rows of A,
integer data); rows not computed keep their sentinel bits.
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


def _compare(D, sent, ref, comp, rows=None, what=""):
    Df = flat_rows(D)
    Sf = flat_rows(sent)
    idx = np.arange(Df.shape[0]) if rows is None else rows
    if comp.any():
        got = check.bf16_to_f64(Df[torch.as_tensor(idx[comp])])
        check.assert_close(got, ref[comp], what)
    if (~comp).any():
        untouched = idx[~comp]
        assert np.array_equal(check.bf16_bits(Df[torch.as_tensor(untouched)]),
                              check.bf16_bits(Sf[torch.as_tensor(untouched)])), f"{what}: a skipped row was written"


def _pack_nibbles(q: torch.Tensor) -> torch.Tensor:
    """[..., K] nibbles -> [..., K/2] bytes, element 2i in the low nibble of byte i."""
    return (q[..., 0::2] | (q[..., 1::2] << 4)).to(torch.uint8).contiguous()


FP4_DENSE = [(1, 16, 128, False), (5, 129, 640, True), (64, 2112, 1024, False), (100, 300, 512, True),
             (257, 515, 1152, False), (300, 1000, 2048, True)]


@pytest.mark.parametrize("M,N,K,with_c", FP4_DENSE)
def test_fp4_dense(oracle, M, N, K, with_c):
    p = gen.make_dense(M, N, K, seed=M + N + K + 9, with_c=with_c, fp4=True)
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    _compare(D, sent, ref, comp, what=f"fp4 dense {M}x{N}x{K}")


def test_fp4_one_hot_maps_nibbles_and_scales(oracle):
    """A row m is 1.0 at column pi(m) and zero elsewhere, with scale 1: D[m, n] is
    2^(eb-127) e2m1(B[n, pi(m)]) exactly, so the result must be the oracle's BF16 bit
    for bit.  This fixes the nibble order, the K position of every lane's codes and
    which of the four 1x32 scale bytes each K element takes."""
    g = torch.Generator().manual_seed(91)
    M, N, K = 256, 192, 512
    pi = torch.randperm(K, generator=g)[:M]
    A = torch.zeros(M, K, dtype=torch.uint8)
    A[torch.arange(M), pi] = 0x38                           # E4M3 1.0
    ea = torch.full((K // 128, M), 127, dtype=torch.int64)  # scale 1
    q = torch.randint(0, 16, (N, K), generator=g, dtype=torch.uint8)
    eb = torch.randint(120, 135, (N, K // 32), generator=g)
    sfb = gen.pack_ue8m0(eb.reshape(N * (K // 128), 4)).reshape(N, K // 128).contiguous()
    p = gen.Problem("dense", A, gen.pack_ue8m0(ea.T).T.contiguous(), _pack_nibbles(q), sfb, ue8m0=True, fp4=True)
    D, _ = run(p)
    ref, _ = oracle_rows(oracle, p)
    assert np.array_equal(check.bf16_bits(D), oracle.bf16_rne(ref).reshape(M, N))


def test_fp4_integer_data_bitwise(oracle):
    """Integer E4M3 codes, every E2M1 code and power-of-two scales: all sums are exact
    in FP32, so D equals the oracle's BF16 bit for bit."""
    g = torch.Generator().manual_seed(92)
    M, N, K = 96, 400, 1664          # 13 K blocks: the last A scale word is partly unused
    A = gen.integer_codes((M, K), g, max_abs=8)
    ea = torch.randint(125, 130, (K // 128, M), generator=g)
    q = torch.randint(0, 16, (N, K), generator=g, dtype=torch.uint8)
    eb = torch.randint(125, 130, (N, K // 32), generator=g)
    sfb = gen.pack_ue8m0(eb.reshape(N * (K // 128), 4)).reshape(N, K // 128).contiguous()
    p = gen.Problem("dense", A, gen.pack_ue8m0(ea.T).T.contiguous(), _pack_nibbles(q), sfb, ue8m0=True, fp4=True)
    D, _ = run(p)
    ref, _ = oracle_rows(oracle, p)
    assert np.array_equal(check.bf16_bits(D), oracle.bf16_rne(ref).reshape(M, N))


def test_fp4_grouped(oracle):
    pm = gen.make_masked(3, 200, 333, 640, seed=41, with_c=True, masked_m=[200, 0, 77], fp4=True)
    D, sent = run(pm)
    ref, comp = oracle_rows(oracle, pm)
    _compare(D, sent, ref, comp, what="fp4 masked")
    pc = gen.make_contiguous([128, 0, 256, 100], 333, 640, seed=42, with_c=True, pad_rows=128, fp4=True)
    D, sent = run(pc)
    ref, comp = oracle_rows(oracle, pc)
    _compare(D, sent, ref, comp, what="fp4 contiguous")


@pytest.mark.parametrize("masked_m", [[0, 0], [256, 256], [-5, 300], [1, 129]])
def test_fp4_masked_edges(oracle, masked_m):
    p = gen.make_masked(2, 256, 520, 512, seed=43, masked_m=masked_m, fp4=True)
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    _compare(D, sent, ref, comp, what=f"fp4 masked {masked_m}")


FP4_FORCED = ["128,128,4,2,2,1,1,0", "256,256,4,2,2,1,1,0", "64,96,2,2,4,2,1,0", "256,224,4,2,2,1,1,0",
              "32,64,1,2,3,4,1,0", "128,112,4,1,3,1,1,0", "128,128,4,2,2,1,1,0,0,256;64,96,2,2,3,1,1,0,256,520",
              "128,224,4,2,4,1,1,0"]


@pytest.mark.parametrize("forced", FP4_FORCED)
def test_fp4_forced_tile_configs(oracle, monkeypatch, forced):
    monkeypatch.setenv("DG_FORCE_CONFIG", forced)
    p = gen.make_dense(300, 520, 1024, seed=17, with_c=True, fp4=True)
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    _compare(D, sent, ref, comp, what=f"fp4 forced {forced}")


@pytest.mark.parametrize("cfg", [0, 1, "1c", 2, 3, 4])
def test_fp4_workloads(oracle, cfg):
    """The five benchmark workloads with FP4 weights, at full size (sampled rows)."""
    p = gen.make_workload(cfg, fp4=True)
    D, sent = run(p)
    # every row except for the contiguous workload (sampled; the FP32-scale form checks it whole)
    rows = sample_rows(p.M, 48, seed=6, block=128) if p.kind == "contiguous" else None
    ref, comp = oracle_rows(oracle, p, rows=rows)
    _compare(D, sent, ref, comp, rows=rows, what="fp4 " + gen.WORKLOAD_NAMES[cfg])
