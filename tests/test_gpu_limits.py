"""GPU parity at the edges of the sizes the C ABI accepts, against the CPU oracle,
through the C ABI:

* the longest K: 2^24 - 128 (131071 K blocks, a prime, so no split-K), where a
  256-row tile's slab of A is just under the 4 GiB that 32-bit buffer offsets
  reach (the ABI rejects one block more), with the default plan and a forced
  256-row tile;
* K = 2^20 split over workgroups, in each scale format (FP32, UE8M0, FP8 x FP4,
  BF16);
* 2^19 + 77 rows of A (dense, with C) and 2^19 rows over four experts
  (contiguous): grids of thousands of tiles, row offsets past 2^27 bytes;
* 2^18 + 40 columns of B with 3 rows;
* masked groups with a long K (2^17) and a partial mask;
* A stored K-outermost with 2^22 + 64 rows (its rewrite spans 65537 column
  blocks).

Outputs are checked on sampled rows (always the first and last and tile
edges) with the bar of the other parity tests: |D - ref| <= 2^-7 |ref| +
1e-3 rms(ref) per element; rows not computed keep their sentinel bits.
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


def _compare(D, sent, ref, comp, rows, what):
    Df, Sf = flat_rows(D), flat_rows(sent)
    idx = torch.as_tensor(rows)
    got = check.bf16_to_f64(Df[idx])
    assert comp.any(), what
    check.assert_close(got[comp], ref[comp], what)
    if (~comp).any():
        un = torch.as_tensor(rows[~comp])
        assert np.array_equal(check.bf16_bits(Df[un]), check.bf16_bits(Sf[un])), f"{what}: a skipped row was written"


def _random_e4m3(shape, seed):
    """Uniformly random E4M3 codes (a seeded PCG64 byte stream) with the two NaN
    codes (0x7f, 0xff) moved to the largest finite magnitude, a few rows at a
    time to bound host memory."""
    rng = np.random.default_rng(seed)
    x = torch.frombuffer(bytearray(rng.bytes(int(np.prod(shape)))), dtype=torch.uint8).view(shape)
    for r in range(0, shape[0], 16):
        blk = x[r:r + 16]
        blk -= ((blk & 0x7F) == 0x7F).to(torch.uint8)
    return x


LONGEST_K = (1 << 24) - 128


@pytest.fixture(scope="module")
def longest_k():
    M, N, K = 256, 16, LONGEST_K
    g = torch.Generator().manual_seed(4242)
    sfa = gen.pow2_scales((K // 128, M), g, lo=-4, hi=0)
    sfb = gen.pow2_scales((1, K // 128), g, lo=-4, hi=0)
    return gen.Problem("dense", _random_e4m3((M, K), 4243), sfa, _random_e4m3((N, K), 4244), sfb)


@pytest.mark.parametrize("forced", [None, "256,16,4,1,2,1,1,0"])
def test_longest_k_at_the_offset_limit(oracle, monkeypatch, longest_k, forced):
    if forced:
        monkeypatch.setenv("DG_FORCE_CONFIG", forced)
    p = longest_k
    D, sent = run(p)
    rows = np.array([0, 1, 127, 128, 254, 255], dtype=np.int64)
    ref, comp = oracle_rows(oracle, p, rows=rows)
    _compare(D, sent, ref, comp, rows, f"dense 256x16x{LONGEST_K} ({forced or 'default plan'})")


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0", "fp8_fp4", "bf16"])
def test_long_k_split(oracle, fmt):
    M, N, K = 32, 144, 1 << 20
    if fmt == "bf16":
        p = gen.make_bf16("dense", seed=77, M=M, N=N, K=K)
    else:
        p = gen.make_dense(M, N, K, seed=76, ue8m0=fmt == "ue8m0", fp4=fmt == "fp8_fp4")
    D, sent = run(p)
    rows = np.array([0, 1, 15, 16, 30, 31], dtype=np.int64)
    ref, comp = oracle_rows(oracle, p, rows=rows)
    _compare(D, sent, ref, comp, rows, f"{fmt} dense {M}x{N}x{K}")


def test_many_rows_dense(oracle):
    M, N, K = (1 << 19) + 77, 96, 256
    p = gen.make_dense(M, N, K, seed=78, with_c=True)
    D, sent = run(p)
    rows = sample_rows(M, 48, block=256, seed=3)
    ref, comp = oracle_rows(oracle, p, rows=rows)
    _compare(D, sent, ref, comp, rows, f"dense {M}x{N}x{K} + C")


def test_many_rows_contiguous(oracle):
    group_rows = [(1 << 17) - 5, 1 << 17, 0, (1 << 17) + 3]
    p = gen.make_contiguous(group_rows, 96, 256, seed=79)
    D, sent = run(p)
    rows = sample_rows(p.M, 64, block=128, seed=4)
    ref, comp = oracle_rows(oracle, p, rows=rows)
    _compare(D, sent, ref, comp, rows, f"contiguous {group_rows} x 96 x 256")


def test_many_columns(oracle):
    M, N, K = 3, (1 << 18) + 40, 512
    p = gen.make_dense(M, N, K, seed=80, with_c=True)
    D, sent = run(p)
    rows = np.arange(M, dtype=np.int64)
    ref, comp = oracle_rows(oracle, p, rows=rows)
    _compare(D, sent, ref, comp, rows, f"dense {M}x{N}x{K} + C")


def test_masked_long_k(oracle):
    G, M_max, N, K = 2, 256, 160, 1 << 17
    p = gen.make_masked(G, M_max, N, K, seed=81, masked_m=[256, 37])
    D, sent = run(p)
    rows = np.concatenate([sample_rows(M_max, 10, seed=5), M_max + sample_rows(M_max, 10, seed=6)])
    ref, comp = oracle_rows(oracle, p, rows=rows)
    _compare(D, sent, ref, comp, rows, f"masked {G}x{M_max}x{N}x{K}")


def test_tt_layout_rewrite_of_many_rows(oracle):
    """A stored K-outermost ([K][M]) with M = 2^22 + 64: its rewrite covers 65537 blocks
    of 64 columns, past what one grid dimension of 65535 would hold."""
    import moe_grouped_gemm_scales_amd as dg
    M, N, K = (1 << 22) + 64, 16, 128
    p = gen.make_dense(M, N, K, seed=82)
    At = p.A.t().contiguous()
    sent = gen.sentinel_like((M, N), 7)
    D = sent.to("cuda")
    dg.dg_fp8_gemm_tt(At.to("cuda"), p.sfa.to("cuda"), p.B.to("cuda"), p.sfb.to("cuda"), None, D)
    torch.cuda.synchronize()
    rows = sample_rows(M, 48, block=64, seed=8)
    ref, comp = oracle_rows(oracle, p, rows=rows)
    _compare(D.cpu(), sent, ref, comp, rows, f"tt layout {M}x{N}x{K}")
