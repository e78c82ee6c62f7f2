"""GPU parity of the unscaled BF16 GEMM (dense, contiguous, masked) against the
CPU oracle, through the C ABI.  Same bar as the FP8 forms; integer data must
match bit for bit; rows not computed keep their sentinel bits."""
import numpy as np
import pytest
import torch

from tests import check, gen
from tests.gpu_util import flat_rows, oracle_rows, run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _compare(D, sent, ref, comp, rows=None, what=""):
    Df, Sf = flat_rows(D), flat_rows(sent)
    idx = np.arange(Df.shape[0]) if rows is None else rows
    if comp.any():
        got = check.bf16_to_f64(Df[torch.as_tensor(idx[comp])])
        check.assert_close(got, ref[comp], what)
    if (~comp).any():
        un = torch.as_tensor(idx[~comp])
        assert np.array_equal(check.bf16_bits(Df[un]), check.bf16_bits(Sf[un])), f"{what}: a skipped row was written"


@pytest.mark.parametrize("M,N,K,with_c", [(1, 16, 64, False), (5, 129, 192, True), (64, 2112, 1024, False),
                                          (100, 300, 512, True), (257, 515, 640, False), (300, 1000, 2048, True)])
def test_bf16_dense(oracle, M, N, K, with_c):
    p = gen.make_bf16("dense", seed=M + N + K + 11, M=M, N=N, K=K, with_c=with_c)
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    _compare(D, sent, ref, comp, what=f"bf16 dense {M}x{N}x{K}")


def test_bf16_integer_data_bitwise(oracle):
    g = torch.Generator().manual_seed(12)
    M, N, K = 96, 400, 256
    A = torch.randint(-20, 21, (M, K), generator=g).to(torch.bfloat16)
    B = torch.randint(-20, 21, (N, K), generator=g).to(torch.bfloat16)
    p = gen.Problem("dense", A, None, B, None, bf16=True)
    D, _ = run(p)
    ref, _ = oracle_rows(oracle, p)
    assert np.array_equal(check.bf16_bits(D), oracle.bf16_rne(ref).reshape(M, N))


def test_bf16_grouped(oracle):
    pc = gen.make_bf16("contiguous", seed=13, N=333, K=640, group_rows=[128, 0, 256, 100], with_c=True, pad_rows=128)
    D, sent = run(pc)
    ref, comp = oracle_rows(oracle, pc)
    _compare(D, sent, ref, comp, what="bf16 contiguous")
    pm = gen.make_bf16("masked", seed=14, N=333, K=640, G=3, M_max=200, masked_m=[200, 0, 77], with_c=True)
    D, sent = run(pm)
    ref, comp = oracle_rows(oracle, pm)
    _compare(D, sent, ref, comp, what="bf16 masked")


@pytest.mark.parametrize("forced", ["128,128,4,2,2,1,1,0", "256,256,4,2,2,1,1,0", "64,96,2,2,4,2,1,0",
                                    "32,64,1,2,3,4,1,0", "256,224,2,2,2,1,1,0",    # AGPR accumulators
                                    "256,256,4,2,2,1,1,4",                         # A ahead
                                    "256,256,4,2,2,1,1,6", "128,128,2,2,3,1,1,6"])  # split refill
def test_bf16_forced_tile_configs(oracle, monkeypatch, forced):
    monkeypatch.setenv("DG_FORCE_CONFIG", forced)
    p = gen.make_bf16("dense", seed=15, M=300, N=520, K=1024, with_c=True)
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    _compare(D, sent, ref, comp, what=f"bf16 forced {forced}")


def test_bf16_large_dense(oracle):
    """The compute-bound dense shape (4096 x 7168 x 16384) in BF16, every element."""
    p = gen.make_bf16("dense", seed=1002, M=4096, N=7168, K=16384)
    D, sent = run(p)
    ref, comp = oracle_rows(oracle, p)
    _compare(D, sent, ref, comp, what="bf16 4096x7168x16384")
