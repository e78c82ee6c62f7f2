"""GPU parity of the NN / TN / TT storage layouts (dense) and the NN contiguous
grouped form against the oracle, through the C ABI.  Same bar as the NT forms;
rows the contiguous form does not compute keep their sentinel bits."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_scales_amd as dg
from tests import check, gen
from tests.gpu_util import sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def stored(p, layout):
    """(A, B) as stored for the layout (CPU tensors)."""
    A = p.A if layout[0] == "n" else p.A.t().contiguous()
    B = p.B if layout[1] == "t" else p.B.transpose(-1, -2).contiguous()
    return A, B


def run_layout(p, layout, sentinel_seed=99):
    A, B = stored(p, layout)
    c = lambda t: None if t is None else t.to("cuda")
    sent = gen.sentinel_like((p.M, p.N), sentinel_seed)
    D = sent.to("cuda")
    if p.kind == "dense":
        getattr(dg, f"dg_fp8_gemm_{layout}")(c(A), c(p.sfa), c(B), c(p.sfb), c(p.C), D)
    else:
        dg.dg_m_grouped_fp8_gemm_nn_contiguous(c(A), c(p.sfa), c(B), c(p.sfb), c(p.m_indices), c(p.C), D)
    torch.cuda.synchronize()
    return D.cpu(), sent, A, B


def check_layout(oracle, p, layout, rows=None):
    D, sent, A, B = run_layout(p, layout)
    mi = None if p.kind == "dense" else p.m_indices.numpy()
    ref, comp = oracle.fp8_gemm_layout(layout, A.numpy(), p.sfa.numpy(), B.numpy(), p.sfb.numpy(),
                                       None if p.C is None else p.C.numpy(), m_indices=mi, rows=rows)
    idx = np.arange(p.M) if rows is None else rows
    got = check.bf16_to_f64(D[torch.as_tensor(idx)])
    if comp.any():
        check.assert_close(got[comp], ref[comp], f"{layout} {p.kind} {p.M}x{p.N}x{p.K}")
    if (~comp).any():
        un = torch.as_tensor(idx[~comp])
        assert np.array_equal(check.bf16_bits(D[un]), check.bf16_bits(sent[un])), "a skipped row was written"


@pytest.mark.parametrize("layout", ["nn", "tn", "tt", "nt"])
@pytest.mark.parametrize("M,N,K,with_c", [(1, 16, 128, False), (5, 129, 384, True), (100, 300, 512, True),
                                          (257, 515, 640, False)])
def test_dense_layouts(oracle, layout, M, N, K, with_c):
    p = gen.make_dense(M, N, K, seed=M + 3 * N + K, with_c=with_c)
    check_layout(oracle, p, layout)


def test_nn_contiguous(oracle):
    p = gen.make_contiguous([128, 0, 256, 100], 333, 640, seed=77, with_c=True, pad_rows=128)
    check_layout(oracle, p, "nn")


@pytest.mark.parametrize("layout", ["nn", "tt"])
def test_layouts_large_dense(oracle, layout):
    """The compute-bound dense workload (4096 x 7168 x 16384) stored in another layout."""
    p = gen.make_workload(2)
    # NN compared whole, TT on sampled rows
    check_layout(oracle, p, layout, rows=None if layout == "nn" else sample_rows(p.M, 32, seed=8, block=256))


def test_nn_contiguous_workload(oracle):
    """The contiguous MoE workload with B stored [G, K, N]."""
    p = gen.make_workload(3)
    check_layout(oracle, p, "nn", rows=sample_rows(p.M, 40, seed=9, block=128))
