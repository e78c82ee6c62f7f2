"""The dense entry point that allocates nothing (dg_fp8_gemm_nt_noalloc),
through the C ABI: its output equals dg_fp8_gemm_nt's bit for bit on two calls
in a row (the second with a smaller input, both split-K plans, so both use the
library's static scratch array), it takes no device memory, and it rejects a
plan whose split-K needs more scratch than the array holds."""
import ctypes

import pytest
import torch

from tests import check, gen
from tests.gpu_util import oracle_rows, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _call(fn, d, D, M, N, K, stream):
    v = lambda t: ctypes.c_void_p(None if t is None else t.data_ptr())
    return fn(v(d["A"]), v(d["sfa"]), v(d["B"]), v(d["sfb"]), v(d["C"]), v(D), M, N, K,
              ctypes.c_void_p(stream.cuda_stream))


def test_noalloc_matches_the_allocating_entry_point(oracle):
    import moe_grouped_gemm_scales_amd.dg as dgm
    lib = dgm.lib
    s_alloc, s_free = torch.cuda.Stream(), torch.cuda.Stream()
    # two calls in a row, the second smaller; both shapes select split-K
    for (M, N, K, seed) in ((64, 2112, 7168, 301), (48, 1536, 7168, 302)):
        desc = dgm.describe_config(0, M, N, K)
        assert "_sk1_" not in desc, f"{desc}: expected a split-K plan"
        p = gen.make_dense(M, N, K, seed=seed, with_c=(seed % 2 == 0))
        d = to_dev(p)
        D_ref = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        with torch.cuda.stream(s_alloc):
            assert _call(lib.dg_fp8_gemm_nt, d, D_ref, M, N, K, s_alloc) == 0   # also loads the kernels
        torch.cuda.synchronize()
        ref, _ = oracle_rows(oracle, p)
        check.assert_close(check.bf16_to_f64(D_ref), ref, f"dg_fp8_gemm_nt {M}x{N}x{K}")
        D = gen.sentinel_like((M, N), seed).to("cuda")
        with torch.cuda.stream(s_free):
            D.add_(0)          # a first launch on the stream, so the runtime has set it up
        torch.cuda.synchronize()
        free_before = torch.cuda.mem_get_info()[0]
        # a stream the allocating path has never seen: it would have created a workspace there
        with torch.cuda.stream(s_free):
            rc = _call(lib.dg_fp8_gemm_nt_noalloc, d, D, M, N, K, s_free)
            assert rc == 0, lib.dg_last_error().decode()
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free_before, "the no-alloc call took device memory"
        assert torch.equal(D.view(torch.int16), D_ref.view(torch.int16)), f"{M}x{N}x{K}: differs from dg_fp8_gemm_nt"


def test_noalloc_needs_loaded_kernels_and_bounded_scratch(monkeypatch):
    import moe_grouped_gemm_scales_amd.dg as dgm
    lib = dgm.lib
    s = torch.cuda.Stream()
    # sizes never called before: nothing loaded, so the call refuses (and allocates nothing)
    p = gen.make_dense(40, 1000, 3072, seed=303)
    d = to_dev(p)
    D = torch.empty(40, 1000, dtype=torch.bfloat16, device="cuda")
    assert _call(lib.dg_fp8_gemm_nt_noalloc, d, D, 40, 1000, 3072, s) == -2
    assert "not loaded" in lib.dg_last_error().decode()
    # 1024 x 2112 x 8192 with 8 forced K splits: 71 MB of partials, more than the scratch
    monkeypatch.setenv("DG_FORCE_CONFIG", "128,128,4,2,2,8,1,0")
    q = gen.make_dense(1024, 2112, 8192, seed=304)
    e = to_dev(q)
    D = torch.empty(1024, 2112, dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(s):
        assert _call(lib.dg_fp8_gemm_nt, e, D, 1024, 2112, 8192, s) == 0
        assert _call(lib.dg_fp8_gemm_nt_noalloc, e, D, 1024, 2112, 8192, s) == -2
    torch.cuda.synchronize()
    assert "more than the scratch holds" in lib.dg_last_error().decode()
