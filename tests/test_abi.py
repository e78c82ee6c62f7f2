"""The C ABI on the CPU: the library loads, exports every symbol that the
headers under include/ declare, and rejects bad arguments before any HIP call."""
import ctypes
import glob
import os
import re

import pytest

import moe_grouped_gemm_scales_amd as pkg
from moe_grouped_gemm_scales_amd import dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")

FAKE = 0x100000   # a 16-byte aligned address that is never dereferenced


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert "dg_fp8_gemm_nt" in names and "dg_m_grouped_fp8_gemm_nt_masked" in names
    lib = ctypes.CDLL(dg.LIB_PATH)
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        for n in declared_functions(h):
            assert hasattr(lib, n), f"{n} declared in {os.path.basename(h)} but not exported"


def test_probe_arguments_rejected_before_launch():
    """Probe entry points validate on the host (no GPU is touched for these)."""
    lib = dg.lib
    v = ctypes.c_void_p
    lib.dg_probe_null.argtypes = [ctypes.c_int, v]
    lib.dg_probe_spin.argtypes = [ctypes.c_int, v]
    lib.dg_probe_stream_read.argtypes = [v, ctypes.c_size_t, v, ctypes.c_int, v]
    lib.dg_probe_mfma_fp8.argtypes = [ctypes.c_int, ctypes.c_int, v, v]
    assert lib.dg_probe_null(0, None) == -1
    assert lib.dg_probe_spin(0, None) == -1
    assert lib.dg_probe_spin(2000000, None) == -1
    assert lib.dg_probe_stream_read(None, 1024, v(FAKE), 4, None) == -1
    assert lib.dg_probe_stream_read(v(FAKE), 1000, v(FAKE), 4, None) == -3
    assert lib.dg_probe_stream_read(v(FAKE + 4), 1024, v(FAKE), 4, None) == -3
    assert lib.dg_probe_mfma_fp8(4, 0, v(FAKE), None) == -1
    assert lib.dg_probe_mfma_fp8(4, 10, None, None) == -1


def test_alignment_query():
    assert pkg.get_mk_alignment_for_contiguous_layout() == 128


def _dense(A=FAKE, sfa=FAKE, B=FAKE, sfb=FAKE, C=None, D=FAKE, M=64, N=64, K=128):
    v = ctypes.c_void_p
    return dg.lib.dg_fp8_gemm_nt(v(A), v(sfa), v(B), v(sfb), v(C), v(D), M, N, K, None)


@pytest.mark.parametrize("kw,status", [
    (dict(A=0), -1), (dict(sfa=0), -1), (dict(B=0), -1), (dict(sfb=0), -1), (dict(D=0), -1),
    (dict(M=-1), -1), (dict(N=0), -1), (dict(K=0), -1),
    (dict(K=100), -2), (dict(K=7168 + 64), -2),
    (dict(A=FAKE + 8), -3), (dict(D=FAKE + 2), -3), (dict(C=FAKE + 4), -3), (dict(sfa=FAKE + 2), -3),
])
def test_dense_validation(kw, status):
    assert _dense(**kw) == status
    assert dg.lib.dg_last_error().decode()


def test_empty_m_is_a_no_op():
    assert _dense(M=0) == 0


def test_grouped_validation():
    v = ctypes.c_void_p
    f = dg.lib.dg_m_grouped_fp8_gemm_nt_contiguous
    assert f(v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, None, v(FAKE), 128, 64, 128, 2, None) == -1
    assert f(v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, v(FAKE), 100, 64, 128, 2, None) == -3
    assert f(v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, v(FAKE), 128, 64, 128, 0, None) == -1
    g = dg.lib.dg_m_grouped_fp8_gemm_nt_masked
    assert g(v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, None, v(FAKE), 64, 64, 128, 2, None) == -1
    assert g(v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE + 2), None, v(FAKE), 64, 64, 128, 2, None) == -3
    assert g(v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, v(FAKE), 0, 64, 128, 2, None) == 0


def test_no_device_is_a_hip_error():
    """Valid arguments on a host without a GPU: the first HIP call fails cleanly."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _dense() == -5


def test_binding_marshalling_errors():
    import torch
    A = torch.zeros(4, 128, dtype=torch.uint8)
    with pytest.raises(ValueError):
        pkg.dg_fp8_gemm_nt(A, torch.zeros(1, 4), A, torch.zeros(1, 1), None, torch.zeros(4, 4, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        pkg.dg_fp8_gemm_nt(A.float(), torch.zeros(1, 4), A, torch.zeros(1, 1), None, None)


def test_fp4_and_ue8m0_validation():
    v = ctypes.c_void_p
    f = dg.lib.dg_fp8_fp4_gemm_nt
    assert f(v(FAKE), v(FAKE), None, v(FAKE), None, v(FAKE), 64, 64, 128, None) == -1      # B NULL
    assert f(v(FAKE), v(FAKE), v(FAKE + 8), v(FAKE), None, v(FAKE), 64, 64, 128, None) == -3   # B misaligned
    assert f(v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, v(FAKE), 64, 64, 96, None) == -2    # K % 128
    assert f(v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, v(FAKE), 0, 64, 128, None) == 0     # M = 0: no-op
    g = dg.lib.dg_m_grouped_fp8_fp4_gemm_nt_masked
    assert g(v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, None, v(FAKE), 64, 64, 128, 2, None) == -1
    h = dg.lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0
    assert h(v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, v(FAKE), 100, 64, 128, 2, None) == -3


def test_k_grouped_validation():
    v = ctypes.c_void_p
    f = dg.lib.dg_k_grouped_fp8_gemm_tn_contiguous
    assert f(v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, None, v(FAKE), 64, 64, 128, 2, None) == -1   # ks NULL
    assert f(v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, v(FAKE), 64, 64, 128, 0, None) == -1  # G = 0
    assert f(v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE + 2), None, v(FAKE), 64, 64, 128, 2, None) == -3
    assert f(v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, v(FAKE), 64, 64, 192, 2, None) == -2  # K % 128
    assert f(v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, v(FAKE), 0, 64, 128, 2, None) == 0    # M = 0


def test_layout_and_bf16_validation():
    v = ctypes.c_void_p
    for name in ("dg_fp8_gemm_nn", "dg_fp8_gemm_tn", "dg_fp8_gemm_tt"):
        f = getattr(dg.lib, name)
        assert f(None, v(FAKE), v(FAKE), v(FAKE), None, v(FAKE), 64, 64, 128, None) == -1
        assert f(v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, v(FAKE), 64, 64, 100, None) == -2
    c = dg.lib.dg_m_grouped_fp8_gemm_nn_contiguous
    assert c(v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, v(FAKE), 100, 64, 128, 2, None) == -3
    b = dg.lib.dg_bf16_gemm_nt
    assert b(None, v(FAKE), None, v(FAKE), 64, 64, 64, None) == -1
    assert b(v(FAKE), v(FAKE), None, v(FAKE), 64, 64, 96, None) == -2          # K % 64
    assert b(v(FAKE), v(FAKE + 4), None, v(FAKE), 64, 64, 64, None) == -3      # B misaligned
    assert b(v(FAKE), v(FAKE), None, v(FAKE), 0, 64, 64, None) == 0           # M = 0: no-op
    bc = dg.lib.dg_m_grouped_bf16_gemm_nt_contiguous
    assert bc(v(FAKE), v(FAKE), v(FAKE), None, v(FAKE), 100, 64, 64, 2, None) == -3   # M % 128
    assert bc(v(FAKE), v(FAKE), None, None, v(FAKE), 128, 64, 64, 2, None) == -1      # m_indices NULL
    bm = dg.lib.dg_m_grouped_bf16_gemm_nt_masked
    assert bm(v(FAKE), v(FAKE), v(FAKE), None, v(FAKE), 64, 64, 64, 0, None) == -1    # G = 0


def test_describe_config_for_new_forms():
    assert pkg.describe_config(0 | pkg.SCALE_FP8_FP4, 128, 24576, 1536, num_cus=256).endswith("_f8f4")
    assert pkg.describe_config(pkg.KIND_K_GROUPED, 4096, 7168, 32768, 4, num_cus=256).startswith("k3")
    key = pkg.describe_config(pkg.KIND_BF16, 4096, 7168, 16384, num_cus=256)
    assert key.endswith("_bf16") and "_K32768_" in key       # BF16 rows counted in bytes


def test_b_is_streamed_only_where_two_row_blocks_at_most_read_it():
    """Plans whose B blocks at most two row blocks of the launch read (dense or
    masked with few rows) carry `_bs`; the large and contiguous plans, whose row
    blocks share B blocks through L2, do not."""
    streamed = [pkg.describe_config(0, 64, 2112, 7168, num_cus=256),
                pkg.describe_config(0, 128, 24576, 1536, num_cus=256),
                pkg.describe_config(0, 128, 24576, 1536, has_c=True, num_cus=256),
                pkg.describe_config(2, 256, 7168, 2048, 4, num_cus=256),
                pkg.describe_config(0 | pkg.SCALE_UE8M0, 128, 24576, 1536, num_cus=256)]
    shared = [pkg.describe_config(0, 4096, 7168, 16384, num_cus=256),
              pkg.describe_config(1, 32768, 4096, 7168, 4, num_cus=256),
              pkg.describe_config(pkg.KIND_K_GROUPED, 4096, 7168, 32768, 4, num_cus=256),
              pkg.describe_config(0, 1024, 4096, 1024, num_cus=256)]
    assert all("_bs" in k for k in streamed), streamed
    assert not any("_bs" in k for k in shared), shared
