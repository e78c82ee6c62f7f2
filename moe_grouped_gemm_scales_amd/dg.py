"""Python binding of libdg.so: argument marshalling only.

Every function here checks the torch tensors' dtypes, shapes, devices and
contiguity, then calls the C entry point of the same name with raw device
pointers and the current HIP stream.  All arithmetic runs in the library's
HIP kernels; there is no other code path.  If libdg.so is missing the import
fails loudly (build it with ``python moe_grouped_gemm_scales_amd/build.py``).

Layouts (DeepGEMM README, "Interfaces / Notes"): D = C + A @ B.T with A
[M, K] and B [N, K] in FP8 E4M3 (torch.float8_e4m3fn or raw uint8 codes),
sfa float32 [K/128, M] (MN-major LHS scales), sfb float32 [ceil(N/128), K/128],
optional float32 C [M, N], bfloat16 D [M, N].  Grouped forms add a leading
group dimension as documented in include/dg.h.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# DG_LIBRARY: load another build of the same C ABI instead of the in-tree one
LIB_PATH = os.environ.get("DG_LIBRARY") or os.path.join(_HERE, "libdg.so")

DG_OK = 0
STATUS_NAMES = {0: "DG_OK", -1: "DG_ERR_INVALID_ARG", -2: "DG_ERR_UNSUPPORTED",
                -3: "DG_ERR_ALIGNMENT", -4: "DG_ERR_JIT", -5: "DG_ERR_HIP"}


class DGError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python moe_grouped_gemm_scales_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.dg_fp8_gemm_nt.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, vp]
    lib.dg_m_grouped_fp8_gemm_nt_contiguous.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp]
    lib.dg_m_grouped_fp8_gemm_nt_masked.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp]
    lib.dg_fp8_gemm_nt_ue8m0.argtypes = lib.dg_fp8_gemm_nt.argtypes
    lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0.argtypes = lib.dg_m_grouped_fp8_gemm_nt_contiguous.argtypes
    lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0.argtypes = lib.dg_m_grouped_fp8_gemm_nt_masked.argtypes
    for name in ("dg_fp8_gemm_nn", "dg_fp8_gemm_tn", "dg_fp8_gemm_tt"):
        getattr(lib, name).argtypes = lib.dg_fp8_gemm_nt.argtypes
        getattr(lib, name).restype = i32
    lib.dg_m_grouped_fp8_gemm_nn_contiguous.argtypes = lib.dg_m_grouped_fp8_gemm_nt_contiguous.argtypes
    lib.dg_m_grouped_fp8_gemm_nn_contiguous.restype = i32
    vp_ = ctypes.c_void_p
    lib.dg_bf16_gemm_nt.argtypes = [vp_, vp_, vp_, vp_, i32, i32, i32, vp_]
    lib.dg_m_grouped_bf16_gemm_nt_contiguous.argtypes = [vp_, vp_, vp_, vp_, vp_, i32, i32, i32, i32, vp_]
    lib.dg_m_grouped_bf16_gemm_nt_masked.argtypes = [vp_, vp_, vp_, vp_, vp_, i32, i32, i32, i32, vp_]
    for f in (lib.dg_bf16_gemm_nt, lib.dg_m_grouped_bf16_gemm_nt_contiguous, lib.dg_m_grouped_bf16_gemm_nt_masked):
        f.restype = i32
    lib.dg_fp4_fp4_gemm_nt.argtypes = lib.dg_fp8_gemm_nt.argtypes
    lib.dg_m_grouped_fp4_fp4_gemm_nt_contiguous.argtypes = lib.dg_m_grouped_fp8_gemm_nt_contiguous.argtypes
    lib.dg_m_grouped_fp4_fp4_gemm_nt_masked.argtypes = lib.dg_m_grouped_fp8_gemm_nt_masked.argtypes
    for f in (lib.dg_fp4_fp4_gemm_nt, lib.dg_m_grouped_fp4_fp4_gemm_nt_contiguous,
              lib.dg_m_grouped_fp4_fp4_gemm_nt_masked):
        f.restype = i32
    lib.dg_k_grouped_fp8_gemm_tn_contiguous.argtypes = lib.dg_m_grouped_fp8_gemm_nt_contiguous.argtypes
    lib.dg_k_grouped_fp8_gemm_tn_contiguous.restype = i32
    lib.dg_fp8_fp4_gemm_nt.argtypes = lib.dg_fp8_gemm_nt.argtypes
    lib.dg_m_grouped_fp8_fp4_gemm_nt_contiguous.argtypes = lib.dg_m_grouped_fp8_gemm_nt_contiguous.argtypes
    lib.dg_m_grouped_fp8_fp4_gemm_nt_masked.argtypes = lib.dg_m_grouped_fp8_gemm_nt_masked.argtypes
    for f in (lib.dg_fp8_gemm_nt, lib.dg_m_grouped_fp8_gemm_nt_contiguous, lib.dg_m_grouped_fp8_gemm_nt_masked,
              lib.dg_fp8_gemm_nt_ue8m0, lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0,
              lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0, lib.dg_fp8_fp4_gemm_nt,
              lib.dg_m_grouped_fp8_fp4_gemm_nt_contiguous, lib.dg_m_grouped_fp8_fp4_gemm_nt_masked):
        f.restype = i32
    lib.dg_last_error.restype = ctypes.c_char_p
    lib.dg_last_error.argtypes = []
    lib.dg_get_mk_alignment_for_contiguous_layout.restype = i32
    lib.dg_set_num_cus.argtypes = [i32]
    lib.dg_set_num_cus.restype = i32
    lib.dg_get_num_cus.restype = i32
    lib.dg_init.restype = i32
    lib.dg_precompile.argtypes = [i32] * 7
    lib.dg_precompile.restype = i32
    lib.dg_describe_config.argtypes = [i32] * 7 + [ctypes.c_char_p, i32]
    lib.dg_describe_config.restype = i32
    lib.dg_fp8_gemm_nt_ue8m0_i16.argtypes = lib.dg_fp8_gemm_nt.argtypes
    lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_i16.argtypes = lib.dg_m_grouped_fp8_gemm_nt_contiguous.argtypes
    lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0_i16.argtypes = lib.dg_m_grouped_fp8_gemm_nt_masked.argtypes
    for f in (lib.dg_fp8_gemm_nt_ue8m0_i16, lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_i16,
              lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0_i16):
        f.restype = i32
    lib.dg_fp8_gemm_nt_noalloc.argtypes = lib.dg_fp8_gemm_nt.argtypes
    lib.dg_fp8_gemm_nt_noalloc.restype = i32
    lib.dg_get_wait_giveups.argtypes = [ctypes.POINTER(ctypes.c_uint)]
    lib.dg_get_wait_giveups.restype = i32
    lib.dg_reset_wait_giveups.argtypes = []
    lib.dg_reset_wait_giveups.restype = i32
    return lib


lib = _load()


def _check(status: int):
    if status != DG_OK:
        raise DGError(status, lib.dg_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# torch's current device and the raw handle of its current stream, without
# building Python device and stream objects (a few microseconds per call)
_cur_device = torch._C._cuda_getDevice
_cur_raw_stream = torch._C._cuda_getCurrentRawStream


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        return ctypes.c_void_p(_cur_raw_stream(_cur_device()))
    return ctypes.c_void_p(stream.cuda_stream)


def _fp8(t: torch.Tensor, name: str):
    if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise TypeError(f"{name} must be float8_e4m3fn or uint8 E4M3 codes, got {t.dtype}")
    _dev(t, name)


def _dev(t: torch.Tensor, name: str):
    d = t.get_device()                  # -1 for host tensors
    if d < 0:
        raise ValueError(f"{name} must be a device tensor")
    if d != _cur_device():
        # the library launches on the current device; another device's memory is not its operand
        raise ValueError(f"{name} is on {t.device}, but the current device is cuda:{_cur_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _f32(t: torch.Tensor, name: str, shape):
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _dev(t, name)


def _scales(sfa, sfb, sfa_kb_mn, sfb_nb_kb, lead=()):
    """Check the scale tensors; True for packed UE8M0 (int32), False for FP32.

    FP32: sfa [*lead, Kb, M] and sfb [*lead, Nb, Kb].  UE8M0: the same with Kb
    replaced by ceil(Kb/4) words, four K blocks to a word.
    """
    (kb, m), (nb, _) = sfa_kb_mn, sfb_nb_kb
    if sfa.dtype == torch.int32:
        w = _cdiv(kb, 4)
        for t, name, shape in ((sfa, "sfa", (*lead, w, m)), (sfb, "sfb", (*lead, nb, w))):
            if t.dtype != torch.int32:
                raise TypeError(f"{name} must be int32 (packed UE8M0) like sfa, got {t.dtype}")
            if tuple(t.shape) != tuple(shape):
                raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
            _dev(t, name)
        return True
    _f32(sfa, "sfa", (*lead, kb, m))
    _f32(sfb, "sfb", (*lead, nb, kb))
    return False


def _out(d: torch.Tensor, shape):
    if d.dtype != torch.bfloat16:
        raise TypeError(f"D must be bfloat16, got {d.dtype}")
    if tuple(d.shape) != tuple(shape):
        raise ValueError(f"D must have shape {tuple(shape)}, got {tuple(d.shape)}")
    _dev(d, "D")


def _cdiv(a, b):
    return (a + b - 1) // b


def dg_fp8_gemm_nt(A, sfa, B, sfb, C, D, stream=None):
    """D = C + A @ B.T (C may be None).  A [M,K], sfa [K/128,M], B [N,K], sfb [ceil(N/128),K/128].

    With int32 scale tensors (packed UE8M0, sfa [ceil(K/512),M], sfb [ceil(N/128),ceil(K/512)])
    this calls dg_fp8_gemm_nt_ue8m0.
    """
    _fp8(A, "A"); _fp8(B, "B")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B must share K")
    e8 = _scales(sfa, sfb, (_cdiv(K, 128), M), (_cdiv(N, 128), _cdiv(K, 128)))
    if C is not None:
        _f32(C, "C", (M, N))
    _out(D, (M, N))
    f = lib.dg_fp8_gemm_nt_ue8m0 if e8 else lib.dg_fp8_gemm_nt
    _check(f(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(C), _ptr(D), M, N, K, _stream(stream)))
    return D


def dg_m_grouped_fp8_gemm_nt_contiguous(A, sfa, B, sfb, m_indices, C, D, stream=None):
    """Contiguous M-grouped: row m uses B[m_indices[m]]; rows with an index outside [0,G) are untouched."""
    _fp8(A, "A"); _fp8(B, "B")
    M, K = A.shape
    G, N = B.shape[0], B.shape[1]
    if B.shape[2] != K:
        raise ValueError("A and B must share K")
    if sfa.dtype == torch.int32:       # packed UE8M0; sfa has no group dimension here
        e8 = _scales(sfa, sfb[0], (_cdiv(K, 128), M), (_cdiv(N, 128), _cdiv(K, 128)))
        if tuple(sfb.shape) != (G, _cdiv(N, 128), _cdiv(_cdiv(K, 128), 4)):
            raise ValueError("sfb must be int32 [G, ceil(N/128), ceil(K/512)]")
    else:
        e8 = False
        _f32(sfa, "sfa", (_cdiv(K, 128), M))
        _f32(sfb, "sfb", (G, _cdiv(N, 128), _cdiv(K, 128)))
    if m_indices.dtype != torch.int32 or tuple(m_indices.shape) != (M,):
        raise ValueError("m_indices must be int32 [M]")
    _dev(m_indices, "m_indices")
    if C is not None:
        _f32(C, "C", (M, N))
    _out(D, (M, N))
    f = lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0 if e8 else lib.dg_m_grouped_fp8_gemm_nt_contiguous
    _check(f(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(m_indices), _ptr(C), _ptr(D), M, N, K, G,
             _stream(stream)))
    return D


def dg_m_grouped_fp8_gemm_nt_masked(A, sfa, B, sfb, masked_m, C, D, stream=None):
    """Masked M-grouped: group g computes rows m < clamp(masked_m[g], 0, M_max); other rows untouched."""
    _fp8(A, "A"); _fp8(B, "B")
    G, M_max, K = A.shape
    N = B.shape[1]
    if B.shape[0] != G or B.shape[2] != K:
        raise ValueError("B must be [G, N, K]")
    e8 = _scales(sfa, sfb, (_cdiv(K, 128), M_max), (_cdiv(N, 128), _cdiv(K, 128)), lead=(G,))
    if masked_m.dtype != torch.int32 or tuple(masked_m.shape) != (G,):
        raise ValueError("masked_m must be int32 [G]")
    _dev(masked_m, "masked_m")
    if C is not None:
        _f32(C, "C", (G, M_max, N))
    _out(D, (G, M_max, N))
    f = lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0 if e8 else lib.dg_m_grouped_fp8_gemm_nt_masked
    _check(f(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(masked_m), _ptr(C), _ptr(D), M_max, N, K, G,
             _stream(stream)))
    return D


def get_mk_alignment_for_contiguous_layout() -> int:
    return int(lib.dg_get_mk_alignment_for_contiguous_layout())


def set_num_cus(n: int) -> None:
    _check(lib.dg_set_num_cus(int(n)))


def get_num_cus() -> int:
    return int(lib.dg_get_num_cus())


def init() -> None:
    _check(lib.dg_init())


def precompile(kind: int, rows: int, N: int, K: int, num_groups: int = 1, has_c: bool = False,
               num_cus: int = 0) -> None:
    _check(lib.dg_precompile(kind, rows, N, K, num_groups, int(has_c), num_cus))


def get_wait_giveups() -> int:
    """Bounded kernel waits on the current device that ran out (0 unless something went wrong)."""
    c = ctypes.c_uint(0)
    _check(lib.dg_get_wait_giveups(ctypes.byref(c)))
    return int(c.value)


def reset_wait_giveups() -> None:
    _check(lib.dg_reset_wait_giveups())


def describe_config(kind: int, rows: int, N: int, K: int, num_groups: int = 1, has_c: bool = False,
                    num_cus: int = 0) -> str:
    """Key of the kernel configuration a call with these sizes selects."""
    buf = ctypes.create_string_buffer(1024)
    _check(lib.dg_describe_config(kind, rows, N, K, num_groups, int(has_c), num_cus, buf, len(buf)))
    return buf.value.decode()


# The packed-UE8M0 entry points by their C names (the functions above also
# dispatch to them when given int32 scale tensors)
SCALE_UE8M0 = 4      # DG_SCALE_UE8M0: OR into `kind` of precompile / describe_config


def dg_fp8_gemm_nt_ue8m0(A, sfa, B, sfb, C, D, stream=None):
    if sfa.dtype != torch.int32:
        raise TypeError("dg_fp8_gemm_nt_ue8m0 takes packed UE8M0 int32 scales")
    return dg_fp8_gemm_nt(A, sfa, B, sfb, C, D, stream)


def dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(A, sfa, B, sfb, m_indices, C, D, stream=None):
    if sfa.dtype != torch.int32:
        raise TypeError("dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0 takes packed UE8M0 int32 scales")
    return dg_m_grouped_fp8_gemm_nt_contiguous(A, sfa, B, sfb, m_indices, C, D, stream)


def dg_m_grouped_fp8_gemm_nt_masked_ue8m0(A, sfa, B, sfb, masked_m, C, D, stream=None):
    if sfa.dtype != torch.int32:
        raise TypeError("dg_m_grouped_fp8_gemm_nt_masked_ue8m0 takes packed UE8M0 int32 scales")
    return dg_m_grouped_fp8_gemm_nt_masked(A, sfa, B, sfb, masked_m, C, D, stream)


# ---------------------------------------------------------------- UE8M0 pairs in int16 (MN-major)
SCALE_UE8M0_I16 = 64   # DG_SCALE_UE8M0_I16: OR into `kind` of precompile / describe_config


def _i16(t: torch.Tensor, name: str, shape):
    if t.dtype != torch.int16:
        raise TypeError(f"{name} must be int16 (UE8M0 pairs), got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _dev(t, name)


def dg_fp8_gemm_nt_ue8m0_i16(A, sfa, B, sfb, C, D, stream=None):
    """D = C + A @ B.T with UE8M0 scale pairs: sfa int16 [ceil(K/256), M], sfb int16 [ceil(K/256), ceil(N/128)]."""
    _fp8(A, "A"); _fp8(B, "B")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B must share K")
    P = _cdiv(_cdiv(K, 128), 2)
    _i16(sfa, "sfa", (P, M))
    _i16(sfb, "sfb", (P, _cdiv(N, 128)))
    if C is not None:
        _f32(C, "C", (M, N))
    _out(D, (M, N))
    _check(lib.dg_fp8_gemm_nt_ue8m0_i16(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(C), _ptr(D), M, N, K,
                                        _stream(stream)))
    return D


def dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_i16(A, sfa, B, sfb, m_indices, C, D, stream=None):
    """Contiguous M-grouped with UE8M0 pairs: sfa int16 [ceil(K/256), M], sfb int16 [G, ceil(K/256), ceil(N/128)]."""
    _fp8(A, "A"); _fp8(B, "B")
    M, K = A.shape
    G, N = B.shape[0], B.shape[1]
    if B.shape[2] != K:
        raise ValueError("A and B must share K")
    P = _cdiv(_cdiv(K, 128), 2)
    _i16(sfa, "sfa", (P, M))
    _i16(sfb, "sfb", (G, P, _cdiv(N, 128)))
    if m_indices.dtype != torch.int32 or tuple(m_indices.shape) != (M,):
        raise ValueError("m_indices must be int32 [M]")
    _dev(m_indices, "m_indices")
    if C is not None:
        _f32(C, "C", (M, N))
    _out(D, (M, N))
    _check(lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_i16(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(m_indices),
                                                             _ptr(C), _ptr(D), M, N, K, G, _stream(stream)))
    return D


def dg_m_grouped_fp8_gemm_nt_masked_ue8m0_i16(A, sfa, B, sfb, masked_m, C, D, stream=None):
    """Masked M-grouped with UE8M0 pairs: sfa int16 [G, ceil(K/256), M_max], sfb int16 [G, ceil(K/256), ceil(N/128)]."""
    _fp8(A, "A"); _fp8(B, "B")
    G, M_max, K = A.shape
    N = B.shape[1]
    if B.shape[0] != G or B.shape[2] != K:
        raise ValueError("B must be [G, N, K]")
    P = _cdiv(_cdiv(K, 128), 2)
    _i16(sfa, "sfa", (G, P, M_max))
    _i16(sfb, "sfb", (G, P, _cdiv(N, 128)))
    if masked_m.dtype != torch.int32 or tuple(masked_m.shape) != (G,):
        raise ValueError("masked_m must be int32 [G]")
    _dev(masked_m, "masked_m")
    if C is not None:
        _f32(C, "C", (G, M_max, N))
    _out(D, (G, M_max, N))
    _check(lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0_i16(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(masked_m),
                                                         _ptr(C), _ptr(D), M_max, N, K, G, _stream(stream)))
    return D


# names without the C prefix, as on the pages
fp8_gemm_nt = dg_fp8_gemm_nt
m_grouped_fp8_gemm_nt_contiguous = dg_m_grouped_fp8_gemm_nt_contiguous
m_grouped_fp8_gemm_nt_masked = dg_m_grouped_fp8_gemm_nt_masked


# ---------------------------------------------------------------- FP8 x FP4
SCALE_FP8_FP4 = 8    # DG_SCALE_FP8_FP4: OR into `kind` of precompile / describe_config


def _i32(t: torch.Tensor, name: str, shape):
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32 (packed UE8M0), got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _dev(t, name)


def _fp4(t: torch.Tensor, name: str, shape):
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must be uint8 (two E2M1 codes per byte), got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _dev(t, name)


def dg_fp8_fp4_gemm_nt(A, sfa, B, sfb, C, D, stream=None):
    """D = C + A @ B.T with E2M1 B.  A [M,K] E4M3, sfa int32 [ceil(K/512),M] (UE8M0, 1x128),
    B uint8 [N,K/2] (element 2i in the low nibble of byte i), sfb int32 [N,K/128] (UE8M0, 1x32)."""
    _fp8(A, "A")
    M, K = A.shape
    N = B.shape[0]
    _fp4(B, "B", (N, K // 2))
    _i32(sfa, "sfa", (_cdiv(_cdiv(K, 128), 4), M))
    _i32(sfb, "sfb", (N, _cdiv(K, 128)))
    if C is not None:
        _f32(C, "C", (M, N))
    _out(D, (M, N))
    _check(lib.dg_fp8_fp4_gemm_nt(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(C), _ptr(D), M, N, K,
                                  _stream(stream)))
    return D


def dg_m_grouped_fp8_fp4_gemm_nt_contiguous(A, sfa, B, sfb, m_indices, C, D, stream=None):
    """Contiguous M-grouped FP8 x FP4: B uint8 [G,N,K/2], sfb int32 [G,N,K/128]; A/sfa as the dense form."""
    _fp8(A, "A")
    M, K = A.shape
    G, N = B.shape[0], B.shape[1]
    _fp4(B, "B", (G, N, K // 2))
    _i32(sfa, "sfa", (_cdiv(_cdiv(K, 128), 4), M))
    _i32(sfb, "sfb", (G, N, _cdiv(K, 128)))
    if m_indices.dtype != torch.int32 or tuple(m_indices.shape) != (M,):
        raise ValueError("m_indices must be int32 [M]")
    _dev(m_indices, "m_indices")
    if C is not None:
        _f32(C, "C", (M, N))
    _out(D, (M, N))
    _check(lib.dg_m_grouped_fp8_fp4_gemm_nt_contiguous(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(m_indices),
                                                       _ptr(C), _ptr(D), M, N, K, G, _stream(stream)))
    return D


def dg_m_grouped_fp8_fp4_gemm_nt_masked(A, sfa, B, sfb, masked_m, C, D, stream=None):
    """Masked M-grouped FP8 x FP4: A [G,M_max,K], sfa int32 [G,ceil(K/512),M_max], B uint8 [G,N,K/2],
    sfb int32 [G,N,K/128]."""
    _fp8(A, "A")
    G, M_max, K = A.shape
    N = B.shape[1]
    _fp4(B, "B", (G, N, K // 2))
    _i32(sfa, "sfa", (G, _cdiv(_cdiv(K, 128), 4), M_max))
    _i32(sfb, "sfb", (G, N, _cdiv(K, 128)))
    if masked_m.dtype != torch.int32 or tuple(masked_m.shape) != (G,):
        raise ValueError("masked_m must be int32 [G]")
    _dev(masked_m, "masked_m")
    if C is not None:
        _f32(C, "C", (G, M_max, N))
    _out(D, (G, M_max, N))
    _check(lib.dg_m_grouped_fp8_fp4_gemm_nt_masked(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(masked_m),
                                                   _ptr(C), _ptr(D), M_max, N, K, G, _stream(stream)))
    return D


fp8_fp4_gemm_nt = dg_fp8_fp4_gemm_nt
m_grouped_fp8_fp4_gemm_nt_contiguous = dg_m_grouped_fp8_fp4_gemm_nt_contiguous
m_grouped_fp8_fp4_gemm_nt_masked = dg_m_grouped_fp8_fp4_gemm_nt_masked


# ---------------------------------------------------------------- K-grouped TN
KIND_K_GROUPED = 3   # `kind` of precompile / describe_config for the K-grouped call


def dg_k_grouped_fp8_gemm_tn_contiguous(A, sfa, B, sfb, ks, C, D, stream=None):
    """D[g] = C[g] + A[seg g]^T @ B[seg g] (FP32 scales per 128 K rows of each column).

    A [K,M] and B [K,N] E4M3 (K outermost), sfa [K/128,M] and sfb [K/128,N] float32,
    ks int32 [G] (device) K rows per group, C None or float32 [G,M,N], D bfloat16 [G,M,N].
    """
    _fp8(A, "A"); _fp8(B, "B")
    K, M = A.shape
    if B.shape[0] != K:
        raise ValueError("A and B must share K (their first dimension)")
    N = B.shape[1]
    _f32(sfa, "sfa", (_cdiv(K, 128), M))
    _f32(sfb, "sfb", (_cdiv(K, 128), N))
    if ks.dtype != torch.int32 or ks.dim() != 1:
        raise ValueError("ks must be int32 [G]")
    _dev(ks, "ks")
    G = ks.shape[0]
    if C is not None:
        _f32(C, "C", (G, M, N))
    _out(D, (G, M, N))
    _check(lib.dg_k_grouped_fp8_gemm_tn_contiguous(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(ks), _ptr(C),
                                                   _ptr(D), M, N, K, G, _stream(stream)))
    return D


k_grouped_fp8_gemm_tn_contiguous = dg_k_grouped_fp8_gemm_tn_contiguous


# ---------------------------------------------------------------- NN / TN / TT layouts
def _dense_layout(layout, A, sfa, B, sfb, C, D, stream):
    """D = C + A_l @ B_l.T where A is stored [M,K] (n) or [K,M] (t) and B [N,K] (t) or [K,N] (n)."""
    _fp8(A, "A"); _fp8(B, "B")
    M, K = A.shape if layout[0] == "n" else A.shape[::-1]
    N, Kb_ = B.shape if layout[1] == "t" else B.shape[::-1]
    if Kb_ != K:
        raise ValueError("A and B must share K")
    _f32(sfa, "sfa", (_cdiv(K, 128), M))
    _f32(sfb, "sfb", (_cdiv(N, 128), _cdiv(K, 128)))
    if C is not None:
        _f32(C, "C", (M, N))
    _out(D, (M, N))
    f = getattr(lib, f"dg_fp8_gemm_{layout}")
    _check(f(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(C), _ptr(D), M, N, K, _stream(stream)))
    return D


def dg_fp8_gemm_nn(A, sfa, B, sfb, C, D, stream=None):
    """A [M,K], B stored [K,N]."""
    return _dense_layout("nn", A, sfa, B, sfb, C, D, stream)


def dg_fp8_gemm_tn(A, sfa, B, sfb, C, D, stream=None):
    """A stored [K,M], B stored [K,N]."""
    return _dense_layout("tn", A, sfa, B, sfb, C, D, stream)


def dg_fp8_gemm_tt(A, sfa, B, sfb, C, D, stream=None):
    """A stored [K,M], B [N,K]."""
    return _dense_layout("tt", A, sfa, B, sfb, C, D, stream)


def dg_m_grouped_fp8_gemm_nn_contiguous(A, sfa, B, sfb, m_indices, C, D, stream=None):
    """Contiguous M-grouped with B stored [G,K,N]; otherwise as the NT form."""
    _fp8(A, "A"); _fp8(B, "B")
    M, K = A.shape
    G, N = B.shape[0], B.shape[2]
    if B.shape[1] != K:
        raise ValueError("B must be [G, K, N]")
    _f32(sfa, "sfa", (_cdiv(K, 128), M))
    _f32(sfb, "sfb", (G, _cdiv(N, 128), _cdiv(K, 128)))
    if m_indices.dtype != torch.int32 or tuple(m_indices.shape) != (M,):
        raise ValueError("m_indices must be int32 [M]")
    _dev(m_indices, "m_indices")
    if C is not None:
        _f32(C, "C", (M, N))
    _out(D, (M, N))
    _check(lib.dg_m_grouped_fp8_gemm_nn_contiguous(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(m_indices),
                                                   _ptr(C), _ptr(D), M, N, K, G, _stream(stream)))
    return D


fp8_gemm_nn, fp8_gemm_tn, fp8_gemm_tt = dg_fp8_gemm_nn, dg_fp8_gemm_tn, dg_fp8_gemm_tt
m_grouped_fp8_gemm_nn_contiguous = dg_m_grouped_fp8_gemm_nn_contiguous


# ---------------------------------------------------------------- BF16 x BF16 (unscaled)
KIND_BF16 = 16       # DG_BF16: OR into `kind` of precompile / describe_config (K in elements)


def _bf(t: torch.Tensor, name: str, shape):
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _dev(t, name)


def dg_bf16_gemm_nt(A, B, C, D, stream=None):
    """D = C + A @ B.T in BF16 without scales.  A [M,K], B [N,K] bfloat16, C None or float32 [M,N]."""
    M, K = A.shape
    N = B.shape[0]
    _bf(A, "A", (M, K)); _bf(B, "B", (N, K))
    if C is not None:
        _f32(C, "C", (M, N))
    _out(D, (M, N))
    _check(lib.dg_bf16_gemm_nt(_ptr(A), _ptr(B), _ptr(C), _ptr(D), M, N, K, _stream(stream)))
    return D


def dg_m_grouped_bf16_gemm_nt_contiguous(A, B, m_indices, C, D, stream=None):
    """Contiguous M-grouped BF16: A [M,K], B [G,N,K], m_indices int32 [M]."""
    M, K = A.shape
    G, N = B.shape[0], B.shape[1]
    _bf(A, "A", (M, K)); _bf(B, "B", (G, N, K))
    if m_indices.dtype != torch.int32 or tuple(m_indices.shape) != (M,):
        raise ValueError("m_indices must be int32 [M]")
    _dev(m_indices, "m_indices")
    if C is not None:
        _f32(C, "C", (M, N))
    _out(D, (M, N))
    _check(lib.dg_m_grouped_bf16_gemm_nt_contiguous(_ptr(A), _ptr(B), _ptr(m_indices), _ptr(C), _ptr(D), M, N, K, G,
                                                    _stream(stream)))
    return D


def dg_m_grouped_bf16_gemm_nt_masked(A, B, masked_m, C, D, stream=None):
    """Masked M-grouped BF16: A [G,M_max,K], B [G,N,K], masked_m int32 [G]."""
    G, M_max, K = A.shape
    N = B.shape[1]
    _bf(A, "A", (G, M_max, K)); _bf(B, "B", (G, N, K))
    if masked_m.dtype != torch.int32 or tuple(masked_m.shape) != (G,):
        raise ValueError("masked_m must be int32 [G]")
    _dev(masked_m, "masked_m")
    if C is not None:
        _f32(C, "C", (G, M_max, N))
    _out(D, (G, M_max, N))
    _check(lib.dg_m_grouped_bf16_gemm_nt_masked(_ptr(A), _ptr(B), _ptr(masked_m), _ptr(C), _ptr(D), M_max, N, K, G,
                                                _stream(stream)))
    return D


bf16_gemm_nt = dg_bf16_gemm_nt
m_grouped_bf16_gemm_nt_contiguous = dg_m_grouped_bf16_gemm_nt_contiguous
m_grouped_bf16_gemm_nt_masked = dg_m_grouped_bf16_gemm_nt_masked


# ---------------------------------------------------------------- FP4 x FP4
SCALE_FP4_FP4 = 32   # DG_SCALE_FP4_FP4: OR into `kind` of precompile / describe_config


def dg_fp4_fp4_gemm_nt(A, sfa, B, sfb, C, D, stream=None):
    """D = C + A @ B.T with E2M1 A and B.  A uint8 [M,K/2], sfa int32 [M,K/128], B uint8 [N,K/2],
    sfb int32 [N,K/128] (one UE8M0 scale per 1x32 block of each row, four to a word)."""
    M, K2 = A.shape
    K = 2 * K2
    N = B.shape[0]
    _fp4(A, "A", (M, K2)); _fp4(B, "B", (N, K2))
    _i32(sfa, "sfa", (M, _cdiv(K, 128))); _i32(sfb, "sfb", (N, _cdiv(K, 128)))
    if C is not None:
        _f32(C, "C", (M, N))
    _out(D, (M, N))
    _check(lib.dg_fp4_fp4_gemm_nt(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(C), _ptr(D), M, N, K,
                                  _stream(stream)))
    return D


def dg_m_grouped_fp4_fp4_gemm_nt_contiguous(A, sfa, B, sfb, m_indices, C, D, stream=None):
    """Contiguous M-grouped FP4 x FP4: A [M,K/2], sfa [M,K/128], B [G,N,K/2], sfb [G,N,K/128]."""
    M, K2 = A.shape
    K = 2 * K2
    G, N = B.shape[0], B.shape[1]
    _fp4(A, "A", (M, K2)); _fp4(B, "B", (G, N, K2))
    _i32(sfa, "sfa", (M, _cdiv(K, 128))); _i32(sfb, "sfb", (G, N, _cdiv(K, 128)))
    if m_indices.dtype != torch.int32 or tuple(m_indices.shape) != (M,):
        raise ValueError("m_indices must be int32 [M]")
    _dev(m_indices, "m_indices")
    if C is not None:
        _f32(C, "C", (M, N))
    _out(D, (M, N))
    _check(lib.dg_m_grouped_fp4_fp4_gemm_nt_contiguous(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(m_indices),
                                                       _ptr(C), _ptr(D), M, N, K, G, _stream(stream)))
    return D


def dg_m_grouped_fp4_fp4_gemm_nt_masked(A, sfa, B, sfb, masked_m, C, D, stream=None):
    """Masked M-grouped FP4 x FP4: A [G,M_max,K/2], sfa [G,M_max,K/128], B [G,N,K/2], sfb [G,N,K/128]."""
    G, M_max, K2 = A.shape
    K = 2 * K2
    N = B.shape[1]
    _fp4(A, "A", (G, M_max, K2)); _fp4(B, "B", (G, N, K2))
    _i32(sfa, "sfa", (G, M_max, _cdiv(K, 128))); _i32(sfb, "sfb", (G, N, _cdiv(K, 128)))
    if masked_m.dtype != torch.int32 or tuple(masked_m.shape) != (G,):
        raise ValueError("masked_m must be int32 [G]")
    _dev(masked_m, "masked_m")
    if C is not None:
        _f32(C, "C", (G, M_max, N))
    _out(D, (G, M_max, N))
    _check(lib.dg_m_grouped_fp4_fp4_gemm_nt_masked(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(masked_m),
                                                   _ptr(C), _ptr(D), M_max, N, K, G, _stream(stream)))
    return D


fp4_fp4_gemm_nt = dg_fp4_fp4_gemm_nt
m_grouped_fp4_fp4_gemm_nt_contiguous = dg_m_grouped_fp4_fp4_gemm_nt_contiguous
m_grouped_fp4_fp4_gemm_nt_masked = dg_m_grouped_fp4_fp4_gemm_nt_masked
