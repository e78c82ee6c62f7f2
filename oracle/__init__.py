"""CPU oracle for block-scaled FP8 GEMM (D = C + A.B^T, NT) and its M-grouped forms.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The GPU library never
imports, links or calls anything here, and nothing here imports the GPU library.

The arithmetic lives in ``oracle.c`` (plain C, FP64, one pthread per core);
this module only compiles it and marshals numpy arrays through ctypes.
Semantics and citations are in the header of ``oracle.c``:

* DeepGEMM README, "Interfaces / Notes": D = C + A @ B.T for the NT layout,
  FP32 scale factors, LHS scales stored MN-major.
* DeepGEMM launch article, section 2: per-block promotion into a
  higher-precision accumulator.
* DeepGEMM README, "Grouped GEMM (contiguous layout)" and "(masked layout)".
* DeepGEMM README, "Interfaces / Notes" (SM100) and the Ascend 950 article:
  UE8M0 scale factors packed four to a 32-bit word; unpacked here to the FP32
  scales they stand for (exactly), after which the GEMM is the FP32-scale one.
* DeepGEMM-Ascend hub page (precision table: FP8 x FP4) and README news
  2026.04.16 (FP8xFP4 GEMM; FP4 weights with UE8M0 scale factors): E2M1
  weights with one UE8M0 scale per 1x32 block, A as in the UE8M0 form.
* DeepGEMM README, "Grouped GEMM (contiguous layout)": the K-axis grouped TN
  call for the MoE weight backward (M and N fixed), both operands K-outermost
  with one FP32 scale per 128 K rows of each column.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

KBLOCK = 128


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile ``oracle.c`` (or a given copy of it) into a shared library."""
    cmd = ["gcc", "-O2", "-Wall", "-shared", "-fPIC", "-pthread", "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _needs_build() -> bool:
    return (not os.path.exists(_LIB_PATH)
            or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC))


def _declare(lib):
    c = ctypes
    p = c.c_void_p
    lib.oracle_e4m3_value.restype = c.c_double
    lib.oracle_e4m3_value.argtypes = [c.c_uint8]
    lib.oracle_e4m3_table.restype = None
    lib.oracle_e4m3_table.argtypes = [p]
    lib.oracle_bf16_rne.restype = c.c_uint16
    lib.oracle_bf16_rne.argtypes = [c.c_double]
    lib.oracle_ue8m0_value.restype = c.c_double
    lib.oracle_ue8m0_value.argtypes = [c.c_uint8]
    lib.oracle_ue8m0_unpack_mn_major.restype = None
    lib.oracle_ue8m0_unpack_mn_major.argtypes = [p, c.c_int64, c.c_int, c.c_int64, p]
    lib.oracle_ue8m0_unpack_k_major.restype = None
    lib.oracle_ue8m0_unpack_k_major.argtypes = [p, c.c_int64, c.c_int, p]
    lib.oracle_ue8m0_pairs_unpack_lhs.restype = None
    lib.oracle_ue8m0_pairs_unpack_lhs.argtypes = [p, c.c_int64, c.c_int, c.c_int64, p]
    lib.oracle_ue8m0_pairs_unpack_rhs.restype = None
    lib.oracle_ue8m0_pairs_unpack_rhs.argtypes = [p, c.c_int64, c.c_int, c.c_int64, p]
    lib.oracle_e2m1_value.restype = c.c_double
    lib.oracle_e2m1_value.argtypes = [c.c_uint8]
    lib.oracle_fp8_fp4_gemm.restype = c.c_int
    lib.oracle_fp8_fp4_gemm.argtypes = [c.c_int, p, p, p, p, p, p, c.c_int64, c.c_int, c.c_int, c.c_int,
                                        p, c.c_int64, p, p, c.c_int]
    lib.oracle_k_grouped_tn.restype = c.c_int
    lib.oracle_k_grouped_tn.argtypes = [p, p, p, p, p, p, c.c_int64, c.c_int, c.c_int, c.c_int,
                                        p, c.c_int64, p, p, c.c_int]
    lib.oracle_fp4_fp4_gemm.restype = c.c_int
    lib.oracle_fp4_fp4_gemm.argtypes = lib.oracle_fp8_fp4_gemm.argtypes
    lib.oracle_bf16_value.restype = c.c_double
    lib.oracle_bf16_value.argtypes = [c.c_uint16]
    lib.oracle_bf16_gemm.restype = c.c_int
    lib.oracle_bf16_gemm.argtypes = [c.c_int, p, p, p, p, c.c_int64, c.c_int, c.c_int, c.c_int,
                                     p, c.c_int64, p, p, c.c_int]
    lib.oracle_default_threads.restype = c.c_int
    lib.oracle_default_threads.argtypes = []
    lib.oracle_fp8_gemm_nt.restype = c.c_int
    lib.oracle_fp8_gemm_nt.argtypes = [p, p, p, p, p, c.c_int64, c.c_int, c.c_int,
                                       p, c.c_int64, p, c.c_int]
    for name in ("oracle_m_grouped_contiguous", "oracle_m_grouped_masked"):
        f = getattr(lib, name)
        f.restype = c.c_int
        f.argtypes = [p, p, p, p, p, p, c.c_int64, c.c_int, c.c_int, c.c_int,
                      p, c.c_int64, p, p, c.c_int]
    return lib


def load(path: str | None = None):
    """Load the oracle library (building it first if missing or stale).

    With ``path`` given, load that file (used for deliberately broken copies
    in the negative-control tests) without caching it.
    """
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        if _needs_build():
            build()
        _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _rows(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, int(r.size)


class Oracle:
    """numpy front-end over one loaded copy of the oracle library."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else load()

    def threads(self) -> int:
        return int(self.lib.oracle_default_threads())

    def e4m3_table(self) -> np.ndarray:
        out = np.empty(256, dtype=np.float64)
        self.lib.oracle_e4m3_table(_ptr(out))
        return out

    def bf16_rne(self, x: np.ndarray) -> np.ndarray:
        x = np.asarray(x, dtype=np.float64).ravel()
        return np.array([self.lib.oracle_bf16_rne(float(v)) for v in x], dtype=np.uint16)

    # ---------------------------------------------------------- UE8M0 scales
    def ue8m0_value(self, e: int) -> float:
        return float(self.lib.oracle_ue8m0_value(int(e)))

    def unpack_sfa_ue8m0(self, packed, Kb: int) -> np.ndarray:
        """[..., ceil(Kb/4), M] int32 -> [..., Kb, M] fp32 (MN-major LHS scales)."""
        pk = _c(packed, np.int32)
        *lead, W, M = pk.shape
        assert W == (Kb + 3) // 4
        n = int(np.prod(lead)) if lead else 1
        out = np.empty((*lead, Kb, M), dtype=np.float32)
        self.lib.oracle_ue8m0_unpack_mn_major(_ptr(pk), n, Kb, M, _ptr(out))
        return out

    def unpack_sfb_ue8m0(self, packed, Kb: int) -> np.ndarray:
        """[..., Nb, ceil(Kb/4)] int32 -> [..., Nb, Kb] fp32 (K-contiguous RHS scales)."""
        pk = _c(packed, np.int32)
        *lead, W = pk.shape
        assert W == (Kb + 3) // 4
        n = int(np.prod(lead)) if lead else 1
        out = np.empty((*lead, Kb), dtype=np.float32)
        self.lib.oracle_ue8m0_unpack_k_major(_ptr(pk), n, Kb, _ptr(out))
        return out

    def fp8_gemm_nt_ue8m0(self, A, sfa, B, sfb, C=None, rows=None, threads=0):
        """Dense form with packed UE8M0 scales sfa [ceil(Kb/4), M], sfb [Nb, ceil(Kb/4)]."""
        Kb = np.shape(A)[-1] // KBLOCK
        return self.fp8_gemm_nt(A, self.unpack_sfa_ue8m0(sfa, Kb), B, self.unpack_sfb_ue8m0(sfb, Kb), C, rows,
                                threads)

    def m_grouped_contiguous_ue8m0(self, A, sfa, B, sfb, m_indices, C=None, rows=None, threads=0):
        Kb = np.shape(A)[-1] // KBLOCK
        return self.m_grouped_contiguous(A, self.unpack_sfa_ue8m0(sfa, Kb), B, self.unpack_sfb_ue8m0(sfb, Kb),
                                         m_indices, C, rows, threads)

    def m_grouped_masked_ue8m0(self, A, sfa, B, sfb, masked_m, C=None, rows=None, threads=0):
        Kb = np.shape(A)[-1] // KBLOCK
        return self.m_grouped_masked(A, self.unpack_sfa_ue8m0(sfa, Kb), B, self.unpack_sfb_ue8m0(sfb, Kb),
                                     masked_m, C, rows, threads)

    # ---------------------------------------------------------- UE8M0 pairs (int16, MN-major)
    def unpack_sfa_ue8m0_pairs(self, pairs, Kb: int) -> np.ndarray:
        """[..., ceil(Kb/2), M] int16 -> [..., Kb, M] fp32 (MN-major LHS scales)."""
        pk = _c(pairs, np.int16)
        *lead, P, M = pk.shape
        assert P == (Kb + 1) // 2
        n = int(np.prod(lead)) if lead else 1
        out = np.empty((*lead, Kb, M), dtype=np.float32)
        self.lib.oracle_ue8m0_pairs_unpack_lhs(_ptr(pk), n, Kb, M, _ptr(out))
        return out

    def unpack_sfb_ue8m0_pairs(self, pairs, Kb: int) -> np.ndarray:
        """[..., ceil(Kb/2), Nb] int16 (MN-major) -> [..., Nb, Kb] fp32 (the FP32 sfb layout)."""
        pk = _c(pairs, np.int16)
        *lead, P, Nb = pk.shape
        assert P == (Kb + 1) // 2
        n = int(np.prod(lead)) if lead else 1
        out = np.empty((*lead, Nb, Kb), dtype=np.float32)
        self.lib.oracle_ue8m0_pairs_unpack_rhs(_ptr(pk), n, Kb, Nb, _ptr(out))
        return out

    def fp8_gemm_nt_ue8m0_pairs(self, A, sfa, B, sfb, C=None, rows=None, threads=0):
        """Dense form with UE8M0 pairs: sfa int16 [ceil(Kb/2), M], sfb int16 [ceil(Kb/2), Nb]."""
        Kb = np.shape(A)[-1] // KBLOCK
        return self.fp8_gemm_nt(A, self.unpack_sfa_ue8m0_pairs(sfa, Kb), B, self.unpack_sfb_ue8m0_pairs(sfb, Kb), C,
                                rows, threads)

    # ---------------------------------------------------------- FP8 x FP4
    def e2m1_value(self, nibble: int) -> float:
        return float(self.lib.oracle_e2m1_value(int(nibble)))

    def fp8_fp4_gemm(self, kind: str, A, sfa, B, sfb, group_info=None, C=None, rows=None, threads=0):
        """(D FP64 [rows, N], computed [rows]) of an FP8 x FP4 GEMM.

        kind "dense" | "contiguous" | "masked".  A E4M3 codes ([M,K] or [G,M_max,K]); sfa packed
        UE8M0 words ([ceil(Kb/4),M] or [G,ceil(Kb/4),M_max]); B E2M1 pairs [(G,)N,K/2] u8 (element
        2i in the low nibble of byte i); sfb [(G,)N,Kb] int32 (byte j: K elements 128 kb + 32 j ..+32).
        """
        A = _c(A, np.uint8); B = _c(B, np.uint8)
        sfa = _c(sfa, np.int32); sfb = _c(sfb, np.int32); C = _c(C, np.float32)
        gi = _c(group_info, np.int32)
        k = {"dense": 0, "contiguous": 1, "masked": 2}[kind]
        if kind == "masked":
            G, M, K = A.shape
        else:
            M, K = A.shape
            G = B.shape[0] if B.ndim == 3 else 1
        N = B.shape[-2]
        r, nr = _rows(rows)
        n_out = nr if r is not None else (G * M if kind == "masked" else M)
        out = np.empty((n_out, N), dtype=np.float64)
        comp = np.zeros(n_out, dtype=np.uint8)
        rc = self.lib.oracle_fp8_fp4_gemm(k, _ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(gi), _ptr(C), M, N, K, G,
                                          _ptr(r), nr, _ptr(out), _ptr(comp), threads)
        if rc != 0:
            raise ValueError("oracle_fp8_fp4_gemm: bad sizes")
        return out, comp.astype(bool)

    # ---------------------------------------------------------- BF16 x BF16
    def bf16_value(self, bits: int) -> float:
        return float(self.lib.oracle_bf16_value(int(bits)))

    def bf16_gemm(self, kind: str, A, B, group_info=None, C=None, rows=None, threads=0):
        """(D FP64 [rows, N], computed [rows]) of the unscaled BF16 GEMM D = C + A . B^T.

        A, B: BF16 bit patterns as uint16 (or int16), A [M,K] (masked [G,M_max,K]), B [(G,)N,K];
        group_info: m_indices (contiguous) or masked_m (masked).
        """
        A = _c(np.asarray(A).view(np.uint16), np.uint16); B = _c(np.asarray(B).view(np.uint16), np.uint16)
        C = _c(C, np.float32); gi = _c(group_info, np.int32)
        k = {"dense": 0, "contiguous": 1, "masked": 2}[kind]
        if kind == "masked":
            G, M, K = A.shape
        else:
            M, K = A.shape
            G = B.shape[0] if B.ndim == 3 else 1
        N = B.shape[-2]
        r, nr = _rows(rows)
        n_out = nr if r is not None else (G * M if kind == "masked" else M)
        out = np.empty((n_out, N), dtype=np.float64)
        comp = np.zeros(n_out, dtype=np.uint8)
        rc = self.lib.oracle_bf16_gemm(k, _ptr(A), _ptr(B), _ptr(gi), _ptr(C), M, N, K, G, _ptr(r), nr, _ptr(out),
                                       _ptr(comp), threads)
        if rc != 0:
            raise ValueError("oracle_bf16_gemm: bad sizes")
        return out, comp.astype(bool)

    # ---------------------------------------------------------- NN / TN / TT layouts
    def fp8_gemm_layout(self, layout: str, A, sfa, B, sfb, C=None, m_indices=None, G=1, rows=None, threads=0):
        """(D FP64, computed) of D = C + A_l . B_l^T for a stored layout (DeepGEMM README,
        "Normal dense GEMM": fp8_gemm_{nt, nn, tn, tt}; "Grouped GEMM (contiguous layout)":
        m_grouped_fp8_gemm_{nt, nn}_contiguous).

        The first letter is how A is stored (N: [M, K], T: [K, M]), the second how B is
        (T: [N, K] or [G, N, K], N: [K, N] or [G, K, N]); the scales keep their logical
        layouts (sfa [K/128, M], sfb [(G,) ceil(N/128), K/128]).  A stored operand is put
        back in the NT arrangement with a plain transpose, then the NT definition applies.
        m_indices given: the contiguous grouped form.
        """
        a_t, b_n = layout[0] == "t", layout[1] == "n"
        A = np.ascontiguousarray(np.asarray(A).T) if a_t else np.asarray(A)
        B = np.asarray(B)
        if b_n:
            B = np.ascontiguousarray(np.swapaxes(B, -1, -2))
        if m_indices is None:
            out = self.fp8_gemm_nt(A, sfa, B, sfb, C, rows=rows, threads=threads)
            return out, np.ones(out.shape[0], dtype=bool)
        return self.m_grouped_contiguous(A, sfa, B, sfb, m_indices, C, rows=rows, threads=threads)

    # ---------------------------------------------------------- K-grouped TN
    def k_grouped_tn(self, A, sfa, B, sfb, ks, C=None, rows=None, threads=0):
        """(D FP64 [rows, N], computed [rows]) of the K-grouped TN GEMM.

        A [K,M] and B [K,N] E4M3 codes (K outermost), sfa [K/128,M] and sfb [K/128,N] FP32,
        ks [G] int32 K rows per group (consecutive segments), C None or [G,M,N] FP32.
        Rows are flat g*M + m (all G*M by default); every row is computed.
        """
        A = _c(A, np.uint8); B = _c(B, np.uint8)
        sfa = _c(sfa, np.float32); sfb = _c(sfb, np.float32); C = _c(C, np.float32)
        ks = _c(ks, np.int32)
        K, M = A.shape
        N = B.shape[1]
        G = ks.shape[0]
        r, nr = _rows(rows)
        n_out = nr if r is not None else G * M
        out = np.empty((n_out, N), dtype=np.float64)
        comp = np.zeros(n_out, dtype=np.uint8)
        rc = self.lib.oracle_k_grouped_tn(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(ks), _ptr(C), M, N, K, G,
                                          _ptr(r), nr, _ptr(out), _ptr(comp), threads)
        if rc != 0:
            raise ValueError("oracle_k_grouped_tn: bad sizes")
        return out, comp.astype(bool)

    def fp4_fp4_gemm(self, kind: str, A, sfa, B, sfb, group_info=None, C=None, rows=None, threads=0):
        """(D FP64 [rows, N], computed [rows]) of an FP4 x FP4 GEMM: A E2M1 pairs [M,K/2] (masked
        [G,M_max,K/2]) with sfa int32 [M,K/128] (masked [G,M_max,K/128]), B and sfb as fp8_fp4_gemm."""
        A = _c(A, np.uint8); B = _c(B, np.uint8)
        sfa = _c(sfa, np.int32); sfb = _c(sfb, np.int32); C = _c(C, np.float32)
        gi = _c(group_info, np.int32)
        k = {"dense": 0, "contiguous": 1, "masked": 2}[kind]
        if kind == "masked":
            G, M, K2 = A.shape
        else:
            M, K2 = A.shape
            G = B.shape[0] if B.ndim == 3 else 1
        K = 2 * K2
        N = B.shape[-2]
        r, nr = _rows(rows)
        n_out = nr if r is not None else (G * M if kind == "masked" else M)
        out = np.empty((n_out, N), dtype=np.float64)
        comp = np.zeros(n_out, dtype=np.uint8)
        rc = self.lib.oracle_fp4_fp4_gemm(k, _ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(gi), _ptr(C), M, N, K, G,
                                          _ptr(r), nr, _ptr(out), _ptr(comp), threads)
        if rc != 0:
            raise ValueError("oracle_fp4_fp4_gemm: bad sizes")
        return out, comp.astype(bool)

    def fp8_gemm_nt(self, A, sfa, B, sfb, C=None, rows=None, threads=0):
        """D (FP64) of the dense form; A [M,K] u8, sfa [K/128,M], B [N,K] u8, sfb [Nb,Kb]."""
        A = _c(A, np.uint8); B = _c(B, np.uint8)
        sfa = _c(sfa, np.float32); sfb = _c(sfb, np.float32); C = _c(C, np.float32)
        M, K = A.shape
        N = B.shape[0]
        r, nr = _rows(rows)
        out = np.empty(((nr if r is not None else M), N), dtype=np.float64)
        rc = self.lib.oracle_fp8_gemm_nt(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(C),
                                         M, N, K, _ptr(r), nr, _ptr(out), threads)
        if rc != 0:
            raise ValueError("oracle_fp8_gemm_nt: bad sizes")
        return out

    def m_grouped_contiguous(self, A, sfa, B, sfb, m_indices, C=None, rows=None, threads=0):
        """(D FP64 [rows,N], computed u8 [rows]) of the contiguous grouped form."""
        A = _c(A, np.uint8); B = _c(B, np.uint8)
        sfa = _c(sfa, np.float32); sfb = _c(sfb, np.float32); C = _c(C, np.float32)
        mi = _c(m_indices, np.int32)
        M, K = A.shape
        G, N = B.shape[0], B.shape[1]
        r, nr = _rows(rows)
        n_out = nr if r is not None else M
        out = np.empty((n_out, N), dtype=np.float64)
        comp = np.zeros(n_out, dtype=np.uint8)
        rc = self.lib.oracle_m_grouped_contiguous(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(mi),
                                                  _ptr(C), M, N, K, G, _ptr(r), nr, _ptr(out),
                                                  _ptr(comp), threads)
        if rc != 0:
            raise ValueError("oracle_m_grouped_contiguous: bad sizes")
        return out, comp.astype(bool)

    def m_grouped_masked(self, A, sfa, B, sfb, masked_m, C=None, rows=None, threads=0):
        """(D FP64 [rows,N], computed u8 [rows]) of the masked grouped form.

        A [G,M_max,K], sfa [G,K/128,M_max], B [G,N,K], sfb [G,Nb,Kb]; rows are flat
        indices g*M_max + m (None: all rows, output shaped [G*M_max, N]).
        """
        A = _c(A, np.uint8); B = _c(B, np.uint8)
        sfa = _c(sfa, np.float32); sfb = _c(sfb, np.float32); C = _c(C, np.float32)
        mm = _c(masked_m, np.int32)
        G, M_max, K = A.shape
        N = B.shape[1]
        r, nr = _rows(rows)
        n_out = nr if r is not None else G * M_max
        out = np.empty((n_out, N), dtype=np.float64)
        comp = np.zeros(n_out, dtype=np.uint8)
        rc = self.lib.oracle_m_grouped_masked(_ptr(A), _ptr(sfa), _ptr(B), _ptr(sfb), _ptr(mm),
                                              _ptr(C), M_max, N, K, G, _ptr(r), nr, _ptr(out),
                                              _ptr(comp), threads)
        if rc != 0:
            raise ValueError("oracle_m_grouped_masked: bad sizes")
        return out, comp.astype(bool)
