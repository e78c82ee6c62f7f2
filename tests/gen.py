"""Seeded synthetic inputs for block-scaled FP8 GEMM, shared by the tests and the bench.

This module draws random numbers and quantises them; it holds none of the
GEMM's arithmetic and imports neither the GPU library nor the oracle.

Quantisation is the caller's job on the pages (DeepGEMM README, "Interfaces /
Notes": FP8 casting and transposition are left to the user), so it lives here,
on the input side:

* A, one scale per 1x128 block (one row, 128 consecutive K), stored MN-major
  as ``sfa[K/128][M]`` (the README's "transposed" LHS-scale layout);
* B, one scale per 128x128 block (128 rows of B, 128 consecutive K), stored
  ``sfb[ceil(N/128)][K/128]``;
* scale = amax/448 in FP32 (1.0 for an all-zero block), code =
  E4M3FN(clamp(x/scale, -448, 448)), rounded to nearest-even by torch's cast.

UE8M0 scales (DeepGEMM README, "Interfaces / Notes": SM100 takes UE8M0 scale
factors, four packed into one 32-bit integer): the block scale is rounded up to
a power of two, s = 2^ceil(log2(amax/448)) (so |x/s| <= 448 still holds), and
its biased exponent e = 127 + log2(s) is stored as one byte; byte j of a word
holds K block 4w + j (unused bytes hold 127).  LHS words are MN-major,
``sfa[ceil(K/512)][M]``; RHS words ``sfb[ceil(N/128)][ceil(K/512)]``.

Workload recipe (sizes from the DeepGEMM launch article, section 3 tables):
values ~N(0,1) from ``torch.Generator('cpu')`` seeded with ``1000 + config``,
drawn in the order A, B, C, masked_m.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

KBLOCK = 128
E4M3_MAX = 448.0


# ---------------------------------------------------------------- quantisers
def _cast_e4m3(x: torch.Tensor) -> torch.Tensor:
    return x.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)


def _block_scale(amax: torch.Tensor, ue8m0: bool):
    """(scale fp32, biased exponent int32 or None) of blocks with the given amax."""
    s = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    if not ue8m0:
        return s, None
    m, e = torch.frexp(s)                      # s = m * 2^e, m in [0.5, 1)
    e = (e - (m == 0.5).to(e.dtype)).to(torch.int32)   # ceil(log2 s)
    return torch.ldexp(torch.ones_like(s), e), e + 127


def pack_ue8m0(e: torch.Tensor) -> torch.Tensor:
    """[..., Kb] biased exponents -> [..., ceil(Kb/4)] int32, byte j = K block 4w + j."""
    *lead, Kb = e.shape
    W = (Kb + 3) // 4
    pad = torch.full((*lead, 4 * W - Kb), 127, dtype=torch.int64)
    b = torch.cat([e.to(torch.int64), pad], dim=-1).reshape(*lead, W, 4)
    w = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)
    return w.to(torch.uint32).view(torch.int32) if hasattr(torch, "uint32") else \
        torch.where(w >= 2**31, w - 2**32, w).to(torch.int32)


def pack_ue8m0_pairs(e: torch.Tensor) -> torch.Tensor:
    """[..., Kb, cols] biased exponents (MN-major) -> [..., ceil(Kb/2), cols] int16:
    byte h of pair word p is K block 2p + h; a missing last block is padded with 127."""
    *lead, Kb, cols = e.shape
    P = (Kb + 1) // 2
    pad = torch.full((*lead, 2 * P - Kb, cols), 127, dtype=torch.int64)
    b = torch.cat([e.to(torch.int64), pad], dim=-2).reshape(*lead, P, 2, cols)
    w = b[..., 0, :] | (b[..., 1, :] << 8)
    return torch.where(w >= 2**15, w - 2**16, w).to(torch.int16)


def unpack_ue8m0_exponents(words: torch.Tensor, Kb: int) -> torch.Tensor:
    """[..., ceil(Kb/4)] int32 words -> [..., Kb] biased exponents (byte j = K block 4w + j)."""
    w = words.to(torch.int64) & 0xFFFFFFFF
    b = torch.stack([(w >> (8 * j)) & 0xFF for j in range(4)], dim=-1)
    return b.reshape(*words.shape[:-1], -1)[..., :Kb]


def to_ue8m0_pairs(p: "Problem") -> "Problem":
    """The same problem with its four-to-a-word UE8M0 scales repacked as int16 pairs
    along K, both stored MN-major: sfa [.., ceil(Kb/2), M], sfb [.., ceil(Kb/2), Nb]."""
    assert p.ue8m0 and not p.fp4, "a packed-UE8M0 FP8 problem"
    Kb = p.K // KBLOCK
    ea = unpack_ue8m0_exponents(p.sfa.transpose(-1, -2), Kb).transpose(-1, -2)   # [.., Kb, M]
    eb = unpack_ue8m0_exponents(p.sfb, Kb).transpose(-1, -2)                      # [.., Kb, Nb]
    return dataclasses.replace(p, sfa=pack_ue8m0_pairs(ea).contiguous(), sfb=pack_ue8m0_pairs(eb).contiguous(),
                               ue8m0=False, ue8m0_pairs=True)


def quantize_1x128(x: torch.Tensor, ue8m0: bool = False):
    """x [..., M, K] fp32 -> (codes u8 [..., M, K], sfa [..., K/128, M] fp32, or
    [..., ceil(K/512), M] int32 packed UE8M0)."""
    *lead, M, K = x.shape
    assert K % KBLOCK == 0
    xb = x.reshape(*lead, M, K // KBLOCK, KBLOCK)
    amax = xb.abs().amax(dim=-1)
    s, e = _block_scale(amax, ue8m0)
    q = _cast_e4m3(xb / s.unsqueeze(-1)).reshape(*lead, M, K)
    if ue8m0:
        return q.contiguous(), pack_ue8m0(e).transpose(-1, -2).contiguous()
    return q.contiguous(), s.transpose(-1, -2).contiguous()


def quantize_128x128(x: torch.Tensor, ue8m0: bool = False):
    """x [..., N, K] fp32 -> (codes u8 [..., N, K], sfb [..., ceil(N/128), K/128] fp32,
    or [..., ceil(N/128), ceil(K/512)] int32 packed UE8M0)."""
    *lead, N, K = x.shape
    assert K % KBLOCK == 0
    Nb = (N + KBLOCK - 1) // KBLOCK
    pad = Nb * KBLOCK - N
    xp = torch.nn.functional.pad(x, (0, 0, 0, pad)) if pad else x
    xb = xp.reshape(*lead, Nb, KBLOCK, K // KBLOCK, KBLOCK)
    amax = xb.abs().amax(dim=(-3, -1))
    s, e = _block_scale(amax, ue8m0)
    q = _cast_e4m3(xb / s[..., :, None, :, None]).reshape(*lead, Nb * KBLOCK, K)
    if ue8m0:
        return q[..., :N, :].contiguous(), pack_ue8m0(e).contiguous()
    return q[..., :N, :].contiguous(), s.contiguous()


# ---------------------------------------------------------------- FP4 weights
E2M1_MAX = 6.0
E2M1_MAGS = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _cast_e2m1(x: torch.Tensor) -> torch.Tensor:
    """Nearest E2M1 code (ties to the even mantissa) of x, |x| <= 6: u8 nibbles 0..15."""
    a = x.abs().clamp(max=E2M1_MAX)
    d = (a.unsqueeze(-1) - E2M1_MAGS).abs()
    best = d.min(dim=-1, keepdim=True).values
    # among equally near magnitudes take the even code (mantissa bit 0)
    cand = (d == best) & (torch.arange(8) % 2 == 0)
    code = torch.where(cand.any(-1), cand.to(torch.int8).argmax(-1), (d == best).to(torch.int8).argmax(-1))
    return (code.to(torch.uint8) | ((x < 0).to(torch.uint8) << 3)) * (a > 0).to(torch.uint8)


def quantize_fp4_1x32(x: torch.Tensor):
    """x [..., N, K] fp32 -> (E2M1 pairs u8 [..., N, K/2], sfb int32 [..., N, K/128]).

    One UE8M0 scale per 1x32 block, s = 2^ceil(log2(amax/6)); element 2i in the low
    nibble of byte i; byte j of word [n][kb] holds the scale of K elements 128 kb + 32 j ..+32.
    """
    *lead, N, K = x.shape
    assert K % KBLOCK == 0
    xb = x.reshape(*lead, N, K // 32, 32)
    amax = xb.abs().amax(dim=-1)
    s = torch.where(amax > 0, amax / E2M1_MAX, torch.ones_like(amax))
    m, e = torch.frexp(s)
    e = (e - (m == 0.5).to(e.dtype)).to(torch.int32)
    s = torch.ldexp(torch.ones_like(s), e)
    q = _cast_e2m1(xb / s.unsqueeze(-1)).reshape(*lead, N, K)
    packed = (q[..., 0::2] | (q[..., 1::2] << 4)).contiguous()
    words = pack_ue8m0((e + 127).reshape(*lead, N, K // KBLOCK, 4).reshape(*lead, N * (K // KBLOCK), 4))
    return packed, words.reshape(*lead, N, K // KBLOCK).contiguous()


# ---------------------------------------------------------------- problems
@dataclasses.dataclass
class Problem:
    kind: str                       # "dense" | "contiguous" | "masked"
    A: torch.Tensor                 # u8 codes
    sfa: torch.Tensor               # fp32
    B: torch.Tensor                 # u8 codes
    sfb: torch.Tensor               # fp32
    C: Optional[torch.Tensor] = None
    m_indices: Optional[torch.Tensor] = None   # int32 [M] (contiguous)
    masked_m: Optional[torch.Tensor] = None    # int32 [G] (masked)
    seed: int = 0
    ue8m0: bool = False             # sfa/sfb are packed UE8M0 int32 words
    fp4: bool = False               # B holds E2M1 pairs [.., N, K/2], sfb [.., N, K/128] words (1x32 blocks)
    bf16: bool = False              # A and B are torch.bfloat16, no scales (sfa, sfb None)
    fp4a: bool = False              # A also E2M1 pairs [.., M, K/2] with sfa [.., M, K/128] words (FP4 x FP4)
    ue8m0_pairs: bool = False       # sfa/sfb are UE8M0 pairs in int16, MN-major ([.., ceil(Kb/2), M|Nb])

    @property
    def M(self):
        return self.A.shape[-2]

    @property
    def N(self):
        return self.B.shape[-2]

    @property
    def K(self):
        return self.A.shape[-1] * (2 if self.fp4a else 1)    # FP4 A holds two codes a byte

    @property
    def G(self):
        return 1 if self.kind == "dense" else self.B.shape[0]


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def _quant_b(b, ue8m0, fp4):
    return quantize_fp4_1x32(b) if fp4 else quantize_128x128(b, ue8m0)


def _quant_a(a, ue8m0, fp4x4):
    return quantize_fp4_1x32(a) if fp4x4 else quantize_1x128(a, ue8m0)


def make_dense(M, N, K, seed, with_c=False, ue8m0=False, fp4=False, fp4x4=False) -> Problem:
    """fp4: FP8 x FP4 (B as E2M1 with 1x32 UE8M0 scales; A with UE8M0 scales);
    fp4x4: FP4 x FP4 (A as E2M1 with 1x32 UE8M0 scales per row, like B)."""
    fp4 = fp4 or fp4x4
    ue8m0 = ue8m0 or fp4
    g = _gen(seed)
    a = torch.randn(M, K, generator=g, dtype=torch.float32)
    b = torch.randn(N, K, generator=g, dtype=torch.float32)
    c = torch.randn(M, N, generator=g, dtype=torch.float32) if with_c else None
    A, sfa = _quant_a(a, ue8m0, fp4x4)
    del a
    B, sfb = _quant_b(b, ue8m0, fp4)
    del b
    return Problem("dense", A, sfa, B, sfb, C=c, seed=seed, ue8m0=ue8m0, fp4=fp4, fp4a=fp4x4)


def make_contiguous(group_rows, N, K, seed, with_c=False, pad_rows=None, align=128, ue8m0=False,
                    fp4=False, fp4x4=False) -> Problem:
    """Experts' tokens concatenated along M, each segment padded to ``align`` rows.

    group_rows[g] valid rows for expert g; padding rows get index -1.  With
    ``pad_rows`` given, that many extra -1 rows are appended.
    """
    G = len(group_rows)
    g = _gen(seed)
    seg = [((r + align - 1) // align) * align for r in group_rows]
    M = sum(seg) + (pad_rows or 0)
    a = torch.randn(M, K, generator=g, dtype=torch.float32)
    b = torch.randn(G, N, K, generator=g, dtype=torch.float32)
    c = torch.randn(M, N, generator=g, dtype=torch.float32) if with_c else None
    idx = torch.full((M,), -1, dtype=torch.int32)
    off = 0
    for e, (r, s) in enumerate(zip(group_rows, seg)):
        idx[off:off + r] = e
        off += s
    fp4 = fp4 or fp4x4
    ue8m0 = ue8m0 or fp4
    A, sfa = _quant_a(a, ue8m0, fp4x4)
    del a
    B, sfb = _quant_b(b, ue8m0, fp4)
    del b
    return Problem("contiguous", A, sfa, B, sfb, C=c, m_indices=idx, seed=seed, ue8m0=ue8m0, fp4=fp4, fp4a=fp4x4)


def make_masked(G, M_max, N, K, seed, with_c=False, masked_m=None, ue8m0=False, fp4=False,
                fp4x4=False) -> Problem:
    g = _gen(seed)
    a = torch.randn(G, M_max, K, generator=g, dtype=torch.float32)
    b = torch.randn(G, N, K, generator=g, dtype=torch.float32)
    c = torch.randn(G, M_max, N, generator=g, dtype=torch.float32) if with_c else None
    if masked_m is None:
        mm = torch.randint(0, M_max + 1, (G,), generator=g, dtype=torch.int32)
    else:
        mm = torch.as_tensor(masked_m, dtype=torch.int32)
    fp4 = fp4 or fp4x4
    ue8m0 = ue8m0 or fp4
    A, sfa = _quant_a(a, ue8m0, fp4x4)
    del a
    B, sfb = _quant_b(b, ue8m0, fp4)
    del b
    return Problem("masked", A, sfa, B, sfb, C=c, masked_m=mm, seed=seed, ue8m0=ue8m0, fp4=fp4, fp4a=fp4x4)


# ---------------------------------------------------------------- BF16 x BF16 (unscaled)
def _bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16).contiguous()


def make_bf16(kind, seed, M=None, N=None, K=None, with_c=False, group_rows=None, G=None, M_max=None,
              masked_m=None, pad_rows=None) -> Problem:
    """BF16 operands ~N(0,1) rounded to BF16 (nearest-even), drawn A, B, C, masked_m."""
    g = _gen(seed)
    if kind == "dense":
        a = torch.randn(M, K, generator=g)
        b = torch.randn(N, K, generator=g)
        c = torch.randn(M, N, generator=g) if with_c else None
        return Problem("dense", _bf16(a), None, _bf16(b), None, C=c, seed=seed, bf16=True)
    if kind == "contiguous":
        G = len(group_rows)
        seg = [((r + 127) // 128) * 128 for r in group_rows]
        Mt = sum(seg) + (pad_rows or 0)
        a = torch.randn(Mt, K, generator=g)
        b = torch.randn(G, N, K, generator=g)
        c = torch.randn(Mt, N, generator=g) if with_c else None
        idx = torch.full((Mt,), -1, dtype=torch.int32)
        off = 0
        for e, (r, sg) in enumerate(zip(group_rows, seg)):
            idx[off:off + r] = e
            off += sg
        return Problem("contiguous", _bf16(a), None, _bf16(b), None, C=c, m_indices=idx, seed=seed, bf16=True)
    a = torch.randn(G, M_max, K, generator=g)
    b = torch.randn(G, N, K, generator=g)
    c = torch.randn(G, M_max, N, generator=g) if with_c else None
    mm = torch.randint(0, M_max + 1, (G,), generator=g, dtype=torch.int32) if masked_m is None else \
        torch.as_tensor(masked_m, dtype=torch.int32)
    return Problem("masked", _bf16(a), None, _bf16(b), None, C=c, masked_m=mm, seed=seed, bf16=True)


# ---------------------------------------------------------------- K-grouped TN
@dataclasses.dataclass
class KGroupedProblem:
    """K-grouped TN: both operands K-outermost, one FP32 scale per 128 K rows of each column."""
    A: torch.Tensor                 # u8 codes [K, M]
    sfa: torch.Tensor               # fp32 [K/128, M]
    B: torch.Tensor                 # u8 codes [K, N]
    sfb: torch.Tensor               # fp32 [K/128, N]
    ks: torch.Tensor                # int32 [G]: K rows of each group, consecutive segments
    C: Optional[torch.Tensor] = None   # fp32 [G, M, N]
    seed: int = 0
    kind: str = "k_grouped"

    @property
    def M(self):
        return self.A.shape[1]

    @property
    def N(self):
        return self.B.shape[1]

    @property
    def K(self):
        return self.A.shape[0]

    @property
    def G(self):
        return self.ks.shape[0]


def quantize_k_blocks(x: torch.Tensor):
    """x [K, M] fp32 -> (codes u8 [K, M], scales fp32 [K/128, M]): one scale per 128 K rows
    of each column (the 1x128 rule of quantize_1x128, applied along K)."""
    q, s = quantize_1x128(x.t().contiguous())
    return q.t().contiguous(), s


def make_k_grouped(ks, M, N, seed, with_c=False) -> KGroupedProblem:
    """Groups g of ks[g] K rows each (multiples of 128), values ~N(0,1) drawn A, B, C."""
    g = _gen(seed)
    K = int(sum(ks))
    a = torch.randn(K, M, generator=g, dtype=torch.float32)
    b = torch.randn(K, N, generator=g, dtype=torch.float32)
    c = torch.randn(len(ks), M, N, generator=g, dtype=torch.float32) if with_c else None
    A, sfa = quantize_k_blocks(a)
    del a
    B, sfb = quantize_k_blocks(b)
    del b
    return KGroupedProblem(A, sfa, B, sfb, torch.as_tensor(ks, dtype=torch.int32), C=c, seed=seed)


def make_k_grouped_workload() -> KGroupedProblem:
    """The weight gradient of the contiguous workload: 4 experts x 8192 tokens, M = 4096, N = 7168."""
    return make_k_grouped([8192] * 4, 4096, 7168, seed=1005)


WORKLOAD_NAMES_EXTRA = {"kg": "k_grouped_4x8192_4096x7168"}


# ---------------------------------------------------------------- the five workloads
# (shapes: DeepGEMM launch article, section 3, dense table and MoE table)
WORKLOADS = {
    0: dict(kind="dense", M=64, N=2112, K=7168),
    1: dict(kind="dense", M=128, N=24576, K=1536),
    "1c": dict(kind="dense", M=128, N=24576, K=1536, with_c=True),
    2: dict(kind="dense", M=4096, N=7168, K=16384),
    3: dict(kind="contiguous", G=4, rows_per_group=8192, N=4096, K=7168),
    4: dict(kind="masked", G=4, M_max=256, N=7168, K=2048),
}

WORKLOAD_NAMES = {
    0: "dense_64x2112x7168",
    1: "dense_128x24576x1536",
    "1c": "dense_128x24576x1536_plusC",
    2: "dense_4096x7168x16384",
    3: "contiguous_4x8192x4096x7168",
    4: "masked_4x256x7168x2048",
}


def workload_seed(cfg) -> int:
    return 1000 + (1 if cfg == "1c" else int(cfg))


def make_workload(cfg, ue8m0=False, fp4=False, fp4x4=False, ue8m0_pairs=False) -> Problem:
    if ue8m0_pairs:
        return to_ue8m0_pairs(make_workload(cfg, ue8m0=True))
    c = WORKLOADS[cfg]
    seed = workload_seed(cfg)
    kw = dict(ue8m0=ue8m0, fp4=fp4, fp4x4=fp4x4)
    if c["kind"] == "dense":
        return make_dense(c["M"], c["N"], c["K"], seed, with_c=c.get("with_c", False), **kw)
    if c["kind"] == "contiguous":
        return make_contiguous([c["rows_per_group"]] * c["G"], c["N"], c["K"], seed, **kw)
    return make_masked(c["G"], c["M_max"], c["N"], c["K"], seed, **kw)


# ---------------------------------------------------------------- structured inputs for pins
E4M3_ONE = 0x38


def integer_codes(shape, gen, max_abs=16):
    """E4M3 codes of random integers in [-max_abs, max_abs] (all exactly representable)."""
    v = torch.randint(-max_abs, max_abs + 1, shape, generator=gen).to(torch.float32)
    return _cast_e4m3(v)


def pow2_scales(shape, gen, lo=-3, hi=3):
    e = torch.randint(lo, hi + 1, shape, generator=gen).to(torch.float32)
    return torch.pow(2.0, e)


def sentinel_like(shape, seed) -> torch.Tensor:
    """Seeded random 16-bit patterns (viewed as bf16) used to prefill D."""
    g = _gen(seed)
    return torch.randint(0, 1 << 16, shape, generator=g, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)


def to_numpy(p: Problem):
    """numpy views of a problem's tensors (for the oracle)."""
    f = lambda t: None if t is None else (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).numpy()
    return dict(A=f(p.A), sfa=f(p.sfa), B=f(p.B), sfb=f(p.sfb), C=f(p.C),
                m_indices=f(p.m_indices), masked_m=f(p.masked_m))
