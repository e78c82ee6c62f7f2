"""Pins of the CPU oracle against things other than itself (all CPU-only).

Each pin is chosen so that a plausible slip in the oracle (a dropped K block,
the FNUZ reading of E4M3, a wrong scale index or layout, a transposed operand,
a lost sign, an ignored C, a wrong group or mask rule) fails at least one of
them; ``test_oracle_mutants.py`` plants those slips and checks that they do.

Pins used:
* library routines: torch's float8_e4m3fn -> float32 decode, torch's
  float32 -> bfloat16 cast, numpy FP64 matmul of dequantised operands;
* exact integer arithmetic: int64 matmul of codes x 512;
* closed forms: all-ones codes, one-hot rows, sign flip, power-of-two scaling;
* group/mask invariants from the grouped-layout sections of the DeepGEMM README.
"""
import json
import os

import numpy as np
import pytest
import torch

from tests import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_decode_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)


def dequant_ref(p, dec):
    """numpy FP64 (A*sfa) @ (B*sfb)^T (+C) for a dense problem; also the |.| bound."""
    A = dec[p.A.numpy()]
    B = dec[p.B.numpy()]
    M, K = A.shape
    N = B.shape[0]
    sa = np.repeat(p.sfa.numpy().astype(np.float64).T, 128, axis=1)            # [M, K]
    sb = np.repeat(np.repeat(p.sfb.numpy().astype(np.float64), 128, axis=0)[:N], 128, axis=1)
    Ad, Bd = A * sa, B * sb
    ref = Ad @ Bd.T
    mag = np.abs(Ad) @ np.abs(Bd).T
    if p.C is not None:
        ref = ref + p.C.numpy().astype(np.float64)
        mag = mag + np.abs(p.C.numpy().astype(np.float64))
    return ref, mag


# ------------------------------------------------------------------ E4M3 decode
def test_e4m3_table_matches_torch_decode(oracle):
    t = oracle.e4m3_table()
    r = torch_decode_table()
    assert np.array_equal(np.isnan(t), np.isnan(r))
    ok = ~np.isnan(t)
    assert np.array_equal(t[ok], r[ok])
    # signed zero as well
    assert np.array_equal(np.signbit(t[ok]), np.signbit(r[ok]))


def test_e4m3_table_format_facts(oracle):
    """Facts fixed by the E4M3FN format (see tests/golden/e4m3_points.json)."""
    t = oracle.e4m3_table()
    with open(os.path.join(GOLDEN, "e4m3_points.json")) as f:
        pts = json.load(f)
    for code, val in pts["points"].items():
        c = int(code, 16)
        if val == "nan":
            assert np.isnan(t[c])
        else:
            assert t[c] == float(val), (code, t[c], val)
    assert int(np.isnan(t).sum()) == 2
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                     # strictly increasing 0x00..0x7E
    assert np.all(t[0x80:0xFF] == -t[0x00:0x7F])        # sign bit is a pure sign
    fin = t[~np.isnan(t)]
    assert np.all(fin * 512 == np.round(fin * 512))     # every value is a multiple of 2^-9
    assert np.max(np.abs(fin)) == 448.0                 # amax/448 scaling hits the top code


# ------------------------------------------------------------------ BF16 rounding
def test_bf16_rne_matches_torch_cast(oracle):
    g = torch.Generator().manual_seed(7)
    x = torch.randn(4000, generator=g) * torch.pow(2.0, torch.randint(-30, 30, (4000,), generator=g).float())
    special = torch.tensor([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 1.0078125 + 2 ** -9, 3.3895313892515355e38,
                            3.4028234663852886e38, 1e-38, 9.183549615799121e-41, 1.1754943508222875e-38,
                            -2.5, 65504.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], dtype=torch.float32)
    x = torch.cat([x, special])
    want = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_rne(x.numpy().astype(np.float64))
    assert np.array_equal(got, want)


# ------------------------------------------------------------------ dense: brute force
@pytest.mark.parametrize("M", [1, 2, 3, 5, 127, 128, 129])
@pytest.mark.parametrize("N", [1, 3, 128, 129])
@pytest.mark.parametrize("K", [128, 384])
def test_dense_vs_numpy_dequant_matmul(oracle, M, N, K):
    p = gen.make_dense(M, N, K, seed=M * 1000 + N * 10 + K, with_c=(M + N) % 2 == 1)
    d = oracle.fp8_gemm_nt(p.A.numpy(), p.sfa.numpy(), p.B.numpy(), p.sfb.numpy(),
                           None if p.C is None else p.C.numpy())
    ref, mag = dequant_ref(p, torch_decode_table())
    assert np.all(np.abs(d - ref) <= 1e-13 * mag + 1e-300)


def test_dense_integer_data_exact_vs_int64(oracle):
    """Integer-valued codes, power-of-two scales: D is exact; compare to int64 matmul."""
    g = torch.Generator().manual_seed(11)
    M, N, K = 37, 300, 512
    A = gen.integer_codes((M, K), g)
    B = gen.integer_codes((N, K), g)
    sfa = gen.pow2_scales((K // 128, M), g)
    sfb = gen.pow2_scales(((N + 127) // 128, K // 128), g)
    d = oracle.fp8_gemm_nt(A.numpy(), sfa.numpy(), B.numpy(), sfb.numpy())
    dec = torch_decode_table()
    Ai = np.rint(dec[A.numpy()] * 512).astype(np.int64)
    Bi = np.rint(dec[B.numpy()] * 512).astype(np.int64)
    exact = np.zeros((M, N), dtype=np.float64)
    for kb in range(K // 128):
        S = Ai[:, kb * 128:(kb + 1) * 128] @ Bi[:, kb * 128:(kb + 1) * 128].T   # exact int64
        sa = sfa.numpy()[kb][:, None].astype(np.float64)
        sb = sfb.numpy()[np.arange(N) // 128, kb][None, :].astype(np.float64)
        exact += S.astype(np.float64) / 2.0 ** 18 * sa * sb
    assert np.array_equal(d, exact)


# ------------------------------------------------------------------ dense: closed forms
def test_all_ones_closed_form(oracle):
    g = torch.Generator().manual_seed(3)
    M, N, K = 19, 260, 640
    A = torch.full((M, K), gen.E4M3_ONE, dtype=torch.uint8)
    B = torch.full((N, K), gen.E4M3_ONE, dtype=torch.uint8)
    sfa = torch.rand(K // 128, M, generator=g) + 0.5
    sfb = torch.rand((N + 127) // 128, K // 128, generator=g) + 0.5
    C = torch.randn(M, N, generator=g)
    d = oracle.fp8_gemm_nt(A.numpy(), sfa.numpy(), B.numpy(), sfb.numpy(), C.numpy())
    nb = np.arange(N) // 128
    want = 128.0 * (sfa.numpy().astype(np.float64).T @ sfb.numpy().astype(np.float64)[nb].T) + C.numpy()
    assert np.allclose(d, want, rtol=1e-14, atol=0)
    # constant scales: K * sA * sB exactly
    d2 = oracle.fp8_gemm_nt(A.numpy(), np.full((K // 128, M), 0.25, np.float32), B.numpy(),
                            np.full(((N + 127) // 128, K // 128), 2.0, np.float32))
    assert np.all(d2 == K * 0.25 * 2.0)


def test_one_hot_rows(oracle):
    """A[m, pi(m)] = 1: D[m, n] = sfa[pi/128][m] * sfb[n/128][pi/128] * e4m3(B[n, pi])."""
    g = torch.Generator().manual_seed(5)
    M, N, K = 40, 200, 768
    pi = torch.randint(0, K, (M,), generator=g)
    A = torch.zeros(M, K, dtype=torch.uint8)
    A[torch.arange(M), pi] = gen.E4M3_ONE
    p = gen.make_dense(1, N, K, seed=99)
    sfa = torch.rand(K // 128, M, generator=g) + 0.1
    d = oracle.fp8_gemm_nt(A.numpy(), sfa.numpy(), p.B.numpy(), p.sfb.numpy())
    dec = torch_decode_table()
    pin = pi.numpy()
    kb = pin // 128
    want = (sfa.numpy()[kb, np.arange(M)][:, None].astype(np.float64)
            * p.sfb.numpy()[np.arange(N)[None, :] // 128, kb[:, None]].astype(np.float64)
            * dec[p.B.numpy()[:, pin].T])
    assert np.array_equal(d, want)


def test_sign_flip_and_pow2_scaling(oracle):
    p = gen.make_dense(33, 257, 384, seed=21)
    A = p.A.numpy()
    base = oracle.fp8_gemm_nt(A, p.sfa.numpy(), p.B.numpy(), p.sfb.numpy())
    flipped = np.where(A != 0, A ^ 0x80, A).astype(np.uint8)
    neg = oracle.fp8_gemm_nt(flipped, p.sfa.numpy(), p.B.numpy(), p.sfb.numpy())
    assert np.array_equal(neg, -base)
    up = oracle.fp8_gemm_nt(A, p.sfa.numpy() * 8.0, p.B.numpy(), p.sfb.numpy())
    assert np.array_equal(up, 8.0 * base)
    # swapping the operands transposes D when both sides carry 128x128 block
    # scales: D[m,n] = sum_kb SA[m/128][kb] SB[n/128][kb] S[m,n,kb] is symmetric
    g = torch.Generator().manual_seed(23)
    Ma, Nb_, K = 256, 384, 512
    A2 = gen.integer_codes((Ma, K), g, max_abs=448)
    B2 = gen.integer_codes((Nb_, K), g, max_abs=448)
    SA = (torch.rand(Ma // 128, K // 128, generator=g) + 0.1).numpy()
    SB = (torch.rand(Nb_ // 128, K // 128, generator=g) + 0.1).numpy()
    sfa_a = np.ascontiguousarray(np.repeat(SA, 128, axis=0).T)          # [Kb, Ma]
    sfa_b = np.ascontiguousarray(np.repeat(SB, 128, axis=0).T)          # [Kb, Nb_]
    d_ab = oracle.fp8_gemm_nt(A2.numpy(), sfa_a, B2.numpy(), SB)
    d_ba = oracle.fp8_gemm_nt(B2.numpy(), sfa_b, A2.numpy(), SA)
    assert np.array_equal(d_ab, d_ba.T)


def test_rows_subset_equals_full(oracle):
    p = gen.make_dense(70, 150, 256, seed=31, with_c=True)
    full = oracle.fp8_gemm_nt(p.A.numpy(), p.sfa.numpy(), p.B.numpy(), p.sfb.numpy(), p.C.numpy())
    rows = np.array([69, 0, 13, 13, 64])
    sub = oracle.fp8_gemm_nt(p.A.numpy(), p.sfa.numpy(), p.B.numpy(), p.sfb.numpy(), p.C.numpy(), rows=rows)
    assert np.array_equal(sub, full[rows])
    one = oracle.fp8_gemm_nt(p.A.numpy(), p.sfa.numpy(), p.B.numpy(), p.sfb.numpy(), p.C.numpy(), threads=1)
    assert np.array_equal(one, full)


def test_c_is_added(oracle):
    p = gen.make_dense(9, 140, 256, seed=41, with_c=True)
    with_c = oracle.fp8_gemm_nt(p.A.numpy(), p.sfa.numpy(), p.B.numpy(), p.sfb.numpy(), p.C.numpy())
    without = oracle.fp8_gemm_nt(p.A.numpy(), p.sfa.numpy(), p.B.numpy(), p.sfb.numpy())
    assert np.allclose(with_c - without, p.C.numpy().astype(np.float64), rtol=0, atol=1e-9)


def test_bad_sizes_rejected(oracle):
    A = np.zeros((4, 100), np.uint8)
    with pytest.raises(ValueError):
        oracle.fp8_gemm_nt(A, np.ones((1, 4), np.float32), np.zeros((4, 100), np.uint8), np.ones((1, 1), np.float32))


# ------------------------------------------------------------------ contiguous grouped
def test_contiguous_segments_equal_dense(oracle):
    p = gen.make_contiguous([128, 0, 256, 100], N=200, K=256, seed=51, with_c=True, pad_rows=128)
    npd = gen.to_numpy(p)
    d, comp = oracle.m_grouped_contiguous(npd["A"], npd["sfa"], npd["B"], npd["sfb"], npd["m_indices"], npd["C"])
    idx = npd["m_indices"]
    assert np.array_equal(comp, (idx >= 0) & (idx < 4))
    assert np.all(np.isnan(d[~comp]))
    for g in range(4):
        rows = np.nonzero(idx == g)[0]
        if rows.size == 0:
            continue
        dd = oracle.fp8_gemm_nt(npd["A"], npd["sfa"], npd["B"][g], npd["sfb"][g], npd["C"], rows=rows)
        assert np.array_equal(d[rows], dd)


def test_contiguous_group_independence_and_permutation(oracle):
    p = gen.make_contiguous([128, 128, 128], N=130, K=256, seed=52)
    npd = gen.to_numpy(p)
    d, _ = oracle.m_grouped_contiguous(npd["A"], npd["sfa"], npd["B"], npd["sfb"], npd["m_indices"])
    B2 = npd["B"].copy()
    B2[1] = np.where(B2[1] != 0, B2[1] ^ 0x80, B2[1])
    d2, _ = oracle.m_grouped_contiguous(npd["A"], npd["sfa"], B2, npd["sfb"], npd["m_indices"])
    idx = npd["m_indices"]
    assert np.array_equal(d2[idx != 1], d[idx != 1])
    assert np.array_equal(d2[idx == 1], -d[idx == 1])
    # relabel the groups: rows follow their expert's weights
    perm = np.array([2, 0, 1])
    idx_p = perm[idx].astype(np.int32)
    Bp = np.empty_like(npd["B"]); sfbp = np.empty_like(npd["sfb"])
    Bp[perm] = npd["B"]; sfbp[perm] = npd["sfb"]
    d3, _ = oracle.m_grouped_contiguous(npd["A"], npd["sfa"], Bp, sfbp, idx_p)
    assert np.array_equal(d3, d)
    # G = 1 with all rows valid is the dense form
    d4, _ = oracle.m_grouped_contiguous(npd["A"], npd["sfa"], npd["B"][:1], npd["sfb"][:1],
                                        np.zeros_like(idx))
    assert np.array_equal(d4, oracle.fp8_gemm_nt(npd["A"], npd["sfa"], npd["B"][0], npd["sfb"][0]))


# ------------------------------------------------------------------ masked grouped
def test_masked_rows_and_groups(oracle):
    G, M_max, N, K = 4, 70, 150, 256
    p = gen.make_masked(G, M_max, N, K, seed=61, with_c=True, masked_m=[0, 70, 33, 200])
    npd = gen.to_numpy(p)
    d, comp = oracle.m_grouped_masked(npd["A"], npd["sfa"], npd["B"], npd["sfb"], npd["masked_m"], npd["C"])
    valid = np.array([0, 70, 33, 70])
    want_comp = (np.arange(M_max)[None, :] < valid[:, None]).ravel()
    assert np.array_equal(comp, want_comp)
    assert np.all(np.isnan(d[~comp]))
    for g in range(G):
        if valid[g] == 0:
            continue
        dd = oracle.fp8_gemm_nt(npd["A"][g], npd["sfa"][g], npd["B"][g], npd["sfb"][g], npd["C"][g])
        assert np.array_equal(d.reshape(G, M_max, N)[g, :valid[g]], dd[:valid[g]])


def test_masked_negative_and_subset(oracle):
    G, M_max, N, K = 2, 16, 40, 128
    p = gen.make_masked(G, M_max, N, K, seed=62, masked_m=[-5, 16])
    npd = gen.to_numpy(p)
    d, comp = oracle.m_grouped_masked(npd["A"], npd["sfa"], npd["B"], npd["sfb"], npd["masked_m"])
    assert not comp[:M_max].any() and comp[M_max:].all()
    rows = np.array([31, 16, 3])
    ds, cs = oracle.m_grouped_masked(npd["A"], npd["sfa"], npd["B"], npd["sfb"], npd["masked_m"], rows=rows)
    assert np.array_equal(cs, comp[rows])
    assert np.array_equal(ds[cs], d[rows][cs])


# ------------------------------------------------------------------ UE8M0 scales
def test_ue8m0_points_from_format(oracle):
    """Decode of single E8M0 bytes against values fixed by the OCP MX definition."""
    pts = json.load(open(os.path.join(GOLDEN, "ue8m0_points.json")))["points"]
    for code, val in pts.items():
        got = oracle.ue8m0_value(int(code, 16))
        if val == "nan":
            assert np.isnan(got), code
        else:
            assert got == float(val), (code, got, val)
    # monotone, each step exactly doubles (no gaps or repeats in 0..254)
    vals = np.array([oracle.ue8m0_value(e) for e in range(255)])
    assert np.all(vals[1:] == 2.0 * vals[:-1])


def test_ue8m0_packing_byte_order_and_layouts(oracle):
    """Byte j of a word is K block 4w + j; LHS words [W][M] (MN-major), RHS [Nb][W]."""
    Kb, M = 6, 3
    e = np.array([[120 + kb + 10 * m for m in range(M)] for kb in range(Kb)])   # [Kb][M]
    words = np.zeros((2, M), dtype=np.int64)
    for kb in range(Kb):
        words[kb // 4] |= e[kb] << (8 * (kb % 4))
    words[1] |= (77 << 16) | (78 << 24)                 # bytes past the last K block: ignored
    sfa = oracle.unpack_sfa_ue8m0(words.astype(np.uint32).view(np.int32), Kb)
    assert sfa.shape == (Kb, M)
    assert np.array_equal(sfa, np.ldexp(1.0, e - 127).astype(np.float32))
    sfb = oracle.unpack_sfb_ue8m0(words.T.copy().astype(np.uint32).view(np.int32), Kb)   # [M as Nb][W]
    assert np.array_equal(sfb, np.ldexp(1.0, e.T - 127).astype(np.float32))
    # grouped leading dimension
    g2 = np.stack([words, words + 1]).astype(np.uint32).view(np.int32)
    u = oracle.unpack_sfa_ue8m0(g2, Kb)
    assert u.shape == (2, Kb, M) and np.array_equal(u[0], sfa)
    assert np.array_equal(u[1, 0], np.ldexp(1.0, e[0] + 1 - 127).astype(np.float32))


def test_ue8m0_all_ones_closed_form(oracle):
    """All-ones codes: D[m,n] = 128 * sum_kb 2^(ea[kb,m]-127) * 2^(eb[n/128,kb]-127) + C, exactly."""
    g = torch.Generator().manual_seed(8)
    M, N, K = 7, 300, 896
    Kb, Nb = K // 128, (N + 127) // 128
    ea = torch.randint(120, 135, (Kb, M), generator=g)
    eb = torch.randint(118, 131, (Nb, Kb), generator=g)
    sfa = gen.pack_ue8m0(ea.T).T.contiguous()               # [W][M]
    sfb = gen.pack_ue8m0(eb)                                # [Nb][W]
    A = torch.full((M, K), gen.E4M3_ONE, dtype=torch.uint8)
    B = torch.full((N, K), gen.E4M3_ONE, dtype=torch.uint8)
    C = torch.randn(M, N, generator=g)
    d = oracle.fp8_gemm_nt_ue8m0(A.numpy(), sfa.numpy(), B.numpy(), sfb.numpy(), C.numpy())
    want = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            want[m, n] = 128.0 * sum(2.0 ** (int(ea[kb, m]) - 127) * 2.0 ** (int(eb[n // 128, kb]) - 127)
                                     for kb in range(Kb)) + float(C[m, n])
    assert np.array_equal(d, want)


# ------------------------------------------------------------------ UE8M0 pairs in int16 (MN-major)
def _hex16(rows):
    return np.array([[int(h, 16) for h in r] for r in rows], dtype=np.uint16).view(np.int16)


def test_ue8m0_pairs_worked_example(oracle):
    """A hand-written example of the pair packing (tests/golden/ue8m0_pairs_layout.json):
    byte h of word p = K block 2p + h, MN-major for both operands, trailing byte ignored."""
    ex = json.load(open(os.path.join(GOLDEN, "ue8m0_pairs_layout.json")))
    Kb = ex["Kb"]
    sfa = oracle.unpack_sfa_ue8m0_pairs(_hex16(ex["lhs_pairs_hex"]), Kb)        # [Kb][M]
    assert np.array_equal(sfa, np.ldexp(1.0, np.array(ex["lhs_scales_log2"])).astype(np.float32))
    sfb = oracle.unpack_sfb_ue8m0_pairs(_hex16(ex["rhs_pairs_hex"]), Kb)        # [Nb][Kb]
    assert np.array_equal(sfb, np.ldexp(1.0, np.array(ex["rhs_scales_log2"])).astype(np.float32))


def test_ue8m0_pairs_equal_quads(oracle):
    """The same exponents packed two to an int16 (MN-major) and four to an int32 unpack to
    the same FP32 scales, and the GEMMs agree bit for bit (odd Kb, grouped lead dims)."""
    g = torch.Generator().manual_seed(12)
    Kb, M, Nb = 7, 5, 3
    ea = torch.randint(100, 150, (2, Kb, M), generator=g)
    eb = torch.randint(100, 150, (2, Nb, Kb), generator=g)
    quad_a = gen.pack_ue8m0(ea.transpose(-1, -2)).transpose(-1, -2).contiguous()   # [2][W][M]
    quad_b = gen.pack_ue8m0(eb)                                                     # [2][Nb][W]
    pair_a = gen.pack_ue8m0_pairs(ea)                                               # [2][P][M]
    pair_b = gen.pack_ue8m0_pairs(eb.transpose(-1, -2))                             # [2][P][Nb]
    assert tuple(pair_a.shape) == (2, 4, M) and tuple(pair_b.shape) == (2, 4, Nb)
    assert np.array_equal(oracle.unpack_sfa_ue8m0_pairs(pair_a.numpy(), Kb),
                          oracle.unpack_sfa_ue8m0(quad_a.numpy(), Kb))
    assert np.array_equal(oracle.unpack_sfb_ue8m0_pairs(pair_b.numpy(), Kb),
                          oracle.unpack_sfb_ue8m0(quad_b.numpy(), Kb))
    p = gen.make_dense(9, 300, 7 * 128, seed=13, with_c=True, ue8m0=True)
    q = gen.to_ue8m0_pairs(p)
    d = gen.to_numpy(p)
    want = oracle.fp8_gemm_nt_ue8m0(d["A"], d["sfa"], d["B"], d["sfb"], d["C"])
    got = oracle.fp8_gemm_nt_ue8m0_pairs(d["A"], q.sfa.numpy(), d["B"], q.sfb.numpy(), d["C"])
    assert np.array_equal(got, want)


def test_ue8m0_pairs_all_ones_closed_form(oracle):
    """All-ones codes with pair-packed scales: D = 128 * sum_kb 2^(ea-127) 2^(eb-127) + C, exactly."""
    g = torch.Generator().manual_seed(14)
    M, N, K = 6, 260, 640
    Kb, Nb = K // 128, (N + 127) // 128
    ea = torch.randint(118, 134, (Kb, M), generator=g)
    eb = torch.randint(121, 132, (Kb, Nb), generator=g)            # MN-major: [Kb][Nb]
    A = torch.full((M, K), gen.E4M3_ONE, dtype=torch.uint8)
    B = torch.full((N, K), gen.E4M3_ONE, dtype=torch.uint8)
    C = torch.randn(M, N, generator=g)
    d = oracle.fp8_gemm_nt_ue8m0_pairs(A.numpy(), gen.pack_ue8m0_pairs(ea).numpy(), B.numpy(),
                                       gen.pack_ue8m0_pairs(eb).numpy(), C.numpy())
    want = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            want[m, n] = 128.0 * sum(2.0 ** (int(ea[kb, m]) - 127) * 2.0 ** (int(eb[kb, n // 128]) - 127)
                                     for kb in range(Kb)) + float(C[m, n])
    assert np.array_equal(d, want)


def test_ue8m0_generator_scales(oracle):
    """The UE8M0 quantiser picks the least power of two >= amax/448 and keeps codes in range."""
    p = gen.make_dense(33, 260, 768, seed=41, ue8m0=True)
    x = torch.randn(33, 768, generator=gen._gen(41))
    sfa = oracle.unpack_sfa_ue8m0(p.sfa.numpy(), 6)                  # [Kb][M]
    amax = x.reshape(33, 6, 128).abs().amax(-1).numpy().T / 448.0    # [Kb][M]
    assert np.all(sfa >= amax) and np.all(sfa < 2 * amax)
    assert np.all(np.log2(sfa) == np.round(np.log2(sfa)))
    dec = torch_decode_table()
    assert np.all(np.abs(dec[p.A.numpy()]) <= 448.0)


# ------------------------------------------------------------------ FP8 x FP4
def _e2m1_golden():
    pts = json.load(open(os.path.join(GOLDEN, "e2m1_points.json")))["points"]
    return np.array([float(pts[f"0x{c:x}"]) for c in range(16)])


def test_e2m1_points_from_format(oracle):
    table = _e2m1_golden()
    for c in range(16):
        got = oracle.e2m1_value(c)
        assert got == table[c] and np.signbit(got) == np.signbit(table[c]), c


def _fp4_dequant_ref(p):
    """numpy FP64 dequantise-and-matmul of a dense FP8 x FP4 problem, from the golden
    E2M1 table, torch's E4M3 decode and 2^(e-127) per byte (independent of the oracle)."""
    dec8 = torch_decode_table()
    t4 = _e2m1_golden()
    A = dec8[p.A.numpy()]
    M, K = A.shape
    Bb = p.B.numpy()
    B = np.empty((Bb.shape[0], K))
    B[:, 0::2] = t4[Bb & 0xF]
    B[:, 1::2] = t4[Bb >> 4]
    wa = p.sfa.numpy().view(np.uint32)                       # [W][M]
    ea = np.stack([(wa[kb // 4] >> (8 * (kb % 4))) & 0xFF for kb in range(K // 128)])   # [Kb][M]
    wb = p.sfb.numpy().view(np.uint32)                       # [N][Kb]
    eb = np.stack([(wb >> (8 * j)) & 0xFF for j in range(4)], axis=-1).reshape(wb.shape[0], -1)   # [N][K/32]
    sa = np.repeat(np.ldexp(1.0, ea.astype(np.int64) - 127).T, 128, axis=1)
    sb = np.repeat(np.ldexp(1.0, eb.astype(np.int64) - 127), 32, axis=1)
    ref = (A * sa) @ (B * sb).T
    if p.C is not None:
        ref = ref + p.C.numpy().astype(np.float64)
    return ref


@pytest.mark.parametrize("M,N,K", [(3, 40, 256), (17, 130, 640)])
def test_fp8_fp4_vs_numpy_dequant_matmul(oracle, M, N, K):
    p = gen.make_dense(M, N, K, seed=M + N, with_c=True, fp4=True)
    d, comp = oracle.fp8_fp4_gemm("dense", p.A.numpy(), p.sfa.numpy(), p.B.numpy(), p.sfb.numpy(), C=p.C.numpy())
    assert comp.all()
    ref = _fp4_dequant_ref(p)
    assert np.allclose(d, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_fp8_fp4_nibble_order_and_block_scales(oracle):
    """One-hot pairs: A[m, k] = 1 and B[n, k] = 1 only at k = m + n; B's 32-blocks scaled 2^j."""
    M, N, K = 4, 6, 256
    A = np.zeros((M, K), np.uint8)
    B = np.zeros((N, K // 2), np.uint8)
    for m in range(M):
        A[m, 31 * m + 1] = gen.E4M3_ONE
    for n in range(N):
        k = 31 * (n % M) + 1
        B[n, k // 2] |= (0x2 << 4) if k & 1 else 0x2      # E2M1 1.0 at element k
    sfa = np.full((1, M), 0x7F7F7F7F, np.uint32).view(np.int32)
    eb = np.array([127 + j for j in range(8)])            # per 32-block of K: 2^j
    sfb = np.stack([eb[0:4], eb[4:8]]).astype(np.uint32)
    sfb = (sfb[:, 0] | (sfb[:, 1] << 8) | (sfb[:, 2] << 16) | (sfb[:, 3] << 24)).view(np.int32)
    sfb = np.tile(sfb, (N, 1))
    d, _ = oracle.fp8_fp4_gemm("dense", A, sfa, B, sfb)
    for m in range(M):
        for n in range(N):
            k = 31 * m + 1
            assert d[m, n] == (2.0 ** (k // 32) if n % M == m else 0.0), (m, n, d[m, n])


def test_fp8_fp4_grouped_equal_dense(oracle):
    pm = gen.make_masked(2, 40, 70, 384, seed=5, masked_m=[40, 17], fp4=True)
    d, comp = oracle.fp8_fp4_gemm("masked", pm.A.numpy(), pm.sfa.numpy(), pm.B.numpy(), pm.sfb.numpy(),
                                  pm.masked_m.numpy())
    assert comp.sum() == 57
    for g in range(2):
        dg_, _ = oracle.fp8_fp4_gemm("dense", pm.A[g].numpy(), pm.sfa[g].numpy(), pm.B[g].numpy(), pm.sfb[g].numpy())
        valid = int(pm.masked_m[g])
        assert np.array_equal(d[g * 40:g * 40 + valid], dg_[:valid])
    pc = gen.make_contiguous([128, 0, 100], 70, 256, seed=6, fp4=True)
    d, comp = oracle.fp8_fp4_gemm("contiguous", pc.A.numpy(), pc.sfa.numpy(), pc.B.numpy(), pc.sfb.numpy(),
                                  pc.m_indices.numpy())
    idx = pc.m_indices.numpy()
    assert np.array_equal(comp, (idx >= 0))
    for e in (0, 2):
        rows = np.nonzero(idx == e)[0]
        de, _ = oracle.fp8_fp4_gemm("dense", pc.A.numpy()[rows], pc.sfa.numpy()[:, rows], pc.B[e].numpy(),
                                    pc.sfb[e].numpy())
        assert np.array_equal(d[rows], de)


def test_fp4_quantiser_rounds_to_nearest(oracle):
    """Every E2M1 code the generator picks is a nearest representable value of x / s."""
    g = torch.Generator().manual_seed(9)
    x = torch.randn(8, 256, generator=g) * 3
    B, sfb = gen.quantize_fp4_1x32(x)
    t4 = _e2m1_golden()
    q = np.empty((8, 256))
    q[:, 0::2] = t4[B.numpy() & 0xF]
    q[:, 1::2] = t4[B.numpy() >> 4]
    w = sfb.numpy().view(np.uint32)
    e = np.stack([(w >> (8 * j)) & 0xFF for j in range(4)], -1).reshape(8, -1)
    s = np.repeat(np.ldexp(1.0, e.astype(np.int64) - 127), 32, axis=1)
    y = x.numpy().astype(np.float64) / s
    mags = np.unique(np.abs(t4))
    err = np.abs(np.abs(y)[..., None] - mags).min(-1)
    assert np.allclose(np.abs(np.abs(q) - np.abs(y)), err)
    assert np.all(np.abs(y) <= 6.0)


# ------------------------------------------------------------------ K-grouped TN
def _kg_dequant_ref(p):
    """numpy FP64 per group: C_g + (A_seg * sfa)^T @ (B_seg * sfb), from torch's E4M3 decode."""
    dec = torch_decode_table()
    A = dec[p.A.numpy()] * np.repeat(p.sfa.numpy().astype(np.float64), 128, axis=0)   # [K, M]
    B = dec[p.B.numpy()] * np.repeat(p.sfb.numpy().astype(np.float64), 128, axis=0)   # [K, N]
    out, off = [], 0
    for g, k in enumerate(p.ks.tolist()):
        d = A[off:off + k].T @ B[off:off + k]
        if p.C is not None:
            d = d + p.C[g].numpy().astype(np.float64)
        out.append(d)
        off += k
    return np.concatenate(out, axis=0)


@pytest.mark.parametrize("ks,M,N", [([128, 256, 0, 384], 37, 129), ([512], 1, 5), ([0, 128], 130, 64)])
def test_k_grouped_vs_numpy_dequant_matmul(oracle, ks, M, N):
    p = gen.make_k_grouped(ks, M, N, seed=sum(ks) + M + N, with_c=True)
    got, comp = oracle.k_grouped_tn(p.A, p.sfa, p.B, p.sfb, p.ks, p.C)
    assert comp.all()
    ref = _kg_dequant_ref(p)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-9)


def test_k_grouped_equals_dense_nt_on_transposed_operands(oracle):
    """With B scales constant over each 128 columns, group g is the dense NT GEMM of
    A_seg^T and B_seg^T with sfb[nb][kb]: the same exact block sums in the same order,
    so the results agree bit for bit (a different oracle entry point, pinned above)."""
    g = torch.Generator().manual_seed(61)
    ks, M, N = [256, 384], 70, 200
    p = gen.make_k_grouped(ks, M, N, seed=62, with_c=True)
    Kb = sum(ks) // 128
    sb_blocks = gen.pow2_scales((Kb, (N + 127) // 128), g)
    sfb = torch.repeat_interleave(sb_blocks, 128, dim=1)[:, :N].contiguous()
    got, _ = oracle.k_grouped_tn(p.A, p.sfa, p.B, sfb, p.ks, p.C)
    got = got.reshape(len(ks), M, N)
    off = 0
    for gi, k in enumerate(ks):
        A = p.A[off:off + k].t().contiguous()
        B = p.B[off:off + k].t().contiguous()
        sfa = p.sfa[off // 128:(off + k) // 128].contiguous()
        sfb_nt = sb_blocks[off // 128:(off + k) // 128].t().contiguous()
        ref = oracle.fp8_gemm_nt(A.numpy(), sfa.numpy(), B.numpy(), sfb_nt.numpy(), p.C[gi].numpy())
        assert np.array_equal(got[gi], ref)
        off += k


def test_k_grouped_operand_swap_transposes(oracle):
    p = gen.make_k_grouped([128, 256], 45, 77, seed=63)
    d, _ = oracle.k_grouped_tn(p.A, p.sfa, p.B, p.sfb, p.ks)
    e, _ = oracle.k_grouped_tn(p.B, p.sfb, p.A, p.sfa, p.ks)
    assert np.array_equal(d.reshape(2, 45, 77), e.reshape(2, 77, 45).transpose(0, 2, 1))


def test_k_grouped_empty_group_and_closed_form(oracle):
    """ks = 0 gives D = C exactly; all-ones codes (E4M3 1.0) with constant power-of-two
    scales give D = ks[g] * sA * sB exactly."""
    ks, M, N = [256, 0, 128], 9, 33
    K = sum(ks)
    ones_a = torch.full((K, M), gen.E4M3_ONE, dtype=torch.uint8)
    ones_b = torch.full((K, N), gen.E4M3_ONE, dtype=torch.uint8)
    sfa = torch.full((K // 128, M), 0.25)
    sfb = torch.full((K // 128, N), 8.0)
    C = torch.randn(3, M, N, generator=torch.Generator().manual_seed(64))
    d, _ = oracle.k_grouped_tn(ones_a, sfa, ones_b, sfb, torch.tensor(ks, dtype=torch.int32), C)
    d = d.reshape(3, M, N)
    for g, k in enumerate(ks):
        assert np.array_equal(d[g], k * 2.0 + C[g].numpy().astype(np.float64))


def test_k_grouped_bad_segments_rejected(oracle):
    p = gen.make_k_grouped([128, 128], 4, 4, seed=65)
    with pytest.raises(ValueError):
        oracle.k_grouped_tn(p.A, p.sfa, p.B, p.sfb, torch.tensor([64, 192], dtype=torch.int32))


# ------------------------------------------------------------------ NN / TN / TT layouts
@pytest.mark.parametrize("layout", ["nt", "nn", "tn", "tt"])
@pytest.mark.parametrize("M,N,K", [(3, 129, 384), (130, 5, 256)])
def test_layouts_vs_numpy_on_stored_operands(oracle, layout, M, N, K):
    """The stored operands, dequantised in place with numpy (no transposes on the oracle's
    side of the comparison): D = C + A_deq @ B_deq^T (nt), A_deq @ B_deq (nn), and so on."""
    p = gen.make_dense(M, N, K, seed=M * N + K, with_c=True)
    dec = torch_decode_table()
    sa = np.repeat(p.sfa.numpy().astype(np.float64), 128, axis=0)                     # [K, M]
    sb = np.repeat(np.repeat(p.sfb.numpy().astype(np.float64), 128, axis=0)[:N], 128, axis=1)   # [N, K]
    A = p.A.numpy() if layout[0] == "n" else np.ascontiguousarray(p.A.numpy().T)      # stored
    B = p.B.numpy() if layout[1] == "t" else np.ascontiguousarray(p.B.numpy().T)
    Ad = dec[A] * (sa.T if layout[0] == "n" else sa)
    Bd = dec[B] * (sb if layout[1] == "t" else sb.T)
    lhs = Ad if layout[0] == "n" else Ad.T                                            # [M, K]
    rhs = Bd.T if layout[1] == "t" else Bd                                            # [K, N]
    ref = lhs @ rhs + p.C.numpy().astype(np.float64)
    got, comp = oracle.fp8_gemm_layout(layout, A, p.sfa.numpy(), B, p.sfb.numpy(), p.C.numpy())
    assert comp.all()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-9)


def test_layout_nn_contiguous_vs_numpy(oracle):
    p = gen.make_contiguous([128, 0, 100], 129, 256, seed=71, with_c=True, pad_rows=128)
    Bn = np.ascontiguousarray(np.swapaxes(p.B.numpy(), -1, -2))                        # [G, K, N]
    got, comp = oracle.fp8_gemm_layout("nn", p.A.numpy(), p.sfa.numpy(), Bn, p.sfb.numpy(), p.C.numpy(),
                                       m_indices=p.m_indices.numpy())
    dec = torch_decode_table()
    Ad = dec[p.A.numpy()] * np.repeat(p.sfa.numpy().astype(np.float64).T, 128, axis=1)
    for m in range(p.M):
        g = int(p.m_indices[m])
        assert comp[m] == (0 <= g < 3)
        if not comp[m]:
            continue
        sb = np.repeat(np.repeat(p.sfb[g].numpy().astype(np.float64), 128, axis=0)[:129], 128, axis=1)  # [N, K]
        ref = Ad[m] @ (dec[Bn[g]] * sb.T) + p.C[m].numpy().astype(np.float64)
        assert np.allclose(got[m], ref, rtol=1e-12, atol=1e-9)


# ------------------------------------------------------------------ BF16 x BF16
def test_bf16_decode_matches_torch_for_every_code(oracle):
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = codes.view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_value(c) for c in range(65536)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    # array_equal cannot see the sign of a zero: 0x8000 must decode to -0
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))
    assert np.signbit(got[0x8000]) and got[0x8000] == 0.0


@pytest.mark.parametrize("M,N,K", [(1, 5, 64), (37, 129, 200), (130, 3, 128)])
def test_bf16_gemm_vs_numpy(oracle, M, N, K):
    p = gen.make_bf16("dense", seed=M + N + K, M=M, N=N, K=K, with_c=True)
    A = p.A.float().numpy().astype(np.float64)
    B = p.B.float().numpy().astype(np.float64)
    ref = A @ B.T + p.C.numpy().astype(np.float64)
    d = gen.to_numpy(p)
    got, comp = oracle.bf16_gemm("dense", d["A"], d["B"], C=d["C"])
    assert comp.all()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-10)


def test_bf16_gemm_integer_data_exact(oracle):
    g = torch.Generator().manual_seed(88)
    A = torch.randint(-20, 21, (50, 256), generator=g)
    B = torch.randint(-20, 21, (70, 256), generator=g)
    got, _ = oracle.bf16_gemm("dense", A.to(torch.bfloat16).view(torch.int16).numpy(),
                              B.to(torch.bfloat16).view(torch.int16).numpy())
    assert np.array_equal(got, (A.to(torch.int64) @ B.to(torch.int64).T).numpy().astype(np.float64))


def test_bf16_grouped_equal_dense(oracle):
    pc = gen.make_bf16("contiguous", seed=81, N=65, K=96, group_rows=[128, 0, 60], with_c=True, pad_rows=128)
    d = gen.to_numpy(pc)
    got, comp = oracle.bf16_gemm("contiguous", d["A"], d["B"], d["m_indices"], d["C"])
    for m in np.flatnonzero(comp):
        g = int(pc.m_indices[m])
        ref, _ = oracle.bf16_gemm("dense", d["A"][m:m + 1], d["B"][g], C=d["C"][m:m + 1])
        assert np.array_equal(got[m], ref[0])
    assert np.array_equal(comp, (pc.m_indices.numpy() >= 0))
    pm = gen.make_bf16("masked", seed=82, N=40, K=64, G=3, M_max=20, masked_m=[20, 0, 7])
    d = gen.to_numpy(pm)
    got, comp = oracle.bf16_gemm("masked", d["A"], d["B"], d["masked_m"])
    assert comp.reshape(3, 20).sum(1).tolist() == [20, 0, 7]
    for g in range(3):
        ref, _ = oracle.bf16_gemm("dense", d["A"][g], d["B"][g])
        valid = comp.reshape(3, 20)[g]
        assert np.array_equal(got.reshape(3, 20, 40)[g][valid], ref[valid])


# ------------------------------------------------------------------ FP4 x FP4
def _e2m1_decode_np(packed):
    """[..., K/2] bytes -> [..., K] values from the golden E2M1 table (element 2i: low nibble)."""
    table = _e2m1_golden()
    vals = np.array([table[c] for c in range(16)])
    lo, hi = packed & 0x0F, packed >> 4
    return vals[np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], -1)]


def _per32_scales(words, K):
    """[..., K/128] int32 words -> [..., K] FP64 scales 2^(e-127), byte j of word kb for K 128kb+32j.."""
    w = words.astype(np.int64) & 0xFFFFFFFF
    e = np.stack([(w >> (8 * j)) & 0xFF for j in range(4)], axis=-1).reshape(*words.shape[:-1], -1)
    return np.repeat(np.ldexp(1.0, e - 127), 32, axis=-1)[..., :K]


@pytest.mark.parametrize("M,N,K", [(1, 5, 128), (17, 130, 384), (129, 3, 256)])
def test_fp4_fp4_vs_numpy_dequant_matmul(oracle, M, N, K):
    p = gen.make_dense(M, N, K, seed=M * 7 + N + K, with_c=True, fp4x4=True)
    A = _e2m1_decode_np(p.A.numpy()) * _per32_scales(p.sfa.numpy(), K)
    B = _e2m1_decode_np(p.B.numpy()) * _per32_scales(p.sfb.numpy(), K)
    ref = A @ B.T + p.C.numpy().astype(np.float64)
    got, comp = oracle.fp4_fp4_gemm("dense", p.A.numpy(), p.sfa.numpy(), p.B.numpy(), p.sfb.numpy(),
                                    C=p.C.numpy())
    assert comp.all()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-9)


def test_fp4_fp4_operand_swap_and_grouped(oracle):
    p = gen.make_dense(40, 72, 256, seed=97, fp4x4=True)
    d, _ = oracle.fp4_fp4_gemm("dense", p.A, p.sfa, p.B, p.sfb)
    e, _ = oracle.fp4_fp4_gemm("dense", p.B, p.sfb, p.A, p.sfa)
    assert np.array_equal(d, e.T)
    pm = gen.make_masked(3, 64, 48, 256, seed=98, masked_m=[64, 0, 9], fp4x4=True)
    got, comp = oracle.fp4_fp4_gemm("masked", pm.A, pm.sfa, pm.B, pm.sfb, pm.masked_m)
    assert comp.reshape(3, 64).sum(1).tolist() == [64, 0, 9]
    for g in range(3):
        ref, _ = oracle.fp4_fp4_gemm("dense", pm.A[g], pm.sfa[g], pm.B[g], pm.sfb[g])
        valid = comp.reshape(3, 64)[g]
        assert np.array_equal(got.reshape(3, 64, 48)[g][valid], ref[valid])
    pc = gen.make_contiguous([128, 60], 48, 256, seed=99, fp4x4=True)
    got, comp = oracle.fp4_fp4_gemm("contiguous", pc.A, pc.sfa, pc.B, pc.sfb, pc.m_indices)
    for m in np.flatnonzero(comp):
        g = int(pc.m_indices[m])
        ref, _ = oracle.fp4_fp4_gemm("dense", pc.A[m:m + 1], pc.sfa[m:m + 1], pc.B[g], pc.sfb[g])
        assert np.array_equal(got[m], ref[0])
