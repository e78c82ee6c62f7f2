/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for block-scaled
 * FP8 GEMM  D = C + A . B^T  (NT layout) and its two M-grouped forms.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call this file.  The GPU
 * library never includes, links or calls it, and it shares no code, header,
 * table or constant with the GPU library.
 *
 * Sources (the pages this follows):
 *  - DeepGEMM README (pigsec.cn mirror), "Interfaces / Notes": kernels compute
 *    D = C + A @ B with the NT input layout, so fp8_gemm_nt is D = C + A @ B.T;
 *    on the SM90 path the scale factors are FP32 and the LHS scales are stored
 *    transposed (MN-major).
 *  - DeepGEMM launch article (2048ai.net), section 2 "FP8": the FP8 tensor-core
 *    partial products are accumulated a second time in higher precision
 *    ("promotion"), i.e. each 128-wide K block is reduced on its own and then
 *    scaled and added into an FP32 accumulator.
 *  - DeepGEMM README, "Grouped GEMM (contiguous layout)": only M is grouped,
 *    N and K are shared, each expert segment is aligned to the GEMM M block.
 *  - DeepGEMM README, "Grouped GEMM (masked layout)": a mask tensor tells the
 *    kernel which part of each group is valid; only that part is computed.
 *  - The FP8 format is E4M3.  The pages do not define the encoding; this file
 *    takes the OCP "E4M3FN" reading (max finite 448, no infinities, NaN only
 *    at S.1111.111), because the workloads scale blocks by amax/448.
 *  - Block sizes: A scales per 1x128 (one row, one K block), B scales per
 *    128x128 (128 rows of B, one K block).
 *  - DeepGEMM README, "Grouped GEMM (contiguous layout)": a K-axis grouped
 *    call (k_grouped_fp8_gemm_tn_contiguous) for the MoE weight backward,
 *    M and N fixed; see compute_row_kgrouped for its reading.
 *
 * What is computed, for every output row m that is computed and every n:
 *     S[m,n,kb] = sum_{k in block kb} e4m3(A[m,k]) * e4m3(B[n,k])      (FP64)
 *     D[m,n]    = C[m,n] + sum_kb (sfa[kb][m] * sfb[n/128][kb]) * S[m,n,kb]
 * in FP64, ascending kb, with no rounding to BF16 (D stays FP64).
 * Every finite E4M3 value is a multiple of 2^-9 and |S| <= 128*448^2 < 2^25,
 * so S needs at most 43 significant bits and FP64 sums it exactly in any order.
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_KBLOCK 128   /* K extent of one scale block (1x128 and 128x128) */
#define ORACLE_NBLOCK 128   /* N extent of one B scale block (128x128)        */

/* ------------------------------------------------------------------ */
/* E4M3 (OCP FN) decode, from the bit fields: sign s = bit 7,          */
/* exponent e = bits 6..3 (bias 7), mantissa m = bits 2..0.            */
/*   e == 0           : (-1)^s * (m/8) * 2^-6         (subnormal)      */
/*   e in 1..15       : (-1)^s * (1 + m/8) * 2^(e-7)  (normal)         */
/*   e == 15 && m == 7: NaN  (the only non-finite pattern; no Inf)     */
/* ------------------------------------------------------------------ */
double oracle_e4m3_value(uint8_t code)
{
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

void oracle_e4m3_table(double *out256)
{
    for (int c = 0; c < 256; ++c)
        out256[c] = oracle_e4m3_value((uint8_t)c);
}

/* ------------------------------------------------------------------ */
/* UE8M0 scale factors (DeepGEMM README, "Interfaces / Notes": on the  */
/* SM100 path the scale factors are UE8M0, four of them packed into    */
/* one 32-bit integer; the Ascend 950 article packs them along K).     */
/* The format is the OCP MX E8M0 one: an unsigned 8-bit exponent e     */
/* with bias 127, value 2^(e - 127); e = 255 is NaN.  Reading of the   */
/* packing: byte j (bits 8j..8j+7) of word w holds the scale of K      */
/* block 4w + j; bytes past the last K block are ignored.              */
/* Every value 2^-127 .. 2^127 is exact in FP32 (2^-127 as a           */
/* subnormal), so unpacking to FP32 scales loses nothing and the GEMM  */
/* is then the FP32-scale one.                                         */
/* ------------------------------------------------------------------ */
double oracle_ue8m0_value(uint8_t e)
{
    if (e == 255)
        return NAN;
    return ldexp(1.0, (int)e - 127);
}

static uint8_t ue8m0_byte(int32_t word, int j)
{
    return (uint8_t)(((uint32_t)word >> (8 * j)) & 0xFFu);
}

/*
 * LHS layout (MN-major, like the FP32 sfa): packed [n_mats][ceil(Kb/4)][M] ->
 * out [n_mats][Kb][M] FP32.
 */
void oracle_ue8m0_unpack_mn_major(const int32_t *packed, int64_t n_mats, int Kb, int64_t M, float *out)
{
    const int W = (Kb + 3) / 4;
    for (int64_t g = 0; g < n_mats; ++g)
        for (int kb = 0; kb < Kb; ++kb)
            for (int64_t m = 0; m < M; ++m) {
                int32_t w = packed[(g * W + kb / 4) * M + m];
                out[(g * Kb + kb) * M + m] = (float)oracle_ue8m0_value(ue8m0_byte(w, kb % 4));
            }
}

/*
 * RHS layout (K-contiguous, like the FP32 sfb): packed [n_rows][ceil(Kb/4)] ->
 * out [n_rows][Kb] FP32, where n_rows counts 128-row blocks of B (times groups).
 */
void oracle_ue8m0_unpack_k_major(const int32_t *packed, int64_t n_rows, int Kb, float *out)
{
    const int W = (Kb + 3) / 4;
    for (int64_t r = 0; r < n_rows; ++r)
        for (int kb = 0; kb < Kb; ++kb)
            out[r * Kb + kb] = (float)oracle_ue8m0_value(ue8m0_byte(packed[r * W + kb / 4], kb % 4));
}

/* ------------------------------------------------------------------ */
/* UE8M0 scale pairs in 16-bit words (DeepGEMM-Ascend news article,    */
/* "Cómo funciona": on Ascend every pair of UE8M0 scale factors along  */
/* K is packed into one int16, and the values are stored MN-major).    */
/* Readings: byte h (bits 8h..8h+7) of pair word p holds the scale of  */
/* K block 2p + h (the earlier K block in the low byte, as in the      */
/* four-to-a-word packing); a trailing high byte past the last K block */
/* is ignored; MN-major for both operands: the LHS words are           */
/* [ceil(Kb/2)][M] and the RHS words [ceil(Kb/2)][Nb], the index of    */
/* the row (LHS) or of the 128-row block of B (RHS) running fastest.   */
/* The block sizes stay 1x128 (LHS) and 128x128 (RHS).                 */
/* ------------------------------------------------------------------ */
static uint8_t ue8m0_pair_half(int16_t word, int h)
{
    return (uint8_t)(((uint16_t)word >> (h ? 8 : 0)) & 0xFFu);
}

/* LHS: pairs [n_mats][ceil(Kb/2)][M] -> out [n_mats][Kb][M] FP32 (the FP32 sfa layout). */
void oracle_ue8m0_pairs_unpack_lhs(const int16_t *pairs, int64_t n_mats, int Kb, int64_t M, float *out)
{
    const int P = (Kb + 1) / 2;
    for (int64_t g = 0; g < n_mats; ++g)
        for (int kb = 0; kb < Kb; ++kb)
            for (int64_t m = 0; m < M; ++m) {
                int16_t w = pairs[(g * P + kb / 2) * M + m];
                out[(g * Kb + kb) * M + m] = (float)oracle_ue8m0_value(ue8m0_pair_half(w, kb % 2));
            }
}

/* RHS: pairs [n_mats][ceil(Kb/2)][Nb] -> out [n_mats][Nb][Kb] FP32 (the FP32 sfb layout). */
void oracle_ue8m0_pairs_unpack_rhs(const int16_t *pairs, int64_t n_mats, int Kb, int64_t Nb, float *out)
{
    const int P = (Kb + 1) / 2;
    for (int64_t g = 0; g < n_mats; ++g)
        for (int64_t nb = 0; nb < Nb; ++nb)
            for (int kb = 0; Kb > kb; ++kb) {
                int16_t pw = pairs[(g * P + kb / 2) * Nb + nb];
                out[(g * Nb + nb) * Kb + kb] = (float)oracle_ue8m0_value(ue8m0_pair_half(pw, kb & 1));
            }
}

/* ------------------------------------------------------------------ */
/* FP4 E2M1 (OCP MX FP4; the pages' FP8 x FP4 GEMM takes FP4 weights:  */
/* DeepGEMM-Ascend hub page, precision table; README news 2026.04.16). */
/* Bits: sign = bit 3, exponent = bits 2..1 (bias 1), mantissa bit 0.  */
/*   e == 0   : (-1)^s * m * 0.5                (0 or 0.5)             */
/*   e in 1..3: (-1)^s * (1 + m/2) * 2^(e-1)    (1, 1.5, 2, 3, 4, 6)   */
/* No infinities or NaN.  Two per byte, element 2i in the low nibble   */
/* of byte i (reading: the OCP MX packing order).                      */
/* ------------------------------------------------------------------ */
double oracle_e2m1_value(uint8_t nibble)
{
    int s = (nibble >> 3) & 1;
    int e = (nibble >> 1) & 3;
    int m = nibble & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -1.0 * mag : mag;
}

/* ------------------------------------------------------------------ */
/* BF16 (1 sign, 8 exponent bits with bias 127, 7 mantissa bits),     */
/* round-to-nearest, ties-to-even, straight from a double.  The        */
/* outputs of all three operations are BF16.                           */
/* ------------------------------------------------------------------ */
static double round_half_even(double v) /* v >= 0, v < 2^52 */
{
    double fl = floor(v);
    double d = v - fl;
    if (d > 0.5)
        return fl + 1.0;
    if (d < 0.5)
        return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

uint16_t oracle_bf16_rne(double x)
{
    if (isnan(x))
        return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return sign | 0x7F80;
    int e;
    (void)frexp(a, &e);          /* a in [2^(e-1), 2^e) */
    int E = e - 1;               /* a = 1.f * 2^E */
    int qexp = (E < -126) ? -133 : E - 7;  /* value of one unit in the last place */
    double r = ldexp(round_half_even(ldexp(a, -qexp)), qexp);
    if (r >= 0x1p128)
        return sign | 0x7F80;    /* rounds past the largest finite BF16 */
    if (r < 0x1p-126)
        return sign | (uint16_t)ldexp(r, 133);        /* subnormal */
    int e2;
    (void)frexp(r, &e2);
    int E2 = e2 - 1;
    uint16_t mant = (uint16_t)(ldexp(r, 7 - E2) - 128.0);
    return sign | (uint16_t)((E2 + 127) << 7) | mant;
}

/* ------------------------------------------------------------------ */
/* One output row: D[n] = C[n] + sum_kb sa(kb) * sfb[n/128][kb] * S    */
/* ------------------------------------------------------------------ */
typedef struct {
    const double *dec;      /* 256-entry decode table */
    const uint8_t *a_row;   /* K codes of this row of A */
    const float *sa;        /* sfa for this row; the kb-th value is sa[kb * sa_stride] */
    int64_t sa_stride;
    const uint8_t *b;       /* B of the selected group, [N][K] codes */
    const float *sfb;       /* sfb of the selected group, [Nb][Kb] */
    const float *c_row;     /* NULL or N floats */
    int N, K;
    double *out;            /* N doubles */
} row_job;

static void compute_row(const row_job *j)
{
    const int Kb = j->K / ORACLE_KBLOCK;
    for (int n = 0; n < j->N; ++n) {
        const uint8_t *b_row = j->b + (int64_t)n * j->K;
        const float *sb = j->sfb + (int64_t)(n / ORACLE_NBLOCK) * Kb;
        double acc = 0.0;
        for (int kb = 0; kb < Kb; ++kb) {
            double s = 0.0;   /* exact block sum */
            const uint8_t *ap = j->a_row + kb * ORACLE_KBLOCK;
            const uint8_t *bp = b_row + kb * ORACLE_KBLOCK;
            for (int k = 0; k < ORACLE_KBLOCK; ++k)
                s += j->dec[ap[k]] * j->dec[bp[k]];
            double scale = (double)j->sa[kb * j->sa_stride] * (double)sb[kb];
            acc += scale * s;
        }
        j->out[n] = acc + (j->c_row ? (double)j->c_row[n] : 0.0);
    }
}

/* ------------------------------------------------------------------ */
/* FP8 x FP4 row: A in E4M3 with one UE8M0 scale per 1x128 block (the  */
/* packed LHS words above), B in E2M1 with one UE8M0 scale per 1x32    */
/* block of its row (reading: the OCP MX block of FP4, 32 elements),   */
/* four 32-blocks of one 128-wide K block packed into one word:        */
/*   D[n] = C[n] + sum_kb sum_j sa(kb) * sb(n, kb, j) * S[n, kb, j],   */
/*   S = sum over the 32 k of block j of e4m3(A[m,k]) * e2m1(B[n,k])   */
/* in FP64 (each S is exact: every term is a multiple of 2^-10 below   */
/* 448 * 6, so 32 of them need far fewer than 53 bits).                */
/* ------------------------------------------------------------------ */
typedef struct {
    const double *dec;      /* E4M3 table */
    double dec4[16];        /* E2M1 table */
    const uint8_t *a_row;   /* K codes */
    const int32_t *sa;      /* packed LHS words of this row; word w at sa[w * sa_stride] */
    int64_t sa_stride;
    const uint8_t *b;       /* B of the group, [N][K/2] bytes */
    const int32_t *sfb;     /* [N][Kb] words of the group */
    const float *c_row;
    int N, K;
    double *out;
} row_job4;

static void compute_row_fp4(const row_job4 *j)
{
    const int Kb = j->K / ORACLE_KBLOCK;
    for (int n = 0; n < j->N; ++n) {
        const uint8_t *b_row = j->b + (int64_t)n * (j->K / 2);
        double acc = 0.0;
        for (int kb = 0; kb != Kb; ++kb) {
            double sa = oracle_ue8m0_value(ue8m0_byte(j->sa[(kb / 4) * j->sa_stride], kb % 4));
            int32_t wb = j->sfb[(int64_t)n * Kb + kb];
            for (int blk = 0; blk < 4; ++blk) {
                double s = 0.0;
                for (int t = 0; t < 32; ++t) {
                    int k = kb * ORACLE_KBLOCK + blk * 32 + t;
                    uint8_t byte = b_row[k / 2];
                    uint8_t nib = (k & 1) ? (byte >> 4) : (byte & 0xF);
                    s += j->dec[j->a_row[k]] * j->dec4[nib];
                }
                acc += sa * oracle_ue8m0_value(ue8m0_byte(wb, blk)) * s;
            }
        }
        j->out[n] = (j->c_row ? (double)j->c_row[n] : 0.0) + acc;
    }
}

/* ------------------------------------------------------------------ */
/* FP4 x FP4 row (DeepGEMM-Ascend hub page, precision table: FP4 x FP4 */
/* for ultra-low-bit inference): A and B both E2M1, two codes a byte,  */
/* each row with one UE8M0 scale per 1x32 block (the four of a K block */
/* in one word, sfa [rows][K/128] like sfb [N][K/128]):                */
/*   D[n] = C[n] + sum_kb sum_j 2^(ea-127) 2^(eb-127) S[n, kb, j],     */
/*   S = sum over the 32 k of block j of e2m1(A[m,k]) * e2m1(B[n,k]).  */
/* ------------------------------------------------------------------ */
static double e2m1_nibble(const uint8_t *row, int k, const double *dec4)
{
    const uint8_t byte = row[k >> 1];
    return dec4[(k % 2 == 0) ? (byte & 0x0F) : (byte >> 4)];
}

static void compute_row_fp4x4(const uint8_t *a_row, const int32_t *sa_row, const uint8_t *b, const int32_t *sfb,
                              const float *c_row, int N, int K, double *out)
{
    double dec4[16];
    for (int c = 0; c < 16; ++c) dec4[c] = oracle_e2m1_value((uint8_t)c);
    const int Kb = K / ORACLE_KBLOCK;
    for (int n = 0; n < N; ++n) {
        const uint8_t *b_row = b + (int64_t)n * (K / 2);
        double total = 0.0;
        for (int kb = 0; Kb > kb; ++kb) {
            for (int j = 0; j < 4; ++j) {
                double blk = 0.0;
                for (int t = 0; t < 32; ++t) {
                    const int k = kb * ORACLE_KBLOCK + 32 * j + t;
                    blk += e2m1_nibble(a_row, k, dec4) * e2m1_nibble(b_row, k, dec4);
                }
                const double sa = oracle_ue8m0_value(ue8m0_byte(sa_row[kb], j));
                const double sb = oracle_ue8m0_value(ue8m0_byte(sfb[(int64_t)n * Kb + kb], j));
                total += sa * sb * blk;
            }
        }
        out[n] = total + (c_row ? (double)c_row[n] : 0.0);
    }
}

/* ------------------------------------------------------------------ */
/* Row scheduling over threads.                                        */
/* ------------------------------------------------------------------ */
enum { KIND_DENSE = 0, KIND_CONTIG = 1, KIND_MASKED = 2, KIND_KGROUP = 3 };

typedef struct {
    int kind;
    const uint8_t *A; const float *sfa; const uint8_t *B; const float *sfb;
    const int32_t *group_info;   /* m_indices (contig) or masked_m (masked) */
    const float *C;
    int64_t M;                   /* rows of A (dense/contig) or M_max (masked) */
    int N, K, G;
    const int64_t *rows; int64_t n_rows;
    double *out; uint8_t *computed;
    double dec[256];
    int fp4;                     /* FP8 x FP4: sfa/sfb are packed UE8M0 words, B is E2M1 */
    const int64_t *k_off;        /* K-grouped: first K row of each group's segment ([G + 1]) */
} problem;

/* ------------------------------------------------------------------ */
/* K-grouped TN (DeepGEMM README, "Grouped GEMM (contiguous layout)":  */
/* a K-axis grouped call for the weight backward of MoE, M and N       */
/* fixed).  Both operands are stored K-outermost ("TN": A [K][M],       */
/* B [K][N]) and group g owns the K rows [k_off[g], k_off[g + 1]):      */
/*   D[g][m][n] = C[g][m][n]                                           */
/*              + sum_{kb in g} sfa[kb][m] * sfb[kb][n] * S[kb][m][n], */
/*   S = sum over the 128 k of block kb of e4m3(A[k][m]) e4m3(B[k][n]) */
/* (reading: both operands carry one FP32 scale per 128 K rows of each */
/* column, 1x128 along K, the granularity of the A scales of the other */
/* forms).  S is exact in FP64 as for the other forms; the outer sum   */
/* runs in ascending kb.  The block sums of all n are formed together  */
/* (k outer, n inner), which changes nothing: each is exact.           */
/* ------------------------------------------------------------------ */
static void compute_row_kgrouped(const problem *p, int64_t g, int64_t m, double *out)
{
    const int N = p->N;
    const int64_t M = p->M;
    const int64_t kb_first = p->k_off[g] / ORACLE_KBLOCK, kb_end = p->k_off[g + 1] / ORACLE_KBLOCK;
    double *s = (double *)malloc(sizeof(double) * (size_t)N);
    for (int n = 0; n < N; ++n)
        out[n] = 0.0;
    for (int64_t kb = kb_first; kb < kb_end; ++kb) {
        for (int n = 0; n < N; ++n)
            s[n] = 0.0;
        for (int64_t k = kb * ORACLE_KBLOCK; k < (kb + 1) * ORACLE_KBLOCK; ++k) {
            const double a = p->dec[p->A[k * M + m]];
            const uint8_t *b_row = p->B + k * (int64_t)N;
            for (int n = 0; n < N; ++n)
                s[n] += a * p->dec[b_row[n]];
        }
        const double sa = (double)p->sfa[kb * M + m];
        const float *sb = p->sfb + kb * (int64_t)N;
        for (int n = 0; n < N; ++n)
            out[n] += sa * (double)sb[n] * s[n];
    }
    free(s);
    if (p->C) {
        const float *c_row = p->C + (g * M + m) * (int64_t)N;
        for (int n = 0; n < N; ++n)
            out[n] += (double)c_row[n];
    }
}

typedef struct { const problem *p; int64_t r0, r1; } slice;

static void do_row(const problem *p, int64_t i)
{
    const int Kb = p->K / ORACLE_KBLOCK;
    const int Nb = (p->N + ORACLE_NBLOCK - 1) / ORACLE_NBLOCK;
    int64_t r = p->rows ? p->rows[i] : i;
    double *out = p->out + i * (int64_t)p->N;
    row_job j;
    j.dec = p->dec; j.N = p->N; j.K = p->K; j.out = out;

    if (p->kind == KIND_KGROUP) {            /* flat row r = g * M + m */
        compute_row_kgrouped(p, r / p->M, r % p->M, out);
        if (p->computed) p->computed[i] = 1;
        return;
    }
    if (p->kind == KIND_DENSE) {
        j.a_row = p->A + r * p->K;
        j.sa = p->sfa + r; j.sa_stride = p->M;
        j.b = p->B; j.sfb = p->sfb;
        j.c_row = p->C ? p->C + r * p->N : NULL;
    } else if (p->kind == KIND_CONTIG) {
        int32_t g = p->group_info[r];
        if (g < 0 || g >= p->G) {            /* padding row: not computed */
            for (int n = 0; n < p->N; ++n) out[n] = NAN;
            if (p->computed) p->computed[i] = 0;
            return;
        }
        j.a_row = p->A + r * p->K;
        j.sa = p->sfa + r; j.sa_stride = p->M;
        j.b = p->B + (int64_t)g * p->N * p->K;
        j.sfb = p->sfb + (int64_t)g * Nb * Kb;
        j.c_row = p->C ? p->C + r * p->N : NULL;
    } else {
        int64_t g = r / p->M, m = r % p->M;
        int64_t valid = p->group_info[g];
        if (valid < 0) valid = 0;
        if (valid > p->M) valid = p->M;
        if (m >= valid) {                    /* masked row: not computed */
            for (int n = 0; n < p->N; ++n) out[n] = NAN;
            if (p->computed) p->computed[i] = 0;
            return;
        }
        j.a_row = p->A + r * p->K;
        j.sa = p->sfa + g * Kb * p->M + m; j.sa_stride = p->M;
        j.b = p->B + g * p->N * (int64_t)p->K;
        j.sfb = p->sfb + g * Nb * (int64_t)Kb;
        j.c_row = p->C ? p->C + r * p->N : NULL;
    }
    if (p->fp4 == 2) {
        /* FP4 x FP4: A rows are K/2 bytes with a word of scales per K block */
        const int32_t *sfa44 = (const int32_t *)p->sfa;
        const int32_t *sfb44 = (const int32_t *)p->sfb;
        int64_t g44 = 0;
        if (p->kind == KIND_CONTIG) g44 = p->group_info[r];
        if (p->kind == KIND_MASKED) g44 = r / p->M;
        compute_row_fp4x4(p->A + r * (int64_t)(p->K / 2), sfa44 + r * (int64_t)Kb,
                          p->B + g44 * (int64_t)p->N * (p->K / 2), sfb44 + g44 * (int64_t)p->N * Kb, j.c_row,
                          p->N, p->K, out);
    } else if (p->fp4) {
        /* same row selection; scales and B reinterpreted for FP8 x FP4 */
        const int W = (Kb + 3) / 4;
        row_job4 j4;
        j4.dec = p->dec; j4.N = p->N; j4.K = p->K; j4.out = out; j4.a_row = j.a_row; j4.c_row = j.c_row;
        for (int c = 0; c < 16; ++c) j4.dec4[c] = oracle_e2m1_value((uint8_t)c);
        const int32_t *sfa4 = (const int32_t *)p->sfa;
        const int32_t *sfb4 = (const int32_t *)p->sfb;
        const uint8_t *B4 = p->B;
        int64_t g = 0, m = r;
        if (p->kind == KIND_CONTIG) g = p->group_info[r];
        if (p->kind == KIND_MASKED) { g = r / p->M; m = r % p->M; }
        j4.sa = sfa4 + (p->kind == KIND_MASKED ? g * W * p->M : 0) + m;
        j4.sa_stride = p->M;
        j4.b = B4 + g * (int64_t)p->N * (p->K / 2);
        j4.sfb = sfb4 + g * (int64_t)p->N * Kb;
        compute_row_fp4(&j4);
    } else {
        compute_row(&j);
    }
    if (p->computed) p->computed[i] = 1;
}

static void *worker(void *arg)
{
    const slice *s = (const slice *)arg;
    for (int64_t i = s->r0; i < s->r1; ++i)
        do_row(s->p, i);
    return NULL;
}

int oracle_default_threads(void)
{
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof(set), &set) == 0) {
        int c = CPU_COUNT(&set);
        if (c > 0) return c;
    }
    return 1;
}

static int run(problem *p, int n_threads)
{
    if (p->K <= 0 || p->K % ORACLE_KBLOCK != 0 || p->N <= 0 || p->M <= 0 || p->n_rows < 0)
        return -1;
    oracle_e4m3_table(p->dec);
    if (n_threads <= 0) n_threads = oracle_default_threads();
    if (n_threads > p->n_rows) n_threads = (int)(p->n_rows > 0 ? p->n_rows : 1);
    if (n_threads > 256) n_threads = 256;
    pthread_t tid[256];
    int joined[256];
    slice sl[256];
    int64_t per = (p->n_rows + n_threads - 1) / n_threads;
    for (int t = 0; t < n_threads; ++t) {
        sl[t].p = p;
        sl[t].r0 = t * per < p->n_rows ? t * per : p->n_rows;
        sl[t].r1 = (t + 1) * per < p->n_rows ? (t + 1) * per : p->n_rows;
        joined[t] = 0;
        if (sl[t].r0 >= sl[t].r1)
            continue;
        if (pthread_create(&tid[t], NULL, worker, &sl[t]) == 0)
            joined[t] = 1;
        else
            worker(&sl[t]);          /* could not start a thread: do it here */
    }
    for (int t = 0; t < n_threads; ++t)
        if (joined[t])
            pthread_join(tid[t], NULL);
    return 0;
}

/*
 * Dense:  D = C + A . B^T.
 *   A [M][K] e4m3 codes, sfa [K/128][M], B [N][K] codes, sfb [ceil(N/128)][K/128],
 *   C NULL or [M][N] fp32.  rows: NULL (all M rows, out is [M][N]) or n_rows row
 *   indices (out is [n_rows][N]).  Returns 0, or -1 on bad sizes.
 */
int oracle_fp8_gemm_nt(const uint8_t *A, const float *sfa, const uint8_t *B, const float *sfb,
                       const float *C, int64_t M, int N, int K,
                       const int64_t *rows, int64_t n_rows, double *out, int n_threads)
{
    problem p;
    memset(&p, 0, sizeof(p));
    p.kind = KIND_DENSE; p.A = A; p.sfa = sfa; p.B = B; p.sfb = sfb; p.C = C;
    p.M = M; p.N = N; p.K = K; p.G = 1;
    p.rows = rows; p.n_rows = rows ? n_rows : M; p.out = out;
    return run(&p, n_threads);
}

/*
 * M-grouped contiguous: row m uses expert g = m_indices[m] (B[g], sfb[g]);
 * rows whose index lies outside [0, G) are padding and are not computed
 * (out row = NaN, computed[i] = 0).
 *   A [M][K], sfa [K/128][M], B [G][N][K], sfb [G][ceil(N/128)][K/128],
 *   m_indices [M] int32, C NULL or [M][N].
 */
int oracle_m_grouped_contiguous(const uint8_t *A, const float *sfa, const uint8_t *B,
                                const float *sfb, const int32_t *m_indices, const float *C,
                                int64_t M, int N, int K, int G,
                                const int64_t *rows, int64_t n_rows, double *out,
                                uint8_t *computed, int n_threads)
{
    problem p;
    memset(&p, 0, sizeof(p));
    p.kind = KIND_CONTIG; p.A = A; p.sfa = sfa; p.B = B; p.sfb = sfb; p.C = C;
    p.group_info = m_indices; p.M = M; p.N = N; p.K = K; p.G = G;
    p.rows = rows; p.n_rows = rows ? n_rows : M; p.out = out; p.computed = computed;
    if (G <= 0) return -1;
    return run(&p, n_threads);
}

/*
 * M-grouped masked: group g computes rows m < clamp(masked_m[g], 0, M_max);
 * the other rows are not computed (out row = NaN, computed[i] = 0).
 *   A [G][M_max][K], sfa [G][K/128][M_max], B [G][N][K], sfb [G][ceil(N/128)][K/128],
 *   masked_m [G] int32, C NULL or [G][M_max][N].
 *   rows are flat indices g*M_max + m (NULL: all G*M_max rows).
 */
int oracle_m_grouped_masked(const uint8_t *A, const float *sfa, const uint8_t *B,
                            const float *sfb, const int32_t *masked_m, const float *C,
                            int64_t M_max, int N, int K, int G,
                            const int64_t *rows, int64_t n_rows, double *out,
                            uint8_t *computed, int n_threads)
{
    problem p;
    memset(&p, 0, sizeof(p));
    p.kind = KIND_MASKED; p.A = A; p.sfa = sfa; p.B = B; p.sfb = sfb; p.C = C;
    p.group_info = masked_m; p.M = M_max; p.N = N; p.K = K; p.G = G;
    p.rows = rows; p.n_rows = rows ? n_rows : (int64_t)G * M_max; p.out = out; p.computed = computed;
    if (G <= 0) return -1;
    return run(&p, n_threads);
}

/*
 * FP8 x FP4 (all three forms; kind 0 dense, 1 contiguous, 2 masked):
 *   A as in the FP32-scale forms; sfa packed UE8M0 words [ceil(Kb/4)][M]
 *   (masked: [G][ceil(Kb/4)][M_max]); B [G][N][K/2] E2M1 pairs (dense: G = 1);
 *   sfb [G][N][Kb] words, byte j = scale of K elements [128 kb + 32 j, +32);
 *   group_info: m_indices (contiguous) or masked_m (masked), NULL for dense.
 */
int oracle_fp8_fp4_gemm(int kind, const uint8_t *A, const int32_t *sfa, const uint8_t *B, const int32_t *sfb,
                        const int32_t *group_info, const float *C, int64_t M, int N, int K, int G,
                        const int64_t *rows, int64_t n_rows, double *out, uint8_t *computed, int n_threads)
{
    problem p;
    memset(&p, 0, sizeof(p));
    if (kind < 0 || kind > 2 || G <= 0) return -1;
    p.kind = kind; p.A = A; p.sfa = (const float *)sfa; p.B = B; p.sfb = (const float *)sfb; p.C = C;
    p.group_info = group_info; p.M = M; p.N = N; p.K = K; p.G = G; p.fp4 = 1;
    p.rows = rows;
    p.n_rows = rows ? n_rows : (kind == KIND_MASKED ? (int64_t)G * M : M);
    p.out = out; p.computed = computed;
    return run(&p, n_threads);
}

/*
 * K-grouped TN contiguous (see compute_row_kgrouped):
 *   A [K][M] e4m3 codes, sfa [K/128][M], B [K][N] codes, sfb [K/128][N] fp32,
 *   ks [G] int32: K rows of each group, in order (reading: each a multiple of
 *   128; a negative count is 0; segments are cut at K), C NULL or [G][M][N].
 *   rows: flat indices g*M + m (NULL: all G*M rows); out [rows][N] FP64.
 *   Returns 0, or -1 on bad sizes (K not a multiple of 128, a segment not
 *   starting on a multiple of 128).
 */
int oracle_k_grouped_tn(const uint8_t *A, const float *sfa, const uint8_t *B, const float *sfb,
                        const int32_t *ks, const float *C, int64_t M, int N, int K, int G,
                        const int64_t *rows, int64_t n_rows, double *out, uint8_t *computed, int n_threads)
{
    problem p;
    memset(&p, 0, sizeof(p));
    if (G <= 0 || K <= 0 || K % ORACLE_KBLOCK != 0) return -1;
    int64_t *off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(G + 1));
    off[0] = 0;
    for (int g = 0; g < G; ++g) {
        int64_t k = ks[g] < 0 ? 0 : ks[g];
        int64_t end = off[g] + k;
        off[g + 1] = end > K ? K : end;
        if (off[g + 1] % ORACLE_KBLOCK != 0) { free(off); return -1; }
    }
    p.kind = KIND_KGROUP; p.A = A; p.sfa = sfa; p.B = B; p.sfb = sfb; p.C = C;
    p.M = M; p.N = N; p.K = K; p.G = G; p.k_off = off;
    p.rows = rows; p.n_rows = rows ? n_rows : (int64_t)G * M; p.out = out; p.computed = computed;
    int rc = run(&p, n_threads);
    free(off);
    return rc;
}

/* ------------------------------------------------------------------ */
/* BF16 x BF16 (DeepGEMM-Ascend hub page, precision table: BF16 x BF16 */
/* for ordinary-precision training; DeepGEMM README intro: GEMM in     */
/* FP8, FP4 and BF16): D = C + A . B^T with no scale factors.          */
/* BF16 decoded from its bit fields: sign bit 15, exponent bits 14..7  */
/* (bias 127), mantissa bits 6..0; exponent 0: subnormal m * 2^-133;   */
/* exponent 255: Inf (m = 0) or NaN.                                   */
/* ------------------------------------------------------------------ */
double oracle_bf16_value(uint16_t bits)
{
    int s = (bits >> 15) & 1;
    int e = (bits >> 7) & 0xFF;
    int m = bits & 0x7F;
    double mag;
    if (e == 0xFF)
        mag = m ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)m, -133);
    else
        mag = ldexp(1.0 + (double)m / 128.0, e - 127);
    /* the sign bit applies to zero as well: 0x8000 is -0 */
    return copysign(mag, s ? -1.0 : 1.0);
}

typedef struct {
    const uint16_t *A, *B;       /* [rows][K], [G][N][K] */
    const float *C;
    const int32_t *group_info;   /* m_indices (kind 1) or masked_m (kind 2) */
    int kind;
    int64_t M;                   /* rows of A (dense, contiguous) or M_max (masked) */
    int N, K, G;
    const int64_t *rows;
    int64_t n_rows;
    double *out;
    uint8_t *computed;
} bf16_problem;

typedef struct { const bf16_problem *p; int64_t r0, r1; } bf16_slice;

/* All 65536 codes decoded once by oracle_bf16_value (a lookup instead of a
 * decode per multiply; the values are the same). */
static double bf16_table[65536];
static pthread_once_t bf16_table_once = PTHREAD_ONCE_INIT;
static void bf16_table_fill(void)
{
    for (int c = 0; c < 65536; ++c) bf16_table[c] = oracle_bf16_value((uint16_t)c);
}

/* One output row: D[n] = C[n] + sum_k bf16(A[m][k]) * bf16(B[n][k]) in FP64,
 * ascending k (every product is exact in FP64; the sum rounds far below the
 * BF16 output's resolution). */
static void *bf16_worker(void *arg)
{
    const bf16_slice *sl = (const bf16_slice *)arg;
    const bf16_problem *p = sl->p;
    double *a = (double *)malloc(sizeof(double) * (size_t)p->K);
    for (int64_t i = sl->r0; i < sl->r1; ++i) {
        int64_t r = p->rows ? p->rows[i] : i;
        double *out = p->out + i * (int64_t)p->N;
        int64_t g = 0;
        if (p->kind == KIND_CONTIG) {
            g = p->group_info[r];
            if (g < 0 || g >= p->G) {
                for (int n = 0; n < p->N; ++n) out[n] = NAN;
                if (p->computed) p->computed[i] = 0;
                continue;
            }
        } else if (p->kind == KIND_MASKED) {
            int64_t valid = p->group_info[r / p->M];
            valid = valid < 0 ? 0 : (valid > p->M ? p->M : valid);
            g = r / p->M;
            if (r % p->M >= valid) {
                for (int n = 0; n < p->N; ++n) out[n] = NAN;
                if (p->computed) p->computed[i] = 0;
                continue;
            }
        }
        for (int k = 0; k < p->K; ++k)
            a[k] = bf16_table[p->A[r * p->K + k]];
        const uint16_t *b = p->B + g * (int64_t)p->N * p->K;
        for (int n = 0; n < p->N; ++n) {
            double acc = 0.0;
            for (int k = 0; k < p->K; ++k)
                acc += a[k] * bf16_table[b[(int64_t)n * p->K + k]];
            out[n] = acc + (p->C ? (double)p->C[r * (int64_t)p->N + n] : 0.0);
        }
        if (p->computed) p->computed[i] = 1;
    }
    free(a);
    return NULL;
}

/*
 * BF16 GEMM, kind 0 dense / 1 contiguous / 2 masked, layouts as the FP8 forms
 * with 2-byte elements and no scales: A [rows][K] (masked [G][M_max][K]),
 * B [G][N][K] (dense: G = 1), C NULL or like D.  rows: flat row indices
 * (NULL: all).  Returns 0, or -1 on bad sizes.
 */
int oracle_bf16_gemm(int kind, const uint16_t *A, const uint16_t *B, const int32_t *group_info, const float *C,
                     int64_t M, int N, int K, int G, const int64_t *rows, int64_t n_rows, double *out,
                     uint8_t *computed, int n_threads)
{
    if (kind < 0 || kind > 2 || M <= 0 || N <= 0 || K <= 0 || G <= 0) return -1;
    pthread_once(&bf16_table_once, bf16_table_fill);
    bf16_problem p = {A, B, C, group_info, kind, M, N, K, G, rows, 0, out, computed};
    p.n_rows = rows ? n_rows : (kind == KIND_MASKED ? (int64_t)G * M : M);
    if (n_threads <= 0) n_threads = oracle_default_threads();
    if (n_threads > 256) n_threads = 256;
    if (n_threads > p.n_rows) n_threads = (int)(p.n_rows > 0 ? p.n_rows : 1);
    pthread_t tid[256];
    bf16_slice sl[256];
    int started[256];
    int64_t per = (p.n_rows + n_threads - 1) / n_threads;
    for (int t = 0; t < n_threads; ++t) {
        sl[t].p = &p;
        sl[t].r0 = t * per < p.n_rows ? t * per : p.n_rows;
        sl[t].r1 = (t + 1) * per < p.n_rows ? (t + 1) * per : p.n_rows;
        started[t] = sl[t].r0 < sl[t].r1 && pthread_create(&tid[t], NULL, bf16_worker, &sl[t]) == 0;
        if (!started[t] && sl[t].r0 < sl[t].r1) bf16_worker(&sl[t]);
    }
    for (int t = 0; t < n_threads; ++t)
        if (started[t]) pthread_join(tid[t], NULL);
    return 0;
}

/*
 * FP4 x FP4 (all three forms; kind 0 dense, 1 contiguous, 2 masked):
 *   A [rows][K/2] E2M1 pairs (masked [G][M_max][K/2]), sfa [rows][K/128] words
 *   (masked [G][M_max][K/128]); B and sfb as for FP8 x FP4; C, group_info and
 *   rows as for the other forms.
 */
int oracle_fp4_fp4_gemm(int kind, const uint8_t *A, const int32_t *sfa, const uint8_t *B, const int32_t *sfb,
                        const int32_t *group_info, const float *C, int64_t M, int N, int K, int G,
                        const int64_t *rows, int64_t n_rows, double *out, uint8_t *computed, int n_threads)
{
    problem p;
    memset(&p, 0, sizeof(p));
    if (kind < 0 || kind > 2 || G <= 0) return -1;
    p.kind = kind; p.A = A; p.sfa = (const float *)sfa; p.B = B; p.sfb = (const float *)sfb; p.C = C;
    p.group_info = group_info; p.M = M; p.N = N; p.K = K; p.G = G; p.fp4 = 2;
    p.rows = rows;
    p.n_rows = rows ? n_rows : (kind == KIND_MASKED ? (int64_t)G * M : M);
    p.out = out; p.computed = computed;
    return run(&p, n_threads);
}
