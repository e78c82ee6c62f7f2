/*
 * dg.h -- C ABI of the MI355X (gfx950) block-scaled FP8 GEMM library (libdg.so).
 *
 * Operation (DeepGEMM README, "Interfaces / Notes"): the kernels follow the
 * naming D = C + A @ B with the NT input layout, so the `_nt` calls compute
 *
 *     D = C + A . B^T
 *
 * with A and B in FP8 E4M3 (OCP "FN" encoding: max 448, no infinities),
 * FP32 accumulation, and BF16 D.  Fine-grained scaling (same section, and
 * the DeepGEMM launch article, section 2 "FP8"): one FP32 scale per 1x128
 * block of A (one row, 128 consecutive K) and one per 128x128 block of B.
 * Every 128-wide K block is reduced on the matrix cores, then multiplied by
 * its two scales and added into an FP32 accumulator ("promotion").
 * Quantisation and any transposition are the caller's job (same section).
 *
 * Notation: Kb = K/128, Nb = ceil(N/128).  All tensors are row-major and
 * densely packed.
 *
 *   A    uint8 (E4M3 codes) [rows][K]
 *   sfa  float [Kb][rows]             MN-major ("transposed") LHS scales, as the
 *                                     README's notes require for the LHS
 *   B    uint8 (E4M3 codes) [N][K]    (the "T" of NT: row n of B is column n of B^T)
 *   sfb  float [Nb][Kb]               rows n in [128 i, 128 i + 128) use sfb[i][kb]
 *   C    float [rows][N] or NULL      added before the single BF16 rounding
 *   D    bf16  [rows][N]              written with round-to-nearest-even
 *
 * Ownership and execution:
 *   - Every tensor pointer is DEVICE memory owned by the caller; the library
 *     never frees or keeps it.  A, B, C and D must be 16-byte aligned; the
 *     scale and index arrays 4-byte aligned.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = default
 *     stream).  They never synchronise the host and never read device data
 *     (group indices, masks) on the host.
 *   - The library owns its compiled-kernel cache and a per-stream device
 *     workspace (split-K partials and arrival counters; the K-contiguous copies
 *     of K-outermost operands), created on first use (or by dg_init) and kept
 *     until process exit.  The first call for a new shape compiles a kernel
 *     (hipRTC) and may allocate; later calls with the same shape neither
 *     compile nor allocate.  A workspace a larger call outgrows is replaced by
 *     one at least twice its size and is never freed, so a HIP graph that
 *     captured calls keeps valid addresses; replay such a graph on the stream
 *     it was captured on (calls on one stream share that stream's workspace).
 *     Two graphs that captured calls on the same stream share its workspace
 *     too, so they must not be replayed concurrently (on other streams) when
 *     their shapes use split-K (few rows, long K) or a K-contiguous rewrite:
 *     that races on the partial sums and arrival counters and is unsupported.
 *     A call that compiles or allocates cannot run under stream capture: make
 *     the first call of each shape on each stream eagerly, then capture.
 *   - Work queued on different streams must not share output buffers.
 *
 * Errors: every call validates its arguments on the host before touching the
 * GPU and returns a dg_status; dg_last_error() gives a message for the last
 * non-OK status of the calling thread.  No exception crosses the ABI.
 * Data-dependent cases are defined behaviour, not errors: masked_m values are
 * clamped to [0, M_max]; m_indices values outside [0, num_groups) mark rows
 * that are not computed (their D rows are left as they were).
 */
#ifndef DG_H_
#define DG_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DG_OK = 0,
    DG_ERR_INVALID_ARG = -1,   /* NULL pointer, non-positive size, bad group count */
    DG_ERR_UNSUPPORTED = -2,   /* K not a multiple of 128, sizes beyond 32-bit offsets */
    DG_ERR_ALIGNMENT = -3,     /* pointer not 16-byte aligned, contiguous M not aligned */
    DG_ERR_JIT = -4,           /* hipRTC compile or code-object load failed, or a forced tile of a
                                  variant that loads B into registers spilled registers */
    DG_ERR_HIP = -5            /* a HIP runtime call failed (no device, launch error) */
} dg_status;

/*
 * Dense:  D[M][N] = C + A[M][K] . B[N][K]^T.
 * DeepGEMM README, "Normal dense GEMM (non-grouped)" (fp8_gemm_nt), and
 * "Interfaces / Notes" for the layouts above.  C may be NULL.
 */
dg_status dg_fp8_gemm_nt(const void *A, const float *sfa, const void *B, const float *sfb,
                         const float *C, void *D, int M, int N, int K, void *stream);

/*
 * The dense call for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same operation, arguments, layouts and errors as dg_fp8_gemm_nt, except:
 *   - It allocates nothing: no hipMalloc or hipFree, no compile, no module
 *     load.  The kernels for the sizes must already be loaded on the device:
 *     call dg_fp8_gemm_nt once with the same M, N, K and C presence first
 *     (otherwise DG_ERR_UNSUPPORTED).
 *   - Split-K partial sums and arrival counters (shapes with few rows and a
 *     long K) live in a static device array of the library, 32 MiB of partial
 *     sums plus 256 KiB of counters per device, held until the process ends,
 *     instead of a per-stream workspace.  A shape whose split-K needs more is
 *     rejected with DG_ERR_UNSUPPORTED.  Each call first zeroes the counters
 *     it uses (a small kernel on `stream`).
 *   - Every call on a device shares that array, which keeps the last call's
 *     contents: calls that overlap in time on one GPU (on other streams, or
 *     graph replays running concurrently) race and give wrong results.
 */
dg_status dg_fp8_gemm_nt_noalloc(const void *A, const float *sfa, const void *B, const float *sfb,
                                 const float *C, void *D, int M, int N, int K, void *stream);

/*
 * M-grouped, contiguous layout (MoE prefill / training forward).
 * DeepGEMM README, "Grouped GEMM (contiguous layout)": only M is grouped, N
 * and K are shared; the experts' tokens are concatenated along M and every
 * expert's segment starts on a multiple of
 * dg_get_mk_alignment_for_contiguous_layout() rows.
 *   A [M][K], sfa [Kb][M], B [G][N][K], sfb [G][Nb][Kb], C NULL or [M][N], D [M][N],
 *   m_indices int32 [M] (device): expert of each row; a value outside [0, G)
 *   marks a padding row, which is not computed and whose D row is untouched.
 * M must be a multiple of the alignment.  Every valid row of an aligned block
 * must name the block's expert, and padding rows come after them.  Outside
 * that layout each row is either computed for its own expert or left
 * untouched (which one depends on the tile size); no row is ever computed
 * with another expert's weights.
 */
dg_status dg_m_grouped_fp8_gemm_nt_contiguous(const void *A, const float *sfa, const void *B,
                                              const float *sfb, const int32_t *m_indices,
                                              const float *C, void *D, int M, int N, int K,
                                              int num_groups, void *stream);

/*
 * M-grouped, masked layout (MoE decode, graph-friendly).
 * DeepGEMM README, "Grouped GEMM (masked layout)": the host does not know how
 * many rows each expert received; a device mask tells the kernel which part
 * to compute.
 *   A [G][M_max][K], sfa [G][Kb][M_max], B [G][N][K], sfb [G][Nb][Kb],
 *   C NULL or [G][M_max][N], D [G][M_max][N],
 *   masked_m int32 [G] (device): group g computes rows m < clamp(masked_m[g], 0, M_max);
 *   D rows at or beyond that are never written.
 */
dg_status dg_m_grouped_fp8_gemm_nt_masked(const void *A, const float *sfa, const void *B,
                                          const float *sfb, const int32_t *masked_m,
                                          const float *C, void *D, int M_max, int N, int K,
                                          int num_groups, void *stream);

/*
 * Storage layouts other than NT (DeepGEMM README, "Normal dense GEMM":
 * fp8_gemm_{nt, nn, tn, tt}; "Grouped GEMM (contiguous layout)":
 * m_grouped_fp8_gemm_{nt, nn}_contiguous).  The operation is the same
 * D = C + A . B^T over the logical A [M][K] and B [N][K]; the letters say how
 * the operands are stored (reading, the pages name the calls only): the first
 * is A, N = [M][K] (K-contiguous), T = [K][M]; the second is B, T = [N][K],
 * N = [K][N] (grouped: [G][K][N]).  The scales keep their logical layouts and
 * block shapes (sfa [Kb][M], sfb [(G)][Nb][Kb]).  An operand stored K-outermost
 * is rewritten K-contiguous into a per-stream device buffer (rows x K bytes,
 * allocated on the first call of a size, kept until exit), then the NT kernels
 * run on it.  Everything else as for the NT calls.
 */
dg_status dg_fp8_gemm_nn(const void *A, const float *sfa, const void *B, const float *sfb,
                         const float *C, void *D, int M, int N, int K, void *stream);
dg_status dg_fp8_gemm_tn(const void *A, const float *sfa, const void *B, const float *sfb,
                         const float *C, void *D, int M, int N, int K, void *stream);
dg_status dg_fp8_gemm_tt(const void *A, const float *sfa, const void *B, const float *sfb,
                         const float *C, void *D, int M, int N, int K, void *stream);
dg_status dg_m_grouped_fp8_gemm_nn_contiguous(const void *A, const float *sfa, const void *B,
                                              const float *sfb, const int32_t *m_indices,
                                              const float *C, void *D, int M, int N, int K,
                                              int num_groups, void *stream);

/*
 * The same three forms with packed UE8M0 scale factors (DeepGEMM README,
 * "Interfaces / Notes": on the SM100 path the scale factors are UE8M0, four
 * of them packed into one 32-bit integer; the Ascend 950 article packs them
 * along K as well).  A UE8M0 byte e stands for the scale 2^(e - 127) (OCP MX
 * E8M0; e = 255 is NaN).  Reading of the packing: byte j (bits 8j..8j+7) of a
 * word holds the scale of K block 4w + j; bytes past the last K block are
 * ignored.  With W = ceil(K/512):
 *   sfa int32 [W][M] (masked: [G][W][M_max]), MN-major like the FP32 sfa;
 *   sfb int32 [Nb][W] (grouped: [G][Nb][W]), K-contiguous like the FP32 sfb.
 * Block sizes, layouts of A, B, C, D, the group and mask rules, ownership and
 * errors are those of the FP32-scale entry points above; the result is
 * D = C + sum_kb 2^(ea-127) 2^(eb-127) P_kb, rounded once to BF16.  On gfx950
 * the MFMA applies these scales itself, so no promotion step is needed.
 */
dg_status dg_fp8_gemm_nt_ue8m0(const void *A, const int32_t *sfa, const void *B, const int32_t *sfb,
                               const float *C, void *D, int M, int N, int K, void *stream);
dg_status dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const void *A, const int32_t *sfa, const void *B,
                                                    const int32_t *sfb, const int32_t *m_indices,
                                                    const float *C, void *D, int M, int N, int K,
                                                    int num_groups, void *stream);
dg_status dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const void *A, const int32_t *sfa, const void *B,
                                                const int32_t *sfb, const int32_t *masked_m,
                                                const float *C, void *D, int M_max, int N, int K,
                                                int num_groups, void *stream);

/*
 * The same three forms with UE8M0 scale factors packed in pairs along K into
 * 16-bit words, stored MN-major (DeepGEMM-Ascend news article, the paragraph
 * on the scale-factor format: on Ascend each pair of UE8M0 factors along K is
 * packed into one int16, values in MN-major order).  Readings: byte h (bits
 * 8h..8h+7) of pair word p holds the scale of K block 2p + h; a trailing byte
 * past the last K block is ignored; both operands are MN-major.  With
 * P = ceil(K/256):
 *   sfa int16 [P][M] (masked: [G][P][M_max]): row m fastest, like the FP32 sfa;
 *   sfb int16 [P][Nb] (grouped: [G][P][Nb]): the 128-row block index of B fastest.
 * The scale arrays must be 2-byte aligned.  Block sizes (1x128, 128x128),
 * A, B, C, D, groups, masks, ownership and errors as for the entry points
 * above; the matrix core applies the scales (no promotion step), and
 * D = C + sum_kb 2^(ea-127) 2^(eb-127) P_kb, rounded once to BF16.
 */
dg_status dg_fp8_gemm_nt_ue8m0_i16(const void *A, const int16_t *sfa, const void *B, const int16_t *sfb,
                                   const float *C, void *D, int M, int N, int K, void *stream);
dg_status dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_i16(const void *A, const int16_t *sfa, const void *B,
                                                        const int16_t *sfb, const int32_t *m_indices,
                                                        const float *C, void *D, int M, int N, int K,
                                                        int num_groups, void *stream);
dg_status dg_m_grouped_fp8_gemm_nt_masked_ue8m0_i16(const void *A, const int16_t *sfa, const void *B,
                                                    const int16_t *sfb, const int32_t *masked_m,
                                                    const float *C, void *D, int M_max, int N, int K,
                                                    int num_groups, void *stream);

/*
 * FP8 x FP4: the same three forms with FP4 weights (DeepGEMM-Ascend hub page,
 * precision table "FP8 x FP4"; DeepGEMM README, news of 2026.04.16: an
 * FP8 x FP4 GEMM with FP4 weights and UE8M0 scale factors).
 *   A, sfa: as in the packed-UE8M0 entry points above (E4M3, one UE8M0 scale
 *     per 1x128 block, sfa int32 [W][M], masked [G][W][M_max]).
 *   B uint8 [N][K/2] (grouped: [G][N][K/2]): OCP MX E2M1 codes, two per
 *     byte, element 2i in the low nibble of byte i (reading: the OCP packing
 *     order).  E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0;
 *     magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN.
 *   sfb int32 [N][Kb] (grouped: [G][N][Kb]): one UE8M0 scale per 1x32 block
 *     of each row of B (reading: the OCP MX block of 32); byte j of word
 *     [n][kb] scales K elements 128 kb + 32 j .. 128 kb + 32 j + 31.
 *   D = C + sum over 32-wide K blocks j of 2^(ea-127) 2^(eb-127) S_j, S_j the
 *   exact block dot product, rounded once to BF16 (the matrix core applies
 *   both scales; FP32 accumulation).
 * C, D, the group and mask rules, ownership and errors are those of the
 * entry points above; B must be 16-byte aligned.
 */
dg_status dg_fp8_fp4_gemm_nt(const void *A, const int32_t *sfa, const void *B, const int32_t *sfb,
                             const float *C, void *D, int M, int N, int K, void *stream);
dg_status dg_m_grouped_fp8_fp4_gemm_nt_contiguous(const void *A, const int32_t *sfa, const void *B,
                                                  const int32_t *sfb, const int32_t *m_indices,
                                                  const float *C, void *D, int M, int N, int K,
                                                  int num_groups, void *stream);
dg_status dg_m_grouped_fp8_fp4_gemm_nt_masked(const void *A, const int32_t *sfa, const void *B,
                                              const int32_t *sfb, const int32_t *masked_m,
                                              const float *C, void *D, int M_max, int N, int K,
                                              int num_groups, void *stream);

/*
 * K-grouped, TN, contiguous (MoE weight backward).  DeepGEMM README, "Grouped
 * GEMM (contiguous layout)": a K-axis grouped call (k_grouped_fp8_gemm_tn_contiguous)
 * with M and N fixed; the groups' K segments are concatenated along K.  The
 * page names the call only, so its layout is a reading:
 *   A uint8 (E4M3) [K][M] and B uint8 (E4M3) [K][N]: both K-outermost ("TN";
 *     row k of A holds the M values of K index k), the layout in which token
 *     gradients and activations are stored for a weight gradient;
 *   sfa float [K/128][M], sfb float [K/128][N]: one FP32 scale per 128 K rows
 *     of each column (1x128 along K for both operands);
 *   ks int32 [G] (device): K rows of each group, in order; group g owns rows
 *     [ks[0] + ... + ks[g-1], + ks[g]).  Each count must be a multiple of 128
 *     (a negative count is taken as 0; the segments are cut at K; a count
 *     that is not a multiple of 128 gives undefined values for that group and
 *     the later ones, but no access outside the buffers);
 *   C float [G][M][N] or NULL, D bf16 [G][M][N]:
 *     D[g] = C[g] + sum over the K blocks kb of group g of
 *            sfa[kb][m] * sfb[kb][n] * (exact block dot product of column m of A
 *            and column n of B), rounded once to BF16.
 * An empty group gets D[g] = C[g] (or zeros).  K must be a multiple of 128.
 * The library rewrites A and B K-contiguous into a per-stream device buffer of
 * (M + N) * ceil(K/1024)*1024 bytes (allocated on the first call of a size,
 * kept until exit), then runs the GEMM on it.  Ownership, streams and errors
 * as above.
 */
dg_status dg_k_grouped_fp8_gemm_tn_contiguous(const void *A, const float *sfa, const void *B,
                                              const float *sfb, const int32_t *ks, const float *C,
                                              void *D, int M, int N, int K, int num_groups,
                                              void *stream);

/*
 * BF16 x BF16 without scale factors (DeepGEMM-Ascend hub page, precision
 * table "BF16 x BF16" for ordinary-precision training; DeepGEMM README intro:
 * GEMM in FP8, FP4 and BF16): D = C + A . B^T with A and B in BF16, FP32
 * accumulation, BF16 D (round-to-nearest-even, once).  Layouts as the FP8 NT
 * forms with 2-byte elements and no sfa/sfb: dense A [M][K], B [N][K];
 * contiguous A [M][K], B [G][N][K], m_indices [M]; masked A [G][M_max][K],
 * B [G][N][K], masked_m [G]; C float like D or NULL.  K must be a multiple of
 * 64 (one 128-byte block; reading, the pages give no rule), M of the
 * contiguous form a multiple of 128.  Ownership, streams, group and mask rules
 * and errors as for the FP8 forms.
 */
dg_status dg_bf16_gemm_nt(const void *A, const void *B, const float *C, void *D, int M, int N, int K,
                          void *stream);
dg_status dg_m_grouped_bf16_gemm_nt_contiguous(const void *A, const void *B, const int32_t *m_indices,
                                               const float *C, void *D, int M, int N, int K,
                                               int num_groups, void *stream);
dg_status dg_m_grouped_bf16_gemm_nt_masked(const void *A, const void *B, const int32_t *masked_m,
                                           const float *C, void *D, int M_max, int N, int K,
                                           int num_groups, void *stream);

/*
 * FP4 x FP4 (DeepGEMM-Ascend hub page, precision table "FP4 x FP4" for
 * ultra-low-bit inference; the page names no call, so the layout is a
 * reading): A as well as B in OCP E2M1 (two codes a byte, element 2i in the
 * low nibble of byte i), each row of each operand with one UE8M0 scale per
 * 1x32 block, the four of a 128-wide K block in one word (byte j: K elements
 * 128 kb + 32 j .. + 31):
 *   A uint8 [M][K/2] (masked [G][M_max][K/2]), sfa int32 [M][K/128]
 *     (masked [G][M_max][K/128]); B and sfb as for FP8 x FP4.
 *   D = C + sum over 32-wide K blocks of 2^(ea-127) 2^(eb-127) S_j, rounded
 *   once to BF16.  C, D, groups, masks, ownership and errors as above.
 */
dg_status dg_fp4_fp4_gemm_nt(const void *A, const int32_t *sfa, const void *B, const int32_t *sfb,
                             const float *C, void *D, int M, int N, int K, void *stream);
dg_status dg_m_grouped_fp4_fp4_gemm_nt_contiguous(const void *A, const int32_t *sfa, const void *B,
                                                  const int32_t *sfb, const int32_t *m_indices,
                                                  const float *C, void *D, int M, int N, int K,
                                                  int num_groups, void *stream);
dg_status dg_m_grouped_fp4_fp4_gemm_nt_masked(const void *A, const int32_t *sfa, const void *B,
                                              const int32_t *sfb, const int32_t *masked_m,
                                              const float *C, void *D, int M_max, int N, int K,
                                              int num_groups, void *stream);

/*
 * Health of the current device's kernels.  The producer/consumer kernel
 * variant (one wave streams the A tiles into an LDS ring, the others wait on
 * per-slot LDS flags; chosen for few rows, e.g. M <= 128) bounds every such
 * wait (about 30 ms) so that a fault in its hand-off can never hang the
 * device.  A wait that runs out adds one to a device-wide counter, and the D of
 * that call is then not to be trusted.  dg_get_wait_giveups() copies the
 * counter to *count and dg_reset_wait_giveups() clears it; both synchronise
 * with the device (not for use inside stream capture).  The counter is 0
 * unless something went wrong.
 */
dg_status dg_get_wait_giveups(unsigned int *count);
dg_status dg_reset_wait_giveups(void);

/* Message for the calling thread's last non-OK status ("" if none).  Owned by the library. */
const char *dg_last_error(void);

/*
 * Row alignment every expert segment of the contiguous layout must start on
 * (DeepGEMM README, utility functions: get_mk_alignment_for_contiguous_layout).
 * Always 128 here.
 */
int dg_get_mk_alignment_for_contiguous_layout(void);

/*
 * Upper bound on the compute units the kernels spread over (README utility
 * functions: set_num_sms / get_num_sms).  n <= 0 or above the device's count
 * restores the device's count.  Affects tile heuristics of later calls only.
 */
dg_status dg_set_num_cus(int n);
int dg_get_num_cus(void);

/*
 * Optional eager set-up on the current device: device query, cache directory,
 * default-stream workspace.  Never needed, but lets a caller keep first-call
 * allocation out of a timed or captured region.
 */
dg_status dg_init(void);

/* Flags OR-ed into `kind` below for the packed-UE8M0 and the FP8 x FP4 entry points. */
#define DG_SCALE_UE8M0 4
#define DG_SCALE_FP8_FP4 8
#define DG_BF16 16           /* BF16 x BF16 without scales (K in elements) */
#define DG_SCALE_FP4_FP4 32  /* FP4 x FP4 */
#define DG_SCALE_UE8M0_I16 64   /* UE8M0 pairs in 16-bit words, MN-major */

/*
 * Compile (or load from the cache) the kernel(s) that a later call with these
 * arguments would use, without launching anything.  kind: 0 dense,
 * 1 contiguous, 2 masked, 3 K-grouped (K = the K rows; the FP32 scale form
 * only) (| DG_SCALE_UE8M0 for packed UE8M0 scales, | DG_SCALE_UE8M0_I16 for
 * UE8M0 pairs in 16-bit words, | DG_SCALE_FP8_FP4 for FP8 x FP4, | DG_BF16,
 * | DG_SCALE_FP4_FP4); has_c:
 * 0/1; rows = M (dense/contiguous) or M_max.
 * Needs no GPU: the code object is built for gfx950 and stored in the cache
 * directory (DG_CACHE_DIR, else <library dir>/jit_cache).
 */
dg_status dg_precompile(int kind, int rows, int N, int K, int num_groups, int has_c, int num_cus);

/*
 * Name of the kernel configuration (tile, waves, LDS stages, split-K, sizes)
 * that a call with these arguments selects on the current device (or for
 * `num_cus` compute units when num_cus > 0), written NUL-terminated into
 * buf[0..len).  A call that launches two kernels over disjoint column ranges
 * (two tile widths) gets both names joined by '+'.  Informational; nothing is
 * compiled or launched.
 */
dg_status dg_describe_config(int kind, int rows, int N, int K, int num_groups, int has_c, int num_cus,
                             char *buf, int len);

#ifdef __cplusplus
}
#endif

#endif /* DG_H_ */
