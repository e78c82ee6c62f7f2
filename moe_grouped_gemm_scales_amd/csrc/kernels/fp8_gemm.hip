// Block-scaled FP8 GEMM for gfx950 (CDNA4):  D = C + A . B^T  (NT layout).
//
// Device code only.  The host library embeds this file as text and compiles
// it at run time with hipRTC, once per shape/tile key, with the key's values
// passed as -D macros (DeepGEMM launch article, section 4.2: matrix sizes and
// tile/pipeline parameters are compile-time constants of a JIT-built kernel).
//
// What it computes (DeepGEMM README, "Interfaces / Notes"; launch article,
// section 2 "FP8" on promotion):
//   A  [rows][K]  E4M3 codes, one FP32 scale per 1x128 block, sfa[K/128][rows]
//   B  [N][K]     E4M3 codes, one FP32 scale per 128x128 block, sfb[ceil(N/128)][K/128]
//   D[m][n] = bf16( C[m][n] + sum_kb sfa[kb][m] * sfb[n/128][kb] * P_kb[m][n] )
// where P_kb is the exact-product, FP32-summed 128-wide block dot product from
// one v_mfma_f32_16x16x128_f8f6f4, promoted into FP32 VGPR accumulators.
//
// Forms (DG_KIND):
//   0 dense
//   1 M-grouped contiguous (README "Grouped GEMM (contiguous layout)"): rows of
//     all experts concatenated; grp = m_indices[rows]; a row block takes its
//     expert from its first row, rows whose index differs are left untouched.
//   2 M-grouped masked (README "Grouped GEMM (masked layout)"): A/D are
//     [G][M_max][.]; grp = masked_m[G]; rows >= clamp(masked_m[g]) untouched.
//   3 K-grouped (README "Grouped GEMM (contiguous layout)": the K-axis grouped
//     call of the MoE weight backward, M and N fixed): D[g] = C[g] + the sum
//     over the K blocks of group g only; grp = ks[G], the K rows of each group
//     in order.  A and B here are the operands already made K-contiguous
//     ([M][K], [N][K] with K the padded row pitch) by dg_transpose_k_major
//     below; B has one FP32 scale per column and K block, sfb[K/128][N].
//
// Layout of the work (MI355X-specific, not from the pages):
//   * MFMA orientation is swapped: the MFMA "row" operand is a 16-row slice of
//     B and the "column" operand a 16-row slice of A, so a lane owns one m and
//     four consecutive n.  Promotion then needs one scale product per
//     (m, 128-wide n block) and the BF16 store is 8 contiguous bytes.
//   * Operand tiles go global -> LDS by buffer_load ... lds (no VGPR staging)
//     into a STAGES-deep ring; each 128-byte row is stored with its 16-byte
//     chunks XOR-swizzled by (row & 7), which makes the fragment reads
//     bank-conflict free (measured with SQ_LDS_BANK_CONFLICT).
//   * A persistent grid walks tiles; split-K partials (dense only) are summed
//     in a fixed order by the last-arriving workgroup of a tile.

typedef unsigned char u8;
typedef unsigned short u16;
typedef unsigned int u32;
typedef unsigned long long u64;
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef u16 v4u16 __attribute__((ext_vector_type(4)));

#ifndef DG_KIND
#define DG_KIND 0
#define DG_BM 128
#define DG_BN 128
#define DG_WM 2
#define DG_WN 2
#define DG_STAGES 2
#define DG_KSTEP 1
#define DG_SPLITK 1
#define DG_HAS_C 0
#define DG_N 256
#define DG_K 256
#define DG_G 1
#endif
#ifndef DG_VARIANT
#define DG_VARIANT 0
#endif
// Scale format: 0 = FP32 scales (sfa [K/128][rows], sfb [ceil(N/128)][K/128]);
// 1 = UE8M0 (DeepGEMM README, "Interfaces / Notes", SM100: four UE8M0 scale
// factors packed into one 32-bit integer): byte j of a word is K block 4w + j,
// sfa words [ceil(K/512)][rows], sfb words [ceil(N/128)][ceil(K/512)].  The
// MFMA applies UE8M0 block scales itself, so there is no promotion step.
// 2 = FP8 x FP4 (DeepGEMM-Ascend hub page, precision table; DeepGEMM README
// news 2026.04.16): A and sfa as for 1; B holds OCP E2M1 codes, two per byte
// (element 2i in the low nibble of byte i), [N][K/2]; sfb holds one UE8M0
// scale per 1x32 block of each row of B, the four of a 128-wide K block in
// one word, [N][K/128] (byte j: K elements 128 kb + 32 j .. + 32).
// 3 = BF16 x BF16 without scales (DeepGEMM-Ascend hub page, precision table;
// DeepGEMM README intro: GEMM in FP8, FP4 and BF16): A [rows][K], B [N][K]
// BF16, D = C + A . B^T.  DG_K is then the row length in BYTES (2 x K), so a
// 128-byte "K block" is 64 BF16 elements, two v_mfma_f32_16x16x32_bf16.
// 4 = FP4 x FP4 (DeepGEMM-Ascend hub page, precision table): A as well as B
// in E2M1, [rows][K/2], each row with one UE8M0 scale per 1x32 block, sfa
// [rows][K/128] words (masked [G][M_max][K/128]) laid out like sfb of 2.
// 5 = UE8M0 scale pairs (DeepGEMM-Ascend news article, scale-factor format:
// every pair of UE8M0 scales along K in one int16, stored MN-major): byte h
// of pair word p is K block 2p + h; sfa int16 [ceil(K/256)][rows] (masked
// [G][.][M_max]), sfb int16 [ceil(K/256)][ceil(N/128)] (grouped [G][.][.]).
// Otherwise as 1: the MFMA applies the scales.
#ifndef DG_SF
#define DG_SF 0
#endif
// Column range of D this kernel computes (a launch may cover part of N, so
// that one call can use two tile widths and fill whole rounds of the grid)
#ifndef DG_NB
#define DG_NB 0
#endif
#ifndef DG_NE
#define DG_NE DG_N
#endif
// DG_BSTREAM: each B block is read by at most two row blocks of the launch, so
// B's loads carry the non-temporal hint (the host sets it for dense and masked
// launches of few rows)
#ifndef DG_BSTREAM
#define DG_BSTREAM 0
#endif

namespace dg {

constexpr int kKind = DG_KIND;
constexpr int BM = DG_BM, BN = DG_BN, WM = DG_WM, WN = DG_WN;
constexpr int NWAVES = WM * WN;
constexpr int NTHREADS = 64 * NWAVES;
// split-K arrival counters: one per output tile and wave, each in a 128-byte
// line of its own (the host sizes the counter buffer with the same stride)
constexpr int CTR_STRIDE = 32;
constexpr int WAVE_M = BM / WM, WAVE_N = BN / WN;
constexpr int TM = WAVE_M / 16, TN = WAVE_N / 16;
constexpr int STAGES = DG_STAGES;
constexpr int KSTEP = DG_KSTEP;             // 128-wide K blocks per LDS stage
constexpr int SPLITK = DG_SPLITK;
constexpr bool HAS_C = DG_HAS_C != 0;
constexpr int N = DG_N, K = DG_K, G = DG_G;
constexpr int KBLK = 128;
constexpr int KBLKS = K / KBLK;
constexpr int NBLKS = (N + KBLK - 1) / KBLK;
constexpr int N_BEGIN = DG_NB, N_END = DG_NE;  // columns [N_BEGIN, N_END) of D; N is the row pitch
static_assert(0 <= N_BEGIN && N_BEGIN < N_END && N_END <= N && N_BEGIN % 16 == 0, "column range");
constexpr int NUM_NT = (N_END - N_BEGIN + BN - 1) / BN;     // n tiles
constexpr bool SF_E8 = DG_SF == 1 || DG_SF == 2 || DG_SF == 4 || DG_SF == 5;
constexpr bool PAIRS = DG_SF == 5;            // UE8M0 pairs in 16-bit words, MN-major (A and B)
constexpr bool FP4B = DG_SF == 2 || DG_SF == 4;   // B in E2M1 with per-row 1x32 UE8M0 scales
constexpr bool FP4A = DG_SF == 4;             // A in E2M1 with per-row 1x32 UE8M0 scales too
constexpr bool BF16 = DG_SF == 3;             // BF16 operands, no scales
constexpr int KW = PAIRS ? (KBLKS + 1) / 2 : (KBLKS + 3) / 4;   // packed UE8M0 words per row of scales
constexpr int SF_KB = SF_E8 ? KW : KBLKS;     // scale entries (floats or words) along K
constexpr int SF_BYTES = PAIRS ? 2 : 4;       // bytes of one scale entry (float, 32-bit or 16-bit word)
constexpr int KB_B = FP4B ? K / 2 : K;        // bytes of one row of B
constexpr int KB_A = FP4A ? K / 2 : K;        // ... of A
// a wave's n range [n0 + wn*WAVE_N, +WAVE_N) never crosses a 128 boundary when
// WAVE_N divides 128 (tiles start at multiples of BN, a multiple of WAVE_N);
// FP4 B has a scale per row, never one per wave
constexpr bool KG = kKind == 3;                // K-grouped: per-column B scales, per-group K ranges
constexpr bool SB_UNIFORM = (KBLK % WAVE_N) == 0 && (DG_NB % WAVE_N) == 0 && !FP4B && !KG && !BF16;
static_assert(!BF16 || (DG_KSTEP == 1 && kKind != 3), "BF16: one K block a stage, M-grouped or dense");
static_assert(!KG || (!SF_E8 && DG_SPLITK == 1 && DG_KSTEP == 1), "K-grouped: FP32 scales, no split-K, one K block a stage");

static_assert(K % KBLK == 0, "K must be a multiple of 128");
static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "wave tiles must be 16-aligned");
static_assert(KSTEP == 1 || KSTEP == 2, "one or two K blocks per stage");
static_assert(KBLKS % (SPLITK * KSTEP) == 0, "split-K and stage depth must divide the K blocks");
static_assert(STAGES >= 2, "at least double buffering");

// Register budget: 256 per lane, as for two waves per SIMD, whatever the wave
// count.  The kernel declares a maximum workgroup size of at least 512 lanes
// (it is launched with NTHREADS; LDS keeps one workgroup per CU): with a
// 256-lane maximum the compiler plans for one wave per SIMD, writes MFMA
// results to AGPRs and copies every one back with v_accvgpr_read before the
// promotion FMA, doubling the VALU work per MFMA.
// Exception: with no promotion step (UE8M0 scales applied by the MFMA, or BF16)
// a 4-wave workgroup with more than 32 sub-tiles per wave keeps its accumulators
// in AGPRs, which the MFMAs read and write directly; it declares its own size.
constexpr bool ACC_IN_AGPR = (DG_SF == 1 || DG_SF == 3 || DG_SF == 5) && NTHREADS == 256 && TM * TN > 32;
constexpr int MAX_THREADS_DECL = (NTHREADS < 512 && !ACC_IN_AGPR) ? 512 : NTHREADS;

struct Params {
    const u8* A;
    const float* sfa;
    const u8* B;
    const float* sfb;
    const float* C;
    u16* D;
    const int* grp;        // m_indices (contiguous) or masked_m (masked); unused for dense
    float* ws;             // split-K partials
    u32* counters;         // split-K arrival counters, zero between calls
    int M;                 // rows of A (dense, contiguous) or M_max (masked)
    int num_tiles;         // total work items for this launch
    int kt;                // K-grouped: K rows of the operands (the groups' segments are cut there)
    u32* status;           // library status words: [0] counts bounded waits that gave up
};

// The kernel's one argument: the pointers and sizes of Params, passed by value in
// one struct.  The HIP runtime prepares every argument of a launch on the host
// (about 0.15-0.2 us each), so one argument instead of thirteen takes about 2 us
// off each call.  The pointers are global memory.
#define DG_GLOBAL __attribute__((address_space(1)))
struct KernArgs {
    const DG_GLOBAL u8* A;
    const DG_GLOBAL float* sfa;
    const DG_GLOBAL u8* B;
    const DG_GLOBAL float* sfb;
    const DG_GLOBAL float* C;
    DG_GLOBAL u16* D;
    const DG_GLOBAL int* grp;
    DG_GLOBAL float* ws;
    DG_GLOBAL u32* counters;
    int M;
    int num_tiles;
    int kt;
    DG_GLOBAL u32* status;
};
static_assert(sizeof(KernArgs) == 96 && __builtin_offsetof(KernArgs, M) == 72 &&
              __builtin_offsetof(KernArgs, status) == 88, "the host fills this layout");

// Promotion scale of one MFMA result: one FP32 per (row, 128-row block of B),
// or, K-grouped, one per column, i.e. a vector over the lane's four columns.
template <bool V> struct ScaleType { typedef float type; };
template <> struct ScaleType<true> { typedef v4f type; };
typedef ScaleType<KG>::type sc_t;
// the first (or only) scale, and its bits (for branches the K-grouped form never takes)
__device__ __forceinline__ float first(float x) { return x; }
__device__ __forceinline__ float first(v4f x) { return x.x; }

// ------------------------------------------------------------ small helpers
__device__ __forceinline__ v4i make_rsrc(const void* base, u32 num_bytes) {
    u64 p = (u64)base;
    v4i r;
    r.x = (int)(u32)p;
    r.y = (int)((u32)(p >> 32) & 0xffffu);   // stride 0
    r.z = (int)num_bytes;
    r.w = 0x00020000;                        // raw buffer, dword data format
    r.x = __builtin_amdgcn_readfirstlane(r.x);
    r.y = __builtin_amdgcn_readfirstlane(r.y);
    r.z = __builtin_amdgcn_readfirstlane(r.z);
    r.w = __builtin_amdgcn_readfirstlane(r.w);
    return r;
}

// One lane-linear LDS DMA: lane l writes its 16 (or 4) bytes to lds + 16*l (or 4*l).
// Issued through inline asm so that the compiler does not answer every later
// LDS read with a blanket wait for all outstanding DMA; the ring's own
// vmcnt waits below give the exact ordering instead.
__device__ __forceinline__ void dma16(v4i rsrc, u32 voff, u32 soff, u32 lds) {
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds) : "memory");
}
// B's 16-byte DMA: with DG_BSTREAM the non-temporal hint rides along
__device__ __forceinline__ void dma16b(v4i rsrc, u32 voff, u32 soff, u32 lds) {
    if constexpr (DG_BSTREAM)
        asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen nt lds"
                     :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds) : "memory");
    else
        dma16(rsrc, voff, soff, lds);
}
__device__ __forceinline__ void dma4(v4i rsrc, u32 voff, u32 soff, u32 lds) {
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dword %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds) : "memory");
}
// Two bytes per lane, zero-extended into the lane's 4-byte LDS word (lds + 4*l).
__device__ __forceinline__ void dma2(v4i rsrc, u32 voff, u32 soff, u32 lds) {
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_ushort %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds) : "memory");
}
// The scale DMA of a stage: 32-bit entries, or 16-bit UE8M0 pairs
__device__ __forceinline__ void dma_sf(v4i rsrc, u32 voff, u32 soff, u32 lds) {
    if constexpr (PAIRS) dma2(rsrc, voff, soff, lds);
    else dma4(rsrc, voff, soff, lds);
}
template <int CNT>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(CNT >= 0 && CNT <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(CNT) : "memory");
}

__device__ __forceinline__ u16 f32_to_bf16(float f) {
    const u32 u = __builtin_bit_cast(u32, f);
    const u32 rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;    // nearest-even
    const u32 qnan = (u >> 16) | 0x40u;                              // NaN: quiet, sign and payload top kept
    return (u16)((u & 0x7fffffffu) > 0x7f800000u ? qnan : rounded);  // a select, not a branch
}

// The lane's index within its wave, computed where it is called (an asm the
// compiler neither hoists nor merges with an earlier copy).
__device__ __forceinline__ int lane_id_now() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// two BF16 values (x in the low half) in one word
__device__ __forceinline__ u32 bf16_pair(float x, float y) { return (u32)f32_to_bf16(x) | ((u32)f32_to_bf16(y) << 16); }

__device__ __forceinline__ u32 lds_addr(const void* p) {
    return (u32)(u64)(const __attribute__((address_space(3))) void*)p;
}
typedef __attribute__((address_space(3))) const v4i lds_v4i;
typedef __attribute__((address_space(3))) const float lds_f32;
typedef __attribute__((address_space(3))) const u8 lds_u8;
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
// the two 16-byte halves of a fragment as BF16 MFMA operands (8 elements each)
__device__ __forceinline__ v8bf bf_lo(v8i x) { return __builtin_bit_cast(v8bf, v4i{x[0], x[1], x[2], x[3]}); }
__device__ __forceinline__ v8bf bf_hi(v8i x) { return __builtin_bit_cast(v8bf, v4i{x[4], x[5], x[6], x[7]}); }
// Fragment read: two 16-byte chunks at lane-specific bases plus a constant
// offset, written as pointer arithmetic so the offset folds into ds_read_b128.
__device__ __forceinline__ v8i lds_read_frag(lds_u8* lo, lds_u8* hi, int off) {
    const v4i a = *(lds_v4i*)(lo + off);
    const v4i b = *(lds_v4i*)(hi + off);
    return v8i{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}
__device__ __forceinline__ float lds_read_f32(lds_u8* base, int off) { return *(lds_f32*)(base + off); }
// FP4 fragment: 32 E2M1 codes in 16 bytes; the MFMA reads only the low four
// registers of an FP4 operand.
__device__ __forceinline__ v8i lds_read_frag4(lds_u8* p, int off) {
    const v4i a = *(lds_v4i*)(p + off);
    return v8i{a.x, a.y, a.z, a.w, 0, 0, 0, 0};
}

// ------------------------------------------------------------ tile decode
struct Tile {
    int m0;          // first row of the tile within its A/D (per-group for masked)
    int n0;          // first column
    int g;           // group (B/sfb select; A/sfa/C/D too for masked)
    int rows;        // valid rows in [m0, m0 + BM) for loads (>= 1)
    int row_limit;   // rows m0 + r with r < row_limit may be stored (masked / dense tail)
    int kb0, kb1;    // K-block range
    int split;       // split index
    int mn;          // output tile index (for split-K bookkeeping)
    int g2;          // contiguous, 256-row blocks: the expert of rows 128.. when it differs, else -1
    bool skip;
};

// Workgroups go to the 8 XCDs (each with its own L2) round-robin by index.
// Within every round of the persistent grid (the last one possibly partial,
// with R < grid work items), give XCD x a contiguous range of the logical
// order, so that the items it runs at the same time are neighbours there and
// share their A and B blocks in its L2.  WG b of the round runs on XCD b % 8
// as the (b / 8)-th of the ceil((R - x) / 8) WGs there; the ranges of the
// XCDs partition [0, R).
__device__ __forceinline__ int xcd_spread(int t, int num_items) {
    const int grid = gridDim.x;
    if (grid % 8 != 0) return t;
    const int r0 = t - t % grid;                          // first item of this round
    const int R = num_items - r0 < grid ? num_items - r0 : grid;
    const int b = t - r0;                                 // < R
    const int x = b % 8;
    return r0 + x * (R / 8) + (x < R % 8 ? x : R % 8) + b / 8;
}

// Dense and contiguous forms: output tile (mt, nt) and K split of work item t.
// Grouped order: walk 8 m-tiles per column sweep so that concurrently resident
// workgroups share A and B tiles in L2.
__device__ __forceinline__ void tile_position(const Params& p, int t, int& mn, int& split, int& mt, int& nt) {
    const int num_mt = (p.M + BM - 1) / BM;
    t = xcd_spread(t, p.num_tiles);
    mn = t / SPLITK;
    split = t % SPLITK;
    constexpr int GROUP_M = 8;
    const int width = GROUP_M * NUM_NT;
    const int first_m = mn / width * GROUP_M;
    const int gsize = num_mt - first_m < GROUP_M ? num_mt - first_m : GROUP_M;
    mt = first_m + (mn % width) % gsize;
    nt = (mn % width) / gsize;
}

// Contiguous form: the experts of the first and (256-row blocks) second 128 rows
// of work item t's row block, read ahead of the tile's decode.
__device__ __forceinline__ void tile_experts(const Params& p, int t, int& g, int& g2) {
    int mn, split, mt, nt;
    tile_position(p, t, mn, split, mt, nt);
    const int m0 = mt * BM;
    g = p.grp[m0];
    g2 = (BM > 128 && m0 + 128 < p.M) ? p.grp[m0 + 128] : -1;
}

// PRE: the contiguous form's experts come from tile_experts() (g_pre, g2_pre)
// instead of being read here.
template <bool PRE = false>
__device__ __forceinline__ Tile decode_tile(const Params& p, int t, int g_pre = 0, int g2_pre = -1) {
    Tile tl;
    tl.skip = false;
    tl.g2 = -1;
    tl.split = 0;
    tl.kb0 = 0;
    tl.kb1 = KBLKS;
    if constexpr (kKind == 2) {
        // Masked: enumerate only the active row blocks, group by group.
        const int nmt_max = (p.M + BM - 1) / BM;
        int g = 0, base = 0;
        int mb = 0, nt = 0, valid = 0;
        tl.skip = true;
        for (; g < G; ++g) {
            int v = p.grp[g];
            v = v < 0 ? 0 : (v > p.M ? p.M : v);
            int nmt = (v + BM - 1) / BM;
            if (nmt > nmt_max) nmt = nmt_max;
            int cnt = nmt * NUM_NT;
            if (t < base + cnt) {
                int local = t - base;
                mb = local % nmt;                 // row blocks fastest: they share B
                nt = local / nmt;
                valid = v;
                tl.skip = false;
                break;
            }
            base += cnt;
        }
        tl.g = g;
        tl.m0 = mb * BM;
        tl.n0 = N_BEGIN + nt * BN;
        tl.rows = p.M - tl.m0 < BM ? p.M - tl.m0 : BM;
        tl.row_limit = valid - tl.m0;
        tl.mn = 0;
    } else if constexpr (kKind == 3) {
        // K-grouped: every group has the same output tiles; its K range is the
        // prefix sum of ks (negative counts taken as 0, cut at kt; a count that
        // is not a multiple of 128 makes this and later groups' values
        // undefined, never an access out of bounds)
        const int num_mt = (p.M + BM - 1) / BM;
        const int per_g = num_mt * NUM_NT;
        t = xcd_spread(t, p.num_tiles);
        const int g = t / per_g;
        const int local = t % per_g;
        int off = 0;
        for (int h = 0; h < g; ++h) off += p.grp[h] > 0 ? p.grp[h] : 0;
        int len = p.grp[g] > 0 ? p.grp[g] : 0;
        const int kbt = p.kt / KBLK;
        int kb0 = off / KBLK, kb1 = (off + len) / KBLK;
        kb0 = kb0 < kbt ? kb0 : kbt;
        kb1 = kb1 < kbt ? kb1 : kbt;
        // grouped order inside the group: 8 row blocks per column sweep
        constexpr int GROUP_M = 8;
        const int width = GROUP_M * NUM_NT;
        const int first_m = local / width * GROUP_M;
        const int gsize = num_mt - first_m < GROUP_M ? num_mt - first_m : GROUP_M;
        const int mt = first_m + (local % width) % gsize, nt = (local % width) / gsize;
        tl.g = g;
        tl.m0 = mt * BM;
        tl.n0 = N_BEGIN + nt * BN;
        tl.rows = p.M - tl.m0 < BM ? p.M - tl.m0 : BM;
        tl.row_limit = tl.rows;
        tl.kb0 = kb0;
        tl.kb1 = kb1 > kb0 ? kb1 : kb0;
        tl.mn = 0;
    } else {
        int mn, mt, nt;
        tile_position(p, t, mn, tl.split, mt, nt);
        tl.mn = mn;
        tl.m0 = mt * BM;
        tl.n0 = N_BEGIN + nt * BN;
        tl.rows = p.M - tl.m0 < BM ? p.M - tl.m0 : BM;
        tl.row_limit = tl.rows;
        tl.kb0 = tl.split * (KBLKS / SPLITK);
        tl.kb1 = tl.kb0 + KBLKS / SPLITK;
        if constexpr (kKind == 1) {
            const int g = PRE ? g_pre : p.grp[tl.m0];
            tl.g = g;
            tl.skip = (g < 0 || g >= G);
            // every 128-row block of the layout names one expert (its first row's):
            // a 256-row block covers two, which may differ
            if constexpr (BM > 128) {
                if (tl.m0 + 128 < p.M) {
                    const int g2 = PRE ? g2_pre : p.grp[tl.m0 + 128];
                    if (g2 >= 0 && g2 < G && g2 != g) tl.g2 = g2;
                }
            }
        } else {
            tl.g = 0;
        }
    }
    return tl;
}


// ------------------------------------------------------------ end of a work item
// Split-K bookkeeping and the epilogue, shared by every kernel variant.  acc
// holds TM_ x TN_ blocks of 16 x 16: lane (l16, q) owns row row0 + 16 a and
// the four columns col0 + 16 b + [0, 4) of each (row0, col0 relative to the
// tile).  Returns after storing, or early when another split finishes this
// wave's slice of the tile.
// Paired 16-byte stores (see the epilogue) need an even number of n sub-tiles
// and 8-column alignment of every row, tile and column range.
template <int TN_>
constexpr bool PAIRED_STORES = TN_ % 2 == 0 && N % 8 == 0 && N_BEGIN % 8 == 0 && N_END % 8 == 0 && BN % 8 == 0;

// GRP_LDS (contiguous form): the expert of the lane's row row0 + 16 a is the
// int at LDS address grp_lds + 64 a, instead of being read from global memory.
template <int TM_, int TN_, bool GRP_LDS = false>
__device__ __forceinline__ void finish_tile(const Params& p, const Tile& tl, v4f (&acc)[TM_][TN_], int row0,
                                            int col0, int tid, u32 grp_lds = 0) {
    // An MFMA reads the operands of every lane of its wave, whatever EXEC
    // holds.  Pin every accumulator here, while the whole wave is active:
    // otherwise, when the K loop is short enough to be laid out straight, the
    // compiler may sink the last MFMAs, with the per-lane values feeding them
    // (scale shifts, fragment reads), into the row-guarded stores below, where
    // those values are only computed for the lanes of rows that are stored.
#pragma unroll
    for (int a = 0; a < TM_; ++a)
#pragma unroll
        for (int b = 0; b < TN_; ++b) asm volatile("" : "+v"(acc[a][b]));
    // ---- split-K: publish the partial, the last arrival sums all in split order
    if constexpr (SPLITK > 1) {
        float* ws = p.ws + ((u64)tl.mn * SPLITK) * (BM * BN);
        // The splits of a tile run on any of the 8 XCDs, each with its own L2, so
        // a partial must be visible across L2s without a cache write-back (an
        // agent-scope release fence writes back the whole L2: 7-10 us per work
        // item, longer than the K loop).  The stores carry the agent-scope cache
        // policy (sc1), which writes them through this XCD's L2 to the
        // device-coherent side (Infinity Fabric, MALL, HBM); the last arrival
        // reads them back with agent-scope loads, which do not take a line from
        // its own L2.  Each wave hands off its own slice of the tile: its lanes
        // write, and the lanes of that wave in the last split read, the same
        // words of every split's partial, and the wave's arrival has a counter of
        // its own, alone in a 128-byte line (atomics on one line are serialised
        // where they are performed: with four counters to a line the hand-off
        // took 0.9 us longer).  The wave waits for its stores' acknowledgement (vmcnt 0)
        // before its agent-scope arrival atomic, so when that count shows every
        // split arrived, every split's slice is at the coherence point.  No
        // workgroup barrier: a wave that is not last returns at once.
        constexpr int CPOL_AGENT = 16;
        // The partials are read once: the reads also carry the non-temporal hint
        // (the scope stays that of sc1), which took 64 x 2112 x 7168 from 10.9 to
        // 9.7 us; on the stores the same hint made it 0.8 us slower.
        constexpr int CPOL_AGENT_NT = CPOL_AGENT | 2;
        constexpr u32 WS_BYTES = SPLITK * BM * BN * 4;
        const __amdgpu_buffer_rsrc_t rs_ws = __builtin_amdgcn_make_buffer_rsrc(ws, 0, WS_BYTES, 0x00020000);
#pragma unroll
        for (int a = 0; a < TM_; ++a)
#pragma unroll
            for (int b = 0; b < TN_; ++b)
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(v4i, acc[a][b]), rs_ws,
                    (tl.split * BM * BN + ((a * TN_ + b) * NTHREADS + tid) * 4) * 4, 0, CPOL_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        u32* const ctr = p.counters + ((u64)tl.mn * NWAVES + (tid >> 6)) * CTR_STRIDE;
        u32 old = 0;
        if ((tid & 63) == 0) {
            old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (old == (u32)(SPLITK - 1)) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (__builtin_amdgcn_readfirstlane(old) != (u32)(SPLITK - 1)) return;
        asm volatile("" ::: "memory");
        // Every partial is summed in split order, the same order on every run,
        // CH splits' loads in flight together without running out of registers.
        // With few sub-tiles this split's own partial is kept in registers (the
        // same bits it stored) and its load is given an offset past the buffer,
        // which returns zeros without a memory access.
        constexpr bool OWN = TM_ * TN_ <= 8;
        v4f own[OWN ? TM_ : 1][OWN ? TN_ : 1];
        if constexpr (OWN) {
#pragma unroll
            for (int a = 0; a < TM_; ++a)
#pragma unroll
                for (int b = 0; b < TN_; ++b) own[a][b] = acc[a][b];
        }
        constexpr int CH0 = 28 / (TM_ * TN_);
        constexpr int CH = CH0 < 1 ? 1 : (CH0 > SPLITK ? SPLITK : CH0);
        int wofs = 0;
#pragma unroll
        for (int s0 = 0; s0 < SPLITK; s0 += CH) {
            v4f part[CH][TM_][TN_];
#pragma unroll
            for (int c = 0; c < CH; ++c)
                if (s0 + c < SPLITK) {
                    const bool mine = OWN && s0 + c == tl.split;
#pragma unroll
                    for (int a = 0; a < TM_; ++a)
#pragma unroll
                        for (int b = 0; b < TN_; ++b)
                            part[c][a][b] = __builtin_bit_cast(
                                v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                         rs_ws,
                                         mine ? WS_BYTES
                                              : (wofs + (s0 + c) * BM * BN + ((a * TN_ + b) * NTHREADS + tid) * 4) * 4,
                                         0, CPOL_AGENT_NT));
                }
#pragma unroll
            for (int c = 0; c < CH; ++c)
                if (s0 + c < SPLITK) {
                    const bool mine = OWN && s0 + c == tl.split;
#pragma unroll
                    for (int a = 0; a < TM_; ++a)
#pragma unroll
                        for (int b = 0; b < TN_; ++b) {
                            v4f v = part[c][a][b];
                            if constexpr (OWN) v = mine ? own[a][b] : v;
                            acc[a][b] = (s0 + c == 0) ? v : acc[a][b] + v;
                        }
                }
            // the next chunk's loads depend on this opaque zero, taken after this
            // chunk's sums, so the compiler cannot hoist them all (and spill them)
            // ahead of those sums
            asm volatile("" : "+s"(wofs) : "v"(acc[0][0]));
        }
    }

    // ---- epilogue: (+C), BF16 nearest-even, store rows that may be written
    // The lane's row and column bases pass through an empty asm here, so the
    // store addresses are computed now: otherwise the compiler computes all of
    // them before the K loop, and with no register left across the loop it
    // spills them, so every store first waits for a scratch reload (and with it
    // for every store issued before it).
    asm volatile("" : "+v"(row0), "+v"(col0));
    u64 row_base;      // element offset of row 0 of this tile in C/D
    if constexpr (kKind == 2 || kKind == 3) row_base = ((u64)tl.g * p.M + tl.m0) * N;
    else row_base = (u64)tl.m0 * N;
#pragma unroll
    for (int a = 0; a < TM_; ++a) {
        const int r = row0 + a * 16;            // row inside the tile
        bool row_ok = r < tl.row_limit;
        if constexpr (kKind == 1) {
            const int gr = GRP_LDS ? *(__attribute__((address_space(3))) const int*)(grp_lds + a * 64)
                                   : p.grp[tl.m0 + r];
            row_ok = row_ok && gr == tl.g;
        }
        if (!row_ok) continue;
        if constexpr (PAIRED_STORES<TN_>) {
            // Sub-tiles b, b + 1 in pairs: lanes q and q ^ 1 (16 apart, same row,
            // same row_ok) swap four values, so that each lane holds 8 consecutive
            // columns and the four lanes of a row cover 64 contiguous bytes: even q
            // keeps its b values and takes its partner's (4 columns on), odd q keeps
            // its b + 1 values and takes its partner's (4 columns before).
            const bool odd = ((col0 >> 2) & 1) != 0;
#pragma unroll
            for (int b = 0; b < TN_; b += 2) {
                const int n = tl.n0 + col0 + b * 16;      // this lane's columns of sub-tile b
                const u64 off = row_base + (u64)r * N + n;
                v4f v0 = acc[a][b], v1 = acc[a][b + 1];
                if constexpr (HAS_C) {
                    if (n < N_END) v0 += *(const v4f*)(p.C + off);
                    if (n + 16 < N_END) v1 += *(const v4f*)(p.C + off + 16);
                }
                const u32 lo0 = bf16_pair(v0.x, v0.y), hi0 = bf16_pair(v0.z, v0.w);
                const u32 lo1 = bf16_pair(v1.x, v1.y), hi1 = bf16_pair(v1.z, v1.w);
                // ds_swizzle, bit mode: lane ^ 16 inside each half of the wave
                const u32 r_lo = (u32)__builtin_amdgcn_ds_swizzle((int)(odd ? lo0 : lo1), 0x401F);
                const u32 r_hi = (u32)__builtin_amdgcn_ds_swizzle((int)(odd ? hi0 : hi1), 0x401F);
                const int n_out = odd ? n + 12 : n;         // odd: columns 16 (b + 1) + 4 (q - 1) ..
                if (n_out >= N_END) continue;
                const v4i o = odd ? v4i{(int)r_lo, (int)r_hi, (int)lo1, (int)hi1}
                                  : v4i{(int)lo0, (int)hi0, (int)r_lo, (int)r_hi};
                *(v4i*)(p.D + row_base + (u64)r * N + n_out) = o;
            }
            continue;
        }
#pragma unroll
        for (int b = 0; b < TN_; ++b) {
            const int n = tl.n0 + col0 + b * 16;
            if (n >= N_END) continue;
            const u64 off = row_base + (u64)r * N + n;
            v4f v = acc[a][b];
            if constexpr (N % 4 == 0 && N_END % 4 == 0) {
                if constexpr (HAS_C) v += *(const v4f*)(p.C + off);
                v4u16 o = {f32_to_bf16(v.x), f32_to_bf16(v.y), f32_to_bf16(v.z), f32_to_bf16(v.w)};
                *(v4u16*)(p.D + off) = o;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (n + e < N_END) {
                        float x = v[e];
                        if constexpr (HAS_C) x += p.C[off + e];
                        p.D[off + e] = f32_to_bf16(x);
                    }
                }
            }
        }
    }
}

// 16 bytes per lane from global memory into VGPRs.  Inline asm, like the DMA,
// so that the compiler leaves the wait to the kernel's own vmcnt accounting;
// the destination is only read after that wait and tie() below.
template <int OFF>
__device__ __forceinline__ v4i load16(v4i rsrc, u32 voff, u32 soff) {
    v4i r;
    if constexpr (DG_BSTREAM)
        asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen offset:%4 nt"
                     : "=v"(r) : "v"(voff), "s"(rsrc), "s"(soff), "n"(OFF) : "memory");
    else
        asm volatile("buffer_load_dwordx4 %0, %1, %2, %3 offen offset:%4"
                     : "=v"(r) : "v"(voff), "s"(rsrc), "s"(soff), "n"(OFF) : "memory");
    return r;
}
// After the wait: a register the loads wrote is redefined here, so no use of it
// can be scheduled before the wait.
__device__ __forceinline__ void tie(v4i& x) { asm volatile("" : "+v"(x)); }

template <int... Is> struct iseq {};
template <int Nn, int... Is> struct make_iseq { using type = typename make_iseq<Nn - 1, Nn - 1, Is...>::type; };
template <int... Is> struct make_iseq<0, Is...> { using type = iseq<Is...>; };
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F& f, iseq<Is...>) { (f.template operator()<Is>(), ...); }
template <int Nn, typename F>
__device__ __forceinline__ void static_for(F&& f) { static_for_impl(f, typename make_iseq<Nn>::type{}); }

#if DG_VARIANT == 0
// ============================================================ variant 0: both operands through LDS
// LDS ring: per stage [A tile BM x ROWB][B tile BN x ROWB][sfa, BM floats per K block, padded].
// A stage holds KSTEP consecutive K blocks, so each tile row is ROWB contiguous
// bytes of its global row: with K = 1536 (a 1.5 KB row pitch) HBM streams B
// far better in 256-byte than in 128-byte pieces.
constexpr int ROWB = 128 * KSTEP;               // bytes of one tile row in a stage
constexpr int RPI = 1024 / ROWB;                // tile rows per 1 KB DMA instruction
// FP4 B: a K block of a row is 64 bytes, 16 rows per instruction, its four
// 16-byte chunks XOR-swizzled by (row >> 2) & 3
constexpr int ROWB_B = FP4B ? 64 : ROWB;
constexpr int RPI_B = 1024 / ROWB_B;
constexpr int ROWB_A = FP4A ? 64 : ROWB;        // FP4 A: the same 64-byte rows as FP4 B
constexpr int RPI_A = 1024 / ROWB_A;
constexpr int NA_INS = BM / RPI_A;              // 1 KB DMA instructions for A
constexpr int NB_INS = BN / RPI_B;              // ... for B
constexpr int NS_PER_KB = BF16 ? 0 : (BM + 63) / 64;   // 256 B DMA instructions for one K block of sfa
constexpr int NS_INS = NS_PER_KB * KSTEP;
constexpr int A_OFF = 0;
constexpr int B_OFF = BM * ROWB_A;
constexpr int S_OFF = B_OFF + BN * ROWB_B;
constexpr int S_BYTES = NS_PER_KB * 256;        // sfa bytes per K block
// sfb of the (at most three) 128-row blocks of B a tile touches, one 256 B
// DMA per K block, so the K loop issues no scalar loads; FP4 B: one word per
// row of the tile, K-grouped: one float per column, 64 per DMA
constexpr int T_OFF = S_OFF + KSTEP * S_BYTES;
constexpr int NT_INS = BF16 ? 0 : (FP4B || KG) ? (BN + 63) / 64 : KSTEP;
constexpr int STAGE_BYTES = T_OFF + NT_INS * 256;
static_assert(BN <= 256, "a tile touches at most three 128-row blocks of B");
static_assert(!SF_E8 || KSTEP == 1, "UE8M0 scales: one K block per stage");
static_assert(!BF16 || (KBLKS >= 1 && K % 128 == 0), "BF16: K bytes a multiple of 128");
// A ahead (DG_AAHEAD, two-slot ring only): the A tiles and their scales get a ring
// of their own with one slot more than B's, so A is requested two K blocks ahead
// and B one; the rings then are [A slots x (A tile, sfa)][B slots x (B tile, sfb)].
#ifndef DG_AAHEAD
#define DG_AAHEAD 0
#endif
constexpr bool AAHEAD = DG_AAHEAD != 0;
static_assert(!AAHEAD || (KSTEP == 1 && STAGES == 2), "A ahead: one K block a stage, two B slots");
static_assert(!AAHEAD || (!FP4A && !FP4B && !KG), "A ahead: FP8 (128x128 B scales) or BF16 operands");
constexpr int A_SLOT = BM * ROWB_A + S_BYTES;                 // A ahead: one A slot
constexpr int B_SLOT = BN * ROWB_B + NT_INS * 256;            // A ahead: one B slot
constexpr int A_SLOTS = STAGES + 1;
constexpr int B_RING = A_SLOTS * A_SLOT;
constexpr int RING_BYTES = AAHEAD ? B_RING + STAGES * B_SLOT : STAGES * STAGE_BYTES;
// Contiguous form: the expert of each of the wave's rows (WAVE_M <= 64 of them),
// brought into LDS by one DMA of the wave at the start of the tile, so the
// epilogue does not wait on global reads of the group index while every CU
// stores its tile.
constexpr bool ROW_GRP_LDS = kKind == 1 && WAVE_M <= 64;
constexpr int GRP_OFF = RING_BYTES;
constexpr int LDS_BYTES = RING_BYTES + (ROW_GRP_LDS ? NWAVES * 256 : 0);
static_assert(BM % RPI_A == 0 && BN % RPI_B == 0, "tiles are loaded RPI rows per instruction");
static_assert(LDS_BYTES <= 160 * 1024, "LDS ring exceeds 160 KB");

// Every wave issues the same number of DMA instructions per stage, so one
// vmcnt immediate fits all waves: instruction i of a category goes to wave
// i % NWAVES, and a wave whose share runs out repeats the category's last
// instruction (identical bytes to identical LDS addresses, so harmless).
constexpr int IA = (NA_INS + NWAVES - 1) / NWAVES;
constexpr int IB = (NB_INS + NWAVES - 1) / NWAVES;
constexpr int IS = (NS_INS + NWAVES - 1) / NWAVES;
constexpr int IT = (NT_INS + NWAVES - 1) / NWAVES;
// One scale instruction per wave: scale instruction i goes to wave i (the A
// scales first, then the B scales) and the waves past them repeat the last B
// one, so a stage costs the CU NWAVES scale instructions instead of
// NWAVES * (IS + IT) (8 instead of 16 for a 256 x 256 tile).  The wave's choice
// is made with scalar selects, so the MFMA sequence it is spread over has no
// branch, and every wave still issues the same count.
#ifndef DG_SCALE_DIET
#define DG_SCALE_DIET 1
#endif
// Wave priority (0-3) while a wave issues one n sub-tile's MFMAs; 0 leaves it alone.
#ifndef DG_SETPRIO
#define DG_SETPRIO 0
#endif
constexpr bool DIET = DG_SCALE_DIET != 0 && !AAHEAD && NS_INS + NT_INS > 0 && NS_INS + NT_INS <= NWAVES;
constexpr int INS_PER_WAVE = DIET ? IA + IB + 1 : IA + IB + IS + IT;
static_assert(INS_PER_WAVE * (STAGES - 1) <= 63, "vmcnt range");
// MFMA steps (n sub-tiles of a stage's first K block) the refill is spread over;
// 0: all at once.  It must be issued before the last sub-tile, where the wait
// for the next stage counts it.
#ifndef DG_SPREAD
#define DG_SPREAD (STAGES == 2 ? (TN + 1) / 2 : TN)
#endif
constexpr int SPREAD = DG_SPREAD < TN - 1 ? DG_SPREAD : TN - 1;

// Split refill (DG_SPLIT): a slot is handed back in two parts.  Its A tile, its
// scales and the B rows of the first half of every wave's n sub-tiles are read
// by the middle of the K block (A and the scales at its start, those B rows by
// sub-tile TN/2 - 1), so after a barrier there they are refilled with the K
// block STAGES ahead (the "mid" group); the B rows of the second half follow
// after the barrier at the end of the block (the "end" group).  Every load then
// has about half a K block more time to land, and the CU keeps more bytes in
// flight.  Each wait is for one group, with the (STAGES - 1) later mid and end
// groups still pending.
#ifndef DG_SPLIT
#define DG_SPLIT 0
#endif
constexpr bool SPLIT = DG_SPLIT != 0;
constexpr int HALF_TN = TN / 2;
constexpr int NB_HALF = NB_INS / 2;                      // B DMA instructions of one half
constexpr int IBH = (NB_HALF + NWAVES - 1) / NWAVES;    // ... per wave
constexpr int NSC_PER_WAVE = INS_PER_WAVE - IA - IB;    // scale DMA instructions per wave
constexpr int G_MID = IA + IBH + NSC_PER_WAVE;
constexpr int G_END = IBH;
constexpr int SPLIT_PENDING = (STAGES - 1) * (G_MID + G_END);
static_assert(!SPLIT || (KSTEP == 1 && !AAHEAD && TN % 2 == 0 && TN >= 4 && !FP4A && !FP4B),
              "split refill: FP8 or BF16 operands, one K block a slot, an even number of n sub-tiles");
// B instruction i covers 8 rows inside one 16-row n sub-tile of one wave column
// (2 TN instructions per column): the first TN of a column are the first half
static_assert(!SPLIT || (RPI == 8 && NB_INS == WN * 2 * TN), "split refill: 8 B rows per instruction");
static_assert(!SPLIT || SPLIT_PENDING <= 63, "vmcnt range");
// The mid group is spread over the sub-tiles from the mid barrier on, the end
// group over the first ones of the next block; each must be issued in full
// before the next wait, which counts it.
constexpr int MID_STEPS = TN - HALF_TN;                  // steps HALF_TN - 1 .. TN - 2
constexpr int END_STEPS = HALF_TN - 1;                   // steps 0 .. HALF_TN - 2

// contiguous form with 256-row blocks: up to two passes over a tile, one per expert
constexpr int PIECES = (kKind == 1 && BM > 128) ? 2 : 1;
static_assert(kKind != 1 || BM <= 128 || BM == 256, "contiguous row blocks: at most 128 rows, or 256");

// Wait until at most PENDING whole stages of this wave's DMA remain in flight.
template <int PENDING>
__device__ __forceinline__ void wait_stages() { wait_vmcnt<PENDING * INS_PER_WAVE>(); }

// ------------------------------------------------------------ the kernel
// Arguments are separate __restrict__ pointers (not one struct) so that the
// compiler may read the uniform ones (sfb, group info) with scalar loads.
extern "C" __global__ void __attribute__((amdgpu_flat_work_group_size(1, MAX_THREADS_DECL)))
dg_fp8_gemm_nt_kernel(const KernArgs ka) {
    const u8* __restrict__ A = (const u8*)ka.A;
    const float* __restrict__ sfa = (const float*)ka.sfa;
    const u8* __restrict__ B = (const u8*)ka.B;
    const float* __restrict__ sfb = (const float*)ka.sfb;
    const float* __restrict__ C = (const float*)ka.C;
    u16* __restrict__ D = (u16*)ka.D;
    const int* __restrict__ grp = (const int*)ka.grp;
    float* __restrict__ ws = (float*)ka.ws;
    u32* __restrict__ counters = (u32*)ka.counters;
    const int M = ka.M, num_tiles = ka.num_tiles, kt = ka.kt;
    u32* __restrict__ status = (u32*)ka.status;
    const Params p{A, sfa, B, sfb, C, D, grp, ws, counters, M, num_tiles, kt, status};
    // Every argument in one round trip of scalar loads: otherwise the loop bound
    // is fetched first and the pointers only after it arrives (~0.5 us each).
    asm volatile("" :: "s"(A), "s"(sfa), "s"(B), "s"(sfb), "s"(C), "s"(D), "s"(grp), "s"(ws), "s"(counters), "s"(M),
                 "s"(num_tiles), "s"(gridDim.x));
    __shared__ __attribute__((aligned(1024))) u8 smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM;          // wave position along m
    const int wn = wave / WM;          // wave position along n
    const int l16 = lane & 15;
    const int q = lane >> 4;
    const u32 smem_base = lds_addr(smem);
    // Every fragment row this lane reads is l16 plus a multiple of 16, so the
    // swizzle term row & 7 is the same for all of them.  Lane group q takes the
    // 16-byte K chunks q and q + 4 of its row (the K order inside one MFMA only
    // has to agree between the two operands, and it does: both use this map);
    // with chunks XOR-swizzled by row & 7 these reads are free of LDS bank
    // conflicts on gfx950, where chunks 2q, 2q + 1 were not.
    // The matrix core pairs the operands by its own K index: in an E4M3
    // operand, bytes 0-15 of lane group q are K 16q .. 16q+15 and bytes 16-31
    // are K 64+16q .. 64+16q+15 (the map above, so these are those K); in an
    // E2M1 operand, the 32 codes of lane group q are K 32q .. 32q+31, which is
    // 16-byte chunk q of B's 64-byte row, and the lane's scale byte applies
    // to them: exactly one 1x32 scale block (mapped with one-hot rows of A).
    const int sw = l16 & 7;
    const u32 chunk_lo = (u32)((q ^ sw) << 4);
    const u32 chunk_hi = (u32)(((q ^ 4) ^ sw) << 4);
    const u32 a_frag_off = (u32)(wm * WAVE_M + l16) * ROWB_A;
    const u32 b_frag_off = (u32)(wn * WAVE_N + l16) * ROWB_B;
    const u32 b_chunk_lo = FP4B ? (u32)((q ^ ((l16 >> 2) & 3)) << 4) : chunk_lo;
    const u32 a_chunk_lo = FP4A ? (u32)((q ^ ((l16 >> 2) & 3)) << 4) : chunk_lo;

    // contiguous form: the experts of the next work item's row block, read one
    // work item ahead so that the decode does not wait for them
    int g_next = 0, g2_next = -1;
    if constexpr (kKind == 1) {
        if ((int)blockIdx.x < p.num_tiles) tile_experts(p, blockIdx.x, g_next, g2_next);
    }
#pragma unroll 1
    for (int t = blockIdx.x; t < p.num_tiles; t += gridDim.x) {
        const Tile tl0 = decode_tile<kKind == 1>(p, t, g_next, g2_next);
        if constexpr (kKind == 1) {
            if (t + (int)gridDim.x < p.num_tiles) tile_experts(p, t + gridDim.x, g_next, g2_next);
        }
        // A contiguous row block of 256 rows holds two 128-row blocks of the
        // layout; when their experts differ the tile is computed once for each
        // (the epilogue stores a row only for its own expert).
#pragma unroll 1
        for (int piece = 0; piece < PIECES; ++piece) {
            Tile tl = tl0;
            if (piece == 1) {
                if (tl0.g2 < 0) break;
                tl.g = tl0.g2;
                tl.skip = false;
            }
            if (tl.skip) continue;

            // ---- per-tile buffer resources (bases advanced to the tile's rows)
            const u8* a_base;
            const float* sfa_base;
            int a_rows_total;        // rows of this A (for sfa stride)
            if constexpr (kKind == 2) {
                a_base = p.A + ((u64)tl.g * p.M + tl.m0) * KB_A;
                sfa_base = (const float*)((const u8*)p.sfa +
                                          (u64)tl.g * (FP4A ? KBLKS : SF_KB) * p.M * (FP4A ? 4u : (u32)SF_BYTES));
            } else {
                a_base = p.A + (u64)tl.m0 * KB_A;
                sfa_base = p.sfa;
            }
            a_rows_total = p.M;
            const int n_rows = N_END - tl.n0 < BN ? N_END - tl.n0 : BN;
            const u8* b_base = p.B + ((u64)(KG ? 0 : tl.g) * N + tl.n0) * KB_B;
            const v4i rs_a = make_rsrc(a_base, (u32)tl.rows * KB_A);
            const v4i rs_b = make_rsrc(b_base, (u32)n_rows * KB_B);
            const v4i rs_s = make_rsrc(sfa_base, (u32)(FP4A ? KBLKS : SF_KB) * a_rows_total * (FP4A ? 4u : (u32)SF_BYTES));
            const v4i rs_t = FP4B ? make_rsrc(p.sfb + ((u64)tl.g * N + tl.n0) * KBLKS, (u32)n_rows * KBLKS * 4u)
                             : KG ? make_rsrc(p.sfb, (u32)(p.kt / KBLK) * N * 4u)
                                  : make_rsrc((const u8*)p.sfb + (u64)tl.g * NBLKS * SF_KB * SF_BYTES,
                                              (u32)NBLKS * SF_KB * (u32)SF_BYTES);
            const int nb_t0 = tl.n0 / KBLK;                  // first 128-row block of B in this tile

            // ---- per-lane DMA offsets (fixed over K).  Lane l of an instruction
            // writes LDS bytes [16 l, 16 l + 16) of its 1 KB: tile row RPI*i + l / (ROWB/16),
            // K block h of the stage, physical chunk p = l % 8, which holds logical
            // chunk p ^ (row & 7).  The lane part is kept in one register (two when
            // RPI = 4, where the swizzle also depends on the parity of i) and the
            // instruction's row offset i*RPI*K is added at issue.  Rows past the tile
            // (ragged M or N) give offsets past the buffer's size: the load returns
            // zeros without touching memory, and those rows are never stored.
            auto lane_voff = [&](int i) {
                const int r = i * RPI + lane / (ROWB / 16);
                const int h = (lane % (ROWB / 16)) / 8;
                const int c = (lane & 7) ^ (r & 7);
                return (u32)(lane / (ROWB / 16)) * K + h * 128 + c * 16;
            };
            constexpr int NPAR = (RPI % 8) == 0 ? 1 : 8 / RPI;   // distinct (i*RPI) & 7 values
            static_assert(NPAR == 1 || NPAR == 2, "rows per instruction");
            u32 voff_rows[NPAR];
#pragma unroll
            for (int par = 0; par < NPAR; ++par) voff_rows[par] = lane_voff(par);
            // FP4 B: lane l writes row l / 4 of the instruction's 16, physical chunk
            // l & 3, which holds logical chunk (l & 3) ^ ((row >> 2) & 3); the row's
            // swizzle term does not depend on the instruction (16 rows each)
            const u32 voff_b4 = (u32)(lane >> 2) * KB_B + (u32)(((lane & 3) ^ ((lane >> 4) & 3)) << 4);
            const u32 voff_b4a = (u32)(lane >> 2) * KB_A + (u32)(((lane & 3) ^ ((lane >> 4) & 3)) << 4);   // FP4 A
            u32 voff_s[IS > 0 ? IS : 1];   // A scales: clamped rows (the offset includes the K block's row of sfa)
#pragma unroll
            for (int j = 0; j < IS; ++j) {
                const int i = min(wave + j * NWAVES, NS_INS - 1);
                const int h = i / NS_PER_KB;
                const int m = tl.m0 + (i % NS_PER_KB) * 64 + lane;
                const int mm = m < a_rows_total ? m : a_rows_total - 1;
                // FP4 A: word [m][kb] (row-major); otherwise sfa [kb][m] (MN-major)
                voff_s[j] = FP4A ? (u32)mm * KBLKS * 4u : (u32)mm * SF_BYTES + (u32)h * a_rows_total * SF_BYTES;
            }
            u32 voff_t[IT > 0 ? IT : 1];
#pragma unroll
            for (int j = 0; j < IT; ++j) {
                // without repeats, wave NS_INS + h issues B-scale instruction h
                const int h = DIET ? min(max(wave - NS_INS, 0), NT_INS - 1) : min(wave + j * NWAVES, NT_INS - 1);
                if constexpr (FP4B) {
                    // word [n0 + 64 h + lane][kb]; rows past the tile read as zero
                    voff_t[j] = (u32)(64 * h + lane) * KBLKS * 4u;
                } else if constexpr (KG) {
                    // sfb[kb][n0 + 64 h + lane], columns past N clamped (never stored)
                    voff_t[j] = (u32)min(tl.n0 + 64 * h + lane, N - 1) * 4u;
                } else {
                    const int nb = min(nb_t0 + lane, NBLKS - 1);
                    // UE8M0 pairs: MN-major [K/256][NBLKS]; otherwise K-contiguous [NBLKS][SF_KB]
                    voff_t[j] = PAIRS ? (u32)nb * 2u : (u32)nb * SF_KB * 4u + (u32)h * 4u;
                }
            }

            // one scale instruction per wave: an A-scale one (waves 0 .. NS_INS-1) or a B-scale one
            const bool is_a_sc = wave < NS_INS;
            const u32 voff_sc = is_a_sc ? voff_s[0] : voff_t[0];
            const u32 lds_sc = __builtin_amdgcn_readfirstlane(
                is_a_sc ? (u32)(S_OFF + wave * 256) : (u32)(T_OFF + min(max(wave - NS_INS, 0), NT_INS - 1) * 256));
            v4i rs_sc = is_a_sc ? rs_s : rs_t;
            rs_sc.x = __builtin_amdgcn_readfirstlane(rs_sc.x);
            rs_sc.y = __builtin_amdgcn_readfirstlane(rs_sc.y);
            rs_sc.z = __builtin_amdgcn_readfirstlane(rs_sc.z);
            rs_sc.w = __builtin_amdgcn_readfirstlane(rs_sc.w);
            // DMA instruction j (0 <= j < INS_PER_WAVE) of one stage for this wave
            // (kb: first K block of the stage)
            // index along K of the scales of K block kb (a word holds four UE8M0 scales)
            auto sf_row = [](int kb) { return PAIRS ? kb >> 1 : SF_E8 ? kb >> 2 : kb; };
            // scalar offset of K block kb's B scales: a row of the MN-major pairs, or a K-contiguous entry
            auto sfb_soff = [](int kb) { return PAIRS ? (u32)(kb >> 1) * NBLKS * 2u : (u32)(SF_E8 ? kb >> 2 : kb) * 4u; };
            // live = false: a placeholder load whose buffer size is zero, so it moves
            // no data (every lane is out of range) but keeps the vmcnt count fixed.
            auto issue_one = [&](int j, int kb, int stage, bool live = true) {
                const u32 st = __builtin_amdgcn_readfirstlane(smem_base + stage * STAGE_BYTES);
                auto lim = [&](v4i r) {
                    r.z = live ? r.z : 0;
                    return r;
                };
                if (j < IA) {
                    const int i = min(wave + j * NWAVES, NA_INS - 1);
                    if constexpr (FP4A)
                        dma16(lim(rs_a), voff_b4a + (u32)__builtin_amdgcn_readfirstlane((u32)(i * RPI_A) * (u32)KB_A),
                              __builtin_amdgcn_readfirstlane((u32)kb * (KBLK / 2)), st + A_OFF + i * 1024);
                    else
                        dma16(lim(rs_a), voff_rows[i % NPAR] + (u32)__builtin_amdgcn_readfirstlane((u32)(i * RPI) * (u32)K),
                              __builtin_amdgcn_readfirstlane((u32)kb * KBLK), st + A_OFF + i * 1024);
                } else if (j < IA + IB) {
                    const int i = min(wave + (j - IA) * NWAVES, NB_INS - 1);
                    if constexpr (FP4B)
                        dma16b(lim(rs_b), voff_b4 + (u32)__builtin_amdgcn_readfirstlane((u32)(i * RPI_B) * (u32)KB_B),
                              __builtin_amdgcn_readfirstlane((u32)kb * (KBLK / 2)), st + B_OFF + i * 1024);
                    else
                        dma16b(lim(rs_b), voff_rows[i % NPAR] + (u32)__builtin_amdgcn_readfirstlane((u32)(i * RPI) * (u32)K),
                              __builtin_amdgcn_readfirstlane((u32)kb * KBLK), st + B_OFF + i * 1024);
                } else if (DIET) {
                    // this wave's scale instruction: resource, lane offset and LDS place chosen
                    // once per tile (rs_sc, voff_sc, lds_sc); only the K block's offset varies
                    const u32 soff = is_a_sc ? (FP4A ? (u32)kb * 4u : (u32)sf_row(kb) * a_rows_total * (u32)SF_BYTES)
                                             : (FP4B ? (u32)kb * 4u : KG ? (u32)kb * N * 4u : sfb_soff(kb));
                    dma_sf(lim(rs_sc), voff_sc, __builtin_amdgcn_readfirstlane(soff),
                           __builtin_amdgcn_readfirstlane(st + lds_sc));
                } else if (j < IA + IB + IS) {
                    const int i = min(wave + (j - IA - IB) * NWAVES, NS_INS - 1);
                    dma_sf(lim(rs_s), voff_s[j - IA - IB],
                           __builtin_amdgcn_readfirstlane(FP4A ? (u32)kb * 4u
                                                               : (u32)sf_row(kb) * a_rows_total * (u32)SF_BYTES),
                           st + S_OFF + i * 256);
                } else {
                    const int h = min(wave + (j - IA - IB - IS) * NWAVES, NT_INS - 1);
                    dma_sf(lim(rs_t), voff_t[j - IA - IB - IS],
                           __builtin_amdgcn_readfirstlane(FP4B ? (u32)kb * 4u : KG ? (u32)kb * N * 4u : sfb_soff(kb)),
                           st + T_OFF + h * 256);
                }
            };
            auto issue_stage = [&](int kb, int stage, bool live = true) {
#pragma unroll
                for (int j = 0; j < INS_PER_WAVE; ++j) issue_one(j, kb, stage, live);
            };
            // split refill: B instruction of half `hi` with index bi inside that half
            auto issue_b_half = [&](int bi, bool hi, int kb, int stage, bool live) {
                const u32 st = __builtin_amdgcn_readfirstlane(smem_base + stage * STAGE_BYTES);
                v4i r = rs_b;
                r.z = live ? r.z : 0;
                const int i = (bi / TN) * (2 * TN) + (hi ? TN : 0) + bi % TN;
                dma16b(r, voff_rows[i % NPAR] + (u32)__builtin_amdgcn_readfirstlane((u32)(i * RPI) * (u32)K),
                      __builtin_amdgcn_readfirstlane((u32)kb * KBLK), st + B_OFF + i * 1024);
            };
            // instruction j of the mid group (A, first-half B rows, scales) and of the end group
            auto issue_mid = [&](int j, int kb, int stage, bool live) {
                if (j < IA) issue_one(j, kb, stage, live);
                else if (j < IA + IBH) issue_b_half(min(wave + (j - IA) * NWAVES, NB_HALF - 1), false, kb, stage, live);
                else issue_one(j - IBH + IB, kb, stage, live);
            };
            auto issue_end = [&](int j, int kb, int stage, bool live) {
                issue_b_half(min(wave + j * NWAVES, NB_HALF - 1), true, kb, stage, live);
            };
            // A ahead: instruction j of one iteration's issue, in the order B, sfb (K block
            // kb_b into B slot sl_b), then A, sfa (K block kb_a into A slot sl_a), so that
            // waiting until only the last IA + IS are in flight lands everything but A's.
            auto issue_one_aa = [&](int j, int kb_a, int sl_a, bool live_a, int kb_b, int sl_b, bool live_b) {
                auto lim = [&](v4i r, bool live) {
                    r.z = live ? r.z : 0;
                    return r;
                };
                const u32 sa_base = __builtin_amdgcn_readfirstlane(smem_base + sl_a * A_SLOT);
                const u32 sb_base = __builtin_amdgcn_readfirstlane(smem_base + B_RING + sl_b * B_SLOT);
                if (j < IB) {
                    const int i = min(wave + j * NWAVES, NB_INS - 1);
                    dma16b(lim(rs_b, live_b), voff_rows[i % NPAR] + (u32)__builtin_amdgcn_readfirstlane((u32)(i * RPI) * (u32)K),
                          __builtin_amdgcn_readfirstlane((u32)kb_b * KBLK), sb_base + i * 1024);
                } else if (j < IB + IT) {
                    const int h = min(wave + (j - IB) * NWAVES, NT_INS - 1);
                    dma_sf(lim(rs_t, live_b), voff_t[j - IB], __builtin_amdgcn_readfirstlane(sfb_soff(kb_b)),
                           sb_base + BN * ROWB_B + h * 256);
                } else if (j < IB + IT + IA) {
                    const int i = min(wave + (j - IB - IT) * NWAVES, NA_INS - 1);
                    dma16(lim(rs_a, live_a), voff_rows[i % NPAR] + (u32)__builtin_amdgcn_readfirstlane((u32)(i * RPI) * (u32)K),
                          __builtin_amdgcn_readfirstlane((u32)kb_a * KBLK), sa_base + i * 1024);
                } else {
                    const int i = min(wave + (j - IB - IT - IA) * NWAVES, NS_INS - 1);
                    dma_sf(lim(rs_s, live_a), voff_s[j - IB - IT - IA],
                           __builtin_amdgcn_readfirstlane((u32)sf_row(kb_a) * a_rows_total * (u32)SF_BYTES),
                           sa_base + BM * ROWB_A + i * 256);
                }
            };

            // ---- accumulators
            v4f acc[TM][TN];
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int b = 0; b < TN; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
            // MFMA results of the last n sub-tile of the previous K block and their
            // scales: promoted while the next K block's first MFMAs run.
            v4f p_carry[TM];
            sc_t s_carry[TM];
#pragma unroll
            for (int a = 0; a < TM; ++a) {
                p_carry[a] = v4f{0.f, 0.f, 0.f, 0.f};
                s_carry[a] = 0.f;
            }

            // Every wave has finished reading the ring (the earlier tile's last K
            // block) before any refills it.  The earlier tile's stores may still be
            // in flight: the loads below overlap them, and each wait of the ring
            // counts only the loads issued after the group it waits for, which
            // complete in order, so a store still pending only delays a wait.
            __syncthreads();
            // the experts of this wave's rows (contiguous form), for the epilogue;
            // rows past M read as 0 and are never stored
            if constexpr (ROW_GRP_LDS) {
                dma4(make_rsrc(p.grp, (u32)p.M * 4u), (u32)(tl.m0 + wm * WAVE_M + lane) * 4u, 0u,
                     __builtin_amdgcn_readfirstlane(smem_base + GRP_OFF + wave * 256));
            }

            const int nst = (tl.kb1 - tl.kb0) / KSTEP;       // stages of this tile
            if constexpr (AAHEAD) {
                // B and A of K block 0, then A of K block 1 (placeholders past the tile)
#pragma unroll
                for (int j = 0; j < INS_PER_WAVE; ++j) issue_one_aa(j, tl.kb0, 0, nst > 0, tl.kb0, 0, nst > 0);
#pragma unroll
                for (int j = IB + IT; j < INS_PER_WAVE; ++j)
                    issue_one_aa(j, tl.kb0 + min(1, nst - 1), 1, nst > 1, tl.kb0, 0, false);
            } else if constexpr (SPLIT) {
                // K blocks 0 .. STAGES-1 without the end group of the last (issued in the
                // first steps of block 0); placeholders past the tile keep the counts fixed
#pragma unroll
                for (int s = 0; s < STAGES; ++s) {
#pragma unroll
                    for (int j = 0; j < G_MID; ++j) issue_mid(j, tl.kb0 + min(s, nst - 1), s, s < nst);
                    if (s + 1 < STAGES) {
#pragma unroll
                        for (int j = 0; j < G_END; ++j) issue_end(j, tl.kb0 + min(s, nst - 1), s, s < nst);
                    }
                }
            } else {
#pragma unroll
                for (int s = 0; s < STAGES - 1; ++s)
                    if (s < nst) issue_stage(tl.kb0 + s * KSTEP, s);
            }

            // row offsets of this lane's fragments inside a stage
            const int a_row0 = wm * WAVE_M + l16;   // + a*16
            const int wave_n0 = tl.n0 + wn * WAVE_N;
            // LDS byte offset of each n sub-tile's sfb inside a K block's sfb slice
            int sb_off[TN];
#pragma unroll
            for (int b = 0; b < TN; ++b) {
                int nblk = (wave_n0 + b * 16) / KBLK;
                nblk = nblk < NBLKS ? nblk : NBLKS - 1;
                sb_off[b] = __builtin_amdgcn_readfirstlane((nblk - nb_t0) * 4);
            }

            if constexpr (KSTEP == 1) {
                // One K block per stage: the barrier sits in the last n sub-tile, where
                // the next K block's fragments are fetched while its MFMAs run.
                // LDS bases of one K block (stage slot, K block h inside the stage)
                const u32 b_frag = b_frag_off + b_chunk_lo, b_frag_hi = b_frag_off + chunk_hi;
                const u32 a_frag = a_frag_off + a_chunk_lo, a_frag_hi = a_frag_off + chunk_hi;
                // B fragment of the sub-tile at byte offset off of a K block (lo/hi:
                // the block's base plus this lane's chunk offsets)
                auto read_fb = [&](lds_u8* lo, lds_u8* hi, int off) __attribute__((always_inline)) {
                    if constexpr (FP4B) return lds_read_frag4(lo, off);
                    else return lds_read_frag(lo, hi, off);
                };
                auto read_fa = [&](lds_u8* lo, lds_u8* hi, int off) __attribute__((always_inline)) {
                    if constexpr (FP4A) return lds_read_frag4(lo, off);
                    else return lds_read_frag(lo, hi, off);
                };
                // FP4 B scales: this lane's row of each n sub-tile, one word per K block
                const int sb4_off = (wn * WAVE_N + l16) * 4;
                const u32 sh_q = 8u * (u32)q;    // lane group q takes byte q (its 32-wide K block)
                // LDS bases of the A tile, the B tile, the A scales and the B scales of a
                // slot (one K block per stage here; with A ahead A and B have rings of their own)
                auto a_tile = [&](int slot) __attribute__((always_inline)) {
                    return (lds_u8*)__builtin_amdgcn_readfirstlane(
                        smem_base + (AAHEAD ? slot * A_SLOT : slot * STAGE_BYTES + A_OFF));
                };
                auto b_tile = [&](int slot) __attribute__((always_inline)) {
                    return (lds_u8*)__builtin_amdgcn_readfirstlane(
                        smem_base + (AAHEAD ? B_RING + slot * B_SLOT : slot * STAGE_BYTES + B_OFF));
                };
                auto a_scales = [&](int slot) __attribute__((always_inline)) {
                    return (lds_u8*)__builtin_amdgcn_readfirstlane(
                        smem_base + (AAHEAD ? slot * A_SLOT + BM * ROWB_A : slot * STAGE_BYTES + S_OFF));
                };
                auto b_scales = [&](int slot) __attribute__((always_inline)) {
                    return (lds_u8*)__builtin_amdgcn_readfirstlane(
                        smem_base + (AAHEAD ? B_RING + slot * B_SLOT + BN * ROWB_B : slot * STAGE_BYTES + T_OFF));
                };
                // Registers of the K block being multiplied: its A fragments, its first
                // (then current) B fragment and the scales.  They are read from LDS one K
                // block ahead, during the last n sub-tile of the previous one.
                v8i fa[TM];
                v8i fb;
                float sa[TM];
                sc_t sb[TN];
                // K-grouped B scales: the lane's four columns of each n sub-tile
                const int sbk_off = (wn * WAVE_N + 4 * q) * 4;
                auto read_scales = [&](int slot_a, int slot_b) __attribute__((always_inline)) {
                    if constexpr (BF16) return;       // no scales
                    lds_u8* const sb_p = b_scales(slot_b);
                    if constexpr (FP4B) {
#pragma unroll
                        for (int b = 0; b < TN; ++b) sb[b] = lds_read_f32(sb_p, sb4_off + b * 64);
                    } else if constexpr (KG) {
#pragma unroll
                        for (int b = 0; b < TN; ++b)
                            sb[b] = *(__attribute__((address_space(3))) const sc_t*)(sb_p + sbk_off + b * 64);
                    } else if constexpr (SB_UNIFORM) {
                        sb[0] = lds_read_f32(sb_p, sb_off[0]);
                    } else {
#pragma unroll
                        for (int b = 0; b < TN; ++b) sb[b] = lds_read_f32(sb_p, sb_off[b]);
                    }
                    lds_u8* const sa_p = a_scales(slot_a) + a_row0 * 4;
#pragma unroll
                    for (int a = 0; a < TM; ++a) sa[a] = lds_read_f32(sa_p, a * 64);
                };

                // stage 0 in LDS (this wave's DMA, then everyone's), then its registers
                if constexpr (AAHEAD) wait_vmcnt<IA + IS>();     // all but A of K block 1
                else if constexpr (SPLIT) wait_vmcnt<SPLIT_PENDING>();   // the mid group of block 0
                else if (STAGES - 1 <= nst) wait_stages<STAGES - 2>();
                else wait_vmcnt<0>();
                __syncthreads();
                {
                    lds_u8* const ka0 = a_tile(0);
                    lds_u8* const kb0 = b_tile(0);
                    read_scales(0, 0);
#pragma unroll
                    for (int a = 0; a < TM; ++a) fa[a] = read_fa(ka0 + a_frag, ka0 + a_frag_hi, a * 16 * ROWB_A);
                    fb = read_fb(kb0 + b_frag, kb0 + b_frag_hi, 0);
                }

#pragma unroll 1
                for (int it = 0; it < nst; ++it) {
                    const int stage = it % STAGES;
                    // The slot of stage it-1 is free: every wave read all of it into
                    // registers before the barrier in the previous iteration.  Its refill
                    // (the stage STAGES-1 ahead) is spread over the first MFMA steps.  In
                    // the last STAGES-1 iterations the refill is a placeholder that moves
                    // no data, so the loop has no branch and the number of stages in
                    // flight is always the same.
                    const bool live = it + STAGES - 1 < nst;
                    const int kb_fill = tl.kb0 + min(it + STAGES - 1, nst - 1) * KSTEP;
                    const int slot_fill = (it + STAGES - 1) % STAGES;
                    // A ahead: A of K block it+2 into its A slot, B of it+1 into its B slot
                    const int a_fill_slot = (it + 2) % A_SLOTS;
                    const int a_fill_kb = tl.kb0 + min(it + 2, nst - 1);
                    const bool a_live = it + 2 < nst;
                    // the K block after the last one of this stage: first of the next stage
                    const int stage_next = (it + 1) % STAGES;
                    const int a_slot = AAHEAD ? it % A_SLOTS : stage;
                    const int a_slot_next = AAHEAD ? (it + 1) % A_SLOTS : stage_next;
#pragma unroll
                    for (int h = 0; h < KSTEP; ++h) {
                    lds_u8* const kbp = b_tile(stage);
                    lds_u8* const b_lo = kbp + b_frag;
                    lds_u8* const b_hi = kbp + b_frag_hi;
                    lds_u8* const kan = a_tile(a_slot_next);
                    lds_u8* const kbn = b_tile(stage_next);
                    (void)a_slot;

                    float sab[TM];           // sa * sb for the uniform case
                    if constexpr (SB_UNIFORM && !SF_E8) {
#pragma unroll
                        for (int a = 0; a < TM; ++a) sab[a] = sa[a] * first(sb[0]);
                    }
                    // UE8M0: this K block's scale bytes, shifted to bits 0-7 of each word
                    int ea[TM], eb[TN];
                    if constexpr (SF_E8) {
                        const u32 sh = 8u * (u32)((tl.kb0 + it) & (PAIRS ? 1 : 3));
#pragma unroll
                        for (int a = 0; a < TM; ++a) ea[a] = (int)(__builtin_bit_cast(u32, sa[a]) >> (FP4A ? sh_q : sh));
#pragma unroll
                        for (int b = 0; b < (SB_UNIFORM ? 1 : TN); ++b)
                            eb[b] = (int)(__builtin_bit_cast(u32, first(sb[b])) >> (FP4B ? sh_q : sh));
                    }

                    // Software pipeline over the n sub-tiles: the MFMAs of sub-tile b
                    // run while the FMAs promote sub-tile b-1 (for b = 0: the carried
                    // last sub-tile of the previous K block).
                    v4f pr[TM];
#pragma unroll
                    for (int b = 0; b < TN; ++b) {
                        if constexpr (SPLIT) {
                            // end group of block it + STAGES - 1 (into the slot block it - 1 used),
                            // then, after the mid barrier, the mid group of block it + STAGES
                            // (into this block's slot)
                            if (b < END_STEPS) {
                                const int f = it + STAGES - 1;
#pragma unroll
                                for (int j = b * G_END / END_STEPS; j < (b + 1) * G_END / END_STEPS; ++j)
                                    issue_end(j, tl.kb0 + min(f, nst - 1), f % STAGES, f < nst);
                            }
                            if (b + 1 == HALF_TN) {
                                wait_vmcnt<SPLIT_PENDING>();      // end group of this block landed
                                __syncthreads();
                            }
                            if (b + 1 >= HALF_TN && b + 1 < TN) {
                                const int f = it + STAGES, sb = b + 1 - HALF_TN;
#pragma unroll
                                for (int j = sb * G_MID / MID_STEPS; j < (sb + 1) * G_MID / MID_STEPS; ++j)
                                    issue_mid(j, tl.kb0 + min(f, nst - 1), stage, f < nst);
                            }
                        } else if (h == 0) {
                            if constexpr (AAHEAD) {
                                const int nspread = SPREAD == 0 ? 1 : SPREAD;
                                if (b < nspread) {
#pragma unroll
                                    for (int j = b * INS_PER_WAVE / nspread; j < (b + 1) * INS_PER_WAVE / nspread; ++j)
                                        issue_one_aa(j, a_fill_kb, a_fill_slot, a_live, kb_fill, slot_fill, live);
                                }
                            } else if constexpr (SPREAD == 0) {
                                if (b == 0) issue_stage(kb_fill, slot_fill, live);
                            } else if (b < SPREAD) {
#pragma unroll
                                for (int j = b * INS_PER_WAVE / SPREAD; j < (b + 1) * INS_PER_WAVE / SPREAD; ++j)
                                    issue_one(j, kb_fill, slot_fill, live);
                            }
                        }
                        const bool last = b + 1 == TN;
                        v8i fb_next;
                        if (!last) fb_next = read_fb(b_lo, b_hi, (b + 1) * 16 * ROWB_B);
                        // scales of sub-tile b-1 (promoted now) and, in the last sub-tile, of
                        // b itself (carried), taken before the next K block's replace them
                        sc_t sc_prev[TM], s_last[TM];
#pragma unroll
                        for (int a = 0; a < TM; ++a) {
                            if constexpr (SF_E8 || BF16) sc_prev[a] = s_last[a] = 0.f;
                            else if constexpr (SB_UNIFORM) sc_prev[a] = s_last[a] = sab[a];
                            else {
                                sc_prev[a] = sa[a] * sb[b > 0 ? b - 1 : 0];
                                if (b == 0) sc_prev[a] = 0.f;
                                s_last[a] = sa[a] * sb[b];
                            }
                        }
                        if (last) {
                            if (h + 1 == KSTEP) {
                                // next stage landed (own DMA; the later stages pending), then
                                // everyone's; all reads of this stage are in registers.  A ahead:
                                // everything but A of K block it+2 (issued last) has landed
                                if constexpr (AAHEAD) wait_vmcnt<IA + IS>();
                                else if constexpr (SPLIT) wait_vmcnt<SPLIT_PENDING>();   // next block's mid group
                                else wait_stages<STAGES - 2>();
                                __syncthreads();
                            }
                            read_scales(a_slot_next, stage_next);
                        }
                        v4f prev[TM];
#pragma unroll
                        for (int a = 0; a < TM; ++a) prev[a] = pr[a];
                        // optional: the wave asks for issue priority while it has MFMAs to issue
                        if constexpr (DG_SETPRIO != 0) __builtin_amdgcn_s_setprio(DG_SETPRIO);
#pragma unroll
                        for (int a = 0; a < TM; ++a) {
                            if constexpr (SF_E8) {
                                // acc += 2^(eb-127) 2^(ea-127) P: the MFMA applies both block
                                // scales (its srcA is B, scaled by eb; its srcB is A, by ea).
                                // operand formats: 0 = E4M3, 4 = E2M1 (srcA: B, srcB: A)
                                acc[a][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                    fb, fa[a], acc[a][b], FP4B ? 4 : 0, FP4A ? 4 : 0, 0, eb[SB_UNIFORM ? 0 : b], 0, ea[a]);
                            } else if constexpr (BF16) {
                                // 64 BF16 elements: K chunks q (elements 8q..8q+7) then q+4 (32+8q..)
                                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf_lo(fb), bf_lo(fa[a]), acc[a][b], 0, 0, 0);
                                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf_hi(fb), bf_hi(fa[a]), acc[a][b], 0, 0, 0);
                            } else {
                                const v4f zero = {0.f, 0.f, 0.f, 0.f};
                                // P[n][m] over this 128-wide K block: exact products, FP32 sums
                                pr[a] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb, fa[a], zero, 0, 0, 0, 0, 0, 0);
                                if (b == 0) acc[a][TN - 1] += p_carry[a] * s_carry[a];
                                else acc[a][b - 1] += prev[a] * sc_prev[a];
                            }
                            // the last sub-tile's MFMA has taken fa[a]: fetch the next K block's
                            // (after the tile's last block these reads are unused)
                            if (last) fa[a] = read_fa(kan + a_frag, kan + a_frag_hi, a * 16 * ROWB_A);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        if constexpr (DG_SETPRIO != 0) __builtin_amdgcn_s_setprio(0);
                        if (!last) {
                            fb = fb_next;
                        } else {
                            fb = read_fb(kbn + b_frag, kbn + b_frag_hi, 0);
#pragma unroll
                            for (int a = 0; a < TM; ++a) s_carry[a] = s_last[a];
                        }
                    }
#pragma unroll
                    for (int a = 0; a < TM; ++a) p_carry[a] = pr[a];
                    }   // K blocks of the stage
                }
                wait_vmcnt<0>();         // no DMA (placeholders included) outlives the tile
            } else {
                // Two K blocks per stage (short K loops): barrier at the top of each
                // stage, fragments read at the start of each K block.
#pragma unroll 1
                for (int it = 0; it < nst; ++it) {
                    const int stage = it % STAGES;
                    // stage `it` has landed (for this wave) once at most the later stages are pending
                    if (it + STAGES - 1 <= nst) wait_stages<STAGES - 2>();
                    else wait_vmcnt<0>();
                    __syncthreads();
                    // Refill the slot every wave finished reading last iteration.  With two
                    // slots the refill is needed by the next iteration, so it goes out
                    // at once; with three or more it is spread over this iteration's
                    // MFMA steps, so no wave stalls on a burst of vector-memory issue.
                    const bool refill = it + STAGES - 1 < nst;
                    const int kb_fill = tl.kb0 + (it + STAGES - 1) * KSTEP, slot_fill = (it + STAGES - 1) % STAGES;
                    if constexpr (STAGES == 2) {
                        if (refill) issue_stage(kb_fill, slot_fill);
                    }

                    const u32 st = __builtin_amdgcn_readfirstlane(smem_base + stage * STAGE_BYTES);
#pragma unroll
                    for (int h = 0; h < KSTEP; ++h) {
                    const int kb = tl.kb0 + it * KSTEP + h;
                    // scale of B from the stage (same address in every lane: a broadcast read)
                    lds_u8* const sb_p = (lds_u8*)(st + T_OFF + h * 256);
                    float sb[TN];
                    if constexpr (SB_UNIFORM) {
                        sb[0] = lds_read_f32(sb_p, sb_off[0]);
                    } else {
#pragma unroll
                        for (int b = 0; b < TN; ++b) sb[b] = lds_read_f32(sb_p, sb_off[b]);
                    }
                    lds_u8* const stp = (lds_u8*)(st + h * 128);
                    lds_u8* const sa_p = (lds_u8*)(st + h * S_BYTES) + a_row0 * 4;
                    lds_u8* const a_lo = stp + a_frag_off + chunk_lo;
                    lds_u8* const a_hi = stp + a_frag_off + chunk_hi;
                    lds_u8* const b_lo = stp + b_frag_off + chunk_lo;
                    lds_u8* const b_hi = stp + b_frag_off + chunk_hi;

                    float sa[TM];
#pragma unroll
                    for (int a = 0; a < TM; ++a) sa[a] = lds_read_f32(sa_p, S_OFF + a * 64);
                    v8i fa[TM];
#pragma unroll
                    for (int a = 0; a < TM; ++a) fa[a] = lds_read_frag(a_lo, a_hi, A_OFF + a * 16 * ROWB);
                    v8i fb = lds_read_frag(b_lo, b_hi, B_OFF);

                    float sab[TM];           // sa * sb for the uniform case
                    if constexpr (SB_UNIFORM && !SF_E8) {
#pragma unroll
                        for (int a = 0; a < TM; ++a) sab[a] = sa[a] * sb[0];
                    }
                    // UE8M0: this K block's scale bytes, shifted to bits 0-7 of each word
                    int ea[TM], eb[TN];
                    if constexpr (SF_E8) {
                        const u32 sh = 8u * (u32)((tl.kb0 + it) & (PAIRS ? 1 : 3));
#pragma unroll
                        for (int a = 0; a < TM; ++a) ea[a] = (int)(__builtin_bit_cast(u32, sa[a]) >> sh);
#pragma unroll
                        for (int b = 0; b < (SB_UNIFORM ? 1 : TN); ++b) eb[b] = (int)(__builtin_bit_cast(u32, sb[b]) >> sh);
                    }

                    // Software pipeline over the n sub-tiles: the MFMAs of sub-tile b
                    // run while the FMAs promote sub-tile b-1 (for b = 0: the carried
                    // last sub-tile of the previous K block).
                    v4f pr[TM];
#pragma unroll
                    for (int b = 0; b < TN; ++b) {
                        if constexpr (STAGES > 2) {
                            if (refill && h == 0) {
#pragma unroll
                                for (int j = b * INS_PER_WAVE / TN; j < (b + 1) * INS_PER_WAVE / TN; ++j)
                                    issue_one(j, kb_fill, slot_fill);
                            }
                        }
                        v8i fb_next;
                        if (b + 1 < TN) fb_next = lds_read_frag(b_lo, b_hi, B_OFF + (b + 1) * 16 * ROWB);
                        v4f prev[TM];
#pragma unroll
                        for (int a = 0; a < TM; ++a) prev[a] = pr[a];
#pragma unroll
                        for (int a = 0; a < TM; ++a) {
                            const v4f zero = {0.f, 0.f, 0.f, 0.f};
                            // P[n][m] over this 128-wide K block: exact products, FP32 sums
                            pr[a] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb, fa[a], zero, 0, 0, 0, 0, 0, 0);
                            if (b == 0) {
                                acc[a][TN - 1] += p_carry[a] * s_carry[a];
                            } else {
                                float sc;
                                if constexpr (SB_UNIFORM) sc = sab[a];
                                else sc = sa[a] * sb[b - 1];
                                acc[a][b - 1] += prev[a] * sc;
                            }
                        }
                        if (b + 1 < TN) fb = fb_next;
                    }
#pragma unroll
                    for (int a = 0; a < TM; ++a) {
                        p_carry[a] = pr[a];
                        if constexpr (SB_UNIFORM) s_carry[a] = sab[a];
                        else s_carry[a] = sa[a] * sb[TN - 1];
                    }
                    }   // K blocks of the stage
                }
            }
            if constexpr (!SF_E8 && !BF16) {
#pragma unroll
                for (int a = 0; a < TM; ++a) acc[a][TN - 1] += p_carry[a] * s_carry[a];
            }

            // (the row experts' DMA has landed: no DMA of this wave outlives the K loop)
            // The lane's row and column bases and its thread index are taken afresh from
            // the lane id here, so that no per-lane value has to live across the K loop
            // for the epilogue.
            const int ln = lane_id_now();
            finish_tile<TM, TN, ROW_GRP_LDS>(p, tl, acc, wm * WAVE_M + (ln & 15), wn * WAVE_N + 4 * (ln >> 4),
                                             wave * 64 + ln, smem_base + GRP_OFF + wave * 256 + (ln & 15) * 4);
        }   // pieces
    }
}

#elif DG_VARIANT == 1 || DG_VARIANT == 2
// ============================================================ variants 1 and 2: B straight into VGPRs
// For few rows (every row of a problem or group in one or two row blocks):
// each wave owns WAVE_N rows of B and loads them from global memory straight
// into VGPRs, DEPTH K blocks ahead of their use.  A wave's B rows are one
// contiguous stretch of memory that it requests within a short window, so HBM
// streams it well, and the bytes in flight per CU are bounded by the register
// file rather than by LDS.  The K range of a work item is unrolled completely,
// so every wait count is a compile-time constant.
//   variant 1: the A tile (read by every wave), its scales and the B scales
//              pass through an LDS ring, one K block per slot, one barrier per
//              K block;
//   variant 2: the A tile of the whole K range is loaded into LDS once per
//              work item (it must fit), so the K loop has no barrier at all
//              and the waves run independently.
constexpr bool ARES = DG_VARIANT == 2;
static_assert(!SF_E8 && !KG && !BF16, "UE8M0 scales, BF16 and the K-grouped form are built for variant 0");
static_assert(WM == 1, "variants 1 and 2 spread their waves along n only");
static_assert(KSTEP == 1, "variants 1 and 2 stage one K block at a time");
constexpr int NKB = KBLKS / SPLITK;               // K blocks of one work item
static_assert(NKB <= 64, "the whole K range of a work item is unrolled");
constexpr int DEPTH = STAGES - 1;                 // K blocks of B requested ahead of use
constexpr int NREG = ARES ? NKB : STAGES;         // K blocks held in LDS (variant 1: ring slots)
constexpr int NA_INS = BM / 8;                    // 1 KB DMA instructions for one K block of A
constexpr int NS_INS = (BM + 63) / 64;            // 256 B DMA instructions for its sfa
// LDS: [sfb][sfa: NREG x NS_INS x 256 B][A: NREG x BM rows x 128 B], where sfb
// is, in variant 1, one row of 64 floats per slot (one per 128-row block of B
// from the tile's first on) and, in variant 2, three rows of 64 floats (the
// tile's 128-row blocks j = 0..2 over the item's K blocks).  The scales come
// first so that their offsets fit a ds_read immediate.
constexpr int T_OFF = 0;
constexpr int S_OFF = T_OFF + (ARES ? 3 : NREG) * 256;
constexpr int A_OFF = S_OFF + NREG * NS_INS * 256;
constexpr int LDS_BYTES = A_OFF + NREG * BM * 128;
// A fragment reads address LDS from a few per-tile base registers 32 KB apart,
// so that every offset fits the 16-bit ds_read immediate
constexpr int A_BANK = 32768;
constexpr int NBANK = (LDS_BYTES + A_BANK - 1) / A_BANK;
static_assert(BM % 8 == 0, "A is loaded 8 rows per DMA instruction");
static_assert(BN <= 256, "a tile touches at most three 128-row blocks of B");
static_assert(LDS_BYTES <= 160 * 1024, "LDS exceeds 160 KB");
// Vector-memory instructions per wave.  Every wave issues the same count
// (repeating its category's last instruction where its share runs out), so
// one vmcnt immediate fits all waves.
constexpr int UB = 2 * TN;                        // B: two 16-byte loads per lane per 16-row sub-tile
// variant 1, per K block: share of the A and sfa DMA, one sfb DMA, the B loads
constexpr int IA = (NA_INS + NWAVES - 1) / NWAVES;
constexpr int IS = (NS_INS + NWAVES - 1) / NWAVES;
constexpr int UNIT = ARES ? UB : IA + IS + 1 + UB;
// variant 2, once per work item: the same A and sfa shares for every K block, and sfb
constexpr int IT_ALL = (3 + NWAVES - 1) / NWAVES;
constexpr int PRE_UNITS = DEPTH < NKB ? DEPTH : NKB;
static_assert(UNIT * (DEPTH - 1) <= 63 && (!ARES || UNIT * PRE_UNITS <= 63), "vmcnt range");
#ifndef DG_FA_AHEAD
#define DG_FA_AHEAD 4
#endif
constexpr int FA_AHEAD = DG_FA_AHEAD < TM ? DG_FA_AHEAD : TM;   // A fragments read ahead of use


extern "C" __global__ void __attribute__((amdgpu_flat_work_group_size(1, MAX_THREADS_DECL)))
dg_fp8_gemm_nt_kernel(const KernArgs ka) {
    const u8* __restrict__ A = (const u8*)ka.A;
    const float* __restrict__ sfa = (const float*)ka.sfa;
    const u8* __restrict__ B = (const u8*)ka.B;
    const float* __restrict__ sfb = (const float*)ka.sfb;
    const float* __restrict__ C = (const float*)ka.C;
    u16* __restrict__ D = (u16*)ka.D;
    const int* __restrict__ grp = (const int*)ka.grp;
    float* __restrict__ ws = (float*)ka.ws;
    u32* __restrict__ counters = (u32*)ka.counters;
    const int M = ka.M, num_tiles = ka.num_tiles, kt = ka.kt;
    u32* __restrict__ status = (u32*)ka.status;
    const Params p{A, sfa, B, sfb, C, D, grp, ws, counters, M, num_tiles, kt, status};
    // Every argument in one round trip of scalar loads: otherwise the loop bound
    // is fetched first and the pointers only after it arrives (~0.5 us each).
    asm volatile("" :: "s"(A), "s"(sfa), "s"(B), "s"(sfb), "s"(C), "s"(D), "s"(grp), "s"(ws), "s"(counters), "s"(M),
                 "s"(num_tiles), "s"(gridDim.x));
    __shared__ __attribute__((aligned(1024))) u8 smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int q = lane >> 4;
    const u32 smem_base = lds_addr(smem);
    // A fragments: the swizzled chunk pair {q, q ^ 4} of row l16 (+16 a), as in variant 0
    const int sw = l16 & 7;
    const u32 chunk_lo = (u32)((q ^ sw) << 4);
    const u32 chunk_hi = (u32)(((q ^ 4) ^ sw) << 4);
    const u32 a_frag_off = (u32)l16 * 128u;
    const int wave_n = wave * WAVE_N;             // first column of this wave inside the tile

#pragma unroll 1
    for (int t = blockIdx.x; t < p.num_tiles; t += gridDim.x) {
        const Tile tl = decode_tile(p, t);
        if (tl.skip) continue;

        const u8* a_base;
        const float* sfa_base;
        if constexpr (kKind == 2) {
            a_base = p.A + ((u64)tl.g * p.M + tl.m0) * K;
            sfa_base = p.sfa + (u64)tl.g * KBLKS * p.M;
        } else {
            a_base = p.A + (u64)tl.m0 * K;
            sfa_base = p.sfa;
        }
        const int n_rows = N_END - tl.n0 < BN ? N_END - tl.n0 : BN;
        const u8* b_base = p.B + ((u64)tl.g * N + tl.n0) * K;
        const v4i rs_b = make_rsrc(b_base, (u32)n_rows * K);
        const int nb_t0 = tl.n0 / KBLK;
        // B: sub-tile b, row l16 (clamped to the valid rows), logical chunks q and q + 4
        u32 bvoff[TN];
#pragma unroll
        for (int b = 0; b < TN; ++b) {
            const int r = wave_n + b * 16 + l16;
            bvoff[b] = (u32)(r < n_rows ? r : n_rows - 1) * K + q * 16;
        }
        auto issue_b = [&](int kb, v4i (&dst)[TN][2]) __attribute__((always_inline)) {
            const u32 ka = __builtin_amdgcn_readfirstlane((u32)kb * KBLK);
#pragma unroll
            for (int b = 0; b < TN; ++b) {
                dst[b][0] = load16<0>(rs_b, bvoff[b], ka);
                dst[b][1] = load16<64>(rs_b, bvoff[b], ka);
            }
        };
        const v4i rs_a = make_rsrc(a_base, (u32)tl.rows * K);
        const v4i rs_s = make_rsrc(sfa_base, (u32)KBLKS * p.M * 4u);
        const v4i rs_t = make_rsrc(p.sfb + (u64)tl.g * NBLKS * KBLKS, (u32)NBLKS * KBLKS * 4u);
        // A DMA: lane l of instruction i (8 tile rows) writes LDS bytes [16 l, 16 l + 16)
        // of its 1 KB = tile row 8 i + l / 8, physical chunk l % 8, which holds
        // logical chunk (l % 8) ^ (row & 7).
        // (the same offsets serve every K block: only the scalar offset moves)
        u32 voff_a[IA], voff_s[IS];
#pragma unroll
        for (int j = 0; j < IA; ++j) {
            const int i = min(wave + j * NWAVES, NA_INS - 1);
            const int r = i * 8 + lane / 8;
            const int c = (lane & 7) ^ (r & 7);
            const int rr = r < tl.rows ? r : tl.rows - 1;
            voff_a[j] = (u32)rr * K + c * 16;
        }
#pragma unroll
        for (int j = 0; j < IS; ++j) {
            const int i = min(wave + j * NWAVES, NS_INS - 1);
            const int m = tl.m0 + i * 64 + lane;
            voff_s[j] = (u32)(m < p.M ? m : p.M - 1) * 4u;
        }
        // this wave's share of one K block of A and sfa, into LDS region ri
        auto issue_a = [&](int kb, int ri) __attribute__((always_inline)) {
            const u32 st = __builtin_amdgcn_readfirstlane(smem_base);
            const u32 ka = __builtin_amdgcn_readfirstlane((u32)kb * KBLK);
#pragma unroll
            for (int j = 0; j < IA; ++j) {
                const int i = min(wave + j * NWAVES, NA_INS - 1);
                dma16(rs_a, voff_a[j], ka, st + A_OFF + ri * (BM * 128) + i * 1024);
            }
#pragma unroll
            for (int j = 0; j < IS; ++j) {
                const int i = min(wave + j * NWAVES, NS_INS - 1);
                dma4(rs_s, voff_s[j], __builtin_amdgcn_readfirstlane((u32)kb * p.M * 4u),
                     st + S_OFF + (ri * NS_INS + i) * 256);
            }
        };
        // variant 1: one K block of A, sfa and sfb into ring slot `slot`
        auto issue_ring = [&](int kb, int slot) __attribute__((always_inline)) {
            issue_a(kb, slot);
            dma4(rs_t, (u32)min(nb_t0 + lane, NBLKS - 1) * KBLKS * 4u, __builtin_amdgcn_readfirstlane((u32)kb * 4u),
                 __builtin_amdgcn_readfirstlane(smem_base) + T_OFF + slot * 256);
        };
        // LDS read pointers, fixed per tile; every K block adds a compile-time
        // offset (which the compiler folds into the ds_read immediates instead
        // of keeping one address register per K block alive).  sb_p[b]: the
        // sub-tile's sfb, variant 1 inside a slot's sfb row (one float per
        // 128-row block), variant 2 the row of its block.
        lds_u8* const lds = (lds_u8*)smem_base;
        lds_u8* sb_p[TN];
#pragma unroll
        for (int b = 0; b < TN; ++b) {
            int nblk = (tl.n0 + wave_n + b * 16) / KBLK;
            nblk = nblk < NBLKS ? nblk : NBLKS - 1;
            sb_p[b] = lds + T_OFF + (nblk - nb_t0) * (ARES ? 256 : 4);
        }
        lds_u8* const sa_p0 = lds + S_OFF + l16 * 4;
        lds_u8* a_lo_bank[NBANK];
        lds_u8* a_hi_bank[NBANK];
#pragma unroll
        for (int k = 0; k < NBANK; ++k) {
            a_lo_bank[k] = lds + k * A_BANK + a_frag_off + chunk_lo;
            a_hi_bank[k] = lds + k * A_BANK + a_frag_off + chunk_hi;
            // opaque, so the compiler keeps these registers instead of re-deriving
            // one address register per K block from the first
            asm volatile("" : "+v"(a_lo_bank[k]), "+v"(a_hi_bank[k]));
        }

        v4f acc[TM][TN];
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int b = 0; b < TN; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
        // the last product of a K block and its scale, promoted under the next block's first MFMA
        v4f p_carry = {0.f, 0.f, 0.f, 0.f};
        float s_carry = 0.f;
        v4i breg[NKB][TN][2];

        // Every wave has finished reading LDS (the earlier tile's) before it is
        // refilled.  The earlier tile's stores may still be in flight: the waits
        // below count only loads issued after the ones they wait for, which
        // complete in order, so a pending store only delays a wait.
        __syncthreads();

        if constexpr (ARES) {
            // the whole K range of A, sfa and sfb, then the first DEPTH K blocks of B
            const u32 st = __builtin_amdgcn_readfirstlane(smem_base);
            static_for<NKB>([&]<int KB>() __attribute__((always_inline)) { issue_a(tl.kb0 + KB, KB); });
#pragma unroll
            for (int j = 0; j < IT_ALL; ++j) {
                const int jb = min(wave + j * NWAVES, 2);
                const int nb = min(nb_t0 + jb, NBLKS - 1);
                const int kb = min(tl.kb0 + lane, KBLKS - 1);
                dma4(rs_t, (u32)(nb * KBLKS + kb) * 4u, 0u, st + T_OFF + jb * 256);
            }
            static_for<PRE_UNITS>([&]<int J>() __attribute__((always_inline)) { issue_b(tl.kb0 + J, breg[J]); });
            // this wave's A share has landed once only the B loads may be pending
            wait_vmcnt<PRE_UNITS * UB>();
            __syncthreads();
        } else {
            static_for<PRE_UNITS>([&]<int J>() __attribute__((always_inline)) {
                issue_ring(tl.kb0 + J, J % NREG);
                issue_b(tl.kb0 + J, breg[J]);
            });
        }

        static_for<NKB>([&]<int IT>() __attribute__((always_inline)) {
            // this wave's loads of K block IT have landed once only the later
            // requested blocks (up to IT + DEPTH - 1) may still be in flight
            constexpr int last = IT + DEPTH - 1 < NKB - 1 ? IT + DEPTH - 1 : NKB - 1;
            wait_vmcnt<(last - IT) * UNIT>();
#pragma unroll
            for (int b = 0; b < TN; ++b) {
                tie(breg[IT][b][0]);
                tie(breg[IT][b][1]);
            }
            // byte offsets of this K block's A, sfa and sfb from the per-tile pointers
            constexpr int ri = ARES ? IT : IT % NREG;          // LDS region of this K block
            constexpr int a_off = A_OFF + ri * (BM * 128);
            constexpr int sa_off = ri * (NS_INS * 256);
            constexpr int sb_off = ARES ? IT * 4 : ri * 256;
            if constexpr (ARES) {
                if constexpr (IT + DEPTH < NKB) issue_b(tl.kb0 + IT + DEPTH, breg[IT + DEPTH]);
            } else {
                // every wave's share of A has landed, and every wave is done with slot IT - 1
                __syncthreads();
                if constexpr (IT + DEPTH < NKB) {
                    issue_ring(tl.kb0 + IT + DEPTH, (IT + DEPTH) % NREG);
                    issue_b(tl.kb0 + IT + DEPTH, breg[IT + DEPTH]);
                }
            }

            float sb[TN];
#pragma unroll
            for (int b = 0; b < TN; ++b) sb[b] = lds_read_f32(sb_p[b], sb_off);
            float sa[TM];
#pragma unroll
            for (int a = 0; a < TM; ++a) sa[a] = lds_read_f32(sa_p0, sa_off + a * 64);
            lds_u8* const a_lo = a_lo_bank[a_off / A_BANK] + a_off % A_BANK;
            lds_u8* const a_hi = a_hi_bank[a_off / A_BANK] + a_off % A_BANK;
            v8i fb[TN];
#pragma unroll
            for (int b = 0; b < TN; ++b) {
                const v4i x = breg[IT][b][0], y = breg[IT][b][1];
                fb[b] = v8i{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
            }
            // A fragments are read FA_AHEAD sub-tiles ahead of their MFMA, so the
            // LDS latency hides behind the MFMAs in between.  Software pipeline
            // over the (a, b) sub-tiles: each MFMA runs while the FMAs promote
            // the previous sub-tile's product.
            v8i fa[TM];
#pragma unroll
            for (int a = 0; a < FA_AHEAD; ++a) fa[a] = lds_read_frag(a_lo, a_hi, a * 16 * 128);
            v4f prev = p_carry;
            float sprev = s_carry;
#pragma unroll
            for (int a = 0; a < TM; ++a) {
                if (a + FA_AHEAD < TM) fa[a + FA_AHEAD] = lds_read_frag(a_lo, a_hi, (a + FA_AHEAD) * 16 * 128);
#pragma unroll
                for (int b = 0; b < TN; ++b) {
                    const v4f zero = {0.f, 0.f, 0.f, 0.f};
                    // P[n][m] over this 128-wide K block: exact products, FP32 sums
                    const v4f pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[b], fa[a], zero, 0, 0, 0, 0, 0, 0);
                    if (a == 0 && b == 0) acc[TM - 1][TN - 1] += prev * sprev;
                    else if (b == 0) acc[a - 1][TN - 1] += prev * sprev;
                    else acc[a][b - 1] += prev * sprev;
                    prev = pr;
                    sprev = sa[a] * sb[b];
                }
                // keep the read-ahead: the scheduler would otherwise sink each
                // fragment read down to its MFMA
                __builtin_amdgcn_sched_barrier(0);
            }
            p_carry = prev;
            s_carry = sprev;
            // Pin the accumulators at the end of every block: with the K range
            // unrolled, the compiler would otherwise sink all promotion FMAs into
            // the epilogue (their only use) and keep every product alive until then.
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int b = 0; b < TN; ++b) asm volatile("" : "+v"(acc[a][b]));
        });
        acc[TM - 1][TN - 1] += p_carry * s_carry;

        finish_tile<TM, TN>(p, tl, acc, l16, wave_n + 4 * q, tid);
    }
}
#elif DG_VARIANT == 3
// ============================================================ variant 3: a producer wave for A
// For few rows, like variant 1, but without any workgroup barrier in the K
// loop.  One extra wave (the last) only loads A and its scales into an LDS
// ring and publishes each K block with an LDS flag; the NWAVES other waves
// each stream their own rows of B straight into VGPRs (DEPTH K blocks ahead),
// wait on the flag of the K block they need rather than on the slowest wave,
// and count themselves off each slot when done with it.  The producer
// refills a slot only once every consumer has counted off, and publishes a
// block LAG blocks after issuing it (LAG < SLOTS, so the slot it waits for
// always holds a published block: no wait can be circular).  Every wait on a
// flag is also bounded, so a fault in this protocol would cost correctness,
// which the tests check, and never hang the device.
static_assert(WM == 1, "variant 3 spreads its consumer waves along n only");
static_assert(!SF_E8 && !KG && !BF16, "UE8M0 scales, BF16 and the K-grouped form are built for variant 0");
static_assert(KSTEP == 1, "variant 3 stages one K block per slot");
constexpr int NKB = KBLKS / SPLITK;               // K blocks of one work item
static_assert(NKB <= 64, "the whole K range of a work item is unrolled");
constexpr int DEPTH = STAGES - 1;                 // K blocks of B requested ahead of use
constexpr int UB = 2 * TN;                        // B loads per lane per K block
constexpr int PRE_UNITS = DEPTH < NKB ? DEPTH : NKB;
static_assert(DEPTH >= 1 && UB * PRE_UNITS <= 63, "vmcnt range");
constexpr int NA_INS = BM / 8;                    // 1 KB DMA instructions for one K block of A
constexpr int NS_INS = (BM + 63) / 64;            // 256 B DMA instructions for its sfa
static_assert(BM % 8 == 0, "A is loaded 8 rows per DMA instruction");
static_assert(BN <= 256, "a tile touches at most three 128-row blocks of B");
// LDS: [sfb: rows j = 0..2 (the tile's 128-row blocks of B) x 64 K blocks]
//      [sfa: SLOTS x NS_INS x 256 B][A: SLOTS x BM rows x 128 B]
constexpr int T_OFF = 0;
constexpr int S_OFF = 3 * 256;
constexpr int SLOT_A = BM * 128;
constexpr int SLOT_S = NS_INS * 256;
constexpr int SLOTS_FIT = (160 * 1024 - 1024 - S_OFF) / (SLOT_A + SLOT_S);
constexpr int SLOTS = SLOTS_FIT < 16 ? SLOTS_FIT : 16;
constexpr int A_OFF = S_OFF + SLOTS * SLOT_S;
constexpr int LDS_BYTES = A_OFF + SLOTS * SLOT_A;
constexpr int PU = NA_INS + NS_INS;               // producer DMA instructions per K block
constexpr int LAG = (SLOTS - 1) < (63 / PU) ? (SLOTS - 1) : (63 / PU);
static_assert(SLOTS >= 2 && LAG >= 1, "ring too small");
constexpr int V3_THREADS = NTHREADS + 64;
constexpr int V3_MAX_DECL = V3_THREADS < 512 ? 512 : V3_THREADS;
#ifndef DG_SPIN_LIMIT
#define DG_SPIN_LIMIT (1 << 20)
#endif
constexpr int SPIN_LIMIT = DG_SPIN_LIMIT;         // about 30 ms of s_sleep 1 before giving up
constexpr int A_BANK = 32768;
constexpr int NBANK = (LDS_BYTES + A_BANK - 1) / A_BANK;
#ifndef DG_FA_AHEAD
#define DG_FA_AHEAD 4
#endif
constexpr int FA_AHEAD = DG_FA_AHEAD < TM ? DG_FA_AHEAD : TM;

// Bounded wait until *flag >= target (an LDS word written by another wave).
// A wait that runs out is counted in the library's status word (one vector
// atomic from the wave's first lane), so the host can tell that this call's D
// is not to be trusted; the wave then goes on, so the grid always drains.
__device__ __forceinline__ void wait_flag(u32* flag, u32 target, u32* status) {
    bool landed = false;
    for (int i = 0; i < SPIN_LIMIT; ++i) {
        const u32 v = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (v >= target) {
            landed = true;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    if (!landed && (threadIdx.x & 63) == 0)
        __hip_atomic_fetch_add(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::: "memory");   // later LDS reads stay after the wait
}

extern "C" __global__ void __attribute__((amdgpu_flat_work_group_size(1, V3_MAX_DECL)))
dg_fp8_gemm_nt_kernel(const KernArgs ka) {
    const u8* __restrict__ A = (const u8*)ka.A;
    const float* __restrict__ sfa = (const float*)ka.sfa;
    const u8* __restrict__ B = (const u8*)ka.B;
    const float* __restrict__ sfb = (const float*)ka.sfb;
    const float* __restrict__ C = (const float*)ka.C;
    u16* __restrict__ D = (u16*)ka.D;
    const int* __restrict__ grp = (const int*)ka.grp;
    float* __restrict__ ws = (float*)ka.ws;
    u32* __restrict__ counters = (u32*)ka.counters;
    const int M = ka.M, num_tiles = ka.num_tiles, kt = ka.kt;
    u32* __restrict__ status = (u32*)ka.status;
    const Params p{A, sfa, B, sfb, C, D, grp, ws, counters, M, num_tiles, kt, status};
    // Every argument in one round trip of scalar loads: otherwise the loop bound
    // is fetched first and the pointers only after it arrives (~0.5 us each).
    asm volatile("" :: "s"(A), "s"(sfa), "s"(B), "s"(sfb), "s"(C), "s"(D), "s"(grp), "s"(ws), "s"(counters), "s"(M),
                 "s"(num_tiles), "s"(gridDim.x));
    __shared__ __attribute__((aligned(1024))) u8 smem[LDS_BYTES];
    __shared__ u32 ready[SLOTS];     // K block index + 1 held by the slot, once landed
    __shared__ u32 freed[SLOTS];     // consumer waves done with the slot's current block

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool producer = wave == NWAVES;
    const int l16 = lane & 15;
    const int q = lane >> 4;
    const u32 smem_base = lds_addr(smem);
    const int sw = l16 & 7;
    const u32 chunk_lo = (u32)((q ^ sw) << 4);
    const u32 chunk_hi = (u32)(((q ^ 4) ^ sw) << 4);
    const u32 a_frag_off = (u32)l16 * 128u;
    const int wave_n = wave * WAVE_N;

#pragma unroll 1
    for (int t = blockIdx.x; t < p.num_tiles; t += gridDim.x) {
        const Tile tl = decode_tile(p, t);
        if (tl.skip) continue;
        // every wave is done with the previous tile: reset the ring's flags
        __syncthreads();
        if (tid < SLOTS) {
            ready[tid] = 0u;
            freed[tid] = 0u;
        }
        __syncthreads();

        const u8* a_base;
        const float* sfa_base;
        if constexpr (kKind == 2) {
            a_base = p.A + ((u64)tl.g * p.M + tl.m0) * K;
            sfa_base = p.sfa + (u64)tl.g * KBLKS * p.M;
        } else {
            a_base = p.A + (u64)tl.m0 * K;
            sfa_base = p.sfa;
        }
        const int n_rows = N_END - tl.n0 < BN ? N_END - tl.n0 : BN;
        const int nb_t0 = tl.n0 / KBLK;

        if (producer) {
            const v4i rs_a = make_rsrc(a_base, (u32)tl.rows * K);
            const v4i rs_s = make_rsrc(sfa_base, (u32)KBLKS * p.M * 4u);
            const v4i rs_t = make_rsrc(p.sfb + (u64)tl.g * NBLKS * KBLKS, (u32)NBLKS * KBLKS * 4u);
            const u32 st = __builtin_amdgcn_readfirstlane(smem_base);
            // sfb of the tile's 128-row blocks over all K blocks (published with block 0)
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const int nb = min(nb_t0 + j, NBLKS - 1);
                const int kb = min(tl.kb0 + lane, KBLKS - 1);
                dma4(rs_t, (u32)(nb * KBLKS + kb) * 4u, 0u, st + T_OFF + j * 256);
            }
            // A DMA: lane l of instruction i (8 tile rows) writes LDS bytes [16 l, 16 l + 16)
            // of its 1 KB = tile row 8 i + l / 8, physical chunk l % 8, which holds
            // logical chunk (l % 8) ^ (row & 7).
            u32 voff_a[NA_INS], voff_s[NS_INS];
#pragma unroll
            for (int i = 0; i < NA_INS; ++i) {
                const int r = i * 8 + lane / 8;
                const int c = (lane & 7) ^ (r & 7);
                voff_a[i] = (u32)(r < tl.rows ? r : tl.rows - 1) * K + c * 16;
            }
#pragma unroll
            for (int i = 0; i < NS_INS; ++i) {
                const int m = tl.m0 + i * 64 + lane;
                voff_s[i] = (u32)(m < p.M ? m : p.M - 1) * 4u;
            }
            auto publish = [&](int kb) __attribute__((always_inline)) {
                if (lane == 0)
                    __hip_atomic_store(&ready[kb % SLOTS], (u32)(kb + 1), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            };
            static_for<NKB>([&]<int KB>() __attribute__((always_inline)) {
                constexpr int slot = KB % SLOTS;
                // the slot's previous block (KB - SLOTS) has been read by every consumer
                if constexpr (KB >= SLOTS) wait_flag(&freed[slot], (u32)(NWAVES * (KB / SLOTS)), p.status);
                const u32 ka = __builtin_amdgcn_readfirstlane((u32)(tl.kb0 + KB) * KBLK);
#pragma unroll
                for (int i = 0; i < NA_INS; ++i) dma16(rs_a, voff_a[i], ka, st + A_OFF + slot * SLOT_A + i * 1024);
#pragma unroll
                for (int i = 0; i < NS_INS; ++i)
                    dma4(rs_s, voff_s[i], __builtin_amdgcn_readfirstlane((u32)(tl.kb0 + KB) * p.M * 4u),
                         st + S_OFF + slot * SLOT_S + i * 256);
                // block KB - LAG has landed once only the LAG newer blocks may be in flight
                if constexpr (KB >= LAG) {
                    wait_vmcnt<LAG * PU>();
                    publish(KB - LAG);
                }
            });
            static_for<(LAG < NKB ? LAG : NKB)>([&]<int J>() __attribute__((always_inline)) {
                constexpr int kb = NKB - (LAG < NKB ? LAG : NKB) + J;   // the unpublished tail, oldest first
                wait_vmcnt<(NKB - 1 - kb) * PU>();
                publish(kb);
            });
            continue;
        }

        // ---------------------------------------------------------- consumer waves
        const u8* b_base = p.B + ((u64)tl.g * N + tl.n0) * K;
        const v4i rs_b = make_rsrc(b_base, (u32)n_rows * K);
        u32 bvoff[TN];
#pragma unroll
        for (int b = 0; b < TN; ++b) {
            const int r = wave_n + b * 16 + l16;
            bvoff[b] = (u32)(r < n_rows ? r : n_rows - 1) * K + q * 16;
        }
        auto issue_b = [&](int kb, v4i (&dst)[TN][2]) __attribute__((always_inline)) {
            const u32 ka = __builtin_amdgcn_readfirstlane((u32)kb * KBLK);
#pragma unroll
            for (int b = 0; b < TN; ++b) {
                dst[b][0] = load16<0>(rs_b, bvoff[b], ka);
                dst[b][1] = load16<64>(rs_b, bvoff[b], ka);
            }
        };
        lds_u8* const lds = (lds_u8*)smem_base;
        lds_u8* sb_p[TN];
#pragma unroll
        for (int b = 0; b < TN; ++b) {
            int nblk = (tl.n0 + wave_n + b * 16) / KBLK;
            nblk = nblk < NBLKS ? nblk : NBLKS - 1;
            sb_p[b] = lds + T_OFF + (nblk - nb_t0) * 256;
        }
        lds_u8* const sa_p0 = lds + S_OFF + l16 * 4;
        lds_u8* a_lo_bank[NBANK];
        lds_u8* a_hi_bank[NBANK];
#pragma unroll
        for (int k = 0; k < NBANK; ++k) {
            a_lo_bank[k] = lds + k * A_BANK + a_frag_off + chunk_lo;
            a_hi_bank[k] = lds + k * A_BANK + a_frag_off + chunk_hi;
            asm volatile("" : "+v"(a_lo_bank[k]), "+v"(a_hi_bank[k]));
        }

        v4f acc[TM][TN];
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int b = 0; b < TN; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
        v4f p_carry = {0.f, 0.f, 0.f, 0.f};
        float s_carry = 0.f;
        v4i breg[NKB][TN][2];

        // (no load of the earlier tile is in flight, only its stores, which the
        // waits below may wait for but never count as loads that landed)
        static_for<PRE_UNITS>([&]<int J>() __attribute__((always_inline)) { issue_b(tl.kb0 + J, breg[J]); });

        static_for<NKB>([&]<int IT>() __attribute__((always_inline)) {
            constexpr int last = IT + DEPTH - 1 < NKB - 1 ? IT + DEPTH - 1 : NKB - 1;
            wait_vmcnt<(last - IT) * UB>();
#pragma unroll
            for (int b = 0; b < TN; ++b) {
                tie(breg[IT][b][0]);
                tie(breg[IT][b][1]);
            }
            constexpr int slot = IT % SLOTS;
            wait_flag(&ready[slot], (u32)(IT + 1), p.status);
            if constexpr (IT + DEPTH < NKB) issue_b(tl.kb0 + IT + DEPTH, breg[IT + DEPTH]);

            constexpr int a_off = A_OFF + slot * SLOT_A;
            float sb[TN];
#pragma unroll
            for (int b = 0; b < TN; ++b) sb[b] = lds_read_f32(sb_p[b], IT * 4);
            float sa[TM];
#pragma unroll
            for (int a = 0; a < TM; ++a) sa[a] = lds_read_f32(sa_p0, slot * SLOT_S + a * 64);
            lds_u8* const a_lo = a_lo_bank[a_off / A_BANK] + a_off % A_BANK;
            lds_u8* const a_hi = a_hi_bank[a_off / A_BANK] + a_off % A_BANK;
            v8i fb[TN];
#pragma unroll
            for (int b = 0; b < TN; ++b) {
                const v4i x = breg[IT][b][0], y = breg[IT][b][1];
                fb[b] = v8i{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
            }
            v8i fa[TM];
#pragma unroll
            for (int a = 0; a < FA_AHEAD; ++a) fa[a] = lds_read_frag(a_lo, a_hi, a * 16 * 128);
            v4f prev = p_carry;
            float sprev = s_carry;
#pragma unroll
            for (int a = 0; a < TM; ++a) {
                if (a + FA_AHEAD < TM) fa[a + FA_AHEAD] = lds_read_frag(a_lo, a_hi, (a + FA_AHEAD) * 16 * 128);
#pragma unroll
                for (int b = 0; b < TN; ++b) {
                    const v4f zero = {0.f, 0.f, 0.f, 0.f};
                    // P[n][m] over this 128-wide K block: exact products, FP32 sums
                    const v4f pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[b], fa[a], zero, 0, 0, 0, 0, 0, 0);
                    if (a == 0 && b == 0) acc[TM - 1][TN - 1] += prev * sprev;
                    else if (b == 0) acc[a - 1][TN - 1] += prev * sprev;
                    else acc[a][b - 1] += prev * sprev;
                    prev = pr;
                    sprev = sa[a] * sb[b];
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            p_carry = prev;
            s_carry = sprev;
            // this wave has read everything of the slot it needs: count off
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (lane == 0) __hip_atomic_fetch_add(&freed[slot], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int b = 0; b < TN; ++b) asm volatile("" : "+v"(acc[a][b]));
        });
        acc[TM - 1][TN - 1] += p_carry * s_carry;

        finish_tile<TM, TN>(p, tl, acc, l16, wave_n + 4 * q, tid);
    }
}
#elif DG_VARIANT == 5
// ============================================================ variant 5: B in VGPRs, A through a deep ring (large tiles)
// For the large, MFMA-bound shapes.  With both operands staged through LDS a
// 256 x 256 tile leaves room for two stages only, so each K block's loads are
// requested about one K block ahead, less than the fabric latency under load.
// Here every wave owns WAVE_N = BN / NWAVES columns (no two waves share a row of
// B) and loads its B fragments straight into VGPRs, DEPTH K blocks ahead of
// their use; only A (shared by all waves) and the scales pass through LDS, in
// a ring of STAGES slots, so A is requested STAGES - 1 K blocks ahead.  Per K
// block each wave issues the same vector-memory instructions: its share of
// the A DMA, one scale DMA (the A scales of 64 rows, or the B scales), and
// its B loads; waiting for its own B loads of a block therefore also waits for
// its A share of that block (issued earlier), and one barrier per K block makes
// the A slot visible to all and frees the slot the previous block used.
static_assert(WM == 1, "variant 5 spreads its waves along n only");
static_assert(!SF_E8 && !KG && !BF16, "variant 5: FP32 scales");
static_assert(KSTEP == 1 && SPLITK == 1, "variant 5: one K block a slot, no split-K");
#ifndef DG_BDEPTH
#define DG_BDEPTH 2
#endif
constexpr int DEPTH = DG_BDEPTH;                  // K blocks of B in flight ahead of the one multiplied
constexpr int NSETS = DEPTH + 1;                  // B register sets; the K loop is unrolled by this
constexpr int SLOTS = STAGES;                     // A ring slots
static_assert(DEPTH >= 1 && SLOTS - 1 >= DEPTH, "A is requested at least as far ahead as B");
constexpr int NA_INS = BM / 8;                    // 1 KB DMA instructions for one K block of A
constexpr int NS_INS = BM / 64;                   // 256 B DMA instructions for its A scales
static_assert(BM % 64 == 0 && NA_INS % NWAVES == 0, "whole A DMA instructions per wave");
static_assert(NS_INS + 1 <= NWAVES, "one scale DMA per wave and K block");
constexpr int IA = NA_INS / NWAVES;
constexpr int UB = 2 * TN;                        // B loads per lane per K block
constexpr int UNIT = IA + 1 + UB;                 // vector-memory instructions per wave per K block
static_assert(UNIT * DEPTH <= 63, "vmcnt range");
static_assert(BN <= 256 && (KBLK % WAVE_N) == 0, "a wave's columns lie in one 128-row block of B");
// LDS slot: [A: BM rows x 128 B][A scales: BM floats][B scales: 64 floats].  The
// A scales are stored so that lane (l16, *) finds those of its rows l16 + 16 a,
// a = 0 .. TM-1, in TM consecutive floats: float i of the slot's scale area
// holds row (i % TM) * 16 + i / TM.
constexpr int S_OFF = BM * 128;
constexpr int T_OFF = S_OFF + BM * 4;
constexpr int SLOT_BYTES = T_OFF + 256;
constexpr int LDS_BYTES = SLOTS * SLOT_BYTES;
static_assert(LDS_BYTES <= 160 * 1024, "LDS exceeds 160 KB");
static_assert(TM % 4 == 0, "A scales are read four at a time");
#ifndef DG_FA_AHEAD
#define DG_FA_AHEAD 1
#endif
constexpr int FA_AHEAD = DG_FA_AHEAD < TM ? DG_FA_AHEAD : TM;   // A fragments read ahead of use

extern "C" __global__ void __attribute__((amdgpu_flat_work_group_size(1, MAX_THREADS_DECL)))
dg_fp8_gemm_nt_kernel(const KernArgs ka) {
    const u8* __restrict__ A = (const u8*)ka.A;
    const float* __restrict__ sfa = (const float*)ka.sfa;
    const u8* __restrict__ B = (const u8*)ka.B;
    const float* __restrict__ sfb = (const float*)ka.sfb;
    const float* __restrict__ C = (const float*)ka.C;
    u16* __restrict__ D = (u16*)ka.D;
    const int* __restrict__ grp = (const int*)ka.grp;
    float* __restrict__ ws = (float*)ka.ws;
    u32* __restrict__ counters = (u32*)ka.counters;
    const int M = ka.M, num_tiles = ka.num_tiles, kt = ka.kt;
    u32* __restrict__ status = (u32*)ka.status;
    const Params p{A, sfa, B, sfb, C, D, grp, ws, counters, M, num_tiles, kt, status};
    asm volatile("" :: "s"(A), "s"(sfa), "s"(B), "s"(sfb), "s"(C), "s"(D), "s"(grp), "s"(M), "s"(num_tiles),
                 "s"(gridDim.x));
    __shared__ __attribute__((aligned(1024))) u8 smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int q = lane >> 4;
    const u32 smem_base = lds_addr(smem);
    // A fragments: the swizzled chunk pair {q, q ^ 4} of row l16 (+16 a), as in variant 0
    const int sw = l16 & 7;
    const u32 chunk_lo = (u32)((q ^ sw) << 4);
    const u32 chunk_hi = (u32)(((q ^ 4) ^ sw) << 4);
    const int wave_n = wave * WAVE_N;             // first column of this wave inside the tile

#pragma unroll 1
    for (int t = blockIdx.x; t < p.num_tiles; t += gridDim.x) {
        const Tile tl = decode_tile(p, t);
        if (tl.skip) continue;

        const u8* a_base;
        const float* sfa_base;
        if constexpr (kKind == 2) {
            a_base = p.A + ((u64)tl.g * p.M + tl.m0) * K;
            sfa_base = p.sfa + (u64)tl.g * KBLKS * p.M;
        } else {
            a_base = p.A + (u64)tl.m0 * K;
            sfa_base = p.sfa;
        }
        const int n_rows = N_END - tl.n0 < BN ? N_END - tl.n0 : BN;
        const int nb_t0 = tl.n0 / KBLK;
        // A rows past the tile's valid rows lie past the buffer: they load as zeros
        const v4i rs_a = make_rsrc(a_base, (u32)tl.rows * K);
        const v4i rs_s = make_rsrc(sfa_base, (u32)KBLKS * p.M * 4u);
        const v4i rs_t = make_rsrc(p.sfb + (u64)tl.g * NBLKS * KBLKS, (u32)NBLKS * KBLKS * 4u);
        const v4i rs_b = make_rsrc(p.B + ((u64)tl.g * N + tl.n0) * K, (u32)n_rows * K);
        // this wave's share of the A DMA: instruction i = wave + j * NWAVES writes tile rows
        // 8 i .. 8 i + 7; lane l: row 8 i + l / 8, physical chunk l % 8 holding logical
        // chunk (l % 8) ^ (row & 7) (8 i is a multiple of 8, so the lane part is fixed)
        const u32 voff_a = (u32)(lane >> 3) * K + (u32)(((lane & 7) ^ ((lane >> 3) & 7)) << 4);
        // the wave's scale DMA: waves 0 .. NS_INS-1 the A scales of 64 rows each (in the
        // slot order above), the others the B scales of the tile's 128-row blocks
        u32 voff_sc;
        if (wave < NS_INS) {
            const int i = wave * 64 + lane;
            const int m = tl.m0 + (i % TM) * 16 + i / TM;
            voff_sc = (u32)(m < p.M ? m : p.M - 1) * 4u;
        } else {
            voff_sc = (u32)min(nb_t0 + lane, NBLKS - 1) * KBLKS * 4u;
        }
        // B: sub-tile b, row l16 (clamped to the valid rows), logical chunks q and q + 4
        u32 bvoff[TN];
#pragma unroll
        for (int b = 0; b < TN; ++b) {
            const int r = wave_n + b * 16 + l16;
            bvoff[b] = (u32)(r < n_rows ? r : n_rows - 1) * K + q * 16;
        }
        // K blocks of this tile, opaque to the compiler: with a short constant count it
        // would unroll the K loop and run out of registers
        int nst = tl.kb1 - tl.kb0;
        asm volatile("" : "+s"(nst));
        // K block `it` of the tile (blocks past the end reload the last one: the loads
        // keep every wave's instruction count fixed, and land in a free slot / set)
        auto kb_of = [&](int it) { return tl.kb0 + (it < nst ? it : nst - 1); };
        auto issue_a = [&](int it) __attribute__((always_inline)) {
            const u32 st = __builtin_amdgcn_readfirstlane(smem_base + (u32)(it % SLOTS) * SLOT_BYTES);
            const int kb = kb_of(it);
            // the instruction's row offset goes into the scalar offset, so the lane offset
            // is one register for all of them (no per-instruction copies kept live)
#pragma unroll
            for (int j = 0; j < IA; ++j) {
                const int i = wave + j * NWAVES;
                dma16(rs_a, voff_a, __builtin_amdgcn_readfirstlane((u32)kb * KBLK + (u32)(i * 8) * (u32)K),
                      st + i * 1024);
            }
            if (wave < NS_INS)
                dma4(rs_s, voff_sc, __builtin_amdgcn_readfirstlane((u32)kb * p.M * 4u), st + S_OFF + wave * 256);
            else
                dma4(rs_t, voff_sc, __builtin_amdgcn_readfirstlane((u32)kb * 4u), st + T_OFF);
        };
        auto issue_b = [&](int it, v4i (&dst)[TN][2]) __attribute__((always_inline)) {
            const u32 ka = __builtin_amdgcn_readfirstlane((u32)kb_of(it) * KBLK);
#pragma unroll
            for (int b = 0; b < TN; ++b) {
                dst[b][0] = load16<0>(rs_b, bvoff[b], ka);
                dst[b][1] = load16<64>(rs_b, bvoff[b], ka);
            }
        };
        lds_u8* const lds = (lds_u8*)smem_base;
        // the wave's B scale: its columns' 128-row block, relative to the tile's first
        int nblk = (tl.n0 + wave_n) / KBLK;
        nblk = nblk < NBLKS ? nblk : NBLKS - 1;
        const int sb_off = T_OFF + (nblk - nb_t0) * 4;
        const int sa_off = S_OFF + l16 * TM * 4;
        const u32 a_frag = (u32)l16 * 128u;

        v4f acc[TM][TN];
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int b = 0; b < TN; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
        // the last product of a K block and its scale, promoted under the next block's first MFMA
        v4f p_carry = {0.f, 0.f, 0.f, 0.f};
        float s_carry = 0.f;
        v4i breg[NSETS][TN][2];

        // every wave has finished reading the ring before it is refilled (the
        // earlier tile's stores may still be in flight; see variant 1)
        __syncthreads();
        // A of K blocks 0 .. SLOTS-2, then B of K blocks 0 .. DEPTH-1
#pragma unroll
        for (int i = 0; i < SLOTS - 1; ++i) issue_a(i);
        static_for<DEPTH>([&]<int J>() __attribute__((always_inline)) { issue_b(J, breg[J]); });

        // One K block.  WAIT: this wave's loads issued after B of block `it` (the first
        // DEPTH-1 blocks follow the prologue's order, the rest the loop's).
        auto kblock = [&]<int SET, int WAIT>(int it) __attribute__((always_inline)) {
            wait_vmcnt<WAIT>();
#pragma unroll
            for (int b = 0; b < TN; ++b) {
                tie(breg[SET][b][0]);
                tie(breg[SET][b][1]);
            }
            // every wave's A share of block `it` has landed, and every wave is done with
            // the slot of block it-1, which is refilled now with block it+SLOTS-1
            __syncthreads();
            issue_a(it + SLOTS - 1);
            issue_b(it + DEPTH, breg[(SET + DEPTH) % NSETS]);

            lds_u8* const slot = lds + (u32)(it % SLOTS) * SLOT_BYTES;
            const float sb = lds_read_f32(slot, sb_off);
            // A scales of four sub-tiles at a time, the next four read one group ahead
            auto read_s4 = [&](int a4) __attribute__((always_inline)) {
                return *(__attribute__((address_space(3))) const v4f*)(slot + sa_off + a4 * 16);
            };
            v4f s4 = read_s4(0), s4_next = s4;
            lds_u8* const a_lo = slot + a_frag + chunk_lo;
            lds_u8* const a_hi = slot + a_frag + chunk_hi;
            v8i fb[TN];
#pragma unroll
            for (int b = 0; b < TN; ++b) {
                const v4i x = breg[SET][b][0], y = breg[SET][b][1];
                fb[b] = v8i{x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
            }
            // A fragments read FA_AHEAD sub-tiles ahead; each MFMA runs while the FMAs
            // promote the previous sub-tile's product
            v8i fa[TM];
#pragma unroll
            for (int a = 0; a < FA_AHEAD; ++a) fa[a] = lds_read_frag(a_lo, a_hi, a * 16 * 128);
            v4f prev = p_carry;
            float sprev = s_carry;
#pragma unroll
            for (int a = 0; a < TM; ++a) {
                if (a + FA_AHEAD < TM) fa[a + FA_AHEAD] = lds_read_frag(a_lo, a_hi, (a + FA_AHEAD) * 16 * 128);
                if (a % 4 == 0 && a + 4 < TM) s4_next = read_s4(a / 4 + 1);
                const float sab = s4[a % 4] * sb;
#pragma unroll
                for (int b = 0; b < TN; ++b) {
                    const v4f zero = {0.f, 0.f, 0.f, 0.f};
                    // P[n][m] over this 128-wide K block: exact products, FP32 sums
                    const v4f pr = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fb[b], fa[a], zero, 0, 0, 0, 0, 0, 0);
                    if (a == 0 && b == 0) acc[TM - 1][TN - 1] += prev * sprev;
                    else if (b == 0) acc[a - 1][TN - 1] += prev * sprev;
                    else acc[a][b - 1] += prev * sprev;
                    prev = pr;
                    sprev = sab;
                }
                if (a % 4 == 3) s4 = s4_next;
                __builtin_amdgcn_sched_barrier(0);
            }
            p_carry = prev;
            s_carry = sprev;
        };
        // blocks 0 .. DEPTH-2: after B of block j come the prologue's B of blocks
        // j+1 .. DEPTH-1 and the loop's first j iterations
        static_for<DEPTH - 1>([&]<int J>() __attribute__((always_inline)) {
            if (J < nst) kblock.template operator()<J % NSETS, (DEPTH - 1 - J) * UB + J * UNIT>(J);
        });
        // the rest, unrolled by NSETS so every B register set has a fixed name
#pragma unroll 1
        for (int it0 = DEPTH - 1; it0 < nst; it0 += NSETS) {
            static_for<NSETS>([&]<int U>() __attribute__((always_inline)) {
                if (it0 + U < nst) kblock.template operator()<(DEPTH - 1 + U) % NSETS, (DEPTH - 1) * UNIT>(it0 + U);
            });
        }
        acc[TM - 1][TN - 1] += p_carry * s_carry;
        // the loads past the tile's last block land before their registers are released
        wait_vmcnt<0>();
#pragma unroll
        for (int s2 = 0; s2 < NSETS; ++s2)
#pragma unroll
            for (int b = 0; b < TN; ++b) {
                tie(breg[s2][b][0]);
                tie(breg[s2][b][1]);
            }

        finish_tile<TM, TN>(p, tl, acc, l16, wave_n + 4 * q, tid);
    }
}
#endif

// ============================================================ operands stored K-outermost
// The K-grouped operands, and A or B of the TN / NN / TT layouts, arrive
// K-outermost (X [rows_k][cols] bytes: a row per K index).  The matrix core
// takes each lane's K values from consecutive bytes, so before the GEMM such an
// operand is rewritten as Xt [cols][K] (row pitch K, the compile-time size;
// K-grouped: padded, and bytes past rows_k are never read); blockIdx.z walks
// the groups of a grouped B ([G][rows_k][cols] -> [G][cols][K]).
// One workgroup moves a 64 x 64 byte block through LDS: four lanes read the 64
// bytes of a K row, then each lane gathers 16 K values of one column from LDS
// and writes them as one 16-byte store.  Bound by HBM bandwidth.  The grid is
// one-dimensional, K blocks fastest, so no grid dimension limits the number of
// rows or columns.  (Column blocks fastest, so that neighbouring workgroups
// share the 128-byte lines of a row, measured 12 % slower: 93 against 83 us per
// 4 x 8192 x 4096 operand.)
extern "C" __global__ void __launch_bounds__(256)
dg_transpose_k_major(const u8* __restrict__ X, u8* __restrict__ Xt, int rows_k, int cols) {
    __shared__ __attribute__((aligned(16))) u8 tile[64][68];   // 68: rows start on different banks
    const int tid = threadIdx.x;
    const u32 nkt = (u32)rows_k >> 6;                            // K blocks (rows_k is a multiple of 64)
    const int k0 = (int)(blockIdx.x % nkt) * 64, c0 = (int)(blockIdx.x / nkt) * 64;
    X += (u64)blockIdx.z * (u64)rows_k * (u64)cols;
    Xt += (u64)blockIdx.z * (u64)cols * (u64)K;
    const int r = tid >> 2, piece = (tid & 3) * 16;
    {
        const int k = k0 + r, c = c0 + piece;
        u32 w[4] = {0u, 0u, 0u, 0u};
        if (k < rows_k) {
            const u8* src = X + (u64)k * (u64)cols + c;
            if ((cols & 15) == 0 && c + 16 <= cols) {
                const v4i x = *(const v4i*)src;           // 16-byte aligned: cols and c are multiples of 16
                w[0] = (u32)x.x; w[1] = (u32)x.y; w[2] = (u32)x.z; w[3] = (u32)x.w;
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (c + i < cols) w[i >> 2] |= (u32)src[i] << (8 * (i & 3));
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) *(u32*)&tile[r][piece + 4 * j] = w[j];
    }
    __syncthreads();
    const int c = c0 + r;
    if (c < cols && k0 + piece < rows_k) {
        u32 w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            w[j] = (u32)tile[piece + 4 * j][r] | ((u32)tile[piece + 4 * j + 1][r] << 8) |
                   ((u32)tile[piece + 4 * j + 2][r] << 16) | ((u32)tile[piece + 4 * j + 3][r] << 24);
        *(v4i*)(Xt + (u64)c * K + k0 + piece) = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
}

}  // namespace dg
