// Tile selection for the block-scaled FP8 GEMM kernels on MI355X.
//
// DeepGEMM picks block sizes per shape so that the grid fills the machine,
// including non-power-of-two widths such as 112 (launch article, section 2.2
// "non-standard block partitioning", and section 7).  The same idea is used
// here with a small cost model of gfx950: 256 CUs, 8 XCDs, 160 KB LDS per CU,
// 8192 dense FP8 FLOP/clk/CU at 2.4 GHz and ~8 TB/s of HBM.  Candidates are
// (tile, wave grid, LDS stages, split-K) tuples; the model charges each
// candidate its wave-quantised MFMA time, its operand traffic and a fixed
// per-tile cost, and the cheapest one wins.  DG_FORCE_CONFIG
// ("bm,bn,wm,wn,stages,splitk[,kstep[,variant[,nb,ne]]]", launches separated
// by ';') overrides the choice for tuning sweeps.
#include <algorithm>
#include <iterator>
#include <cmath>
#include <cstdio>
#include <cstdlib>

#include "dg_internal.h"

namespace dg {
namespace {

constexpr double kClockHz = 2.4e9;
constexpr double kMfmaFlopPerClkCu = 8192.0;
constexpr double kHbmBytesPerS = 8.0e12;
constexpr double kCuLoadBytesPerS = 64.0 * kClockHz;   // one CU's share of L2 fabric
constexpr int kLdsBytes = 160 * 1024;

int round_up(int x, int m) { return (x + m - 1) / m * m; }

int vgpr_estimate(int tm, int tn) {
    // accumulators + A fragments + two B fragments + products + addressing
    return tm * tn * 4 + tm * 8 + 16 + tm * tn / 2 + 48;
}

int occupancy(const KernelConfig& c) {
    int lds = c.lds_bytes();
    int by_lds = kLdsBytes / std::max(lds, 1);
    int tm = c.bm / c.wm / 16, tn = c.bn / c.wn / 16;
    int v = round_up(vgpr_estimate(tm, tn), 8);
    int waves_per_simd = std::min(8, 512 / std::max(v, 8));
    int by_regs = waves_per_simd * 4 / (c.wm * c.wn);
    return std::max(1, std::min(by_lds, by_regs));
}

struct Estimate {
    double seconds;
    KernelConfig cfg;
};

double estimate(const Problem& p, const KernelConfig& c, int num_cus, double valid_rows) {
    const int mt = (p.kind == kMasked) ? (int)std::ceil(valid_rows / std::max(p.g, 1) / c.bm) * p.g
                                       : (p.rows + c.bm - 1) / c.bm * (p.kind == kKGrouped ? p.g : 1);
    const int nt = (p.n + c.bn - 1) / c.bn;
    const double tiles = (double)mt * nt * c.splitk;
    const int occ = occupancy(c);
    const double slots = (double)num_cus * occ;
    const double waves = std::ceil(tiles / slots);
    // K-grouped: a tile covers one group's share of K (taken as an even split)
    const double kspan = (double)p.k / c.splitk / (p.kind == kKGrouped ? std::max(p.g, 1) : 1);
    const double kblocks = kspan / 128.0;
    const int nw = c.wm * c.wn;
    const double waves_per_simd = std::max(1.0, occ * nw / 4.0);
    // Per-CU cycle counts of one tile (measured shape of the kernel on gfx950):
    //  * MFMA: 32 cycles per 16x16x128 step on each of 4 SIMDs, shared by the
    //    occ resident workgroups;
    //  * VALU: one FMA per output element per K block plus a scale product per
    //    sub-tile, 4 cycles per wave64 instruction; only part of it hides under
    //    the MFMAs of the same SIMD;
    //  * a fixed cost per LDS stage (barrier, first LDS reads) that a second
    //    wave per SIMD mostly hides.
    const double mfma_cyc = (double)c.bm * c.bn * kspan * 2.0 / kMfmaFlopPerClkCu * occ /
                            std::min(1.0, nw * occ / 4.0);
    const double valu_cyc = (double)c.bm * c.bn / 64.0 * kblocks * 1.3 * 4.0 / 4.0 * occ;
    const double compute_cyc = std::max(mfma_cyc, valu_cyc) + 0.35 * std::min(mfma_cyc, valu_cyc);
    const double stage_cyc = 900.0 / waves_per_simd * (kblocks / c.kstep);
    const double t_compute = (compute_cyc + stage_cyc) / kClockHz;
    // operand tiles mostly come from L2/MALL (they are shared between tiles);
    // the HBM bound of the whole launch is applied below
    const double t_load = ((c.sf == 4 ? 0.5 : 1.0) * c.bm + (c.sf == 2 || c.sf == 4 ? 0.5 : 1.0) * c.bn) * kspan /
                          (kCuLoadBytesPerS / occ);
    // pipeline fill, epilogue and scheduling per tile; split-K adds a round trip
    double t_fixed = 1.2e-6 + (c.splitk > 1 ? 1.0e-6 * c.splitk + c.bm * c.bn * 8.0 * c.splitk / kCuLoadBytesPerS : 0.0);
    double t = waves * (std::max(t_compute, t_load) + t_fixed);
    // whole-device floor: HBM traffic.  Row blocks that share a B column block
    // re-read it; they only hit in L2 when they run close together, which the
    // grouped tile order gives for large M (8 row blocks per sweep) but not for
    // a handful of row blocks spread over the whole grid.
    const double groups_b = (p.kind == kDense) ? 1.0 : p.g;
    const double rows_per_group = valid_rows / groups_b;
    const double b_reads = rows_per_group <= 512 ? std::ceil(rows_per_group / c.bm)
                                                 : std::max(1.0, std::ceil(rows_per_group / c.bm) / 8.0);
    const double b_row_bytes = (p.sf == 2 || p.sf == 4) ? p.k / 2.0 : (double)p.k;
    const double bytes = valid_rows * p.k + b_reads * groups_b * p.n * b_row_bytes +
                         valid_rows * p.n * (2.0 + 4.0 * p.has_c);
    t = std::max(t, bytes / kHbmBytesPerS);
    return t;
}

int dma_per_wave(const KernelConfig& c) {
    const int nw = c.wm * c.wn;
    const int rpi = 8 / c.kstep;
    const int na = c.sf == 4 ? c.bm / 16 : c.bm / rpi, nb = (c.sf == 2 || c.sf == 4) ? c.bn / 16 : c.bn / rpi;
    const int ns = c.sf == 3 ? 0 : (c.bm + 63) / 64 * c.kstep;
    const int nt = c.sf == 3 ? 0 : (c.sf == 2 || c.sf == 4 || c.kind == kKGrouped) ? (c.bn + 63) / 64 : c.kstep;
    return (na + nw - 1) / nw + (nb + nw - 1) / nw + (ns + nw - 1) / nw + (nt + nw - 1) / nw;
}

// Vector-memory instructions per wave per K block of variant 1 (A/sfa DMA
// share, one sfb DMA, two 16-byte B loads per 16-row sub-tile).
int unit_per_wave_v1(const KernelConfig& c) {
    const int nw = c.wm * c.wn;
    return (c.bm / 8 + nw - 1) / nw + ((c.bm + 63) / 64 + nw - 1) / nw + 1 + 2 * (c.bn / c.wn / 16);
}

// Mirrors the kernel's static_asserts, so a selected config always compiles.
bool valid(const KernelConfig& c, const Problem& p) {
    if (c.bm % (16 * c.wm) || c.bn % (16 * c.wn)) return false;
    if (c.ne > 0 && (c.nb < 0 || c.nb % 16 || c.nb >= c.ne || c.ne > p.n)) return false;
    if (c.splitk < 1 || (c.splitk > 1 && p.kind != kDense)) return false;   // split-K: dense only
    if (c.sf != p.sf) return false;
    // variant 4: variant 0 with A requested a K block ahead of B (two B slots, three A
    // slots), for FP8 operands with FP32 or UE8M0 scales and the M forms
    if (c.variant == 4 && (c.kstep != 1 || c.stages != 2 || c.sf == 2 || c.sf == 4 || p.kind == kKGrouped))
        return false;
    // variant 6: variant 0 with the split refill (FP8 operands with FP32 or UE8M0 scales,
    // or BF16; one K block a stage, an even number of n sub-tiles per wave)
    if (c.variant == 6 && (c.kstep != 1 || c.sf == 2 || c.sf == 4 ||
                           (c.bn / c.wn / 16) % 2 || c.bn / c.wn / 16 < 4))
        return false;
    if (c.sf && ((c.variant != 0 && c.variant != 4 && c.variant != 6) || c.kstep != 1)) return false;   // UE8M0, FP4: variant 0, one K block a stage
    if (p.kind == kKGrouped && (c.sf || (c.variant != 0 && c.variant != 6) || c.kstep != 1)) return false;   // K-grouped: the same
    if (c.variant < 0 || c.variant > 6) return false;
    int tm = c.bm / c.wm / 16, tn = c.bn / c.wn / 16;
    if (c.lds_bytes() > kLdsBytes) return false;
    if (c.bn > 256) return false;
    if (c.variant == 5) {
        // B in VGPRs (each wave its own columns), A through a ring of `stages` slots;
        // FP32 scales, one K block a slot, no split-K, the M forms
        const int nw = c.wm * c.wn;
        if (c.sf || c.kstep != 1 || c.splitk != 1 || c.wm != 1 || p.kind == kKGrouped) return false;
        if (c.bm % 64 || (c.bm / 8) % nw || c.bm / 64 + 1 > nw || c.stages < 3) return false;
        if (128 % (c.bn / nw) || tm % 4 || tm * tn > 32 || tn < 1) return false;
        if (p.kind == kContiguous && c.bm > 128) return false;   // one expert per row block
        return (c.bm / 8 / nw + 1 + 2 * tn) * 2 <= 63;           // vmcnt field (two K blocks of B ahead)
    }
    if (p.kind == kContiguous && 128 % c.bm != 0 && c.bm % 128 != 0) return false;
    // one expert per row block; 256-row blocks (both operands through LDS) make one
    // pass per expert of their two 128-row blocks
    if (p.kind == kContiguous && c.bm > 128 && !(c.bm == 256 && (c.variant == 0 || c.variant == 4 || c.variant == 6)))
        return false;
    if (c.variant != 0 && c.variant != 4 && c.variant != 6) {
        // waves along n only, one K block at a time, the whole K range of a
        // work item unrolled, B registers of stages - 1 blocks in flight
        if (c.wm != 1 || c.kstep != 1 || c.stages < 2) return false;
        if ((p.k / 128) % c.splitk || p.k / 128 / c.splitk > 64) return false;
        const int ub = 2 * (c.bn / c.wn / 16);
        const int nkb = p.k / 128 / c.splitk, pre = std::min(c.stages - 1, nkb);
        if (c.variant == 1 && unit_per_wave_v1(c) * (c.stages - 2) > 63) return false;
        if (c.variant == 2 && (ub * (c.stages - 2) > 63 || ub * pre > 63)) return false;
        if (c.variant == 3 && (ub * pre > 63 || c.bm * 128 + 256 > 78 * 1024)) return false;
        if (tm < 1 || tn < 1 || tm > 16 || tn > 4 || tm * tn > 32) return false;
        if (c.bm % 8) return false;
        return true;
    }
    if (c.kstep != 1 && c.kstep != 2) return false;
    if (c.bm % (8 / c.kstep) || c.bn % (8 / c.kstep) || c.stages < 2) return false;
    if (dma_per_wave(c) * (c.stages - 1) > 63) return false;   // vmcnt field
    if (c.variant == 6 && (dma_per_wave(c) + 1) * (c.stages - 1) > 63) return false;   // split groups round up
    // more than 32 sub-tiles per wave: only 4-wave groups without promotion (accumulators in AGPRs)
    const bool agpr_acc = (c.sf == 1 || c.sf == 3 || c.sf == 5) && c.wm * c.wn == 4;
    if (tm < 1 || tn < 1 || tm > 8 || tn > 8 || tm * tn > (agpr_acc ? 64 : 32)) return false;
    if ((p.k / 128) % (c.splitk * c.kstep)) return false;
    return true;
}

// Configurations measured fastest on an MI355X (graph-replayed back-to-back
// launches, tile/wave/stage/split sweeps) for the shapes of the DeepGEMM
// launch article's benchmark tables; other shapes go through the model.
// Consecutive rows of one shape with column ranges [nb, ne) are launched in
// turn (none at present: 4096 x 7168 as 256 x 256 tiles over [0, 4096) then
// 256 x 192 over [4096, 7168) fills two whole rounds of 256 CUs instead of
// 1.75, yet measured the same as 448 tiles of 256 x 256, 459 us each: the
// part runs at its power limit there, so idle CUs in a partial round are not
// lost time).
struct Tuned {
    int kind, rows, n, k, g, has_c;
    int bm, bn, wm, wn, stages, splitk, kstep, variant;
    int nb, ne;
};
const Tuned kTuned[] = {
    {kDense, 64, 2112, 7168, 1, 0, 64, 64, 1, 4, 4, 7, 1, 2, 0, 0},
    {kDense, 128, 24576, 1536, 1, 0, 128, 96, 1, 6, 3, 1, 1, 3, 0, 0},
    {kDense, 128, 24576, 1536, 1, 1, 128, 96, 4, 2, 2, 1, 2, 0, 0, 0},
    // the large shapes: 256 x 256 with the split refill (variant 6): 426-434 us against
    // 449 us for the one-part refill and 447-465 us for 256 x 224 (512 tiles, two full
    // rounds); contiguous: 808 us against 862 us for the one-part refill (one box)
    {kDense, 4096, 7168, 16384, 1, 0, 256, 256, 4, 2, 2, 1, 1, 6, 0, 0},
    {kContiguous, -1, 4096, 7168, 4, 0, 256, 256, 4, 2, 2, 1, 1, 6, 0, 0},
    // the masked decode shape, B streamed: 128 x 128 on variant 0 with three stages
    // 17.47-17.58 us against 17.97-18.10 us for the producer variant with 128 x 112
    // (one box; before B was streamed the producer variant led, 20.6 against 20.4-21.7)
    {kMasked, 256, 7168, 2048, 4, 0, 128, 128, 4, 2, 3, 1, 1, 0, 0, 0},
    // K-grouped weight gradient of the contiguous workload (K: the row pitch of the
    // K-contiguous operands, 4 x 8192 tokens): 192 x 256 with two stages measured 2-4 %
    // under 128 x 256 with three (22 row tiles, the last one a third full); with the split
    // refill 1274-1280 us against 1310-1344 us
    {kKGrouped, 4096, 7168, 32768, 4, 0, 192, 256, 4, 2, 2, 1, 1, 6, 0, 0},
};

// Packed UE8M0 scales (one K block a stage; no promotion in the K loop).  The
// large shapes use 256 x 256 with the split refill (variant 6): 399-404 us against
// 411 us for four waves of 128 x 128 with accumulators in AGPRs; contiguous 739-746 us
// against 790 us for the four-wave tile and 845 us for it without the split (one box)
const Tuned kTunedE8[] = {
    {kDense, 64, 2112, 7168, 1, 0, 64, 64, 2, 2, 4, 7, 1, 0, 0, 0},
    {kDense, 128, 24576, 1536, 1, 0, 128, 96, 4, 2, 3, 1, 1, 0, 0, 0},
    // with C: 15.8 us against 16.7-16.8 us for the model's 128 x 128 with 2 x 4 waves (one box)
    {kDense, 128, 24576, 1536, 1, 1, 128, 96, 4, 2, 4, 1, 1, 0, 0, 0},
    {kDense, 4096, 7168, 16384, 1, 0, 256, 256, 4, 2, 2, 1, 1, 6, 0, 0},
    {kContiguous, -1, 4096, 7168, 4, 0, 256, 256, 4, 2, 2, 1, 1, 6, 0, 0},
    {kMasked, 256, 7168, 2048, 4, 0, 128, 128, 4, 2, 3, 1, 1, 0, 0, 0},
};

// FP8 x FP4 and FP4 x FP4 (variant 0; B, and for FP4 x FP4 also A, tiles are half
// the bytes of the FP8 ones, so 256 x 256 fits three LDS stages: measured 429 us
// (FP8 x FP4) and 403 us (FP4 x FP4) against 485 and 465 us with two, the K loop
// of the large tile being bound by how far ahead its loads are issued)
const Tuned kTunedF4[] = {
    {kDense, 64, 2112, 7168, 1, 0, 64, 64, 2, 2, 4, 7, 1, 0, 0, 0},
    {kDense, 128, 24576, 1536, 1, 0, 128, 96, 4, 2, 3, 1, 1, 0, 0, 0},
    {kDense, 4096, 7168, 16384, 1, 0, 256, 256, 4, 2, 3, 1, 1, 0, 0, 0},
    // contiguous: 256-row blocks with three stages, 849-854 us against 1100-1111 us
    // for 128 x 224 with four (one box)
    {kContiguous, -1, 4096, 7168, 4, 0, 256, 256, 4, 2, 3, 1, 1, 0, 0, 0},
    {kMasked, 256, 7168, 2048, 4, 0, 128, 128, 4, 2, 3, 1, 1, 0, 0, 0},
};

// FP4 x FP4: the FP8 x FP4 choices (contiguous: 724-728 us against 917-924 us for
// 128 x 256 with three stages)
const Tuned kTunedF4F4[] = {
    {kDense, 64, 2112, 7168, 1, 0, 64, 64, 2, 2, 4, 7, 1, 0, 0, 0},
    {kDense, 128, 24576, 1536, 1, 0, 128, 96, 4, 2, 3, 1, 1, 0, 0, 0},
    {kDense, 4096, 7168, 16384, 1, 0, 256, 256, 4, 2, 3, 1, 1, 0, 0, 0},
    {kContiguous, -1, 4096, 7168, 4, 0, 256, 256, 4, 2, 3, 1, 1, 0, 0, 0},
    {kMasked, 256, 7168, 2048, 4, 0, 128, 128, 4, 2, 3, 1, 1, 0, 0, 0},
};

// BF16 x BF16 (k here is the row length in bytes, 2 x K).  A 128-byte K block is
// 64 elements, half the MFMA time of an FP8 one, so the loads' lead matters more:
// variant 4 (A one K block further ahead) 794 us against 865 us for variant 0; the split
// refill with 256 x 256 812-816 us against 819-839 us for variant 4 with 256 x 224
const Tuned kTunedBF16[] = {
    {kDense, 4096, 7168, 32768, 1, 0, 256, 256, 4, 2, 2, 1, 1, 6, 0, 0},
};

std::vector<KernelConfig> tuned(const Problem& p, int num_cus, const KernelConfig& base) {
    std::vector<KernelConfig> out;
    if (num_cus != 256) return out;       // measured on the full 256-CU part
    // FP4 x FP4 starts from the FP8 x FP4 table (same structure, A half the bytes)
    const Tuned* first = p.sf == 3 ? std::begin(kTunedBF16) : p.sf == 4 ? std::begin(kTunedF4F4)
                       : p.sf == 2 ? std::begin(kTunedF4) : p.sf ? std::begin(kTunedE8) : std::begin(kTuned);
    const Tuned* last = p.sf == 3 ? std::end(kTunedBF16) : p.sf == 4 ? std::end(kTunedF4F4)
                      : p.sf == 2 ? std::end(kTunedF4) : p.sf ? std::end(kTunedE8) : std::end(kTuned);
    for (const Tuned* it = first; it != last; ++it) {
        const Tuned& t = *it;
        if (t.kind != p.kind || t.n != p.n || t.k != p.k || t.g != p.g || t.has_c != p.has_c) continue;
        if (t.rows >= 0 && t.rows != p.rows) continue;
        if (t.rows < 0 && p.rows < 4096) continue;   // contiguous: any large token count
        KernelConfig c = base;
        c.bm = t.bm; c.bn = t.bn; c.wm = t.wm; c.wn = t.wn;
        c.stages = t.stages; c.splitk = t.splitk; c.kstep = t.kstep; c.variant = t.variant;
        c.nb = t.nb; c.ne = t.ne;
        out.push_back(c);
    }
    return out;
}

// DG_FORCE_CONFIG="bm,bn,wm,wn,stages,splitk[,kstep[,variant[,nb,ne]]]", or
// several such launches over column ranges [nb, ne) separated by ';'.
std::vector<KernelConfig> parse_forced(const KernelConfig& base) {
    const char* env = std::getenv("DG_FORCE_CONFIG");
    if (!env || !*env) return {};
    std::vector<KernelConfig> out;
    std::string all(env);
    size_t pos = 0;
    while (pos <= all.size()) {
        size_t end = all.find(';', pos);
        if (end == std::string::npos) end = all.size();
        const std::string one = all.substr(pos, end - pos);
        pos = end + 1;
        int bm, bn, wm, wn, st, sk, ks = 1, var = 0, nb = 0, ne = 0;
        int got = std::sscanf(one.c_str(), "%d,%d,%d,%d,%d,%d,%d,%d,%d,%d", &bm, &bn, &wm, &wn, &st, &sk, &ks, &var,
                              &nb, &ne);
        if (got < 6 || got == 9) return {};
        KernelConfig c = base;
        c.bm = bm; c.bn = bn; c.wm = wm; c.wn = wn; c.stages = st; c.splitk = sk; c.kstep = ks;
        c.variant = var;
        c.nb = nb; c.ne = ne;
        out.push_back(c);
    }
    return out;
}

// A B block that at most two row blocks of the launch read (dense or masked
// with few rows) is streamed: its loads carry the non-temporal hint.  Measured
// (one box, alternating): 128x24576x1536 15.1 against 15.5 us, with C 16.0
// against 18.8, UE8M0 14.6 against 15.4, the masked decode shape 18.3 against
// 19.7; where four row blocks share each B block through L2 (the large
// shapes) the hint cost 1-9 %.
std::vector<KernelConfig> with_b_streams(std::vector<KernelConfig> plan, const Problem& p) {
    for (KernelConfig& c : plan)
        c.bstream = (p.kind == kDense || p.kind == kMasked) && p.rows <= 2 * c.bm ? 1 : 0;
    return plan;
}

// The launches cover [0, N) in order, each valid.
bool valid_plan(const std::vector<KernelConfig>& plan, const Problem& p) {
    if (plan.empty()) return false;
    int next = 0;
    for (const KernelConfig& c : plan) {
        if (!valid(c, p) || c.n_begin() != next) return false;
        next = c.n_end();
    }
    return next == p.n;
}

}  // namespace

int64_t num_work_items(const KernelConfig& c, int rows) {
    const int64_t mt = (rows + c.bm - 1) / c.bm;
    const int64_t nt = (c.n_end() - c.n_begin() + c.bn - 1) / c.bn;
    if (c.kind == kMasked || c.kind == kKGrouped) return mt * nt * c.g;
    return mt * nt * c.splitk;
}

std::vector<KernelConfig> select_plan(const Problem& p, int num_cus) {
    KernelConfig base;
    base.kind = p.kind;
    base.has_c = p.has_c;
    base.sf = p.sf;
    base.n = p.n;
    base.k = p.k;
    base.g = (p.kind == kDense) ? 1 : p.g;

    std::vector<KernelConfig> forced = parse_forced(base);
    if (valid_plan(forced, p)) return with_b_streams(forced, p);
    std::vector<KernelConfig> table = with_b_streams(tuned(p, num_cus, base), p);
    if (valid_plan(table, p)) {
        if (env_flag("DG_PRINT_CONFIGS"))
            for (const KernelConfig& c : table)
                std::fprintf(stderr, "[dg] kind=%d rows=%d N=%d K=%d G=%d -> %s (measured)\n", p.kind, p.rows, p.n,
                             p.k, p.g, c.key().c_str());
        return table;
    }

    // masked: the host cannot see masked_m; plan for half the rows being valid
    const double valid_rows = (p.kind == kMasked) ? 0.5 * p.rows * p.g : (double)p.rows;
    const int kb = p.k / 128;
    static const int bms[] = {16, 32, 64, 128, 256};
    static const int bns[] = {16, 32, 48, 64, 96, 112, 128, 160, 192, 224, 256};
    static const int wgs[][2] = {{1, 4}, {2, 2}, {4, 1}, {2, 4}, {4, 2}, {1, 8}, {8, 1}, {1, 1}, {1, 2}, {2, 1}};
    const int max_bm = round_up(std::max(p.rows, 16), 16);
    // Skinny row counts: one row block covers every row (of a group), so each B
    // tile is fetched from HBM once instead of once per row block.
    // (masked groups are not: their row blocks past masked_m[g] are skipped)
    const bool one_row_block = p.kind == kDense && p.rows <= 256;

    // Structure the measurements favour on gfx950: two waves per SIMD (8-wave
    // workgroups) for large tiles, four waves otherwise, wave grids no more
    // than 4:1, row blocks of 64+ rows unless the problem has fewer rows, and
    // split-K only when the output tiles alone cannot fill the device.
    const int out_tiles_128 = ((p.rows + 127) / 128) * ((p.n + 127) / 128);
    Estimate best{1e30, base};
    for (int bm : bms) {
        if (bm > max_bm && bm > 16 && bm / 2 >= max_bm) continue;   // no tile twice the rows
        if (one_row_block && bm < max_bm) continue;
        if (bm < 64 && max_bm >= 64) continue;
        for (int bn : bns) {
            if (bn > round_up(p.n, 16) && bn / 2 >= round_up(p.n, 16)) continue;
            for (auto& w : wgs) {
                const int nw = w[0] * w[1];
                const bool tiny = bm * bn < 64 * 64;
                if (!tiny && nw < 4) continue;
                if (bm * bn >= 128 * 96 && nw < 8) continue;
                if (bm * bn < 128 * 96 && nw > 4) continue;
                if (w[0] > 2 * w[1] || w[1] > 2 * w[0]) {
                    if (!tiny) continue;
                }
                for (int sk = 1; sk <= 16; ++sk) {
                  for (int ks = 1; ks <= (p.sf ? 1 : 2); ++ks) {
                    if (sk > 1 && (p.kind != kDense || kb % sk || kb / sk < 2)) continue;
                    if (sk > 1 && out_tiles_128 * 2 >= num_cus) continue;
                    if (sk > 1 && bm * bn < 64 * 128) continue;   // small split tiles measured slow
                    KernelConfig c = base;
                    c.bm = bm; c.bn = bn; c.wm = w[0]; c.wn = w[1]; c.splitk = sk; c.kstep = ks;
                    c.stages = std::min(4, kLdsBytes / c.stage_bytes());
                    while (c.stages > 2 && dma_per_wave(c) * (c.stages - 1) > 63) --c.stages;
                    if (c.stages < 2) continue;
                    if (!valid(c, p)) continue;
                    double t = estimate(p, c, num_cus, valid_rows);
                    // prefer bigger wave tiles on ties (fewer LDS reads per MFMA)
                    t *= 1.0 + 0.01 / (c.bm / c.wm / 16 * (c.bn / c.wn / 16));
                    if (t < best.seconds) best = {t, c};
                  }
                }
            }
        }
    }
    std::vector<KernelConfig> plan = with_b_streams({best.cfg}, p);
    if (env_flag("DG_PRINT_CONFIGS"))
        std::fprintf(stderr, "[dg] kind=%d rows=%d N=%d K=%d G=%d -> %s (model %.2f us)\n", p.kind, p.rows, p.n,
                     p.k, p.g, plan[0].key().c_str(), best.seconds * 1e6);
    return plan;
}

}  // namespace dg
