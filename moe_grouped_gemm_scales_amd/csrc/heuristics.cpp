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
// ("bm,bn,wm,wn,stages,splitk") overrides the choice for tuning sweeps.
#include <algorithm>
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

double mfma_efficiency(int tm, int tn) {
    // fraction of MFMA peak one wave tile sustains: small tiles spend more issue
    // slots on LDS reads, scale products and loop overhead per MFMA
    double per_mfma_overhead = 2.0 / tm + 2.0 / tn;   // fragment reads per MFMA
    return 0.85 / (1.0 + 0.25 * per_mfma_overhead);
}

struct Estimate {
    double seconds;
    KernelConfig cfg;
};

double estimate(const Problem& p, const KernelConfig& c, int num_cus, double valid_rows) {
    const int mt = (p.kind == kMasked) ? (int)std::ceil(valid_rows / std::max(p.g, 1) / c.bm) * p.g
                                       : (p.rows + c.bm - 1) / c.bm;
    const int nt = (p.n + c.bn - 1) / c.bn;
    const double tiles = (double)mt * nt * c.splitk;
    const int occ = occupancy(c);
    const double slots = (double)num_cus * occ;
    const double waves = std::ceil(tiles / slots);
    const double active = std::min(tiles, slots);
    const double kspan = (double)p.k / c.splitk;
    const int tm = c.bm / c.wm / 16, tn = c.bn / c.wn / 16;
    // a CU has 4 SIMDs: fewer than 4 resident waves leave matrix cores idle
    const double simd_use = std::min(1.0, occ * c.wm * c.wn / 4.0);
    const double mfma_rate = kMfmaFlopPerClkCu * kClockHz * mfma_efficiency(tm, tn) * simd_use / occ;
    const double t_compute = 2.0 * c.bm * c.bn * kspan / mfma_rate;
    // operand tiles mostly come from L2/MALL (they are shared between tiles);
    // the HBM bound of the whole launch is applied below
    (void)active;
    const double t_load = (double)(c.bm + c.bn) * kspan / (kCuLoadBytesPerS / occ);
    // pipeline fill, epilogue and scheduling per tile; split-K adds a round trip
    double t_fixed = 1.2e-6 + (c.splitk > 1 ? 1.0e-6 + c.bm * c.bn * 8.0 * c.splitk / kCuLoadBytesPerS : 0.0);
    double t = waves * (std::max(t_compute, t_load) + t_fixed);
    // whole-device floors: HBM traffic for the operands read once, D written once
    const double groups_b = (p.kind == kDense) ? 1.0 : p.g;
    const double bytes = valid_rows * p.k + groups_b * p.n * p.k + valid_rows * p.n * (2.0 + 4.0 * p.has_c);
    t = std::max(t, bytes / kHbmBytesPerS);
    return t;
}

int dma_per_wave(const KernelConfig& c) {
    const int nw = c.wm * c.wn;
    const int na = c.bm / 8, nb = c.bn / 8, ns = (c.bm + 63) / 64;
    return (na + nw - 1) / nw + (nb + nw - 1) / nw + (ns + nw - 1) / nw;
}

// Mirrors the kernel's static_asserts, so a selected config always compiles.
bool valid(const KernelConfig& c, const Problem& p) {
    if (c.bm % (16 * c.wm) || c.bn % (16 * c.wn)) return false;
    if (c.bm % 8 || c.bn % 8 || c.stages < 2) return false;
    if (dma_per_wave(c) * (c.stages - 1) > 63) return false;   // vmcnt field
    int tm = c.bm / c.wm / 16, tn = c.bn / c.wn / 16;
    if (tm < 1 || tn < 1 || tm > 8 || tn > 8 || tm * tn > 32) return false;
    if (c.lds_bytes() > kLdsBytes) return false;
    if ((p.k / 128) % c.splitk) return false;
    if (p.kind == kContiguous && 128 % c.bm != 0 && c.bm % 128 != 0) return false;
    if (p.kind == kContiguous && c.bm > 128) return false;   // one expert per row block
    return true;
}

bool parse_forced(KernelConfig* c) {
    const char* s = std::getenv("DG_FORCE_CONFIG");
    if (!s || !*s) return false;
    int bm, bn, wm, wn, st, sk;
    if (std::sscanf(s, "%d,%d,%d,%d,%d,%d", &bm, &bn, &wm, &wn, &st, &sk) != 6) return false;
    c->bm = bm; c->bn = bn; c->wm = wm; c->wn = wn; c->stages = st; c->splitk = sk;
    return true;
}

}  // namespace

int64_t num_work_items(const KernelConfig& c, int rows) {
    const int64_t mt = (rows + c.bm - 1) / c.bm;
    const int64_t nt = (c.n + c.bn - 1) / c.bn;
    if (c.kind == kMasked) return mt * nt * c.g;
    return mt * nt * c.splitk;
}

KernelConfig select_config(const Problem& p, int num_cus) {
    KernelConfig base;
    base.kind = p.kind;
    base.has_c = p.has_c;
    base.n = p.n;
    base.k = p.k;
    base.g = (p.kind == kDense) ? 1 : p.g;

    KernelConfig forced = base;
    if (parse_forced(&forced) && valid(forced, p)) return forced;

    // masked: the host cannot see masked_m; plan for half the rows being valid
    const double valid_rows = (p.kind == kMasked) ? 0.5 * p.rows * p.g : (double)p.rows;
    const int kb = p.k / 128;
    static const int bms[] = {16, 32, 64, 128, 256};
    static const int bns[] = {16, 32, 48, 64, 96, 112, 128, 160, 192, 224, 256};
    static const int wgs[][2] = {{1, 4}, {2, 2}, {4, 1}, {2, 4}, {4, 2}, {1, 8}, {8, 1}, {1, 1}, {1, 2}, {2, 1}};
    const int max_bm = round_up(std::max(p.rows, 16), 16);

    Estimate best{1e30, base};
    for (int bm : bms) {
        if (bm > max_bm && bm > 16 && bm / 2 >= max_bm) continue;   // no tile twice the rows
        for (int bn : bns) {
            if (bn > round_up(p.n, 16) && bn / 2 >= round_up(p.n, 16)) continue;
            for (auto& w : wgs) {
                for (int sk = 1; sk <= 16; ++sk) {
                    if (sk > 1 && (p.kind != kDense || kb % sk || kb / sk < 2)) continue;
                    KernelConfig c = base;
                    c.bm = bm; c.bn = bn; c.wm = w[0]; c.wn = w[1]; c.splitk = sk;
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
    if (env_flag("DG_PRINT_CONFIGS"))
        std::fprintf(stderr, "[dg] kind=%d rows=%d N=%d K=%d G=%d -> %s (model %.2f us)\n", p.kind, p.rows, p.n,
                     p.k, p.g, best.cfg.key().c_str(), best.seconds * 1e6);
    return best.cfg;
}

}  // namespace dg
