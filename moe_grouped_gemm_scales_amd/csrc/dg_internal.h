// Internal declarations of libdg.so (host side).
#pragma once

#include <algorithm>
#include <cstdint>
#include <string>
#include <vector>

#include "dg.h"

namespace dg {

enum Kind : int { kDense = 0, kContiguous = 1, kMasked = 2, kKGrouped = 3 };

// One compiled specialisation of the kernel.  Everything here becomes a -D
// macro of the hipRTC compile; N and K are compile-time constants (the
// DeepGEMM launch article, section 4.2, bakes the matrix sizes into each JIT
// kernel), M stays a run-time argument so a changing token count reuses code.
struct KernelConfig {
    int kind = kDense;
    int bm = 128, bn = 128;    // workgroup tile (rows of A, rows of B)
    int wm = 2, wn = 2;        // waves along m and n
    int stages = 2;            // LDS ring depth
    int kstep = 1;             // 128-wide K blocks per LDS stage (1 or 2)
    int splitk = 1;            // K splits (dense only)
    int variant = 0;           // 0: A and B through LDS; 1: B straight into VGPRs, A through an LDS
                               // ring; 2: B straight into VGPRs, A of the K range resident in LDS;
                               // 3: as 1, with an extra producer wave for A and no K-loop barrier;
                               // 4: as 0, with A requested one K block further ahead than B;
                               // 5: B straight into VGPRs (each wave its own columns), A through a
                               //    ring of `stages` LDS slots (large tiles)
                               // 6: as 0, each slot refilled in two parts: A, the scales and the
                               //    first half of B after a barrier in the middle of the K block,
                               //    the second half of B after the block
    int has_c = 0;
    int n = 0, k = 0, g = 1;
    int sf = 0;                // scale format: 0 FP32, 1 packed UE8M0, 2 FP8 x FP4 (E2M1 B, 1x32 UE8M0),
                               // 3 BF16 x BF16 without scales (k is then the row length in bytes),
                               // 4 FP4 x FP4 (E2M1 A and B, 1x32 UE8M0 per row),
                               // 5 UE8M0 pairs in 16-bit words, MN-major (A and B)
    int nb = 0, ne = 0;        // columns [nb, ne) of D (ne = 0: all N); one call may
                               // launch two column ranges with different tile widths
    int bstream = 0;           // each B block is read by at most two row blocks of the launch
                               // (dense or masked, few rows): B loads carry the non-temporal hint

    int n_begin() const { return nb; }
    int n_end() const { return ne > 0 ? ne : n; }

    int threads() const { return 64 * (wm * wn + (variant == 3 ? 1 : 0)); }   // variant 3: + producer wave
    int stage_bytes() const {
        if (variant == 1) return bm * 128 + (bm + 63) / 64 * 256 + 256;
        if (sf == 2) return bm * 128 + bn * 64 + (bm + 63) / 64 * 256 + (bn + 63) / 64 * 256;
        if (sf == 3) return (bm + bn) * 128;   // BF16: no scales
        if (sf == 4) return (bm + bn) * 64 + (bm + 63) / 64 * 256 + (bn + 63) / 64 * 256;   // FP4 x FP4
        if (kind == kKGrouped) return (bm + bn) * 128 + (bm + 63) / 64 * 256 + (bn + 63) / 64 * 256;
        return (bm + bn) * 128 * kstep + kstep * ((bm + 63) / 64) * 256 + kstep * 256;
    }
    // variants 0, 4 and 6 of the contiguous form: 256 bytes per wave for the experts of its rows
    int row_group_bytes() const {
        const bool v046 = variant == 0 || variant == 4 || variant == 6;
        return v046 && kind == kContiguous && bm / wm <= 64 ? 256 * wm * wn : 0;
    }
    int lds_bytes() const {
        if (variant == 4) {   // three A slots (tile + sfa), two B slots (tile + sfb); BF16: no scales
            const int sa = sf == 3 ? 0 : (bm + 63) / 64 * 256, sb = sf == 3 ? 0 : 256;
            return (stages + 1) * (bm * 128 + sa) + stages * (bn * 128 + sb) + row_group_bytes();
        }
        if (variant == 2) return k / 128 / splitk * (bm * 128 + (bm + 63) / 64 * 256) + 3 * 256;
        if (variant == 5) return stages * (bm * 128 + bm * 4 + 256);   // A ring: tile, A scales, B scales
        if (variant == 3) {   // as many ring slots as fit (at most 16), see the kernel
            const int slot = bm * 128 + (bm + 63) / 64 * 256;
            const int slots = std::min(16, (160 * 1024 - 1024 - 768) / slot);
            return 768 + slots * slot;
        }
        return stages * stage_bytes() + row_group_bytes();
    }
    std::string key() const;
};

struct Problem {
    int kind;
    int rows;      // M (dense, contiguous) or M_max (masked)
    int n, k, g;
    int has_c;
    int sf = 0;    // scale format: as KernelConfig::sf
    int kt = 0;    // K-grouped: K rows of the operands (n, k above: N and the padded pitch)
    int a_k_outer = 0, b_k_outer = 0;   // A stored [K][rows] (T), B stored [(G)][K][N] (N)
};

// Tile heuristics (heuristics.cpp): the launches of one call, in order (one,
// or two over disjoint column ranges).
std::vector<KernelConfig> select_plan(const Problem& p, int num_cus);
// Output tiles times splits, i.e. the launch's work items; for masked the
// worst case (every row of every group valid).
int64_t num_work_items(const KernelConfig& c, int rows);

// JIT (jit.cpp).  compile_code() needs no GPU; get_function() loads on the
// current device (the GEMM kernel, or another kernel of the same module).
dg_status compile_code(const KernelConfig& c, std::vector<char>* code);
// DG_JIT_EXTRA_OPTION (one more hipRTC option), part of every cache key
std::string jit_extra_option();
dg_status get_function(const KernelConfig& c, void** function /* hipFunction_t */,
                       const char* name = "dg_fp8_gemm_nt_kernel");

// K-grouped operands are rewritten K-contiguous with this row pitch (the
// compile-time K of the kernels; a new pitch means a new compile)
inline int k_grouped_pitch(int k) { return (k + 1023) / 1024 * 1024; }
std::string cache_dir();

// Device address of the library's status words on the current device
// (device.hip); [0] counts bounded waits in the kernels that gave up.
dg_status status_words(unsigned int** out);

// Split-K arrival counters of a launch of `items` work items: one per output
// tile and computing wave (each wave hands off its own slice of the tile), each
// alone in a 128-byte line (the kernel's CTR_STRIDE of 32 words).
constexpr size_t kCounterStrideBytes = 128;
inline size_t split_k_counter_bytes(const KernelConfig& c, int items) {
    return (size_t)(items / c.splitk) * (size_t)(c.wm * c.wn) * kCounterStrideBytes;
}

// Scratch of dg_fp8_gemm_nt_noalloc (device.hip): a static device array of
// split-K partial sums followed by arrival counters, one copy per device.
constexpr size_t kScratchPartialBytes = size_t(32) << 20;
constexpr size_t kScratchCounterBytes = size_t(256) << 10;
// its device address on the current device (hipGetSymbolAddress)
dg_status scratch_address(void** out);
// zero n words at p on the stream with a small kernel (no memset node, so the
// call can be captured in a graph)
dg_status clear_words(uint32_t* p, int n, void* stream);

// Errors (api.cpp).
dg_status set_error(dg_status s, const std::string& msg);
bool env_flag(const char* name);

}  // namespace dg
