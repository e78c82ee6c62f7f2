// The C ABI of libdg.so: argument checks, tile selection, JIT lookup,
// workspace management and the kernel launch.  The operations and their
// layouts are specified in include/dg.h.
#include <algorithm>
#include <climits>
#include <cstddef>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <atomic>
#include <mutex>
#include <string>
#include <tuple>

#include <hip/hip_runtime.h>

#include "dg_internal.h"

namespace dg {

namespace {

thread_local std::string t_last_error;

// The kernel's arguments, in order.
struct LaunchParams {
    const void* A;
    const void* sfa;
    const void* B;
    const void* sfb;
    const float* C;
    void* D;
    const int32_t* grp;
    float* ws;
    uint32_t* counters;
    int M;
    int num_tiles;
    int kt;
    unsigned int* status;
};
// The GEMM kernel takes these fields as its one by-value argument (KernArgs in
// the kernel source, same layout): one launch argument instead of thirteen.
static_assert(sizeof(LaunchParams) == 96 && offsetof(LaunchParams, M) == 72 && offsetof(LaunchParams, status) == 88,
              "the kernel reads this layout");

struct Workspace {
    float* partials = nullptr;
    size_t partial_bytes = 0;
    uint32_t* counters = nullptr;
    size_t counter_bytes = 0;
    uint8_t* kmajor = nullptr;       // K-grouped operands rewritten K-contiguous
    size_t kmajor_bytes = 0;
    // Buffers a larger call outgrew.  They stay allocated until the process ends:
    // a HIP graph captured earlier still holds their addresses.
    std::vector<void*> retired;
};

// One kernel launch of a call.
struct Segment {
    KernelConfig cfg;
    hipFunction_t fn = nullptr;
    int grid = 0;
    int64_t items = 0;
};
// Everything a call needs besides the pointers, computed once per shape: its
// launches in order (two when the columns are split between tile widths).
struct Plan {
    std::vector<Segment> segs;
    hipFunction_t transpose = nullptr;   // K-grouped: the K-contiguous rewrite of the operands
};

using PlanKey = std::tuple<int, int, int, int, int, int, int, int, std::string>;

struct DeviceState {
    int num_cus = 0;
    unsigned int* status = nullptr;   // the device's status words (device.hip)
    void* scratch = nullptr;          // the device's copy of the no-alloc entry point's scratch (device.hip)
    std::map<hipStream_t, Workspace> ws;
    std::map<PlanKey, Plan> plans;
};

std::mutex g_mu;
std::map<int, DeviceState> g_dev;
std::atomic<int> g_num_cus_limit{0};   // 0: use the device's count

// The calling thread's previous call, kept so that a repeated call (same sizes,
// format, device, stream, CU limit and configuration environment) launches
// without the lock, the plan lookup or any allocation.  Plans live in std::map
// nodes that are never erased, and workspaces a call outgrows are retired, not
// freed, so the pointers stay valid.
struct WarmCall {
    int kind = -1, rows = 0, n = 0, k = 0, g = 0, has_c = 0, sf = 0, dev = -1, limit = 0;
    uint64_t env = 0;
    hipStream_t stream = nullptr;
    const Plan* plan = nullptr;
    float* partials = nullptr;       // split-K workspace of the plan's launches on this stream
    uint32_t* counters = nullptr;
    unsigned int* status = nullptr;
};
thread_local WarmCall t_warm;

dg_status hip_fail(hipError_t e, const char* what);

uint64_t fnv1a_str(const char* s, uint64_t h) {
    if (!s) return h ^ 0x9e37u;
    for (; *s; ++s) h = (h ^ (unsigned char)*s) * 1099511628211ull;
    return h;
}

// Launches of one plan, in order (they share the split-K workspace: each leaves
// its arrival counters at zero).
dg_status launch_segments(const Plan& plan, const Problem& p, const void* A, const void* sfa, const void* B,
                          const void* sfb, const int32_t* grp, const float* C, void* D, hipStream_t stream,
                          float* partials, uint32_t* counters, unsigned int* status) {
    for (const Segment& seg : plan.segs) {
        const KernelConfig& cfg = seg.cfg;
        if (seg.items <= 0) continue;
        LaunchParams lp{};
        lp.A = A; lp.sfa = sfa; lp.B = B; lp.sfb = sfb; lp.C = C; lp.D = D; lp.grp = grp;
        lp.M = p.rows;
        lp.num_tiles = (int)seg.items;
        lp.kt = p.kt;
        lp.status = status;
        if (cfg.splitk > 1) {
            lp.ws = partials;
            lp.counters = counters;
        }
        void* args[] = {&lp};
        hipError_t e = hipModuleLaunchKernel(seg.fn, seg.grid, 1, 1, cfg.threads(), 1, 1, 0, stream, args, nullptr);
        if (e != hipSuccess) return hip_fail(e, "hipModuleLaunchKernel");
    }
    return DG_OK;
}

dg_status hip_fail(hipError_t e, const char* what) {
    return set_error(DG_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

dg_status device_state(DeviceState** out, int* dev_out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    auto& st = g_dev[dev];
    if (st.num_cus == 0) {
        int n = 0;
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(MultiprocessorCount)");
        st.num_cus = n;
    }
    if (!st.status) {
        dg_status s = status_words(&st.status);
        if (s != DG_OK) return s;
    }
    if (!st.scratch) {
        // set-up, once per device, with the device current: the device address
        // of the static scratch array (the host-side symbol is not it)
        dg_status s = scratch_address(&st.scratch);
        if (s != DG_OK) return s;
    }
    *out = &st;
    *dev_out = dev;
    return DG_OK;
}

int effective_cus(const DeviceState& st) {
    const int limit = g_num_cus_limit.load();
    if (limit > 0 && limit < st.num_cus) return limit;
    return st.num_cus;
}

// Grow (never shrink) the stream's workspace, at least doubling it.  An outgrown
// buffer is retired, not freed, so graphs that captured it stay valid.  New
// arrival counters start at zero; kernels leave them at zero again when they finish.
dg_status ensure_workspace(DeviceState& st, hipStream_t stream, size_t partial_bytes, size_t counter_bytes,
                           Workspace** out) {
    Workspace& w = st.ws[stream];
    if (w.partial_bytes < partial_bytes) {
        if (w.partials) w.retired.push_back(w.partials);
        w.partials = nullptr;
        size_t bytes = std::max({partial_bytes, size_t(8) << 20, 2 * w.partial_bytes});
        w.partial_bytes = 0;
        hipError_t e = hipMalloc((void**)&w.partials, bytes);
        if (e != hipSuccess) return hip_fail(e, "hipMalloc(split-K workspace)");
        w.partial_bytes = bytes;
    }
    if (w.counter_bytes < counter_bytes) {
        if (w.counters) w.retired.push_back(w.counters);
        w.counters = nullptr;
        size_t bytes = std::max({counter_bytes, size_t(64) << 10, 2 * w.counter_bytes});
        w.counter_bytes = 0;
        hipError_t e = hipMalloc((void**)&w.counters, bytes);
        if (e != hipSuccess) return hip_fail(e, "hipMalloc(split-K counters)");
        e = hipMemset(w.counters, 0, bytes);
        if (e != hipSuccess) return hip_fail(e, "hipMemset(split-K counters)");
        w.counter_bytes = bytes;
    }
    *out = &w;
    return DG_OK;
}

// Grow (never shrink) the stream's buffer for operands rewritten K-contiguous,
// retiring (not freeing) an outgrown one, as for the workspace above.
dg_status ensure_kmajor(DeviceState& st, hipStream_t stream, size_t need, uint8_t** out) {
    Workspace& w = st.ws[stream];
    if (w.kmajor_bytes < need) {
        if (w.kmajor) w.retired.push_back(w.kmajor);
        w.kmajor = nullptr;
        const size_t bytes = std::max(need, 2 * w.kmajor_bytes);
        w.kmajor_bytes = 0;
        hipError_t e = hipMalloc((void**)&w.kmajor, bytes);
        if (e != hipSuccess) return hip_fail(e, "hipMalloc(K-contiguous operands)");
        w.kmajor_bytes = bytes;
    }
    *out = w.kmajor;
    return DG_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

dg_status check_common(const void* A, const void* sfa, const void* B, const void* sfb, const float* C,
                       const void* D, int rows, int N, int K, size_t sf_align = 4) {
    if (!A || !sfa || !B || !sfb || !D) return set_error(DG_ERR_INVALID_ARG, "A, sfa, B, sfb and D must be non-NULL");
    if (rows < 0 || N <= 0 || K <= 0)
        return set_error(DG_ERR_INVALID_ARG, "sizes must be positive (M may be 0)");
    if (K % 128 != 0) return set_error(DG_ERR_UNSUPPORTED, "K must be a multiple of 128 (the scale block)");
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16) || (C && !aligned(C, 16)))
        return set_error(DG_ERR_ALIGNMENT, "A, B, C and D must be 16-byte aligned");
    if (!aligned(sfa, sf_align) || !aligned(sfb, sf_align))
        return set_error(DG_ERR_ALIGNMENT, sf_align == 4 ? "scales must be 4-byte aligned"
                                                         : "16-bit scale words must be 2-byte aligned");
    // per-tile buffer offsets are 32-bit: one scale plane of A and one 256-row slab must fit
    if ((uint64_t)(K / 128) * (uint64_t)rows * 4u >= (1ull << 32) || (uint64_t)K * 256u >= (1ull << 32))
        return set_error(DG_ERR_UNSUPPORTED, "sizes exceed 32-bit buffer offsets");
    return DG_OK;
}

// noalloc: the plan must already be loaded on the device (no compile, no module
// load), split-K partials and counters go to the library's static scratch array
// instead of the stream's workspace, and nothing is allocated.
dg_status launch(const Problem& p, const void* A, const void* sfa, const void* B, const void* sfb,
                 const int32_t* grp, const float* C, void* D, void* stream_ptr, bool noalloc = false) {
    hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
    const bool rewrite = p.kind == kKGrouped || p.a_k_outer || p.b_k_outer;
    // ---- warm call: the previous call of this thread had the same key
    int dev_now = 0;
    if (hipGetDevice(&dev_now) != hipSuccess) dev_now = -1;
    const uint64_t env = fnv1a_str(std::getenv("DG_JIT_EXTRA_OPTION"),
                                   fnv1a_str(std::getenv("DG_FORCE_CONFIG"), 14695981039346656037ull));
    const int limit = g_num_cus_limit.load(std::memory_order_relaxed);
    WarmCall& w = t_warm;
    if (!noalloc && !rewrite && w.plan && w.kind == p.kind && w.rows == p.rows && w.n == p.n && w.k == p.k &&
        w.g == p.g && w.has_c == p.has_c && w.sf == p.sf && w.dev == dev_now && w.stream == stream &&
        w.env == env && w.limit == limit)
        return launch_segments(*w.plan, p, A, sfa, B, sfb, grp, C, D, stream, w.partials, w.counters, w.status);
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState* st = nullptr;
    int dev = 0;
    dg_status s = device_state(&st, &dev);
    if (s != DG_OK) return s;
    const int cus = effective_cus(*st);
    const char* forced = std::getenv("DG_FORCE_CONFIG");
    PlanKey key{p.kind, p.rows, p.n, p.k, p.g, p.has_c, p.sf, cus,
                std::string(forced ? forced : "") + "|" + jit_extra_option()};
    auto it = st->plans.find(key);
    if (noalloc) {
        if (it == st->plans.end())
            return set_error(DG_ERR_UNSUPPORTED,
                             "dg_fp8_gemm_nt_noalloc: the kernels for these sizes are not loaded on this device; "
                             "call dg_fp8_gemm_nt once with the same M, N, K and C presence first");
        size_t partial_bytes = 0, counter_bytes = 0;
        for (const Segment& seg : it->second.segs) {
            if (seg.cfg.splitk <= 1 || seg.items <= 0) continue;
            partial_bytes = std::max(partial_bytes, (size_t)seg.items * seg.cfg.bm * seg.cfg.bn * sizeof(float));
            counter_bytes = std::max(counter_bytes, split_k_counter_bytes(seg.cfg, seg.items));
        }
        if (partial_bytes > kScratchPartialBytes || counter_bytes > kScratchCounterBytes)
            return set_error(DG_ERR_UNSUPPORTED,
                             "dg_fp8_gemm_nt_noalloc: this shape's split-K needs " + std::to_string(partial_bytes) +
                                 " bytes of partial sums and " + std::to_string(counter_bytes) +
                                 " of counters, more than the scratch holds (" +
                                 std::to_string(kScratchPartialBytes) + " and " +
                                 std::to_string(kScratchCounterBytes) + ")");
        float* partials = static_cast<float*>(st->scratch);
        uint32_t* counters = reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(st->scratch) +
                                                         kScratchPartialBytes);
        if (counter_bytes > 0) {
            // the array keeps the last call's contents: its arrival counters start at zero here
            s = clear_words(counters, (int)(counter_bytes / sizeof(uint32_t)), stream);
            if (s != DG_OK) return s;
        }
        for (const Segment& seg : it->second.segs) {
            const KernelConfig& cfg = seg.cfg;
            if (seg.items <= 0) continue;
            LaunchParams lp{};
            lp.A = A; lp.sfa = sfa; lp.B = B; lp.sfb = sfb; lp.C = C; lp.D = D; lp.grp = grp;
            lp.M = p.rows;
            lp.num_tiles = (int)seg.items;
            lp.kt = p.kt;
            lp.status = st->status;
            if (cfg.splitk > 1) {
                lp.ws = partials;
                lp.counters = counters;
            }
            void* args[] = {&lp};
            hipError_t e = hipModuleLaunchKernel(seg.fn, seg.grid, 1, 1, cfg.threads(), 1, 1, 0, stream, args,
                                                 nullptr);
            if (e != hipSuccess) return hip_fail(e, "hipModuleLaunchKernel");
        }
        return DG_OK;
    }
    if (it == st->plans.end()) {
        Plan plan;
        for (const KernelConfig& c : select_plan(p, cus)) {
            Segment seg;
            seg.cfg = c;
            void* fptr = nullptr;
            s = get_function(c, &fptr);
            if (s != DG_OK) return s;
            seg.fn = static_cast<hipFunction_t>(fptr);
            seg.items = num_work_items(c, p.rows);
            if (seg.items > INT_MAX) return set_error(DG_ERR_UNSUPPORTED, "too many tiles");
            int occ = 1;
            if (hipModuleOccupancyMaxActiveBlocksPerMultiprocessor(&occ, seg.fn, c.threads(), 0) != hipSuccess ||
                occ < 1)
                occ = 1;
            seg.grid = (int)std::min<int64_t>(seg.items, (int64_t)cus * occ);
            plan.segs.push_back(seg);
        }
        it = st->plans.emplace(key, plan).first;
    }
    if (rewrite && !it->second.transpose) {
        void* fptr = nullptr;
        s = get_function(it->second.segs.front().cfg, &fptr, "dg_transpose_k_major");
        if (s != DG_OK) return s;
        it->second.transpose = static_cast<hipFunction_t>(fptr);
    }
    // rewrite of a K-outermost operand X [groups][rows_k][cols] as [groups][cols][pitch]
    // (one workgroup per 64 x 64 byte block, K blocks fastest; grid.z: groups)
    auto rewrite_k_major = [&](const void* x, void* xt, int rows_k, int cols, int groups) -> dg_status {
        const uint64_t blocks = (uint64_t)(rows_k / 64) * (uint64_t)((cols + 63) / 64);
        if (blocks >= (1ull << 31) || groups > 65535)
            return set_error(DG_ERR_UNSUPPORTED, "operand too large for the K-contiguous rewrite");
        if (blocks == 0) return DG_OK;
        void* args[] = {&x, &xt, &rows_k, &cols};
        hipError_t e = hipModuleLaunchKernel(it->second.transpose, (unsigned)blocks, 1, (unsigned)groups, 256, 1, 1, 0,
                                             stream, args, nullptr);
        return e == hipSuccess ? DG_OK : hip_fail(e, "hipModuleLaunchKernel(transpose)");
    };
    // TN / NN / TT layouts: the K-outermost operand(s) rewritten K-contiguous in the
    // stream's workspace, then the NT kernels run on them
    if (p.kind != kKGrouped && (p.a_k_outer || p.b_k_outer)) {
        const size_t a_bytes = p.a_k_outer ? (size_t)p.rows * (size_t)p.k : 0;
        const size_t b_bytes = p.b_k_outer ? (size_t)p.g * (size_t)p.n * (size_t)p.k : 0;
        uint8_t* buf = nullptr;
        s = ensure_kmajor(*st, stream, a_bytes + b_bytes, &buf);
        if (s != DG_OK) return s;
        if (p.a_k_outer) {
            s = rewrite_k_major(A, buf, p.k, p.rows, 1);
            if (s != DG_OK) return s;
            A = buf;
        }
        if (p.b_k_outer) {
            s = rewrite_k_major(B, buf + a_bytes, p.k, p.n, p.g);
            if (s != DG_OK) return s;
            B = buf + a_bytes;
        }
    }
    // K-grouped: rewrite A [kt][M] and B [kt][N] as [M][k] and [N][k] (k: the
    // padded pitch) in the stream's workspace; the GEMM reads those
    if (p.kind == kKGrouped) {
        uint8_t* buf = nullptr;
        s = ensure_kmajor(*st, stream, ((size_t)p.rows + (size_t)p.n) * (size_t)p.k, &buf);
        if (s != DG_OK) return s;
        uint8_t* at = buf;
        uint8_t* bt = buf + (size_t)p.rows * (size_t)p.k;
        s = rewrite_k_major(A, at, p.kt, p.rows, 1);
        if (s != DG_OK) return s;
        s = rewrite_k_major(B, bt, p.kt, p.n, 1);
        if (s != DG_OK) return s;
        A = at;
        B = bt;
    }
    // the split-K workspace the plan's launches need on this stream
    float* partials = nullptr;
    uint32_t* counters = nullptr;
    size_t need_p = 0, need_c = 0;
    for (const Segment& seg : it->second.segs) {
        if (seg.cfg.splitk <= 1 || seg.items <= 0) continue;
        need_p = std::max(need_p, (size_t)seg.items * seg.cfg.bm * seg.cfg.bn * sizeof(float));
        need_c = std::max(need_c, split_k_counter_bytes(seg.cfg, seg.items));
    }
    if (need_p > 0) {
        Workspace* ws = nullptr;
        s = ensure_workspace(*st, stream, need_p, need_c, &ws);
        if (s != DG_OK) return s;
        partials = ws->partials;
        counters = ws->counters;
    }
    const bool print = env_flag("DG_PRINT_CONFIGS");
    if (print)
        for (const Segment& seg : it->second.segs)
            std::fprintf(stderr, "[dg] launch %s grid=%d block=%d items=%lld lds=%d\n", seg.cfg.key().c_str(),
                         seg.grid, seg.cfg.threads(), (long long)seg.items, seg.cfg.lds_bytes());
    s = launch_segments(it->second, p, A, sfa, B, sfb, grp, C, D, stream, partials, counters, st->status);
    if (s != DG_OK) return s;
    if (!rewrite && !print) {
        WarmCall& r = t_warm;
        r.kind = p.kind; r.rows = p.rows; r.n = p.n; r.k = p.k; r.g = p.g; r.has_c = p.has_c; r.sf = p.sf;
        r.dev = dev; r.limit = limit; r.env = env; r.stream = stream; r.plan = &it->second;
        r.partials = partials; r.counters = counters; r.status = st->status;
    }
    return DG_OK;
}

}  // namespace

dg_status set_error(dg_status s, const std::string& msg) {
    t_last_error = msg;
    if (env_flag("DG_DEBUG")) std::fprintf(stderr, "[dg] error %d: %s\n", (int)s, msg.c_str());
    return s;
}

bool env_flag(const char* name) {
    const char* v = std::getenv(name);
    return v && *v && std::strcmp(v, "0") != 0;
}

}  // namespace dg

using namespace dg;

namespace {

// The three forms, for each scale format (sf: 0 FP32, 1 packed UE8M0, 2 FP8 x
// FP4 with E2M1 B; the scale pointers are only passed through to the kernel).
dg_status dense(const void* A, const void* sfa, const void* B, const void* sfb, const float* C, void* D, int M,
                int N, int K, int sf, void* stream, int a_k_outer = 0, int b_k_outer = 0) {
    dg_status s = check_common(A, sfa, B, sfb, C, D, M, N, K, sf == 5 ? 2 : 4);
    if (s != DG_OK) return s;
    if (M == 0) return DG_OK;
    Problem p{kDense, M, N, K, 1, C ? 1 : 0, sf};
    p.a_k_outer = a_k_outer;
    p.b_k_outer = b_k_outer;
    return launch(p, A, sfa, B, sfb, nullptr, C, D, stream);
}

dg_status contiguous(const void* A, const void* sfa, const void* B, const void* sfb, const int32_t* m_indices,
                     const float* C, void* D, int M, int N, int K, int num_groups, int sf, void* stream,
                     int b_k_outer = 0) {
    dg_status s = check_common(A, sfa, B, sfb, C, D, M, N, K, sf == 5 ? 2 : 4);
    if (s != DG_OK) return s;
    if (!m_indices) return set_error(DG_ERR_INVALID_ARG, "m_indices must be non-NULL");
    if (num_groups <= 0) return set_error(DG_ERR_INVALID_ARG, "num_groups must be positive");
    if (!aligned(m_indices, 4)) return set_error(DG_ERR_ALIGNMENT, "m_indices must be 4-byte aligned");
    if (M % dg_get_mk_alignment_for_contiguous_layout() != 0)
        return set_error(DG_ERR_ALIGNMENT, "contiguous M must be a multiple of the M alignment (128)");
    if (M == 0) return DG_OK;
    Problem p{kContiguous, M, N, K, num_groups, C ? 1 : 0, sf};
    p.b_k_outer = b_k_outer;
    return launch(p, A, sfa, B, sfb, m_indices, C, D, stream);
}

dg_status masked(const void* A, const void* sfa, const void* B, const void* sfb, const int32_t* masked_m,
                 const float* C, void* D, int M_max, int N, int K, int num_groups, int sf, void* stream) {
    dg_status s = check_common(A, sfa, B, sfb, C, D, M_max, N, K, sf == 5 ? 2 : 4);
    if (s != DG_OK) return s;
    if (!masked_m) return set_error(DG_ERR_INVALID_ARG, "masked_m must be non-NULL");
    if (num_groups <= 0) return set_error(DG_ERR_INVALID_ARG, "num_groups must be positive");
    if (!aligned(masked_m, 4)) return set_error(DG_ERR_ALIGNMENT, "masked_m must be 4-byte aligned");
    if (M_max == 0) return DG_OK;
    Problem p{kMasked, M_max, N, K, num_groups, C ? 1 : 0, sf};
    return launch(p, A, sfa, B, sfb, masked_m, C, D, stream);
}

// BF16 x BF16, the three M forms: no scales; the kernels count K in bytes
dg_status bf16_gemm(int kind, const void* A, const void* B, const int32_t* grp, const float* C, void* D, int rows,
                    int N, int K, int num_groups, void* stream) {
    if (!A || !B || !D) return set_error(DG_ERR_INVALID_ARG, "A, B and D must be non-NULL");
    if (rows < 0 || N <= 0 || K <= 0) return set_error(DG_ERR_INVALID_ARG, "sizes must be positive (M may be 0)");
    if (K % 64 != 0) return set_error(DG_ERR_UNSUPPORTED, "BF16: K must be a multiple of 64 (one 128-byte block)");
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16) || (C && !aligned(C, 16)))
        return set_error(DG_ERR_ALIGNMENT, "A, B, C and D must be 16-byte aligned");
    if ((uint64_t)K * 2u * 256u >= (1ull << 32)) return set_error(DG_ERR_UNSUPPORTED, "sizes exceed 32-bit buffer offsets");
    if (kind != kDense) {
        if (!grp) return set_error(DG_ERR_INVALID_ARG, "m_indices / masked_m must be non-NULL");
        if (num_groups <= 0) return set_error(DG_ERR_INVALID_ARG, "num_groups must be positive");
        if (!aligned(grp, 4)) return set_error(DG_ERR_ALIGNMENT, "m_indices / masked_m must be 4-byte aligned");
    }
    if (kind == kContiguous && rows % dg_get_mk_alignment_for_contiguous_layout() != 0)
        return set_error(DG_ERR_ALIGNMENT, "contiguous M must be a multiple of the M alignment (128)");
    if (rows == 0) return DG_OK;
    Problem p{kind, rows, N, 2 * K, kind == kDense ? 1 : num_groups, C ? 1 : 0, 3};
    return launch(p, A, nullptr, B, nullptr, grp, C, D, stream);
}

dg_status k_grouped(const void* A, const float* sfa, const void* B, const float* sfb, const int32_t* ks,
                    const float* C, void* D, int M, int N, int K, int num_groups, void* stream) {
    dg_status s = check_common(A, sfa, B, sfb, C, D, M, N, K);
    if (s != DG_OK) return s;
    if (!ks) return set_error(DG_ERR_INVALID_ARG, "ks must be non-NULL");
    if (num_groups <= 0) return set_error(DG_ERR_INVALID_ARG, "num_groups must be positive");
    if (!aligned(ks, 4)) return set_error(DG_ERR_ALIGNMENT, "ks must be 4-byte aligned");
    const int pitch = k_grouped_pitch(K);
    // the K-contiguous operands are addressed with 32-bit offsets per 256-row slab, the
    // B scales as one buffer
    if ((uint64_t)pitch * 256u >= (1ull << 32) || (uint64_t)(K / 128) * (uint64_t)N * 4u >= (1ull << 32))
        return set_error(DG_ERR_UNSUPPORTED, "sizes exceed 32-bit buffer offsets");
    if (M == 0) return DG_OK;
    Problem p{kKGrouped, M, N, pitch, num_groups, C ? 1 : 0, 0};
    p.kt = K;
    return launch(p, A, sfa, B, sfb, ks, C, D, stream);
}

}  // namespace

extern "C" {

const char* dg_last_error(void) { return t_last_error.c_str(); }

int dg_get_mk_alignment_for_contiguous_layout(void) { return 128; }

dg_status dg_set_num_cus(int n) {
    std::lock_guard<std::mutex> lock(g_mu);
    g_num_cus_limit = n > 0 ? n : 0;
    return DG_OK;
}

int dg_get_num_cus(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState* st = nullptr;
    int dev = 0;
    const int limit = g_num_cus_limit.load();
    if (device_state(&st, &dev) != DG_OK) return limit > 0 ? limit : 0;
    return effective_cus(*st);
}

dg_status dg_init(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState* st = nullptr;
    int dev = 0;
    dg_status s = device_state(&st, &dev);
    if (s != DG_OK) return s;
    Workspace* w = nullptr;
    return ensure_workspace(*st, nullptr, 0, 0, &w);
}

dg_status dg_get_wait_giveups(unsigned int* count) {
    if (!count) return set_error(DG_ERR_INVALID_ARG, "count must be non-NULL");
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState* st = nullptr;
    int dev = 0;
    dg_status s = device_state(&st, &dev);
    if (s != DG_OK) return s;
    hipError_t e = hipMemcpy(count, st->status, sizeof(unsigned int), hipMemcpyDeviceToHost);
    return e == hipSuccess ? DG_OK : hip_fail(e, "hipMemcpy(status words)");
}

dg_status dg_reset_wait_giveups(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState* st = nullptr;
    int dev = 0;
    dg_status s = device_state(&st, &dev);
    if (s != DG_OK) return s;
    const unsigned int zero = 0;
    hipError_t e = hipMemcpy(st->status, &zero, sizeof(zero), hipMemcpyHostToDevice);
    return e == hipSuccess ? DG_OK : hip_fail(e, "hipMemcpy(status words)");
}

// Scale format encoded in `kind` by the DG_SCALE_* flags
int scale_format(int* kind) {
    const int sf = (*kind & DG_SCALE_UE8M0_I16) ? 5 : (*kind & DG_SCALE_FP4_FP4) ? 4 : (*kind & DG_BF16) ? 3
                 : (*kind & DG_SCALE_FP8_FP4) ? 2 : (*kind & DG_SCALE_UE8M0) ? 1 : 0;
    *kind &= ~(DG_SCALE_UE8M0 | DG_SCALE_FP8_FP4 | DG_BF16 | DG_SCALE_FP4_FP4 | DG_SCALE_UE8M0_I16);
    return sf;
}

// the kernels' K: BF16 rows are counted in bytes; K-grouped operands use the padded pitch
int kernel_k(int kind, int sf, int K) {
    if (sf == 3) return 2 * K;
    return kind == kKGrouped ? k_grouped_pitch(K) : K;
}

dg_status dg_precompile(int kind, int rows, int N, int K, int num_groups, int has_c, int num_cus) {
    const int sf = scale_format(&kind);
    if (kind < 0 || kind > 3 || rows <= 0 || N <= 0 || K <= 0 || num_groups <= 0)
        return set_error(DG_ERR_INVALID_ARG, "dg_precompile: bad arguments");
    if (K % (sf == 3 ? 64 : 128)) return set_error(DG_ERR_UNSUPPORTED, "K must be a multiple of 128 (BF16: 64)");
    Problem p{kind, rows, N, kernel_k(kind, sf, K), kind == kDense ? 1 : num_groups, has_c ? 1 : 0, sf};
    for (const KernelConfig& cfg : select_plan(p, num_cus > 0 ? num_cus : 256)) {
        std::vector<char> code;
        dg_status s = compile_code(cfg, &code);
        if (s != DG_OK) return s;
    }
    return DG_OK;
}

dg_status dg_describe_config(int kind, int rows, int N, int K, int num_groups, int has_c, int num_cus, char* buf,
                             int len) {
    const int sf = scale_format(&kind);
    if (kind < 0 || kind > 3 || rows <= 0 || N <= 0 || K <= 0 || num_groups <= 0 || !buf || len <= 0)
        return set_error(DG_ERR_INVALID_ARG, "dg_describe_config: bad arguments");
    if (K % (sf == 3 ? 64 : 128)) return set_error(DG_ERR_UNSUPPORTED, "K must be a multiple of 128 (BF16: 64)");
    int cus = num_cus;
    if (cus <= 0) {
        std::lock_guard<std::mutex> lock(g_mu);
        DeviceState* st = nullptr;
        int dev = 0;
        dg_status s = device_state(&st, &dev);
        if (s != DG_OK) return s;
        cus = effective_cus(*st);
    }
    Problem p{kind, rows, N, kernel_k(kind, sf, K), kind == kDense ? 1 : num_groups, has_c ? 1 : 0, sf};
    std::string key;
    for (const KernelConfig& c : select_plan(p, cus)) key += (key.empty() ? "" : "+") + c.key();
    std::snprintf(buf, (size_t)len, "%s", key.c_str());
    return DG_OK;
}

dg_status dg_fp8_gemm_nt(const void* A, const float* sfa, const void* B, const float* sfb, const float* C, void* D,
                         int M, int N, int K, void* stream) {
    return dense(A, sfa, B, sfb, C, D, M, N, K, 0, stream);
}

dg_status dg_fp8_gemm_nt_noalloc(const void* A, const float* sfa, const void* B, const float* sfb, const float* C,
                                 void* D, int M, int N, int K, void* stream) {
    dg_status s = check_common(A, sfa, B, sfb, C, D, M, N, K);
    if (s != DG_OK) return s;
    if (M == 0) return DG_OK;
    Problem p{kDense, M, N, K, 1, C ? 1 : 0, 0};
    return launch(p, A, sfa, B, sfb, nullptr, C, D, stream, true);
}

dg_status dg_m_grouped_fp8_gemm_nt_contiguous(const void* A, const float* sfa, const void* B, const float* sfb,
                                              const int32_t* m_indices, const float* C, void* D, int M, int N, int K,
                                              int num_groups, void* stream) {
    return contiguous(A, sfa, B, sfb, m_indices, C, D, M, N, K, num_groups, 0, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_masked(const void* A, const float* sfa, const void* B, const float* sfb,
                                          const int32_t* masked_m, const float* C, void* D, int M_max, int N, int K,
                                          int num_groups, void* stream) {
    return masked(A, sfa, B, sfb, masked_m, C, D, M_max, N, K, num_groups, 0, stream);
}

dg_status dg_fp8_gemm_nt_ue8m0(const void* A, const int32_t* sfa, const void* B, const int32_t* sfb, const float* C,
                               void* D, int M, int N, int K, void* stream) {
    return dense(A, sfa, B, sfb, C, D, M, N, K, 1, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(const void* A, const int32_t* sfa, const void* B,
                                                    const int32_t* sfb, const int32_t* m_indices, const float* C,
                                                    void* D, int M, int N, int K, int num_groups, void* stream) {
    return contiguous(A, sfa, B, sfb, m_indices, C, D, M, N, K, num_groups, 1, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_masked_ue8m0(const void* A, const int32_t* sfa, const void* B,
                                                const int32_t* sfb, const int32_t* masked_m, const float* C,
                                                void* D, int M_max, int N, int K, int num_groups, void* stream) {
    return masked(A, sfa, B, sfb, masked_m, C, D, M_max, N, K, num_groups, 1, stream);
}

dg_status dg_fp8_gemm_nt_ue8m0_i16(const void* A, const int16_t* sfa, const void* B, const int16_t* sfb,
                                   const float* C, void* D, int M, int N, int K, void* stream) {
    return dense(A, sfa, B, sfb, C, D, M, N, K, 5, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0_i16(const void* A, const int16_t* sfa, const void* B,
                                                        const int16_t* sfb, const int32_t* m_indices, const float* C,
                                                        void* D, int M, int N, int K, int num_groups, void* stream) {
    return contiguous(A, sfa, B, sfb, m_indices, C, D, M, N, K, num_groups, 5, stream);
}

dg_status dg_m_grouped_fp8_gemm_nt_masked_ue8m0_i16(const void* A, const int16_t* sfa, const void* B,
                                                    const int16_t* sfb, const int32_t* masked_m, const float* C,
                                                    void* D, int M_max, int N, int K, int num_groups, void* stream) {
    return masked(A, sfa, B, sfb, masked_m, C, D, M_max, N, K, num_groups, 5, stream);
}

dg_status dg_fp8_fp4_gemm_nt(const void* A, const int32_t* sfa, const void* B, const int32_t* sfb, const float* C,
                             void* D, int M, int N, int K, void* stream) {
    return dense(A, sfa, B, sfb, C, D, M, N, K, 2, stream);
}

dg_status dg_m_grouped_fp8_fp4_gemm_nt_contiguous(const void* A, const int32_t* sfa, const void* B,
                                                  const int32_t* sfb, const int32_t* m_indices, const float* C,
                                                  void* D, int M, int N, int K, int num_groups, void* stream) {
    return contiguous(A, sfa, B, sfb, m_indices, C, D, M, N, K, num_groups, 2, stream);
}

dg_status dg_m_grouped_fp8_fp4_gemm_nt_masked(const void* A, const int32_t* sfa, const void* B,
                                              const int32_t* sfb, const int32_t* masked_m, const float* C, void* D,
                                              int M_max, int N, int K, int num_groups, void* stream) {
    return masked(A, sfa, B, sfb, masked_m, C, D, M_max, N, K, num_groups, 2, stream);
}

dg_status dg_k_grouped_fp8_gemm_tn_contiguous(const void* A, const float* sfa, const void* B, const float* sfb,
                                              const int32_t* ks, const float* C, void* D, int M, int N, int K,
                                              int num_groups, void* stream) {
    return k_grouped(A, sfa, B, sfb, ks, C, D, M, N, K, num_groups, stream);
}

// Layout letters: the first says how A is stored (N [M][K], T [K][M]), the
// second how B is (T [N][K], N [K][N]); the K-outermost ones are rewritten.
dg_status dg_fp8_gemm_nn(const void* A, const float* sfa, const void* B, const float* sfb, const float* C, void* D,
                         int M, int N, int K, void* stream) {
    return dense(A, sfa, B, sfb, C, D, M, N, K, 0, stream, 0, 1);
}

dg_status dg_fp8_gemm_tn(const void* A, const float* sfa, const void* B, const float* sfb, const float* C, void* D,
                         int M, int N, int K, void* stream) {
    return dense(A, sfa, B, sfb, C, D, M, N, K, 0, stream, 1, 1);
}

dg_status dg_fp8_gemm_tt(const void* A, const float* sfa, const void* B, const float* sfb, const float* C, void* D,
                         int M, int N, int K, void* stream) {
    return dense(A, sfa, B, sfb, C, D, M, N, K, 0, stream, 1, 0);
}

dg_status dg_m_grouped_fp8_gemm_nn_contiguous(const void* A, const float* sfa, const void* B, const float* sfb,
                                              const int32_t* m_indices, const float* C, void* D, int M, int N, int K,
                                              int num_groups, void* stream) {
    return contiguous(A, sfa, B, sfb, m_indices, C, D, M, N, K, num_groups, 0, stream, 1);
}

dg_status dg_bf16_gemm_nt(const void* A, const void* B, const float* C, void* D, int M, int N, int K, void* stream) {
    return bf16_gemm(kDense, A, B, nullptr, C, D, M, N, K, 1, stream);
}

dg_status dg_m_grouped_bf16_gemm_nt_contiguous(const void* A, const void* B, const int32_t* m_indices, const float* C,
                                               void* D, int M, int N, int K, int num_groups, void* stream) {
    return bf16_gemm(kContiguous, A, B, m_indices, C, D, M, N, K, num_groups, stream);
}

dg_status dg_m_grouped_bf16_gemm_nt_masked(const void* A, const void* B, const int32_t* masked_m, const float* C,
                                           void* D, int M_max, int N, int K, int num_groups, void* stream) {
    return bf16_gemm(kMasked, A, B, masked_m, C, D, M_max, N, K, num_groups, stream);
}

dg_status dg_fp4_fp4_gemm_nt(const void* A, const int32_t* sfa, const void* B, const int32_t* sfb, const float* C,
                             void* D, int M, int N, int K, void* stream) {
    return dense(A, sfa, B, sfb, C, D, M, N, K, 4, stream);
}

dg_status dg_m_grouped_fp4_fp4_gemm_nt_contiguous(const void* A, const int32_t* sfa, const void* B,
                                                  const int32_t* sfb, const int32_t* m_indices, const float* C,
                                                  void* D, int M, int N, int K, int num_groups, void* stream) {
    return contiguous(A, sfa, B, sfb, m_indices, C, D, M, N, K, num_groups, 4, stream);
}

dg_status dg_m_grouped_fp4_fp4_gemm_nt_masked(const void* A, const int32_t* sfa, const void* B,
                                              const int32_t* sfb, const int32_t* masked_m, const float* C, void* D,
                                              int M_max, int N, int K, int num_groups, void* stream) {
    return masked(A, sfa, B, sfb, masked_m, C, D, M_max, N, K, num_groups, 4, stream);
}

}  // extern "C"
