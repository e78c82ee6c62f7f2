// Device code built into libdg.so itself (hipcc, gfx950).  The GEMM kernels
// are not here: they are compiled per shape at run time (kernels/fp8_gemm.hip,
// hipRTC).  This file holds
//   * the library's status words, which every GEMM launch receives as a kernel
//     argument (the count of bounded waits that gave up), and
//   * measurement probes that put the GEMM timings in context: an empty
//     kernel (launch floor), a streaming read of a large buffer (the HBM read
//     rate this part reaches), back-to-back FP8 MFMAs (the matrix-core rate it
//     reaches under load) and a timed spin (keeps the GPU busy while the host
//     enqueues a timed launch).
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "dg_internal.h"
#include "dg_probe.h"

namespace dg {

// [0]: bounded waits (LDS flag waits of the producer/consumer kernel variant)
// that gave up before their flag was set.  Each device holds its own copy.
__device__ unsigned int g_status[4];

// Scratch of dg_fp8_gemm_nt_noalloc, the entry point for callers that cannot
// allocate: split-K partial sums (kScratchPartialBytes), then the arrival
// counters (kScratchCounterBytes).  Each device holds its own copy until the
// process ends; every call on a device shares it.  Host code must use the
// address hipGetSymbolAddress gives for it (scratch_address below), never the
// array's name.
static __device__ __align__(256) unsigned char scratch[kScratchPartialBytes + kScratchCounterBytes];

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ void dg_probe_null_kernel() {}

__global__ void __launch_bounds__(256) dg_clear_words_kernel(unsigned int* __restrict__ p, int n) {
    for (int i = (int)(blockIdx.x * 256u + threadIdx.x); i < n; i += (int)(gridDim.x * 256u)) p[i] = 0u;
}

// Every lane reads 16 bytes per step, four steps in flight, grid-stride over
// the buffer; the XOR of everything read is stored only if it equals a value it
// practically never has, so the loads cannot be dropped and nothing is written.
__global__ void __launch_bounds__(256) dg_probe_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                            unsigned int* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * 256u;
    size_t i = (size_t)blockIdx.x * 256u + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= src[i];
    const unsigned int x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x9e3779b9u) sink[blockIdx.x] = x;
}

// Eight independent accumulator chains of v_mfma_f32_16x16x128_f8f6f4 per
// wave (E4M3 x E4M3, 65536 FLOP each), eight waves per workgroup (two per
// SIMD), as in the GEMM's large tile.  The operands are arbitrary codes; only
// the time is used.
__global__ void __launch_bounds__(512) dg_probe_mfma_kernel(int iters, float* __restrict__ sink) {
    const int t = (int)threadIdx.x;
    const i32x8 a = {t, t + 1, t + 2, t + 3, t + 4, t + 5, t + 6, t + 7};
    const i32x8 b = {7 * t, 7 * t + 1, 7 * t + 2, 7 * t + 3, 7 * t + 4, 7 * t + 5, 7 * t + 6, 7 * t + 7};
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j], 0, 0, 0, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j].x + acc[j].y + acc[j].z + acc[j].w;
    if (s == 1.25e-30f) sink[blockIdx.x] = s;
}

// One wave that returns once `ticks` of the 100 MHz real-time counter have
// passed: queued ahead of a timed launch, it keeps the GPU busy while the host
// enqueues the launch and its events, so an event pair measures the launch
// alone and not the host's submission gap.
__global__ void dg_probe_spin_kernel(unsigned long long ticks) {
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

}  // namespace

dg_status status_words(unsigned int** out) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_status));
    if (e != hipSuccess)
        return set_error(DG_ERR_HIP, std::string("hipGetSymbolAddress(status words): ") + hipGetErrorString(e));
    *out = static_cast<unsigned int*>(p);
    return DG_OK;
}

dg_status scratch_address(void** out) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
        return set_error(DG_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    *out = ptr;
    return DG_OK;
}

dg_status clear_words(uint32_t* p, int n, void* stream) {
    if (n <= 0) return DG_OK;
    const int grid = (n + 255) / 256 < 64 ? (n + 255) / 256 : 64;
    hipLaunchKernelGGL(dg_clear_words_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), p, n);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? DG_OK : set_error(DG_ERR_HIP, std::string("clear_words: ") + hipGetErrorString(e));
}

}  // namespace dg

using namespace dg;

extern "C" {

dg_status dg_probe_null(int grid, void* stream) {
    if (grid <= 0) return set_error(DG_ERR_INVALID_ARG, "dg_probe_null: grid must be positive");
    hipLaunchKernelGGL(dg_probe_null_kernel, dim3(grid), dim3(64), 0, static_cast<hipStream_t>(stream));
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? DG_OK : set_error(DG_ERR_HIP, std::string("dg_probe_null: ") + hipGetErrorString(e));
}

dg_status dg_probe_spin(int microseconds, void* stream) {
    if (microseconds <= 0 || microseconds > 1000000)
        return set_error(DG_ERR_INVALID_ARG, "dg_probe_spin: microseconds must be in (0, 1e6]");
    hipLaunchKernelGGL(dg_probe_spin_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                       (unsigned long long)microseconds * 100ull);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? DG_OK : set_error(DG_ERR_HIP, std::string("dg_probe_spin: ") + hipGetErrorString(e));
}

dg_status dg_probe_stream_read(const void* src, size_t bytes, unsigned int* sink, int grid, void* stream) {
    if (!src || !sink || grid <= 0 || bytes == 0)
        return set_error(DG_ERR_INVALID_ARG, "dg_probe_stream_read: NULL pointer, empty buffer or no grid");
    if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0)
        return set_error(DG_ERR_ALIGNMENT, "dg_probe_stream_read: buffer must be 16-byte aligned and sized");
    hipLaunchKernelGGL(dg_probe_read_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), bytes / 16, sink);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? DG_OK
                           : set_error(DG_ERR_HIP, std::string("dg_probe_stream_read: ") + hipGetErrorString(e));
}

dg_status dg_probe_mfma_fp8(int grid, int iters, float* sink, void* stream) {
    if (!sink || grid <= 0 || iters <= 0)
        return set_error(DG_ERR_INVALID_ARG, "dg_probe_mfma_fp8: NULL sink, or grid or iterations not positive");
    hipLaunchKernelGGL(dg_probe_mfma_kernel, dim3(grid), dim3(512), 0, static_cast<hipStream_t>(stream), iters,
                       sink);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? DG_OK
                           : set_error(DG_ERR_HIP, std::string("dg_probe_mfma_fp8: ") + hipGetErrorString(e));
}

dg_status dg_probe_call_floor(const void*, const void*, const void*, const void*, const float*, void*, int, int, int,
                              void*) {
    return DG_OK;
}

}  // extern "C"
