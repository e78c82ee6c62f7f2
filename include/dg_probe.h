/*
 * dg_probe.h -- measurement probes exported by libdg.so.
 *
 * They compute nothing of the GEMM.  They put its timings in context: the
 * launch floor of an empty kernel, the HBM read rate this part reaches with a
 * plain streaming kernel, and the FP8 matrix-core rate it reaches with
 * back-to-back MFMAs, so that a GEMM's roofline fraction can be stated against
 * measured peaks as well as against the published ones (5.0 PFLOP/s dense FP8,
 * 8 TB/s HBM).  Calls are asynchronous on `stream` (a hipStream_t, NULL = the
 * default stream), validate their arguments first and return a dg_status
 * (message in dg_last_error()).  All pointers are caller-owned device memory.
 */
#ifndef DG_PROBE_H_
#define DG_PROBE_H_

#include <stddef.h>

#include "dg.h"

#ifdef __cplusplus
extern "C" {
#endif

/* An empty kernel: `grid` workgroups of one wave. */
dg_status dg_probe_null(int grid, void *stream);

/*
 * One wave that spins until `microseconds` (1 .. 10^6) of the device's
 * 100 MHz real-time counter have passed.  Queued ahead of an event pair and a
 * launch, it keeps the GPU busy while the host enqueues them, so the pair
 * times the launch and not the host's submission gap.
 */
dg_status dg_probe_spin(int microseconds, void *stream);

/*
 * Streaming read: `grid` workgroups of 256 lanes read all `bytes` of `src`
 * (16 bytes per lane and step, grid-stride) and combine them; `sink` must hold
 * `grid` words and is written only in the (practically impossible) case that
 * a workgroup's combination equals a fixed value.  `src` and `bytes` must be
 * multiples of 16.  Bytes read per launch: `bytes`.
 */
dg_status dg_probe_stream_read(const void *src, size_t bytes, unsigned int *sink, int grid, void *stream);

/*
 * FP8 MFMA rate: `grid` workgroups of eight waves, each wave issuing
 * 8 * iters dependent-in-eight-chains v_mfma_f32_16x16x128_f8f6f4 (E4M3 x
 * E4M3, 65536 FLOP each).  FLOPs per launch: grid * 8 * 8 * iters * 65536.
 * `sink` must hold `grid` floats and is written only in a practically
 * impossible case.
 */
dg_status dg_probe_mfma_fp8(int grid, int iters, float *sink, void *stream);

/*
 * Does nothing and returns DG_OK.  It takes the arguments of dg_fp8_gemm_nt,
 * so that timing calls of both through the same foreign-function layer (for
 * instance Python's ctypes) and subtracting gives the library's own host cost
 * of a call, without the cost of passing its arguments.
 */
dg_status dg_probe_call_floor(const void *A, const void *sfa, const void *B, const void *sfb, const float *C,
                              void *D, int M, int N, int K, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DG_PROBE_H_ */
