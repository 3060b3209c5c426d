/*
 * ar_probe.h -- the benchmark's probes (libar_probe.so), not part of the all-reduce library:
 *   ar_probe_stream  a streaming-bandwidth calibration: it moves the same streams as the fused
 *                    kernels with no arithmetic that matters, no row reduction and no rounding,
 *                    to show what the memory system delivers for that traffic pattern here;
 *   ar_probe_phases  where the time of a decode-size call goes: the library's kernels compiled
 *                    again with their phase hooks recording a clock per block and phase.
 */
#ifndef AR_PROBE_H
#define AR_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* For i < nvec: reads the 16-byte vector i of each of the `nr` input streams (non-temporal),
 * combines them with XOR and writes the result to out0[i] and, when nw == 2, out0[i] + 1 to
 * out1[i] (non-temporal stores).  One vector per thread, `threads` per block (a multiple of 64,
 * at most 1024), a grid that covers nvec.
 *   inputs : host array of nr device pointers (16-byte aligned), nr in {1, 2, 4, 8, 9, 16}
 *   nw     : 1 or 2 output streams (out1 is ignored for nw == 1)
 * Returns 0, 1 for a bad argument (nothing launched), 2 if the launch failed. */
int ar_probe_stream(const void* const* inputs, int nr, int nw, int64_t nvec, void* out0,
                    void* out1, int threads, void* stream);

/* Phase timing of one launch shape of the library's kernels (bfloat16, W in {2, 4, 8, 16}):
 * the kernel is captured `calls` times in a hipGraph over rotated buffer sets (the benchmark's
 * layout: each tensor role one allocation, enough sets to touch >= 512 MiB per replay) and the
 * graph replayed 6 times (the first untimed).  Thread 0 of every block stores the 100 MHz real-time
 * clock at each phase (after the value the phase produces is available).
 *   kind     : 0 kAllReduce sum kernel, 1 one-block-per-row kARResidualRMSNorm kernel, 2 split
 *              kernel (`segments` blocks per row), 3 an empty kernel (launch floor)
 *   threads, vpt, grid : the launch shape (vpt 1 or 2; split: grid = M * segments)
 *   out[0]   : µs per call (graph replay, events)      out[1] : kernel span, µs (first block's
 *              phase 0 to the last block's phase 7)     out[2] : gap to the next kernel, µs
 *   out[3..8]: phases 1..6, µs after the kernel's first phase 0 (latest block; -1 if none)
 *   out[9]   : rotation sets                           out[10] : calls per graph
 * Medians over every call of the 5 timed replays.  Returns 0, 1 for a bad argument, 2 for a HIP
 * error.  Allocates its buffers, so it is for measurement only. */
int ar_probe_phases(int kind, int W, int M, int H, int threads, int vpt, int grid, int segments,
                    double* out);

#ifdef __cplusplus
}
#endif

#endif /* AR_PROBE_H */
