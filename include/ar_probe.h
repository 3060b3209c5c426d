/*
 * ar_probe.h -- streaming-bandwidth probe used by the benchmark as a calibration (libar_probe.so).
 * Not part of the all-reduce path: it moves the same streams as the fused kernels with no
 * arithmetic that matters, no row reduction and no rounding, to show what the memory system
 * delivers for that traffic pattern on this GPU.
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
 *   inputs : host array of nr device pointers (16-byte aligned), nr = 8 or 9
 *   nw     : 1 or 2 output streams (out1 is ignored for nw == 1)
 * Returns 0, 1 for a bad argument (nothing launched), 2 if the launch failed. */
int ar_probe_stream(const void* const* inputs, int nr, int nw, int64_t nvec, void* out0,
                    void* out1, int threads, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AR_PROBE_H */
