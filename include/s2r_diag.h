/* s2r_diag.h -- measurement helpers exported by libs2r.so (gfx950).  Not part of the
 * aggregation path: the benchmark uses them to put its figures next to what the GPU it
 * runs on achieves. */
#ifndef S2R_DIAG_H
#define S2R_DIAG_H

#include <stddef.h>

#include "s2r.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Streams `bytes` of device memory once -- 128-bit non-temporal loads, several in flight per
 * lane, the load form of the bitmap pass -- folds them into one value and writes it to *sink
 * (device memory), on `stream`.  The duration of the call, taken with events on that stream,
 * gives the achievable HBM read rate.  buf 16-byte aligned, bytes a multiple of 16.
 * Errors: S2R_ERR_NULL, S2R_ERR_ALIGN, S2R_ERR_HIP. */
s2r_status s2r_diag_stream_read(const void* buf, size_t bytes, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* S2R_DIAG_H */
