/* s2r_diag.h -- measurement helpers exported by libs2r.so (gfx950).  Not part of the
 * aggregation path: the benchmark uses them to put its figures next to what the GPU it
 * runs on achieves. */
#ifndef S2R_DIAG_H
#define S2R_DIAG_H

#include <stddef.h>
#include <stdint.h>

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

/* Fills `bytes` of device memory with `value` once -- 128-bit non-temporal stores, one
 * workgroup per 32 KiB, the store form of the decode's output pass -- on `stream`.  The
 * duration of the call, taken with events on that stream, gives the achievable HBM write
 * rate.  buf 16-byte aligned, bytes a multiple of 16.
 * Errors: S2R_ERR_NULL, S2R_ERR_ALIGN, S2R_ERR_DIM (more than 2^31 - 1 workgroups),
 * S2R_ERR_HIP. */
s2r_status s2r_diag_stream_write(void* buf, size_t bytes, float value, void* stream);

#define S2R_TRACE_MAX 64

/* Kernel-level timing with HIP events on the stream each kernel runs on.
 *   capacity  in: number of events[] the caller created (at most S2R_TRACE_MAX)
 *   count     in/out: events used so far (the caller sets it to 0 before a traced run)
 *   events    in: hipEvent_t handles created by the caller (timing enabled)
 *   names     out: names[i] = the kernel launched right after events[i] was recorded, or
 *             "end" for the event a call records after its last launch (static strings)
 * The time between events[i] and events[i + 1] is the duration of kernel names[i] (for
 * names[i] != "end"), measured on the stream the kernel was launched on. */
typedef struct {
  uint32_t capacity;
  uint32_t count;
  void* events[S2R_TRACE_MAX];
  const char* names[S2R_TRACE_MAX];
} s2r_trace;

/* Attaches `t` to the calling host thread, or detaches with t == NULL.  While attached,
 * every library call made from this thread records events[count] on its stream before
 * each kernel launch and once more after its last launch, advancing count, and records
 * nothing more once count reaches capacity.  Only this thread's calls are traced; `t` must
 * stay valid until it is detached.  Launches, results and other threads are unaffected.
 * Errors: S2R_ERR_DIM (capacity > S2R_TRACE_MAX or count > capacity). */
s2r_status s2r_diag_trace_attach(s2r_trace* t);

#ifdef __cplusplus
}
#endif

#endif /* S2R_DIAG_H */
