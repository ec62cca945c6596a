/*
 * slora_probe.h - bandwidth probes of libslora (measurement only).
 *
 * Not part of the LoRA delta: two plain kernels that read HBM the two ways the
 * delta does, so a benchmark can state what MI355X delivers for a launch of
 * the same size next to what the delta kernels reach.
 *
 *   slora_probe_read    one launch that streams `bytes` contiguous bytes, every
 *                       16-byte chunk read exactly once;
 *   slora_probe_gather  one launch that reads whole rows at the given row ids
 *                       of up to two row arrays (the page classes of a pool),
 *                       every listed row once, as the delta reads adapter pages.
 *
 * Both only read (the one store they contain depends on the data read and
 * never executes for finite data), are asynchronous on `stream`, and record
 * the caller's HIP events (hipEvent_t as void*, either may be NULL) from the
 * dispatch itself, like slora_lora_delta_timed.  Device pointers are
 * caller-owned and 16-byte aligned; byte counts are multiples of 16.
 * Errors: SLORA_E_INVAL on a bad argument, SLORA_E_HIP on a launch failure;
 * the message is in slora_last_error().
 */
#ifndef SLORA_PROBE_H
#define SLORA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "slora.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read src[0 .. bytes) once.  items: 16-byte loads each thread keeps in flight
 * (1, 2, 4, 8 or 16); nontemporal: 1 to read with the streaming hint.  sink:
 * device memory of at least 16 bytes (written only if the data hold an
 * impossible pattern). */
slora_status slora_probe_read(const void* src, int64_t bytes, int32_t items, int32_t nontemporal,
                              void* sink, void* stream, void* start_event, void* stop_event);

/* Read rows rows0[0 .. n0) of the array at base0 (rows of row_bytes0 bytes,
 * row i at base0 + i * stride0) and rows rows1[0 .. n1) of the array at base1
 * (n1 may be 0), in one launch, with the streaming hint.  rows0 and rows1 are
 * device arrays of int32 row ids; the caller guarantees that every id is in
 * range.  A workgroup reads whole rows, or one piece of a long row, so its
 * row ids are uniform.  items as for slora_probe_read: rows of up to items
 * 4 KB passes share a workgroup, longer rows take several.  n0, n1 and the
 * 16-byte chunks of a row must each stay below 2^31. */
slora_status slora_probe_gather(const void* base0, int64_t stride0, int64_t row_bytes0,
                                const int32_t* rows0, int64_t n0, const void* base1, int64_t stride1,
                                int64_t row_bytes1, const int32_t* rows1, int64_t n1, int32_t items,
                                void* sink, void* stream, void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* SLORA_PROBE_H */
