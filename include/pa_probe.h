/*
 * pa_probe.h — HBM measurement kernels shipped in libpa.so.
 *
 * These are not part of the paged-attention method; they exist so that
 * bandwidth figures can be put next to what the memory system delivers to a
 * plain streaming kernel, and so that hardware byte counters can be
 * calibrated against a kernel whose traffic is known exactly.
 *
 * Both take device pointers, 16-byte aligned, and a byte count that is a
 * multiple of 16; they enqueue one kernel on `stream` and return.
 */
#ifndef PA_PROBE_H_
#define PA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` from src with 128-bit loads; a 16-byte checksum-like value per
 * workgroup is written to sink (sink must hold 16 * 2048 bytes) so the loads
 * cannot be elided. */
pa_status pa_probe_read(const void* src, size_t bytes, void* sink, void* stream);

/* Copy `bytes` from src to dst with 128-bit loads and stores. */
pa_status pa_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H_ */
