/*
 * libdblock measurement aid -- not a step of the decoding iteration.
 *
 * The iteration's large kernels are bound by how fast HBM can be read.  The
 * datasheet gives 8 TB/s; what a kernel can actually pull on the part is
 * lower.  This probe streams a buffer once with the load pattern the LM head
 * uses for its weight stream (16-byte loads, each wave instruction covering
 * 1 KiB of contiguous bytes, i.e. whole 128-byte lines), so the benchmark can
 * report achieved bandwidth against a measured read ceiling beside the
 * datasheet peak.
 *
 * dblk_probe_read
 *   buf          device pointer, 16-byte aligned, `bytes` readable bytes
 *   bytes        multiple of 32768, > 0
 *   nontemporal  nonzero: loads carry the streaming (nontemporal) hint
 *   grid         workgroups (256 threads each), 1 <= grid <= 65535; each
 *                workgroup reads 32 KiB per trip, grid-strided over the buffer
 *   sink         device uint32 [grid * 256] out: an XOR of the data read (it
 *                keeps the loads from being optimised away; its value is
 *                meaningless)
 *   stream       hipStream_t (NULL = null stream)
 * Returns a dblk_status code (include/dblock.h); validation happens before
 * any launch, as for every other call.
 */
#ifndef DBLOCK_PROBE_H_
#define DBLOCK_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int32_t dblk_probe_read(const void *buf, size_t bytes, int32_t nontemporal, int32_t grid,
                        uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DBLOCK_PROBE_H_ */
