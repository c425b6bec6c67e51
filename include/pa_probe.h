/*
 * pa_probe.h -- a measurement aid of libpa_mi355x.so: the rate at which this
 * GPU streams a large buffer out of HBM.
 *
 * Decode attention is memory-bound ("vLLM 与 PagedAttention"
 * (inference.mavenzero.com/case-studies/vllm), section 一: every generated
 * token reads the whole KV history again, with little arithmetic per byte),
 * so its kernels are judged by the HBM bandwidth they reach.  The nominal
 * peak is not reachable by any read stream; this probe measures what a plain
 * read of contiguous memory does reach, the practical ceiling next to which
 * a decode kernel's fraction of the peak is read.
 */
#ifndef PA_MI355X_PA_PROBE_H_
#define PA_MI355X_PA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pa_probe_stream_read -- read `bytes` of device memory at `src` once, with
 * 16-byte non-temporal loads, and store one 32-bit XOR of the words each
 * workgroup read to sink[workgroup] (the XOR over all of sink equals the XOR
 * of every 32-bit word of the buffer).
 *
 *   src         device memory, 16-byte aligned; bytes a positive multiple of 16
 *   sink        device memory of `workgroups` uint32 values, written in full
 *   workgroups  1 .. 2^20 workgroups of 256 threads
 *   mode        0: each workgroup reads one contiguous 1/workgroups share of
 *               the buffer; 1: the workgroups stride through the buffer in
 *               32 KiB steps (grid stride); 2: the buffer is read as 4 KiB
 *               blocks in a scattered order (logical block i is physical block
 *               i * 0x9E3779B1 modulo the block count), the access pattern of
 *               a paged pool -- bytes must then be 4 KiB times a power of two
 *
 * Enqueued on `stream`; time it with events around the call.  Errors:
 * PA_ERR_INVALID_ARG (null or misaligned pointer, size, count or mode out of
 * range; nothing is enqueued), PA_ERR_HIP (the launch failed).
 */
pa_status pa_probe_stream_read(const void *src, size_t bytes, uint32_t *sink, int workgroups, int mode,
                               void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_MI355X_PA_PROBE_H_ */
