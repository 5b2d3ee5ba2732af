/*
 * libkvq2 read-bandwidth probes: the HBM read ceilings the decode kernel is
 * measured against on the machine it runs on.  They are measurement
 * utilities, not part of the attention path, and live in the same shared
 * library (libkvq2.so).
 *
 * The decode kernel's roofline is the 8 TB/s HBM peak of the MI355X data
 * sheet; these two kernels show what plain reads reach on the same box:
 *   kvq_probe_stream_read  one sequential pass over a buffer with 16-byte
 *                          non-temporal loads, one contiguous block per
 *                          work-group (every byte read once);
 *   kvq_probe_chunk_read   the decode's own access pattern: a list of
 *                          1152-byte INT2 chunks (byte offsets into the pool)
 *                          read through the same non-temporal global->LDS
 *                          loads, four tiles of two chunks in flight per
 *                          wave, each wave taking a contiguous slice of the
 *                          list.
 * Both fold what they read into `sink` (one uint32 per work-group) so that no
 * load is removed.  Asynchronous on `stream`; return 0 or a negative
 * kvq_status (KVQ_ERR_ARG for a null or misaligned pointer or a bad size,
 * KVQ_ERR_HIP for a launch failure).  All device pointers 16-byte aligned.
 */
#ifndef KVQ2_PROBE_H
#define KVQ2_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* src: device buffer of `bytes` bytes (a positive multiple of 16);
 * sink: device uint32 [work_groups]; work_groups in [1, 65536]. */
int kvq_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t work_groups,
                          void* stream);

/* pool: device bytes; chunk_off: device int64 [n_chunks], each a byte offset
 * of a 1152-byte chunk inside the pool (a multiple of 16, caller-checked);
 * sink: device uint32 [work_groups]; n_chunks >= 1; work_groups in [1, 65536]. */
int kvq_probe_chunk_read(const uint8_t* pool, const int64_t* chunk_off, int64_t n_chunks,
                         uint32_t* sink, int32_t work_groups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ2_PROBE_H */
