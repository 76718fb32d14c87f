/*
 * kvq_testing.h -- C ABI of libkvq_testing.so: hooks for tests and
 * measurement that sit beside libkvq.so (include/kvq.h) and are not part of
 * the method.  They compute nothing a caller of the cache needs:
 *
 *  - the FP8 encoders of kvq_append applied to plain float arrays, so that a
 *    test can sweep every float32 input through the device conversion;
 *  - a plain streaming read of a device buffer, the attainable HBM read rate
 *    the decode kernels are compared with;
 *  - the split plan of the decode kernels run on the host for a given batch
 *    (how many work ranges, segments and partial slots it uses).
 *
 * Same conventions as kvq.h: pointers are device pointers owned by the
 * caller unless stated otherwise, work goes on the caller's stream, scalars
 * are validated before any HIP call and return a kvq_status.
 */
#ifndef KVQ_TESTING_H
#define KVQ_TESTING_H

#include <stddef.h>
#include <stdint.h>

#include "kvq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The FP8 E4M3 encoder of kvq_append on n float32 values: nearest-even,
 * saturating at +-448, sign of zero kept, NaN -> 0x7F.
 * x: device fp32 [n];  codes: device u8 [n]. */
kvq_status kvq_e4m3_encode(const float* x, uint8_t* codes, int64_t n, hipStream_t stream);

/* The E5M2 encoder of kvq_append (KVQ_FP8_E5M2 caches) on n float32 values:
 * nearest-even, saturating at +-57344 (no infinities), sign of zero kept,
 * NaN -> 0x7F.  x: device fp32 [n];  codes: device u8 [n]. */
kvq_status kvq_e5m2_encode(const float* x, uint8_t* codes, int64_t n, hipStream_t stream);

/* A plain streaming read of `bytes` bytes at `buf`: blocks_per_cu x (compute
 * units) workgroups of 256 threads step through the buffer in windows of
 * loads_per_thread x 4 KiB, each thread keeping loads_per_thread 16-byte loads
 * (one per 4 KiB of its window) in flight.  buf: device, 16-byte aligned,
 * bytes a multiple of 16.  sink: one device uint32 the kernel may write (in
 * practice never).  blocks_per_cu in 1..32; loads_per_thread 1, 2, 3, 4, 6
 * or 8. */
kvq_status kvq_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int32_t blocks_per_cu,
                          int32_t loads_per_thread, hipStream_t stream);

/* What the decode kernels' split plan does with one batch, computed on the
 * host by the same plan functions the kernels run. */
typedef struct kvq_plan_info {
    int64_t chunk;                 /* range length, weight units (pages, plus a start-up
                                      cost per item in ragged batches)              */
    int64_t ranges_per_head;       /* ranges of one KV head's weight space           */
    int64_t busy_ranges_per_head;  /* ranges holding at least one page              */
    int64_t segments_per_head;     /* (item, range) pieces with pages               */
    int64_t slots_used;            /* highest partial slot written + 1 (per head)    */
    int64_t slots;                 /* partial slots per head the workspace holds     */
    int32_t cost;                  /* start-up weight per item (0: uniform batch)    */
    int32_t max_segments_per_item; /* pieces of the most-cut item                    */
} kvq_plan_info;

/* context_lens: HOST int32 [num_seqs].  total_waves: resident waves of the
 * launch (compute units x workgroups per CU x 4).  partition_pages as in
 * kvq_decode_attention.  Host only: no HIP call. */
kvq_status kvq_plan_stats(int32_t page_size, int32_t num_kv_heads, int32_t total_waves,
                          const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                          int32_t partition_pages, kvq_plan_info* info);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_TESTING_H */
