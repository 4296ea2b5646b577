/*
 * moe_int4_measure.h -- calibration call for the benchmark's roofline (not
 * part of the layer): the rate a plain read-only kernel attains on the same
 * bytes the decode FFN streams.
 *
 * Same conventions as moe_int4.h (device pointers owned by the caller,
 * asynchronous on `stream`, arguments checked before anything is enqueued).
 */
#ifndef MOE_INT4_MEASURE_H
#define MOE_INT4_MEASURE_H

#include "moe_int4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read n_blocks device blocks of block_bytes each once: every block split
 * into wpb = workgroups / n_blocks equal shares, one workgroup of
 * 256 threads (16-byte loads) per share, wpb * n_blocks workgroups in all;
 * the loaded words are folded into one uint32 per workgroup in sink.
 *  blocks      HOST array of n_blocks device pointers (1 <= n_blocks <= 64),
 *              each 16-byte aligned
 *  block_bytes a positive multiple of 16
 *  workgroups  n_blocks .. 65536 (else MOE_ERR_SHAPE)
 *  sink        device uint32 [wpb * n_blocks] (at most `workgroups`
 *              entries), 4-byte aligned (contents unused) */
moe_status moe_measure_stream_read(const uint8_t* const* blocks, int32_t n_blocks,
                                   size_t block_bytes, int32_t workgroups, uint32_t* sink,
                                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_INT4_MEASURE_H */
