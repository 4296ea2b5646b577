/*
 * moe_int4_static.h -- the one-call decode layer without a workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, and hosts that forbid hipMalloc.
 *
 * Same conventions as moe_int4.h (which this header includes).
 */
#ifndef MOE_INT4_STATIC_H
#define MOE_INT4_STATIC_H

#include "moe_int4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the library's static scratch array on each GPU (4 MiB): the
 * largest workspace moe_layer_decode_static can stand in for. */
size_t moe_layer_decode_static_max_bytes(void);

/* moe_layer_decode with the same arguments except the workspace, and the
 * same outputs bit for bit: the router's partial sums and the FFN's
 * intermediate h go to a file-scope device array of
 * moe_layer_decode_static_max_bytes() bytes, one per GPU, held until the
 * process ends.  The call allocates nothing (no hipMalloc, no library
 * allocator); on the first call on a device it looks up that device's copy
 * of the array (hipGetSymbolAddress), so call it with the intended device
 * current.
 *  Shapes whose moe_layer_decode_workspace_bytes() exceeds the array return
 *  MOE_ERR_WORKSPACE with nothing enqueued; every other check, and the
 *  supported batches (1 <= T <= 8, T*top_k <= 64, n_experts <= 256, int4
 *  blocks), are moe_layer_decode's.  MOE_ERR_HIP if the array's address
 *  cannot be found.
 *  Every call on one GPU shares that GPU's array: calls that may overlap in
 *  time on one GPU (two streams, two host threads) race on it and must be
 *  ordered by the caller.  Nothing in the array needs initial contents. */
moe_status moe_layer_decode_static(const moe_shape* shape, int32_t T, const void* x,
                                   moe_dtype x_dt, const float* w_router, const float* bias,
                                   const uint8_t* experts, const uint8_t* shared,
                                   int32_t* topk_idx, float* topk_w, int32_t* counts,
                                   int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                   int32_t* active, int32_t* n_active, void* y, void* y_shared,
                                   void* out, moe_dtype out_dt, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_INT4_STATIC_H */
