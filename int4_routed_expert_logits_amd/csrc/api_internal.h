// Argument checks shared by C-ABI entry points in more than one source file.
#pragma once

#include "moe_int4.h"

namespace moe {

// Every argument check of moe_layer_decode except the workspace's (api.cpp):
// MOE_OK, or the status moe_layer_decode would return for these arguments.
moe_status layer_decode_check(const moe_shape* shape, int32_t T, const void* x, moe_dtype x_dt,
                              const float* w_router, const float* bias, const uint8_t* experts,
                              const uint8_t* shared, const int32_t* topk_idx,
                              const float* topk_w, const int32_t* counts,
                              const int32_t* offsets, const int32_t* perm,
                              const int32_t* inv_perm, const int32_t* active,
                              const int32_t* n_active, const void* y, const void* y_shared,
                              const void* out, moe_dtype out_dt);

}  // namespace moe
