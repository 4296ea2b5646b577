// Internal host-side launchers, one per kernel family.  Arguments have been
// validated by the C-ABI layer (api.cpp) before any of these is called; each
// returns the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace moe {

// Launch through hipLaunchKernel so the launch status comes back directly,
// without touching the thread's sticky last-error state.
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                  hipStream_t stream, Args&&... args) {
  std::tuple<KArgs...> held(static_cast<KArgs>(std::forward<Args>(args))...);
  return std::apply(
      [&](auto&... a) {
        void* ptrs[] = {static_cast<void*>(&a)...};
        return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, shmem,
                               stream);
      },
      held);
}

// route.hip: float64 logits then top-k + renormalised softmax.  The
// workspace holds float64 logits, split into route_parts() partial sums per
// (token, expert) and part of d.
int route_parts(int T, int d, int E);
size_t route_workspace(int T, int d, int E);
hipError_t launch_route(int T, int d, int E, int k, const void* x, bool x_bf16,
                        const float* w_router, const float* bias, double* logits,
                        int32_t* topk_idx, float* topk_w, hipStream_t stream);

// union.hip: batch-union grouping in one workgroup.
hipError_t launch_union(int n_slots, int E, const int32_t* topk_idx, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* active,
                        int32_t* n_active, hipStream_t stream);

// The batch-union outputs (moe_union's arrays).
struct UnionOut {
  int32_t *counts, *offsets, *perm, *inv_perm, *active, *n_active;
};

// route.hip: the router and the batch-union of its result; small batches run
// top-k and union in one kernel, the rest as launch_route + launch_union.
hipError_t launch_route_union(int T, int d, int E, int k, const void* x, bool x_bf16,
                              const float* w_router, const float* bias, double* logits,
                              int32_t* topk_idx, float* topk_w, const UnionOut& u,
                              hipStream_t stream);

// route.hip: only the float64 logit partial sums of launch_route (the
// workspace's [T][E][route_parts()] doubles).
hipError_t launch_router_logits(int T, int d, int E, const void* x, bool x_bf16,
                                const float* w_router, double* part, hipStream_t stream);

// quant.hip: float weights -> int4 codes + float16 scales (per 64-column
// group, or per row).
hipError_t launch_quantize(int N, int K, const void* w, bool f32, bool per_row, uint8_t* codes,
                           void* scales, hipStream_t stream);

struct FfnProblem {
  int T, d, f, E, k;
  bool has_shared;
  bool x_bf16;
  bool mxfp4 = false;  // MXFP4 blocks instead of int4 gs64
  size_t block_bytes;
  const void* x;
  const uint8_t* experts;
  const uint8_t* shared;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* active;
  const int32_t* n_active;
  void* y;
  void* y_shared;
  void* workspace;
};

// ffn_decode.hip: int4 GEMV, float32 intermediate and outputs.
size_t ffn_decode_workspace(int T, int k, int E, int d, int f, bool has_shared);
hipError_t launch_ffn_decode(const FfnProblem& p, hipStream_t stream);

// ffn_decode.hip: the same FFN for a small batch whose top-k and grouping
// the gate/up kernel derives itself from the router's partial sums (part,
// P parts per logit), writing them to topk_idx / topk_w and u (p.offsets,
// p.perm, p.active and p.n_active must be u's arrays).
struct RouteGroup {
  const double* part;
  int P;
  const float* bias;
  int32_t* topk_idx;
  float* topk_w;
  UnionOut u;
};
// Whether launch_ffn_decode_grouping takes this problem (batch size, experts,
// parts per logit, LDS).
bool ffn_decode_groups_batch(const FfnProblem& p, int P);
hipError_t launch_ffn_decode_grouping(const FfnProblem& p, const RouteGroup& rg,
                                      hipStream_t stream);

// ffn_prefill.hip: grouped GEMM on bf16 MFMA, bf16 intermediate and outputs.
size_t ffn_prefill_workspace(int T, int k, int E, int d, int f, bool has_shared);
hipError_t launch_ffn_prefill(const FfnProblem& p, hipStream_t stream);

// pack.hip: canonical -> packed expert blocks (int4 gs64, or MXFP4).
hipError_t launch_pack(int d, int f, long long n_blocks, size_t block_bytes, const uint8_t* src,
                       uint8_t* dst, hipStream_t stream);
hipError_t launch_pack_mxfp4(int d, int f, long long n_blocks, size_t block_bytes,
                             const uint8_t* src, uint8_t* dst, hipStream_t stream);

// combine.hip
hipError_t launch_combine(int T, int d, int k, const void* y, const void* y_shared, bool y_bf16,
                          const int32_t* inv_perm, const float* topk_w, void* out,
                          bool out_bf16, hipStream_t stream);

}  // namespace moe
