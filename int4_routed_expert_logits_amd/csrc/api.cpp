// C ABI of the library (declared in include/moe_int4.h).  Every argument is
// checked here, on the host, before anything is enqueued; the checks use no
// HIP call, so every error path is exercised without a GPU.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "api_internal.h"
#include "launch.h"
#include "moe_int4.h"

namespace {

constexpr int kMaxDim = 8192;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int64_t kMaxSlots = int64_t(1) << 24;  // T * top_k
constexpr size_t kWorkspaceAlign = 256;
// moe_layer_decode: batches of at most this many tokens let every gate/up
// workgroup derive the top-k and the grouping itself (a launch fewer); larger
// ones group once.  Measured on the d=6144, f=2048 layer (HIP graphs): 1
// token 50.5 us against 52.3 us; 2 tokens 90.4 us against 82.5 us; 8 tokens
// 330 us against 240 us.
constexpr int kLayerDecodePrologueMaxT = 1;
constexpr int kMaxQuantK = 65536;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t n) { return (n + kWorkspaceAlign - 1) / kWorkspaceAlign * kWorkspaceAlign; }

// group 64: int4 codes with a float16 scale per 64 elements; group 32:
// MXFP4 (E2M1 codes with an E8M0 scale per 32 elements), which only the
// calls that pass mxfp4_ok take (the rest of the library is int4 only).
constexpr int kGroupInt4 = 64;
constexpr int kGroupMxfp4 = 32;

moe_status check_shape(const moe_shape* s, bool mxfp4_ok = false) {
  if (!s) return MOE_ERR_NULL;
  if (s->d <= 0 || s->f <= 0 || s->n_experts <= 0 || s->top_k <= 0 || s->group <= 0 ||
      s->f_shared < 0)
    return MOE_ERR_SHAPE;
  if (s->group != kGroupInt4 && !(mxfp4_ok && s->group == kGroupMxfp4))
    return MOE_ERR_UNSUPPORTED;
  if (s->d % 64 != 0 || s->f % 64 != 0) return MOE_ERR_SHAPE;
  if (s->d > kMaxDim || s->f > kMaxDim) return MOE_ERR_UNSUPPORTED;
  if (s->n_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (s->top_k > s->n_experts) return MOE_ERR_SHAPE;
  if (s->top_k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if (s->f_shared != 0 && s->f_shared != s->f) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_tokens(const moe_shape* s, int32_t T) {
  if (T < 0) return MOE_ERR_SHAPE;
  if (static_cast<int64_t>(T) * s->top_k > kMaxSlots) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The workspace sizes are 0 for a token count the calls reject.
bool shape_tokens_ok(const moe_shape* s, int32_t T) { return check_tokens(s, T) == MOE_OK; }

moe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  if (e == hipErrorNotSupported) return MOE_ERR_UNSUPPORTED;
  return MOE_ERR_HIP;
}

}  // namespace

namespace moe {

// Every argument check of moe_layer_decode except the workspace's.
moe_status layer_decode_check(const moe_shape* shape, int32_t T, const void* x, moe_dtype x_dt,
                              const float* w_router, const float* bias, const uint8_t* experts,
                              const uint8_t* shared, const int32_t* topk_idx,
                              const float* topk_w, const int32_t* counts,
                              const int32_t* offsets, const int32_t* perm,
                              const int32_t* inv_perm, const int32_t* active,
                              const int32_t* n_active, const void* y, const void* y_shared,
                              const void* out, moe_dtype out_dt) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(shape, T)) != MOE_OK) return st;
  if (x_dt != MOE_F32 && x_dt != MOE_BF16) return MOE_ERR_DTYPE;
  if (out_dt != MOE_F32 && out_dt != MOE_BF16) return MOE_ERR_DTYPE;
  const int E = shape->n_experts, d = shape->d;
  const bool has_shared = shape->f_shared != 0;
  moe::FfnProblem p{};
  p.T = T;
  p.d = d;
  p.f = shape->f;
  p.E = E;
  p.k = shape->top_k;
  p.has_shared = has_shared;
  p.x_bf16 = x_dt == MOE_BF16;
  p.block_bytes = moe_expert_bytes(shape->d, shape->f, shape->group);
  if (T > 0 && !moe::ffn_decode_groups_batch(p, moe::route_parts(T, d, E)))
    return MOE_ERR_UNSUPPORTED;
  if (!counts || !offsets || !active || !n_active) return MOE_ERR_NULL;
  if (!aligned(counts, 4) || !aligned(offsets, 4) || !aligned(active, 4) || !aligned(n_active, 4))
    return MOE_ERR_ALIGN;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !experts || !topk_idx || !topk_w || !perm || !inv_perm || !y || !out)
    return MOE_ERR_NULL;
  if (has_shared != (shared != nullptr) || has_shared != (y_shared != nullptr))
    return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_router, 16) || (bias && !aligned(bias, 4)) ||
      !aligned(experts, 16) || (shared && !aligned(shared, 16)) || !aligned(topk_idx, 4) ||
      !aligned(topk_w, 4) || !aligned(perm, 4) || !aligned(inv_perm, 4) || !aligned(y, 16) ||
      (y_shared && !aligned(y_shared, 16)) || !aligned(out, 16))
    return MOE_ERR_ALIGN;
  return MOE_OK;
}

}  // namespace moe

extern "C" {

size_t moe_expert_bytes(int32_t d, int32_t f, int32_t group) {
  if ((group != kGroupInt4 && group != kGroupMxfp4) || d <= 0 || f <= 0 || d % 64 || f % 64)
    return 0;
  const size_t n = 3ull * static_cast<size_t>(d) * static_cast<size_t>(f);
  // int4: half a byte per code + a float16 per 64; MXFP4: half a byte per
  // code + one byte per 32 (the same total)
  return group == kGroupInt4 ? n / 2 + n / group * 2 : n / 2 + n / group;
}

moe_status moe_pack_experts(const moe_shape* shape, int64_t n_blocks, const uint8_t* src,
                            uint8_t* dst, void* stream) {
  moe_status st = check_shape(shape, true);
  if (st != MOE_OK) return st;
  if (n_blocks < 0) return MOE_ERR_SHAPE;
  if (n_blocks == 0) return MOE_OK;
  if (!src || !dst) return MOE_ERR_NULL;
  if (!aligned(src, 16) || !aligned(dst, 16)) return MOE_ERR_ALIGN;
  const size_t bb = moe_expert_bytes(shape->d, shape->f, shape->group);
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t len = static_cast<uintptr_t>(bb) * static_cast<uintptr_t>(n_blocks);
  if (s0 < d0 + len && d0 < s0 + len) return MOE_ERR_SHAPE;  // overlapping buffers
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(shape->group == kGroupMxfp4
                        ? moe::launch_pack_mxfp4(shape->d, shape->f, n_blocks, bb, src, dst, s)
                        : moe::launch_pack(shape->d, shape->f, n_blocks, bb, src, dst, s));
}

moe_status moe_quantize(int32_t N, int32_t K, const void* w, moe_dtype w_dt, moe_quant_mode mode,
                        uint8_t* codes, void* scales, void* stream) {
  if (N < 0 || K <= 0 || K % 64 != 0) return MOE_ERR_SHAPE;
  if (K > kMaxQuantK) return MOE_ERR_UNSUPPORTED;
  if (mode != MOE_QUANT_GS64 && mode != MOE_QUANT_ROW) return MOE_ERR_UNSUPPORTED;
  if (w_dt != MOE_F32 && w_dt != MOE_BF16) return MOE_ERR_DTYPE;
  if (N == 0) return MOE_OK;
  if (!w || !codes || !scales) return MOE_ERR_NULL;
  if (!aligned(w, 16) || !aligned(codes, 4) || !aligned(scales, 2)) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_quantize(N, K, w, w_dt == MOE_F32, mode == MOE_QUANT_ROW, codes,
                                         scales, static_cast<hipStream_t>(stream)));
}

size_t moe_route_workspace_bytes(const moe_shape* shape, int32_t T) {
  if (check_shape(shape, true) != MOE_OK || !shape_tokens_ok(shape, T)) return 0;
  return round_up(moe::route_workspace(T, shape->d, shape->n_experts));
}

moe_status moe_route(const moe_shape* shape, int32_t T, const void* x, moe_dtype x_dt,
                     const float* w_router, const float* bias, int32_t* topk_idx,
                     float* topk_w, void* workspace, size_t workspace_bytes, void* stream) {
  moe_status st = check_shape(shape, true);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(shape, T)) != MOE_OK) return st;
  if (x_dt != MOE_F32 && x_dt != MOE_BF16) return MOE_ERR_DTYPE;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !topk_idx || !topk_w || !workspace) return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(workspace, kWorkspaceAlign) ||
      !aligned(topk_idx, 4) || !aligned(topk_w, 4) || (bias && !aligned(bias, 4)))
    return MOE_ERR_ALIGN;
  if (workspace_bytes < moe_route_workspace_bytes(shape, T)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_route(T, shape->d, shape->n_experts, shape->top_k, x,
                                      x_dt == MOE_BF16, w_router, bias,
                                      static_cast<double*>(workspace), topk_idx, topk_w,
                                      static_cast<hipStream_t>(stream)));
}

moe_status moe_union(const moe_shape* shape, int32_t T, const int32_t* topk_idx,
                     int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                     int32_t* active, int32_t* n_active, void* stream) {
  moe_status st = check_shape(shape, true);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(shape, T)) != MOE_OK) return st;
  if (!counts || !offsets || !active || !n_active) return MOE_ERR_NULL;
  if (T > 0 && (!topk_idx || !perm || !inv_perm)) return MOE_ERR_NULL;
  if (!aligned(counts, 4) || !aligned(offsets, 4) || !aligned(active, 4) ||
      !aligned(n_active, 4) || (T > 0 && (!aligned(topk_idx, 4) || !aligned(perm, 4) ||
                                          !aligned(inv_perm, 4))))
    return MOE_ERR_ALIGN;
  return hip_status(moe::launch_union(T * shape->top_k, shape->n_experts, topk_idx, counts,
                                      offsets, perm, inv_perm, active, n_active,
                                      static_cast<hipStream_t>(stream)));
}

moe_status moe_route_union(const moe_shape* shape, int32_t T, const void* x, moe_dtype x_dt,
                           const float* w_router, const float* bias, int32_t* topk_idx,
                           float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* inv_perm, int32_t* active, int32_t* n_active,
                           void* workspace, size_t workspace_bytes, void* stream) {
  moe_status st = check_shape(shape, true);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(shape, T)) != MOE_OK) return st;
  if (x_dt != MOE_F32 && x_dt != MOE_BF16) return MOE_ERR_DTYPE;
  if (!counts || !offsets || !active || !n_active) return MOE_ERR_NULL;
  if (!aligned(counts, 4) || !aligned(offsets, 4) || !aligned(active, 4) || !aligned(n_active, 4))
    return MOE_ERR_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0)  // an empty batch: the empty grouping, as moe_union writes it
    return hip_status(moe::launch_union(0, shape->n_experts, nullptr, counts, offsets, nullptr,
                                        nullptr, active, n_active, s));
  if (!x || !w_router || !topk_idx || !topk_w || !workspace || !perm || !inv_perm)
    return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(workspace, kWorkspaceAlign) ||
      !aligned(topk_idx, 4) || !aligned(topk_w, 4) || (bias && !aligned(bias, 4)) ||
      !aligned(perm, 4) || !aligned(inv_perm, 4))
    return MOE_ERR_ALIGN;
  if (workspace_bytes < moe_route_workspace_bytes(shape, T)) return MOE_ERR_WORKSPACE;
  const moe::UnionOut u{counts, offsets, perm, inv_perm, active, n_active};
  return hip_status(moe::launch_route_union(T, shape->d, shape->n_experts, shape->top_k, x,
                                            x_dt == MOE_BF16, w_router, bias,
                                            static_cast<double*>(workspace), topk_idx, topk_w, u,
                                            s));
}

size_t moe_ffn_workspace_bytes(const moe_shape* shape, int32_t T, moe_path path) {
  if (check_shape(shape, true) != MOE_OK || !shape_tokens_ok(shape, T)) return 0;
  const bool sh = shape->f_shared != 0;
  if (path == MOE_PATH_DECODE_F32)
    return round_up(moe::ffn_decode_workspace(T, shape->top_k, shape->n_experts, shape->d,
                                              shape->f, sh));
  if (path == MOE_PATH_PREFILL_BF16)
    return round_up(moe::ffn_prefill_workspace(T, shape->top_k, shape->n_experts, shape->d, shape->f, sh));
  return 0;
}

moe_status moe_expert_ffn(const moe_shape* shape, int32_t T, const void* x, moe_dtype x_dt,
                          const uint8_t* experts, const uint8_t* shared,
                          const int32_t* offsets, const int32_t* perm, const int32_t* active,
                          const int32_t* n_active, moe_path path, void* y, void* y_shared,
                          void* workspace, size_t workspace_bytes, void* stream) {
  moe_status st = check_shape(shape, true);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(shape, T)) != MOE_OK) return st;
  if (path != MOE_PATH_DECODE_F32 && path != MOE_PATH_PREFILL_BF16) return MOE_ERR_UNSUPPORTED;
  const bool mxfp4 = shape->group == kGroupMxfp4;
  if (x_dt != MOE_F32 && x_dt != MOE_BF16) return MOE_ERR_DTYPE;
  if (path == MOE_PATH_PREFILL_BF16 && x_dt != MOE_BF16) return MOE_ERR_DTYPE;
  const bool has_shared = shape->f_shared != 0;
  if (T == 0) return MOE_OK;
  if (!x || !experts || !offsets || !perm || !active || !n_active || !y || !workspace)
    return MOE_ERR_NULL;
  if (has_shared != (shared != nullptr) || has_shared != (y_shared != nullptr))
    return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(experts, 16) || (shared && !aligned(shared, 16)) ||
      !aligned(y, 16) || (y_shared && !aligned(y_shared, 16)) ||
      !aligned(workspace, kWorkspaceAlign) || !aligned(offsets, 4) || !aligned(perm, 4) ||
      !aligned(active, 4) || !aligned(n_active, 4))
    return MOE_ERR_ALIGN;
  if (workspace_bytes < moe_ffn_workspace_bytes(shape, T, path)) return MOE_ERR_WORKSPACE;
  moe::FfnProblem p{};
  p.T = T;
  p.d = shape->d;
  p.f = shape->f;
  p.E = shape->n_experts;
  p.k = shape->top_k;
  p.has_shared = has_shared;
  p.x_bf16 = x_dt == MOE_BF16;
  p.block_bytes = moe_expert_bytes(shape->d, shape->f, shape->group);
  p.mxfp4 = mxfp4;
  p.x = x;
  p.experts = experts;
  p.shared = shared;
  p.offsets = offsets;
  p.perm = perm;
  p.active = active;
  p.n_active = n_active;
  p.y = y;
  p.y_shared = y_shared;
  p.workspace = workspace;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(path == MOE_PATH_DECODE_F32 ? moe::launch_ffn_decode(p, s)
                                                : moe::launch_ffn_prefill(p, s));
}

moe_status moe_combine(const moe_shape* shape, int32_t T, const void* y, const void* y_shared,
                       moe_dtype y_dt, const int32_t* inv_perm, const float* topk_w, void* out,
                       moe_dtype out_dt, void* stream) {
  moe_status st = check_shape(shape, true);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(shape, T)) != MOE_OK) return st;
  if ((y_dt != MOE_F32 && y_dt != MOE_BF16) || (out_dt != MOE_F32 && out_dt != MOE_BF16))
    return MOE_ERR_DTYPE;
  if (T == 0) return MOE_OK;
  if (!y || !inv_perm || !topk_w || !out) return MOE_ERR_NULL;
  if ((shape->f_shared != 0) != (y_shared != nullptr)) return MOE_ERR_NULL;
  if (!aligned(y, 16) || (y_shared && !aligned(y_shared, 16)) || !aligned(out, 16) ||
      !aligned(inv_perm, 4) || !aligned(topk_w, 4))
    return MOE_ERR_ALIGN;
  return hip_status(moe::launch_combine(T, shape->d, shape->top_k, y, y_shared,
                                        y_dt == MOE_BF16, inv_perm, topk_w, out,
                                        out_dt == MOE_BF16, static_cast<hipStream_t>(stream)));
}

size_t moe_layer_decode_workspace_bytes(const moe_shape* shape, int32_t T) {
  if (check_shape(shape) != MOE_OK || !shape_tokens_ok(shape, T)) return 0;
  return moe_route_workspace_bytes(shape, T) + moe_ffn_workspace_bytes(shape, T, MOE_PATH_DECODE_F32);
}

moe_status moe_layer_decode(const moe_shape* shape, int32_t T, const void* x, moe_dtype x_dt,
                            const float* w_router, const float* bias, const uint8_t* experts,
                            const uint8_t* shared, int32_t* topk_idx, float* topk_w,
                            int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                            int32_t* active, int32_t* n_active, void* y, void* y_shared,
                            void* out, moe_dtype out_dt, void* workspace, size_t workspace_bytes,
                            void* stream) {
  moe_status st = moe::layer_decode_check(shape, T, x, x_dt, w_router, bias, experts, shared,
                                          topk_idx, topk_w, counts, offsets, perm, inv_perm,
                                          active, n_active, y, y_shared, out, out_dt);
  if (st != MOE_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int E = shape->n_experts, k = shape->top_k, d = shape->d;
  if (T == 0)
    return hip_status(moe::launch_union(0, E, nullptr, counts, offsets, nullptr, nullptr, active,
                                        n_active, s));
  if (!workspace) return MOE_ERR_NULL;
  if (!aligned(workspace, kWorkspaceAlign)) return MOE_ERR_ALIGN;
  if (workspace_bytes < moe_layer_decode_workspace_bytes(shape, T)) return MOE_ERR_WORKSPACE;
  moe::FfnProblem p{};
  p.T = T;
  p.d = d;
  p.f = shape->f;
  p.E = E;
  p.k = k;
  p.has_shared = shape->f_shared != 0;
  p.x_bf16 = x_dt == MOE_BF16;
  p.block_bytes = moe_expert_bytes(shape->d, shape->f, shape->group);
  // workspace: the router's partial sums, then the FFN's intermediate h
  const size_t route_bytes = moe_route_workspace_bytes(shape, T);
  double* part = static_cast<double*>(workspace);
  p.x = x;
  p.experts = experts;
  p.shared = shared;
  p.offsets = offsets;
  p.perm = perm;
  p.active = active;
  p.n_active = n_active;
  p.y = y;
  p.y_shared = y_shared;
  p.workspace = static_cast<uint8_t*>(workspace) + route_bytes;
  const moe::UnionOut u{counts, offsets, perm, inv_perm, active, n_active};
  hipError_t err;
  if (T <= kLayerDecodePrologueMaxT) {
    // router logits, then gate/up workgroups that take the top-k and the
    // grouping themselves (one launch fewer)
    const moe::RouteGroup rg{part, moe::route_parts(T, d, E), bias, topk_idx, topk_w, u};
    err = moe::launch_router_logits(T, d, E, x, x_dt == MOE_BF16, w_router, part, s);
    if (err == hipSuccess) err = moe::launch_ffn_decode_grouping(p, rg, s);
  } else {
    // the separate calls' kernels: routing and grouping once for the batch
    err = moe::launch_route_union(T, d, E, k, x, x_dt == MOE_BF16, w_router, bias, part,
                                  topk_idx, topk_w, u, s);
    if (err == hipSuccess) err = moe::launch_ffn_decode(p, s);
  }
  if (err == hipSuccess)
    err = moe::launch_combine(T, d, k, y, y_shared, false, inv_perm, topk_w, out,
                              out_dt == MOE_BF16, s);
  return hip_status(err);
}

const char* moe_status_str(moe_status status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or sizes disagree";
    case MOE_ERR_DTYPE: return "dtype not allowed for this call or path";
    case MOE_ERR_ALIGN: return "a pointer is not aligned as documented";
    case MOE_ERR_UNSUPPORTED: return "well-formed request this library does not provide";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "a HIP launch failed";
    case MOE_STATUS_INT_MIN_:
    case MOE_STATUS_INT_MAX_: break;  // range members, not statuses
  }
  return "unknown status";
}

}  // extern "C"
