// Gate-weighted combine of each token's k routed-expert outputs with the
// shared expert (pages: zhichai.net, section on MoE sparsity -- 8 routed
// experts plus the always-active "+1" shared expert per layer).
//   out[t] = sum_{j<k} w[t,j] * y[inv_perm[t*k+j]] + y_shared[t]
// summed in j order in float32; each thread owns 4 (f32) or 8 (bf16)
// consecutive columns of one token, so there are no atomics and the result
// is bitwise reproducible.
#include "common.h"
#include "launch.h"

#pragma clang fp contract(off)  // the fused multiply-adds are written out

namespace moe {

namespace {

template <bool BF16>
struct Vec;
template <>
struct Vec<false> {
  __device__ static void load(const void* p, size_t i, float (&v)[4]) {
    const float4 q = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
};
template <>
struct Vec<true> {
  __device__ static void load(const void* p, size_t i, float (&v)[8]) {
    const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
};

template <bool YBF16>
__device__ __forceinline__ void load_row8(const void* base, size_t i, float (&v)[8]) {
  if constexpr (YBF16) {
    Vec<true>::load(base, i, v);
  } else {
    float a[4], b[4];
    Vec<false>::load(base, i, a);
    Vec<false>::load(base, i + 4, b);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = a[q];
      v[4 + q] = b[q];
    }
  }
}

// All k row indices and weights of a token are loaded before any y row, and
// the y rows of 8 slots are in flight together; empty slots (inv_perm < 0)
// leave the sum untouched.
template <bool YBF16, bool OBF16>
__global__ __launch_bounds__(64) void combine_kernel(const void* __restrict__ y,
                                                     const void* __restrict__ y_shared,
                                                     const int32_t* __restrict__ inv_perm,
                                                     const float* __restrict__ topk_w,
                                                     void* __restrict__ out,
                                                     int /*T, the grid's y extent*/, int d,
                                                     int k) {
  constexpr int V = 8;   // columns per thread
  constexpr int KU = 8;  // slots in flight
  const int t = blockIdx.y;
  const int c0 = (blockIdx.x * blockDim.x + threadIdx.x) * V;
  if (c0 >= d) return;
  float acc[V];
#pragma unroll
  for (int q = 0; q < V; ++q) acc[q] = 0.0f;
  // the shared expert's row needs no index: it goes out first
  float vs[V];
  if (y_shared) load_row8<YBF16>(y_shared, static_cast<size_t>(t) * d + c0, vs);
  for (int j0 = 0; j0 < k; j0 += KU) {
    int p[KU];
    float w[KU];
#pragma unroll
    for (int jj = 0; jj < KU; ++jj) {
      const int j = j0 + jj;
      p[jj] = j < k ? inv_perm[static_cast<size_t>(t) * k + j] : -1;
      w[jj] = j < k ? topk_w[static_cast<size_t>(t) * k + j] : 0.0f;
    }
    float v[KU][V];
#pragma unroll
    for (int jj = 0; jj < KU; ++jj) {
      const size_t row = p[jj] >= 0 ? static_cast<size_t>(p[jj]) : 0;
      load_row8<YBF16>(y, row * d + c0, v[jj]);
    }
#pragma unroll
    for (int jj = 0; jj < KU; ++jj) {
      if (p[jj] >= 0) {
#pragma unroll
        for (int q = 0; q < V; ++q) acc[q] = fmaf(w[jj], v[jj][q], acc[q]);
      }
    }
  }
  if (y_shared) {
#pragma unroll
    for (int q = 0; q < V; ++q) acc[q] += vs[q];
  }
  if constexpr (OBF16) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = static_cast<uint32_t>(f32_to_bf16(acc[2 * j])) |
             (static_cast<uint32_t>(f32_to_bf16(acc[2 * j + 1])) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + static_cast<size_t>(t) * d + c0) =
        make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    float* o = static_cast<float*>(out) + static_cast<size_t>(t) * d + c0;
    *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

}  // namespace

hipError_t launch_combine(int T, int d, int k, const void* y, const void* y_shared, bool y_bf16,
                          const int32_t* inv_perm, const float* topk_w, void* out,
                          bool out_bf16, hipStream_t stream) {
  const dim3 block(64);
  const dim3 grid((d / 8 + 63) / 64, T);
  if (y_bf16)
    return out_bf16 ? launch(combine_kernel<true, true>, grid, block, 0, stream, y, y_shared,
                             inv_perm, topk_w, out, T, d, k)
                    : launch(combine_kernel<true, false>, grid, block, 0, stream, y, y_shared,
                             inv_perm, topk_w, out, T, d, k);
  return out_bf16 ? launch(combine_kernel<false, true>, grid, block, 0, stream, y, y_shared,
                           inv_perm, topk_w, out, T, d, k)
                  : launch(combine_kernel<false, false>, grid, block, 0, stream, y, y_shared,
                           inv_perm, topk_w, out, T, d, k);
}

}  // namespace moe
