// Router: float64 logits, top-k with lower-id tie break, softmax over the
// chosen k (pages: zhichai.net, section on MoE sparsity -- the router picks
// 8 of 256 experts for every token; yunpan.plus article, "capability 4" --
// router semantics never change silently, hence float64 logits whose top-k
// does not depend on summation order).
//
// Two logit kernels: for small batches one wavefront per expert streams that
// expert's router row once for all tokens (the router matrix, 6.3 MB at
// d=6144/E=256, is spread over E/4 workgroups); for large batches a tiled
// float64 product reuses each router row across 64 tokens.  Every product
// x*w is exact in float64 (bf16 or fp32 times fp32), so only the summation
// order can differ from any other float64 evaluation.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

template <bool XBF16>
__device__ __forceinline__ void load_x4(const void* x, size_t idx, float (&v)[4]) {
  if constexpr (XBF16) {
    const uint2 r = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + idx);
    v[0] = __uint_as_float(r.x << 16);
    v[1] = __uint_as_float(r.x & 0xFFFF0000u);
    v[2] = __uint_as_float(r.y << 16);
    v[3] = __uint_as_float(r.y & 0xFFFF0000u);
  } else {
    const float4 r = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + idx);
    v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
  }
}

template <typename T>
__device__ __forceinline__ float x_at(const void* x, size_t idx);
template <>
__device__ __forceinline__ float x_at<uint16_t>(const void* x, size_t idx) {
  return bf16_to_f32(static_cast<const uint16_t*>(x)[idx]);
}
template <>
__device__ __forceinline__ float x_at<float>(const void* x, size_t idx) {
  return static_cast<const float*>(x)[idx];
}

// One wavefront per expert; 4 tokens per sweep of the router row.
template <bool XBF16>
__global__ __launch_bounds__(256) void logits_per_expert(const void* __restrict__ x,
                                                          const float* __restrict__ w,
                                                          const float* __restrict__ bias,
                                                          double* __restrict__ logits, int T,
                                                          int d, int E) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const float* wr = w + static_cast<size_t>(e) * d;
  const double b = bias ? static_cast<double>(bias[e]) : 0.0;
  for (int t0 = 0; t0 < T; t0 += 4) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int i = lane * 4; i < d; i += 256) {
      const float4 wv = *reinterpret_cast<const float4*>(wr + i);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        if (t0 + tt < T) {
          float xv[4];
          load_x4<XBF16>(x, static_cast<size_t>(t0 + tt) * d + i, xv);
          acc[tt] = fma(static_cast<double>(xv[0]), static_cast<double>(wv.x), acc[tt]);
          acc[tt] = fma(static_cast<double>(xv[1]), static_cast<double>(wv.y), acc[tt]);
          acc[tt] = fma(static_cast<double>(xv[2]), static_cast<double>(wv.z), acc[tt]);
          acc[tt] = fma(static_cast<double>(xv[3]), static_cast<double>(wv.w), acc[tt]);
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const double s = wave_sum_f64(acc[tt]);
      if (lane == 0 && t0 + tt < T) logits[static_cast<size_t>(t0 + tt) * E + e] = s + b;
    }
  }
}

// 64 tokens x 64 experts per workgroup, 4x4 outputs per thread, K step 16.
constexpr int kTile = 64;
constexpr int kStep = 16;

template <typename XT>
__global__ __launch_bounds__(256) void logits_tiled(const void* __restrict__ x,
                                                     const float* __restrict__ w,
                                                     const float* __restrict__ bias,
                                                     double* __restrict__ logits, int T, int d,
                                                     int E) {
  __shared__ double xs[kStep][kTile + 1];
  __shared__ double ws[kStep][kTile + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int e0 = blockIdx.x * kTile, t0 = blockIdx.y * kTile;
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
  for (int k0 = 0; k0 < d; k0 += kStep) {
    for (int i = threadIdx.x; i < kTile * kStep; i += 256) {
      const int r = i / kStep, c = i % kStep;
      const int t = t0 + r, e = e0 + r;
      xs[c][r] = t < T ? static_cast<double>(x_at<XT>(x, static_cast<size_t>(t) * d + k0 + c)) : 0.0;
      ws[c][r] = e < E ? static_cast<double>(w[static_cast<size_t>(e) * d + k0 + c]) : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kStep; ++c) {
      double a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[c][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j] = ws[c][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], bb[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) logits[static_cast<size_t>(t) * E + e] = acc[i][j] + (bias ? static_cast<double>(bias[e]) : 0.0);
    }
  }
}

// One wavefront per token: k rounds of a wave-wide argmax over (logit desc,
// expert id asc), then the softmax of the chosen logits in float64.
constexpr int kMaxPerLane = 16;  // E <= 1024
constexpr int kMaxK = 32;

__global__ __launch_bounds__(256) void topk_softmax(const double* __restrict__ logits, int T,
                                                    int E, int k, int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
  __shared__ double sel_v[4][kMaxK];
  __shared__ int sel_e[4][kMaxK];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;
  const double* lg = logits + static_cast<size_t>(t) * E;
  double v[kMaxPerLane];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    double val = e < E ? lg[e] : -__builtin_inf();
    v[i] = val != val ? -__builtin_inf() : val;  // NaN ranks as -inf
    if (e >= E) taken |= 1u << i;
  }
  for (int j = 0; j < k; ++j) {
    double bv = -__builtin_inf();
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      if (!(taken >> i & 1u) && (v[i] > bv || (v[i] == bv && e < be))) {
        bv = v[i];
        be = e;
      }
    }
    for (int off = 32; off > 0; off >>= 1) {
      const double ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == 0) {
      sel_v[wv][j] = bv;
      sel_e[wv][j] = be;
    }
  }
  __builtin_amdgcn_wave_barrier();
  if (lane == 0) {
    const double m = sel_v[wv][0];
    double p[kMaxK];
    double z = 0.0;
    for (int j = 0; j < k; ++j) {
      p[j] = exp(sel_v[wv][j] - m);
      z += p[j];
    }
    for (int j = 0; j < k; ++j) {
      topk_idx[static_cast<size_t>(t) * k + j] = sel_e[wv][j];
      topk_w[static_cast<size_t>(t) * k + j] = static_cast<float>(p[j] / z);
    }
  }
}

}  // namespace

hipError_t launch_route(int T, int d, int E, int k, const void* x, bool x_bf16,
                        const float* w_router, const float* bias, double* logits,
                        int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  hipError_t err;
  if (T <= 32) {
    const dim3 grid((E + 3) / 4);
    err = x_bf16 ? launch(logits_per_expert<true>, grid, dim3(256), 0, stream, x, w_router, bias,
                          logits, T, d, E)
                 : launch(logits_per_expert<false>, grid, dim3(256), 0, stream, x, w_router,
                          bias, logits, T, d, E);
  } else {
    const dim3 grid((E + kTile - 1) / kTile, (T + kTile - 1) / kTile);
    err = x_bf16 ? launch(logits_tiled<uint16_t>, grid, dim3(256), 0, stream, x, w_router, bias,
                          logits, T, d, E)
                 : launch(logits_tiled<float>, grid, dim3(256), 0, stream, x, w_router, bias,
                          logits, T, d, E);
  }
  if (err != hipSuccess) return err;
  return launch(topk_softmax, dim3((T + 3) / 4), dim3(256), 0, stream,
                static_cast<const double*>(logits), T, E, k, topk_idx, topk_w);
}

}  // namespace moe
