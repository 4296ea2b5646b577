// Router: float64 logits, top-k with lower-id tie break, softmax over the
// chosen k (pages: zhichai.net, section on MoE sparsity -- the router picks
// 8 of 256 experts for every token; yunpan.plus article, "capability 4" --
// router semantics never change silently, hence float64 logits whose top-k
// does not depend on summation order).
//
// Two logit kernels: for small batches each router row is split into P
// parts and one wavefront per (expert, part) streams it once for all tokens,
// so the router matrix (6.3 MB at d=6144/E=256) is read by E*P wavefronts at
// HBM rate; for large batches a tiled float64 product reuses each router row
// across 64 tokens.  Every product x*w is exact in float64 (bf16 or fp32
// times fp32), so only the summation order can differ from any other
// float64 evaluation, and that order is fixed for a given batch-size class.
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

// Small batches: one wavefront per (expert, part of d).  Spreading each
// router row over P parts puts E*P wavefronts in flight, enough to stream the
// router matrix at HBM rate; every wavefront keeps up to 8 tokens' float64
// sums and writes part[t][e][p] (tree-summed over its lanes).
constexpr int kTokGroup = 8;
constexpr int kSplitMaxT = 32;  // larger batches use the tiled kernel

template <bool XBF16>
__global__ __launch_bounds__(256) void logits_split(const void* __restrict__ x,
                                                     const float* __restrict__ w,
                                                     double* __restrict__ part, int T, int d,
                                                     int E, int P, int L) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= E * P) return;
  const int e = item / P, p = item - e * P;
  const int i0 = p * L, i1 = min(d, i0 + L);
  const float* wr = w + static_cast<size_t>(e) * d;
  for (int t0 = 0; t0 < T; t0 += kTokGroup) {
    double acc[kTokGroup];
#pragma unroll
    for (int tt = 0; tt < kTokGroup; ++tt) acc[tt] = 0.0;
    for (int i = i0 + lane * 4; i < i1; i += 256) {
      const float4 wv = *reinterpret_cast<const float4*>(wr + i);
#pragma unroll
      for (int tt = 0; tt < kTokGroup; ++tt) {
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
    for (int tt = 0; tt < kTokGroup; ++tt) {
      if (t0 + tt < T) {
        const double s = wave_sum_f64_tree(acc[tt]);
        if (lane == 0) part[(static_cast<size_t>(t0 + tt) * E + e) * P + p] = s;
      }
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

// Top-k and softmax, one wavefront per token, E <= 64*NPL.
//
// The logit of expert e is the in-order sum of its P partial sums plus the
// bias.  Selection is exact on the float64 logits with ties to the lower id.
// It first narrows the field with float32 copies: rounding to float32 is
// monotone, so the k best experts all have float32 keys at or above the k-th
// largest float32 key tau, found by a 32-step bitwise search with ballots.
// The (usually exactly k) candidates at or above tau are then ranked by
// (float64 logit desc, id asc) against each other.  If more than 64
// candidates share the cut (mass ties), k rounds of a wave-wide argmax over
// all experts decide instead.
constexpr int kMaxK = 32;

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int NPL>
__global__ __launch_bounds__(256) void topk_softmax(const double* __restrict__ part, int P,
                                                    const float* __restrict__ bias, int T, int E,
                                                    int k, int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
  __shared__ double cand_v[4][64];
  __shared__ int cand_e[4][64];
  __shared__ double sel_v[4][kMaxK];
  __shared__ int sel_e[4][kMaxK];
  __shared__ double sel_p[4][kMaxK];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;
  const uint64_t lower = (1ull << lane) - 1ull;
  double v[NPL];
  uint32_t key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    double s = -__builtin_inf();
    if (e < E) {
      const double* q = part + (static_cast<size_t>(t) * E + e) * P;
      s = q[0];
      for (int pp = 1; pp < P; ++pp) s += q[pp];
      if (bias) s += static_cast<double>(bias[e]);
      if (s != s) s = -__builtin_inf();  // NaN ranks as -inf
    }
    v[i] = s;
    key[i] = e < E ? order_key(static_cast<float>(s)) : 0u;
  }
  uint32_t tau = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = tau | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) cnt += __popcll(__ballot(key[i] >= c));
    if (cnt >= k) tau = c;
  }
  int nc = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const bool in = key[i] >= tau;
    const uint64_t m = __ballot(in);
    const int pos = nc + __popcll(m & lower);
    if (in && pos < 64) {
      cand_v[wv][pos] = v[i];
      cand_e[wv][pos] = lane + 64 * i;
    }
    nc += __popcll(m);
  }
  __builtin_amdgcn_wave_barrier();
  if (nc <= 64) {
    if (lane < nc) {
      const double mv = cand_v[wv][lane];
      const int me = cand_e[wv][lane];
      int rank = 0;
      for (int q = 0; q < nc; ++q) {
        const double ov = cand_v[wv][q];
        const int oe = cand_e[wv][q];
        rank += (ov > mv || (ov == mv && oe < me)) ? 1 : 0;
      }
      if (rank < k) {
        sel_v[wv][rank] = mv;
        sel_e[wv][rank] = me;
      }
    }
  } else {
    uint32_t taken = 0;
    for (int j = 0; j < k; ++j) {
      double bv = -__builtin_inf();
      int be = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E && !(taken >> i & 1u) && (v[i] > bv || (v[i] == bv && e < be))) {
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
  }
  __builtin_amdgcn_wave_barrier();
  // softmax over the chosen k in float64: p_j = exp(l_j - l_0), z summed in j order
  const double m = sel_v[wv][0];
  const double pj = lane < k ? exp(sel_v[wv][lane] - m) : 0.0;
  if (lane < k) sel_p[wv][lane] = pj;
  __builtin_amdgcn_wave_barrier();
  double z = 0.0;
  for (int j = 0; j < k; ++j) z += sel_p[wv][j];
  if (lane < k) {
    topk_idx[static_cast<size_t>(t) * k + lane] = sel_e[wv][lane];
    topk_w[static_cast<size_t>(t) * k + lane] = static_cast<float>(pj / z);
  }
}

}  // namespace

int route_parts(int T, int d, int E) {
  if (T > kSplitMaxT) return 0;
  int P = 2048 / E;
  P = P < 1 ? 1 : (P > 16 ? 16 : P);
  const int by_len = d / 256;
  if (P > by_len) P = by_len < 1 ? 1 : by_len;
  return P;
}

size_t route_workspace(int T, int d, int E) {
  const int P = route_parts(T, d, E);
  return static_cast<size_t>(T) * E * (P > 0 ? P : 1) * sizeof(double);
}

hipError_t launch_route(int T, int d, int E, int k, const void* x, bool x_bf16,
                        const float* w_router, const float* bias, double* logits,
                        int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  hipError_t err;
  int P = route_parts(T, d, E);
  const float* topk_bias = bias;
  if (P > 0) {
    const int L = ((d + P - 1) / P + 3) / 4 * 4;
    const dim3 grid((E * P + 3) / 4);
    err = x_bf16 ? launch(logits_split<true>, grid, dim3(256), 0, stream, x, w_router, logits, T,
                          d, E, P, L)
                 : launch(logits_split<false>, grid, dim3(256), 0, stream, x, w_router, logits,
                          T, d, E, P, L);
  } else {
    P = 1;
    topk_bias = nullptr;  // the tiled kernel adds the bias itself
    const dim3 grid((E + kTile - 1) / kTile, (T + kTile - 1) / kTile);
    err = x_bf16 ? launch(logits_tiled<uint16_t>, grid, dim3(256), 0, stream, x, w_router, bias,
                          logits, T, d, E)
                 : launch(logits_tiled<float>, grid, dim3(256), 0, stream, x, w_router, bias,
                          logits, T, d, E);
  }
  if (err != hipSuccess) return err;
  const dim3 grid((T + 3) / 4);
  const double* part = logits;
  if (E <= 64)
    return launch(topk_softmax<1>, grid, dim3(256), 0, stream, part, P, topk_bias, T, E, k,
                  topk_idx, topk_w);
  if (E <= 128)
    return launch(topk_softmax<2>, grid, dim3(256), 0, stream, part, P, topk_bias, T, E, k,
                  topk_idx, topk_w);
  if (E <= 256)
    return launch(topk_softmax<4>, grid, dim3(256), 0, stream, part, P, topk_bias, T, E, k,
                  topk_idx, topk_w);
  if (E <= 512)
    return launch(topk_softmax<8>, grid, dim3(256), 0, stream, part, P, topk_bias, T, E, k,
                  topk_idx, topk_w);
  return launch(topk_softmax<16>, grid, dim3(256), 0, stream, part, P, topk_bias, T, E, k,
                topk_idx, topk_w);
}

}  // namespace moe
