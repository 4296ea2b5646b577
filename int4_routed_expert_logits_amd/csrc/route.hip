// Router: float64 logits, top-k with lower-id tie break, softmax over the
// chosen k (pages: zhichai.net, section on MoE sparsity -- the router picks
// 8 of 256 experts for every token; yunpan.plus article, "capability 4" --
// router semantics never change silently, hence float64 logits whose top-k
// does not depend on summation order).
//
// Two logit kernels: for small batches each router row is split into P
// parts and one wavefront per (expert, part) streams it once for all tokens,
// so the router matrix (6.3 MB at d=6144/E=256) is read by E*P wavefronts at
// HBM rate; large batches run the product on the float64 matrix cores in
// 64-token x 128-expert tiles.  Every product x*w is exact in float64 (bf16 or fp32
// times fp32), so only the summation order can differ from any other
// float64 evaluation, and that order is fixed for a given batch-size class.
#include "common.h"
#include "launch.h"
#include "topk_wave.h"
#include "union_wave.h"

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

// Small batches: one wavefront per (expert, part of d).  Spreading each
// router row over P parts puts E*P wavefronts in flight, enough to stream the
// router matrix at HBM rate; every wavefront keeps up to 8 tokens' float64
// sums and writes part[t][e][p] (tree-summed over its lanes).
constexpr int kTokGroup = 8;
constexpr int kSplitMaxT = 32;  // larger batches use the matrix-core kernel

// Partial float64 sums of tokens t0 .. t0+kTokGroup-1 against router row e
// over columns [i0, i1), each lane its strided share.
template <bool XBF16>
__device__ __forceinline__ void logits_part(const void* __restrict__ x, const float* __restrict__ w,
                                            int T, int d, int e, int i0, int i1, int t0, int lane,
                                            double (&acc)[kTokGroup]) {
  const float* wr = w + static_cast<size_t>(e) * d;
#pragma unroll
  for (int tt = 0; tt < kTokGroup; ++tt) acc[tt] = 0.0;
  // four 256-column steps per pass, their router loads issued together
  for (int ib = i0 + lane * 4; ib < i1; ib += 4 * 256) {
    float4 wv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = ib + u * 256;
      wv[u] = i < i1 ? *reinterpret_cast<const float4*>(wr + i) : make_float4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = ib + u * 256;
      if (i >= i1) break;
#pragma unroll
      for (int tt = 0; tt < kTokGroup; ++tt) {
        if (t0 + tt < T) {
          float xv[4];
          load_x4<XBF16>(x, static_cast<size_t>(t0 + tt) * d + i, xv);
          acc[tt] = fma(static_cast<double>(xv[0]), static_cast<double>(wv[u].x), acc[tt]);
          acc[tt] = fma(static_cast<double>(xv[1]), static_cast<double>(wv[u].y), acc[tt]);
          acc[tt] = fma(static_cast<double>(xv[2]), static_cast<double>(wv[u].z), acc[tt]);
          acc[tt] = fma(static_cast<double>(xv[3]), static_cast<double>(wv[u].w), acc[tt]);
        }
      }
    }
  }
}

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
  for (int t0 = 0; t0 < T; t0 += kTokGroup) {
    double acc[kTokGroup];
    logits_part<XBF16>(x, w, T, d, e, i0, i1, t0, lane, acc);
#pragma unroll
    for (int tt = 0; tt < kTokGroup; ++tt) {
      if (t0 + tt < T) {
        const double s = wave_sum_f64_tree(acc[tt]);
        if (lane == 0) part[(static_cast<size_t>(t0 + tt) * E + e) * P + p] = s;
      }
    }
  }
}

// Large batches on the float64 matrix cores (v_mfma_f64_16x16x4_f64): a
// workgroup computes 64 tokens x 128 experts over one of P parts of d, each
// wavefront 64 tokens x 32 experts as 4 x 2 tiles of 16 x 16.  x and w are
// staged in LDS in their own types, 32 columns at a time (the next chunk's
// loads in flight during the current one's MFMAs); each lane reads its eight
// columns of a row with one vector read and widens them to float64 --
// exactly -- one per MFMA step.  Operand layout of the 16x16x4 f64
// MFMA: lane l holds A[l % 16][l / 16] and B[l / 16][l % 16]; it receives
// D[l / 16 + 4 * v][l % 16], v = 0..3.  Parts are multiples of 32 columns.
typedef double f64x4_t __attribute__((ext_vector_type(4)));
constexpr int kMT = 64, kME = 128, kMK = 32;
constexpr int kXPad = 8, kWPad = 4;  // LDS row padding (elements)

template <typename XT>
struct MfmaLogitsLds {
  static constexpr int kXLd = kMK + kXPad * (4 / static_cast<int>(sizeof(XT)));  // x row stride
  static constexpr int kWLd = kMK + kWPad;
  XT x[2][kMT][kXLd];
  float w[2][kME][kWLd];
  // each lane reads 8 consecutive columns of a row as 16-byte pieces
  static_assert(kXLd * sizeof(XT) % 16 == 0 && kWLd * sizeof(float) % 16 == 0 &&
                    sizeof(x) % 16 == 0 && kMK == 32,
                "16-byte aligned rows, four lanes of 8 columns per chunk");
};

template <typename XT>
__global__ __launch_bounds__(256) void logits_mfma(const void* __restrict__ x,
                                                    const float* __restrict__ w,
                                                    double* __restrict__ part, int T, int d,
                                                    int E, int P, int L) {
  using S = MfmaLogitsLds<XT>;
  __shared__ __align__(16) S sh;
  const int e0 = blockIdx.x * kME, t0 = blockIdx.y * kMT, p = blockIdx.z;
  const int k_begin = p * L, k_end = min(d, k_begin + L);
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  // staging: x rows as 16-byte pieces (XP per row), w rows as 8 pieces
  constexpr int XP = kMK * static_cast<int>(sizeof(XT)) / 16;  // 4 (bf16) or 8 (f32)
  constexpr int XN = kMT * XP / 256;                             // pieces per thread: 1 or 2
  const XT* xb = static_cast<const XT*>(x);
  uint4 rx[XN], rw[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < XN; ++u) {
      const int i = tid + 256 * u, r = i / XP, c = i % XP;
      const int t = min(t0 + r, T - 1);  // rows past T are zeroed at the store
      rx[u] = *reinterpret_cast<const uint4*>(xb + static_cast<size_t>(t) * d + k0 +
                                               c * (16 / static_cast<int>(sizeof(XT))));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 256 * u, r = i / 8, c = i % 8;
      const int e = min(e0 + r, E - 1);
      rw[u] = *reinterpret_cast<const uint4*>(w + static_cast<size_t>(e) * d + k0 + c * 4);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int u = 0; u < XN; ++u) {
      const int i = tid + 256 * u, r = i / XP, c = i % XP;
      const uint4 v = t0 + r < T ? rx[u] : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(&sh.x[buf][r][c * (16 / static_cast<int>(sizeof(XT)))]) = v;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 256 * u, r = i / 8, c = i % 8;
      const uint4 v = e0 + r < E ? rw[u] : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(&sh.w[buf][r][c * 4]) = v;
    }
  };
  f64x4_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  const int fr = lane & 15, fk = lane >> 4;  // fragment row / column of this lane
  if (k_begin < k_end) {
    load(k_begin);
    store(0);
  }
  __syncthreads();
  int buf = 0;
  for (int k0 = k_begin; k0 < k_end; k0 += kMK) {
    const bool more = k0 + kMK < k_end;
    if (more) load(k0 + kMK);
    // lane (fr, fk) takes columns 8 fk .. 8 fk + 7 of the chunk, one per
    // MFMA step (step s multiplies columns s, 8 + s, 16 + s, 24 + s), so its
    // operands are one contiguous LDS read per row
    XT xa[4][8];
    float wb[2][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (sizeof(XT) == 2) {
        const uint4 v = *reinterpret_cast<const uint4*>(&sh.x[buf][i * 16 + fr][8 * fk]);
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xa[i][2 * q] = static_cast<XT>(u[q] & 0xFFFFu);
          xa[i][2 * q + 1] = static_cast<XT>(u[q] >> 16);
        }
      } else {
        const float4 v0 = *reinterpret_cast<const float4*>(&sh.x[buf][i * 16 + fr][8 * fk]);
        const float4 v1 = *reinterpret_cast<const float4*>(&sh.x[buf][i * 16 + fr][8 * fk + 4]);
        const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) xa[i][q] = f[q];
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float4 v0 = *reinterpret_cast<const float4*>(&sh.w[buf][wv * 32 + j * 16 + fr][8 * fk]);
      const float4 v1 = *reinterpret_cast<const float4*>(&sh.w[buf][wv * 32 + j * 16 + fr][8 * fk + 4]);
      const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) wb[j][q] = f[q];
    }
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      double a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (sizeof(XT) == 2)
          a[i] = static_cast<double>(bf16_to_f32(xa[i][st]));
        else
          a[i] = static_cast<double>(xa[i][st]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = static_cast<double>(wb[j][st]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) store(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = t0 + i * 16 + fk + 4 * v;
      if (t >= T) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = e0 + wv * 32 + j * 16 + fr;
        if (e < E) part[(static_cast<size_t>(t) * E + e) * P + p] = acc[i][j][v];
      }
    }
  }
}

template <int NPL, int MP>
__global__ __launch_bounds__(256) void topk_softmax(const double* __restrict__ part, int P,
                                                    const float* __restrict__ bias, int T, int E,
                                                    int k, int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
  __shared__ TopkLds sh[4];
  const int wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;
  topk_token<NPL, MP>(part, P, bias, t, E, k, topk_idx, topk_w, sh[wv]);
}

// Top-k and batch-union in one workgroup, for batches whose T * k slots one
// wavefront can group (T <= kFusedMaxT, T * k <= 64): wavefront t runs the
// top-k of token t exactly as topk_softmax does, then wavefront 0 groups the
// chosen ids, read back from LDS, exactly as the stand-alone union kernel
// does.  One launch less per decode step.
constexpr int kFusedMaxT = 8;

template <int NPL, int MP, int EPL>
__global__ __launch_bounds__(64 * kFusedMaxT) void topk_union(
    const double* __restrict__ part, int P, const float* __restrict__ bias, int T, int E, int k,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active) {
  __shared__ TopkLds sh[kFusedMaxT];
  __shared__ int cnt[64 * EPL];
  __shared__ int first[64 * EPL];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wv < T) topk_token<NPL, MP>(part, P, bias, wv, E, k, topk_idx, topk_w, sh[wv]);
  __syncthreads();
  if (wv != 0) return;
  const int n = T * k;
  const int e = lane < n ? sh[lane / k].sel_e[lane % k] : -1;
  union_wave<EPL>(e, n, E, counts, offsets, perm, inv_perm, active, n_active, cnt, first);
}

}  // namespace

// Parts of d per logit, the same rule for every batch in a size class: the
// split kernel spreads the router matrix over E*P wavefronts; the matrix-core
// kernel cuts d into parts of at least 768 columns (384 measured slower for
// the 2048-token batch: twice the float64 partial sums to write and re-read).  The top-k kernel holds
// up to 16 parts for E <= 256, 8 for E <= 512, 4 beyond.
int route_parts(int T, int d, int E) {
  const int cap = E <= 256 ? 16 : (E <= 512 ? 8 : 4);
  int P;
  if (T <= kSplitMaxT) {
    P = 2048 / E;
    const int by_len = d / 256;
    if (P > by_len) P = by_len;
  } else {
    P = d / 768;
  }
  return P < 1 ? 1 : (P > cap ? cap : P);
}

size_t route_workspace(int T, int d, int E) {
  return static_cast<size_t>(T) * E * route_parts(T, d, E) * sizeof(double);
}

namespace {

hipError_t launch_logits(int T, int d, int E, int P, const void* x, bool x_bf16,
                         const float* w_router, double* logits, hipStream_t stream) {
  if (T <= kSplitMaxT) {
    const int L = ((d + P - 1) / P + 3) / 4 * 4;
    const dim3 grid((E * P + 3) / 4);
    return x_bf16 ? launch(logits_split<true>, grid, dim3(256), 0, stream, x, w_router, logits, T,
                          d, E, P, L)
                  : launch(logits_split<false>, grid, dim3(256), 0, stream, x, w_router, logits,
                           T, d, E, P, L);
  }
  const int L = ((d + P - 1) / P + kMK - 1) / kMK * kMK;
  const dim3 grid((E + kME - 1) / kME, (T + kMT - 1) / kMT, P);
  return x_bf16 ? launch(logits_mfma<uint16_t>, grid, dim3(256), 0, stream, x, w_router, logits,
                         T, d, E, P, L)
                : launch(logits_mfma<float>, grid, dim3(256), 0, stream, x, w_router, logits, T,
                         d, E, P, L);
}

// Parts held per logit by the top-k kernels: the next of 4, 8, 16 at or
// above P (route_parts caps P at 16 for E <= 256, 8 for E <= 512, 4 beyond).
template <int NPL>
hipError_t launch_topk(int T, int E, int k, int P, const double* part, const float* bias,
                       int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  constexpr int kCap = NPL <= 4 ? 16 : (NPL == 8 ? 8 : 4);
  const dim3 grid((T + 3) / 4), block(256);
  if (P <= 4)
    return launch(topk_softmax<NPL, 4>, grid, block, 0, stream, part, P, bias, T, E, k, topk_idx,
                  topk_w);
  if (P <= 8 || kCap == 8)
    return launch(topk_softmax<NPL, (kCap < 8 ? kCap : 8)>, grid, block, 0, stream, part, P, bias,
                  T, E, k, topk_idx, topk_w);
  return launch(topk_softmax<NPL, kCap>, grid, block, 0, stream, part, P, bias, T, E, k, topk_idx,
                topk_w);
}

hipError_t launch_topk_any(int T, int E, int k, int P, const double* part, const float* bias,
                           int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  if (E <= 64) return launch_topk<1>(T, E, k, P, part, bias, topk_idx, topk_w, stream);
  if (E <= 128) return launch_topk<2>(T, E, k, P, part, bias, topk_idx, topk_w, stream);
  if (E <= 256) return launch_topk<4>(T, E, k, P, part, bias, topk_idx, topk_w, stream);
  if (E <= 512) return launch_topk<8>(T, E, k, P, part, bias, topk_idx, topk_w, stream);
  return launch_topk<16>(T, E, k, P, part, bias, topk_idx, topk_w, stream);
}

template <int NPL, int EPL>
hipError_t launch_topk_union(int T, int E, int k, int P, const double* part, const float* bias,
                             int32_t* topk_idx, float* topk_w, const UnionOut& u,
                             hipStream_t stream) {
  const dim3 grid(1), block(64 * kFusedMaxT);
  if (P <= 8)
    return launch(topk_union<NPL, 8, EPL>, grid, block, 0, stream, part, P, bias, T, E, k,
                  topk_idx, topk_w, u.counts, u.offsets, u.perm, u.inv_perm, u.active,
                  u.n_active);
  return launch(topk_union<NPL, 16, EPL>, grid, block, 0, stream, part, P, bias, T, E, k, topk_idx,
                topk_w, u.counts, u.offsets, u.perm, u.inv_perm, u.active, u.n_active);
}

}  // namespace

hipError_t launch_route(int T, int d, int E, int k, const void* x, bool x_bf16,
                        const float* w_router, const float* bias, double* logits,
                        int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  const int P = route_parts(T, d, E);
  const hipError_t err = launch_logits(T, d, E, P, x, x_bf16, w_router, logits, stream);
  if (err != hipSuccess) return err;
  return launch_topk_any(T, E, k, P, logits, bias, topk_idx, topk_w, stream);
}

hipError_t launch_router_logits(int T, int d, int E, const void* x, bool x_bf16,
                                const float* w_router, double* part, hipStream_t stream) {
  return launch_logits(T, d, E, route_parts(T, d, E), x, x_bf16, w_router, part, stream);
}

hipError_t launch_route_union(int T, int d, int E, int k, const void* x, bool x_bf16,
                              const float* w_router, const float* bias, double* logits,
                              int32_t* topk_idx, float* topk_w, const UnionOut& u,
                              hipStream_t stream) {
  const int P = route_parts(T, d, E);
  hipError_t err = launch_logits(T, d, E, P, x, x_bf16, w_router, logits, stream);
  if (err != hipSuccess) return err;
  if (T <= kFusedMaxT && T * k <= 64 && E <= 256) {
    if (E <= 64)
      return launch_topk_union<1, 4>(T, E, k, P, logits, bias, topk_idx, topk_w, u, stream);
    if (E <= 128)
      return launch_topk_union<2, 4>(T, E, k, P, logits, bias, topk_idx, topk_w, u, stream);
    return launch_topk_union<4, 4>(T, E, k, P, logits, bias, topk_idx, topk_w, u, stream);
  }
  err = launch_topk_any(T, E, k, P, logits, bias, topk_idx, topk_w, stream);
  if (err != hipSuccess) return err;
  return launch_union(T * k, E, topk_idx, u.counts, u.offsets, u.perm, u.inv_perm, u.active,
                      u.n_active, stream);
}

}  // namespace moe
