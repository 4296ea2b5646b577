// Weight quantiser: float weights -> int4 codes + float16 scales, the
// one-time conversion the pages' engine runs on a checkpoint before serving
// (ssnai.com digest, first-command section; yunpan.plus article, "capability
// 4": int4 experts with gs64 scales, compared there with one scale per row).
//
//   s = float16(float32(absmax) / 7)     absmax over a 64-column group (GS64)
//                                        or over the whole row (ROW)
//   q = nearest integer to w / s, ties to even, in [-8, 7]; s == 0 gives q = 0
//
// Codes go out in the canonical layout (row-major [N][K/2], element 2j in the
// low nibble of byte j).  The rounding of every code is decided exactly: a
// product with an approximate reciprocal settles every code that is not near
// a half-way point, and for those the half-way points (2q +- 1) * s, exact in
// float32 (a float16 times an odd number below 17), are compared with 2w.  Memory-bound: 2 (bf16) or 4 (f32) bytes read and
// ~0.53 bytes written per weight.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

template <bool F32>
__device__ __forceinline__ void load8(const void* w, size_t idx, float (&v)[8]) {
  if constexpr (F32) {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(w) + idx);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(w) + idx + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(w) + idx);
    const uint32_t u[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  }
}

__device__ __forceinline__ float scale_of(float absmax) {
  // float32 division (correctly rounded), then round to float16
  return static_cast<float>(static_cast<_Float16>(absmax / 7.0f));
}

// The nearest integer to w / s with ties to even, clipped to [-8, 7].  inv is
// an approximate 1 / s (0 when s is 0): t = w * inv is within 1e-5 of w / s,
// so rounding t is exact unless t lies within 1e-4 of a half-integer; only
// then are the half-way points compared with 2w exactly.
__device__ __forceinline__ int code_of(float w, float s, float inv) {
  const float t = w * inv;
  const float qf = rintf(t);
  int q = static_cast<int>(qf);
  if (fabsf(t - qf) > 0.4999f) {
    q = max(-9, min(8, q));
    const float w2 = 2.0f * w;
    const float lo = static_cast<float>(2 * q - 1) * s, hi = static_cast<float>(2 * q + 1) * s;
    if (w2 < lo) {
      --q;
    } else if (w2 > hi) {
      ++q;
    } else if (w2 == lo) {
      if (q & 1) --q;  // tie between q - 1 and q: the even one
    } else if (w2 == hi) {
      if (q & 1) ++q;
    }
  }
  return max(-8, min(7, q));
}

__device__ __forceinline__ uint32_t pack8(const float (&v)[8], float s) {
  const float inv = s != 0.0f ? __builtin_amdgcn_rcpf(s) : 0.0f;
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) r |= (static_cast<uint32_t>(code_of(v[i], s, inv)) & 0xFu) << (4 * i);
  return r;
}

// GS64: 8 lanes per group, 8 consecutive weights per lane; the group's
// absolute maximum is reduced over its 8 lanes.
template <bool F32>
__global__ __launch_bounds__(256) void quant_gs64(const void* __restrict__ w, int /*K*/, long long groups,
                                                  uint32_t* __restrict__ codes,
                                                  _Float16* __restrict__ scales) {
  const long long t = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const long long grp = t >> 3;
  const bool live = grp < groups;
  const long long gg = live ? grp : groups - 1;  // lanes past the end redo the last group
  const int part = threadIdx.x & 7;
  const size_t idx = static_cast<size_t>(gg) * 64 + part * 8;
  float v[8];
  load8<F32>(w, idx, v);
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  m = fmaxf(m, __shfl_xor(m, 1, kWave));
  m = fmaxf(m, __shfl_xor(m, 2, kWave));
  m = fmaxf(m, __shfl_xor(m, 4, kWave));
  const float s = scale_of(m);
  if (!live) return;
  codes[idx / 8] = pack8(v, s);
  if (part == 0) scales[gg] = static_cast<_Float16>(s);
}

// ROW: one workgroup per row; the row's absolute maximum first, then the codes
// (the second read of the row hits the cache).
template <bool F32>
__global__ __launch_bounds__(256) void quant_row(const void* __restrict__ w, int K,
                                                 uint32_t* __restrict__ codes,
                                                 _Float16* __restrict__ scales) {
  __shared__ float wmax[4];
  const int r = blockIdx.x;
  const size_t base = static_cast<size_t>(r) * K;
  float m = 0.0f;
  for (int c = threadIdx.x * 8; c < K; c += 256 * 8) {
    float v[8];
    load8<F32>(w, base + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = scale_of(m);
  for (int c = threadIdx.x * 8; c < K; c += 256 * 8) {
    float v[8];
    load8<F32>(w, base + c, v);
    codes[(base + c) / 8] = pack8(v, s);
  }
  if (threadIdx.x == 0) scales[r] = static_cast<_Float16>(s);
}

}  // namespace

hipError_t launch_quantize(int N, int K, const void* w, bool f32, bool per_row, uint8_t* codes,
                           void* scales, hipStream_t stream) {
  uint32_t* c = reinterpret_cast<uint32_t*>(codes);
  _Float16* s = static_cast<_Float16*>(scales);
  if (per_row)
    return f32 ? launch(quant_row<true>, dim3(N), dim3(256), 0, stream, w, K, c, s)
               : launch(quant_row<false>, dim3(N), dim3(256), 0, stream, w, K, c, s);
  const long long groups = static_cast<long long>(N) * (K / 64);
  const unsigned grid = static_cast<unsigned>((groups * 8 + 255) / 256);
  return f32 ? launch(quant_gs64<true>, dim3(grid), dim3(256), 0, stream, w, K, groups, c, s)
             : launch(quant_gs64<false>, dim3(grid), dim3(256), 0, stream, w, K, groups, c, s);
}

}  // namespace moe
