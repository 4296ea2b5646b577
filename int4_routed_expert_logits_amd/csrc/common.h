// Device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;  // CDNA wavefront width

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// a.lo*b.lo + a.hi*b.hi + c with both operands holding two bfloat16 values;
// the products are exact in float32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// (v & mask) | bits in one VALU instruction (v_and_or_b32).  With both
// constants known, the compiler emits an AND and an OR with a literal each (a
// gfx9 VOP3 instruction reads at most one scalar or literal operand); an
// empty asm statement hides the value of `bits` in a vector register, so the
// and-or pattern is selected with the mask in a scalar register.  The asm
// emits no instruction: every instruction here is the compiler's own, and so
// is the hazard bookkeeping between it and the matrix instructions that
// read its result.
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t c) {
  asm("" : "+v"(c));
  return c;
}

__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t mask, uint32_t bits_vgpr) {
  return (v & mask) | bits_vgpr;
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64);
// every lane of a group receives the group's sum.
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Lane permutation of a double inside rows of 16 lanes (DPP control CTRL).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      0, static_cast<int>(static_cast<uint32_t>(b)), CTRL, 0xF, 0xF, false));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
      0, static_cast<int>(static_cast<uint32_t>(b >> 32)), CTRL, 0xF, 0xF, false));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(b)), lane));
  const uint32_t hi = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(b >> 32)), lane));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// Wave-wide float64 sum over a fixed tree (pairs, quads, 8s, 16s inside each
// row through DPP, then the four row sums), so the result does not depend on
// scheduling; every lane receives it.  Addition is commutative in IEEE
// arithmetic, so both lanes of each exchange hold the same partial sum.
__device__ __forceinline__ double wave_sum_f64_tree(double v) {
  v += dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f64<0x141>(v);  // row_half_mirror
  v += dpp_f64<0x140>(v);  // row_mirror
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// E8M0 scale byte (MX formats) -> 2^(E - 127) as float32: E = 0 is the
// subnormal 2^-127, E = 255 is NaN.  E << 23 is the float for E in 1 .. 254;
// bit 22 turns E = 0 into 2^-127 and E = 255 (infinity) into a quiet NaN.
// Written without branches, so it costs two compares and no control flow.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  const uint32_t edge = static_cast<uint32_t>(e == 0u) | static_cast<uint32_t>(e == 255u);
  return __uint_as_float((e << 23) | (edge << 22));
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

}  // namespace moe
