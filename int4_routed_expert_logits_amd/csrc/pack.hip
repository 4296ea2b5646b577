// Canonical expert block -> packed expert block (a byte bijection of the
// same size), the one-time conversion the kernels read from (the pages'
// engine also converts its checkpoint once before serving: ssnai.com digest,
// "第一步命令" (first command); yunpan.plus article, quick-start section).
//
// For every matrix W [N][K] of a block (gate, up, down) the codes are
// regrouped into tiles of 64 rows: tile t, 32-column chunk c, row-in-tile l
// holds 16 bytes at
//     q_off + t*(64*K/2) + c*1024 + l*16
// so one 16-byte load per lane of a wavefront reads 64 rows x 32 columns as
// one contiguous kilobyte.  Inside each 4-byte word (8 columns 8w..8w+7) the
// nibble of column 8w+j moves to bit 4*(j/2) + 16*(j%2), so that
// (word >> 4i) & 0x000F000F holds columns (8w+2i, 8w+2i+1) in its two
// 16-bit halves, and each nibble is stored in offset binary (the
// two's-complement code q with its top bit flipped, i.e. q + 8 in [0, 15]),
// so that one OR with 0x43004300 turns such a pair into the exact bf16 pair
// (136 + q_a, 136 + q_b).  Scales follow the same 64-row tiles, group-major inside a
// tile: row t*64+l, group g goes to
//     s_off + (t*(K/64)*64 + g*64 + l)*2
// so the scales of one group for a whole tile are one 128-byte run (a
// kernel that walks the groups reads whole lines), and a tile's scales are
// still one contiguous piece.  The offsets q_off / s_off of the six
// sub-arrays are those of the canonical block.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace moe {

namespace {

struct PackArgs {
  const uint8_t* src;
  uint8_t* dst;
  size_t block_bytes;
  int d, f;
  long long units_per_block;   // code units (16 B) of the three matrices
  long long sunits_per_block;  // scale units (2 B) of the three matrices
  long long n_blocks;
};

__device__ __forceinline__ uint32_t interleave_word(uint32_t w) {
  uint32_t out = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) out |= ((w >> (4 * j)) & 0xFu) << (4 * (j >> 1) + 16 * (j & 1));
  return out ^ 0x88888888u;  // q -> q + 8 in every nibble
}

struct MatGeom {
  int N, K;
  size_t q_off, s_off;
  long long units, sunits;
};

__device__ __forceinline__ void geom(const PackArgs& a, int m, MatGeom& g) {
  const size_t dd = a.d, ff = a.f;
  const size_t s0 = 3 * dd * ff / 2;
  if (m == 0) {
    g.N = a.f; g.K = a.d; g.q_off = 0; g.s_off = s0;
  } else if (m == 1) {
    g.N = a.f; g.K = a.d; g.q_off = ff * dd / 2; g.s_off = s0 + ff * (dd / 64) * 2;
  } else {
    g.N = a.d; g.K = a.f; g.q_off = ff * dd; g.s_off = s0 + 2 * ff * (dd / 64) * 2;
  }
  g.units = static_cast<long long>(g.N) * (g.K / 32);
  g.sunits = static_cast<long long>(g.N) * (g.K / 64);
}

__global__ __launch_bounds__(256) void pack_codes(PackArgs a) {
  const long long total = a.units_per_block * a.n_blocks;
  for (long long i = blockIdx.x * 256ll + threadIdx.x; i < total; i += 256ll * gridDim.x) {
    const long long b = i / a.units_per_block;
    long long u = i - b * a.units_per_block;
    MatGeom g;
    int m = 0;
    for (; m < 3; ++m) {
      geom(a, m, g);
      if (u < g.units) break;
      u -= g.units;
    }
    const int cpr = g.K / 32;  // chunks per row
    const int r = static_cast<int>(u / cpr), c = static_cast<int>(u % cpr);
    const uint8_t* blk_src = a.src + b * a.block_bytes;
    uint8_t* blk_dst = a.dst + b * a.block_bytes;
    const uint4 v = *reinterpret_cast<const uint4*>(blk_src + g.q_off +
                                                    static_cast<size_t>(r) * (g.K / 2) + c * 16);
    const uint4 o = make_uint4(interleave_word(v.x), interleave_word(v.y), interleave_word(v.z),
                               interleave_word(v.w));
    const size_t dst_off = g.q_off + static_cast<size_t>(r / 64) * (64 * static_cast<size_t>(g.K) / 2) +
                           static_cast<size_t>(c) * 1024 + static_cast<size_t>(r % 64) * 16;
    *reinterpret_cast<uint4*>(blk_dst + dst_off) = o;
  }
}

__global__ __launch_bounds__(256) void pack_scales(PackArgs a) {
  const long long total = a.sunits_per_block * a.n_blocks;
  for (long long i = blockIdx.x * 256ll + threadIdx.x; i < total; i += 256ll * gridDim.x) {
    const long long b = i / a.sunits_per_block;
    long long u = i - b * a.sunits_per_block;
    MatGeom g;
    int m = 0;
    for (; m < 3; ++m) {
      geom(a, m, g);
      if (u < g.sunits) break;
      u -= g.sunits;
    }
    const uint16_t* s = reinterpret_cast<const uint16_t*>(a.src + b * a.block_bytes + g.s_off);
    uint16_t* d = reinterpret_cast<uint16_t*>(a.dst + b * a.block_bytes + g.s_off);
    const int G = g.K / 64;
    const long long r = u / G, grp = u - r * G;
    d[(r / 64) * G * 64 + grp * 64 + r % 64] = s[u];
  }
}

// MXFP4 blocks (E2M1 nibbles, one E8M0 byte per 32 elements): the codes move
// to the same 64-row tiles but keep their nibble order and values (the
// hardware's FP4 -> bf16 conversion takes a byte as two neighbouring
// elements); the scale bytes follow the tiles block-major: row t*64+l, block
// b at s_off + t*(K/32)*64 + b*64 + l.
__device__ __forceinline__ void geom_mx(const PackArgs& a, int m, MatGeom& g) {
  const size_t dd = a.d, ff = a.f;
  const size_t s0 = 3 * dd * ff / 2;
  if (m == 0) {
    g.N = a.f; g.K = a.d; g.q_off = 0; g.s_off = s0;
  } else if (m == 1) {
    g.N = a.f; g.K = a.d; g.q_off = ff * dd / 2; g.s_off = s0 + ff * (dd / 32);
  } else {
    g.N = a.d; g.K = a.f; g.q_off = ff * dd; g.s_off = s0 + 2 * ff * (dd / 32);
  }
  g.units = static_cast<long long>(g.N) * (g.K / 32);
  g.sunits = static_cast<long long>(g.N) * (g.K / 32);
}

__global__ __launch_bounds__(256) void pack_codes_mx(PackArgs a) {
  const long long total = a.units_per_block * a.n_blocks;
  for (long long i = blockIdx.x * 256ll + threadIdx.x; i < total; i += 256ll * gridDim.x) {
    const long long b = i / a.units_per_block;
    long long u = i - b * a.units_per_block;
    MatGeom g;
    int m = 0;
    for (; m < 3; ++m) {
      geom_mx(a, m, g);
      if (u < g.units) break;
      u -= g.units;
    }
    const int cpr = g.K / 32;
    const int r = static_cast<int>(u / cpr), c = static_cast<int>(u % cpr);
    const uint4 v = *reinterpret_cast<const uint4*>(a.src + b * a.block_bytes + g.q_off +
                                                    static_cast<size_t>(r) * (g.K / 2) + c * 16);
    const size_t dst_off = g.q_off + static_cast<size_t>(r / 64) * (64 * static_cast<size_t>(g.K) / 2) +
                           static_cast<size_t>(c) * 1024 + static_cast<size_t>(r % 64) * 16;
    *reinterpret_cast<uint4*>(a.dst + b * a.block_bytes + dst_off) = v;
  }
}

__global__ __launch_bounds__(256) void pack_scales_mx(PackArgs a) {
  const long long total = a.sunits_per_block * a.n_blocks;
  for (long long i = blockIdx.x * 256ll + threadIdx.x; i < total; i += 256ll * gridDim.x) {
    const long long b = i / a.sunits_per_block;
    long long u = i - b * a.sunits_per_block;
    MatGeom g;
    int m = 0;
    for (; m < 3; ++m) {
      geom_mx(a, m, g);
      if (u < g.sunits) break;
      u -= g.sunits;
    }
    const uint8_t* s = a.src + b * a.block_bytes + g.s_off;
    uint8_t* d = a.dst + b * a.block_bytes + g.s_off;
    const int G = g.K / 32;
    const long long r = u / G, blk = u - r * G;
    d[(r / 64) * G * 64 + blk * 64 + r % 64] = s[u];
  }
}

}  // namespace

hipError_t launch_pack_mxfp4(int d, int f, long long n_blocks, size_t block_bytes,
                             const uint8_t* src, uint8_t* dst, hipStream_t stream) {
  PackArgs a{};
  a.src = src;
  a.dst = dst;
  a.block_bytes = block_bytes;
  a.d = d;
  a.f = f;
  a.units_per_block = 3ll * d * f / 32;
  a.sunits_per_block = 3ll * d * f / 32;
  a.n_blocks = n_blocks;
  const long long total = a.units_per_block * n_blocks;
  const unsigned grid = static_cast<unsigned>(std::min<long long>((total + 255) / 256, 1 << 16));
  hipError_t e = launch(pack_codes_mx, dim3(grid), dim3(256), 0, stream, a);
  if (e != hipSuccess) return e;
  return launch(pack_scales_mx, dim3(grid), dim3(256), 0, stream, a);
}

hipError_t launch_pack(int d, int f, long long n_blocks, size_t block_bytes, const uint8_t* src,
                       uint8_t* dst, hipStream_t stream) {
  PackArgs a{};
  a.src = src;
  a.dst = dst;
  a.block_bytes = block_bytes;
  a.d = d;
  a.f = f;
  a.units_per_block = 3ll * d * f / 32;
  a.sunits_per_block = 3ll * d * f / 64;
  a.n_blocks = n_blocks;
  const long long total = a.units_per_block * n_blocks;
  const unsigned grid = static_cast<unsigned>(std::min<long long>((total + 255) / 256, 1 << 16));
  hipError_t e = launch(pack_codes, dim3(grid), dim3(256), 0, stream, a);
  if (e != hipSuccess) return e;
  const long long stotal = a.sunits_per_block * n_blocks;
  const unsigned sgrid = static_cast<unsigned>(std::min<long long>((stotal + 255) / 256, 1 << 16));
  return launch(pack_scales, dim3(sgrid), dim3(256), 0, stream, a);
}

}  // namespace moe
