// Calibration kernel for the benchmark's roofline: a plain streaming read of
// a set of equal-size blocks (the expert blocks one decode step reads), split
// evenly over the workgroups, with no arithmetic beyond folding the loaded
// words together.  Its rate is what a read-only kernel of the same bytes
// attains on this GPU, the ceiling the decode FFN is compared with beside the
// published HBM peak.
#include <hip/hip_runtime.h>

#include "launch.h"
#include "moe_int4_measure.h"

namespace moe {
namespace {

constexpr int kReadThreads = 256;
constexpr int kMaxReadBlocks = 64;
constexpr int kUnroll = 4;  // 16-byte loads in flight per thread and iteration

struct ReadArgs {
  const uint8_t* blocks[kMaxReadBlocks];
};

// Workgroup w reads share w % wpb of block w / wpb (wpb workgroups per
// block, each share a whole number of 16-byte pieces); each thread XORs what
// it loads and one word per workgroup is written, so no load can be dropped.
__global__ __launch_bounds__(kReadThreads) void stream_read(ReadArgs a, int wpb,
                                                            unsigned long long block_bytes,
                                                            unsigned long long per,
                                                            uint32_t* sink) {
  const int b = blockIdx.x / wpb, s = blockIdx.x - b * wpb;
  const unsigned long long lo = per * s;
  const unsigned long long hi = lo + per < block_bytes ? lo + per : block_bytes;
  const uint8_t* base = a.blocks[b];
  uint4 acc = make_uint4(0u, 0u, 0u, 0u);
  constexpr unsigned long long kStride = 16ull * kReadThreads * kUnroll;
  for (unsigned long long o = lo + 16ull * threadIdx.x; o < hi; o += kStride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const unsigned long long p = o + 16ull * kReadThreads * u;
      v[u] = p < hi ? *reinterpret_cast<const uint4*>(base + p) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      acc.x ^= v[u].x;
      acc.y ^= v[u].y;
      acc.z ^= v[u].z;
      acc.w ^= v[u].w;
    }
  }
  uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int off = 32; off > 0; off >>= 1) r ^= __shfl_xor(r, off, 64);
  __shared__ uint32_t part[kReadThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = r;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace
}  // namespace moe

extern "C" {

moe_status moe_measure_stream_read(const uint8_t* const* blocks, int32_t n_blocks,
                                   size_t block_bytes, int32_t workgroups, uint32_t* sink,
                                   void* stream) {
  if (!blocks || !sink) return MOE_ERR_NULL;
  if (n_blocks < 1 || n_blocks > moe::kMaxReadBlocks || workgroups < n_blocks ||
      workgroups > 65536 || block_bytes == 0 || block_bytes % 16)
    return MOE_ERR_SHAPE;
  moe::ReadArgs a{};
  for (int i = 0; i < n_blocks; ++i) {
    if (!blocks[i]) return MOE_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(blocks[i]) % 16) return MOE_ERR_ALIGN;
    a.blocks[i] = blocks[i];
  }
  if (reinterpret_cast<uintptr_t>(sink) % 4) return MOE_ERR_ALIGN;
  // wpb equal shares of every block, each a whole number of 16-byte pieces;
  // wpb * n_blocks <= workgroups, the size of sink
  const int wpb = workgroups / n_blocks;
  unsigned long long per = (static_cast<unsigned long long>(block_bytes) + wpb - 1) / wpb;
  per = (per + 15) / 16 * 16;
  const hipError_t err =
      moe::launch(moe::stream_read, dim3(wpb * n_blocks), dim3(moe::kReadThreads), 0,
                  static_cast<hipStream_t>(stream), a, wpb,
                  static_cast<unsigned long long>(block_bytes), per, sink);
  return err == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
