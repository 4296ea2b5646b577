// Batch-union grouping (pages: yunpan.plus article, "capability 2" -- an
// expert needed by several positions of one batch is read once; "capability
// 3" -- a worker receives one layer's routed batch-union and runs the FFN).
//
// One workgroup of 1024 threads does the whole grouping in LDS: a histogram
// of the T*k routing slots per expert, an exclusive scan into offsets, the
// active-expert list, then a stable counting sort of the slots.  Slots are
// taken in chunks of 1024 in id order; inside a chunk each wavefront ranks its
// lanes among equal keys with ballots, and wavefronts are ordered by a
// per-chunk table of per-wave key counts, so the permutation is the stable
// one regardless of the order in which hardware atomics land.
#include "common.h"
#include "launch.h"
#include "union_wave.h"

namespace moe {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxE = 1024;

// Exclusive scan of n <= 2 * kThreads ints in LDS (in place), returns the
// total.
__device__ int block_exclusive_scan(int* a, int n, int* tmp) {
  // each thread owns two consecutive entries
  const int tid = threadIdx.x;
  const int i0 = 2 * tid, i1 = 2 * tid + 1;
  const int v0 = i0 < n ? a[i0] : 0;
  const int v1 = i1 < n ? a[i1] : 0;
  int s = v0 + v1;
  // inclusive scan of s over the threads: wave scan then wave totals
  const int lane = tid & 63, wv = tid >> 6;
  int incl = s;
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) tmp[wv] = incl;
  __syncthreads();
  int wave_base = 0;
  for (int w = 0; w < wv; ++w) wave_base += tmp[w];
  int total = 0;
  for (int w = 0; w < kWaves; ++w) total += tmp[w];
  const int excl = wave_base + incl - s;
  __syncthreads();
  if (i0 < n) a[i0] = excl;
  if (i1 < n) a[i1] = excl + v0;
  __syncthreads();
  return total;
}

__device__ __forceinline__ int key_of(const int32_t* __restrict__ topk_idx, int s, int n, int E) {
  const int e = s < n ? topk_idx[s] : -1;
  return (e >= 0 && e < E) ? e : -1;
}

// Dynamic LDS: wave_cnt and wave_pre, kWaves * E ints each.
__global__ __launch_bounds__(kThreads) void batch_union(const int32_t* __restrict__ topk_idx,
                                                        int n, int E, int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ perm,
                                                        int32_t* __restrict__ inv_perm,
                                                        int32_t* __restrict__ active,
                                                        int32_t* __restrict__ n_active) {
  __shared__ int cnt[kMaxE];
  __shared__ int start[kMaxE];    // next free grouped position per expert
  __shared__ int flag[kMaxE];
  __shared__ int scan_tmp[kWaves];
  extern __shared__ int dyn[];
  int* wave_cnt = dyn;            // [kWaves][E] slots of the chunk per wave and expert
  int* wave_pre = dyn + kWaves * E;  // [kWaves][E] first grouped position of each
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;

  for (int e = tid; e < E; e += kThreads) cnt[e] = 0;
  for (int i = tid; i < kWaves * E; i += kThreads) wave_cnt[i] = 0;
  __syncthreads();
  // histogram: four keys per thread in flight at a time
  for (int s0 = tid; s0 < n; s0 += 4 * kThreads) {
    int e[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) e[u] = key_of(topk_idx, s0 + u * kThreads, n, E);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (e[u] >= 0) atomicAdd(&cnt[e[u]], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    counts[e] = cnt[e];
    start[e] = cnt[e];
    flag[e] = cnt[e] > 0 ? 1 : 0;
  }
  __syncthreads();
  const int total = block_exclusive_scan(start, E, scan_tmp);
  const int n_act = block_exclusive_scan(flag, E, scan_tmp);
  for (int e = tid; e < E; e += kThreads) {
    offsets[e] = start[e];
    if (cnt[e] > 0) active[flag[e]] = e;
  }
  for (int i = n_act + tid; i < E; i += kThreads) active[i] = -1;
  if (tid == 0) {
    offsets[E] = total;
    n_active[0] = n_act;
  }
  __syncthreads();

  // Stable placement, one chunk of kThreads slots at a time (the next
  // chunk's keys are loaded while this one is placed).  A slot's position is
  // its expert's next free position, plus the expert's slots in lower
  // wavefronts of the chunk, plus its rank among the lower lanes of its own
  // wavefront with the same expert.
  const int nbits = key_bits(E);
  int e_next = key_of(topk_idx, tid, n, E);
  for (int c0 = 0; c0 < n; c0 += kThreads) {
    const int s = c0 + tid;
    const int e = e_next;
    e_next = key_of(topk_idx, s + kThreads, n, E);
    const bool valid = e >= 0;
    const uint64_t same = match_key(e, valid, nbits);
    const int rank = __popcll(same & ((1ull << lane) - 1ull));
    // the expert's lowest lane in the wavefront writes its count
    if (valid && rank == 0) wave_cnt[wv * E + e] = __popcll(same);
    __syncthreads();
    // per expert: exclusive prefix over the wavefronts, from its next free
    // position
    for (int ee = tid; ee < E; ee += kThreads) {
      int run = start[ee];
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        wave_pre[w * E + ee] = run;
        run += wave_cnt[w * E + ee];
      }
      start[ee] = run;
    }
    __syncthreads();
    if (s < n) {
      if (valid) {
        const int pos = wave_pre[wv * E + e] + rank;
        perm[pos] = s;
        inv_perm[s] = pos;
      } else {
        inv_perm[s] = -1;
      }
    }
    // the lane of rank 0 of each expert in a wavefront is the one that wrote
    // its count: it clears it for the next chunk
    if (valid && rank == 0) wave_cnt[wv * E + e] = 0;
    __syncthreads();
  }
}

// Small batches (at most 64 slots, e.g. decode up to 8 tokens at k=8): one
// wavefront, no workgroup barriers (union_wave.h).
template <int EPL>
__global__ __launch_bounds__(64) void batch_union_small(const int32_t* __restrict__ topk_idx,
                                                         int n, int E,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ perm,
                                                         int32_t* __restrict__ inv_perm,
                                                         int32_t* __restrict__ active,
                                                         int32_t* __restrict__ n_active) {
  __shared__ int cnt[64 * EPL];
  __shared__ int first[64 * EPL];
  const int lane = threadIdx.x;
  const int e = lane < n ? topk_idx[lane] : -1;
  union_wave<EPL>(e, n, E, counts, offsets, perm, inv_perm, active, n_active, cnt, first);
}

}  // namespace

hipError_t launch_union(int n_slots, int E, const int32_t* topk_idx, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* active,
                        int32_t* n_active, hipStream_t stream) {
  if (n_slots <= 64) {
    if (E <= 256)
      return launch(batch_union_small<4>, dim3(1), dim3(64), 0, stream, topk_idx, n_slots, E,
                    counts, offsets, perm, inv_perm, active, n_active);
    return launch(batch_union_small<16>, dim3(1), dim3(64), 0, stream, topk_idx, n_slots, E,
                  counts, offsets, perm, inv_perm, active, n_active);
  }
  const int lds = 2 * kWaves * E * static_cast<int>(sizeof(int));
  if (lds > 48 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(batch_union),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  return launch(batch_union, dim3(1), dim3(kThreads), lds, stream, topk_idx, n_slots, E, counts,
                offsets, perm, inv_perm, active, n_active);
}

}  // namespace moe
