// Batch-union grouping (pages: yunpan.plus article, "capability 2" -- an
// expert needed by several positions of one batch is read once; "capability
// 3" -- a worker receives one layer's routed batch-union and runs the FFN).
//
// One workgroup of 1024 threads does the whole grouping in LDS: a stable
// counting sort of the T*k routing slots by expert.  Each of the 16
// wavefronts owns a contiguous range of the slots.  It counts its slots per
// expert (LDS atomic adds: a count does not depend on the order they land
// in); a prefix over the wavefronts per expert and an exclusive scan over the
// experts give the offsets, the active-expert list and each wavefront's first
// position per expert; then each wavefront walks its range again in slot
// order and places every slot at its expert's next position plus its rank
// among the lanes of its 64-slot step with the same expert (ballots).  Three
// barriers between the phases, and the permutation is the stable one by
// construction.
#include "common.h"
#include "launch.h"
#include "union_wave.h"

namespace moe {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxE = 1024;
constexpr int kKeys = 16;  // slot keys a lane holds at a time

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
  __shared__ int start[kMaxE];    // the experts' counts, then their offsets
  __shared__ int flag[kMaxE];
  __shared__ int scan_tmp[kWaves];
  extern __shared__ int tab[];    // [kWaves][E]: slots per wavefront and expert, then the
                                  // wavefront's next grouped position per expert
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int nbits = key_bits(E);
  // wavefront wv owns the slots [s0, s0 + 64 * spw), whole 64-slot steps
  const int spw = ((n + 63) / 64 + kWaves - 1) / kWaves;
  const int s0 = wv * spw * 64;
  for (int i = tid; i < kWaves * E; i += kThreads) tab[i] = 0;
  __syncthreads();
  // counts per wavefront and expert: LDS atomic adds (counts do not depend
  // on the order the adds land in; 16 keys in flight per lane)
  for (int b0 = 0; b0 < spw; b0 += kKeys) {
    int key[kKeys];
#pragma unroll
    for (int u = 0; u < kKeys; ++u)  // (steps past the wavefront's range are not its slots)
      key[u] = b0 + u < spw ? key_of(topk_idx, s0 + (b0 + u) * 64 + lane, n, E) : -1;
#pragma unroll
    for (int u = 0; u < kKeys; ++u)
      if (key[u] >= 0) atomicAdd(&tab[wv * E + key[u]], 1);
  }
  __syncthreads();
  // per expert: exclusive prefix over the wavefronts, and the total
  for (int e = tid; e < E; e += kThreads) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int c = tab[w * E + e];
      tab[w * E + e] = run;
      run += c;
    }
    counts[e] = run;
    cnt[e] = run;
    start[e] = run;
    flag[e] = run > 0 ? 1 : 0;
  }
  __syncthreads();
  const int total = block_exclusive_scan(start, E, scan_tmp);
  const int n_act = block_exclusive_scan(flag, E, scan_tmp);
  for (int e = tid; e < E; e += kThreads) {
    offsets[e] = start[e];
    if (cnt[e] > 0) active[flag[e]] = e;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tab[w * E + e] += start[e];
  }
  for (int i = n_act + tid; i < E; i += kThreads) active[i] = -1;
  if (tid == 0) {
    offsets[E] = total;
    n_active[0] = n_act;
  }
  __syncthreads();
  // Stable placement: each wavefront walks its slots in order; a slot goes
  // to its expert's next position for this wavefront plus its rank among the
  // lower lanes of its step with the same expert, and the expert's lowest
  // lane then advances that position past the step's lanes.
  for (int b0 = 0; b0 < spw; b0 += kKeys) {
    int key[kKeys];
#pragma unroll
    for (int u = 0; u < kKeys; ++u) key[u] = key_of(topk_idx, s0 + (b0 + u) * 64 + lane, n, E);
#pragma unroll
    for (int u = 0; u < kKeys; ++u) {
      if (b0 + u >= spw) break;  // (uniform)
      const int s = s0 + (b0 + u) * 64 + lane;
      const bool valid = key[u] >= 0;
      const uint64_t same = match_key(key[u], valid, nbits);
      const int rank = __popcll(same & ((1ull << lane) - 1ull));
      if (valid) {
        const int pos = tab[wv * E + key[u]] + rank;
        perm[pos] = s;
        inv_perm[s] = pos;
      } else if (s < n) {
        inv_perm[s] = -1;
      }
      __builtin_amdgcn_wave_barrier();
      if (valid && rank == 0) tab[wv * E + key[u]] += __popcll(same);
      __builtin_amdgcn_wave_barrier();
    }
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
  const int lds = kWaves * E * static_cast<int>(sizeof(int));
  if (lds > 48 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(batch_union),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  return launch(batch_union, dim3(1), dim3(kThreads), lds, stream, topk_idx, n_slots, E, counts,
                offsets, perm, inv_perm, active, n_active);
}

}  // namespace moe
