// Batch-union grouping of at most 64 routing slots by one wavefront, shared
// by the stand-alone union kernel and the fused route + union kernel (pages:
// yunpan.plus article, "capability 2" -- an expert needed by several
// positions of one batch is read once).
//
// Lane s holds slot s; the histogram is built with LDS atomics, every lane
// scans a contiguous block of EPL experts, and a slot's grouped position is
// its expert's offset plus the number of lower slots with the same expert
// (match_key rank), which is the stable order by (expert, slot).  Ids outside
// [0, E) are not grouped (inv_perm = -1).
#pragma once

#include "common.h"

namespace moe {

// Mask of the lanes of this wavefront whose key equals this lane's, among
// the lanes with valid set: one ballot per key bit (keys < 2^nbits), each
// lane keeping the lanes that agree with it on that bit.  No loop over the
// distinct keys.
__device__ __forceinline__ uint64_t match_key(int key, bool valid, int nbits) {
  uint64_t same = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t m = __ballot(bit);
    same &= bit ? m : ~m;
  }
  return same;
}

// Bits of an expert id below E.
__device__ __forceinline__ int key_bits(int E) { return E > 1 ? 32 - __clz(E - 1) : 0; }

// cnt, first: LDS scratch of 64 * EPL ints each.  e: this lane's slot's
// expert id (any value for lanes >= n).
template <int EPL>
__device__ __forceinline__ void union_wave(int e, int n, int E, int32_t* __restrict__ counts,
                                           int32_t* __restrict__ offsets,
                                           int32_t* __restrict__ perm,
                                           int32_t* __restrict__ inv_perm,
                                           int32_t* __restrict__ active,
                                           int32_t* __restrict__ n_active, int* cnt, int* first) {
  const int lane = threadIdx.x & 63;
  const bool valid = lane < n && e >= 0 && e < E;
  if (!valid) e = -1;
#pragma unroll
  for (int i = 0; i < EPL; ++i) cnt[lane * EPL + i] = 0;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (valid) atomicAdd(&cnt[e], 1);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  int c[EPL];
  int sum = 0, act = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    c[i] = cnt[lane * EPL + i];
    sum += c[i];
    act += c[i] > 0 ? 1 : 0;
  }
  int isum = sum, iact = act;  // inclusive scans over lanes
  for (int off = 1; off < 64; off <<= 1) {
    const int os = __shfl_up(isum, off, 64);
    const int oa = __shfl_up(iact, off, 64);
    if (lane >= off) {
      isum += os;
      iact += oa;
    }
  }
  int base = isum - sum, abase = iact - act;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int ee = lane * EPL + i;
    if (ee < E) {
      counts[ee] = c[i];
      offsets[ee] = base;
      if (c[i] > 0) active[abase++] = ee;
    }
    first[ee] = base;
    base += c[i];
  }
  const int total = __shfl(isum, 63, 64);
  const int n_act = __shfl(iact, 63, 64);
  for (int i = n_act + lane; i < E; i += 64) active[i] = -1;
  if (lane == 0) {
    offsets[E] = total;
    n_active[0] = n_act;
  }
  __builtin_amdgcn_wave_barrier();
  const uint64_t lower = (1ull << lane) - 1ull;
  const int rank = __popcll(match_key(e, valid, key_bits(E)) & lower);
  if (lane < n) {
    if (valid) {
      const int pos = first[e] + rank;
      perm[pos] = lane;
      inv_perm[lane] = pos;
    } else {
      inv_perm[lane] = -1;
    }
  }
}

}  // namespace moe
