// Top-k and renormalised softmax of one token by one wavefront, shared by
// the router kernels and the decode gate/up kernel that groups a small batch
// itself (pages: zhichai.net, section on MoE sparsity -- 8 of 256 experts per
// token; yunpan.plus article, "capability 4" -- router semantics never change
// silently, so the selection is exact on float64 logits).
#pragma once

#include "common.h"

namespace moe {

namespace {

// Top-k and softmax of one token by one wavefront, E <= 64*NPL.
//
// The logit of expert e is the in-order sum of its P partial sums plus the
// bias.  Selection is exact on the float64 logits with ties to the lower id.
// It first narrows the field with float32 copies: rounding to float32 is
// monotone, so the k best experts all have float32 keys at or above tau, the
// k-th largest float32 key (found by k rounds of a wave-wide maximum, each
// taking one key out).  The (usually exactly k) candidates at or above tau
// are then ranked by (float64 logit desc, id asc) against each other.  If
// more than 64 candidates share the cut (mass ties), k rounds of a wave-wide
// argmax over all experts decide instead.
constexpr int kMaxK = 32;

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

// Maximum over the wavefront, in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));  // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));  // row_mirror
  const uint32_t a = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0));
  const uint32_t b = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16));
  const uint32_t c = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 32));
  const uint32_t d = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 48));
  return max(max(a, b), max(c, d));
}

// LDS scratch of one wavefront.
struct TopkLds {
  double cand_v[64];
  int cand_e[64];
  double sel_v[kMaxK];
  int sel_e[kMaxK];
  double sel_p[kMaxK];
};

// MP: parts loaded per logit (P <= MP); every lane's partial sums are
// loaded before any is added.  The chosen ids (sh.sel_e, best first) stay in
// LDS; topk_idx / topk_w receive them too unless topk_idx is null.
template <int NPL, int MP>
__device__ __forceinline__ void topk_token(const double* __restrict__ part, int P,
                                           const float* __restrict__ bias, int t, int E, int k,
                                           int32_t* __restrict__ topk_idx,
                                           float* __restrict__ topk_w, TopkLds& sh) {
  const int lane = threadIdx.x & 63;
  const uint64_t lower = (1ull << lane) - 1ull;
  double v[NPL];
  uint32_t key[NPL];
  constexpr int kMaxParts = MP;
  double pv[NPL][kMaxParts];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = min(lane + 64 * i, E - 1);
    const double* q = part + (static_cast<size_t>(t) * E + e) * P;
#pragma unroll
    for (int pp = 0; pp < kMaxParts; ++pp) pv[i][pp] = q[min(pp, P - 1)];
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    double s = -__builtin_inf();
    if (e < E) {
      s = pv[i][0];
#pragma unroll
      for (int pp = 1; pp < kMaxParts; ++pp)
        if (pp < P) s += pv[i][pp];
      if (bias) s += static_cast<double>(bias[e]);
      if (s != s) s = -__builtin_inf();  // NaN ranks as -inf
    }
    v[i] = s;
    key[i] = e < E ? order_key(static_cast<float>(s)) : 0u;  // real keys are > 0
  }
  // tau: take the largest remaining key out, k times
  uint32_t wk[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) wk[i] = key[i];
  uint32_t tau = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t lm = wk[0];
#pragma unroll
    for (int i = 1; i < NPL; ++i) lm = max(lm, wk[i]);
    tau = wave_max_u32(lm);
    const uint64_t who = __ballot(lm == tau);
    if (lane == __ffsll(static_cast<unsigned long long>(who)) - 1) {
      bool done = false;
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        if (!done && wk[i] == tau) {
          wk[i] = 0;
          done = true;
        }
      }
    }
  }
  int nc = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const bool in = key[i] >= tau;
    const uint64_t m = __ballot(in);
    const int pos = nc + __popcll(m & lower);
    if (in && pos < 64) {
      sh.cand_v[pos] = v[i];
      sh.cand_e[pos] = lane + 64 * i;
    }
    nc += __popcll(m);
  }
  __builtin_amdgcn_wave_barrier();
  if (nc <= 64) {
    if (lane < nc) {
      const double mv = sh.cand_v[lane];
      const int me = sh.cand_e[lane];
      int rank = 0;
      for (int q = 0; q < nc; ++q) {
        const double ov = sh.cand_v[q];
        const int oe = sh.cand_e[q];
        rank += (ov > mv || (ov == mv && oe < me)) ? 1 : 0;
      }
      if (rank < k) {
        sh.sel_v[rank] = mv;
        sh.sel_e[rank] = me;
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
        sh.sel_v[j] = bv;
        sh.sel_e[j] = be;
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  // softmax over the chosen k in float64: p_j = exp(l_j - l_0), z summed in j order
  const double m = sh.sel_v[0];
  const double pj = lane < k ? exp(sh.sel_v[lane] - m) : 0.0;
  if (lane < k) sh.sel_p[lane] = pj;
  __builtin_amdgcn_wave_barrier();
  double z = 0.0;
  for (int j = 0; j < k; ++j) z += sh.sel_p[j];
  if (topk_idx != nullptr && lane < k) {
    topk_idx[static_cast<size_t>(t) * k + lane] = sh.sel_e[lane];
    topk_w[static_cast<size_t>(t) * k + lane] = static_cast<float>(pj / z);
  }
  __builtin_amdgcn_wave_barrier();
}

}  // namespace

}  // namespace moe
