// Decode-path expert FFN: an HBM-bound int4 GEMV over the batch-union
// (pages: zhichai.net, sections on MoE sparsity and the three storage tiers
// -- 8 routed + 1 shared int4 expert per token, each a ~19 MB block;
// yunpan.plus article, "capability 2" -- each routed expert read once for all
// tokens of the batch that chose it).
//
// Two stream-ordered kernels over the packed expert blocks (pack.hip):
//   gate/up  h[p] = silu(W_gate x) * (W_up x)   for every grouped position p
//   down     y[p] = W_down h[p]
// Each is a pure streaming pass: every wavefront reads its own rows once and
// writes finished outputs, with no counters, no partial sums in memory and
// no waiting on other workgroups; the kernel boundary is the only
// synchronisation between the phases (h goes through the workspace).
//
// Lanes split rows and the input dimension: a gate/up wavefront owns 8 rows
// of gate and of up, each row spread over 8 lanes that take one eighth of
// the input columns; a down wavefront owns 16 rows over 4 lanes each.  A
// lane's partial sums are combined over its row's lanes by a fixed butterfly
// inside the wavefront, so the summation order is fixed by the layer shape
// and a token's result does not depend on the batch it comes in.  With 8
// gate/up rows per wavefront a 1-token step of the ~19 MB-expert layer has
// 9 x 256 equal gate/up wavefronts (9 per CU) and 9 x 384 down wavefronts.
//
// Codes stream through buffer loads, 16 bytes (32 nibbles of one row) per
// lane; the 16-byte pieces of 8 (or 16) neighbouring rows are contiguous in
// the packed tile, so every load instruction reads whole 128-byte lines.
// The activations of the workgroup's tokens (x for gate/up, h for down) are
// staged once in LDS; the parts of a row are skewed by 16 bytes so that the
// lanes of one LDS read hit different banks.
//
// Dequant: with the packed nibble order (offset-binary nibbles q + 8),
// ((w >> 4i) & 0x000F000F) | 0x43004300 is the bf16 pair (136 + q_a, 136 + q_b)
// of two neighbouring columns, exactly (the OR sets the exponent 2^7 above the
// 7-bit mantissa q + 8): one shift and one and-or per pair.  v_dot2_f32_bf16 multiplies it with the activation pair (products
// exact in fp32); the 136 offset is removed with the chunk's activation sum
// and the fp16 group scale applied once per 32 codes.  float32 activations
// and the float32 h fed to the down projection are carried as bf16 hi + lo
// pairs (16 significant bits); accumulation is float32 throughout.
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "topk_wave.h"
#include "union_wave.h"

// Every fused multiply-add below is written out; no other contraction, so a
// token's arithmetic is the same however many tokens share a sweep.
#pragma clang fp contract(off)

namespace moe {

namespace {

constexpr int kStep = 2;  // chunks per matrix per pipeline step (3 and 4 measured slower)
constexpr uint32_t kMask = 0x000F000Fu;
constexpr uint32_t kMagic = 0x43004300u;  // bf16 exponent 2^7 in both halves
constexpr float kOffset = 136.0f;

constexpr int kGuRows = 8;     // gate/up rows per wavefront
constexpr int kGuParts = 8;    // lanes per gate/up row
constexpr int kGuWaves = 4;    // wavefronts per gate/up workgroup (32 rows)
constexpr int kDnRows = 16;    // down rows per wavefront
constexpr int kDnParts = 4;    // lanes per down row
constexpr int kDnWaves = 4;    // wavefronts per down workgroup (64 rows)
constexpr int kSkewWords = 4;  // LDS skew between the parts of a row (16 bytes)
constexpr int kScalePad = 8;   // LDS padding (fp16) after each group's row scales
static_assert(kGuRows * kGuParts == kWave && kDnRows * kDnParts == kWave, "lane split");
static_assert(64 % (kGuRows * kGuWaves) == 0 && 64 % (kDnRows * kDnWaves) == 0,
              "a workgroup's rows stay inside one packed 64-row tile");

struct FfnArgs {
  const uint8_t* experts;
  const uint8_t* shared;
  size_t block_bytes;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* active;
  const int32_t* n_active;
  int top_k;
  int T;
  int has_shared;
  int d, f;
  size_t q_gate, q_up, q_down, s_gate, s_up, s_down;
  const void* x;  // [T][d] bf16 or f32
  uint32_t* hp;   // h as bf16 pairs: [T*k + T][f/32][32] (16 hi words, 16 lo words)
  float* y;       // [T*k][d]
  float* y_shared;  // [T][d]
};

// The router half of a small decode batch that the gate/up kernel groups
// itself: float64 logit partial sums from the router kernel, and where the
// top-k and the grouping go.
struct RouteArgs {
  const double* part;  // [T][E][P]
  const float* bias;   // [E] or null
  int P, E;
  int32_t* topk_idx;
  float* topk_w;
  int32_t *counts, *offsets, *perm, *inv_perm, *active, *n_active;
};

constexpr int kRouteMaxT = 8;     // tokens a grouping workgroup takes (2 per wavefront)
constexpr int kRouteMaxE = 256;   // experts (4 per lane in the grouping wavefront)
constexpr int kRouteEpl = kRouteMaxE / kWave;

// LDS of the grouping prologue: one top-k scratch per wavefront, the chosen
// ids of every token, and the grouping itself.
struct RouteLds {
  TopkLds tk[kGuWaves];
  int sel[kRouteMaxT][kMaxK];
  int cnt[kRouteMaxE], first[kRouteMaxE];
  int counts[kRouteMaxE], offsets[kRouteMaxE + 4], active[kRouteMaxE];
  int perm[kWave], inv_perm[kWave];
  int n_active[4];
};

struct Slot {
  const uint8_t* blk;
  int M;   // tokens
  int p0;  // first grouped position (routed experts)
  bool shared;
  bool live;
};

// Expert slot s of the launch: the shared expert first (if any), then
// active[0 ..].  Everything here is the same for every lane; keeping it in
// scalar registers keeps the buffer descriptors built from it scalar.
// active / offsets: the grouping, in global memory or (when the gate/up
// kernel grouped the batch itself) in LDS.
__device__ __forceinline__ Slot resolve_slot(const FfnArgs& g, int slot,
                                             const int32_t* active, const int32_t* offsets) {
  Slot s{nullptr, 0, 0, false, false};
  if (slot < g.has_shared) {
    s.blk = g.shared;
    s.M = g.T;
    s.shared = true;
    s.live = true;
    return s;
  }
  // active[] is -1 past the n_active experts of the batch, so one load tells
  // both whether the slot is live and which expert it holds
  const int e = __builtin_amdgcn_readfirstlane(active[slot - g.has_shared]);
  if (e < 0) return s;
  s.blk = g.experts + static_cast<size_t>(e) * g.block_bytes;
  s.p0 = __builtin_amdgcn_readfirstlane(offsets[e]);
  s.M = __builtin_amdgcn_readfirstlane(offsets[e + 1]) - s.p0;
  s.live = true;
  return s;
}

// Position of token m of a slot in the h row space (shared rows follow the
// T*k routed positions).
__device__ __forceinline__ int row_of(const FfnArgs& g, const Slot& sl, int m) {
  return sl.shared ? g.T * g.top_k + m : sl.p0 + m;
}

constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit buffer access
constexpr int kLoadNonTemporal = 2;     // buffer-load cache policy: streaming (nt)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcWord3);
}

// One pipeline step: kStep chunks of codes (16 bytes per lane) for NM
// matrices.
template <int NM>
struct Step {
  uint4 q[NM][kStep];
};

// Codes of one 64-row tile for NM matrices, as buffer resources: a 128-bit
// scalar descriptor plus one lane offset per load.
template <int NM>
struct TileRes {
  __amdgpu_buffer_rsrc_t q[NM];
};

// Chunks [c, c + kStep) of this lane's range [cb, ce).  Loads are
// unconditional (indices past the range are clamped to its last chunk, a
// cache hit), so every path has the same loads in flight and the compiler
// waits for exactly the step it needs.  rt: the lane's row inside the tile.
template <int NM>
__device__ __forceinline__ void load_step(const TileRes<NM>& res, int c, int cb, int ce, int rt,
                                          Step<NM>& d) {
#pragma unroll
  for (int i = 0; i < kStep; ++i) {
    const int cc = max(min(c + i, ce - 1), cb);
#pragma unroll
    for (int mat = 0; mat < NM; ++mat) {
      // non-temporal: every code is read once per step (measured 4% faster
      // on the 1-token step of the ~19 MB-expert layer than plain loads)
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(res.q[mat], cc * 1024 + rt * 16, 0,
                                                           kLoadNonTemporal);
      d.q[mat][i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }
}

// Math of one step.  xl: this lane's activations, local chunk cl of token m
// at xl[m * tok_words + cl * XW]; xs: chunk sums at xs[m * sum_words + cl];
// sc[mat]: the fp16 group scales of this lane's row, group j at
// sc[mat][j * kSst] (the lane's range starts at chunk cb).  XW = 16 (bf16
// pairs) or 32 (16 hi pairs, then 16 lo pairs).
// MXFP4 (MX): byte i of a code word is two E2M1 elements, columns 2i and
// 2i + 1 of the word's eight; the hardware conversion gives them as a bf16
// pair exactly.
template <int I>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, I));
}

template <int NM, int MT, int XW, int kSst, bool MX>
__device__ __forceinline__ void math_step(const Step<NM>& d, int cl, int nl, int cb, int nt,
                                          const uint32_t* xl, int tok_words, const float* xs,
                                          int sum_words, const void* const (&sc)[NM],
                                          float (&acc)[NM][MT]) {
#pragma unroll
  for (int i = 0; i < kStep; ++i) {
    const int c = cl + i;
    if (c >= nl) break;
    float tc[NM][MT];
    const uint32_t mg = opaque_vgpr(kMagic);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // the activation pairs of this 8-column word, once for every matrix
      uint4 xh[MT], xo[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < nt) {
          xh[m] = *reinterpret_cast<const uint4*>(xl + m * tok_words + c * XW + 4 * w);
          if constexpr (XW == 32)
            xo[m] = *reinterpret_cast<const uint4*>(xl + m * tok_words + c * XW + 16 + 4 * w);
        }
      }
#pragma unroll
      for (int mat = 0; mat < NM; ++mat) {
        const uint32_t u = w == 0 ? d.q[mat][i].x : w == 1 ? d.q[mat][i].y : w == 2 ? d.q[mat][i].z : d.q[mat][i].w;
        uint32_t b0, b1, b2, b3;
        if constexpr (MX) {
          b0 = fp4_pair<0>(u);
          b1 = fp4_pair<1>(u);
          b2 = fp4_pair<2>(u);
          b3 = fp4_pair<3>(u);
        } else {
          b0 = and_or(u, kMask, mg);
          b1 = and_or((u >> 4), kMask, mg);
          b2 = and_or((u >> 8), kMask, mg);
          b3 = and_or((u >> 12), kMask, mg);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < nt) {
            float t = w == 0 ? 0.0f : tc[mat][m];
            t = dot2_bf16(b0, xh[m].x, t);
            t = dot2_bf16(b1, xh[m].y, t);
            t = dot2_bf16(b2, xh[m].z, t);
            t = dot2_bf16(b3, xh[m].w, t);
            if constexpr (XW == 32) {
              t = dot2_bf16(b0, xo[m].x, t);
              t = dot2_bf16(b1, xo[m].y, t);
              t = dot2_bf16(b2, xo[m].z, t);
              t = dot2_bf16(b3, xo[m].w, t);
            }
            tc[mat][m] = t;
          }
        }
      }
    }
#pragma unroll
    for (int mat = 0; mat < NM; ++mat) {
      if constexpr (MX) {
        // one E8M0 scale per 32-column chunk; the elements are exact, no offset
        const float sv = e8m0_to_f32(static_cast<const uint8_t*>(sc[mat])[(cb + c) * kSst]);
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m < nt) acc[mat][m] = fmaf(sv, tc[mat][m], acc[mat][m]);
      } else {
        const float sv = static_cast<float>(static_cast<const _Float16*>(sc[mat])[((cb + c) >> 1) * kSst]);
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m < nt)
            acc[mat][m] = fmaf(sv, fmaf(-kOffset, xs[m * sum_words + c], tc[mat][m]), acc[mat][m]);
      }
    }
  }
}

// This lane's partial sums over its chunks [cb, ce) of the tile: two step
// buffers, the next step's loads in flight while the current step's math
// runs.  Every lane runs the same number of steps (nmax = the longest part);
// lanes past their own range do no math.
//
// `a` and `b` hold the first two steps' loads, issued by the caller before
// it staged the activations, so their latency overlaps the staging.
template <int NM, int MT, int XW, int kSst, bool MX>
__device__ __forceinline__ void sweep(const TileRes<NM>& res, int cb, int ce, int nmax, int rt,
                                      int nt, const uint32_t* xl, int tok_words, const float* xs,
                                      int sum_words, const void* const (&sc)[NM], Step<NM>& a,
                                      Step<NM>& b, float (&acc)[NM][MT]) {
#pragma unroll
  for (int mat = 0; mat < NM; ++mat)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[mat][m] = 0.0f;
  const int nl = ce - cb;
  for (int c0 = 0; c0 < nmax; c0 += 2 * kStep) {
    math_step<NM, MT, XW, kSst, MX>(a, c0, nl, cb, nt, xl, tok_words, xs, sum_words, sc, acc);
    load_step<NM>(res, cb + c0 + 2 * kStep, cb, ce, rt, a);
    math_step<NM, MT, XW, kSst, MX>(b, c0 + kStep, nl, cb, nt, xl, tok_words, xs, sum_words, sc, acc);
    load_step<NM>(res, cb + c0 + 3 * kStep, cb, ce, rt, b);
  }
}

// LDS layout of a workgroup's staged activations: token m, part p, local
// chunk cl at word m * tok_words + p * part_words + cl * xw (part_words =
// cpp_max * xw + kSkewWords); chunk sums at m * sum_words + p * cpp_max + cl.
// Part p covers chunks [p * chunks / parts, (p + 1) * chunks / parts).
struct StageLayout {
  int parts, chunks, cpp_max, xw, part_words, tok_words, sum_words;
  __device__ __forceinline__ int cb(int p) const { return p * chunks / parts; }
  __device__ __forceinline__ int part_of(int c) const {
    int p = c * parts / chunks;
    while (cb(p + 1) <= c) ++p;
    while (cb(p) > c) --p;
    return p;
  }
};

__device__ __forceinline__ StageLayout stage_layout(int chunks, int parts, int xw) {
  StageLayout s;
  s.parts = parts;
  s.chunks = chunks;
  s.cpp_max = (chunks + parts - 1) / parts;
  s.xw = xw;
  s.part_words = s.cpp_max * xw + kSkewWords;
  s.tok_words = parts * s.part_words;
  s.sum_words = parts * s.cpp_max;
  return s;
}

// The fp16 scales of `rows` consecutive rows, starting at row o of a packed
// 64-row tile (the block's scales are group-major inside a tile: group j of
// the tile's 64 rows at tile + j * 128 bytes), into LDS as
// [groups][rows + kScalePad].
__device__ __forceinline__ void stage_scales(const uint8_t* tile, int o, int rows, int groups,
                                             uint32_t* dst) {
  const int per = rows / 8;  // 16-byte pieces per group (rows is a multiple of 8)
  for (int i = threadIdx.x; i < groups * per; i += blockDim.x) {
    const int j = i / per, pc = i - j * per;
    const uint4 v = *reinterpret_cast<const uint4*>(tile + (j * 64 + o) * 2 + pc * 16);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(dst) + (j * (rows + kScalePad) + pc * 8) * 2) = v;
  }
}

// MXFP4: the E8M0 bytes of `rows` consecutive rows from row o of a packed
// 64-row tile (block b of the tile's rows at tile + b * 64), into LDS as
// [blocks][rows + kScalePadMx] bytes.
constexpr int kScalePadMx = 16;
__device__ __forceinline__ void stage_scales_mx(const uint8_t* tile, int o, int rows, int blocks,
                                                uint32_t* dst) {
  const int per = rows / 16;  // 16-byte pieces per block (rows is a multiple of 16)
  for (int i = threadIdx.x; i < blocks * per; i += blockDim.x) {
    const int b = i / per, pc = i - b * per;
    const uint4 v = *reinterpret_cast<const uint4*>(tile + b * 64 + o + pc * 16);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(dst) + b * (rows + kScalePadMx) + pc * 16) = v;
  }
}

// x rows of the gate/up phase: bf16 copied as pairs, or f32 split into hi/lo
// bf16; plus each chunk's sum of the values the dot products see.
template <bool XF32>
__device__ void stage_x(const FfnArgs& g, const Slot& sl, const int32_t* perm, int m0, int nt,
                        const StageLayout& L, uint32_t* xl, float* xs) {
  for (int i = threadIdx.x; i < nt * L.chunks; i += blockDim.x) {
    const int m = i / L.chunks, c = i - m * L.chunks;
    const int p = L.part_of(c), cl = c - L.cb(p);
    const int tok = sl.shared ? m0 + m : (g.T == 1 ? 0 : perm[sl.p0 + m0 + m] / g.top_k);
    uint32_t* dst = xl + m * L.tok_words + p * L.part_words + cl * L.xw;
    float s = 0.0f;
    if constexpr (!XF32) {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(g.x) +
                                                        static_cast<size_t>(tok) * g.d + c * 32);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 v = src[j];
        reinterpret_cast<uint4*>(dst)[j] = v;
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) s += __uint_as_float(w[q] << 16) + __uint_as_float(w[q] & 0xFFFF0000u);
      }
    } else {
      const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(g.x) +
                                                          static_cast<size_t>(tok) * g.d + c * 32);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float4 v = src[j];
        const float e[4] = {v.x, v.y, v.z, v.w};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          hi[q] = f32_to_bf16(e[q]);
          const float hf = __uint_as_float(hi[q] << 16);
          lo[q] = f32_to_bf16(e[q] - hf);
          s += hf + __uint_as_float(lo[q] << 16);
        }
        dst[2 * j] = hi[0] | (hi[1] << 16);
        dst[2 * j + 1] = hi[2] | (hi[3] << 16);
        dst[16 + 2 * j] = lo[0] | (lo[1] << 16);
        dst[16 + 2 * j + 1] = lo[2] | (lo[3] << 16);
      }
    }
    xs[m * L.sum_words + p * L.cpp_max + cl] = s;
  }
}

// h rows of the down phase (hi/lo pairs), plus each chunk's sum.  Four
// threads share a chunk, each copying a quarter (two 16-byte pieces: hi
// words 4q.., lo words 4q..) and summing its 16 values; the quarter sums are
// added in a fixed order ((q0 + q1) + (q2 + q3)).
__device__ void stage_h(const FfnArgs& g, const Slot& sl, int m0, int nt, const StageLayout& L,
                        uint32_t* xl, float* xs) {
  const int q = threadIdx.x & 3;
  const int items = nt * L.chunks;
  // every thread of a quad runs the same iterations (the shuffles need all four)
  for (int i0 = threadIdx.x >> 2; i0 < (items + blockDim.x / 4 - 1) / (blockDim.x / 4) * (blockDim.x / 4);
       i0 += blockDim.x / 4) {
    const int i = min(i0, items - 1);
    const int m = i / L.chunks, c = i - m * L.chunks;
    const int p = L.part_of(c), cl = c - L.cb(p);
    const size_t row = row_of(g, sl, m0 + m);
    const uint4* src = reinterpret_cast<const uint4*>(g.hp + (row * L.chunks + c) * 32);
    uint32_t* dst = xl + m * L.tok_words + p * L.part_words + cl * 32;
    const uint4 vh = src[q], vl = src[4 + q];
    float s = 0.0f;
    const uint32_t w[8] = {vh.x, vh.y, vh.z, vh.w, vl.x, vl.y, vl.z, vl.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) s += __uint_as_float(w[k] << 16) + __uint_as_float(w[k] & 0xFFFF0000u);
    s += __shfl_xor(s, 1, kWave);
    s += __shfl_xor(s, 2, kWave);
    if (i0 < items) {
      reinterpret_cast<uint4*>(dst)[q] = vh;
      reinterpret_cast<uint4*>(dst)[4 + q] = vl;
      if (q == 0) xs[m * L.sum_words + p * L.cpp_max + cl] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// gate/up: one workgroup per (expert slot, 64-row tile of f), 8 wavefronts
// of 8 rows; lane = 8 * part + row
// ---------------------------------------------------------------------------

// Words of a gate/up workgroup's LDS before the grouping prologue's region
// (a multiple of 4, so the region is 16-byte aligned).
__host__ __device__ constexpr int gu_scale_words(int d, bool mx) {
  // two matrices: fp16 per (row, 64 columns), or one E8M0 byte per (row, 32 columns)
  return mx ? (kGuWaves * kGuRows + kScalePadMx) * (d / 32) / 2
            : (kGuWaves * kGuRows + kScalePad) * (d / 64);
}

__host__ __device__ constexpr int gu_words(int d, int mt, bool xf32, bool mx = false) {
  return (gu_scale_words(d, mx) +
          mt * (kGuParts * (((d / 32 + kGuParts - 1) / kGuParts) * (xf32 ? 32 : 16) + kSkewWords) +
                kGuParts * ((d / 32 + kGuParts - 1) / kGuParts)) +
          3) / 4 * 4;
}

// The grouping prologue (RMP > 0, small batches): the routed workgroups take
// the top-k of every token from the router's partial sums (RMP = parts held
// per logit) and group the batch in LDS, each for itself, with the same
// device code as the route + union kernel, so every workgroup derives the same
// grouping.  One of them also writes the top-k and the grouping out for the
// down and combine kernels.  The shared expert's workgroups need no grouping
// and go straight to their weights.
template <int RMP>
__device__ __forceinline__ void group_batch(const FfnArgs& g, const RouteArgs& r, RouteLds& rl) {
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int k = g.top_k, n = g.T * k;
  const bool writer = blockIdx.x == 0 && blockIdx.y == static_cast<unsigned>(g.has_shared);
  for (int t = wv; t < g.T; t += kGuWaves) {
    topk_token<kRouteEpl, RMP>(r.part, r.P, r.bias, t, r.E, k, writer ? r.topk_idx : nullptr,
                               r.topk_w, rl.tk[wv]);
    if (lane < k) rl.sel[t][lane] = rl.tk[wv].sel_e[lane];
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  if (wv == 0) {
    const int e = lane < n ? rl.sel[lane / k][lane % k] : -1;
    union_wave<kRouteEpl>(e, n, r.E, rl.counts, rl.offsets, rl.perm, rl.inv_perm, rl.active,
                          rl.n_active, rl.cnt, rl.first);
  }
  __syncthreads();
  if (writer) {
    for (int i = threadIdx.x; i < r.E; i += blockDim.x) {
      r.counts[i] = rl.counts[i];
      r.offsets[i] = rl.offsets[i];
      r.active[i] = rl.active[i];
    }
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      r.perm[i] = rl.perm[i];
      r.inv_perm[i] = rl.inv_perm[i];
    }
    if (threadIdx.x == 0) {
      r.offsets[r.E] = rl.offsets[r.E];
      r.n_active[0] = rl.n_active[0];
    }
  }
}

template <int MT, bool XF32, int RMP, bool MX>
__global__ __launch_bounds__(kGuWaves * kWave) void decode_gateup(FfnArgs g, RouteArgs rt_args) {
  static_assert(!(MX && RMP > 0), "the grouping prologue runs with int4 blocks only");
  extern __shared__ __align__(16) uint32_t lds[];
  constexpr int XW = XF32 ? 32 : 16;
  const int32_t* perm = g.perm;
  const int32_t* active = g.active;
  const int32_t* offsets = g.offsets;
  if constexpr (RMP > 0) {
    if (blockIdx.y >= static_cast<unsigned>(g.has_shared)) {
      RouteLds& rl = *reinterpret_cast<RouteLds*>(lds + gu_words(g.d, MT, XF32));
      group_batch<RMP>(g, rt_args, rl);
      perm = rl.perm;
      active = rl.active;
      offsets = rl.offsets;
    }
  }
  const Slot sl = resolve_slot(g, blockIdx.y, active, offsets);
  if (!sl.live) return;
  // The two 32-row halves of a 64-row tile go to workgroups x and x + 8,
  // which run on the same XCD (workgroups are dealt to the 8 XCDs in turn),
  // so the tile's 128-byte scale runs are fetched into one L2 once.
  static_assert(kGuWaves * kGuRows == 32, "two workgroups per 64-row tile");
  const int xb = blockIdx.x, nb = g.f / 32;  // workgroups along f
  const int row0 = (nb % 16 == 0 ? (xb / 16) * 512 + (xb % 8) * 64 + ((xb / 8) & 1) * 32
                                 : xb * 32);  // first f-row of the workgroup
  const int tile = row0 / 64;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane % kGuRows, p = lane / kGuRows;
  const int rt = row0 % 64 + wv * kGuRows + r;  // row inside the tile
  const StageLayout L = stage_layout(g.d / 32, kGuParts, XW);
  constexpr int kRowsWg = kGuWaves * kGuRows;
  const int groups = g.d / 64;
  // scale strides: fp16 elements per group row, or bytes per MXFP4 block row
  constexpr int kSst = MX ? kRowsWg + kScalePadMx : kRowsWg + kScalePad;
  const int blocks = g.d / 32;
  uint32_t* scl = lds;                                    // [2][groups][kSst] fp16 or [2][blocks][kSst] u8
  uint32_t* xl = lds + gu_scale_words(g.d, MX);           // staged x
  float* xs = reinterpret_cast<float*>(xl + MT * L.tok_words);
  const int cb = L.cb(p), ce = L.cb(p + 1);

  const size_t tq = static_cast<size_t>(tile) * 64 * (g.d / 2);
  TileRes<2> res;
  res.q[0] = make_rsrc(sl.blk + g.q_gate + tq, 32u * g.d);
  res.q[1] = make_rsrc(sl.blk + g.q_up + tq, 32u * g.d);
  const int rl = wv * kGuRows + r;  // row inside the workgroup
  const void* sc[2];
  if constexpr (MX) {
    sc[0] = reinterpret_cast<const uint8_t*>(scl) + rl;
    sc[1] = reinterpret_cast<const uint8_t*>(scl) + kSst * blocks + rl;
    const size_t ts = static_cast<size_t>(tile) * 64 * blocks;  // the tile's scale bytes
    stage_scales_mx(sl.blk + g.s_gate + ts, row0 % 64, kRowsWg, blocks, scl);
    stage_scales_mx(sl.blk + g.s_up + ts, row0 % 64, kRowsWg, blocks, scl + kSst * blocks / 4);
  } else {
    sc[0] = reinterpret_cast<const _Float16*>(scl) + rl;
    sc[1] = reinterpret_cast<const _Float16*>(scl) + kSst * groups + rl;
    const size_t ts = static_cast<size_t>(tile) * 64 * groups * 2;  // the tile's scales
    stage_scales(sl.blk + g.s_gate + ts, row0 % 64, kRowsWg, groups, scl);
    stage_scales(sl.blk + g.s_up + ts, row0 % 64, kRowsWg, groups, scl + kSst * groups / 2);
  }
  const int fchunks = g.f / 32;
  const int frow = row0 + wv * kGuRows + r;

  for (int m0 = 0; m0 < sl.M; m0 += MT) {
    const int nt = min(MT, sl.M - m0);
    Step<2> first, second;
    load_step<2>(res, cb, cb, ce, rt, first);
    load_step<2>(res, cb + kStep, cb, ce, rt, second);
    __syncthreads();
    stage_x<XF32>(g, sl, perm, m0, nt, L, xl, xs);
    __syncthreads();
    float acc[2][MT];
    sweep<2, MT, XW, kSst, MX>(res, cb, ce, L.cpp_max, rt, nt, xl + p * L.part_words, L.tok_words,
                     xs + p * L.cpp_max, L.sum_words, sc, first, second, acc);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= nt) break;
      // sum over the row's lanes (one per part), fixed order
      float gs = acc[0][m], us = acc[1][m];
#pragma unroll
      for (int off = kGuRows; off < kWave; off <<= 1) {
        gs += __shfl_xor(gs, off, kWave);
        us += __shfl_xor(us, off, kWave);
      }
      const float h = silu(gs) * us;
      const uint32_t hi = f32_to_bf16(h);
      const uint32_t lo = f32_to_bf16(h - __uint_as_float(hi << 16));
      const uint32_t hi_o = __shfl_xor(hi, 1, kWave), lo_o = __shfl_xor(lo, 1, kWave);
      // f-row frow sits in chunk frow/32, pair (frow%32)/2
      const size_t row = row_of(g, sl, m0 + m);
      uint32_t* hrow = g.hp + (row * fchunks + (frow >> 5)) * 32;
      const int j = (frow & 31) >> 1;
      if (p == 0 && (r & 1) == 0) hrow[j] = hi | (hi_o << 16);
      if (p == 1 && (r & 1) == 1) hrow[16 + j] = lo_o | (lo << 16);
    }
  }
}

// ---------------------------------------------------------------------------
// down: one workgroup per (expert slot, 64-row tile of d), 4 wavefronts of
// 16 rows; lane = 16 * part + row
// ---------------------------------------------------------------------------

template <int MT, bool MX>
__global__ __launch_bounds__(kDnWaves * kWave) void decode_down(FfnArgs g) {
  extern __shared__ __align__(16) uint32_t lds[];
  const Slot sl = resolve_slot(g, blockIdx.y, g.active, g.offsets);
  if (!sl.live) return;
  const int row0 = blockIdx.x * kDnWaves * kDnRows;  // first d-row of the workgroup
  const int tile = row0 / 64;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane % kDnRows, p = lane / kDnRows;
  const int rt = row0 % 64 + wv * kDnRows + r;
  const StageLayout L = stage_layout(g.f / 32, kDnParts, 32);
  constexpr int kRowsWg = kDnWaves * kDnRows;
  const int groups = g.f / 64;
  constexpr int kSst = MX ? kRowsWg + kScalePadMx : kRowsWg + kScalePad;
  const int blocks = g.f / 32;
  uint32_t* scl = lds;                                    // [groups][kSst] fp16 or [blocks][kSst] u8
  uint32_t* xl = lds + (MX ? kSst * blocks / 4 : kSst * groups / 2);  // staged h
  float* xs = reinterpret_cast<float*>(xl + MT * L.tok_words);
  const int cb = L.cb(p), ce = L.cb(p + 1);

  TileRes<1> res;
  res.q[0] = make_rsrc(sl.blk + g.q_down + static_cast<size_t>(tile) * 64 * (g.f / 2), 32u * g.f);
  const int rl = wv * kDnRows + r;
  const void* sc[1];
  if constexpr (MX) {
    sc[0] = reinterpret_cast<const uint8_t*>(scl) + rl;
    stage_scales_mx(sl.blk + g.s_down + static_cast<size_t>(tile) * 64 * blocks, row0 % 64,
                    kRowsWg, blocks, scl);
  } else {
    sc[0] = reinterpret_cast<const _Float16*>(scl) + rl;
    stage_scales(sl.blk + g.s_down + static_cast<size_t>(tile) * 64 * groups * 2, row0 % 64,
                 kRowsWg, groups, scl);
  }
  const int drow = row0 + wv * kDnRows + r;

  for (int m0 = 0; m0 < sl.M; m0 += MT) {
    const int nt = min(MT, sl.M - m0);
    Step<1> first, second;
    load_step<1>(res, cb, cb, ce, rt, first);
    load_step<1>(res, cb + kStep, cb, ce, rt, second);
    __syncthreads();
    stage_h(g, sl, m0, nt, L, xl, xs);
    __syncthreads();
    float acc[1][MT];
    sweep<1, MT, 32, kSst, MX>(res, cb, ce, L.cpp_max, rt, nt, xl + p * L.part_words, L.tok_words,
                     xs + p * L.cpp_max, L.sum_words, sc, first, second, acc);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= nt) break;
      float ys = acc[0][m];
#pragma unroll
      for (int off = kDnRows; off < kWave; off <<= 1) ys += __shfl_xor(ys, off, kWave);
      if (p == 0) {
        float* out = sl.shared ? g.y_shared + static_cast<size_t>(m0 + m) * g.d
                               : g.y + static_cast<size_t>(sl.p0 + m0 + m) * g.d;
        out[drow] = ys;
      }
    }
  }
}

int gu_lds_bytes(int d, int mt, bool xf32, bool mx = false) {
  const int chunks = d / 32, cpp = (chunks + kGuParts - 1) / kGuParts, xw = xf32 ? 32 : 16;
  const int scales = gu_scale_words(d, mx);  // words: two matrices
  return (scales + mt * (kGuParts * (cpp * xw + kSkewWords) + kGuParts * cpp)) * 4;
}

int dn_lds_bytes(int f, int mt, bool mx = false) {
  const int chunks = f / 32, cpp = (chunks + kDnParts - 1) / kDnParts;
  const int scales = mx ? (kDnWaves * kDnRows + kScalePadMx) * (f / 32) / 4
                        : (kDnWaves * kDnRows + kScalePad) * (f / 64) / 2;
  return (scales + mt * (kDnParts * (cpp * 32 + kSkewWords) + kDnParts * cpp)) * 4;
}

constexpr int kMaxLds = 64 * 1024;

int gu_route_lds_bytes(int d, int mt, bool xf32) {
  return gu_words(d, mt, xf32) * 4 + static_cast<int>(sizeof(RouteLds));
}

// RMP = 0: the grouping comes from global memory; 8 or 16: the gate/up
// kernel groups the batch (RouteArgs) and writes the grouping for the down
// kernel.
template <int MT, bool XF32, int RMP, bool MX>
hipError_t launch_mt(const FfnArgs& g, const RouteArgs& r, int slots, hipStream_t s) {
  const dim3 g1(g.f / (kGuWaves * kGuRows), slots), g2(g.d / (kDnWaves * kDnRows), slots);
  const int gu_lds = RMP > 0 ? gu_route_lds_bytes(g.d, MT, XF32) : gu_lds_bytes(g.d, MT, XF32, MX);
  hipError_t err = launch(decode_gateup<MT, XF32, RMP, MX>, g1, dim3(kGuWaves * kWave), gu_lds, s, g, r);
  if (err != hipSuccess) return err;
  return launch(decode_down<MT, MX>, g2, dim3(kDnWaves * kWave), dn_lds_bytes(g.f, MT, MX), s, g);
}

template <int RMP, bool MX = false>
hipError_t launch_any_mt(const FfnArgs& g, const RouteArgs& r, int slots, int mt, bool xf32,
                         hipStream_t s) {
  if (xf32) {
    if (mt == 4) return launch_mt<4, true, RMP, MX>(g, r, slots, s);
    if (mt == 2) return launch_mt<2, true, RMP, MX>(g, r, slots, s);
    return launch_mt<1, true, RMP, MX>(g, r, slots, s);
  }
  if (mt == 4) return launch_mt<4, false, RMP, MX>(g, r, slots, s);
  if (mt == 2) return launch_mt<2, false, RMP, MX>(g, r, slots, s);
  return launch_mt<1, false, RMP, MX>(g, r, slots, s);
}

FfnArgs ffn_args(const FfnProblem& p) {
  const size_t dd = p.d, ff = p.f;
  FfnArgs g{};
  g.experts = p.experts;
  g.shared = p.shared;
  g.block_bytes = p.block_bytes;
  g.offsets = p.offsets;
  g.perm = p.perm;
  g.active = p.active;
  g.n_active = p.n_active;
  g.top_k = p.k;
  g.T = p.T;
  g.has_shared = p.has_shared ? 1 : 0;
  g.d = p.d;
  g.f = p.f;
  g.q_gate = 0;
  g.q_up = ff * dd / 2;
  g.q_down = ff * dd;
  g.s_gate = 3 * dd * ff / 2;
  if (p.mxfp4) {  // one E8M0 byte per 32 elements
    g.s_up = g.s_gate + ff * (dd / 32);
    g.s_down = g.s_up + ff * (dd / 32);
  } else {        // one float16 per 64 elements
    g.s_up = g.s_gate + ff * (dd / 64) * 2;
    g.s_down = g.s_up + ff * (dd / 64) * 2;
  }
  g.x = p.x;
  g.hp = static_cast<uint32_t*>(p.workspace);
  g.y = static_cast<float*>(p.y);
  g.y_shared = static_cast<float*>(p.y_shared);
  return g;
}

// Tokens per sweep: as many as the batch offers, up to 4, LDS permitting
// (gu_extra: bytes the gate/up kernel needs beyond its staging); 0 if even
// one token does not fit.
int pick_mt(const FfnProblem& p, int gu_extra) {
  const bool xf32 = !p.x_bf16;
  int mt = p.T >= 4 ? 4 : (p.T >= 2 ? 2 : 1);
  auto fits = [&](int m) {
    return gu_words(p.d, m, xf32, p.mxfp4) * 4 + gu_extra <= kMaxLds &&
           dn_lds_bytes(p.f, m, p.mxfp4) <= kMaxLds;
  };
  while (mt > 1 && !fits(mt)) mt /= 2;
  return fits(mt) ? mt : 0;
}

}  // namespace

size_t ffn_decode_workspace(int T, int k, int /*E*/, int /*d*/, int f, bool has_shared) {
  const size_t rows = static_cast<size_t>(T) * (k + (has_shared ? 1 : 0));
  return rows * f * 4;  // h as bf16 hi/lo pairs
}

hipError_t launch_ffn_decode(const FfnProblem& p, hipStream_t stream) {
  const FfnArgs g = ffn_args(p);
  const int slots = g.has_shared + std::min(p.E, p.T * p.k);
  const int mt = pick_mt(p, 0);
  if (mt == 0) return hipErrorNotSupported;
  return p.mxfp4 ? launch_any_mt<0, true>(g, RouteArgs{}, slots, mt, !p.x_bf16, stream)
                 : launch_any_mt<0, false>(g, RouteArgs{}, slots, mt, !p.x_bf16, stream);
}

bool ffn_decode_groups_batch(const FfnProblem& p, int P) {
  return p.T >= 1 && p.T <= kRouteMaxT && p.T * p.k <= kWave && p.E <= kRouteMaxE &&
         p.k <= kMaxK && P <= 16 && pick_mt(p, static_cast<int>(sizeof(RouteLds))) > 0;
}

hipError_t launch_ffn_decode_grouping(const FfnProblem& p, const RouteGroup& rg,
                                      hipStream_t stream) {
  if (!ffn_decode_groups_batch(p, rg.P)) return hipErrorNotSupported;
  const FfnArgs g = ffn_args(p);
  RouteArgs r{};
  r.part = rg.part;
  r.bias = rg.bias;
  r.P = rg.P;
  r.E = p.E;
  r.topk_idx = rg.topk_idx;
  r.topk_w = rg.topk_w;
  r.counts = rg.u.counts;
  r.offsets = rg.u.offsets;
  r.perm = rg.u.perm;
  r.inv_perm = rg.u.inv_perm;
  r.active = rg.u.active;
  r.n_active = rg.u.n_active;
  const int slots = g.has_shared + std::min(p.E, p.T * p.k);
  const int mt = pick_mt(p, static_cast<int>(sizeof(RouteLds)));
  if (mt == 0) return hipErrorNotSupported;
  if (rg.P <= 8) return launch_any_mt<8>(g, r, slots, mt, !p.x_bf16, stream);
  return launch_any_mt<16>(g, r, slots, mt, !p.x_bf16, stream);
}

}  // namespace moe
