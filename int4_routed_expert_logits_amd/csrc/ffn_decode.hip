// Decode-path expert FFN: an HBM-bound int4 GEMV over the batch-union
// (pages: zhichai.net, sections on MoE sparsity and the three storage tiers
// -- 8 routed + 1 shared int4 expert per token, each a ~19 MB block;
// yunpan.plus article, "capability 2" -- each routed expert read once for all
// tokens of the batch that chose it).
//
// One launch, two phases over the packed expert blocks (pack.hip):
//   gate/up  h[p] = silu(W_gate x) * (W_up x)   for every grouped position p
//   down     y[p] = W_down h[p]
// A work item is one wavefront: one 64-row tile of one expert's matrix
// (gate and up together in the first phase) over one part of the input
// dimension.  Each lane owns one row and accumulates it over the part, so
// there is no cross-lane reduction per row.  Splitting the input dimension
// into P parts gives enough equal, independent wavefronts to spread over all
// 256 CUs (a 1-token step has only 9 experts x 32 gate/up tiles); the parts'
// partial sums go to the workspace and the part that finishes last adds them
// in part order (so the result does not depend on timing) and finishes the
// tile: h = silu(g) * u, or the y row.  The activations of the item's tokens
// are staged in LDS and read back as broadcasts.  Codes stream through
// buffer loads, 16 bytes per lane, two 32-column chunks per matrix per
// pipeline step, with the next step's loads in flight during the current
// step's math.
//
// Dequant: with the packed nibble order, ((w >> 4i) & 0x000F000F) ^ 0x43084308
// is the bf16 pair (136 + q_a, 136 + q_b) of two neighbouring columns, exactly
// (the XOR sets the exponent 2^7 and turns the two's-complement nibble q into
// q + 8).  v_dot2_f32_bf16 multiplies it with the activation pair (products
// exact in fp32); the 136 offset is removed with the chunk's activation sum
// and the fp16 group scale applied once per 32 codes.  float32 activations
// and the float32 h fed to the down projection are carried as bf16 hi + lo
// pairs (16 significant bits); accumulation is float32 throughout.
//
// Both phases run in one persistent grid of single-wavefront workgroups.
// Items [0, n_items1) are gate/up parts, the rest down parts, expert-slot
// major; workgroup b takes items b, b + grid, ... in order.  The grid never
// exceeds what the GPU holds at once, so every workgroup is resident, and a
// workgroup finishes its gate/up items before it reaches a down item: a down
// item waiting for its slot's h always sees it finish.  Data that crosses
// workgroups (partial sums, h) goes through device-scope stores and loads,
// which bypass the per-XCD L2 caches that are not coherent with each other,
// and is published by a counter increment after the stores have completed.
#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

#include "common.h"
#include "launch.h"

// Every fused multiply-add below is written out; no other contraction, so a
// token's arithmetic is the same in every code path (one or two tokens per
// sweep) and its result does not depend on the batch it is in.
#pragma clang fp contract(off)

namespace moe {

namespace {

constexpr int kStep = 2;  // chunks per matrix per pipeline step
constexpr uint32_t kMask = 0x000F000Fu;
constexpr uint32_t kMagicX = 0x43084308u;  // bf16 exponent 2^7 | nibble sign flip
constexpr float kOffset = 136.0f;

// Control block (int32 words) at the head of the workspace: per expert slot,
// on its own 128-byte line, the number of gate/up tiles that have published
// h and the number of down tiles that have finished; a flag raised if a wait
// ever timed out; then one arrival counter per (slot, tile) of each phase.
// Zero before the first call; every counter is zeroed again by the last
// wavefront that uses it, so each call leaves the block zero.
constexpr int kLineWords = 32;
constexpr int kMaxSlots = 1025;  // 1024 experts + shared
constexpr int kTimeout = kMaxSlots * kLineWords;
constexpr int kTileCounters = kTimeout + kLineWords;
constexpr uint64_t kSpinLimit = 200000000ull;  // 2 s of the 100 MHz wall clock

struct DecodeArgs {
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
  int slots;           // shared first (if any), then active[0 ..]
  int d, f;
  size_t q_gate, q_up, q_down, s_gate, s_up, s_down;
  const void* x;       // [T][d] bf16 or f32
  uint32_t* hp;        // h as bf16 pairs: [T*k + T][f/32][32] (hi pairs, then lo pairs)
  float* hs;           // h chunk sums:    [T*k + T][f/32]
  float* y;            // [T*k][d]
  float* y_shared;     // [T][d]
  int* ctrl;
  int* tcnt1;          // [slots][tiles1] arrival counters (gate/up)
  int* tcnt2;          // [slots][tiles2] arrival counters (down)
  float* part1;        // [rows][tiles1][P1][2][64] gate/up partial sums (P1 > 1)
  float* part2;        // [rows][tiles2][P2][64] down partial sums (P2 > 1)
  int tiles1, tiles2;  // f/64, d/64
  int P1, P2;          // input-dimension parts per tile
  int n_items1, n_items2;
};

struct Slot {
  const uint8_t* blk;
  int M;         // tokens
  int p0;        // first grouped position (routed experts)
  bool shared;
  bool live;
};

__device__ __forceinline__ Slot resolve_slot(const DecodeArgs& g, int slot) {
  Slot s{nullptr, 0, 0, false, false};
  if (slot < g.has_shared) {
    s.blk = g.shared;
    s.M = g.T;
    s.shared = true;
    s.live = true;
    return s;
  }
  // the same for every lane: keep it in scalar registers, so the buffer
  // descriptors built from it are scalar too
  const int ra = slot - g.has_shared;
  if (ra >= __builtin_amdgcn_readfirstlane(g.n_active[0])) return s;
  const int e = __builtin_amdgcn_readfirstlane(g.active[ra]);
  s.blk = g.experts + static_cast<size_t>(e) * g.block_bytes;
  s.p0 = __builtin_amdgcn_readfirstlane(g.offsets[e]);
  s.M = __builtin_amdgcn_readfirstlane(g.offsets[e + 1]) - s.p0;
  s.live = true;
  return s;
}

// Position of token m of a slot in the h / y row space (shared rows follow
// the T*k routed positions).
__device__ __forceinline__ int row_of(const DecodeArgs& g, const Slot& sl, int m) {
  return sl.shared ? g.T * g.top_k + m : sl.p0 + m;
}

// ---------------------------------------------------------------------------
// one pipeline step of codes + scales for NM matrices of a tile
// ---------------------------------------------------------------------------

template <int NM>
struct Step {
  uint4 q[NM][kStep];
  float s[NM][kStep];
};

// Buffer resources of one tile's codes and scales for NM matrices: loads go
// through a 128-bit scalar descriptor plus one lane offset, so no per-load
// 64-bit addresses occupy vector registers, and a read past the tile returns
// zero instead of touching other memory.
template <int NM>
struct TileRes {
  __amdgpu_buffer_rsrc_t q[NM];
  __amdgpu_buffer_rsrc_t s[NM];
};

constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit buffer access

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcWord3);
}

// Loads are unconditional (chunk indices past the wavefront's range are
// clamped to its last chunk, a cache hit), so the compiler sees the same
// number of loads in flight on every path and can wait for exactly the step
// it needs instead of for everything.
template <int NM>
__device__ __forceinline__ void load_step(const TileRes<NM>& res, int c0, int ce, int cbase,
                                          int lane, Step<NM>& d) {
#pragma unroll
  for (int i = 0; i < kStep; ++i) {
    const int c = cbase + min(c0 + i, ce - 1);
#pragma unroll
    for (int mat = 0; mat < NM; ++mat) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(res.q[mat], lane * 16, c * 1024, 0);
      d.q[mat][i] = make_uint4(v[0], v[1], v[2], v[3]);
      const unsigned short h =
          __builtin_amdgcn_raw_buffer_load_b16(res.s[mat], lane * 2, (c >> 1) * 128, 0);
      d.s[mat][i] = static_cast<float>(__builtin_bit_cast(_Float16, h));
    }
  }
}

// XW: activation words per chunk in LDS (16: bf16 pairs; 32: hi pairs then lo pairs)
template <int NM, int MT, int XW>
__device__ __forceinline__ void math_step(const Step<NM>& d, int c0, int ce, int nt,
                                          const uint32_t* xl, const float* xs, int chunks,
                                          float (&acc)[NM][MT]) {
#pragma unroll
  for (int i = 0; i < kStep; ++i) {
    const int c = c0 + i;
    if (c >= ce) break;
    float tc[NM][MT];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // the activation pairs of this 8-column word, once for every matrix
      uint4 xh[MT], xo[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < nt) {
          xh[m] = *reinterpret_cast<const uint4*>(xl + (m * chunks + c) * XW + 4 * w);
          if constexpr (XW == 32)
            xo[m] = *reinterpret_cast<const uint4*>(xl + (m * chunks + c) * XW + 16 + 4 * w);
        }
      }
#pragma unroll
      for (int mat = 0; mat < NM; ++mat) {
        const uint32_t u = w == 0 ? d.q[mat][i].x : w == 1 ? d.q[mat][i].y : w == 2 ? d.q[mat][i].z : d.q[mat][i].w;
        const uint32_t b0 = (u & kMask) ^ kMagicX;
        const uint32_t b1 = ((u >> 4) & kMask) ^ kMagicX;
        const uint32_t b2 = ((u >> 8) & kMask) ^ kMagicX;
        const uint32_t b3 = ((u >> 12) & kMask) ^ kMagicX;
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
    for (int mat = 0; mat < NM; ++mat)
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < nt)
          acc[mat][m] = fmaf(d.s[mat][i], fmaf(-kOffset, xs[m * chunks + c], tc[mat][m]), acc[mat][m]);
  }
}

// Partial sums of this wavefront over chunks cbase + [0, nc) of the tile,
// whose activations sit in LDS at local chunk indices [0, nc): two step
// buffers, the next step's loads in flight while the current step's math
// runs.
template <int NM, int MT, int XW>
__device__ __forceinline__ void tile_sweep(const TileRes<NM>& res, int cbase, int nc, int nt,
                                           const uint32_t* xl, const float* xs, int lane,
                                           float (&acc)[NM][MT]) {
#pragma unroll
  for (int mat = 0; mat < NM; ++mat)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[mat][m] = 0.0f;
  if (nc <= 0) return;
  Step<NM> a, b;
  load_step<NM>(res, 0, nc, cbase, lane, a);
  for (int c0 = 0; c0 < nc; c0 += 2 * kStep) {
    load_step<NM>(res, c0 + kStep, nc, cbase, lane, b);
    math_step<NM, MT, XW>(a, c0, nc, nt, xl, xs, nc, acc);
    load_step<NM>(res, c0 + 2 * kStep, nc, cbase, lane, a);
    math_step<NM, MT, XW>(b, c0 + kStep, nc, nt, xl, xs, nc, acc);
  }
}

// ---------------------------------------------------------------------------
// LDS staging of the item's activations (chunks [cb, ce) of the input)
// ---------------------------------------------------------------------------

// x rows of the gate/up phase: bf16 copied as pairs, or f32 split into hi/lo.
template <bool XF32>
__device__ __forceinline__ void stage_x(const DecodeArgs& g, const Slot& sl, int m0, int nt,
                                        int cb, int ce, uint32_t* xl, float* xs) {
  constexpr int XW = XF32 ? 32 : 16;
  const int nc = ce - cb;
  for (int i = threadIdx.x; i < nt * nc; i += kWave) {
    const int m = i / nc, cc = i - m * nc, c = cb + cc;
    const int tok = sl.shared ? m0 + m : g.perm[sl.p0 + m0 + m] / g.top_k;
    uint32_t* dst = xl + (m * nc + cc) * XW;
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
    xs[m * nc + cc] = s;
  }
}

// h rows of the down phase (already hi/lo pairs), read at device scope.
__device__ __forceinline__ void stage_h(const DecodeArgs& g, const Slot& sl, int m0, int nt,
                                        int cb, int ce, uint32_t* xl, float* xs) {
  const int chunks = g.f / 32, nc = ce - cb;
  for (int i = threadIdx.x; i < nt * nc * 32; i += kWave) {
    const int m = i / (nc * 32), rest = i - m * nc * 32;
    const size_t row = row_of(g, sl, m0 + m);
    xl[m * nc * 32 + rest] = __hip_atomic_load(g.hp + (row * chunks + cb) * 32 + rest, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
  }
  for (int i = threadIdx.x; i < nt * nc; i += kWave) {
    const int m = i / nc, cc = i - m * nc;
    const size_t row = row_of(g, sl, m0 + m);
    xs[m * nc + cc] =
        __hip_atomic_load(g.hs + row * chunks + cb + cc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ void wait_for(const DecodeArgs& g, const int* counter, int need) {
  const uint64_t t0 = wall_clock64();
  while (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
    __builtin_amdgcn_s_sleep(2);
    if (wall_clock64() - t0 > kSpinLimit) {
      atomicOr(g.ctrl + kTimeout, 1);
      break;
    }
  }
}

__device__ __forceinline__ float load_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publish this wavefront's device-scope stores, then bump a counter; returns
// the counter's previous value (the same in every lane).
__device__ __forceinline__ int publish(int* counter) {
  __builtin_amdgcn_s_waitcnt(0);  // the stores above have completed
  __syncthreads();
  int old = 0;
  if (threadIdx.x == 0)
    old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __shfl(old, 0, kWave);
}

// h of one token for this tile's 64 rows, written as bf16 hi/lo pairs plus
// the 32-row chunk sums the down phase needs.
__device__ __forceinline__ void write_h(const DecodeArgs& g, size_t row, int tile, float gs, float us) {
  const int lane = threadIdx.x;
  const int fchunks = g.f / 32;
  const float h = silu(gs) * us;
  const uint32_t hi = f32_to_bf16(h);
  const uint32_t lo = f32_to_bf16(h - __uint_as_float(hi << 16));
  const uint32_t hi_o = __shfl_xor(hi, 1, kWave), lo_o = __shfl_xor(lo, 1, kWave);
  // row r = tile*64 + lane sits in chunk tile*2 + lane/32, pair (lane%32)/2
  const int c = tile * 2 + (lane >> 5), j = (lane & 31) >> 1;
  uint32_t* hrow = g.hp + (row * fchunks + c) * 32;
  if ((lane & 1) == 0)
    __hip_atomic_store(hrow + j, hi | (hi_o << 16), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    __hip_atomic_store(hrow + 16 + j, lo_o | (lo << 16), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  float part = __uint_as_float(hi << 16) + __uint_as_float(lo << 16);
  part = group_sum(part, 32);
  if ((lane & 31) == 0) store_dev(g.hs + row * fchunks + c, part);
}

// ---------------------------------------------------------------------------
// the two phases
// ---------------------------------------------------------------------------

template <int MT, bool XF32>
__device__ void gateup_item(const DecodeArgs& g, const Slot& sl, int slot, int tile, int kp,
                            uint32_t* xl, float* xs) {
  constexpr int XW = XF32 ? 32 : 16;
  const int lane = threadIdx.x;
  const int chunks = g.d / 32;
  const int cb = kp * chunks / g.P1, ce = (kp + 1) * chunks / g.P1;
  const size_t tq = static_cast<size_t>(tile) * 64 * (g.d / 2), ts = static_cast<size_t>(tile) * 2 * g.d;
  TileRes<2> res;
  res.q[0] = make_rsrc(sl.blk + g.q_gate + tq, 32u * g.d);
  res.q[1] = make_rsrc(sl.blk + g.q_up + tq, 32u * g.d);
  res.s[0] = make_rsrc(sl.blk + g.s_gate + ts, 2u * g.d);
  res.s[1] = make_rsrc(sl.blk + g.s_up + ts, 2u * g.d);
  for (int m0 = 0; m0 < sl.M; m0 += MT) {
    const int nt = min(MT, sl.M - m0);
    __syncthreads();
    stage_x<XF32>(g, sl, m0, nt, cb, ce, xl, xs);
    __syncthreads();
    float acc[2][MT];
    tile_sweep<2, MT, XW>(res, cb, ce - cb, nt, xl, xs, lane, acc);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= nt) break;
      const size_t row = row_of(g, sl, m0 + m);
      if (g.P1 == 1) {
        write_h(g, row, tile, acc[0][m], acc[1][m]);
      } else {
        float* pp = g.part1 + ((row * g.tiles1 + tile) * g.P1 + kp) * 128;
        store_dev(pp + lane, acc[0][m]);
        store_dev(pp + 64 + lane, acc[1][m]);
      }
    }
  }
  if (g.P1 > 1) {
    // the last part to arrive adds the parts in order and writes h
    int* tc = g.tcnt1 + slot * g.tiles1 + tile;
    if (publish(tc) != g.P1 - 1) return;
    for (int m = 0; m < sl.M; ++m) {
      const size_t row = row_of(g, sl, m);
      const float* pp = g.part1 + (row * g.tiles1 + tile) * g.P1 * 128;
      float gs = 0.0f, us = 0.0f;
      for (int q = 0; q < g.P1; ++q) {
        gs += load_dev(pp + q * 128 + lane);
        us += load_dev(pp + q * 128 + 64 + lane);
      }
      write_h(g, row, tile, gs, us);
    }
    if (lane == 0) __hip_atomic_store(tc, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // h of this tile is complete for every token of the slot
  publish(g.ctrl + slot * kLineWords);
}

template <int MT>
__device__ void down_item(const DecodeArgs& g, const Slot& sl, int slot, int tile, int kp,
                          uint32_t* xl, float* xs) {
  const int lane = threadIdx.x;
  const int chunks = g.f / 32;
  const int cb = kp * chunks / g.P2, ce = (kp + 1) * chunks / g.P2;
  TileRes<1> res;
  res.q[0] = make_rsrc(sl.blk + g.q_down + static_cast<size_t>(tile) * 64 * (g.f / 2), 32u * g.f);
  res.s[0] = make_rsrc(sl.blk + g.s_down + static_cast<size_t>(tile) * 2 * g.f, 2u * g.f);
  int* line = g.ctrl + slot * kLineWords;
  if (lane == 0) wait_for(g, line, g.tiles1);
  __syncthreads();
  for (int m0 = 0; m0 < sl.M; m0 += MT) {
    const int nt = min(MT, sl.M - m0);
    __syncthreads();
    stage_h(g, sl, m0, nt, cb, ce, xl, xs);
    __syncthreads();
    float acc[1][MT];
    tile_sweep<1, MT, 32>(res, cb, ce - cb, nt, xl, xs, lane, acc);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m >= nt) break;
      const size_t row = row_of(g, sl, m0 + m);
      if (g.P2 == 1) {
        float* out = sl.shared ? g.y_shared + static_cast<size_t>(m0 + m) * g.d
                               : g.y + static_cast<size_t>(sl.p0 + m0 + m) * g.d;
        out[tile * 64 + lane] = acc[0][m];
      } else {
        store_dev(g.part2 + ((row * g.tiles2 + tile) * g.P2 + kp) * 64 + lane, acc[0][m]);
      }
    }
  }
  if (g.P2 > 1) {
    int* tc = g.tcnt2 + slot * g.tiles2 + tile;
    if (publish(tc) != g.P2 - 1) return;
    for (int m = 0; m < sl.M; ++m) {
      const size_t row = row_of(g, sl, m);
      const float* pp = g.part2 + (row * g.tiles2 + tile) * g.P2 * 64;
      float ys = 0.0f;
      for (int q = 0; q < g.P2; ++q) ys += load_dev(pp + q * 64 + lane);
      float* out = sl.shared ? g.y_shared + static_cast<size_t>(m) * g.d
                             : g.y + static_cast<size_t>(sl.p0 + m) * g.d;
      out[tile * 64 + lane] = ys;
    }
    if (lane == 0) __hip_atomic_store(tc, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the slot's last down tile clears both slot counters for the next call
  __syncthreads();
  if (lane == 0 &&
      __hip_atomic_fetch_add(line + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g.tiles2 - 1) {
    __hip_atomic_store(line, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(line + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int MT, bool XF32>
__global__ __launch_bounds__(kWave) void decode_ffn(DecodeArgs g, int lds_words) {
  extern __shared__ __align__(16) uint32_t lds[];
  uint32_t* xl = lds;                                   // activations of the part
  float* xs = reinterpret_cast<float*>(lds + lds_words);  // their chunk sums
  const int n_items = g.n_items1 + g.n_items2;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    if (item < g.n_items1) {
      const int per_slot = g.tiles1 * g.P1;
      const int slot = item / per_slot, r = item - slot * per_slot;
      const Slot sl = resolve_slot(g, slot);
      if (!sl.live) continue;
      gateup_item<MT, XF32>(g, sl, slot, r / g.P1, r % g.P1, xl, xs);
    } else {
      const int it = item - g.n_items1;
      const int per_slot = g.tiles2 * g.P2;
      const int slot = it / per_slot, r = it - slot * per_slot;
      const Slot sl = resolve_slot(g, slot);
      if (!sl.live) continue;
      down_item<MT>(g, sl, slot, r / g.P2, r % g.P2, xl, xs);
    }
  }
}

// Parts per tile: from the layer shape alone (about 24 gate/up or 16 down
// chunks per part, a power of two up to 16), so a token's summation order --
// and its result, bit for bit -- does not depend on the batch it comes in.
// The 1-token step of the ~19 MB-expert layer gets 9 x 32 x 8 = 2304 gate/up
// and 9 x 96 x 4 = 3456 down wavefronts.  Batches of more than 64 tokens have
// enough tiles by themselves and use one part (no partial-sum traffic).
constexpr int kSplitMaxTokens = 64;

int parts_for(int chunks, int per_part, int T) {
  if (T > kSplitMaxTokens) return 1;
  int p = 1;
  while (chunks / p > per_part && p < 16) p *= 2;
  return p;
}

struct Layout {
  int P1, P2;
  size_t ctrl_words, hp, hs, part1, part2, total;  // byte offsets / sizes
};

Layout layout_for(int T, int k, int E, int d, int f, bool has_shared) {
  Layout l{};
  const int slots = (has_shared ? 1 : 0) + std::min(E, T * k);
  const int tiles1 = f / 64, tiles2 = d / 64;
  l.P1 = parts_for(d / 32, 24, T);
  l.P2 = parts_for(f / 32, 16, T);
  const size_t rows = static_cast<size_t>(T) * (k + (has_shared ? 1 : 0));
  l.ctrl_words = kTileCounters + static_cast<size_t>(slots) * (tiles1 + tiles2);
  size_t off = (l.ctrl_words * 4 + 255) / 256 * 256;
  l.hp = off;
  off += rows * f * 4;
  l.hs = off;
  off += (rows * (f / 32) * 4 + 255) / 256 * 256;
  l.part1 = off;
  if (l.P1 > 1) off += rows * tiles1 * l.P1 * 128 * 4;
  l.part2 = off;
  if (l.P2 > 1) off += rows * tiles2 * l.P2 * 64 * 4;
  l.total = off;
  return l;
}

int lds_words_for(int d, int f, int P1, int P2, int mt, bool xf32) {
  const int c1 = (d / 32 + P1 - 1) / P1, c2 = (f / 32 + P2 - 1) / P2;
  return mt * std::max(c1 * (xf32 ? 32 : 16), c2 * 32);
}

size_t lds_bytes_for(int d, int f, int P1, int P2, int mt, bool xf32) {
  const int c1 = (d / 32 + P1 - 1) / P1, c2 = (f / 32 + P2 - 1) / P2;
  return (static_cast<size_t>(lds_words_for(d, f, P1, P2, mt, xf32)) + mt * std::max(c1, c2)) * 4;
}

constexpr size_t kMaxLds = 64 * 1024;

// Workgroups of a kernel the GPU holds at once, for a given LDS size: the
// persistent grid must not exceed it.  Cached per (kernel, device, LDS size).
int resident_capacity(const void* kernel, size_t lds) {
  static std::mutex mu;
  static std::vector<std::pair<std::pair<const void*, int>, std::pair<size_t, int>>> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& e : cache)
    if (e.first.first == kernel && e.first.second == dev && e.second.first == lds) return e.second.second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kWave, lds) != hipSuccess ||
      per_cu <= 0)
    return 0;
  cache.push_back({{kernel, dev}, {lds, cus * per_cu}});
  return cus * per_cu;
}

template <int MT, bool XF32>
hipError_t launch_mt(const DecodeArgs& g, hipStream_t s) {
  auto kernel = decode_ffn<MT, XF32>;
  const int words = lds_words_for(g.d, g.f, g.P1, g.P2, MT, XF32);
  const size_t lds = lds_bytes_for(g.d, g.f, g.P1, g.P2, MT, XF32);
  const int cap = resident_capacity(reinterpret_cast<const void*>(kernel), lds);
  if (cap <= 0) return hipErrorInvalidValue;
  const int grid = std::min(cap, g.n_items1 + g.n_items2);
  return launch(kernel, dim3(static_cast<unsigned>(grid)), dim3(kWave), lds, s, g, words);
}

}  // namespace

size_t ffn_decode_workspace(int T, int k, int E, int d, int f, bool has_shared) {
  return layout_for(T, k, E, d, f, has_shared).total;
}

hipError_t launch_ffn_decode(const FfnProblem& p, hipStream_t stream) {
  const size_t dd = p.d, ff = p.f;
  const Layout l = layout_for(p.T, p.k, p.E, p.d, p.f, p.has_shared);
  DecodeArgs g{};
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
  g.slots = g.has_shared + std::min(p.E, p.T * p.k);
  g.d = p.d;
  g.f = p.f;
  g.q_gate = 0;
  g.q_up = ff * dd / 2;
  g.q_down = ff * dd;
  g.s_gate = 3 * dd * ff / 2;
  g.s_up = g.s_gate + ff * (dd / 64) * 2;
  g.s_down = g.s_up + ff * (dd / 64) * 2;
  g.x = p.x;
  char* ws = static_cast<char*>(p.workspace);
  g.ctrl = reinterpret_cast<int*>(ws);
  g.tcnt1 = g.ctrl + kTileCounters;
  g.tiles1 = p.f / 64;
  g.tiles2 = p.d / 64;
  g.tcnt2 = g.tcnt1 + static_cast<size_t>(g.slots) * g.tiles1;
  g.hp = reinterpret_cast<uint32_t*>(ws + l.hp);
  g.hs = reinterpret_cast<float*>(ws + l.hs);
  g.part1 = reinterpret_cast<float*>(ws + l.part1);
  g.part2 = reinterpret_cast<float*>(ws + l.part2);
  g.y = static_cast<float*>(p.y);
  g.y_shared = static_cast<float*>(p.y_shared);
  g.P1 = l.P1;
  g.P2 = l.P2;
  g.n_items1 = g.slots * g.tiles1 * g.P1;
  g.n_items2 = g.slots * g.tiles2 * g.P2;
  const bool xf32 = !p.x_bf16;
  // two tokens per sweep when experts can hold several and the LDS fits
  const bool two = p.T >= 2 && lds_bytes_for(p.d, p.f, l.P1, l.P2, 2, xf32) <= kMaxLds;
  if (!two && lds_bytes_for(p.d, p.f, l.P1, l.P2, 1, xf32) > kMaxLds) return hipErrorNotSupported;
  if (xf32) return two ? launch_mt<2, true>(g, stream) : launch_mt<1, true>(g, stream);
  return two ? launch_mt<2, false>(g, stream) : launch_mt<1, false>(g, stream);
}

}  // namespace moe
