// Decode-path expert FFN: an HBM-bound int4 GEMV over the batch-union
// (pages: zhichai.net, sections on MoE sparsity and the three storage tiers
// -- 8 routed + 1 shared int4 expert per token, each a ~19 MB block;
// yunpan.plus article, "capability 2" -- each routed expert read once for all
// tokens of the batch that chose it).
//
// Two launches per call:
//   gate/up  h[p] = silu(W_gate x) * (W_up x)   for every grouped position p
//   down     y[p] = W_down h[p]
// Both run one kernel template.  A workgroup is one wavefront that owns a
// block of output rows of one expert and sweeps them for all of that expert's
// tokens (several tokens per sweep), so every weight byte is fetched from HBM
// once per expert.  Lanes split a row's input dimension into 16-byte chunks
// (32 int4 codes); `lpr` lanes work on one row, 64/lpr rows per sweep step.
//
// Dequant: a code byte pair word v (8 nibbles, XOR 0x88888888 turns each
// two's-complement nibble n into n+8) gives four bf16 pairs with one
// and-or each: (v >> 4i) & 0x000F000F | 0x43004300 is the bf16 pair
// (136 + n_a, 136 + n_b), exactly.  v_dot2_f32_bf16 multiplies them with the
// matching activation pairs (products exact in fp32); the 136 offset is
// removed with the chunk's precomputed activation sum, and the fp16 group
// scale is applied once per 32 codes.  float32 activations (and the float32 h
// fed to the down projection) are split into bf16 hi + lo parts first, so
// they keep 16 significant bits; accumulation is float32 throughout.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace moe {

namespace {

struct GemvArgs {
  const uint8_t* experts;
  const uint8_t* shared;
  size_t block_bytes;
  int K;                // input dimension of the matrices
  int N;                // output rows
  size_t q_off[2];      // byte offsets of the code matrices inside a block
  size_t s_off[2];      // byte offsets of their fp16 scales
  const void* in;       // input rows, K wide
  int in_gather;        // 1: routed position p reads in[perm[p] / top_k]; 0: in[p]
  int shared_in_row0;   // input row of shared-expert token 0
  float* out;           // routed position p writes out + p*N
  float* out_shared;    // shared token m writes out_shared + m*N
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* active;
  const int32_t* n_active;
  int top_k;
  int T;
  int has_shared;
  int lpr;              // lanes per row: 8, 16, 32 or 64
  int rows_per_block;
  int row_blocks;
};

constexpr uint32_t kMagic = 0x43004300u;  // bf16 pair (128, 128)
constexpr float kOffset = 136.0f;         // 128 + 8

// Activation chunk (32 consecutive inputs) of one token, as bf16 pairs laid
// out to match the nibble pairing (col+p, col+p+4), p = 0..3, per 8-column
// word; XF32 adds the low halves after the high halves.
template <bool XF32>
struct XChunk {
  static constexpr int kWords = XF32 ? 32 : 16;
};

template <bool XF32>
__device__ __forceinline__ void load_chunk(const void* in, size_t elem0, bool ok,
                                           uint32_t (&xv)[XChunk<XF32>::kWords], float& xsum) {
  if (!ok) {
#pragma unroll
    for (int j = 0; j < XChunk<XF32>::kWords; ++j) xv[j] = 0u;
    xsum = 0.0f;
    return;
  }
  if constexpr (!XF32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(in) + elem0);
    uint32_t r[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = p[j];
      r[4 * j + 0] = v.x; r[4 * j + 1] = v.y; r[4 * j + 2] = v.z; r[4 * j + 3] = v.w;
    }
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a = r[4 * w + 0], b = r[4 * w + 1], c = r[4 * w + 2], d = r[4 * w + 3];
      xv[4 * w + 0] = (a & 0xFFFFu) | (c << 16);
      xv[4 * w + 1] = (a >> 16) | (c & 0xFFFF0000u);
      xv[4 * w + 2] = (b & 0xFFFFu) | (d << 16);
      xv[4 * w + 3] = (b >> 16) | (d & 0xFFFF0000u);
      s += __uint_as_float(a << 16) + __uint_as_float(a & 0xFFFF0000u) +
           __uint_as_float(b << 16) + __uint_as_float(b & 0xFFFF0000u) +
           __uint_as_float(c << 16) + __uint_as_float(c & 0xFFFF0000u) +
           __uint_as_float(d << 16) + __uint_as_float(d & 0xFFFF0000u);
    }
    xsum = s;
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(in) + elem0);
    float v[32];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 q = p[j];
      v[4 * j + 0] = q.x; v[4 * j + 1] = q.y; v[4 * j + 2] = q.z; v[4 * j + 3] = q.w;
    }
    uint32_t hi[32], lo[32];
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      hi[j] = f32_to_bf16(v[j]);
      const float hf = __uint_as_float(hi[j] << 16);
      lo[j] = f32_to_bf16(v[j] - hf);
      s += hf + __uint_as_float(lo[j] << 16);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        xv[4 * w + p] = hi[8 * w + p] | (hi[8 * w + p + 4] << 16);
        xv[16 + 4 * w + p] = lo[8 * w + p] | (lo[8 * w + p + 4] << 16);
      }
    }
    xsum = s;
  }
}

template <int NCH, int NT, bool XF32, bool GATEUP>
__device__ __forceinline__ void gemv_pass(const GemvArgs& a, const uint8_t* blk, bool is_shared,
                                          int p0, int m0, int lane) {
  constexpr int NM = GATEUP ? 2 : 1;
  constexpr int XW = XChunk<XF32>::kWords;
  const int lpr = a.lpr;
  const int rpp = kWave / lpr;
  const int q = lane / lpr, sub = lane % lpr;
  const int chunks = a.K >> 5;

  uint32_t xv[NT][NCH][XW];
  float xs[NT][NCH];
  float* orow[NT];
#pragma unroll
  for (int m = 0; m < NT; ++m) {
    int row;
    if (is_shared) {
      row = a.shared_in_row0 + m0 + m;
      orow[m] = a.out_shared + static_cast<size_t>(m0 + m) * a.N;
    } else {
      const int p = p0 + m0 + m;
      row = a.in_gather ? a.perm[p] / a.top_k : p;
      orow[m] = a.out + static_cast<size_t>(p) * a.N;
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = sub + lpr * i;
      load_chunk<XF32>(a.in, static_cast<size_t>(row) * a.K + static_cast<size_t>(c) * 32,
                       c < chunks, xv[m][i], xs[m][i]);
    }
  }

  const int r_begin = (blockIdx.x % a.row_blocks) * a.rows_per_block;
  const int r_end = min(a.N, r_begin + a.rows_per_block);
  for (int r0 = r_begin; r0 < r_end; r0 += rpp) {
    const int r = r0 + q;
    const bool rv = r < r_end;
    float acc[NM][NT];
#pragma unroll
    for (int mat = 0; mat < NM; ++mat) {
#pragma unroll
      for (int m = 0; m < NT; ++m) acc[mat][m] = 0.0f;
      const uint8_t* qrow = blk + a.q_off[mat] + static_cast<size_t>(r) * (a.K >> 1);
      const _Float16* srow = reinterpret_cast<const _Float16*>(blk + a.s_off[mat]) +
                             static_cast<size_t>(r) * (a.K >> 6);
      uint4 code[NCH];
      float scale[NCH];
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = sub + lpr * i;
        if (rv && c < chunks) {
          code[i] = *reinterpret_cast<const uint4*>(qrow + static_cast<size_t>(c) * 16);
          scale[i] = static_cast<float>(srow[c >> 1]);
        } else {
          code[i] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
          scale[i] = 0.0f;
        }
      }
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const uint32_t u[4] = {code[i].x, code[i].y, code[i].z, code[i].w};
        float t[NT];
#pragma unroll
        for (int m = 0; m < NT; ++m) t[m] = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t v = u[w] ^ 0x88888888u;
          const uint32_t b0 = (v & 0x000F000Fu) | kMagic;
          const uint32_t b1 = ((v >> 4) & 0x000F000Fu) | kMagic;
          const uint32_t b2 = ((v >> 8) & 0x000F000Fu) | kMagic;
          const uint32_t b3 = ((v >> 12) & 0x000F000Fu) | kMagic;
#pragma unroll
          for (int m = 0; m < NT; ++m) {
            t[m] = dot2_bf16(b0, xv[m][i][4 * w + 0], t[m]);
            t[m] = dot2_bf16(b1, xv[m][i][4 * w + 1], t[m]);
            t[m] = dot2_bf16(b2, xv[m][i][4 * w + 2], t[m]);
            t[m] = dot2_bf16(b3, xv[m][i][4 * w + 3], t[m]);
            if constexpr (XF32) {
              t[m] = dot2_bf16(b0, xv[m][i][16 + 4 * w + 0], t[m]);
              t[m] = dot2_bf16(b1, xv[m][i][16 + 4 * w + 1], t[m]);
              t[m] = dot2_bf16(b2, xv[m][i][16 + 4 * w + 2], t[m]);
              t[m] = dot2_bf16(b3, xv[m][i][16 + 4 * w + 3], t[m]);
            }
          }
        }
#pragma unroll
        for (int m = 0; m < NT; ++m)
          acc[mat][m] = fmaf(scale[i], t[m] - kOffset * xs[m][i], acc[mat][m]);
      }
#pragma unroll
      for (int m = 0; m < NT; ++m) acc[mat][m] = group_sum(acc[mat][m], lpr);
    }
    if (rv && sub == 0) {
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        float v = acc[0][m];
        if constexpr (GATEUP) v = silu(acc[0][m]) * acc[1][m];
        orow[m][r] = v;
      }
    }
  }
}

template <int NCH, int MT, bool XF32, bool GATEUP>
__global__ __launch_bounds__(64) void int4_gemv(GemvArgs a) {
  const int lane = threadIdx.x;
  const int slot = blockIdx.x / a.row_blocks;
  const uint8_t* blk;
  int M, p0;
  bool is_shared;
  if (slot < a.has_shared) {
    blk = a.shared;
    M = a.T;
    p0 = 0;
    is_shared = true;
  } else {
    const int ra = slot - a.has_shared;
    if (ra >= a.n_active[0]) return;
    const int e = a.active[ra];
    blk = a.experts + static_cast<size_t>(e) * a.block_bytes;
    p0 = a.offsets[e];
    M = a.offsets[e + 1] - p0;
    is_shared = false;
  }
  for (int m0 = 0; m0 < M; m0 += MT) {
    const int nt = min(MT, M - m0);
    if constexpr (MT >= 4) {
      if (nt == 4) { gemv_pass<NCH, 4, XF32, GATEUP>(a, blk, is_shared, p0, m0, lane); continue; }
      if (nt == 3) { gemv_pass<NCH, 3, XF32, GATEUP>(a, blk, is_shared, p0, m0, lane); continue; }
    }
    if constexpr (MT >= 2) {
      if (nt == 2) { gemv_pass<NCH, 2, XF32, GATEUP>(a, blk, is_shared, p0, m0, lane); continue; }
    }
    gemv_pass<NCH, 1, XF32, GATEUP>(a, blk, is_shared, p0, m0, lane);
  }
}

// Per-lane activation registers of a sweep: NCH chunks x MT tokens x words.
template <int NCH, int MT, bool XF32>
constexpr bool fits() {
  return NCH * MT * XChunk<XF32>::kWords <= 128;
}

template <int NCH, bool XF32, bool GATEUP>
hipError_t launch_mt(int mt, const GemvArgs& a, dim3 grid, hipStream_t s) {
  if constexpr (fits<NCH, 4, XF32>())
    if (mt == 4) return launch(int4_gemv<NCH, 4, XF32, GATEUP>, grid, dim3(64), 0, s, a);
  if constexpr (fits<NCH, 2, XF32>())
    if (mt == 2) return launch(int4_gemv<NCH, 2, XF32, GATEUP>, grid, dim3(64), 0, s, a);
  if (mt != 1) return hipErrorInvalidValue;
  return launch(int4_gemv<NCH, 1, XF32, GATEUP>, grid, dim3(64), 0, s, a);
}

template <bool XF32, bool GATEUP>
hipError_t launch_nch(int nch, int mt, const GemvArgs& a, dim3 grid, hipStream_t s) {
  switch (nch) {
    case 1: return launch_mt<1, XF32, GATEUP>(mt, a, grid, s);
    case 2: return launch_mt<2, XF32, GATEUP>(mt, a, grid, s);
    case 3: return launch_mt<3, XF32, GATEUP>(mt, a, grid, s);
    case 4: return launch_mt<4, XF32, GATEUP>(mt, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

struct Tiling {
  int lpr, nch, mt;
};

// Lanes per row and chunks per lane for an input dimension K: fewest idle
// lanes first, then the most chunks per lane (fewest cross-lane reduction
// steps per weight) within a per-lane register budget for the activations.
Tiling choose_tiling(int K, bool split, int max_tokens) {
  const int chunks = K / 32;
  const int cap = split ? 2 : 3;
  Tiling best{64, (chunks + 63) / 64, 1};
  int best_waste = 1 << 30;
  for (int lpr = 64; lpr >= 8; lpr >>= 1) {
    const int nch = (chunks + lpr - 1) / lpr;
    if (nch > 4 || (nch > cap && lpr != 64)) continue;
    const int waste = nch * lpr - chunks;
    if (waste < best_waste || (waste == best_waste && nch > best.nch)) {
      best = {lpr, nch, 1};
      best_waste = waste;
    }
  }
  const int words = split ? 32 : 16;
  int mt = 1;
  while (mt < 4 && mt * 2 <= max_tokens && best.nch * words * mt * 2 <= 128) mt *= 2;
  best.mt = mt;
  return best;
}

}  // namespace

size_t ffn_decode_workspace(int T, int k, int f, bool has_shared) {
  return static_cast<size_t>(T) * (k + (has_shared ? 1 : 0)) * f * sizeof(float);
}

hipError_t launch_ffn_decode(const FfnProblem& p, hipStream_t stream) {
  const size_t dd = p.d, ff = p.f;
  const size_t q_gate = 0, q_up = ff * dd / 2, q_down = ff * dd;
  const size_t s_gate = 3 * dd * ff / 2, s_up = s_gate + ff * (dd / 64) * 2,
               s_down = s_up + ff * (dd / 64) * 2;
  const int slots = (p.has_shared ? 1 : 0) + std::min(p.E, p.T * p.k);
  float* h = static_cast<float*>(p.workspace);
  float* h_shared = h + static_cast<size_t>(p.T) * p.k * p.f;

  // gate/up
  GemvArgs g{};
  g.experts = p.experts;
  g.shared = p.shared;
  g.block_bytes = p.block_bytes;
  g.K = p.d;
  g.N = p.f;
  g.q_off[0] = q_gate; g.q_off[1] = q_up;
  g.s_off[0] = s_gate; g.s_off[1] = s_up;
  g.in = p.x;
  g.in_gather = 1;
  g.shared_in_row0 = 0;
  g.out = h;
  g.out_shared = h_shared;
  g.offsets = p.offsets; g.perm = p.perm; g.active = p.active; g.n_active = p.n_active;
  g.top_k = p.k;
  g.T = p.T;
  g.has_shared = p.has_shared ? 1 : 0;
  const Tiling t1 = choose_tiling(p.d, !p.x_bf16, p.T);
  g.lpr = t1.lpr;
  {
    const int rpp = 64 / t1.lpr;
    const int bytes_per_row = 2 * (p.d / 2);
    int rows = std::max(1, 32768 / bytes_per_row);
    rows = std::max(rpp, rows / rpp * rpp);
    g.rows_per_block = rows;
    g.row_blocks = (p.f + rows - 1) / rows;
  }
  const dim3 grid1(static_cast<unsigned>(slots) * g.row_blocks);
  hipError_t err = p.x_bf16 ? launch_nch<false, true>(t1.nch, t1.mt, g, grid1, stream)
                            : launch_nch<true, true>(t1.nch, t1.mt, g, grid1, stream);
  if (err != hipSuccess) return err;

  // down
  GemvArgs dn = g;
  dn.K = p.f;
  dn.N = p.d;
  dn.q_off[0] = q_down; dn.q_off[1] = q_down;
  dn.s_off[0] = s_down; dn.s_off[1] = s_down;
  dn.in = h;
  dn.in_gather = 0;
  dn.shared_in_row0 = p.T * p.k;
  dn.out = static_cast<float*>(p.y);
  dn.out_shared = static_cast<float*>(p.y_shared);
  const Tiling t2 = choose_tiling(p.f, true, p.T);
  dn.lpr = t2.lpr;
  {
    const int rpp = 64 / t2.lpr;
    const int bytes_per_row = p.f / 2;
    int rows = std::max(1, 32768 / bytes_per_row);
    rows = std::max(rpp, rows / rpp * rpp);
    dn.rows_per_block = rows;
    dn.row_blocks = (p.d + rows - 1) / rows;
  }
  const dim3 grid2(static_cast<unsigned>(slots) * dn.row_blocks);
  return launch_nch<true, false>(t2.nch, t2.mt, dn, grid2, stream);
}

}  // namespace moe
