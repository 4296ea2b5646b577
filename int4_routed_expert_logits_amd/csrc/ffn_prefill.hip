// Prefill-path expert FFN: a grouped GEMM over the batch-union on bf16 MFMA
// (pages: yunpan.plus article, "capability 2" -- the positions of a batch
// that chose an expert are grouped and share one read of its weights;
// zhichai.net, section on MoE sparsity -- 8 routed int4 experts plus the
// shared one per token).
//
//   gate/up  H[rows of slot s] = silu(X_s W_gate^T) * (X_s W_up^T)   (bf16 H)
//   down     Y[rows of slot s] = H_s W_down^T                         (bf16 Y)
//
// Work: for every expert slot (the shared expert first, then the active
// routed experts) its rows -- the grouped positions, i.e. the tokens that
// chose it -- are cut into M-tiles of 32.  A workgroup of 4 wavefronts takes
// one M-tile and 256 output columns; each wavefront computes 32 rows x 64
// columns with v_mfma_f32_32x32x16_bf16, streaming its weights straight from
// the packed tile into registers.  A small kernel first lists the M-tiles.
//
// Dequant into the MFMA: a 4-byte word of the packed codes holds 8
// consecutive input columns, and ((w >> 4i) & 0x000F000F) ^ 0x43084308 is
// the bf16 pair (136 + q) of columns 2i, 2i+1 -- exact -- so one word is one
// 8-element B operand.  Per 64-column scale group g the MFMAs accumulate
// P = sum_k x[m,k] (136 + q[k,n]) on top of a correction C = -136 S_g[m]
// (S_g the row's activation sum over the group, split into three bf16 parts
// and multiplied by -136 in one extra MFMA), and the group scale is applied
// once: acc += s[n,g] * P.  The weights therefore enter the products
// exactly; only the float32 accumulation and the bf16 rounding of H and Y
// round.  Activations are bf16 (an f32 x is rejected by the C ABI).
#include <algorithm>

#include "common.h"
#include "launch.h"

#pragma clang fp contract(off)

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 32;        // rows per M-tile
constexpr int kWaveCols = 64;  // output columns per wavefront
constexpr int kWaves = 4;      // wavefronts per workgroup
constexpr int kWgCols = kWaves * kWaveCols;
constexpr uint32_t kMask = 0x000F000Fu;
constexpr uint32_t kMagicX = 0x43084308u;
constexpr int kRsrcWord3 = 0x00020000;

struct PrefillArgs {
  const uint8_t* experts;
  const uint8_t* shared;
  size_t block_bytes;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* active;
  int top_k;
  int T;
  int has_shared;
  int slots;
  int d, f;
  size_t q_gate, q_up, q_down, s_gate, s_up, s_down;
  const uint16_t* x;   // [T][d] bf16
  uint16_t* h;         // [T*k + T][f] bf16
  uint16_t* y;         // [T*k][d] bf16
  uint16_t* y_shared;  // [T][d] bf16
  int2* tiles;         // (slot, first row) of every M-tile
  int* n_tiles;
};

struct Slot {
  const uint8_t* blk;
  int M;
  int p0;
  bool shared;
};

__device__ __forceinline__ Slot resolve_slot(const PrefillArgs& g, int slot) {
  Slot s{nullptr, 0, 0, false};
  if (slot < g.has_shared) {
    s.blk = g.shared;
    s.M = g.T;
    s.shared = true;
    return s;
  }
  const int e = __builtin_amdgcn_readfirstlane(g.active[slot - g.has_shared]);
  if (e < 0) return s;
  s.blk = g.experts + static_cast<size_t>(e) * g.block_bytes;
  s.p0 = __builtin_amdgcn_readfirstlane(g.offsets[e]);
  s.M = __builtin_amdgcn_readfirstlane(g.offsets[e + 1]) - s.p0;
  return s;
}

__device__ __forceinline__ int row_of(const PrefillArgs& g, const Slot& sl, int m) {
  return sl.shared ? g.T * g.top_k + m : sl.p0 + m;
}

// ---------------------------------------------------------------------------
// M-tile list: one workgroup, slots in chunks of 1024
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void prefill_tiles(PrefillArgs g) {
  __shared__ int wave_tot[16];
  __shared__ int base_s;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) base_s = 0;
  __syncthreads();
  for (int s0 = 0; s0 < g.slots; s0 += 1024) {
    const int slot = s0 + tid;
    int M = 0;
    if (slot < g.slots) {
      if (slot < g.has_shared) {
        M = g.T;
      } else {
        const int e = g.active[slot - g.has_shared];
        if (e >= 0) M = g.offsets[e + 1] - g.offsets[e];
      }
    }
    const int nt = (M + kBM - 1) / kBM;
    int incl = nt;
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wave_tot[wv] = incl;
    __syncthreads();
    int before = base_s;
    for (int w = 0; w < wv; ++w) before += wave_tot[w];
    int total = 0;
    for (int w = 0; w < 16; ++w) total += wave_tot[w];
    const int pos = before + incl - nt;
    for (int i = 0; i < nt; ++i) g.tiles[pos + i] = make_int2(slot, i * kBM);
    __syncthreads();
    if (tid == 0) base_s += total;
    __syncthreads();
  }
  if (tid == 0) g.n_tiles[0] = base_s;
}

// ---------------------------------------------------------------------------
// shared GEMM core
// ---------------------------------------------------------------------------

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// The 8-element B operand of packed word w: bf16 pairs (136 + q).
__device__ __forceinline__ bf16x8_t dequant_word(uint32_t w) {
  const uint4 b = make_uint4((w & kMask) ^ kMagicX, ((w >> 4) & kMask) ^ kMagicX,
                             ((w >> 8) & kMask) ^ kMagicX, ((w >> 12) & kMask) ^ kMagicX);
  return as_bf16x8(b);
}

__device__ __forceinline__ uint32_t word_of(const uint4& q, int j) {
  return j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
}

// Sum of the 8 bf16 values of a fragment, in order.
__device__ __forceinline__ float frag_sum(const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += __uint_as_float(w[i] << 16) + __uint_as_float(w[i] & 0xFFFF0000u);
  return s;
}

// -136 * S for the 32 rows of the tile, replicated over every column, as an
// MFMA result: A holds S split into three bf16 parts in k = 0..2 (lanes of
// the first half), B holds -136 there.
__device__ __forceinline__ f32x16_t offset_correction(float S, int half) {
  const uint32_t s_hi = f32_to_bf16(S);
  const float r1 = S - __uint_as_float(s_hi << 16);
  const uint32_t s_mid = f32_to_bf16(r1);
  const float r2 = r1 - __uint_as_float(s_mid << 16);
  const uint32_t s_lo = f32_to_bf16(r2);
  const uint32_t m136 = f32_to_bf16(-136.0f);
  uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
  if (half == 0) {
    a = make_uint4(s_hi | (s_mid << 16), s_lo, 0, 0);
    b = make_uint4(m136 | (m136 << 16), m136, 0, 0);
  }
  f32x16_t z = {};
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), z, 0, 0, 0);
}

// One K step (a 64-column scale group) of NM matrices x 2 column halves.
template <int NM>
struct KStep {
  uint4 a[4];         // A fragments j = 0..3 (8 bf16 each)
  uint4 q[NM][2];     // codes: 16 bytes = 4 words = 4 B fragments
  float s[NM][2];     // group scales of this lane's columns
};

template <int NM>
__device__ __forceinline__ void load_kstep(const uint16_t* arow, bool arow_ok, int grp,
                                           const __amdgpu_buffer_rsrc_t (&rq)[NM],
                                           const uint16_t* const (&srow)[NM][2], int col,
                                           int half, KStep<NM>& st) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    st.a[j] = arow_ok ? *reinterpret_cast<const uint4*>(arow + grp * 64 + half * 32 + j * 8)
                      : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int mat = 0; mat < NM; ++mat) {
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(
          rq[mat], (2 * grp + half) * 1024 + (ns * 32 + col) * 16, 0, 0);
      st.q[mat][ns] = make_uint4(v[0], v[1], v[2], v[3]);
      st.s[mat][ns] = static_cast<float>(__builtin_bit_cast(_Float16, srow[mat][ns][grp]));
    }
  }
}

template <int NM>
__device__ __forceinline__ void math_kstep(const KStep<NM>& st, int half,
                                           f32x16_t (&acc)[NM][2]) {
  float S = frag_sum(st.a[0]) + frag_sum(st.a[1]) + frag_sum(st.a[2]) + frag_sum(st.a[3]);
  S += __shfl_xor(S, 32, kWave);
  const f32x16_t corr = offset_correction(S, half);
#pragma unroll
  for (int mat = 0; mat < NM; ++mat) {
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
      f32x16_t p = corr;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(st.a[j]),
                                                    dequant_word(word_of(st.q[mat][ns], j)), p,
                                                    0, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mat][ns][i] = fmaf(st.s[mat][ns], p[i], acc[mat][ns][i]);
    }
  }
}

// acc[mat][ns] = this wavefront's 32 x 64 tile of A [32 x K] times the
// packed matrices (rows n0 .. n0+63 of each, K input columns), K/64 steps,
// the next step's loads in flight during the current step's MFMAs.
template <int NM>
__device__ __forceinline__ void gemm_tile(const uint16_t* arow, bool arow_ok, int groups,
                                          const __amdgpu_buffer_rsrc_t (&rq)[NM],
                                          const uint16_t* const (&srow)[NM][2], int col,
                                          int half, f32x16_t (&acc)[NM][2]) {
#pragma unroll
  for (int mat = 0; mat < NM; ++mat)
#pragma unroll
    for (int ns = 0; ns < 2; ++ns)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mat][ns][i] = 0.0f;
  KStep<NM> cur, nxt;
  load_kstep<NM>(arow, arow_ok, 0, rq, srow, col, half, cur);
  for (int grp = 0; grp < groups; ++grp) {
    if (grp + 1 < groups) load_kstep<NM>(arow, arow_ok, grp + 1, rq, srow, col, half, nxt);
    math_kstep<NM>(cur, half, acc);
    cur = nxt;
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcWord3);
}

// Output element i of a 32x32 MFMA tile held by lane (col, half) is row
// (i/4)*8 + half*4 + i%4, column col.
__device__ __forceinline__ int out_row(int i, int half) { return (i >> 2) * 8 + half * 4 + (i & 3); }

// ---------------------------------------------------------------------------
// gate/up
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kWaves * kWave) void prefill_gateup(PrefillArgs g) {
  const int ti = blockIdx.y;
  if (ti >= __builtin_amdgcn_readfirstlane(g.n_tiles[0])) return;
  const int2 tile = g.tiles[ti];
  const int slot = __builtin_amdgcn_readfirstlane(tile.x);
  const int m0 = __builtin_amdgcn_readfirstlane(tile.y);
  const Slot sl = resolve_slot(g, slot);
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * kWgCols + wv * kWaveCols;  // first f-row of this wavefront
  if (n0 >= g.f) return;
  const int col = lane & 31, half = lane >> 5;
  const int m = m0 + col;
  const bool ok = m < sl.M;
  int tok = 0;
  if (ok) tok = sl.shared ? m : g.perm[sl.p0 + m] / g.top_k;
  const uint16_t* arow = g.x + static_cast<size_t>(tok) * g.d;
  const size_t tq = static_cast<size_t>(n0 / 64) * 64 * (g.d / 2);
  const __amdgpu_buffer_rsrc_t rq[2] = {make_rsrc(sl.blk + g.q_gate + tq, 32u * g.d),
                                        make_rsrc(sl.blk + g.q_up + tq, 32u * g.d)};
  const int groups = g.d / 64;
  const uint16_t* sg = reinterpret_cast<const uint16_t*>(sl.blk + g.s_gate);
  const uint16_t* su = reinterpret_cast<const uint16_t*>(sl.blk + g.s_up);
  const uint16_t* const srow[2][2] = {
      {sg + static_cast<size_t>(n0 + col) * groups, sg + static_cast<size_t>(n0 + 32 + col) * groups},
      {su + static_cast<size_t>(n0 + col) * groups, su + static_cast<size_t>(n0 + 32 + col) * groups}};
  f32x16_t acc[2][2];
  gemm_tile<2>(arow, ok, groups, rq, srow, col, half, acc);
#pragma unroll
  for (int ns = 0; ns < 2; ++ns) {
    const int n = n0 + ns * 32 + col;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int mm = m0 + out_row(i, half);
      if (mm < sl.M) {
        const float hv = silu(acc[0][ns][i]) * acc[1][ns][i];
        g.h[static_cast<size_t>(row_of(g, sl, mm)) * g.f + n] = f32_to_bf16(hv);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// down
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kWaves * kWave) void prefill_down(PrefillArgs g) {
  const int ti = blockIdx.y;
  if (ti >= __builtin_amdgcn_readfirstlane(g.n_tiles[0])) return;
  const int2 tile = g.tiles[ti];
  const int slot = __builtin_amdgcn_readfirstlane(tile.x);
  const int m0 = __builtin_amdgcn_readfirstlane(tile.y);
  const Slot sl = resolve_slot(g, slot);
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * kWgCols + wv * kWaveCols;  // first d-row of this wavefront
  if (n0 >= g.d) return;
  const int col = lane & 31, half = lane >> 5;
  const int m = m0 + col;
  const bool ok = m < sl.M;
  const uint16_t* arow = g.h + static_cast<size_t>(ok ? row_of(g, sl, m) : 0) * g.f;
  const size_t tq = static_cast<size_t>(n0 / 64) * 64 * (g.f / 2);
  const __amdgpu_buffer_rsrc_t rq[1] = {make_rsrc(sl.blk + g.q_down + tq, 32u * g.f)};
  const int groups = g.f / 64;
  const uint16_t* sd = reinterpret_cast<const uint16_t*>(sl.blk + g.s_down);
  const uint16_t* const srow[1][2] = {
      {sd + static_cast<size_t>(n0 + col) * groups, sd + static_cast<size_t>(n0 + 32 + col) * groups}};
  f32x16_t acc[1][2];
  gemm_tile<1>(arow, ok, groups, rq, srow, col, half, acc);
#pragma unroll
  for (int ns = 0; ns < 2; ++ns) {
    const int n = n0 + ns * 32 + col;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int mm = m0 + out_row(i, half);
      if (mm < sl.M) {
        uint16_t* out = sl.shared ? g.y_shared + static_cast<size_t>(mm) * g.d
                                  : g.y + static_cast<size_t>(sl.p0 + mm) * g.d;
        out[n] = f32_to_bf16(acc[0][ns][i]);
      }
    }
  }
}

// Upper bound of the M-tiles of a launch: every slot's rows rounded up.
int max_tiles(int T, int k, int slots, bool has_shared) {
  return (T * k + (has_shared ? T : 0)) / kBM + slots;
}

struct PrefillLayout {
  size_t h, tiles, n_tiles, total;
};

PrefillLayout prefill_layout(int T, int k, int E, int f, bool has_shared) {
  PrefillLayout l{};
  const int slots = (has_shared ? 1 : 0) + std::min(E, T * k);
  const size_t rows = static_cast<size_t>(T) * (k + (has_shared ? 1 : 0));
  l.h = 0;
  size_t off = (rows * f * 2 + 255) / 256 * 256;
  l.tiles = off;
  off += (static_cast<size_t>(max_tiles(T, k, slots, has_shared)) * sizeof(int2) + 255) / 256 * 256;
  l.n_tiles = off;
  off += 256;
  l.total = off;
  return l;
}

}  // namespace

size_t ffn_prefill_workspace(int T, int k, int E, int f, bool has_shared) {
  return prefill_layout(T, k, E, f, has_shared).total;
}

hipError_t launch_ffn_prefill(const FfnProblem& p, hipStream_t stream) {
  const size_t dd = p.d, ff = p.f;
  const PrefillLayout l = prefill_layout(p.T, p.k, p.E, p.f, p.has_shared);
  PrefillArgs g{};
  g.experts = p.experts;
  g.shared = p.shared;
  g.block_bytes = p.block_bytes;
  g.offsets = p.offsets;
  g.perm = p.perm;
  g.active = p.active;
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
  g.x = static_cast<const uint16_t*>(p.x);
  char* ws = static_cast<char*>(p.workspace);
  g.h = reinterpret_cast<uint16_t*>(ws + l.h);
  g.tiles = reinterpret_cast<int2*>(ws + l.tiles);
  g.n_tiles = reinterpret_cast<int*>(ws + l.n_tiles);
  g.y = static_cast<uint16_t*>(p.y);
  g.y_shared = static_cast<uint16_t*>(p.y_shared);
  const int mt = max_tiles(p.T, p.k, g.slots, p.has_shared);
  hipError_t err = launch(prefill_tiles, dim3(1), dim3(1024), 0, stream, g);
  if (err != hipSuccess) return err;
  err = launch(prefill_gateup, dim3((p.f + kWgCols - 1) / kWgCols, mt), dim3(kWaves * kWave), 0,
               stream, g);
  if (err != hipSuccess) return err;
  return launch(prefill_down, dim3((p.d + kWgCols - 1) / kWgCols, mt), dim3(kWaves * kWave), 0,
                stream, g);
}

}  // namespace moe
