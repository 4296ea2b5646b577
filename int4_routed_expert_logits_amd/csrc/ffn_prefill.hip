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
// chose it -- are cut into M-tiles: 128-row tiles while at least 96 rows are
// left, the rest in 32-row tiles.  A small kernel lists both kinds.
//  * 128-row tiles (the heavy experts of a Zipf-routed batch, the shared
//    expert): compute-bound.  A workgroup of 4 wavefronts fetches the
//    activations, codes, scales and row sums of one 64-column scale group
//    straight into LDS (three stages, one group fetched while another is
//    multiplied), and each wavefront computes 64 rows x 32 or 64 columns
//    (int4) or 64 or 128 columns (MXFP4, which has no per-group scale
//    multiply-adds and so the registers for twice the columns) with
//    v_mfma_f32_32x32x16_bf16.
//  * 32-row tiles (the many experts with a handful of tokens): they stream
//    the weights, one read per tile, near the read rate their access
//    pattern reaches, with the vector ALUs about half busy.  The activations of a group go through LDS, each
//    wavefront keeps 4 groups of its own codes in flight in registers and
//    multiplies both 16-row blocks with v_mfma_f32_16x16x32_bf16.
// The weights are read once per tile; the codes go from memory straight to
// MFMA operands (in registers, or through LDS where 4 wavefronts share
// them).
//
// Dequant into the MFMA: a 4-byte word of the packed codes holds 8
// consecutive input columns as offset-binary nibbles (q + 8), and
// ((w >> 4i) & 0x000F000F) | 0x43004300 is the bf16 pair (136 + q) of columns
// 2i, 2i+1 -- exact -- so one word is one 8-element B operand (seven VALU
// instructions).  Per 64-column scale group g the MFMAs accumulate
// P = sum_k x[m,k] (136 + q[k,n]) on top of a correction C = -136 S_g[m]
// (S_g the row's activation sum over the group), and the group scale is
// applied once: acc += s[n,g] * P.  C is the same for every column, so it
// is formed once per row block and group and shared by every column tile:
// in the 32-row tiles by the same MFMA with a B operand that is -136
// everywhere; in the 128-row tiles by one MFMA whose A operand holds the
// row's group sum, precomputed per row and split into three bf16 parts
// (prefill_rowsums), against -136 in the three matching B elements.
// The weights enter the products exactly (so do x * 136); only the float32
// accumulation and the bf16 rounding of H and Y round.  Activations are
// bf16 (an f32 x is rejected by the C ABI).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"

#pragma clang fp contract(off)

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBM = 32;        // rows per small M-tile
constexpr int kBigM = 128;     // rows per big M-tile
constexpr int kBigMinRows = 96;  // fewest rows a big tile is used for
constexpr uint32_t kMask = 0x000F000Fu;
constexpr uint32_t kMagic = 0x43004300u;
constexpr int kRsrcWord3 = 0x00020000;
// E8M0 exponents for which every E2M1 value times 2^(E - 127) is a normal
// bf16 (0.5 * 2^-125 .. 6 * 2^125), so the scale can be folded into the
// element conversion exactly; groups with other exponents take the
// unfolded form.
constexpr uint32_t kMxFoldLo = 2, kMxFoldHi = 252;

// True if any of the four E8M0 bytes of v lies outside kMxFoldLo .. kMxFoldHi.
__device__ __forceinline__ bool mx_wide(uint32_t v) {
  bool w = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) w |= ((v >> (8 * i)) & 0xFFu) - kMxFoldLo > kMxFoldHi - kMxFoldLo;
  return w;
}

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
  int2* tiles;         // (slot, first row) of every 32-row M-tile
  int* n_tiles;
  int2* big_tiles;     // (slot, first row) of every 128-row M-tile
  int* n_big;
  // Per row and 64-column group, the row's sum over the group split into
  // three bf16 parts (hi | mid << 16, lo): of the x tokens [T][d/64] and of
  // the h rows [T*k + T][f/64].  The 128-row tiles form the -136 * sum
  // correction from them with one MFMA.
  uint2* sum_x;
  uint2* sum_h;
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
// M-tile lists: one workgroup, slots in chunks of 1024.  A slot's rows go to
// 128-row tiles while at least 96 rows are left for the next one, the rest
// to 32-row tiles.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void big_small(int M, int& nb, int& ns) {
  nb = M / kBigM + ((M % kBigM) >= kBigMinRows ? 1 : 0);
  const int rem = max(0, M - nb * kBigM);
  ns = (rem + kBM - 1) / kBM;
}

__global__ __launch_bounds__(1024) void prefill_tiles(PrefillArgs g) {
  __shared__ int tot_b[16], tot_s[16];
  __shared__ int base_b, base_s;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) {
    base_b = 0;
    base_s = 0;
  }
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
    int nb, ns;
    big_small(M, nb, ns);
    int ib = nb, is = ns;  // inclusive scans over the workgroup
    for (int off = 1; off < 64; off <<= 1) {
      const int ob = __shfl_up(ib, off, 64), os = __shfl_up(is, off, 64);
      if (lane >= off) {
        ib += ob;
        is += os;
      }
    }
    if (lane == 63) {
      tot_b[wv] = ib;
      tot_s[wv] = is;
    }
    __syncthreads();
    int pb = base_b, ps = base_s, all_b = 0, all_s = 0;
    for (int w = 0; w < 16; ++w) {
      if (w < wv) {
        pb += tot_b[w];
        ps += tot_s[w];
      }
      all_b += tot_b[w];
      all_s += tot_s[w];
    }
    pb += ib - nb;
    ps += is - ns;
    for (int i = 0; i < nb; ++i) g.big_tiles[pb + i] = make_int2(slot, i * kBigM);
    for (int i = 0; i < ns; ++i) g.tiles[ps + i] = make_int2(slot, nb * kBigM + i * kBM);
    __syncthreads();
    if (tid == 0) {
      base_b += all_b;
      base_s += all_s;
    }
    __syncthreads();
  }
  if (tid == 0) {
    g.n_tiles[0] = base_s;
    g.n_big[0] = base_b;
  }
}

// ---------------------------------------------------------------------------
// Row sums per 64-column group: thread (row, group) adds the group's 64 bf16
// values in float32 in a fixed order (eight runs of eight, then the runs in
// order) and splits the sum s into bf16 parts hi + mid + lo (each the
// nearest bf16 of what the parts before leave), which carry s to about 24
// bits.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void prefill_rowsums(const uint16_t* src, int rows, int K,
                                                       uint2* dst) {
  const int groups = K / 64;
  const long long i = blockIdx.x * 256ll + threadIdx.x;
  if (i >= static_cast<long long>(rows) * groups) return;
  const long long r = i / groups;
  const int grp = static_cast<int>(i - r * groups);
  const uint4* p = reinterpret_cast<const uint4*>(src + r * K + grp * 64);
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint4 v = p[j];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float run = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      run += __uint_as_float(w[q] << 16);
      run += __uint_as_float(w[q] & 0xFFFF0000u);
    }
    sum += run;
  }
  const uint32_t hi = f32_to_bf16(sum);
  const float r1 = sum - bf16_to_f32(static_cast<uint16_t>(hi));
  const uint32_t mid = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(static_cast<uint16_t>(mid));
  const uint32_t lo = f32_to_bf16(r2);
  dst[i] = make_uint2(hi | (mid << 16), lo);
}

// ---------------------------------------------------------------------------
// shared GEMM core
// ---------------------------------------------------------------------------

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// The 8-element B operand of packed word w: bf16 pairs (136 + q).
__device__ __forceinline__ bf16x8_t dequant_word(uint32_t w) {
  const uint32_t mg = opaque_vgpr(kMagic);
  const uint4 b = make_uint4(and_or(w, kMask, mg), and_or(w >> 4, kMask, mg),
                             and_or(w >> 8, kMask, mg), and_or(w >> 12, kMask, mg));
  return as_bf16x8(b);
}

// MXFP4: the 8-element B operand of code word w (byte i holds elements 2i and
// 2i + 1, low nibble first), each E2M1 value times the block scale sv as bf16,
// one hardware conversion per pair.  Exact while every product is a normal
// bf16, i.e. for E8M0 exponents 2 .. 252 (callers pass sv = 1 and scale the
// products in float32 for groups with other exponents).
__device__ __forceinline__ bf16x8_t dequant_word_mx(uint32_t w, float sv) {
  const uint4 b = make_uint4(
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sv, 0)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sv, 1)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sv, 2)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sv, 3)));
  return as_bf16x8(b);
}


// B operand holding -136 in every element (bf16 0xC308).  With codes dequantised
// to 136 + q, the product with it gives the -136 * sum(A) that turns
// A * (136 + q) into A * q, for every column of the tile at once.
__device__ __forceinline__ bf16x8_t minus136() {
  return as_bf16x8(make_uint4(0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u));
}

// Buffer descriptor for `bytes` bytes at `base`.  The base is the same in
// every lane; reading it through readfirstlane keeps the descriptor in
// scalar registers even where the compiler cannot prove that.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b >> 32)));
  void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, static_cast<short>(0), static_cast<int>(bytes),
                                           kRsrcWord3);
}

// Output element i of a 32x32 MFMA tile held by lane (col, half) is row
// (i/4)*8 + half*4 + i%4, column col.
__device__ __forceinline__ int out_row(int i, int half) { return (i >> 2) * 8 + half * 4 + (i & 3); }

// ---------------------------------------------------------------------------
// 32-row tiles (small experts and the rows big tiles leave): they stream
// their weights at ~4.5-4.9 TB/s, near the read rate their access pattern
// reaches on the whole GPU, and on fewer CUs they are held by issue and
// latency (their time then grows almost in proportion).
// The workgroup stages the tile's activations for one
// 64-column group at a time in LDS (double-buffered, with each row's sum);
// every wavefront owns 16*NSUB columns of each of NM matrices, keeps kRing
// groups of its codes in flight in registers, and multiplies both 16-row
// blocks with v_mfma_f32_16x16x32_bf16, so each code is loaded and
// dequantized once per tile.
//
// K order inside a 64-column group: lane quarter kq (lane / 16) covers the
// 16 columns 16*kq .. 16*kq + 15, the first 8 in MFMA step 0 and the next 8
// in step 1 -- for the codes one 8-byte load (words 2*(kq%2), +1 of chunk
// kq/2), for the activations one 32-byte run.
// ---------------------------------------------------------------------------

// Work item of this workgroup on a 1-D grid.  Workgroup b runs on XCD
// b % 8 (workgroups are dealt to the 8 XCDs in turn), as the (b / 8)-th of
// that XCD.  The items -- (tile, column block), tile-major -- are cut into 8
// contiguous runs, one per XCD, so every column block of a tile and the
// neighbouring tiles of the same expert share one L2: the tile's
// activations and the expert's weights are fetched into it once.
constexpr int kXcds = 8;

__device__ __forceinline__ bool xcd_item(int ntiles, int ncols, int& tile, int& col) {
  const int items = ntiles * ncols, per = (items + kXcds - 1) / kXcds;
  const int b = blockIdx.x, j = b / kXcds, w = (b % kXcds) * per + j;
  if (j >= per || w >= items) return false;
  tile = w / ncols;
  col = w - tile * ncols;
  return true;
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kRing = 4;  // groups of codes in flight per wavefront
constexpr int kSmallRB = 2;  // 16-row blocks per small tile
constexpr int kALdS = 72;    // LDS row stride of the small tile's A (bf16)
constexpr int kSmallNSubGU = 4;  // 16-column subtiles per wavefront: gate/up (x2 matrices)
constexpr int kSmallNSubDN = 8;  //   and down

template <int NM, int NSUB>
struct SmallCodes {
  uint2 q[NM][NSUB];  // 2 words = 2 B fragments per subtile
};

template <int NM, int NSUB>
__device__ __forceinline__ void small_codes(int grp, int groups, int kq,
                                            const __amdgpu_buffer_rsrc_t (&rq)[NM], int rt0,
                                            SmallCodes<NM, NSUB>& st) {
  const int gg = min(grp, groups - 1);
#pragma unroll
  for (int mat = 0; mat < NM; ++mat) {
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) {
      const int rt = rt0 + sb * 16;  // row from the first packed tile of the wavefront
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(
          rq[mat], (rt >> 6) * 32 * (groups * 64) + (2 * gg + (kq >> 1)) * 1024 + (rt & 63) * 16 +
                       (kq & 1) * 8, 0, 0);
      st.q[mat][sb] = make_uint2(v[0], v[1]);
    }
  }
}

// Group scales of one ring pass (kRing groups) for all the workgroup's output
// rows, staged in LDS as [kRing][row] fp16.  The workgroup's 512 rows are 8
// packed 64-row tiles, whose scales are group-major: one group of one tile
// is a 128-byte run, so a pass is 8 x 4 such runs, one 16-byte piece per
// thread (tile t / 32, group (t / 8) % 4, rows 8 * (t % 8) ..).  Groups past
// the matrix repeat its last group (unused).
constexpr int kScaleRows = 512;  // output rows (all matrices) of one workgroup
static_assert(kRing == 4 && kScaleRows / 64 * kRing * 8 == 256, "one scale piece per thread");

// src: this thread's run at group 0 of its tile
__device__ __forceinline__ uint4 small_scale_load(const uint8_t* src, int pass, int groups) {
  const int j = min(pass * kRing + ((threadIdx.x >> 3) & 3), groups - 1);
  return *reinterpret_cast<const uint4*>(src + j * 128);
}

__device__ __forceinline__ void small_scale_store(uint16_t* sbuf, const uint4& v) {
  const int t = threadIdx.x;
  reinterpret_cast<uint4*>(sbuf + ((t >> 3) & 3) * kScaleRows + (t >> 5) * 64 + (t & 7) * 8)[0] = v;
}

// abuf: [32 rows][kALdS] bf16.
// sc: this lane's scale of subtile 0 of matrix 0 for this group in the LDS
// scale buffer (bytes).  int4: fp16 scales, one per row: subtile sb of matrix
// mat sits (mat * 64 * NSUB + sb * 16) rows further.  MX: per 64-row tile
// the E8M0 bytes of the group's first block of 32 (rows 0..63), then of its
// second, and the lane's pointer already selects the block of its 16 columns
// of K.
template <int NM, int NSUB, bool MX>
__device__ __forceinline__ void small_math(const uint32_t* abuf, const SmallCodes<NM, NSUB>& st,
                                           const uint8_t* sc, int col, int kq,
                                           f32x4_t (&acc)[kSmallRB][NM][NSUB]) {
  uint4 a[kSmallRB][2];
  f32x4_t corr[kSmallRB];
#pragma unroll
  for (int rb = 0; rb < kSmallRB; ++rb) {
    const int r = rb * 16 + col;
    const uint4* ap = reinterpret_cast<const uint4*>(abuf + (r * kALdS + kq * 16) / 2);
    a[rb][0] = ap[0];
    a[rb][1] = ap[1];
    if constexpr (MX) continue;
    // -136 * (row sums of the group), the same for every column
    corr[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[rb][0]), minus136(),
                                                       f32x4_t{}, 0, 0, 0);
    corr[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[rb][1]), minus136(), corr[rb],
                                                       0, 0, 0);
  }
  if constexpr (MX) {
    // power-of-two scales folded into the conversion (every scale byte of
    // the tile lies in 2 .. 252: prefill_small sends other tiles to
    // small_tile_wide): the products accumulate straight into acc
#pragma unroll
    for (int mat = 0; mat < NM; ++mat) {
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb) {
        const float sv = e8m0_to_f32(sc[2 * mat * 64 * NSUB + (sb >> 2) * 128 + (sb & 3) * 16]);
        const bf16x8_t b0 = dequant_word_mx(st.q[mat][sb].x, sv);
        const bf16x8_t b1 = dequant_word_mx(st.q[mat][sb].y, sv);
#pragma unroll
        for (int rb = 0; rb < kSmallRB; ++rb) {
          acc[rb][mat][sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[rb][0]), b0,
                                                                     acc[rb][mat][sb], 0, 0, 0);
          acc[rb][mat][sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[rb][1]), b1,
                                                                     acc[rb][mat][sb], 0, 0, 0);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int mat = 0; mat < NM; ++mat) {
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) {
      const bf16x8_t b0 = dequant_word(st.q[mat][sb].x), b1 = dequant_word(st.q[mat][sb].y);
      const float sv = static_cast<float>(__builtin_bit_cast(
          _Float16, reinterpret_cast<const uint16_t*>(sc)[mat * 64 * NSUB + sb * 16]));
#pragma unroll
      for (int rb = 0; rb < kSmallRB; ++rb) {
        f32x4_t p = corr[rb];
        p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[rb][0]), b0, p, 0, 0, 0);
        p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[rb][1]), b1, p, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[rb][mat][sb][e] = fmaf(sv, p[e], acc[rb][mat][sb][e]);
      }
    }
  }
}

// Staging of one group of the tile's A: thread t holds 8 columns of row
// t / 8.  The load
// is unconditional (rows past the slot read a valid row) and the value is
// masked only at the store, so the load is waited for where it is stored and
// not earlier, with the codes behind it still in flight.
__device__ __forceinline__ uint4 small_a_load(const uint16_t* arow, int grp) {
  return *reinterpret_cast<const uint4*>(arow + grp * 64 + (threadIdx.x & 7) * 8);
}

// keep: all ones for a row of the slot, zero for rows past it
__device__ __forceinline__ void small_a_store(uint32_t* abuf, const uint4& raw, uint32_t keep) {
  const uint4 v = make_uint4(raw.x & keep, raw.y & keep, raw.z & keep, raw.w & keep);
  const int t = threadIdx.x, r = t >> 3, c8 = t & 7;
  reinterpret_cast<uint4*>(abuf + (r * kALdS + c8 * 8) / 2)[0] = v;
}

constexpr int kSmallBufWords = 32 * kALdS / 2;

// MXFP4 32-row tiles with a scale byte outside 2 .. 252 (an E2M1 value
// times 2^(E - 127) that is not a normal bf16, or E = 255), a case real
// checkpoints do not produce: one group at a time, without the ring of
// codes in flight.  Each lane loads word kq of both 32-column chunks of the
// group, so MFMA step b covers block b alone; the elements convert unscaled
// (exact) and the block's scale multiplies the step's sum in float32, as on
// the decode path.  Entered before anything of the fast path is live, so its
// registers do not add to the fast path's.
// sbase[mat]: the matrix's E8M0 bytes; tile0 / ntiles: the wavefront's first
// packed 64-row tile and the matrix's tile count.
template <int NM, int NSUB>
__device__ __forceinline__ void small_tile_wide(uint32_t* abuf, const uint16_t* srcrow,
                                                uint32_t akeep, int groups, int kq, int col,
                                                const __amdgpu_buffer_rsrc_t (&rq)[NM], int rt0,
                                                const uint8_t* const (&sbase)[2], int tile0,
                                                int ntiles, bool active,
                                                f32x4_t (&acc)[kSmallRB][NM][NSUB]) {
  for (int grp = 0; grp < groups; ++grp) {
    const uint4 araw = small_a_load(srcrow, grp);
    uint2 q[NM][NSUB];
    float sv[NM][NSUB][2];
    if (active) {
#pragma unroll
      for (int mat = 0; mat < NM; ++mat) {
#pragma unroll
        for (int sb = 0; sb < NSUB; ++sb) {
          const int rt = rt0 + sb * 16;
          const int base = (rt >> 6) * 32 * (groups * 64) + (rt & 63) * 16 + kq * 4;
          q[mat][sb] = make_uint2(
              __builtin_amdgcn_raw_buffer_load_b32(rq[mat], base + (2 * grp) * 1024, 0, 0),
              __builtin_amdgcn_raw_buffer_load_b32(rq[mat], base + (2 * grp + 1) * 1024, 0, 0));
          const int tg = min(tile0 + (rt >> 6), ntiles - 1);
          const uint8_t* e = sbase[mat] + static_cast<size_t>(tg) * groups * 128 + 2 * grp * 64 +
                             (rt & 63);
          sv[mat][sb][0] = e8m0_to_f32(e[0]);
          sv[mat][sb][1] = e8m0_to_f32(e[64]);
        }
      }
    }
    __syncthreads();  // the previous group's A has been read
    small_a_store(abuf, araw, akeep);
    __syncthreads();
    if (!active) continue;
    uint4 a[kSmallRB][2];
#pragma unroll
    for (int rb = 0; rb < kSmallRB; ++rb) {
      const int r = rb * 16 + col;
      a[rb][0] = *reinterpret_cast<const uint4*>(abuf + (r * kALdS + kq * 8) / 2);
      a[rb][1] = *reinterpret_cast<const uint4*>(abuf + (r * kALdS + 32 + kq * 8) / 2);
    }
#pragma unroll
    for (int mat = 0; mat < NM; ++mat) {
#pragma unroll
      for (int sb = 0; sb < NSUB; ++sb) {
        const bf16x8_t w0 = dequant_word_mx(q[mat][sb].x, 1.0f);
        const bf16x8_t w1 = dequant_word_mx(q[mat][sb].y, 1.0f);
#pragma unroll
        for (int rb = 0; rb < kSmallRB; ++rb) {
          const f32x4_t p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[rb][0]), w0,
                                                                     f32x4_t{}, 0, 0, 0);
          const f32x4_t p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[rb][1]), w1,
                                                                     f32x4_t{}, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[rb][mat][sb][i] = fmaf(sv[mat][sb][0], p0[i], acc[rb][mat][sb][i]);
            acc[rb][mat][sb][i] = fmaf(sv[mat][sb][1], p1[i], acc[rb][mat][sb][i]);
          }
        }
      }
    }
  }
}

template <int NM, int NSUB, bool DOWN, bool MX>
__global__ __launch_bounds__(256) void prefill_small(PrefillArgs g) {
  constexpr int kWaveN = 16 * NSUB;
  __shared__ __align__(16) uint32_t abufs[2][kSmallBufWords];
  __shared__ __align__(16) uint16_t sbufs[2][kRing * kScaleRows];  // scales of a ring pass
  const int N = DOWN ? g.d : g.f, K = DOWN ? g.f : g.d;
  int ti, cblk;
  if (!xcd_item(__builtin_amdgcn_readfirstlane(g.n_tiles[0]), (N + 4 * kWaveN - 1) / (4 * kWaveN),
                ti, cblk))
    return;
  const int2 tile = g.tiles[ti];
  const int slot = __builtin_amdgcn_readfirstlane(tile.x);
  const int m0 = __builtin_amdgcn_readfirstlane(tile.y);
  const Slot sl = resolve_slot(g, slot);
  const int groups = K / 64;
  // A staging: thread t -> row t / 8 of the tile (rows past the slot read
  // the slot's first row and are zeroed)
  const int am = m0 + (threadIdx.x >> 3);
  const bool aok = am < sl.M;
  const uint32_t akeep = aok ? 0xFFFFFFFFu : 0u;
  const uint16_t* srcrow;
  {
    const int m = aok ? am : m0;
    if (DOWN) {
      srcrow = g.h + static_cast<size_t>(row_of(g, sl, m)) * g.f;
    } else {
      const int tok = sl.shared ? m : g.perm[sl.p0 + m] / g.top_k;
      srcrow = g.x + static_cast<size_t>(tok) * g.d;
    }
  }
  // the wavefront index is uniform: keep it (and the descriptors built from
  // it) in scalar registers
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n0 = (cblk * 4 + wv) * kWaveN;  // first output column of this wavefront
  const bool active = n0 < N;                     // (barriers below need every wavefront)
  const int col = lane & 15, kq = lane >> 4;
  const int nb = active ? n0 : 0;
  const size_t tq = static_cast<size_t>(nb / 64) * 32 * K;
  const size_t qoff[2] = {DOWN ? g.q_down : g.q_gate, g.q_up};
  const size_t soff[2] = {DOWN ? g.s_down : g.s_gate, g.s_up};
  // packed tiles of this wavefront inside the matrix (reads past them give 0)
  const int ntv = min((kWaveN + 63) / 64, (N - nb) / 64);
  __amdgpu_buffer_rsrc_t rq[NM];
#pragma unroll
  for (int mat = 0; mat < NM; ++mat) rq[mat] = make_rsrc(sl.blk + qoff[mat] + tq, 32u * K * ntv);
  const int rt0 = nb % 64 + col;  // this lane's row inside the packed tile (subtile 0)
  // this thread's scale piece: tile t / 32 of the workgroup's rows
  // (matrix-major, then column), rows 8 * (t % 8) .. of the tile
  constexpr int kWgN = 4 * kWaveN;
  static_assert(NM * kWgN == kScaleRows && kWgN % 64 == 0, "scale rows per workgroup");
  const uint8_t* ssrc;
  {
    const int ti8 = threadIdx.x >> 5, mat = ti8 * 64 / kWgN;
    const int pt = min((cblk * kWgN + ti8 * 64 % kWgN) / 64, N / 64 - 1);  // packed tile
    ssrc = sl.blk + (mat == 0 ? soff[0] : soff[NM - 1]) +
           (static_cast<size_t>(pt) * groups * 64 + (threadIdx.x & 7) * 8) * 2;
  }
  // this lane's scale (subtile 0 of matrix 0, first group of a pass) in scale
  // buffer 0; a group's slot is 2 * kScaleRows bytes.  MX: the 64-row tiles of
  // the slot are 128 bytes each, the block of K columns kq * 16.. is
  // kq / 2 of the group's two.
  const uint8_t* scl = reinterpret_cast<const uint8_t*>(sbufs) +
                       (MX ? 2 * wv * kWaveN + col + (kq >> 1) * 64 : 2 * (wv * kWaveN + col));

  f32x4_t acc[kSmallRB][NM][NSUB];
#pragma unroll
  for (int rb = 0; rb < kSmallRB; ++rb)
#pragma unroll
    for (int mat = 0; mat < NM; ++mat)
#pragma unroll
      for (int s = 0; s < NSUB; ++s) acc[rb][mat][s] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // MX: a tile with a scale byte outside 2 .. 252 takes small_tile_wide (this
  // thread checks the scale pieces it would stage in every pass)
  bool wide = false;
  if constexpr (MX) {
    for (int ps = 0; ps < (groups + kRing - 1) / kRing; ++ps) {
      const uint4 v = small_scale_load(ssrc, ps, groups);
      wide |= mx_wide(v.x) | mx_wide(v.y) | mx_wide(v.z) | mx_wide(v.w);
    }
    wide = __syncthreads_or(wide);
  }
  if (MX && wide) {
    const uint8_t* const sbase[2] = {sl.blk + soff[0], sl.blk + soff[NM - 1]};
    small_tile_wide<NM, NSUB>(abufs[0], srcrow, akeep, groups, kq, col, rq, rt0, sbase, nb / 64,
                              N / 64, active, acc);
  } else {
  // Loads are issued in the order they are consumed (scales of pass 0, A of
  // groups 0..2, codes of groups 0..kRing-1, scales of pass 1), and in the
  // loop A of group grp+3 goes out ahead of the codes of group grp+kRing.
  // Counters drain in order, so each wait then covers exactly the data it
  // needs and leaves the later codes in flight.
  const uint4 s0 = small_scale_load(ssrc, 0, groups);
  const uint4 a0 = small_a_load(srcrow, 0);
  uint4 areg[2];  // A of group j lives in areg[j & 1] until its store
  areg[1] = small_a_load(srcrow, min(1, groups - 1));
  areg[0] = small_a_load(srcrow, min(2, groups - 1));
  __builtin_amdgcn_sched_barrier(0);  // keep the issue order
  SmallCodes<NM, NSUB> ring[kRing];
#pragma unroll
  for (int i = 0; i < kRing; ++i) small_codes<NM, NSUB>(i, groups, kq, rq, rt0, ring[i]);
  __builtin_amdgcn_sched_barrier(0);
  uint4 snext = small_scale_load(ssrc, 1, groups);
  small_scale_store(sbufs[0], s0);
  small_a_store(abufs[0], a0, akeep);
  __syncthreads();
  // Full rings first: straight-line bodies, so the compiler can count the
  // loads in flight and wait for exactly the group it needs.
  const int full = groups / kRing * kRing;
  for (int g0 = 0; g0 < full; g0 += kRing) {
    const int pb = (g0 / kRing) & 1;  // scale buffer of this pass
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      const int grp = g0 + i;
      if (active)
        small_math<NM, NSUB, MX>(abufs[i & 1], ring[i], scl + (pb * kRing + i) * 2 * kScaleRows,
                                 col, kq, acc);
      small_a_store(abufs[(i + 1) & 1], areg[(i + 1) & 1], akeep);
      if (i == kRing - 1) small_scale_store(sbufs[pb ^ 1], snext);
      __syncthreads();
      areg[(i + 1) & 1] = small_a_load(srcrow, min(grp + 3, groups - 1));
      __builtin_amdgcn_sched_barrier(0);
      small_codes<NM, NSUB>(grp + kRing, groups, kq, rq, rt0, ring[i]);
      if (i == kRing - 1) snext = small_scale_load(ssrc, g0 / kRing + 2, groups);
    }
  }
  {
    const int pb = (full / kRing) & 1;
#pragma unroll
    for (int i = 0; i < kRing; ++i) {  // the last groups % kRing groups
      const int grp = full + i;
      if (grp < groups) {
        if (active)
          small_math<NM, NSUB, MX>(abufs[i & 1], ring[i],
                                   scl + (pb * kRing + i) * 2 * kScaleRows, col, kq, acc);
        small_a_store(abufs[(i + 1) & 1], areg[(i + 1) & 1], akeep);
        __syncthreads();
        areg[(i + 1) & 1] = small_a_load(srcrow, min(grp + 3, groups - 1));
      }
    }
  }
  }  // fast path
  if (!active) return;
  // lane (col, kq) holds rows 4*kq + e of each block, column col of every subtile
#pragma unroll
  for (int rb = 0; rb < kSmallRB; ++rb) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int mm = m0 + rb * 16 + 4 * kq + e;
      if (mm >= sl.M) continue;
      if constexpr (DOWN) {
        uint16_t* out = sl.shared ? g.y_shared + static_cast<size_t>(mm) * g.d
                                  : g.y + static_cast<size_t>(sl.p0 + mm) * g.d;
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
          if (n0 + s * 16 + col < N) out[n0 + s * 16 + col] = f32_to_bf16(acc[rb][0][s][e]);
      } else {
        uint16_t* hrow = g.h + static_cast<size_t>(row_of(g, sl, mm)) * g.f;
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
          hrow[n0 + s * 16 + col] = f32_to_bf16(silu(acc[rb][0][s][e]) * acc[rb][1][s][e]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 128-row tiles: a workgroup of 4 wavefronts, 2 along M x 2 along N, each
// computing 64 rows x 32 * NS columns of each of NM matrices with
// v_mfma_f32_32x32x16_bf16.  int4: NM * NS = 2 (64 columns of gate and up,
// or 128 of down, per workgroup); MXFP4: NM * NS = 4 (128, or 256).
// ---------------------------------------------------------------------------

template <int NM, int NS>
struct Big {
  static constexpr int kWaveCols = 32 * NS;
  static constexpr int kWgCols = 2 * kWaveCols;
  static constexpr int kTilesN = kWgCols / 64;            // packed 64-row tiles per matrix
  static constexpr int kPieces = NM * kTilesN;            // 128-byte scale pieces per group
  static constexpr int kRuns = kPieces / 2;               // 1 KB code runs per wavefront
  // one stage: A, the codes, the scales, the row sums
  static constexpr int kB = kPieces * 2048;
  static constexpr int kS = kPieces * 128;
  static constexpr int kBytes = kBigM * 128 + kB + kS + kBigM * 8;
  static_assert(kPieces == 2 || kPieces == 4, "two or four scale pieces (one or two code runs per wavefront)");
};

// B operand of the correction: -136 at k = 0, 1, 2 (the three sum parts),
// zero elsewhere.
__device__ __forceinline__ bf16x8_t minus136_x3() {
  return as_bf16x8(make_uint4(0xC308C308u, 0x0000C308u, 0u, 0u));
}

// The operands of a 64-column scale group go from
// memory straight into LDS (global_load_lds, 16 bytes per lane), three
// groups deep, with no staging registers and one barrier per group.
//  * A stage holds one group: A [128 rows][64 bf16] with the eight 16-byte
//    segments of row r stored in the order seg ^ ((r >> 1) & 7) (a 1 KB DMA
//    write is contiguous, so the layout is chosen by which segment each lane
//    fetches; the swizzle keeps the 32-row fragment reads of the MFMAs free
//    of bank conflicts without padding); the codes of the group
//    [(mat * 2 + half) * kWgCols + column] x 16 bytes, as packed (one or two
//    1 KB runs per wavefront); the scales of the group, 128 bytes per packed
//    64-row tile (a quarter per wavefront); the row sums of the group, 8
//    bytes per row.
//  * Group g + 2 is fetched while group g is multiplied, into the stage group
//    g - 1 used; the stages are three distinct LDS arrays and the loop is
//    unrolled by three, so each read names its stage and the compiler's own
//    waits do not cover the fetches of the other stages.
// The arithmetic: exact bf16 (136 + q)
// operands, the -136 * row-sum correction by one MFMA per row block, the
// fp16 scale per group in float32; MXFP4 blocks fold E8M0 into the
// conversion, or take the per-block float32 scaling (tiles with a scale
// byte outside 2 .. 252).
// ---------------------------------------------------------------------------

constexpr int kSt2A = kBigM * 128;                      // A, 16 KB

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Byte offset of A[row][8 * seg ..] in a stage.
__device__ __forceinline__ int a2_off(int row, int seg) {
  return row * 128 + ((seg ^ ((row >> 1) & 7)) << 4);
}

// s_waitcnt vmcnt(N) lgkmcnt(0), expcnt untouched (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// This lane's sources of group 0 (each advanced by the group index).
struct Big2Src {
  const uint8_t* a[4];  // A: its 16-byte segment of row 8 * (4 * wv + j) + lane / 8
  const uint8_t* b[2];  // codes: its 16 bytes of each of the wavefront's 1 KB runs
  const uint8_t* s;     // scales: its 16 bytes (lanes 0..3, or 0..7 with four pieces)
  const uint8_t* r;     // row sums: its 4 bytes
};

// DMA instructions per group and wavefront.
template <class C, bool MX>
constexpr int big2_dmas() { return 4 + C::kRuns + 1 + (MX ? 0 : 1); }

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_u8*)p));
}

// One LDS DMA instruction: every active lane's 16 (or 4) bytes at g go to LDS
// at m0 + 16 (or 4) * lane.  Written as asm rather than the builtin: the
// compiler's own wait bookkeeping cannot tell the three stages apart and
// would wait for every fetch in flight before each read of a stage; these
// fetches are waited for explicitly (wait_vm_lgkm0) instead.  The statement
// has no register outputs; the address register is read when it issues.
__device__ __forceinline__ void dma16(const uint8_t* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const uint8_t* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}

template <class C, bool MX>
__device__ __forceinline__ void big2_issue(const Big2Src& src, int grp, uint8_t* st, int wv,
                                           int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) dma16(src.a[j] + grp * 128, lds_addr(st + (wv * 4 + j) * 1024));
#pragma unroll
  for (int u = 0; u < C::kRuns; ++u)
    dma16(src.b[u] + grp * 2048, lds_addr(st + kSt2A + (wv * C::kRuns + u) * 1024));
  // each wavefront fetches a quarter of the scales (64 or 128 bytes)
  if (lane < C::kS / 64) dma16(src.s + grp * 128, lds_addr(st + kSt2A + C::kB + wv * C::kS / 4));
  if constexpr (!MX) dma4(src.r + grp * 8, lds_addr(st + kSt2A + C::kB + C::kS + wv * 256));
}

template <int NM, int NS, bool MX, bool WIDE>
__device__ __forceinline__ void big2_math(const uint8_t* st, int wm, int wn, int col, int half,
                                          f32x16_t (&acc)[2][NM][NS]) {
  using C = Big<NM, NS>;
  u32x4_t a[2][4];
  f32x16_t corr[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = wm * 64 + i * 32 + col;
#pragma unroll
    for (int j = 0; j < 4; ++j) a[i][j] = *reinterpret_cast<const u32x4_t*>(st + a2_off(r, half * 4 + j));
    if constexpr (MX) continue;
    // -136 * (row sums of the group): one MFMA per row block from the sum
    // parts of the lane's row (the lanes of the upper K half pass zeros)
    const u32x2_t rs = *reinterpret_cast<const u32x2_t*>(st + kSt2A + C::kB + C::kS + r * 8);
    const u32x4_t op = half ? u32x4_t{0u, 0u, 0u, 0u} : u32x4_t{rs.x, rs.y, 0u, 0u};
    corr[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, op),
                                                      minus136_x3(), f32x16_t{}, 0, 0, 0);
  }
  const uint8_t* bq = st + kSt2A;
  const uint8_t* sc = st + kSt2A + C::kB;
  auto bword = [&](int mat, int n) -> u32x4_t {
    return *reinterpret_cast<const u32x4_t*>(bq + ((mat * 2 + half) * C::kWgCols + n) * 16);
  };
  if constexpr (MX) {
    auto ebyte = [&](int mat, int n, int b) -> uint32_t {
      return sc[(mat * C::kTilesN + (n >> 6)) * 128 + b * 64 + (n & 63)];
    };
    if constexpr (!WIDE) {
#pragma unroll
      for (int mat = 0; mat < NM; ++mat) {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          const int n = wn * C::kWaveCols + ns * 32 + col;
          const u32x4_t q = bword(mat, n);
          const float sv = e8m0_to_f32(ebyte(mat, n, half));
          bf16x8_t bw[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) bw[j] = dequant_word_mx(q[j], sv);
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[i][mat][ns] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8_t, a[i][j]), bw[j], acc[i][mat][ns], 0, 0, 0);
        }
      }
      return;
    }
#pragma unroll
    for (int mat = 0; mat < NM; ++mat) {
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const int n = wn * C::kWaveCols + ns * 32 + col;
        const u32x4_t q = bword(mat, n);
#pragma unroll 1
        for (int b = 0; b < 2; ++b) {  // (a loop: one block's operands live at a time)
          const float sv = e8m0_to_f32(ebyte(mat, n, b));
          bf16x8_t bw[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) bw[j] = dequant_word_mx(half == b ? q[j] : 0u, 1.0f);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            f32x16_t pp = f32x16_t{};
#pragma unroll
            for (int j = 0; j < 4; ++j)
              pp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[i][j]),
                                                           bw[j], pp, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][mat][ns][e] = fmaf(sv, pp[e], acc[i][mat][ns][e]);
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int mat = 0; mat < NM; ++mat) {
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      const int n = wn * C::kWaveCols + ns * 32 + col;
      const u32x4_t q = bword(mat, n);
      const float sv = static_cast<float>(*reinterpret_cast<const _Float16*>(
          sc + (mat * C::kTilesN + (n >> 6)) * 128 + (n & 63) * 2));
      bf16x8_t bw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bw[j] = dequant_word(q[j]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        f32x16_t pp = corr[i];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[i][j]), bw[j],
                                                       pp, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][mat][ns][e] = fmaf(sv, pp[e], acc[i][mat][ns][e]);
      }
    }
  }
}

template <int NM, int NS, bool DOWN, bool MX>
__global__ __launch_bounds__(256) void prefill_big(PrefillArgs g) {
  using C = Big<NM, NS>;
  __shared__ __align__(16) uint8_t st0[C::kBytes];
  __shared__ __align__(16) uint8_t st1[C::kBytes];
  __shared__ __align__(16) uint8_t st2[C::kBytes];
  const int N = DOWN ? g.d : g.f, K = DOWN ? g.f : g.d;
  int ti, cblk;
  if (!xcd_item(__builtin_amdgcn_readfirstlane(g.n_big[0]), (N + C::kWgCols - 1) / C::kWgCols, ti,
                cblk))
    return;
  const int n0 = cblk * C::kWgCols;
  const int2 tile = g.big_tiles[ti];
  const int slot = __builtin_amdgcn_readfirstlane(tile.x);
  const int m0 = __builtin_amdgcn_readfirstlane(tile.y);
  const Slot sl = resolve_slot(g, slot);
  const int groups = K / 64;
  const int ntv = min(C::kTilesN, (N - n0) / 64);  // packed tiles inside the matrix
  const int t = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const size_t soff[2] = {DOWN ? g.s_down : g.s_gate, g.s_up};
  const size_t qoff[2] = {DOWN ? g.q_down : g.q_gate, g.q_up};
  // tile row m -> this row's activations and row sums (rows past the slot
  // read the slot's first row; their outputs are never stored)
  auto row_src = [&](int m, const uint8_t*& rp, const uint8_t*& sp) {
    const int mr = m < sl.M ? m : m0;
    if (DOWN) {
      const size_t hr = row_of(g, sl, mr);
      rp = reinterpret_cast<const uint8_t*>(g.h + hr * g.f);
      sp = reinterpret_cast<const uint8_t*>(g.sum_h + hr * groups);
    } else {
      const int tok = sl.shared ? mr : g.perm[sl.p0 + mr] / g.top_k;
      rp = reinterpret_cast<const uint8_t*>(g.x + static_cast<size_t>(tok) * g.d);
      sp = reinterpret_cast<const uint8_t*>(g.sum_x + static_cast<size_t>(tok) * groups);
    }
  };
  Big2Src src;
  {
    const uint8_t* sp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 8 * (wv * 4 + j) + (lane >> 3);
      const uint8_t* rp;
      row_src(m0 + r, rp, sp);
      src.a[j] = rp + ((lane & 7) ^ ((r >> 1) & 7)) * 16;
    }
    // codes: runs pc = wv * kRuns + u = (mat * 2 + half) * kTilesN + tt
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int pc = min(wv * C::kRuns + u, 4 * C::kRuns - 1);
      const int tt = min(pc % C::kTilesN, ntv - 1), hh = (pc / C::kTilesN) & 1,
                mat = pc / (2 * C::kTilesN);
      src.b[u] = sl.blk + qoff[mat] + static_cast<size_t>(n0 / 64 + tt) * 32 * K + hh * 1024 +
                 lane * 16;
    }
    // scales: quarter wv of the kPieces pieces (piece ps = mat * kTilesN + tt;
    // two quarters per piece with two pieces, one with four)
    const int ps = wv * C::kPieces / 4, smat = ps / C::kTilesN;
    const int spt = min(n0 / 64 + ps % C::kTilesN, N / 64 - 1);
    const int sq = C::kPieces == 2 ? (wv & 1) * 64 : 0;  // byte offset of the quarter in its piece
    src.s = sl.blk + soff[smat] + static_cast<size_t>(spt) * groups * 128 + sq +
            min(lane, C::kS / 64 - 1) * 16;
    // row sums: 4-byte part (wv * 64 + lane) & 1 of row (wv * 64 + lane) / 2
    const int d = wv * 64 + lane;
    const uint8_t* rp;
    row_src(m0 + (d >> 1), rp, sp);
    src.r = sp + (d & 1) * 4;
  }
  const int wm = wv & 1, wn = wv >> 1, col = lane & 31, half = lane >> 5;
  // MX: whether any scale byte of the tile leaves 2 .. 252 (this thread reads
  // its share of the tile's scale runs once)
  bool wide = false;
  if constexpr (MX) {
    const int run = groups * 128;  // bytes per piece
    for (int e = t * 16; e < C::kPieces * run; e += 256 * 16) {
      const int ps = e / run, smat = ps / C::kTilesN;
      const int spt = min(n0 / 64 + ps % C::kTilesN, N / 64 - 1);
      const uint4 v = *reinterpret_cast<const uint4*>(sl.blk + soff[smat] +
                                                      static_cast<size_t>(spt) * run + e % run);
      wide |= mx_wide(v.x) | mx_wide(v.y) | mx_wide(v.z) | mx_wide(v.w);
    }
    wide = __syncthreads_or(wide);
  }
  f32x16_t acc[2][NM][NS];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int mat = 0; mat < NM; ++mat)
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][mat][ns][e] = 0.0f;
  constexpr int kD = big2_dmas<C, MX>();
  auto main_loop = [&](auto wide_tag) {
    constexpr bool W = decltype(wide_tag)::value;
    big2_issue<C, MX>(src, 0, st0, wv, lane);
    big2_issue<C, MX>(src, min(1, groups - 1), st1, wv, lane);
    // step of group grp in stage `cur`: its fetches done (the next group's
    // may still run), every wavefront done with the previous group (whose
    // stage `nxt2` receives group grp + 2), then the math
    auto step = [&](int grp, uint8_t* cur, uint8_t* nxt2) {
      wait_vm_lgkm0<kD>();
      __builtin_amdgcn_s_barrier();
      big2_math<NM, NS, MX, W>(cur, wm, wn, col, half, acc);
      big2_issue<C, MX>(src, min(grp + 2, groups - 1), nxt2, wv, lane);
    };
    for (int g0 = 0; g0 < groups; g0 += 3) {
      step(g0, st0, st2);
      if (g0 + 1 < groups) step(g0 + 1, st1, st0);
      if (g0 + 2 < groups) step(g0 + 2, st2, st1);
    }
    wait_vm_lgkm0<0>();  // no fetch into LDS outlives the workgroup
  };
  if constexpr (MX) {
    if (wide)
      main_loop(std::true_type{});
    else
      main_loop(std::false_type{});
  } else {
    main_loop(std::false_type{});
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int mm = m0 + wm * 64 + i * 32 + out_row(e, half);
      if (mm >= sl.M) continue;
      if constexpr (DOWN) {
        uint16_t* out = sl.shared ? g.y_shared + static_cast<size_t>(mm) * g.d
                                  : g.y + static_cast<size_t>(sl.p0 + mm) * g.d;
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          const int n = n0 + wn * C::kWaveCols + ns * 32 + col;
          if (n < N) out[n] = f32_to_bf16(acc[i][0][ns][e]);
        }
      } else {
        uint16_t* hrow = g.h + static_cast<size_t>(row_of(g, sl, mm)) * g.f;
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          const int n = n0 + wn * C::kWaveCols + ns * 32 + col;
          if (n < N) hrow[n] = f32_to_bf16(silu(acc[i][0][ns][e]) * acc[i][1][ns][e]);
        }
      }
    }
  }
}

// Upper bounds of the M-tiles of a launch.  Every 128-row tile holds at
// least kBigMinRows rows; a slot leaves fewer than kBigMinRows rows to
// 16-row tiles, so at most six of them.
int rows_of(int T, int k, bool has_shared) { return T * k + (has_shared ? T : 0); }
int max_small(int T, int k, int slots, bool has_shared) {
  return std::min(rows_of(T, k, has_shared) / kBM + slots, (kBigMinRows + kBM - 1) / kBM * slots);
}
int max_big(int T, int k, bool has_shared) { return rows_of(T, k, has_shared) / kBigMinRows + 1; }

struct PrefillLayout {
  size_t h, tiles, big_tiles, counts, sum_x, sum_h, total;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

PrefillLayout prefill_layout(int T, int k, int E, int d, int f, bool has_shared) {
  PrefillLayout l{};
  const int slots = (has_shared ? 1 : 0) + std::min(E, T * k);
  const size_t rows = rows_of(T, k, has_shared);
  l.h = 0;
  size_t off = align256(rows * f * 2);
  l.tiles = off;
  off += align256(static_cast<size_t>(max_small(T, k, slots, has_shared)) * sizeof(int2));
  l.big_tiles = off;
  off += align256(static_cast<size_t>(max_big(T, k, has_shared)) * sizeof(int2));
  l.counts = off;
  off += 256;
  l.sum_x = off;
  off += align256(static_cast<size_t>(T) * (d / 64) * sizeof(uint2));
  l.sum_h = off;
  off += align256(rows * (f / 64) * sizeof(uint2));
  l.total = off;
  return l;
}

}  // namespace

namespace {

// The launches of one prefill FFN.  int4 blocks: the row-sum pass over x
// before gate/up and over h before down (the offset correction); MXFP4 blocks
// have no offset and skip both.
template <bool MX>
hipError_t prefill_kernels(const FfnProblem& p, const PrefillArgs& g, hipStream_t stream) {
  const int ms = max_small(p.T, p.k, g.slots, p.has_shared);
  const int mb = max_big(p.T, p.k, p.has_shared);
  // int4: gate/up 64 columns of both matrices per workgroup, down 128
  // (three LDS stages of 21.3 KB each; two workgroups per CU).  MXFP4 blocks,
  // with no scale multiply-adds, fit twice the columns in two waves per SIMD:
  // 128 and 256 (stages of 25.5 KB).
  using GU = Big<2, MX ? 2 : 1>;
  using DN = Big<1, MX ? 4 : 2>;
  hipError_t err;
  if ((err = launch(prefill_tiles, dim3(1), dim3(1024), 0, stream, g)) != hipSuccess) return err;
  // 1-D grids: enough workgroups for the largest possible tile lists, in
  // whole rounds of the XCDs
  auto grid = [](int tiles, int cols) {
    return dim3((static_cast<unsigned>(tiles) * cols + kXcds - 1) / kXcds * kXcds);
  };
  const int cgu = (p.f + GU::kWgCols - 1) / GU::kWgCols, cdn = (p.d + DN::kWgCols - 1) / DN::kWgCols;
  const int sgu = (p.f + 64 * kSmallNSubGU - 1) / (64 * kSmallNSubGU);
  const int sdn = (p.d + 64 * kSmallNSubDN - 1) / (64 * kSmallNSubDN);
  auto rowsums = [&](const uint16_t* src, int rows, int K, uint2* dst) {
    const long long n = static_cast<long long>(rows) * (K / 64);
    return launch(prefill_rowsums, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                  stream, src, rows, K, dst);
  };
  if (!MX && (err = rowsums(g.x, p.T, p.d, g.sum_x)) != hipSuccess) return err;
  err = launch(prefill_big<2, GU::kWaveCols / 32, false, MX>, grid(mb, cgu), dim3(256), 0, stream, g);
  if (err != hipSuccess) return err;
  err = launch(prefill_small<2, kSmallNSubGU, false, MX>, grid(ms, sgu), dim3(256), 0, stream, g);
  if (err != hipSuccess) return err;
  if (!MX && (err = rowsums(g.h, rows_of(p.T, p.k, p.has_shared), p.f, g.sum_h)) != hipSuccess)
    return err;
  err = launch(prefill_big<1, DN::kWaveCols / 32, true, MX>, grid(mb, cdn), dim3(256), 0, stream, g);
  if (err != hipSuccess) return err;
  return launch(prefill_small<1, kSmallNSubDN, true, MX>, grid(ms, sdn), dim3(256), 0, stream, g);
}

}  // namespace

size_t ffn_prefill_workspace(int T, int k, int E, int d, int f, bool has_shared) {
  return prefill_layout(T, k, E, d, f, has_shared).total;
}

hipError_t launch_ffn_prefill(const FfnProblem& p, hipStream_t stream) {
  const size_t dd = p.d, ff = p.f;
  const PrefillLayout l = prefill_layout(p.T, p.k, p.E, p.d, p.f, p.has_shared);
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
  g.s_up = g.s_gate + ff * (dd / 64) * 2;  // (MXFP4: ff * (dd / 32) bytes, the same)
  g.s_down = g.s_up + ff * (dd / 64) * 2;
  g.x = static_cast<const uint16_t*>(p.x);
  char* ws = static_cast<char*>(p.workspace);
  g.h = reinterpret_cast<uint16_t*>(ws + l.h);
  g.tiles = reinterpret_cast<int2*>(ws + l.tiles);
  g.big_tiles = reinterpret_cast<int2*>(ws + l.big_tiles);
  g.n_tiles = reinterpret_cast<int*>(ws + l.counts);
  g.n_big = g.n_tiles + 1;
  g.sum_x = reinterpret_cast<uint2*>(ws + l.sum_x);
  g.sum_h = reinterpret_cast<uint2*>(ws + l.sum_h);
  g.y = static_cast<uint16_t*>(p.y);
  g.y_shared = static_cast<uint16_t*>(p.y_shared);
  return p.mxfp4 ? prefill_kernels<true>(p, g, stream) : prefill_kernels<false>(p, g, stream);
}

}  // namespace moe
