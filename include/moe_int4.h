/*
 * moe_int4.h -- C ABI of one MoE layer's routed-expert FFN over int4
 * group-quantised weights, on one AMD Instinct MI355X (gfx950).
 *
 * The layer (pages: zhichai.net, "744亿参数塞进25GB内存：colibrì如何用1300行C代码把
 * 不可能变成可能", section on MoE sparsity; yunpan.plus article on Colibrì,
 * sections "capability 2" and "capability 3"):
 *
 *   moe_route       router logits, top-k of E experts per token, softmax
 *                   renormalised over the chosen k
 *   moe_union       batch-union: group the T*k routing slots by expert so an
 *                   expert's weights are read once for all tokens routed to it
 *                   (the unit a cluster worker receives: one layer's routed
 *                   batch-union)
 *   moe_expert_ffn  int4 gs64 dequant fused into a SwiGLU expert for every
 *                   expert in the union, plus the always-active shared expert
 *   moe_combine     gate-weighted sum of each token's k expert outputs plus
 *                   the shared expert's output
 *   moe_route_union moe_route and moe_union in one call (one launch fewer
 *                   for decode batches)
 *   moe_layer_decode the whole layer (route, union, expert FFN, combine) for
 *                   a decode batch of at most 8 tokens in one call
 *   moe_cache_*     a per-layer cache of experts in HBM (LRU, pinned experts)
 *                   whose misses stream from pinned host memory while the
 *                   resident experts compute
 *   moe_quantize    float weights -> int4 codes + float16 scales (the
 *                   one-time conversion of a checkpoint)
 *   moe_pack_experts one-time byte bijection of the expert blocks into the
 *                   tiled layout the FFN kernels stream
 *
 * Conventions common to every call:
 *  - Every pointer argument except `shape` is a DEVICE pointer owned by the
 *    caller.  The library allocates nothing, keeps no state between calls,
 *    and never synchronises the host.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    legacy default stream).  Data-dependent sizes (counts, n_active) stay on
 *    the device: later calls read them there.
 *  - Arguments are checked before anything is enqueued.  On any error the call
 *    returns a non-zero status, enqueues nothing and leaves every output
 *    untouched.  There is never a silent fallback to another precision or
 *    algorithm (the pages' rule that precision and router semantics never
 *    change silently: yunpan.plus article, "capability 4").
 *  - A kernel launch failure returns MOE_ERR_HIP; faults during execution
 *    surface at the caller's next synchronisation of `stream`.
 *  - Calls are thread-safe.  Calls that share a workspace buffer must be
 *    ordered (same stream, or synchronised); moe_expert_ffn's workspace is
 *    reserved for moe_expert_ffn (see there).
 *  - T == 0 (an empty batch) is valid: moe_union writes empty grouping
 *    outputs; the other calls enqueue nothing and return MOE_OK.
 */
#ifndef MOE_INT4_H
#define MOE_INT4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL                      */
  MOE_ERR_SHAPE = 2,       /* a size is out of range or sizes disagree        */
  MOE_ERR_DTYPE = 3,       /* dtype not allowed for this call or path         */
  MOE_ERR_ALIGN = 4,       /* a pointer is not aligned as documented          */
  MOE_ERR_UNSUPPORTED = 5, /* well-formed but not provided (e.g. group 16)    */
  MOE_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required      */
  MOE_ERR_HIP = 7,         /* a HIP launch failed                             */
  /* The *_INT_MIN_ / *_INT_MAX_ members of this and the enums below are not
   * values to pass or expect: they give each type the range of a 32-bit int,
   * so that the (C++) implementation may hold whatever int a C caller passes
   * and reject it with a status instead of having undefined behaviour. */
  MOE_STATUS_INT_MIN_ = -2147483647 - 1,
  MOE_STATUS_INT_MAX_ = 2147483647
} moe_status;

typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_DTYPE_INT_MIN_ = -2147483647 - 1,
  MOE_DTYPE_INT_MAX_ = 2147483647
} moe_dtype;

/* Which expert-FFN kernel family runs (moe_expert_ffn):
 *  DECODE_F32    HBM-bound int4 GEMV for small batches; activations bf16 or
 *                f32; h, y and y_shared are float32 (fp32 accumulation).
 *  PREFILL_BF16  grouped GEMM on bf16 MFMA for large batches; activations
 *                must be bf16; h, y and y_shared are bfloat16 (fp32
 *                accumulation).  An f32 x is rejected, never rounded. */
typedef enum {
  MOE_PATH_DECODE_F32 = 0,
  MOE_PATH_PREFILL_BF16 = 1,
  MOE_PATH_INT_MIN_ = -2147483647 - 1,
  MOE_PATH_INT_MAX_ = 2147483647
} moe_path;

/* Scale granularity of moe_quantize: one float16 scale per 64 consecutive
 * input columns of a row (the layout every other call reads), or one per row
 * (for comparison only). */
typedef enum {
  MOE_QUANT_GS64 = 0,
  MOE_QUANT_ROW = 1,
  MOE_QUANT_INT_MIN_ = -2147483647 - 1,
  MOE_QUANT_INT_MAX_ = 2147483647
} moe_quant_mode;

/* Layer geometry.
 *  d          hidden size; multiple of 64, 64..8192
 *  f          routed-expert intermediate size; multiple of 64, 64..8192
 *  n_experts  routed experts E, 1..1024
 *  top_k      experts per token k, 1..min(E, 32)
 *             (every call taking T tokens: T >= 0 (MOE_ERR_SHAPE) and
 *             T * top_k <= 2^24 (MOE_ERR_UNSUPPORTED))
 *  group      the expert block format, named by its quantisation group along
 *             the input dimension:
 *               64  int4 codes with a float16 scale per 64 elements (gs64,
 *                   the grouping the pages recommend over per-row scales:
 *                   yunpan.plus article, "capability 4"; ssnai.com digest,
 *                   prerequisites);
 *               32  MXFP4 (OCP Microscaling v1.0): FP4 E2M1 codes with an
 *                   E8M0 scale per 32 elements (the format the pages' Kimi K3
 *                   engine streams its experts in: ssnai.com digest,
 *                   prerequisites).  Taken by moe_expert_bytes,
 *                   moe_pack_experts, moe_ffn_workspace_bytes and
 *                   moe_expert_ffn on both paths, and by the calls that
 *                   do not read expert blocks (moe_route, moe_union,
 *                   moe_route_union, moe_combine and the route workspace
 *                   size); moe_layer_decode and the expert cache return
 *                   MOE_ERR_UNSUPPORTED for it.
 *             Anything else is MOE_ERR_UNSUPPORTED.
 *  f_shared   0 = no shared expert; otherwise the shared expert's
 *             intermediate size, which must equal f (same block layout) */
typedef struct {
  int32_t d;
  int32_t f;
  int32_t n_experts;
  int32_t top_k;
  int32_t group;
  int32_t f_shared;
} moe_shape;

/* Bytes of one expert block; 0 if d, f or group is not valid.  An expert
 * is one contiguous block (the pages keep and evict each ~19 MB int4 expert
 * as one piece: zhichai.net, section on why mmap falls short), laid out as
 *
 *   q_gate[f][d/2] | q_up[f][d/2] | q_down[d][f/2] |
 *   s_gate[f][d/64] | s_up[f][d/64] | s_down[d][f/64]
 *
 * q_*: int4 codes, row-major [out][in], element 2j of a row in the low
 *      nibble of byte j, each nibble a two's-complement value in [-8, 7];
 * s_*: IEEE float16 scales, one per 64 consecutive input elements of a row;
 * weight[r][c] = q[r][c] * s[r][c/64].
 * Gate and up are [f][d] (input d), down is [d][f] (input f).
 * Equals 3*d*f/2 + 3*d*f/group*2; 20,054,016 bytes at d=6144, f=2048.
 *
 * MXFP4 blocks (group 32) have the same size and order, with
 *   s_gate[f][d/32] | s_up[f][d/32] | s_down[d][f/32]
 * as E8M0 bytes E (scale 2^(E-127), E = 255 NaN), and each nibble an FP4
 * E2M1 code (sign, two exponent bits with bias 1, one mantissa bit:
 * +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}); weight[r][c] = e2m1(q[r][c]) * 2^(E[r][c/32]-127). */
size_t moe_expert_bytes(int32_t d, int32_t f, int32_t group);

/* Convert expert blocks from the layout above to the packed layout that
 * moe_expert_ffn reads: a bijection of each block's bytes (a permutation of
 * the nibbles and scales, and every code stored as q + 8), same size, done
 * once when the experts are loaded (as the pages' engine converts its
 * checkpoint once before serving: ssnai.com digest, first-command section).
 * For each matrix W [N][K] of the block (N, K multiples of 64) the codes are
 * regrouped into tiles of 64 rows: row t*64+l, columns 32c..32c+31 go to
 *     q_off + t*(64*K/2) + c*1024 + l*16
 * and inside each 4-byte word (columns 8w..8w+7) the nibble of column 8w+j
 * moves to bit 4*(j/2) + 16*(j%2), stored in offset binary (the
 * two's-complement code q with its top bit flipped: q + 8 in [0, 15]), where
 * q_off is the sub-array offset of the canonical block.  Scales follow the same tiles, group-major inside a
 * tile: the scale of row t*64+l, group g goes to
 *     s_off + (t*(K/64)*64 + g*64 + l)*2
 * where s_off is the scale sub-array offset of the canonical block.
 * MXFP4 blocks (group 32) go to the same 64-row tiles with their nibbles
 * unchanged (no reordering, no offset), and their E8M0 bytes block-major
 * inside a tile: row t*64+l, block b at s_off + t*(K/32)*64 + b*64 + l.
 *  n_blocks  number of consecutive blocks in src (0 is a no-op)
 *  src       canonical blocks, 16-byte aligned
 *  dst       packed blocks, 16-byte aligned, must not overlap src */
moe_status moe_pack_experts(const moe_shape* shape, int64_t n_blocks, const uint8_t* src,
                            uint8_t* dst, void* stream);

/* int4 quantiser: float weights W [N][K] -> codes and float16 scales, the
 * one-time conversion of a checkpoint (pages: ssnai.com digest, first-command
 * section -- the engine converts the weights once; yunpan.plus article,
 * "capability 4" -- int4 experts with gs64 scales, compared with one scale per
 * row).  The rule is not on the pages; this library's reading:
 *   s = float16(float32(absmax) / 7)   absmax over the 64-column group
 *                                      (GS64) or over the row (ROW), both
 *                                      roundings to nearest even
 *   q = the integer nearest to w / s, ties to even, in [-8, 7]; s == 0 gives
 *       q = 0 (a group of zeros)
 * Every code is decided exactly (no rounding of w / s can move it).
 *  N, K      rows and columns; K a positive multiple of 64, K <= 65536
 *  w         [N][K] bf16 or f32 (w_dt), row-major, 16-byte aligned
 *  codes     out [N][K/2] bytes, element 2j of a row in the low nibble of
 *            byte j (the canonical expert-block layout), 4-byte aligned
 *  scales    out float16: [N][K/64] (GS64) or [N] (ROW), 2-byte aligned
 * To build a canonical expert block, call it for W_gate, W_up and W_down with
 * the block's sub-array pointers (moe_expert_bytes gives the layout).
 * N == 0 is a no-op.  Non-finite weights give unspecified codes. */
moe_status moe_quantize(int32_t N, int32_t K, const void* w, moe_dtype w_dt, moe_quant_mode mode,
                        uint8_t* codes, void* scales, void* stream);

/* Scratch bytes moe_route needs for T tokens (router logits, float64); 0 for
 * a shape the call rejects, T < 0 or T * top_k > 2^24. */
size_t moe_route_workspace_bytes(const moe_shape* shape, int32_t T);

/* Router: for every token t,
 *   l[t][e] = sum_i x[t][i] * w_router[e][i] + bias[e]     (float64)
 *   S_t     = the top_k experts with the largest l[t][e]; equal logits are
 *             ordered by lower expert id; S_t is written in descending logit
 *             order
 *   w[t][j] = exp(l_j - l_0) / sum_{j'} exp(l_j' - l_0) over S_t
 * (pages: zhichai.net, MoE sparsity section -- the router picks 8 of 256
 * experts per token; the gating function, precision and tie rule are not on
 * the pages: softmax renormalised over the chosen k, float64 logits so the
 * selection does not depend on summation order, lower id first on ties).
 *  x         [T][d], bf16 or f32 (x_dt), row-major, 16-byte aligned
 *  w_router  [E][d] float32, row-major, 16-byte aligned
 *  bias      [E] float32, or NULL for none; added before both selection and
 *            weighting
 *  topk_idx  out [T][top_k] int32 expert ids
 *  topk_w    out [T][top_k] float32 gate weights (sum to 1 per token)
 *  workspace >= moe_route_workspace_bytes(shape, T) bytes, 256-byte aligned
 * Non-finite logits give unspecified (but in-range) results. */
moe_status moe_route(const moe_shape* shape, int32_t T, const void* x, moe_dtype x_dt,
                     const float* w_router, const float* bias, int32_t* topk_idx,
                     float* topk_w, void* workspace, size_t workspace_bytes, void* stream);

/* Batch-union grouping of the T*top_k routing slots (slot id s = t*top_k + j
 * routes token t to expert topk_idx[t][j]); pages: yunpan.plus article,
 * "capability 2" (an expert needed by several positions of a batch is read
 * once) and "capability 3" (a worker runs the FFN on one layer's routed
 * batch-union).
 *  counts    out [E]    slots routed to each expert
 *  offsets   out [E+1]  exclusive prefix sum of counts (offsets[E] = slots)
 *  perm      out [T*k]  slot id at each grouped position, ordered by expert
 *                       ascending, then slot id ascending
 *  inv_perm  out [T*k]  grouped position of each slot
 *  active    out [E]    experts with counts > 0 ascending, then -1 padding
 *  n_active  out [1]    number of such experts
 * The result is deterministic (no dependence on atomic ordering).  An entry
 * of topk_idx outside [0, E) is not grouped: it gets inv_perm = -1, is not
 * counted, and moe_combine treats it as a zero contribution. */
moe_status moe_union(const moe_shape* shape, int32_t T, const int32_t* topk_idx,
                     int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                     int32_t* active, int32_t* n_active, void* stream);

/* moe_route followed by moe_union, in one call: the same outputs, bit for
 * bit, as the two calls in sequence (arguments as there; the workspace is
 * moe_route's).  Batches with T <= 8 and T*top_k <= 64 (and E <= 256) run
 * the top-k and the grouping in a single kernel, one launch fewer per
 * decode step; larger batches run exactly the two calls' kernels.
 * T == 0 writes the empty grouping, as moe_union does. */
moe_status moe_route_union(const moe_shape* shape, int32_t T, const void* x, moe_dtype x_dt,
                           const float* w_router, const float* bias, int32_t* topk_idx,
                           float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                           int32_t* inv_perm, int32_t* active, int32_t* n_active,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Scratch bytes moe_expert_ffn needs for T tokens on `path`; 0 for a shape
 * or path the call rejects, T < 0 or T * top_k > 2^24. */
size_t moe_ffn_workspace_bytes(const moe_shape* shape, int32_t T, moe_path path);

/* Expert FFN over the batch-union: for every active expert e and each of its
 * grouped positions p in [offsets[e], offsets[e+1]), with token
 * t = perm[p] / top_k,
 *   y[p] = W_down_e ( silu(W_gate_e x[t]) * (W_up_e x[t]) ),  silu(z) = z/(1+e^-z)
 * with every weight dequantised from int4 as q * s (group 64 along the input
 * dimension; MXFP4 blocks: E2M1 value times 2^(E - 127) per 32 elements, for
 * every E8M0 byte: products of activations and E2M1 values are exact, and
 * each block's scale multiplies its partial sum in float32 -- or, on
 * PREFILL for tiles whose scale bytes all lie in 2 .. 252, is folded exactly
 * into the bf16 weight operand; E = 255 makes the block's weights NaN); and
 * for the
 * shared expert (if shape->f_shared) and every token,
 *   y_shared[t] = the same SwiGLU with the shared block
 * (pages: zhichai.net, MoE sparsity and three-tier sections -- 8 routed + 1
 * shared expert active per layer, int4 experts; the SwiGLU form is not on
 * the pages and is this library's reading).
 *  x         [T][d]; DECODE: bf16 or f32; PREFILL: bf16 only
 *  experts   E blocks of moe_expert_bytes(d, f, group) bytes, back to back,
 *            in the packed layout (moe_pack_experts), 16-byte aligned
 *  shared    one packed block, or NULL iff shape->f_shared == 0
 *  offsets, perm, active, n_active: moe_union's outputs for this batch
 *  y         out [T*top_k][d], grouped order; float32 (DECODE) or bf16
 *            (PREFILL); rows of unused positions are not written
 *  y_shared  out [T][d] same dtype, or NULL iff no shared expert
 *  workspace >= moe_ffn_workspace_bytes(shape, T, path), 256-byte aligned,
 *            no initial contents required: it carries the intermediate h
 *            from the gate/up kernel to the down kernel.  Never share one
 *            workspace between two calls that may run at the same time. */
moe_status moe_expert_ffn(const moe_shape* shape, int32_t T, const void* x, moe_dtype x_dt,
                          const uint8_t* experts, const uint8_t* shared,
                          const int32_t* offsets, const int32_t* perm, const int32_t* active,
                          const int32_t* n_active, moe_path path, void* y, void* y_shared,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Gate-weighted combine:
 *   out[t] = sum_{j < top_k} topk_w[t][j] * y[inv_perm[t*top_k + j]] + y_shared[t]
 * summed in j order in float32, no atomics (pages: zhichai.net, MoE
 * sparsity section -- 8 routed experts plus the "+1" shared expert; weights
 * on the shared expert are not on the pages: it is added with weight 1).
 *  y         [T*top_k][d] (y_dt), grouped order, from moe_expert_ffn
 *  y_shared  [T][d] (y_dt) or NULL for none
 *  inv_perm  [T*top_k] from moe_union
 *  topk_w    [T][top_k] from moe_route
 *  out       out [T][d], out_dt (f32 or bf16, round to nearest even)
 * y, y_shared and out must be 16-byte aligned. */
moe_status moe_combine(const moe_shape* shape, int32_t T, const void* y, const void* y_shared,
                       moe_dtype y_dt, const int32_t* inv_perm, const float* topk_w, void* out,
                       moe_dtype out_dt, void* stream);

/* Scratch bytes moe_layer_decode needs for T tokens; 0 for a shape the call
 * rejects, T < 0 or T * top_k > 2^24. */
size_t moe_layer_decode_workspace_bytes(const moe_shape* shape, int32_t T);

/* The whole layer for a small decode batch -- moe_route_union, then
 * moe_expert_ffn on the DECODE path, then moe_combine -- in one call with
 * the same outputs, bit for bit, as those three calls in sequence (pages:
 * zhichai.net, section on MTP speculative decoding -- the main model checks
 * 2-3 drafted tokens per forward pass, and draft and check must compute the
 * same function).  For one token the gate/up kernel derives the top-k and
 * the grouping itself from the router's float64 partial sums, so the step is
 * four launches (router logits, gate/up, down, combine) instead of five;
 * from two tokens on, where each gate/up workgroup redoing the top-k of the
 * whole batch costs more than the launch it saves, the call runs the
 * separate calls' kernels (route + union, gate/up, down, combine).
 *  arguments as in the three calls; every output of theirs is written:
 *  topk_idx, topk_w, counts, offsets, perm, inv_perm, active, n_active, y and
 *  y_shared (float32), and out (out_dt).
 *  workspace >= moe_layer_decode_workspace_bytes(shape, T), 256-byte
 *            aligned, no initial contents required; never shared between
 *            calls that may run at the same time.
 * Supported: 1 <= T <= 8, T*top_k <= 64, n_experts <= 256 (anything else is
 * MOE_ERR_UNSUPPORTED; larger batches use the separate calls).  T == 0 writes
 * the empty grouping, as moe_route_union does. */
moe_status moe_layer_decode(const moe_shape* shape, int32_t T, const void* x, moe_dtype x_dt,
                            const float* w_router, const float* bias, const uint8_t* experts,
                            const uint8_t* shared, int32_t* topk_idx, float* topk_w,
                            int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                            int32_t* active, int32_t* n_active, void* y, void* y_shared,
                            void* out, moe_dtype out_dt, void* workspace, size_t workspace_bytes,
                            void* stream);

/* ------------------------------------------------------------------------
 * Per-layer expert cache (pages: zhichai.net, section on why mmap falls
 * short -- every layer keeps an LRU cache of whole experts, and pinned hot
 * experts take no part in eviction; yunpan.plus article, "capability 1" --
 * per-layer LRU plus a pinned hot-store, and "capability 2" -- missing
 * experts load asynchronously while the resident ones compute).
 *
 * A cache holds n_slots expert blocks in HBM for one layer whose E blocks
 * live in pinned host memory.  Policy (host side, deterministic): a step's
 * distinct experts that a slot holds are hits; the missing ones, in
 * ascending id order, take the lowest empty slot, else the slot whose expert
 * was used least recently (ties: the lower slot), never a pinned expert's
 * slot or one used by the same step.  The cache object lives in host memory
 * (allocated by moe_cache_create, freed by moe_cache_destroy); its first
 * decode step also allocates a small pinned staging buffer and an event.
 * Unlike the calls above, a cache keeps state: the calls on one cache must
 * not overlap.
 * ------------------------------------------------------------------------ */
typedef struct moe_expert_cache moe_expert_cache;

/* n_slots in [top_k, E].  device_slots: n_slots * moe_expert_bytes() bytes
 * of device memory, 256-byte aligned; host_blocks: the layer's E packed
 * blocks (moe_pack_experts layout) in pinned host memory (hipHostMalloc),
 * 16-byte aligned.  Both stay owned by the caller and must outlive the
 * cache.  Both NULL gives a planning-only cache (moe_cache_plan). */
moe_status moe_cache_create(const moe_shape* shape, int32_t n_slots, uint8_t* device_slots,
                            const uint8_t* host_blocks, moe_expert_cache** cache);
void moe_cache_destroy(moe_expert_cache* cache);

/* Pin (pinned != 0) or unpin an expert: a resident pinned expert is never
 * evicted; pinning loads nothing by itself.  MOE_ERR_UNSUPPORTED if more
 * than n_slots - top_k experts would be pinned. */
moe_status moe_cache_pin(moe_expert_cache* cache, int32_t expert, int32_t pinned);

/* One step of the policy on a planning-only cache, on the host (no GPU):
 * experts [n] (host, ids in [0, E), repeats allowed) -> slot_of [n] (host
 * out), and the experts the step fetches, in placement order: fetched [k']
 * with evicted [k'] (the expert each displaced, -1 for an empty slot),
 * k' = *n_fetched (arrays of n entries suffice).  MOE_ERR_UNSUPPORTED
 * (state unchanged) if the pinned experts leave too few slots; on a cache
 * with device slots MOE_ERR_UNSUPPORTED (the slots would no longer match
 * what the device holds). */
moe_status moe_cache_plan(moe_expert_cache* cache, int32_t n, const int32_t* experts,
                          int32_t* slot_of, int32_t* fetched, int32_t* evicted,
                          int32_t* n_fetched);

/* Counters since creation: hits and misses (one per distinct expert of a
 * step) and the bytes copied host -> HBM.  Any pointer may be NULL. */
moe_status moe_cache_stats(const moe_expert_cache* cache, int64_t* hits, int64_t* misses,
                           int64_t* bytes_fetched);

/* The experts the latest step of this cache (moe_cache_layer_decode or
 * moe_cache_plan) fetched, in placement order: fetched [k'] with evicted [k']
 * (the expert each displaced, -1 for an empty slot), k' = *n_fetched.  A
 * step whose copies could not all be queued records nothing (its slots are
 * left empty).  capacity: entries the two host arrays hold (n_experts always
 * suffices); MOE_ERR_SHAPE if fewer than k'. */
moe_status moe_cache_last_fetch(const moe_expert_cache* cache, int32_t capacity, int32_t* fetched,
                                int32_t* evicted, int32_t* n_fetched);

/* Undo the latest step's placements (what moe_cache_last_fetch reports):
 * the slots it filled become empty, its misses are taken back, and the
 * latest-step record is cleared; the experts it displaced stay evicted.
 * For callers of moe_cache_plan whose own copies into the slots failed;
 * moe_cache_layer_decode does the same when its copies cannot be queued.
 * Calling it twice in a row changes nothing the second time. */
moe_status moe_cache_unplan_last(moe_expert_cache* cache);

/* Device scratch bytes of moe_cache_layer_decode; 0 for a shape the cache
 * rejects, T < 0, n_slots < 1 or T * top_k > 1024. */
size_t moe_cache_workspace_bytes(const moe_shape* shape, int32_t T, int32_t n_slots);

/* One decode step of the layer through the cache: the router (as
 * moe_route: topk_idx, topk_w), then -- after the one host wait of the
 * call, for the routing -- the misses are copied from host_blocks into
 * their slots on copy_stream while the FFN of the resident experts and the
 * shared expert runs on `stream`; `stream` then waits for the copies, runs
 * the FFN of the fetched experts and the combine.  out (out_dt) is, bit for
 * bit, the layer output of the separate calls with every expert resident;
 * y (float32 [T*k][d]) is in the cache's grouped order (by slot);
 * y_shared (float32 [T][d]) as moe_expert_ffn writes it.
 *  x: bf16 or f32 [T][d]; w_router, bias, shared: as for moe_route and
 *  moe_expert_ffn.  workspace >= moe_cache_workspace_bytes(shape, T,
 *  n_slots), 256-byte aligned.
 * T * top_k <= 1024, and n_slots - (pinned experts) >= min(E, T * top_k)
 * (else MOE_ERR_UNSUPPORTED, nothing enqueued).  MOE_ERR_NULL on a
 * planning-only cache.  If a host -> slot copy cannot be queued, the call
 * returns MOE_ERR_HIP with the step's fetched experts unmapped (their slots
 * empty), so no later step reads a partly written slot as a hit. */
moe_status moe_cache_layer_decode(moe_expert_cache* cache, int32_t T, const void* x,
                                  moe_dtype x_dt, const float* w_router, const float* bias,
                                  const uint8_t* shared, int32_t* topk_idx, float* topk_w,
                                  void* y, void* y_shared, void* out, moe_dtype out_dt,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  void* copy_stream);

/* Static text for a status code. */
const char* moe_status_str(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_INT4_H */
