"""Plain, slow, float64 CPU oracle of one MoE layer's routed-expert FFN over
int4 group-quantised weights.

TEST INFRASTRUCTURE ONLY: imported by tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the GPU library.  It shares no code,
table or helper with the HIP path; the only thing both sides share is the
seeded input generator in ``synth/`` (which holds none of this arithmetic).

Every step is the plain definition of what the layer computes, written out in
the order the pages describe the layer, in float64 throughout:

  O1 router logits   l[t,e] = sum_i x[t,i] W_r[e,i] + b[e]
  O2 top-k           the k largest logits of a token (ties: lower expert id
                     first), ordered by descending logit
  O3 gate weights    softmax over the k selected logits (= softmax over all
                     experts renormalised over the chosen k)
  O4 batch-union     counting sort of the T*k routing slots by expert, giving
                     counts, offsets, the slot permutation, its inverse and
                     the list of experts that received at least one slot
  O5 int4 dequant    W[r,c] = q[r,c] * s[r, c // 64], q a two's-complement
                     nibble in [-8, 7], s an IEEE float16 group scale
  O6 expert FFN      SwiGLU: y = W_down (silu(W_gate x) * (W_up x))
  O7 shared expert   the same FFN applied to every token
  O8 combine         out[t] = sum_j w[t,j] y[slot(t,j)] + y_shared[t]
  O9 quantiser       float weights -> int4 codes and float16 scales, per
                     64-column group or per row (the one-time conversion)

Sources (the pages, by title and section):

* zhichai.net, "744亿参数塞进25GB内存：colibrì如何用1300行C代码把不可能变成可能",
  section "漏洞在哪里：MoE 架构的稀疏性" (the sparsity loophole): 256 experts per
  layer, 8 + 1 active, the router choosing 8 experts per token dynamically;
  section "三层存储层级" (three storage tiers): the "+1" shared expert active in
  every layer, each routed expert one ~19 MB int4 block.
* yunpan.plus article on Colibrì, section "核心能力二：I/O 不是后勤，而是推理的前线"
  (capability 2, I/O as the front line): an expert needed by several positions
  of one batch is read once (batch-union); section "核心能力三：无 GPU 能跑，有
  GPU 更快" (capability 3): a cluster worker receives one layer's routed
  batch-union and runs the FFN on it; section "核心能力四：语义硬保证" (capability
  4, semantic guarantee): gs64 group quantisation of the int4 experts, and the
  rule that precision and router semantics never change silently.
* ssnai.com digest, "colibri：纯C把744B至2.8T MoE跑在本地硬件上", section "前置条件"
  (prerequisites): the gs64 int4 expert container.

Readings where the pages are silent (each also listed in the design notes):
the gate is a softmax renormalised over the chosen k (no routed scaling
factor); ties go to the lower expert id; a router bias, when present, is added
before both selection and weighting; int4 codes are symmetric two's-complement
nibbles, low nibble first, no zero point; groups run along the input
dimension; scales are float16; the FFN is SwiGLU without biases; the shared
expert is added with weight 1; slots are ordered by (expert, token).
"""
from __future__ import annotations

import numpy as np

GROUP = 64


# ----------------------------------------------------------------------------
# Expert block layout and int4 decoding (O5)
# ----------------------------------------------------------------------------

def expert_block_bytes(d: int, f: int, group: int = GROUP) -> int:
    """Bytes of one expert: 3*d*f int4 codes (half a byte each) plus one
    float16 scale per group of 64 codes.  The pages give ~19 MB per routed int4
    expert (zhichai.net, three storage tiers; yunpan.plus, capability 1)."""
    return 3 * d * f // 2 + 3 * d * f // group * 2


def split_block(block: np.ndarray, d: int, f: int, group: int = GROUP):
    """Cut one expert block into its six sub-arrays (codes row-major
    [out][in/2], scales [out][in/group] float16)."""
    block = np.asarray(block, dtype=np.uint8)
    parts = []
    pos = 0
    for rows, cols in ((f, d), (f, d), (d, f)):
        n = rows * cols // 2
        parts.append(block[pos:pos + n].reshape(rows, cols // 2))
        pos += n
    for rows, cols in ((f, d), (f, d), (d, f)):
        n = rows * (cols // group) * 2
        parts.append(block[pos:pos + n].view(np.float16).reshape(rows, cols // group))
        pos += n
    assert pos == block.size, "block size does not match (d, f)"
    return parts  # q_gate, q_up, q_down, s_gate, s_up, s_down


def unpack_int4(codes: np.ndarray) -> np.ndarray:
    """Bytes [rows, cols/2] -> signed codes [rows, cols] (int64).
    Element 2j sits in the low nibble of byte j, element 2j+1 in the high
    nibble; a nibble v encodes v for v < 8 and v - 16 otherwise."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, half = codes.shape
    out = np.empty((rows, 2 * half), dtype=np.int64)
    low = (codes & 0x0F).astype(np.int64)
    high = (codes >> 4).astype(np.int64)
    out[:, 0::2] = np.where(low >= 8, low - 16, low)
    out[:, 1::2] = np.where(high >= 8, high - 16, high)
    return out


def dequant(codes: np.ndarray, scales: np.ndarray, group: int = GROUP) -> np.ndarray:
    """O5: W[r, c] = q[r, c] * s[r, c // group], in float64 (exact: a 4-bit
    integer times a float16 fits float64 without rounding)."""
    q = unpack_int4(codes).astype(np.float64)
    s = np.repeat(np.asarray(scales, dtype=np.float64), group, axis=1)
    assert s.shape == q.shape
    return q * s


def expert_weights(block: np.ndarray, d: int, f: int, group: int = GROUP):
    """Dequantised (W_gate [f,d], W_up [f,d], W_down [d,f]) of one block."""
    qg, qu, qd, sg, su, sd = split_block(block, d, f, group)
    return dequant(qg, sg, group), dequant(qu, su, group), dequant(qd, sd, group)


def quantize_with_scales(w: np.ndarray, scales: np.ndarray, group: int = GROUP) -> np.ndarray:
    """Inverse of ``dequant`` for given scales: the nearest code in [-8, 7]
    for every element, packed low nibble first.  Used to check that
    quantising a dequantised matrix with its own scales gives the codes back."""
    s = np.repeat(np.asarray(scales, dtype=np.float64), group, axis=1)
    q = np.clip(np.rint(np.asarray(w, dtype=np.float64) / s), -8, 7).astype(np.int64)
    nib = (q & 0x0F).astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


# ----------------------------------------------------------------------------
# Quantiser (O9): float weights -> int4 codes + float16 scales
# ----------------------------------------------------------------------------
# The step the pages' engine runs once on a checkpoint before serving (ssnai.com
# digest, first command; P1 "capability 4": int4 experts with gs64 scales,
# compared there against one scale per row).  The pages give no rounding rule;
# the reading here is the plain symmetric one:
#   s = float16(float32(absmax) / float32(7))   (absmax over the group or row)
#   q = the integer nearest to w / s, ties to even, clipped to [-8, 7];
#       a group of zeros has s = 0 and q = 0.

def quant_scale(absmax) -> np.ndarray:
    """float16 scale(s) for the given absolute maxima (float32 division by 7,
    then rounding to float16, both round-to-nearest-even)."""
    a = np.asarray(absmax, dtype=np.float32)
    return (a / np.float32(7.0)).astype(np.float16)


def quant_codes(w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Signed codes (int64): nearest integer to w / s, ties to even, clipped
    to [-8, 7]; 0 where s == 0.  w / s is evaluated in float64, where it is
    never rounded onto a half-integer it is not exactly equal to."""
    w = np.asarray(w, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(np.where(s != 0.0, w / np.where(s != 0.0, s, 1.0), 0.0))
    return np.clip(q, -8, 7).astype(np.int64)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Signed codes [rows, cols] -> bytes [rows, cols/2], element 2j in the low
    nibble of byte j (the inverse of ``unpack_int4``)."""
    nib = (np.asarray(q, dtype=np.int64) & 0x0F).astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def quantize_gs64(w: np.ndarray, group: int = GROUP):
    """O9, group mode: w [N, K] (float32 or bf16 values) -> (codes [N, K/2]
    uint8, scales [N, K/group] float16)."""
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    g = w.reshape(n, k // group, group)
    s = quant_scale(np.max(np.abs(g), axis=2))
    q = quant_codes(g, s[:, :, None].astype(np.float64)).reshape(n, k)
    return pack_int4(q), s


def quantize_rows(w: np.ndarray):
    """O9, per-row mode: one scale per row -> (codes [N, K/2], scales [N])."""
    w = np.asarray(w, dtype=np.float64)
    s = quant_scale(np.max(np.abs(w), axis=1))
    q = quant_codes(w, s[:, None].astype(np.float64))
    return pack_int4(q), s


# ----------------------------------------------------------------------------
# Routing (O1-O3)
# ----------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """O1: l[t, e] = sum_i x[t, i] * W_r[e, i] (+ b[e]), float64.
    Each product of a bf16/fp32 activation and an fp32 weight is exact in
    float64, so only the summation order separates two correct answers."""
    lg = np.asarray(x, dtype=np.float64) @ np.asarray(w_router, dtype=np.float64).T
    if bias is not None:
        lg = lg + np.asarray(bias, dtype=np.float64)[None, :]
    return lg


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """O2: per token, sort all (logit, expert) pairs by logit descending and
    expert id ascending, keep the first k."""
    T, E = logits.shape
    ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((ids, -logits), axis=-1)   # last key is the primary key
    return order[:, :k].astype(np.int32)


def gate_weights(logits: np.ndarray, topk_idx: np.ndarray) -> np.ndarray:
    """O3: w[t, j] = exp(l_j - m) / sum_j' exp(l_j' - m) over the chosen k
    (m = the largest chosen logit), computed in float64, returned float32
    (round to nearest even)."""
    sel = np.take_along_axis(logits, topk_idx.astype(np.int64), axis=1)
    m = sel.max(axis=1, keepdims=True)
    p = np.exp(sel - m)
    return (p / p.sum(axis=1, keepdims=True)).astype(np.float32)


def route(x, w_router, bias, k):
    """O1-O3 for a batch.  Returns (topk_idx int32 [T,k], topk_w float32
    [T,k], logits float64 [T,E])."""
    lg = router_logits(x, w_router, bias)
    idx = topk_select(lg, k)
    return idx, gate_weights(lg, idx), lg


# ----------------------------------------------------------------------------
# Batch-union grouping (O4)
# ----------------------------------------------------------------------------

def batch_union(topk_idx: np.ndarray, n_experts: int):
    """O4: group the T*k routing slots (slot id s = t*k + j) by expert so each
    expert's weights are read once for all of its tokens.

    counts[e]   slots routed to expert e
    offsets     exclusive prefix sum of counts, length E+1
    perm[i]     the slot id at grouped position i; slots are ordered by expert
                ascending, then by slot id ascending (= token ascending)
    inv_perm[s] the grouped position of slot s
    active      experts with counts > 0, ascending (first n_active entries;
                the rest is filled with -1)

    A slot whose expert id lies outside [0, E) is not grouped: it is not
    counted, has no grouped position (inv_perm = -1) and adds nothing in the
    combine.  (The pages never produce such ids; this is the library's rule.)
    """
    flat = [int(e) for e in np.asarray(topk_idx).reshape(-1)]
    n = len(flat)
    counts = [0] * n_experts
    for e in flat:
        if 0 <= e < n_experts:
            counts[e] += 1
    offsets = [0] * (n_experts + 1)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = list(offsets[:n_experts])
    perm = [-1] * n
    for s, e in enumerate(flat):          # slots visited in id order: stable
        if 0 <= e < n_experts:
            perm[fill[e]] = s
            fill[e] += 1
    inv_perm = [-1] * n
    for i, s in enumerate(perm[:offsets[n_experts]]):
        inv_perm[s] = i
    active = [e for e in range(n_experts) if counts[e] > 0]
    n_active = len(active)
    active = active + [-1] * (n_experts - n_active)
    as32 = lambda v: np.asarray(v, dtype=np.int32)
    return (as32(counts), as32(offsets), as32(perm), as32(inv_perm), as32(active),
            np.asarray([n_active], dtype=np.int32))


# ----------------------------------------------------------------------------
# Expert FFN (O6, O7) and combine (O8)
# ----------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(X: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """O6 for a group of rows X [M, d]: Y = (silu(X Wg^T) * (X Wu^T)) Wd^T."""
    G = X @ Wg.T
    U = X @ Wu.T
    return (silu(G) * U) @ Wd.T


def expert_ffn(x, experts, shared, offsets, perm, active, n_active, top_k, d, f,
               group: int = GROUP, weights=None):
    """O6-O7: for every expert with routed slots, gather its tokens
    (token of slot s = s // k) and run the SwiGLU expert on them; results go to
    ``y`` in grouped (permuted) order.  The shared expert runs on every token
    in token order.  Returns (y [T*k, d], y_shared [T, d] or None), float64.
    ``weights(block, d, f)`` decodes a block (default: the int4 gs64 block)."""
    if weights is None:
        weights = lambda blk, d_, f_: expert_weights(blk, d_, f_, group)  # noqa: E731
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    y = np.zeros((T * top_k, d), dtype=np.float64)
    for a in range(int(np.asarray(n_active).reshape(-1)[0])):
        e = int(active[a])
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        tokens = np.asarray(perm[lo:hi], dtype=np.int64) // top_k
        Wg, Wu, Wd = weights(experts[e], d, f)
        y[lo:hi] = swiglu(x[tokens], Wg, Wu, Wd)
    y_shared = None
    if shared is not None:
        Wg, Wu, Wd = weights(shared, d, f)
        y_shared = swiglu(x, Wg, Wu, Wd)
    return y, y_shared


def combine(y, y_shared, inv_perm, topk_w, top_k):
    """O8: out[t] = sum_{j<k} w[t,j] * y[inv_perm[t*k+j]] + y_shared[t],
    summed in j order, float64."""
    w = np.asarray(topk_w, dtype=np.float64)
    T = w.shape[0]
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for j in range(top_k):
        rows = np.asarray(inv_perm, dtype=np.int64).reshape(T, top_k)[:, j]
        routed = rows >= 0
        out[routed] += w[routed, j:j + 1] * y[rows[routed]]
    if y_shared is not None:
        out += y_shared
    return out


def moe_layer(x, w_router, bias, experts, shared, d, f, n_experts, top_k, group: int = GROUP,
              weights=None):
    """The whole layer, O1-O8.  Returns a dict of every intermediate.
    ``weights``: the block decoder (default int4 gs64; oracle.mxfp4's
    expert_weights for MXFP4 blocks)."""
    idx, w, lg = route(x, w_router, bias, top_k)
    counts, offsets, perm, inv_perm, active, n_active = batch_union(idx, n_experts)
    y, ys = expert_ffn(x, experts, shared, offsets, perm, active, n_active, top_k, d, f, group,
                       weights)
    out = combine(y, ys, inv_perm, w, top_k)
    return dict(logits=lg, topk_idx=idx, topk_w=w, counts=counts, offsets=offsets, perm=perm,
                inv_perm=inv_perm, active=active, n_active=n_active, y=y, y_shared=ys, out=out)
