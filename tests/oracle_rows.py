"""Oracle rows of a large layer, for GPU parity tests at full size.

At the sizes where the whole oracle would take minutes (the ~19 MB-expert
layer with hundreds of routed experts), the tests compare selected rows
only: the oracle routes and groups the whole batch (that is cheap), then
evaluates the SwiGLU of each needed expert for just the tokens asked for.
Experts are decoded one per worker thread (numpy releases the GIL in the
decoding and the products), each expert's weights held only while its rows
are computed.  Everything here calls ``oracle`` functions; nothing comes
from the GPU path.
"""
from __future__ import annotations

import concurrent.futures
import os

import numpy as np

import oracle


def workers() -> int:
    # the GPU hosts give a job 16 CPU threads; stay within what is there
    return max(1, min(16, os.cpu_count() or 1))


def expert_rows(L, xf, requests, weights=None):
    """requests: {expert id or "shared": [token, ...]} -> {(key, token): y row
    (float64 [d])}.  weights: the oracle's block decoder (int4 gs64 default)."""
    weights = oracle.expert_weights if weights is None else weights
    sh = L.shape
    x = np.asarray(xf, dtype=np.float64)

    def one(item):
        key, toks = item
        blk = L.shared if key == "shared" else L.experts[key]
        wg, wu, wd = weights(blk, sh.d, sh.f)
        toks = sorted(set(int(t) for t in toks))
        res = oracle.swiglu(x[toks], wg, wu, wd)
        return {(key, t): r for t, r in zip(toks, res)}

    out = {}
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers()) as ex:
        for part in ex.map(one, list(requests.items())):
            out.update(part)
    return out


def oracle_sampled(L, xf, sample_tokens, weights=None, bias="layer"):
    """Oracle routing and grouping for the whole batch; expert outputs and
    layer outputs only for the sampled tokens.  bias: the router bias
    ("layer" = the layer's own)."""
    sh = L.shape
    b = L.bias if isinstance(bias, str) else bias
    idx, w, lg = oracle.route(xf, L.w_router, b, sh.top_k)
    union = oracle.batch_union(idx, sh.n_experts)
    inv = union[3]
    need = {}
    for t in sample_tokens:
        for j in range(sh.top_k):
            need.setdefault(int(idx[t, j]), []).append(t)
        if L.shared is not None:
            need.setdefault("shared", []).append(t)
    rows = expert_rows(L, xf, need, weights)
    y, ysh, out = {}, {}, {}
    for t in sample_tokens:
        acc = np.zeros(sh.d)
        for j in range(sh.top_k):
            p = int(inv[t * sh.top_k + j])
            y[p] = rows[(int(idx[t, j]), t)]
            acc += float(w[t, j]) * y[p]
        ysh[t] = rows[("shared", t)] if L.shared is not None else np.zeros(sh.d)
        out[t] = acc + ysh[t]
    return dict(topk_idx=idx, topk_w=w, union=union, y=y, y_shared=ysh, out=out, logits=lg)


def prefill_tiles(M: int):
    """(first row, last row) of every M-tile the prefill path cuts an expert
    of M rows into: 128-row tiles while at least 96 rows are left, then
    32-row tiles (the grouping rule of the library's tile lists)."""
    nb = M // 128 + (1 if M % 128 >= 96 else 0)
    tiles = [(i * 128, min(M, i * 128 + 128) - 1) for i in range(nb)]
    r = nb * 128
    while r < M:
        tiles.append((r, min(M, r + 32) - 1))
        r += 32
    return tiles
