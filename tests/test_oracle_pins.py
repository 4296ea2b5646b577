"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks the oracle against a value the pages fix, a closed form, a
brute-force evaluation written independently (its own byte decoding, its own
loops), an invariant, or a library routine the oracle does not call.  Together
they are meant to catch a dropped term, a wrong sign or index, or a transposed
operand anywhere in the oracle.
"""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# int4 decoding and dequantisation
# ----------------------------------------------------------------------------

def test_nibble_decode_all_256_bytes_by_arithmetic_shift():
    # independent decode: move the nibble to the top of a signed byte, shift back
    b = np.arange(256, dtype=np.uint8)
    low = ((b << 4).astype(np.uint8).view(np.int8) >> 4).astype(np.int64)
    high = (b.view(np.int8) >> 4).astype(np.int64)
    got = oracle.unpack_int4(b.reshape(256, 1))
    assert np.array_equal(got[:, 0], low)
    assert np.array_equal(got[:, 1], high)


@pytest.mark.parametrize("byte,low,high", [
    (0x00, 0, 0), (0x7F, -1, 7), (0x80, 0, -8), (0xF8, -8, -1), (0x12, 2, 1), (0x9E, -2, -7)])
def test_nibble_worked_bytes(byte, low, high):
    got = oracle.unpack_int4(np.array([[byte]], dtype=np.uint8))
    assert got.tolist() == [[low, high]]


def test_dequant_is_exact_product():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 256, size=(3, 64), dtype=np.uint8)
    scales = rng.uniform(0.005, 0.02, size=(3, 2)).astype(np.float16)
    w = oracle.dequant(codes, scales)
    for r in range(3):
        for c in range(128):
            byte = int(codes[r, c // 2])
            nib = (byte >> 4) if c % 2 else (byte & 15)
            q = nib - 16 if nib >= 8 else nib
            exact = Fraction(q) * Fraction(float(scales[r, c // 64]))
            assert Fraction(float(w[r, c])) == exact


def test_group_scale_lands_on_its_64_columns():
    # a single code of 1 at (r, c) must come back as scale[r, c // 64] at (r, c) only
    scales = (2.0 ** -np.arange(1, 9)).astype(np.float16).reshape(2, 4)  # distinct per group
    for r, c in [(0, 0), (0, 63), (0, 64), (1, 130), (1, 255)]:
        q = np.zeros((2, 256), dtype=np.int64)
        q[r, c] = 1
        nib = (q & 15).astype(np.uint8)
        codes = nib[:, 0::2] | (nib[:, 1::2] << 4)
        w = oracle.dequant(codes, scales)
        expect = np.zeros((2, 256))
        expect[r, c] = float(scales[r, c // 64])
        assert np.array_equal(w, expect)


def test_quantise_dequantised_codes_round_trip():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, size=(8, 96), dtype=np.uint8)
    scales = rng.uniform(0.005, 0.02, size=(8, 3)).astype(np.float16)
    back = oracle.quantize_with_scales(oracle.dequant(codes, scales), scales)
    assert np.array_equal(back, codes)


def test_bf16_codes_are_exact():
    # every code value is exactly representable in bfloat16
    q = np.arange(-8, 8, dtype=np.float32)
    bits = synth.bf16_round(q)
    assert np.array_equal(synth.bf16_to_f32(bits), q)


# ----------------------------------------------------------------------------
# Routing
# ----------------------------------------------------------------------------

def _brute_route(x, w_router, bias, k):
    """Pure-Python routing: correctly rounded logits (math.fsum of exact
    products), a full sort with Python's sorted(), softmax with math.exp."""
    T, d = x.shape
    E = w_router.shape[0]
    idx, wts = [], []
    for t in range(T):
        lg = []
        for e in range(E):
            v = math.fsum(float(x[t, i]) * float(w_router[e, i]) for i in range(d))
            if bias is not None:
                v = math.fsum([v, float(bias[e])])
            lg.append((v, e))
        top = sorted(lg, key=lambda p: (-p[0], p[1]))[:k]
        m = top[0][0]
        ex = [math.exp(v - m) for v, _ in top]
        z = math.fsum(ex)
        idx.append([e for _, e in top])
        wts.append([v / z for v in ex])
    return np.array(idx), np.array(wts)


def test_route_matches_brute_force_sort():
    rng = np.random.default_rng(2)
    T, d, E, k = 5, 64, 12, 3
    x = rng.standard_normal((T, d)).astype(np.float32)
    w = (rng.standard_normal((E, d)) * 0.02).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    idx, wt, _ = oracle.route(x, w, b, k)
    bidx, bwt = _brute_route(x, w, b, k)
    assert np.array_equal(idx, bidx)
    assert np.max(np.abs(wt - bwt)) <= 1e-7


def test_route_workload1_matches_brute_force_sort():
    layer = synth.make_layer(1, experts=[])
    _, x = synth.make_tokens(1, 4)
    idx, wt, _ = oracle.route(x, layer.w_router, layer.bias, layer.shape.top_k)
    bidx, bwt = _brute_route(x, layer.w_router, layer.bias, layer.shape.top_k)
    assert np.array_equal(idx, bidx)
    assert np.max(np.abs(wt - bwt)) <= 1e-7


def test_k_equal_E_is_the_full_softmax():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, 64)).astype(np.float32)
    w = (rng.standard_normal((8, 64)) * 0.05).astype(np.float32)
    idx, wt, lg = oracle.route(x, w, None, 8)
    full = scipy.special.softmax(x.astype(np.float64) @ w.astype(np.float64).T, axis=1)
    expect = -np.sort(-full, axis=1)
    assert np.max(np.abs(wt - expect)) <= 1e-7
    assert np.array_equal(np.sort(idx, axis=1), np.tile(np.arange(8), (6, 1)))


def test_two_experts_closed_form_sigmoid():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((10, 64)).astype(np.float32)
    w = (rng.standard_normal((2, 64)) * 0.1).astype(np.float32)
    idx, wt, lg = oracle.route(x, w, None, 2)
    for t in range(10):
        l0, l1 = lg[t, idx[t, 0]], lg[t, idx[t, 1]]
        assert l0 >= l1
        assert abs(wt[t, 0] - scipy.special.expit(l0 - l1)) <= 1e-7
        assert abs(wt[t, 1] - scipy.special.expit(l1 - l0)) <= 1e-7


def test_k1_gives_weight_one():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 64)).astype(np.float32)
    w = rng.standard_normal((9, 64)).astype(np.float32)
    idx, wt, lg = oracle.route(x, w, None, 1)
    assert np.all(wt == 1.0)
    assert np.array_equal(idx[:, 0], np.argmax(lg, axis=1))


def test_ties_go_to_lower_expert_id():
    x = np.zeros((1, 64), dtype=np.float32)
    w = np.zeros((5, 64), dtype=np.float32)
    b = np.array([0.0, 1.0, 1.0, 0.5, 1.0], dtype=np.float32)
    idx, wt, _ = oracle.route(x, w, b, 3)
    assert idx.tolist() == [[1, 2, 4]]
    assert np.allclose(wt, 1.0 / 3.0, atol=1e-7)
    idx, wt, _ = oracle.route(x, w, b, 4)
    assert idx.tolist() == [[1, 2, 4, 3]]


def test_constant_logit_shift_changes_nothing():
    layer = synth.make_layer(3, experts=[])
    _, x = synth.make_tokens(3, 16)
    idx, wt, _ = oracle.route(x, layer.w_router, layer.bias, 8)
    idx2, wt2, _ = oracle.route(x, layer.w_router, layer.bias + np.float32(3.25), 8)
    assert np.array_equal(idx, idx2)
    assert np.max(np.abs(wt - wt2)) <= 1e-7


def test_permuting_experts_permutes_indices():
    layer = synth.make_layer(3, experts=[])
    _, x = synth.make_tokens(3, 16)
    pi = np.random.default_rng(6).permutation(256)
    idx, wt, _ = oracle.route(x, layer.w_router, layer.bias, 8)
    idx2, wt2, _ = oracle.route(x, layer.w_router[pi], layer.bias[pi], 8)
    assert np.array_equal(pi[idx2], idx)
    assert np.array_equal(wt, wt2)


@pytest.mark.parametrize("cfg,T", [(2, 16), (3, 64), (4, 8)])
def test_gate_weights_sum_to_one_and_descend(cfg, T):
    layer = synth.make_layer(cfg, experts=[])
    _, x = synth.make_tokens(cfg, T)
    idx, wt, lg = oracle.route(x, layer.w_router, layer.bias, layer.shape.top_k)
    assert np.max(np.abs(wt.astype(np.float64).sum(axis=1) - 1.0)) <= 1e-6
    sel = np.take_along_axis(lg, idx.astype(np.int64), axis=1)
    assert np.all(np.diff(sel, axis=1) < 0)
    assert np.all([len(set(r)) == len(r) for r in idx.tolist()])


# ----------------------------------------------------------------------------
# Batch-union grouping
# ----------------------------------------------------------------------------

def test_union_worked_example():
    # 3 tokens, k = 2, 4 experts; slot s = t*k + j routes to topk[t][j]
    topk = np.array([[2, 0], [0, 1], [2, 1]], dtype=np.int32)
    counts, offsets, perm, inv, active, n_active = oracle.batch_union(topk, 4)
    assert counts.tolist() == [2, 2, 2, 0]
    assert offsets.tolist() == [0, 2, 4, 6, 6]
    assert perm.tolist() == [1, 2, 3, 5, 0, 4]
    assert inv.tolist() == [4, 0, 1, 2, 5, 3]
    assert active.tolist() == [0, 1, 2, -1]
    assert n_active.tolist() == [3]


@pytest.mark.parametrize("T,k,E,seed", [(1, 8, 64, 0), (16, 8, 64, 1), (64, 8, 256, 2), (300, 4, 16, 3)])
def test_union_matches_library_stable_sort(T, k, E, seed):
    rng = np.random.default_rng(seed)
    topk = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, inv, active, n_active = oracle.batch_union(topk, E)
    flat = topk.reshape(-1)
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(inv[perm], np.arange(T * k))
    uniq = np.unique(flat)
    assert n_active[0] == len(uniq)
    assert np.array_equal(active[:len(uniq)], uniq) and np.all(active[len(uniq):] == -1)
    # grouped order: expert ascending, token ascending within an expert
    key = [(int(flat[s]), s // k) for s in perm]
    assert key == sorted(key)


# ----------------------------------------------------------------------------
# Expert FFN and combine
# ----------------------------------------------------------------------------

def _raw_matrix(block, d, f, which):
    """Independent reading of the block layout: byte offsets computed here,
    codes decoded with (v ^ 8) - 8, scales read with struct."""
    sizes = [f * d // 2, f * d // 2, d * f // 2]
    rows, cols = [(f, d), (f, d), (d, f)][which]
    qoff = sum(sizes[:which])
    soff = sum(sizes) + sum(r * (c // 64) * 2 for r, c in [(f, d), (f, d), (d, f)][:which])
    raw = bytes(block)

    def w(r, c):
        byte = raw[qoff + r * (cols // 2) + c // 2]
        nib = (byte >> 4) if (c & 1) else (byte & 15)
        q = (nib ^ 8) - 8
        (s,) = struct.unpack_from("<e", raw, soff + (r * (cols // 64) + c // 64) * 2)
        return q * s
    return rows, cols, w


def _brute_expert(block, d, f, xt):
    """One token through one expert with scalar Python loops."""
    _, _, wg = _raw_matrix(block, d, f, 0)
    _, _, wu = _raw_matrix(block, d, f, 1)
    _, _, wd = _raw_matrix(block, d, f, 2)
    h = []
    for r in range(f):
        g = math.fsum(wg(r, c) * float(xt[c]) for c in range(d))
        u = math.fsum(wu(r, c) * float(xt[c]) for c in range(d))
        h.append(g / (1.0 + math.exp(-g)) * u)
    return np.array([math.fsum(wd(r, c) * h[c] for c in range(f)) for r in range(d)])


def test_expert_ffn_matches_scalar_brute_force():
    rng = np.random.default_rng(7)
    d, f, E, k, T = 128, 64, 3, 2, 3
    bb = oracle.expert_block_bytes(d, f)
    blocks = np.zeros((E, bb), dtype=np.uint8)
    for e in range(E):
        blocks[e, :3 * d * f // 2] = rng.integers(0, 256, 3 * d * f // 2, dtype=np.uint8)
        blocks[e, 3 * d * f // 2:] = rng.uniform(0.005, 0.02, 3 * d * f // 64).astype(np.float16).view(np.uint8)
    shared = blocks[0].copy()
    x = rng.standard_normal((T, d)).astype(np.float32)
    w = (rng.standard_normal((E, d)) * 0.3).astype(np.float32)
    res = oracle.moe_layer(x, w, None, blocks, shared, d, f, E, k)
    for t in range(T):
        for j in range(k):
            e = int(res["topk_idx"][t, j])
            ref = _brute_expert(blocks[e], d, f, x[t])
            got = res["y"][res["inv_perm"][t * k + j]]
            assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
        ref_s = _brute_expert(shared, d, f, x[t])
        assert np.max(np.abs(res["y_shared"][t] - ref_s)) <= 1e-12 * max(1.0, np.max(np.abs(ref_s)))


def test_expert_ffn_single_weight_closed_form():
    # gate code 3 at (5, 70) with scale 0.5, up code -2 at (5, 3) with scale 0.25,
    # down code 7 at (100, 5) with scale 0.125 -> only y[100] is non-zero:
    # y[100] = 0.875 * silu(1.5 x[70]) * (-0.5 x[3])
    d, f = 128, 64
    bb = oracle.expert_block_bytes(d, f)
    blk = np.zeros(bb, dtype=np.uint8)
    qg, qu, qd = 0, f * d // 2, 2 * f * d // 2
    sg = 3 * d * f // 2
    su = sg + f * (d // 64) * 2
    sd = su + f * (d // 64) * 2
    blk[qg + 5 * (d // 2) + 35] = 0x03          # col 70: low nibble of byte 35
    blk[qu + 5 * (d // 2) + 1] = 0xE0           # col 3: high nibble of byte 1, -2
    blk[qd + 100 * (f // 2) + 2] = 0x70         # col 5: high nibble of byte 2, 7
    blk[sg:sg + f * (d // 64) * 2] = np.full(f * (d // 64), 9.0, np.float16).view(np.uint8)
    blk[su:sd] = np.full(f * (d // 64), 9.0, np.float16).view(np.uint8)
    blk[sd:] = np.full(d * (f // 64), 9.0, np.float16).view(np.uint8)
    blk[sg + (5 * 2 + 1) * 2: sg + (5 * 2 + 1) * 2 + 2] = np.array([0.5], np.float16).view(np.uint8)
    blk[su + (5 * 2 + 0) * 2: su + (5 * 2 + 0) * 2 + 2] = np.array([0.25], np.float16).view(np.uint8)
    blk[sd + (100 * 1 + 0) * 2: sd + (100 * 1 + 0) * 2 + 2] = np.array([0.125], np.float16).view(np.uint8)
    x = np.random.default_rng(8).standard_normal((2, d))
    y, _ = oracle.expert_ffn(x, blk[None], None, np.array([0, 2]), np.array([0, 1]),
                             np.array([0]), np.array([1]), 1, d, f)
    g = 1.5 * x[:, 70]
    expect = 0.875 * (g / (1.0 + np.exp(-g))) * (-0.5 * x[:, 3])
    mask = np.ones(d, dtype=bool)
    mask[100] = False
    assert np.all(y[:, mask] == 0.0)
    assert np.allclose(y[:, 100], expect, rtol=1e-15, atol=0)


def test_silu_special_values():
    z = np.array([0.0, 30.0, -30.0, 1.0])
    s = oracle.silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 30.0) < 1e-11
    assert abs(s[2]) < 1e-11
    assert abs(s[3] - scipy.special.expit(1.0)) < 1e-16


def test_doubling_down_scales_doubles_y_exactly():
    layer = synth.make_layer(1)
    _, x = synth.make_tokens(1, 4)
    sh = layer.shape
    res = oracle.moe_layer(x, layer.w_router, None, layer.experts, None, sh.d, sh.f, sh.n_experts, sh.top_k)
    blocks = layer.experts.copy()
    sd = 3 * sh.d * sh.f // 2 + 2 * sh.f * (sh.d // 64) * 2
    for e in range(sh.n_experts):
        s = blocks[e, sd:].view(np.float16)
        s *= np.float16(2.0)
    res2 = oracle.moe_layer(x, layer.w_router, None, blocks, None, sh.d, sh.f, sh.n_experts, sh.top_k)
    assert np.array_equal(res2["y"], 2.0 * res["y"])


def _torch_dense_masked(x, w_router, bias, blocks, shared, d, f, E, k, idx, wts):
    """Every expert evaluated for every token (torch float64, its own decoding
    of the block layout), gates zero outside each token's chosen k."""
    xt = torch.from_numpy(np.asarray(x, dtype=np.float64))
    T = xt.shape[0]

    def mats(blk):
        b = torch.from_numpy(np.asarray(blk, dtype=np.uint8).copy()).to(torch.int64)
        out = []
        qpos = 0
        spos = 3 * d * f // 2
        for rows, cols in ((f, d), (f, d), (d, f)):
            q = b[qpos:qpos + rows * cols // 2].reshape(rows, cols // 2)
            lo, hi = q & 15, q >> 4
            lo = lo - ((lo & 8) << 1)
            hi = hi - ((hi & 8) << 1)
            codes = torch.stack([lo, hi], dim=2).reshape(rows, cols).to(torch.float64)
            nb = rows * (cols // 64) * 2
            s = torch.from_numpy(np.asarray(blk[spos:spos + nb]).view(np.float16).astype(np.float64))
            s = s.reshape(rows, cols // 64).repeat_interleave(64, dim=1)
            out.append(codes * s)
            qpos += rows * cols // 2
            spos += nb
        return out

    gate = torch.zeros((T, E), dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            gate[t, int(idx[t, j])] = float(wts[t, j])
    out = torch.zeros((T, d), dtype=torch.float64)
    for e in range(E):
        wg, wu, wd = mats(blocks[e])
        y = (torch.nn.functional.silu(xt @ wg.T) * (xt @ wu.T)) @ wd.T
        out += gate[:, e:e + 1] * y
    if shared is not None:
        wg, wu, wd = mats(shared)
        out += (torch.nn.functional.silu(xt @ wg.T) * (xt @ wu.T)) @ wd.T
    return out.numpy()


@pytest.mark.parametrize("cfg,T", [(1, 4), (2, 1), (6, 16)])
def test_sparse_layer_equals_dense_masked_gates(cfg, T):
    layer = synth.make_layer(cfg)
    _, x = synth.make_tokens(cfg, T)
    sh = layer.shape
    res = oracle.moe_layer(x, layer.w_router, layer.bias, layer.experts, layer.shared,
                           sh.d, sh.f, sh.n_experts, sh.top_k)
    dense = _torch_dense_masked(x, layer.w_router, layer.bias, layer.experts, layer.shared,
                                sh.d, sh.f, sh.n_experts, sh.top_k, res["topk_idx"], res["topk_w"])
    scale = np.max(np.abs(dense))
    assert np.max(np.abs(res["out"] - dense)) <= 1e-12 * scale


def test_layer_with_shared_equals_dense_masked_gates():
    # small layer with a shared expert and skew-free routing, k = 3 of 6
    rng = np.random.default_rng(9)
    d, f, E, k, T = 128, 64, 6, 3, 5
    bb = oracle.expert_block_bytes(d, f)
    blocks = np.zeros((E, bb), dtype=np.uint8)
    for e in range(E):
        blocks[e, :3 * d * f // 2] = rng.integers(0, 256, 3 * d * f // 2, dtype=np.uint8)
        blocks[e, 3 * d * f // 2:] = rng.uniform(0.005, 0.02, 3 * d * f // 64).astype(np.float16).view(np.uint8)
    shared = blocks[E - 1].copy()
    shared[:100] ^= 0x5A
    x = rng.standard_normal((T, d)).astype(np.float32)
    w = (rng.standard_normal((E, d)) * 0.2).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    res = oracle.moe_layer(x, w, b, blocks, shared, d, f, E, k)
    dense = _torch_dense_masked(x, w, b, blocks, shared, d, f, E, k, res["topk_idx"], res["topk_w"])
    assert np.max(np.abs(res["out"] - dense)) <= 1e-12 * np.max(np.abs(dense))


def test_token_alone_equals_token_in_batch():
    layer = synth.make_layer(1)
    _, x = synth.make_tokens(1, 4)
    sh = layer.shape
    full = oracle.moe_layer(x, layer.w_router, None, layer.experts, None, sh.d, sh.f, sh.n_experts, sh.top_k)
    for t in range(4):
        one = oracle.moe_layer(x[t:t + 1], layer.w_router, None, layer.experts, None,
                               sh.d, sh.f, sh.n_experts, sh.top_k)
        assert np.allclose(one["out"][0], full["out"][t], rtol=0, atol=1e-12 * np.max(np.abs(full["out"])))


def test_combine_one_hot_is_y_plus_shared():
    rng = np.random.default_rng(10)
    T, d = 5, 16
    y = rng.standard_normal((T, d))
    ys = rng.standard_normal((T, d))
    inv = np.array([3, 0, 4, 1, 2])
    out = oracle.combine(y, ys, inv, np.ones((T, 1), np.float32), 1)
    assert np.array_equal(out, y[inv] + ys)


# ----------------------------------------------------------------------------
# Geometry of the pages' layer
# ----------------------------------------------------------------------------

def test_expert_geometry_matches_the_pages():
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    v = lambda key: facts[key]["value"]
    sh = synth.WORKLOADS[4]["shape"]
    assert sh.n_experts == v("routed_experts_per_layer")
    assert sh.top_k == v("active_routed_per_token") and sh.f_shared > 0
    blk = oracle.expert_block_bytes(sh.d, sh.f)
    assert blk == synth.block_bytes(sh.d, sh.f) == 20_054_016
    mib = blk / 2 ** 20
    assert abs(mib - v("routed_expert_megabytes_approx")) / v("routed_expert_megabytes_approx") < 0.05
    layers = v("routed_experts_total") / v("routed_experts_per_layer")
    assert layers == int(layers) == 76
    total_gb = v("routed_experts_total") * blk / 1e9
    assert abs(total_gb - v("routed_experts_total_gigabytes_approx")) / v("routed_experts_total_gigabytes_approx") < 0.06
    per_tok_gb = v("active_routed_per_token") * blk * layers / 1e9
    assert abs(per_tok_gb - v("routed_gigabytes_changing_per_token_approx")) / 11 < 0.15
    assert v("total_params_billion") * 0.5 == v("int4_model_gigabytes")


def test_union_skips_out_of_range_ids():
    topk = np.array([[2, 9], [-1, 1], [2, 1]], dtype=np.int32)   # E = 4: 9 and -1 are not experts
    counts, offsets, perm, inv, active, n_active = oracle.batch_union(topk, 4)
    assert counts.tolist() == [0, 2, 2, 0]
    assert offsets.tolist() == [0, 0, 2, 4, 4]
    assert perm[:4].tolist() == [3, 5, 0, 4]
    assert inv.tolist() == [2, -1, -1, 0, 3, 1]
    out = oracle.combine(np.arange(12.0).reshape(6, 2), None, inv, np.ones((3, 2)), 2)
    assert out.tolist() == [[4.0, 5.0], [0.0, 1.0], [6.0 + 2.0, 7.0 + 3.0]]


# ----------------------------------------------------------------------------
# Quantiser (O9)
# ----------------------------------------------------------------------------

def _round_frac(x: Fraction, mant_bits: int, min_exp: int) -> Fraction:
    """Round a positive Fraction to the nearest binary float with mant_bits
    bits of mantissa (implicit one included), ties to even; min_exp is the
    exponent of the smallest normal (subnormals keep that exponent)."""
    if x == 0:
        return Fraction(0)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    e = max(e, min_exp)
    ulp = Fraction(2) ** (e - mant_bits + 1)
    n = x / ulp
    lo = math.floor(n)
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return lo * ulp


def test_scale_rule_by_exact_rounding():
    # s = float16(float32(absmax / 7)): two round-to-nearest-even steps, here
    # done on exact fractions, independently of numpy's casts
    rng = np.random.default_rng(9)
    a = np.concatenate([rng.uniform(0, 3, 300), rng.uniform(0, 0.02, 300), [1.0, 7.0, 0.0, 3.5]])
    a = a.astype(np.float32)
    got = oracle.quant_scale(a)
    for ai, gi in zip(a, got):
        f32 = _round_frac(Fraction(float(ai)) / 7, 24, -126)
        f16 = _round_frac(f32, 11, -14)
        assert Fraction(float(gi)) == f16, (ai, gi)


def test_quant_codes_brute_force_nearest_with_ties_to_even():
    # every code is the q in [-8, 7] minimising |w - q*s| (exact fractions),
    # ties to the even q -- including exact half-way points
    rng = np.random.default_rng(10)
    s = np.float16(0.013671875)
    halfway = (np.arange(-8, 7) + 0.5) * float(s)
    w = np.concatenate([rng.uniform(-0.11, 0.11, 400), halfway, [0.0, -0.0]])
    q = oracle.quant_codes(w, float(s))
    for wi, qi in zip(w, q):
        best = None
        for c in range(-8, 8):
            err = abs(Fraction(float(wi)) - c * Fraction(float(s)))
            if best is None or err < best[0] or (err == best[0] and c % 2 == 0):
                best = (err, c)
        assert qi == best[1], (wi, qi, best)


def test_quantise_exact_grid_round_trips():
    # weights already on the grid q*s, with a +-7 in every group: quantising
    # gives back the same scales and codes
    rng = np.random.default_rng(11)
    n, k = 6, 256
    q = rng.integers(-7, 8, size=(n, k))
    q[:, ::64] = rng.choice([-7, 7], size=(n, k // 64))
    s = rng.uniform(0.004, 0.03, size=(n, k // 64)).astype(np.float16)
    w = q * np.repeat(s.astype(np.float64), 64, axis=1)
    codes, scales = oracle.quantize_gs64(w)
    assert np.array_equal(scales, s)
    assert np.array_equal(oracle.unpack_int4(codes), q)


def test_quantise_error_bound_and_zero_groups():
    rng = np.random.default_rng(12)
    w = synth.bf16_to_f32(synth.bf16_round(rng.standard_normal((8, 512)).astype(np.float32)))
    w[3, 64:128] = 0.0
    codes, scales = oracle.quantize_gs64(w)
    assert scales[3, 1] == 0 and not oracle.unpack_int4(codes)[3, 64:128].any()
    back = oracle.dequant(codes, scales)
    bound = np.repeat(scales.astype(np.float64), 64, axis=1) / 2
    assert np.all(np.abs(back - w) <= bound)
    # a group's largest magnitude maps to +-7
    q = oracle.unpack_int4(codes).reshape(8, 8, 64)
    assert np.all(np.max(np.abs(q), axis=2)[scales != 0] == 7)


def test_row_mode_is_group_mode_for_one_group_per_row():
    rng = np.random.default_rng(13)
    w = rng.standard_normal((5, 64)).astype(np.float32)
    c1, s1 = oracle.quantize_rows(w)
    c2, s2 = oracle.quantize_gs64(w)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2[:, 0])


def test_group_scales_beat_one_scale_per_row_on_gaussian_weights():
    # the kind of comparison the pages make (yunpan.plus, "capability 4";
    # ssnai.com digest, caveats): gs64 keeps more of a Gaussian matrix than one
    # scale per row
    rng = np.random.default_rng(14)
    w = rng.standard_normal((64, 2048))
    cg, sg = oracle.quantize_gs64(w)
    cr, sr = oracle.quantize_rows(w)
    eg = np.linalg.norm(oracle.dequant(cg, sg) - w)
    er = np.linalg.norm(oracle.unpack_int4(cr) * sr.astype(np.float64)[:, None] - w)
    assert eg < er
