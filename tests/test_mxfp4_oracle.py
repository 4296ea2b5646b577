"""Pins of the MXFP4 oracle (oracle/mxfp4.py) against the OCP MX v1.0
specification's tables (tests/golden/mxfp4_e2m1.json), exact-fraction brute
force and dense evaluation; CPU only."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import moe_oracle as oracle
from oracle import mxfp4 as mx

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mxfp4_e2m1.json")))
E2M1 = [GOLD["e2m1"][str(c)] for c in range(16)]


def test_e2m1_codes_match_the_specification_table():
    got = mx.decode_e2m1(np.arange(16))
    assert np.array_equal(got, np.array(E2M1))
    assert np.signbit(got[8]) and not np.signbit(got[0])      # -0 and +0
    assert GOLD["block_size"] == mx.MX_BLOCK


def test_e8m0_scales_match_the_specification():
    got = mx.decode_e8m0([0, 126, 127, 128, 254, 255])
    assert got[0] == 2.0 ** -127 and got[4] == 2.0 ** 127
    assert list(got[1:4]) == [GOLD["e8m0"]["126"], GOLD["e8m0"]["127"], GOLD["e8m0"]["128"]]
    assert np.isnan(got[5])


def test_dequant_of_a_hand_built_block():
    # one row of 64 elements = two blocks; element 2j in the low nibble of byte j
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, 0] = 0x71          # elements 0, 1: codes 1 (0.5), 7 (6)
    codes[0, 1] = 0xF9          # elements 2, 3: codes 9 (-0.5), 15 (-6)
    codes[0, 16] = 0x35         # elements 32, 33: codes 5 (3), 3 (1.5)
    scales = np.array([[125, 129]], dtype=np.uint8)           # 0.25, 4
    w = mx.dequant(codes, scales)
    assert list(w[0, :4]) == [0.125, 1.5, -0.125, -1.5]
    assert list(w[0, 32:34]) == [12.0, 6.0]
    assert np.count_nonzero(w[0, 4:32]) == 0 and np.count_nonzero(w[0, 34:]) == 0


def _spec_quantize_block(vals):
    """The specification's conversion for one block, in exact fractions:
    X = 2^(floor(log2 max|v|) - 2); each v / X to the nearest E2M1 value,
    ties to the even mantissa, saturating at 6."""
    vals = [Fraction(float(v)) for v in vals]
    amax = max(abs(v) for v in vals)
    if amax == 0:
        return 0, [0] * len(vals)
    p = 0                                   # largest p with 2^p <= amax
    while Fraction(2) ** (p + 1) <= amax:
        p += 1
    while Fraction(2) ** p > amax:
        p -= 1
    e = min(max(p - 2 + 127, 0), 254)
    X = Fraction(2) ** (e - 127)
    mags = [Fraction(GOLD["e2m1"][str(c)]) for c in range(8)]
    codes = []
    for v in vals:
        r = min(abs(v) / X, Fraction(6))
        best = min(abs(r - m) for m in mags)
        near = [c for c in range(8) if abs(r - mags[c]) == best]
        c = near[0] if len(near) == 1 else [c for c in near if c % 2 == 0][0]
        codes.append(c + 8 if (v < 0 and c > 0) else c)
    return e, codes


def test_quantizer_matches_exact_brute_force():
    rng = np.random.default_rng(5)
    w = rng.standard_normal((6, 64)) * np.exp2(rng.integers(-6, 3, size=(6, 1)))
    w[0, :32] = 0.0                                           # an all-zero block
    w[1, 5] = 7.0 * np.max(np.abs(w[1, :32]))                 # forces saturation
    # exact half-way points: with X = 1 (block max in [4, 8)), 0.25, 0.75, 1.25,
    # 1.75, 2.5, 3.5 and 5 lie half-way between two E2M1 values
    w[2, 32:40] = [4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    w[2, 40:64] = 0.5
    codes, scales = mx.quantize(w)
    q = mx.unpack_nibbles(codes)
    for r in range(w.shape[0]):
        for b in range(w.shape[1] // 32):
            e, c = _spec_quantize_block(w[r, 32 * b:32 * b + 32])
            assert int(scales[r, b]) == e, (r, b)
            assert list(q[r, 32 * b:32 * b + 32]) == c, (r, b)


def test_quantizer_grid_round_trip_and_error_bound():
    rng = np.random.default_rng(6)
    q = rng.choice([c for c in range(16) if c != 8], size=(4, 128))   # no -0
    q[:, ::32] = 7                                              # every block holds +6
    e = rng.integers(110, 140, size=(4, 4)).astype(np.uint8)
    w = mx.dequant(mx.pack_nibbles(q), e)
    codes, scales = mx.quantize(w)
    assert np.array_equal(scales, e)
    assert np.array_equal(mx.unpack_nibbles(codes), q)
    # off the grid: within one spacing of the top interval (X), and the block
    # maximum scales into [4, 8)
    g = rng.standard_normal((8, 256))
    codes, scales = mx.quantize(g)
    X = np.repeat(mx.decode_e8m0(scales), 32, axis=1)
    back = mx.dequant(codes, scales)
    unsat = np.abs(g) <= 6 * X
    assert np.all(np.abs(back - g)[unsat] <= X[unsat])
    amax = np.max(np.abs(g.reshape(8, 8, 32)), axis=2) / mx.decode_e8m0(scales)
    assert np.all((amax >= 4) & (amax < 8))


def test_block_has_the_int4_containers_size():
    for d, f in ((512, 256), (6144, 2048)):
        assert mx.block_bytes(d, f) == oracle.expert_block_bytes(d, f)


def _dense_masked_table(x, w_router, bias, blocks, shared, d, f, E, k, idx, wts):
    """Every expert for every token, gates zero outside the chosen k; blocks
    decoded through the specification's table (torch float64)."""
    table = torch.tensor(E2M1, dtype=torch.float64)

    def mats(blk):
        b = torch.from_numpy(np.asarray(blk, dtype=np.uint8).copy()).to(torch.int64)
        out, qpos, spos = [], 0, 3 * d * f // 2
        for rows, cols in ((f, d), (f, d), (d, f)):
            qb = b[qpos:qpos + rows * cols // 2].reshape(rows, cols // 2)
            codes = torch.stack([qb & 15, qb >> 4], dim=2).reshape(rows, cols)
            eb = b[spos:spos + rows * cols // 32].reshape(rows, cols // 32).to(torch.float64)
            out.append(table[codes] * torch.pow(2.0, eb - 127.0).repeat_interleave(32, dim=1))
            qpos += rows * cols // 2
            spos += rows * cols // 32
        return out

    xt = torch.from_numpy(np.asarray(x, dtype=np.float64))
    T = xt.shape[0]
    gate = torch.zeros((T, E), dtype=torch.float64)
    for t in range(T):
        for j in range(k):
            gate[t, int(idx[t, j])] = float(wts[t, j])
    out = torch.zeros((T, d), dtype=torch.float64)
    for e in range(E):
        Wg, Wu, Wd = mats(blocks[e])
        h = torch.nn.functional.silu(xt @ Wg.T) * (xt @ Wu.T)
        out += gate[:, e:e + 1] * (h @ Wd.T)
    if shared is not None:
        Wg, Wu, Wd = mats(shared)
        out += (torch.nn.functional.silu(xt @ Wg.T) * (xt @ Wu.T)) @ Wd.T
    return out.numpy()


@pytest.mark.parametrize("with_shared", [False, True])
def test_mxfp4_layer_equals_dense_masked_gates(with_shared):
    rng = np.random.default_rng(10 + with_shared)
    d, f, E, k, T = 128, 64, 6, 2, 5
    bb = mx.block_bytes(d, f)
    nq = 3 * d * f // 2
    blocks = np.zeros((E + 1, bb), dtype=np.uint8)
    for e in range(E + 1):
        blocks[e, :nq] = rng.integers(0, 256, nq, dtype=np.uint8)
        blocks[e, nq:] = rng.integers(118, 125, bb - nq, dtype=np.uint8)   # 2^-9 .. 2^-3
    shared = blocks[E] if with_shared else None
    x = rng.standard_normal((T, d)).astype(np.float32)
    w = (rng.standard_normal((E, d)) * 0.2).astype(np.float32)
    res = oracle.moe_layer(x, w, None, blocks[:E], shared, d, f, E, k, weights=mx.expert_weights)
    dense = _dense_masked_table(x, w, None, blocks[:E], shared, d, f, E, k,
                                res["topk_idx"], res["topk_w"])
    assert np.max(np.abs(res["out"] - dense)) <= 1e-12 * np.max(np.abs(dense))
