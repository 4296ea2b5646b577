"""GPU parity: every step of the layer through the C ABI against the CPU
oracle on the same seeded inputs.

Routing indices and the batch-union grouping must match bit-exactly; gate
weights within 1e-6; expert outputs and the layer output within
2e-3 * rms(reference) on the float32 decode path.  Workloads run at their
full sizes; where the oracle would need minutes (the 8-token decode batch of
the ~19 MB-expert layer touches ~57 experts) it computes sampled tokens one
by one instead.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import int4_routed_expert_logits_amd as moe
from int4_routed_expert_logits_amd.layer import LayerBuffers, run_layer, run_layer_decode
from oracle_rows import oracle_sampled, expert_rows, prefill_tiles

pytestmark = pytest.mark.gpu

DEC = moe.MOE_PATH_DECODE_F32
TOL_DECODE = 2e-3


def say(msg):
    print(msg, flush=True)


# ----------------------------------------------------------------------------
# inputs on the device
# ----------------------------------------------------------------------------

_layers = {}


def dev_layer(cfg, router_only=False):
    key = (cfg, router_only)
    if key not in _layers:
        if not router_only:
            for k in [k for k in _layers if not k[1]]:
                del _layers[k]
            torch.cuda.empty_cache()
        L = synth.make_layer(cfg, experts=[] if router_only else None)
        sh = moe.shape_of(L.shape)
        dev = dict(
            w_router=torch.from_numpy(L.w_router).cuda(),
            bias=None if L.bias is None else torch.from_numpy(L.bias).cuda(),
            experts=None if router_only else packed(sh, L.experts),
            shared=None if (router_only or L.shared is None) else packed(sh, L.shared[None])[0],
        )
        _layers[key] = (L, dev)
    return _layers[key]


def packed(sh, blocks):
    """Canonical host blocks [n, bytes] -> packed device blocks (moe_pack_experts)."""
    src = torch.from_numpy(np.ascontiguousarray(blocks)).cuda()
    dst = torch.empty_like(src)
    moe.moe_pack_experts(sh, src.shape[0], src, dst)
    torch.cuda.synchronize()
    del src
    return dst


def dev_x(bits):
    if bits.dtype == np.uint16:
        return torch.from_numpy(bits.view(np.int16).copy()).cuda().view(torch.bfloat16)
    return torch.from_numpy(bits.copy()).cuda()


def tokens(cfg, T, batch=0):
    bits, xf = synth.make_tokens(cfg, T, batch)
    return dev_x(bits), xf


def rel_err(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref))) / max(rms, 1e-300)


def min_gap(logits, k):
    s = -np.sort(-logits, axis=1)
    return float(np.min(s[:, k - 1] - s[:, k])) if logits.shape[1] > k else float("inf")


# ----------------------------------------------------------------------------
# router
# ----------------------------------------------------------------------------

# (1, 100): float32 x on the matrix-core path (more than 32 tokens)
ROUTE_CASES = [(1, 4), (1, 3), (1, 100), (2, 1), (2, 16), (3, 64), (3, 5), (4, 1), (4, 8), (4, 33),
               (5, 2048)]


@pytest.mark.parametrize("cfg,T", ROUTE_CASES)
def test_route_parity(cfg, T):
    say(f"route cfg={cfg} T={T}")
    L, dev = dev_layer(cfg, router_only=True)
    x, xf = tokens(cfg, T)
    sh = moe.shape_of(L.shape)
    k = sh.top_k
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_route_workspace_bytes(sh, T), dtype=torch.uint8, device="cuda")
    moe.moe_route(sh, x, dev["w_router"], dev["bias"], idx, w, ws)
    torch.cuda.synchronize()
    ridx, rw, lg = oracle.route(xf, L.w_router, L.bias, k)
    gap = min_gap(lg, k)
    assert np.array_equal(idx.cpu().numpy(), ridx), f"top-k differs (smallest k/k+1 logit gap {gap:.3e})"
    assert np.max(np.abs(w.cpu().numpy() - rw)) <= 1e-6
    # the gpu logits themselves (float64, summation order aside): the workspace
    # holds P partial sums per (token, expert); their in-order sum plus the
    # bias is the logit
    P = route_parts(T, sh.d, sh.n_experts)
    part = ws[: T * sh.n_experts * P * 8].view(torch.float64).cpu().numpy().reshape(T, sh.n_experts, P)
    glg = part[:, :, 0].copy()
    for p in range(1, P):
        glg += part[:, :, p]
    if L.bias is not None:
        glg += L.bias.astype(np.float64)
    assert np.max(np.abs(glg - lg)) <= 1e-12 * max(1.0, np.max(np.abs(lg)))


@pytest.mark.parametrize("T", [1, 7, 40])
def test_route_parity_largest_router(T):
    """The largest router the library takes: E = 1024 experts, top_k = 32,
    d = 8192, with a router bias; T = 1 and 7 on the split kernel, 40 on
    the matrix-core kernel, and the top-k kernels' form for E > 512.  Then
    moe_union on the routing, all against the oracle."""
    say(f"route E=1024 k=32 d=8192 T={T}")
    E, k, d = 1024, 32, 8192
    rng = np.random.default_rng(8192 + T)
    xb = synth.bf16_round(rng.standard_normal((T, d)).astype(np.float32))
    xf = synth.bf16_to_f32(xb)
    wr = (rng.standard_normal((E, d)) * 0.02).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
    sh = moe.Shape(d, 64, E, k, 64, 0)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_route_workspace_bytes(sh, T), dtype=torch.uint8, device="cuda")
    moe.moe_route(sh, dev_x(xb), torch.from_numpy(wr).cuda(), torch.from_numpy(bias).cuda(),
                  idx, w, ws)
    torch.cuda.synchronize()
    ridx, rw, lg = oracle.route(xf, wr, bias, k)
    gap = min_gap(lg, k)
    assert np.array_equal(idx.cpu().numpy(), ridx), f"top-k differs (smallest k/k+1 logit gap {gap:.3e})"
    assert np.max(np.abs(w.cpu().numpy() - rw)) <= 1e-6
    check_union(ridx, E)


def route_parts(T, d, E):
    """Parts of d per router logit; mirrors the library's host rule."""
    cap = 16 if E <= 256 else (8 if E <= 512 else 4)
    if T <= 32:
        P = min(2048 // E, d // 256)
    else:
        P = d // 768
    return max(1, min(P, cap))


def _route_fine(E, k, T=1):
    """Logits 1 + e*2^-30 (exact in float64, all equal after rounding to
    float32), so only the float64 comparison can order them."""
    sh = moe.Shape(64, 64, E, k, 64, 0)
    x = torch.zeros((T, 64), dtype=torch.float32, device="cuda")
    x[:, 0] = 1.0
    x[:, 1] = 2.0 ** -30
    wr = torch.zeros((E, 64), dtype=torch.float32, device="cuda")
    wr[:, 0] = 1.0
    wr[:, 1] = torch.arange(E, dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_route_workspace_bytes(sh, T), dtype=torch.uint8, device="cuda")
    moe.moe_route(sh, x, wr, None, idx, w, ws)
    torch.cuda.synchronize()
    ridx, rw, _ = oracle.route(x.cpu().numpy(), wr.cpu().numpy(), None, k)
    return idx.cpu().numpy(), w.cpu().numpy(), ridx, rw


def test_route_float64_order_below_float32_resolution():
    """64 experts whose float32 keys all tie: the candidate ranking decides."""
    say("route fine float64 order, E=64")
    idx, w, ridx, rw = _route_fine(64, 4)
    assert idx.tolist() == [[63, 62, 61, 60]]
    assert np.array_equal(idx, ridx) and np.max(np.abs(w - rw)) <= 1e-6


def test_route_mass_tie_fallback():
    """More than 64 experts share the float32 cut: the exact argmax rounds."""
    say("route mass tie, E=100")
    idx, w, ridx, rw = _route_fine(100, 8, T=3)
    assert idx.tolist() == [list(range(99, 91, -1))] * 3
    assert np.array_equal(idx, ridx) and np.max(np.abs(w - rw)) <= 1e-6
    # all-equal logits: lowest ids win, equal weights
    sh = moe.Shape(64, 64, 128, 8, 64, 0)
    x = torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros((128, 64), dtype=torch.float32, device="cuda")
    idx = torch.empty((2, 8), dtype=torch.int32, device="cuda")
    w = torch.empty((2, 8), dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_route_workspace_bytes(sh, 2), dtype=torch.uint8, device="cuda")
    moe.moe_route(sh, x, wr, None, idx, w, ws)
    torch.cuda.synchronize()
    assert idx.cpu().tolist() == [list(range(8))] * 2
    assert np.allclose(w.cpu().numpy(), 0.125, atol=0)


def test_route_ties_go_to_lower_id():
    say("route ties")
    sh = moe.Shape(64, 64, 6, 3, 64, 0)
    x = torch.zeros((2, 64), dtype=torch.float32, device="cuda")
    wr = torch.zeros((6, 64), dtype=torch.float32, device="cuda")
    b = torch.tensor([0.0, 1.0, 1.0, 0.5, 1.0, 1.0], device="cuda")
    idx = torch.empty((2, 3), dtype=torch.int32, device="cuda")
    w = torch.empty((2, 3), dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_route_workspace_bytes(sh, 2), dtype=torch.uint8, device="cuda")
    moe.moe_route(sh, x, wr, b, idx, w, ws)
    torch.cuda.synchronize()
    assert idx.cpu().tolist() == [[1, 2, 4], [1, 2, 4]]
    assert np.allclose(w.cpu().numpy(), 1.0 / 3.0, atol=1e-7)


# ----------------------------------------------------------------------------
# batch-union
# ----------------------------------------------------------------------------

def run_union(topk, E):
    T, k = topk.shape
    sh = moe.Shape(64, 64, E, k, 64, 0)
    i32 = dict(dtype=torch.int32, device="cuda")
    n = max(T * k, 1)
    outs = dict(counts=torch.full((E,), -7, **i32), offsets=torch.full((E + 1,), -7, **i32),
                perm=torch.full((n,), -7, **i32), inv_perm=torch.full((n,), -7, **i32),
                active=torch.full((E,), -7, **i32), n_active=torch.full((1,), -7, **i32))
    ti = torch.from_numpy(np.ascontiguousarray(topk, dtype=np.int32)).cuda() if T else None
    moe.moe_union(sh, T, ti, outs["counts"], outs["offsets"], outs["perm"], outs["inv_perm"],
                  outs["active"], outs["n_active"])
    torch.cuda.synchronize()
    return {k_: v.cpu().numpy() for k_, v in outs.items()}


def check_union(topk, E):
    got = run_union(topk, E)
    counts, offsets, perm, inv, active, n_active = oracle.batch_union(topk, E)
    n = topk.size
    assert np.array_equal(got["counts"], counts)
    assert np.array_equal(got["offsets"], offsets)
    assert np.array_equal(got["n_active"], n_active)
    assert np.array_equal(got["active"], active)
    g = int(offsets[E])
    assert np.array_equal(got["perm"][:g], perm[:g])
    assert np.array_equal(got["inv_perm"][:n], inv)


@pytest.mark.parametrize("cfg,T", [(1, 4), (2, 16), (3, 64), (4, 8), (5, 2048)])
def test_union_parity_on_workload_routing(cfg, T):
    say(f"union cfg={cfg} T={T}")
    L, _ = dev_layer(cfg, router_only=True)
    _, xf = synth.make_tokens(cfg, T)
    idx, _, _ = oracle.route(xf, L.w_router, L.bias, L.shape.top_k)
    check_union(idx, L.shape.n_experts)


# (65, 1, ...): one slot past the one-wavefront kernel; (3000, 6, ...) and
# (6250, 8, ...): wavefront ranges longer than one block of held keys
@pytest.mark.parametrize("T,k,E,seed", [(1, 1, 1, 0), (1000, 1, 8, 1), (100, 32, 1024, 2),
                                        (777, 8, 256, 3), (3000, 6, 40, 4), (513, 2, 3, 5),
                                        (65, 1, 7, 6), (6250, 8, 256, 7)])
def test_union_parity_random(T, k, E, seed):
    say(f"union random T={T} k={k} E={E}")
    rng = np.random.default_rng(seed)
    topk = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    check_union(topk, E)


# (8, 5): E = 4; (9, 1), (9, 3): E = 1024, top-32 (the two-kernel form)
@pytest.mark.parametrize("cfg,T", [(1, 4), (2, 1), (2, 8), (2, 9), (2, 16), (3, 64), (4, 1),
                                   (4, 8), (8, 5), (9, 1), (9, 3)])
def test_route_union_equals_route_then_union(cfg, T):
    """moe_route_union (one kernel for top-k + grouping up to 8 tokens) gives
    exactly moe_route's and moe_union's outputs."""
    say(f"route_union cfg={cfg} T={T}")
    L, dev = dev_layer(cfg, router_only=True)
    x, _ = tokens(cfg, T, 1)
    sh = moe.shape_of(L.shape)
    a = LayerBuffers.allocate(sh, T, DEC)
    b = LayerBuffers.allocate(sh, T, DEC)
    moe.moe_route(sh, x, dev["w_router"], dev["bias"], a.topk_idx, a.topk_w, a.workspace)
    moe.moe_union(sh, T, a.topk_idx, a.counts, a.offsets, a.perm, a.inv_perm, a.active,
                  a.n_active)
    moe.moe_route_union(sh, x, dev["w_router"], dev["bias"], b.topk_idx, b.topk_w, b.counts,
                        b.offsets, b.perm, b.inv_perm, b.active, b.n_active, b.workspace)
    torch.cuda.synchronize()
    n = T * sh.top_k
    for name in ("topk_idx", "topk_w", "counts", "offsets", "active", "n_active"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    assert torch.equal(a.perm[:n], b.perm[:n]) and torch.equal(a.inv_perm[:n], b.inv_perm[:n])


def test_route_union_empty_batch():
    say("route_union empty batch")
    L, dev = dev_layer(1, router_only=True)
    sh = moe.shape_of(L.shape)
    b = LayerBuffers.allocate(sh, 0, DEC)
    b.counts.fill_(7)
    b.n_active.fill_(7)
    x = torch.empty((0, sh.d), dtype=torch.float32, device="cuda")
    moe.moe_route_union(sh, x, dev["w_router"], None, b.topk_idx, b.topk_w, b.counts, b.offsets,
                        b.perm, b.inv_perm, b.active, b.n_active, b.workspace)
    torch.cuda.synchronize()
    assert not b.counts.any() and int(b.n_active.item()) == 0


def test_union_all_slots_to_one_expert():
    say("union single expert")
    check_union(np.full((4096, 1), 5, dtype=np.int32), 8)


def test_union_skips_out_of_range_ids():
    say("union invalid ids")
    topk = np.array([[2, 9], [-1, 1], [2, 1], [3, 0]], dtype=np.int32)
    check_union(topk, 4)


def test_union_empty_batch():
    say("union empty")
    got = run_union(np.zeros((0, 4), dtype=np.int32), 16)
    assert np.all(got["counts"] == 0) and np.all(got["offsets"] == 0)
    assert got["n_active"][0] == 0 and np.all(got["active"] == -1)


# ----------------------------------------------------------------------------
# combine
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("ybf16,obf16,shared", [(False, False, True), (False, False, False),
                                               (True, True, True), (False, True, True)])
def test_combine_parity(ybf16, obf16, shared):
    say(f"combine ybf16={ybf16} obf16={obf16} shared={shared}")
    rng = np.random.default_rng(11)
    T, k, d, E = 37, 8, 640, 64
    topk = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    _, _, _, inv, _, _ = oracle.batch_union(topk, E)
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    y = rng.standard_normal((T * k, d)).astype(np.float32)
    ys = rng.standard_normal((T, d)).astype(np.float32) if shared else None
    ydt = torch.bfloat16 if ybf16 else torch.float32
    yd = torch.from_numpy(y).cuda().to(ydt)
    ysd = torch.from_numpy(ys).cuda().to(ydt) if shared else None
    out = torch.empty((T, d), dtype=torch.bfloat16 if obf16 else torch.float32, device="cuda")
    sh = moe.Shape(d, 64, E, k, 64, 64 if shared else 0)
    moe.moe_combine(sh, yd, ysd, torch.from_numpy(inv).cuda(), torch.from_numpy(w).cuda(), out)
    torch.cuda.synchronize()
    yr = yd.float().cpu().numpy()
    ysr = ysd.float().cpu().numpy() if shared else None
    ref = oracle.combine(yr, ysr, inv, w, k)
    got = out.float().cpu().numpy()
    if obf16:
        # round-to-nearest bf16 output: within half an ulp, at most 2^-8 |v|
        rms = np.sqrt(np.mean(ref ** 2))
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5 * rms)
    else:
        assert rel_err(got, ref) <= 1e-6


# ----------------------------------------------------------------------------
# whole layer, decode path
# ----------------------------------------------------------------------------

def gpu_layer(cfg, T, batch=0, path=DEC, experts_override=None, fused=False):
    L, dev = dev_layer(cfg)
    x, xf = tokens(cfg, T, batch)
    sh = moe.shape_of(L.shape)
    buf = LayerBuffers.allocate(sh, T, path)
    ex = dev["experts"] if experts_override is None else experts_override
    run = run_layer_decode if fused else run_layer
    run(x, dev["w_router"], dev["bias"], ex, dev["shared"], buf)
    torch.cuda.synchronize()
    return L, xf, buf


def check_routing_and_union(buf, ref_idx, ref_w, union):
    counts, offsets, perm, inv, active, n_active = union
    assert np.array_equal(buf.topk_idx.cpu().numpy(), ref_idx)
    assert np.max(np.abs(buf.topk_w.cpu().numpy() - ref_w)) <= 1e-6
    assert np.array_equal(buf.counts.cpu().numpy(), counts)
    assert np.array_equal(buf.offsets.cpu().numpy(), offsets)
    n = ref_idx.size
    assert np.array_equal(buf.perm.cpu().numpy()[:n], perm)
    assert np.array_equal(buf.inv_perm.cpu().numpy()[:n], inv)
    assert np.array_equal(buf.active.cpu().numpy(), active)
    assert np.array_equal(buf.n_active.cpu().numpy(), n_active)


# (8, 1), (8, 5): d = f = 64, the smallest sizes taken; (9, 1), (9, 3): 1024
# experts, top-32 (the separate calls only: moe_layer_decode takes E <= 256)
FULL_CASES = [(1, 4), (1, 3), (2, 1), (2, 16), (2, 5), (3, 64), (3, 13), (4, 1), (6, 8), (6, 37),
              (8, 1), (8, 5), (9, 1), (9, 3)]


# the separate calls, and (batches of at most 8 tokens) the one-call moe_layer_decode
@pytest.mark.parametrize("cfg,T,fused", [(c, T, f) for c, T in FULL_CASES
                                         for f in ((False, True) if T <= 8 and c != 9 else (False,))])
def test_layer_decode_parity(cfg, T, fused):
    say(f"layer decode cfg={cfg} T={T} fused={fused}")
    L, xf, buf = gpu_layer(cfg, T, fused=fused)
    sh = L.shape
    ref = oracle.moe_layer(xf, L.w_router, L.bias, L.experts, L.shared, sh.d, sh.f,
                           sh.n_experts, sh.top_k)
    check_routing_and_union(buf, ref["topk_idx"], ref["topk_w"],
                            (ref["counts"], ref["offsets"], ref["perm"], ref["inv_perm"],
                             ref["active"], ref["n_active"]))
    ey = rel_err(buf.y.cpu().numpy()[: T * sh.top_k], ref["y"])
    assert ey <= TOL_DECODE, f"y error {ey:.2e} rms"
    if L.shared is not None:
        es = rel_err(buf.y_shared.cpu().numpy()[:T], ref["y_shared"])
        assert es <= TOL_DECODE, f"y_shared error {es:.2e} rms"
    eo = rel_err(buf.out.cpu().numpy(), ref["out"])
    assert eo <= TOL_DECODE, f"out error {eo:.2e} rms"


def test_layer_decode_parity_19mb_layer_8_tokens_sampled():
    say("layer decode cfg=4 T=8 (sampled)")
    L, xf, buf = gpu_layer(4, 8)
    ref = oracle_sampled(L, xf, [0, 5])
    check_routing_and_union(buf, ref["topk_idx"], ref["topk_w"], ref["union"])
    y = buf.y.cpu().numpy()
    ys = np.stack(list(ref["y"].values()))
    got = np.stack([y[p] for p in ref["y"]])
    assert rel_err(got, ys) <= TOL_DECODE
    out = buf.out.cpu().numpy()
    ro = np.stack([ref["out"][t] for t in sorted(ref["out"])])
    assert rel_err(out[sorted(ref["out"])], ro) <= TOL_DECODE


LAYER_OUTPUTS = ("topk_idx", "topk_w", "counts", "offsets", "perm", "inv_perm", "active",
                 "n_active", "y", "y_shared", "out")


@pytest.mark.parametrize("cfg,T,out_bf16", [(1, 4, False), (1, 3, True), (2, 1, False),
                                            (2, 8, False), (2, 5, True), (3, 8, False),
                                            (3, 1, False), (4, 1, False), (4, 2, False),
                                            (4, 3, True), (4, 4, False), (4, 8, True)])
def test_layer_decode_call_equals_the_separate_calls(cfg, T, out_bf16):
    """moe_layer_decode writes every output of route_union + expert_ffn +
    combine, bit for bit (the same function computed with fewer launches)."""
    say(f"moe_layer_decode vs separate calls cfg={cfg} T={T} out_bf16={out_bf16}")
    L, dev = dev_layer(cfg)
    x, _ = tokens(cfg, T)
    sh = moe.shape_of(L.shape)
    odt = torch.bfloat16 if out_bf16 else None
    a = LayerBuffers.allocate(sh, T, DEC, out_dtype=odt)
    b = LayerBuffers.allocate(sh, T, DEC, out_dtype=odt)
    for t in (a.y, b.y):  # rows of unused positions are never written: same filler
        t.fill_(0.0)
    run_layer(x, dev["w_router"], dev["bias"], dev["experts"], dev["shared"], a)
    run_layer_decode(x, dev["w_router"], dev["bias"], dev["experts"], dev["shared"], b)
    torch.cuda.synchronize()
    n = T * sh.top_k
    for name in LAYER_OUTPUTS:
        ta, tb = getattr(a, name), getattr(b, name)
        if ta is None:
            assert tb is None
            continue
        if name in ("perm", "inv_perm", "y"):
            ta, tb = ta[:n], tb[:n]
        assert torch.equal(ta.cpu(), tb.cpu()), name


def test_layer_decode_mtp_verify_batch_sampled():
    """A multi-token-prediction verify batch (3 tokens: the pages' 2.2-2.8
    tokens per forward) of the 19 MB-expert layer through moe_layer_decode:
    routing and grouping exact, every expert output and layer output of all
    three tokens against the oracle."""
    say("moe_layer_decode MTP verify batch cfg=4 T=3")
    L, xf, buf = gpu_layer(4, 3, fused=True)
    ref = oracle_sampled(L, xf, [0, 1, 2])
    check_routing_and_union(buf, ref["topk_idx"], ref["topk_w"], ref["union"])
    y = buf.y.cpu().numpy()
    got = np.stack([y[p] for p in ref["y"]])
    assert rel_err(got, np.stack(list(ref["y"].values()))) <= TOL_DECODE
    assert rel_err(buf.out.cpu().numpy(), np.stack([ref["out"][t] for t in range(3)])) <= TOL_DECODE


@pytest.mark.parametrize("cfg,T", [(2, 1), (4, 1), (4, 3)])
def test_layer_decode_call_replays_in_a_hip_graph(cfg, T):
    """The benchmark's form of the decode step: moe_layer_decode captured in a
    HIP graph and replayed, each replay on new tokens copied into the
    captured input buffer, with eager work and synchronisations between the
    replays; every replay's outputs equal an eager call's on the same tokens,
    bit for bit."""
    say(f"moe_layer_decode in a HIP graph cfg={cfg} T={T}")
    L, dev = dev_layer(cfg)
    sh = moe.shape_of(L.shape)
    xs = [tokens(cfg, T, batch=b)[0] for b in range(4)]
    x_in = xs[0].clone()
    g_buf = LayerBuffers.allocate(sh, T, DEC)
    run = lambda buf, x: run_layer_decode(x, dev["w_router"], dev["bias"], dev["experts"],
                                          dev["shared"], buf)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        run(g_buf, x_in)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(g_buf, x_in)
    torch.cuda.synchronize()
    for rep, x in enumerate([xs[1], xs[2], xs[1], xs[3]]):
        e_buf = LayerBuffers.allocate(sh, T, DEC)
        run(e_buf, x)  # eager, on the same tokens
        torch.cuda.synchronize()
        x_in.copy_(x)
        graph.replay()
        torch.cuda.synchronize()
        n = T * sh.top_k
        for name in LAYER_OUTPUTS:
            ta, tb = getattr(e_buf, name), getattr(g_buf, name)
            if ta is None:
                continue
            if name in ("perm", "inv_perm", "y"):
                ta, tb = ta[:n], tb[:n]
            assert torch.equal(ta.cpu(), tb.cpu()), (rep, name)
    del graph


def test_layer_decode_call_reuses_its_workspace():
    say("moe_layer_decode workspace reuse")
    for cfg, T in ((4, 1), (2, 8)):
        L, dev = dev_layer(cfg)
        sh = moe.shape_of(L.shape)
        buf = LayerBuffers.allocate(sh, T, DEC)
        outs = []
        for batch in (0, 1, 0, 1):
            bits, _ = synth.make_tokens(cfg, T, batch=batch)
            run_layer_decode(dev_x(bits), dev["w_router"], dev["bias"], dev["experts"],
                             dev["shared"], buf)
            torch.cuda.synchronize()
            outs.append(buf.out.cpu().numpy().copy())
        assert np.isfinite(outs[0]).all()
        assert np.array_equal(outs[0], outs[2]) and np.array_equal(outs[1], outs[3])
        assert not np.array_equal(outs[0], outs[1])


def test_layer_decode_call_empty_batch():
    say("moe_layer_decode T=0")
    L, dev = dev_layer(2)
    sh = moe.shape_of(L.shape)
    buf = LayerBuffers.allocate(sh, 0, DEC)
    buf.counts.fill_(7)
    buf.n_active.fill_(7)
    x = torch.empty((0, sh.d), dtype=torch.bfloat16, device="cuda")
    run_layer_decode(x, dev["w_router"], dev["bias"], dev["experts"], dev["shared"], buf)
    torch.cuda.synchronize()
    assert int(buf.n_active.item()) == 0
    assert int(buf.counts.sum().item()) == 0
    assert int(buf.offsets[-1].item()) == 0


def test_decode_is_deterministic_and_batch_invariant():
    say("decode determinism / batch invariance")
    L, xf, buf1 = gpu_layer(2, 16)
    out1 = buf1.out.cpu().numpy().copy()
    _, _, buf2 = gpu_layer(2, 16)
    assert np.array_equal(out1, buf2.out.cpu().numpy())
    # each token alone gives bitwise the same row as inside the batch
    Ld, dev = dev_layer(2)
    bits, _ = synth.make_tokens(2, 16)
    sh = moe.shape_of(Ld.shape)
    for t in (0, 7, 15):
        b1 = LayerBuffers.allocate(sh, 1, DEC)
        run_layer(dev_x(bits[t:t + 1]), dev["w_router"], dev["bias"], dev["experts"], dev["shared"], b1)
        torch.cuda.synchronize()
        assert np.array_equal(b1.out.cpu().numpy()[0], out1[t])


def test_decode_reuses_its_workspace():
    """Back-to-back calls on one set of buffers, with another batch in
    between, repeat bit for bit (nothing carried over in the workspace)."""
    say("decode workspace reuse")
    for cfg, T in ((4, 1), (2, 16)):
        L, dev = dev_layer(cfg)
        sh = moe.shape_of(L.shape)
        buf = LayerBuffers.allocate(sh, T, DEC)
        outs = []
        for batch in (0, 1, 0, 1, 0):
            bits, _ = synth.make_tokens(cfg, T, batch=batch)
            run_layer(dev_x(bits), dev["w_router"], dev["bias"], dev["experts"], dev["shared"], buf)
            torch.cuda.synchronize()
            outs.append(buf.out.cpu().numpy().copy())
        assert np.isfinite(outs[0]).all()
        assert np.array_equal(outs[0], outs[2]) and np.array_equal(outs[0], outs[4])
        assert np.array_equal(outs[1], outs[3])
        assert not np.array_equal(outs[0], outs[1])


def test_doubling_down_scales_doubles_y():
    say("down-scale doubling")
    L, dev = dev_layer(1)
    sh = L.shape
    blocks = L.experts.copy()
    sd = 3 * sh.d * sh.f // 2 + 2 * sh.f * (sh.d // 64) * 2
    for e in range(sh.n_experts):
        s = blocks[e, sd:].view(np.float16)
        s *= np.float16(2.0)
    _, _, b1 = gpu_layer(1, 4)
    y1 = b1.y.cpu().numpy().copy()
    _, _, b2 = gpu_layer(1, 4, experts_override=packed(moe.shape_of(sh), blocks))
    assert np.array_equal(b2.y.cpu().numpy(), 2.0 * y1)


def test_empty_batch_is_a_no_op():
    say("empty batch")
    L, dev = dev_layer(1)
    sh = moe.shape_of(L.shape)
    buf = LayerBuffers.allocate(sh, 0, DEC)
    run_layer(torch.empty((0, sh.d), dtype=torch.float32, device="cuda"), dev["w_router"],
              dev["bias"], dev["experts"], dev["shared"], buf)
    torch.cuda.synchronize()
    assert int(buf.n_active.item()) == 0


# ----------------------------------------------------------------------------
# packed expert layout
# ----------------------------------------------------------------------------

def np_pack_block(blk, d, f):
    """The packed layout, restated with numpy reshapes: 64-row tiles, 32-column
    chunks of 16 bytes per row, nibble j of each 4-byte word moved to bit
    4*(j//2) + 16*(j%2) and stored as q + 8 (offset binary: the top bit of
    each two's-complement nibble flipped); scales in the same 64-row tiles,
    group-major."""
    blk = np.asarray(blk, dtype=np.uint8)
    out = np.empty_like(blk)
    s0 = 3 * d * f // 2
    mats = [(f, d, 0, s0), (f, d, f * d // 2, s0 + f * (d // 64) * 2),
            (d, f, f * d, s0 + 2 * f * (d // 64) * 2)]
    for N, K, qo, so in mats:
        nq = N * K // 2
        words = blk[qo:qo + nq].view("<u4").reshape(N // 64, 64, K // 32, 4).astype(np.uint64)
        new = np.zeros_like(words)
        for j in range(8):
            q = ((words >> np.uint64(4 * j)) & np.uint64(0xF)).astype(np.int64)
            q = np.where(q >= 8, q - 16, q)                        # two's-complement code
            new |= (q + 8).astype(np.uint64) << np.uint64(4 * (j // 2) + 16 * (j % 2))
        tiled = new.astype("<u4").transpose(0, 2, 1, 3)          # [tile][chunk][row][word]
        out[qo:qo + nq] = np.ascontiguousarray(tiled).view(np.uint8).reshape(-1)
        ns = N * (K // 64) * 2
        sc = blk[so:so + ns].view("<u2").reshape(N // 64, 64, K // 64).transpose(0, 2, 1)
        out[so:so + ns] = np.ascontiguousarray(sc).view(np.uint8).reshape(-1)
    return out


@pytest.mark.parametrize("d,f,n", [(128, 192, 3), (512, 256, 2), (6144, 2048, 1)])
def test_pack_matches_layout_definition(d, f, n):
    say(f"pack d={d} f={f} n={n}")
    rng = np.random.default_rng(d + f)
    bb = oracle.expert_block_bytes(d, f)
    blocks = rng.integers(0, 256, size=(n, bb), dtype=np.uint8)
    sh = moe.Shape(d, f, 8, 2, 64, 0)
    got = packed(sh, blocks).cpu().numpy()
    for b in range(n):
        assert np.array_equal(got[b], np_pack_block(blocks[b], d, f)), f"block {b}"


# ----------------------------------------------------------------------------
# whole layer, prefill path (bf16 MFMA grouped GEMM)
# ----------------------------------------------------------------------------

PRE = moe.MOE_PATH_PREFILL_BF16
TOL_PREFILL = 2e-2


# An ideal kernel that keeps h and y in bf16 (the prefill path's storage
# format) already reaches 1.6-2.5e-2 * rms at the worst element of the int4
# parity layers (float64 simulation), above the 2e-2 * rms of the
# arithmetic, so the bound is element-wise with the format's own rounding;
# the strict max|err| / rms is printed beside it.


def prefill_err(got, ref, name="", extra=None):
    """Largest error of a bf16 prefill output in units of the bound actually
    checked, element by element: 2e-2 * rms(ref) for the arithmetic plus
    half an ulp of the bf16 result at |ref| (at most 2^-8 * |ref|: outputs
    here reach ~6.5 rms, where that rounding alone is ~2.5e-2 rms), plus
    `extra` (per element) where a test adds an allowance; <= 1 passes.
    Prints the strict max|err| / rms(ref) and asserts the strict form of the
    same bound: max|err| <= 2e-2 * rms + 2^-8 * max|ref|."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    strict = float(np.max(np.abs(got - ref))) / rms
    allow = TOL_PREFILL * rms + 2.0 ** -8 * np.abs(ref)
    if extra is not None:
        allow = allow + np.asarray(extra, dtype=np.float64)
    bound = float(np.max(np.abs(got - ref) / allow))
    cap = TOL_PREFILL + 2.0 ** -8 * float(np.max(np.abs(ref))) / rms
    say(f"  {name}: strict max|err|/rms = {strict:.4f} (strict bound {cap:.4f}), "
        f"element-wise bound ratio = {bound:.3f}")
    assert strict <= cap, f"{name}: strict error {strict:.4f} * rms > {cap:.4f}"
    return bound
# (6, 512) and (6, 97): 128-row tiles (full and partial), odd group counts
# along d and f, partial column tiles, an unrouted expert
# (8, 5), (8, 300): d = f = 64 (one group along K, columns past the matrix);
# (9, 40): 1024 experts, top-32, 1025 slots (two chunks of the tile lists)
PREFILL_FULL = [(2, 16), (2, 5), (3, 64), (3, 13), (6, 512), (6, 97), (8, 5), (8, 300), (9, 40)]


@pytest.mark.parametrize("cfg,T", PREFILL_FULL)
def test_layer_prefill_parity(cfg, T):
    """bf16 x through route, union, the MFMA FFN and a bf16 combine, against
    the float64 oracle at the 2e-2 * rms bound of the bf16 path."""
    say(f"layer prefill cfg={cfg} T={T}")
    L, xf, buf = gpu_layer(cfg, T, path=PRE)
    sh = L.shape
    ref = oracle.moe_layer(xf, L.w_router, L.bias, L.experts, L.shared, sh.d, sh.f,
                           sh.n_experts, sh.top_k)
    check_routing_and_union(buf, ref["topk_idx"], ref["topk_w"],
                            (ref["counts"], ref["offsets"], ref["perm"], ref["inv_perm"],
                             ref["active"], ref["n_active"]))
    ey = prefill_err(buf.y.float().cpu().numpy()[: T * sh.top_k], ref["y"], "y")
    assert ey <= 1.0, f"y error {ey:.2f} x bound"
    if L.shared is not None:
        es = prefill_err(buf.y_shared.float().cpu().numpy()[:T], ref["y_shared"], "y_shared")
        assert es <= 1.0, f"y_shared error {es:.2f} x bound"
    eo = prefill_err(buf.out.float().cpu().numpy(), ref["out"], "out (bf16)")
    assert eo <= 1.0, f"out error {eo:.2f} x bound"
    # the same y combined into a float32 out: only y's bf16 storage and the
    # arithmetic remain
    out32 = torch.empty((T, sh.d), dtype=torch.float32, device="cuda")
    moe.moe_combine(moe.shape_of(sh), buf.y, buf.y_shared, buf.inv_perm, buf.topk_w, out32)
    torch.cuda.synchronize()
    e32 = prefill_err(out32.cpu().numpy(), ref["out"], "out (f32 combine)")
    assert e32 <= 1.0, f"out (f32) error {e32:.2f} x bound"


@pytest.mark.parametrize("cfg,T,sample", [(4, 40, [0, 17, 39]), (5, 2048, [0, 1000, 2047])])
def test_layer_prefill_parity_19mb_layer_sampled(cfg, T, sample):
    """The ~19 MB-expert layer: 40 tokens (many one-token experts) and the
    2048-token Zipf-routed batch (experts of up to ~1600 rows, the shared
    expert over all 2048); every expert output of the sampled tokens and
    their layer outputs against the oracle."""
    say(f"layer prefill cfg={cfg} T={T} (sampled {sample})")
    L, xf, buf = gpu_layer(cfg, T, path=PRE)
    ref = oracle_sampled(L, xf, sample)
    check_routing_and_union(buf, ref["topk_idx"], ref["topk_w"], ref["union"])
    y = buf.y.float().cpu().numpy()
    got = np.stack([y[p] for p in ref["y"]])
    assert prefill_err(got, np.stack(list(ref["y"].values())), "y") <= 1.0
    ysh = buf.y_shared.float().cpu().numpy()
    assert prefill_err(ysh[sample], np.stack([ref["y_shared"][t] for t in sample]),
                       "y_shared") <= 1.0
    out = buf.out.float().cpu().numpy()
    assert prefill_err(out[sample], np.stack([ref["out"][t] for t in sample]), "out") <= 1.0


def _largest_layer_check(T, path):
    L, xf, buf = gpu_layer(7, T, path=path)
    sh = L.shape
    ref = oracle_sampled(L, xf, list(range(T)))
    check_routing_and_union(buf, ref["topk_idx"], ref["topk_w"], ref["union"])
    pos = sorted(ref["y"])
    y = buf.y.float().cpu().numpy()
    ysh = buf.y_shared.float().cpu().numpy()
    out = buf.out.float().cpu().numpy()
    got = [y[pos], ysh[:T], out[:T]]
    want = [np.stack([ref["y"][p] for p in pos]), np.stack([ref["y_shared"][t] for t in range(T)]),
            np.stack([ref["out"][t] for t in range(T)])]
    return L, buf, got, want


@pytest.mark.timeout(600)
def test_layer_decode_parity_largest_layer():
    """d = f = 8192 (the largest sizes the library takes) on the decode path,
    through the separate calls and through moe_layer_decode: every output of
    the 3-token batch against the oracle."""
    say("layer decode cfg=7 (d = f = 8192) T=3")
    _, _, got, want = _largest_layer_check(3, DEC)
    for g, r, name in zip(got, want, ("y", "y_shared", "out")):
        e = rel_err(g, r)
        say(f"  {name}: max|err|/rms = {e:.2e}")
        assert e <= TOL_DECODE, name
    L, dev = dev_layer(7)
    x, _ = tokens(7, 3)
    sh = moe.shape_of(L.shape)
    a = LayerBuffers.allocate(sh, 3, DEC)
    b = LayerBuffers.allocate(sh, 3, DEC)
    run_layer(x, dev["w_router"], dev["bias"], dev["experts"], dev["shared"], a)
    run_layer_decode(x, dev["w_router"], dev["bias"], dev["experts"], dev["shared"], b)
    torch.cuda.synchronize()
    assert torch.equal(a.out, b.out) and torch.equal(a.y_shared, b.y_shared)


@pytest.mark.timeout(600)
def test_layer_prefill_parity_largest_layer():
    """d = f = 8192 on the prefill path: 160 tokens, whose Zipf routing gives
    an expert of more than 96 rows and the shared expert's 160 (128-row tiles
    and 32-row tiles, 128 groups along K); every output against the oracle."""
    say("layer prefill cfg=7 (d = f = 8192) T=160")
    L, buf, got, want = _largest_layer_check(160, PRE)
    counts = buf.counts.cpu().numpy()
    say(f"  rows per expert {counts.tolist()}")
    assert counts.max() >= 96  # a 128-row tile of a routed expert
    for g, r, name in zip(got, want, ("y", "y_shared", "out")):
        assert prefill_err(g, r, name) <= 1.0


@pytest.mark.timeout(900)
def test_layer_prefill_parity_2048_every_tile():
    """The 2048-token Zipf-routed batch of the ~19 MB-expert layer at full
    size: the first and the last row of every 128-row and every 32-row M-tile
    of every expert (and of the shared expert's tiles), plus every row of the
    heaviest expert and of the one-row experts, against the oracle."""
    say("layer prefill cfg=5 T=2048, every tile's first and last row")
    L, xf, buf = gpu_layer(5, 2048, path=PRE)
    sh = L.shape
    idx, w, _ = oracle.route(xf, L.w_router, L.bias, sh.top_k)
    union = oracle.batch_union(idx, sh.n_experts)
    counts, offsets, perm, inv, active, n_active = union
    check_routing_and_union(buf, idx, w, union)
    requests, positions = {}, []
    heavy = int(np.argmax(counts))
    n_tiles = 0
    for a in range(int(n_active[0])):
        e = int(active[a])
        lo, M = int(offsets[e]), int(counts[e])
        tiles = prefill_tiles(M)
        n_tiles += len(tiles)
        rows = sorted({r for t in tiles for r in t}) if e != heavy and M > 1 else range(M)
        for r in rows:
            p = lo + r
            positions.append((e, p, int(perm[p]) // sh.top_k))
            requests.setdefault(e, []).append(int(perm[p]) // sh.top_k)
    shared_rows = sorted({r for t in prefill_tiles(2048) for r in t})
    requests["shared"] = shared_rows
    say(f"  {n_tiles} routed M-tiles over {int(n_active[0])} experts, {len(positions)} rows; "
        f"heaviest expert {heavy} with {int(counts[heavy])} rows")
    rows = expert_rows(L, xf, requests)
    y = buf.y.float().cpu().numpy()
    got = np.stack([y[p] for _, p, _ in positions])
    ref = np.stack([rows[(e, t)] for e, _, t in positions])
    assert prefill_err(got, ref, "y (tile rows)") <= 1.0
    ysh = buf.y_shared.float().cpu().numpy()
    assert prefill_err(ysh[shared_rows], np.stack([rows[("shared", t)] for t in shared_rows]),
                       "y_shared (tile rows)") <= 1.0


def test_prefill_empty_batch():
    """T = 0 is a valid call that enqueues nothing."""
    say("prefill empty batch")
    L, dev = dev_layer(2)
    sh = moe.shape_of(L.shape)
    buf = LayerBuffers.allocate(sh, 0, PRE)
    x = torch.empty((0, sh.d), dtype=torch.bfloat16, device="cuda")
    moe.moe_expert_ffn(sh, x, dev["experts"], None, buf.offsets, buf.perm, buf.active,
                       buf.n_active, PRE, buf.y, None, buf.ffn_workspace)
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------
# quantiser (the one-time conversion of a checkpoint)
# ----------------------------------------------------------------------------

def gpu_quantize(w_np, dt, mode):
    """Quantise w_np (float32 values; bf16-rounded first when dt is bf16) on
    the GPU; returns (codes, scales, the exact input values)."""
    if dt == "bf16":
        bits = synth.bf16_round(np.asarray(w_np, dtype=np.float32))
        vals = synth.bf16_to_f32(bits)
        w = torch.from_numpy(bits.view(np.int16).copy()).cuda().view(torch.bfloat16)
    else:
        vals = np.asarray(w_np, dtype=np.float32)
        w = torch.from_numpy(vals.copy()).cuda()
    n, k = vals.shape
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda")
    ns = k // 64 if mode == moe.MOE_QUANT_GS64 else 1
    scales = torch.empty((n, ns), dtype=torch.float16, device="cuda")
    moe.moe_quantize(w, mode, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), vals


@pytest.mark.parametrize("n,k", [(1, 64), (3, 192), (17, 1024), (64, 2048)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("mode", [0, 1])
def test_quantize_parity(n, k, dt, mode):
    say(f"quantize n={n} k={k} {dt} mode={mode}")
    rng = np.random.default_rng(n * 7 + k)
    w = (rng.standard_normal((n, k)) * rng.uniform(0.001, 3.0, size=(n, 1))).astype(np.float32)
    w[0, :64] = 0.0  # a group (and, at k = 64, a row) of zeros
    codes, scales, vals = gpu_quantize(w, dt, mode)
    if mode == moe.MOE_QUANT_GS64:
        rc, rs = oracle.quantize_gs64(vals)
    else:
        rc, rs = oracle.quantize_rows(vals)
        rs = rs[:, None]
    assert np.array_equal(scales.view(np.uint16), rs.view(np.uint16))
    assert np.array_equal(codes, rc)


def test_quantize_exact_ties_go_to_even():
    say("quantize ties")
    # groups whose absmax is 7 * s exactly, the rest at half-way points (q + 1/2) * s
    s = np.float16(0.013671875)
    base = (np.arange(-7, 7) + 0.5) * float(s)
    row = np.concatenate([[7 * float(s)], np.tile(base, 5)[:63]])
    w = np.stack([row, -row, row[::-1].copy()]).astype(np.float32)
    codes, scales, vals = gpu_quantize(w, "f32", moe.MOE_QUANT_GS64)
    rc, rs = oracle.quantize_gs64(vals)
    assert np.all(scales == s)
    assert np.array_equal(codes, rc)
    q = oracle.unpack_int4(codes)
    assert np.all(q[np.abs(vals) < 7 * float(s)] % 2 == 0)


def test_quantize_full_expert_matrix_and_round_trip_through_the_ffn():
    """A 6144 x 2048 matrix (the down projection of the ~19 MB experts) is
    bit-exact with the oracle; and a whole block quantised on the GPU from
    float weights runs through the decode FFN like the oracle's block."""
    say("quantize full matrix")
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((6144, 2048)) * 0.05).astype(np.float32)
    codes, scales, vals = gpu_quantize(w, "bf16", moe.MOE_QUANT_GS64)
    rc, rs = oracle.quantize_gs64(vals)
    assert np.array_equal(scales.view(np.uint16), rs.view(np.uint16))
    assert np.array_equal(codes, rc)
    # small layer: quantise gate, up, down of 8 experts into canonical blocks
    d, f, E, k = 512, 256, 8, 2
    sh = moe.Shape(d, f, E, k, 64, 0)
    bb = oracle.expert_block_bytes(d, f)
    mats = [(f, d), (f, d), (d, f)]
    blocks = torch.zeros((E, bb), dtype=torch.uint8, device="cuda")
    ref_blocks = np.zeros((E, bb), dtype=np.uint8)
    s0 = 3 * d * f // 2
    for e in range(E):
        qo, so = 0, s0
        for (rows, cols) in mats:
            wm = (rng.standard_normal((rows, cols)) * 0.03).astype(np.float32)
            c_gpu = blocks[e, qo:qo + rows * cols // 2].view(rows, cols // 2)
            s_gpu = blocks[e, so:so + rows * cols // 64 * 2].view(torch.float16).view(rows, cols // 64)
            moe.moe_quantize(torch.from_numpy(wm).cuda(), moe.MOE_QUANT_GS64, c_gpu, s_gpu)
            rc, rs = oracle.quantize_gs64(wm)
            ref_blocks[e, qo:qo + rows * cols // 2] = rc.reshape(-1)
            ref_blocks[e, so:so + rows * cols // 64 * 2] = rs.view(np.uint8).reshape(-1)
            qo += rows * cols // 2
            so += rows * cols // 64 * 2
    torch.cuda.synchronize()
    assert np.array_equal(blocks.cpu().numpy(), ref_blocks)
    x = rng.standard_normal((4, d)).astype(np.float32)
    wr = (rng.standard_normal((E, d)) * 0.02).astype(np.float32)
    buf = LayerBuffers.allocate(sh, 4, DEC)
    run_layer(torch.from_numpy(x).cuda(), torch.from_numpy(wr).cuda(), None, packed(sh, ref_blocks),
              None, buf)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(x, wr, None, ref_blocks, None, d, f, E, k)
    assert rel_err(buf.out.cpu().numpy(), ref["out"]) <= TOL_DECODE


# ----------------------------------------------------------------------------
# MXFP4 experts (E2M1 codes, one E8M0 scale per 32 elements): shape group 32
# ----------------------------------------------------------------------------

from oracle import mxfp4 as oracle_mx  # noqa: E402


def mx_shape(L):
    s = L.shape
    return moe.Shape(s.d, s.f, s.n_experts, s.top_k, 32, s.f_shared)


def np_pack_block_mx(blk, d, f):
    """The MXFP4 packed layout, restated with numpy reshapes: codes in 64-row
    tiles of 32-column chunks (16 bytes per row, nibbles unchanged); scale
    bytes in the same tiles, block-major."""
    blk = np.asarray(blk, dtype=np.uint8)
    out = np.empty_like(blk)
    s0 = 3 * d * f // 2
    mats = [(f, d, 0, s0), (f, d, f * d // 2, s0 + f * d // 32),
            (d, f, f * d, s0 + 2 * f * d // 32)]
    for N, K, qo, so in mats:
        nq = N * K // 2
        q = blk[qo:qo + nq].reshape(N // 64, 64, K // 32, 16).transpose(0, 2, 1, 3)
        out[qo:qo + nq] = np.ascontiguousarray(q).reshape(-1)
        ns = N * K // 32
        sc = blk[so:so + ns].reshape(N // 64, 64, K // 32).transpose(0, 2, 1)
        out[so:so + ns] = np.ascontiguousarray(sc).reshape(-1)
    return out


@pytest.mark.parametrize("d,f,n", [(128, 192, 3), (6144, 2048, 1)])
def test_pack_mxfp4_matches_layout_definition(d, f, n):
    say(f"pack mxfp4 d={d} f={f} n={n}")
    rng = np.random.default_rng(d + f + 1)
    bb = oracle_mx.block_bytes(d, f)
    blocks = rng.integers(0, 256, size=(n, bb), dtype=np.uint8)
    sh = moe.Shape(d, f, 8, 2, 32, 0)
    assert moe.moe_expert_bytes(d, f, 32) == bb
    got = packed(sh, blocks).cpu().numpy()
    for b in range(n):
        assert np.array_equal(got[b], np_pack_block_mx(blocks[b], d, f)), f"block {b}"


_mx_layers = {}


def mx_layer(cfg):
    if cfg not in _mx_layers:
        _mx_layers.clear()
        torch.cuda.empty_cache()
        L = synth.make_layer(cfg, fmt="mxfp4")
        sh = mx_shape(L)
        dev = dict(
            w_router=torch.from_numpy(L.w_router).cuda(),
            bias=None if L.bias is None else torch.from_numpy(L.bias).cuda(),
            experts=packed(sh, L.experts),
            shared=None if L.shared is None else packed(sh, L.shared[None])[0],
        )
        _mx_layers[cfg] = (L, sh, dev)
    return _mx_layers[cfg]


# (7, 3): d = f = 8192, the largest sizes taken
@pytest.mark.parametrize("cfg,T", [(6, 8), (6, 37), (2, 1), (2, 16), (4, 1), (7, 3), (8, 5),
                                   (9, 3)])
def test_layer_decode_parity_mxfp4(cfg, T):
    """MXFP4 experts through route, union, the decode FFN (shape group 32)
    and combine, against the float64 oracle with MXFP4 block decoding."""
    say(f"layer decode mxfp4 cfg={cfg} T={T}")
    L, sh, dev = mx_layer(cfg)
    x, xf = tokens(cfg, T, 0)
    buf = LayerBuffers.allocate(sh, T, DEC)
    run_layer(x, dev["w_router"], dev["bias"], dev["experts"], dev["shared"], buf)
    torch.cuda.synchronize()
    s = L.shape
    ref = oracle.moe_layer(xf, L.w_router, L.bias, L.experts, L.shared, s.d, s.f, s.n_experts,
                           s.top_k, weights=oracle_mx.expert_weights)
    check_routing_and_union(buf, ref["topk_idx"], ref["topk_w"],
                            (ref["counts"], ref["offsets"], ref["perm"], ref["inv_perm"],
                             ref["active"], ref["n_active"]))
    ey = rel_err(buf.y.cpu().numpy()[: T * s.top_k], ref["y"])
    assert ey <= TOL_DECODE, f"y error {ey:.2e} rms"
    if L.shared is not None:
        es = rel_err(buf.y_shared.cpu().numpy()[:T], ref["y_shared"])
        assert es <= TOL_DECODE, f"y_shared error {es:.2e} rms"
    eo = rel_err(buf.out.cpu().numpy(), ref["out"])
    assert eo <= TOL_DECODE, f"out error {eo:.2e} rms"


# (6, 512) and (6, 97): 128-row tiles full and partial, odd group counts,
# partial column tiles; (3, 64): 256 experts with the shared expert;
# (7, 160): d = f = 8192, both tile kinds over 256 MXFP4 blocks along K;
# layer 9 (f = 128) at T = 40 has a test of its own below
@pytest.mark.parametrize("cfg,T", [(6, 512), (6, 97), (2, 16), (3, 64), (7, 160), (8, 300)])
def test_layer_prefill_parity_mxfp4(cfg, T):
    """bf16 x through route, union, the MFMA FFN over MXFP4 blocks (the E8M0
    scale folded into the E2M1 -> bf16 conversion) and a bf16 combine,
    against the float64 oracle with MXFP4 block decoding, at the 2e-2 * rms
    bound of the bf16 path."""
    say(f"layer prefill mxfp4 cfg={cfg} T={T}")
    L, sh, dev = mx_layer(cfg)
    x, xf = tokens(cfg, T, 0)
    buf = LayerBuffers.allocate(sh, T, PRE)
    run_layer(x, dev["w_router"], dev["bias"], dev["experts"], dev["shared"], buf)
    torch.cuda.synchronize()
    s = L.shape
    ref = oracle.moe_layer(xf, L.w_router, L.bias, L.experts, L.shared, s.d, s.f, s.n_experts,
                           s.top_k, weights=oracle_mx.expert_weights)
    check_routing_and_union(buf, ref["topk_idx"], ref["topk_w"],
                            (ref["counts"], ref["offsets"], ref["perm"], ref["inv_perm"],
                             ref["active"], ref["n_active"]))
    ey = prefill_err(buf.y.float().cpu().numpy()[: T * s.top_k], ref["y"], "y")
    assert ey <= 1.0, f"y error {ey:.2f} x bound"
    if L.shared is not None:
        es = prefill_err(buf.y_shared.float().cpu().numpy()[:T], ref["y_shared"], "y_shared")
        assert es <= 1.0, f"y_shared error {es:.2f} x bound"
    eo = prefill_err(buf.out.float().cpu().numpy(), ref["out"], "out (bf16)")
    assert eo <= 1.0, f"out error {eo:.2f} x bound"


def test_layer_prefill_parity_mxfp4_one_h_term_dominant():
    """Layer 9 (f = 128, 1024 experts top-32) over MXFP4 blocks at T = 40.
    With 128 terms in the down sum and heavy-tailed MXFP4 weights, one term
    w_j * h_j can dominate an output whose terms cancel, and storing h in
    bf16 (as the prefill path does) moves that output by up to
    2^-9 * sum_j |w_dn[n][j]| |h_j|, more than 2^-8 |y|: an exact evaluation
    that stores h and y in bf16 reaches 1.13 of the usual element-wise bound
    here.  Checked: the strict bound as everywhere, and element-wise the
    usual bound plus that term (computed from the oracle's exact h)."""
    cfg, T = 9, 40
    say(f"layer prefill mxfp4 cfg={cfg} T={T} (h rounding allowance)")
    L, sh, dev = mx_layer(cfg)
    x, xf = tokens(cfg, T, 0)
    buf = LayerBuffers.allocate(sh, T, PRE)
    run_layer(x, dev["w_router"], dev["bias"], dev["experts"], dev["shared"], buf)
    torch.cuda.synchronize()
    s = L.shape
    ref = oracle.moe_layer(xf, L.w_router, L.bias, L.experts, L.shared, s.d, s.f, s.n_experts,
                           s.top_k, weights=oracle_mx.expert_weights)
    check_routing_and_union(buf, ref["topk_idx"], ref["topk_w"],
                            (ref["counts"], ref["offsets"], ref["perm"], ref["inv_perm"],
                             ref["active"], ref["n_active"]))
    xd = np.asarray(xf, dtype=np.float64)

    def h_abs_sum(block, rows):
        wg, wu, wd = oracle_mx.expert_weights(block, s.d, s.f)
        g = xd[rows] @ wg.T
        h = oracle.silu(g) * (xd[rows] @ wu.T)
        return np.abs(h) @ np.abs(wd).T

    perm, offs = ref["perm"], ref["offsets"]
    cy = np.zeros_like(ref["y"])
    for e in np.nonzero(np.diff(offs))[0]:
        cy[offs[e]:offs[e + 1]] = h_abs_sum(L.experts[e], perm[offs[e]:offs[e + 1]] // s.top_k)
    cs = h_abs_sum(L.shared, np.arange(T))
    inv = ref["inv_perm"].reshape(T, s.top_k)
    co = np.einsum("tj,tjd->td", ref["topk_w"].astype(np.float64), cy[inv]) + cs
    ey = prefill_err(buf.y.float().cpu().numpy()[: T * s.top_k], ref["y"], "y", 2.0 ** -9 * cy)
    es = prefill_err(buf.y_shared.float().cpu().numpy()[:T], ref["y_shared"], "y_shared",
                     2.0 ** -9 * cs)
    eo = prefill_err(buf.out.float().cpu().numpy(), ref["out"], "out (bf16)", 2.0 ** -9 * co)
    assert max(ey, es, eo) <= 1.0, f"errors {ey:.2f}, {es:.2f}, {eo:.2f} x bound"


def test_layer_prefill_parity_mxfp4_2048_sampled():
    """The 2048-token Zipf-routed batch over the d=6144, f=2048 layer with
    MXFP4 blocks: every expert output of three sampled tokens and their layer
    outputs against the oracle."""
    sample = [0, 1000, 2047]
    say(f"layer prefill mxfp4 cfg=5 T=2048 (sampled {sample})")
    L, sh, dev = mx_layer(5)
    x, xf = tokens(5, 2048, 0)
    buf = LayerBuffers.allocate(sh, 2048, PRE)
    run_layer(x, dev["w_router"], dev["bias"], dev["experts"], dev["shared"], buf)
    torch.cuda.synchronize()
    ref = oracle_sampled(L, xf, sample, weights=oracle_mx.expert_weights)
    check_routing_and_union(buf, ref["topk_idx"], ref["topk_w"], ref["union"])
    y = buf.y.float().cpu().numpy()
    got = np.stack([y[p] for p in ref["y"]])
    assert prefill_err(got, np.stack(list(ref["y"].values())), "y") <= 1.0
    ysh = buf.y_shared.float().cpu().numpy()
    assert prefill_err(ysh[sample], np.stack([ref["y_shared"][t] for t in sample]),
                       "y_shared") <= 1.0
    out = buf.out.float().cpu().numpy()
    assert prefill_err(out[sample], np.stack([ref["out"][t] for t in sample]), "out") <= 1.0


# MXFP4 scale bytes at and beyond the range where E2M1 * 2^(E - 127) is a
# normal bf16 (2 .. 252), and the NaN byte.
MX_EDGE_E = [0, 1, 2, 126, 252, 253, 254, 255]


def mx_edge_layer(E):
    """Layer 6 with MXFP4 blocks whose gate and up scale bytes are all E (every
    routed expert and the shared one), and bf16 tokens scaled by a power of two
    that keeps each product E2M1 * 2^(E - 127) * x, and the sums of 32 of
    them, inside the float32 range: x * 2^117 for E <= 2, x * 2^-118 for
    E >= 252 (every |x| first raised to at least 2^-8, so the scaled tokens
    stay normal bf16 numbers).  The down blocks keep their drawn scales."""
    L = synth.make_layer(6, fmt="mxfp4")
    s = L.shape
    n_gu = 2 * s.f * s.d // 32  # gate and up scale bytes, right after the codes
    q_end = 3 * s.d * s.f // 2
    L.experts[:, q_end:q_end + n_gu] = E
    L.shared[q_end:q_end + n_gu] = E
    k = 117 if E <= 2 else (-118 if 252 <= E <= 254 else 0)
    return L, k


def mx_edge_tokens(T, k):
    bits, xf = synth.make_tokens(6, T, 5)
    xf = np.sign(xf) * np.maximum(np.abs(xf), 2.0 ** -8)  # exact in bf16
    xf = (xf * 2.0 ** k).astype(np.float32)  # a power of two: exact
    bits = (xf.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(synth.bf16_to_f32(bits), xf)
    return bits, xf


@pytest.mark.parametrize("path,T", [("decode", 37), ("prefill", 300)])
@pytest.mark.parametrize("E", MX_EDGE_E)
def test_mxfp4_every_scale_byte(E, path, T):
    """MXFP4 blocks are decoded exactly for every E8M0 byte, on both paths:
    the edge exponents 0, 1, 2, 252, 253, 254 (whose weights are bf16
    subnormals or overflow bf16 when folded into the element conversion) and
    E = 255, which makes every weight of the block NaN, as in the oracle.
    The prefill batch has 128-row and 32-row tiles and the shared expert."""
    say(f"mxfp4 scale byte E={E} path={path} T={T}")
    L, k = mx_edge_layer(E)
    sh = mx_shape(L)
    s = L.shape
    bits, xf = mx_edge_tokens(T, k)
    x = torch.from_numpy(bits.view(np.int16).copy()).cuda().view(torch.bfloat16)
    experts = packed(sh, L.experts)
    shared = packed(sh, L.shared[None])[0]
    P = PRE if path == "prefill" else DEC
    buf = LayerBuffers.allocate(sh, T, P)
    run_layer(x, torch.from_numpy(L.w_router).cuda(), torch.from_numpy(L.bias).cuda(), experts,
              shared, buf)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(xf, L.w_router, L.bias, L.experts, L.shared, s.d, s.f, s.n_experts,
                           s.top_k, weights=oracle_mx.expert_weights)
    check_routing_and_union(buf, ref["topk_idx"], ref["topk_w"],
                            (ref["counts"], ref["offsets"], ref["perm"], ref["inv_perm"],
                             ref["active"], ref["n_active"]))
    n = T * s.top_k
    got = dict(y=buf.y.float().cpu().numpy()[:n], y_shared=buf.y_shared.float().cpu().numpy()[:T],
               out=buf.out.float().cpu().numpy())
    for name in ("y", "y_shared", "out"):
        g, r = got[name], ref[name]
        if E == 255:
            assert np.isnan(r).all() and np.isnan(g).all(), name
            continue
        assert np.isfinite(r).all() and np.isfinite(g).all(), name
        if P == PRE:
            assert prefill_err(g, r, name) <= 1.0, name
        else:
            e = rel_err(g, r)
            say(f"  {name}: max|err|/rms = {e:.2e}")
            assert e <= TOL_DECODE, name


@pytest.mark.parametrize("fmt,path,T", [("int4", "prefill", 300), ("mxfp4", "prefill", 300),
                                         ("int4", "decode", 8), ("mxfp4", "decode", 8)])
def test_layer_all_tokens_to_the_same_experts(fmt, path, T):
    """Degenerate routing: a router bias of +1000 on experts 0 and 1 sends
    every token to the same two experts (each holds all T rows: full and
    partial 128-row tiles plus 32-row tiles on the prefill path), every other
    expert is unrouted; layer against the oracle."""
    say(f"layer all tokens to experts 0,1 fmt={fmt} path={path} T={T}")
    if fmt == "int4":
        L, dev = dev_layer(6)
        sh = moe.shape_of(L.shape)
        weights = None
    else:
        L, sh, dev = mx_layer(6)
        weights = oracle_mx.expert_weights
    s = L.shape
    bias = np.zeros(s.n_experts, dtype=np.float32)
    bias[: s.top_k] = 1000.0
    x, xf = tokens(6, T, 3)
    P = PRE if path == "prefill" else DEC
    buf = LayerBuffers.allocate(sh, T, P)
    run_layer(x, dev["w_router"], torch.from_numpy(bias).cuda(), dev["experts"], dev["shared"],
              buf)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(xf, L.w_router, bias, L.experts, L.shared, s.d, s.f, s.n_experts,
                           s.top_k, **({} if weights is None else {"weights": weights}))
    assert set(np.unique(ref["topk_idx"])) == set(range(s.top_k))
    check_routing_and_union(buf, ref["topk_idx"], ref["topk_w"],
                            (ref["counts"], ref["offsets"], ref["perm"], ref["inv_perm"],
                             ref["active"], ref["n_active"]))
    n = T * s.top_k
    if P == PRE:
        assert prefill_err(buf.y.float().cpu().numpy()[:n], ref["y"], "y") <= 1.0
        assert prefill_err(buf.y_shared.float().cpu().numpy()[:T], ref["y_shared"],
                           "y_shared") <= 1.0
        assert prefill_err(buf.out.float().cpu().numpy(), ref["out"], "out") <= 1.0
    else:
        assert rel_err(buf.y.cpu().numpy()[:n], ref["y"]) <= TOL_DECODE
        assert rel_err(buf.y_shared.cpu().numpy()[:T], ref["y_shared"]) <= TOL_DECODE
        assert rel_err(buf.out.cpu().numpy(), ref["out"]) <= TOL_DECODE


def test_mxfp4_rejected_where_not_built():
    """The one-call layer refuses MXFP4 shapes (group 32) with
    MOE_ERR_UNSUPPORTED rather than running them as int4."""
    L, sh, dev = mx_layer(6)
    assert moe.moe_layer_decode_workspace_bytes(sh, 8) == 0
    x, _ = tokens(6, 8, 0)
    buf = LayerBuffers.allocate(moe.shape_of(L.shape), 8, DEC)  # int4 sizes
    with pytest.raises(moe.MoeError):
        moe.moe_layer_decode(sh, x, dev["w_router"], dev["bias"], dev["experts"], dev["shared"],
                             buf.topk_idx, buf.topk_w, buf.counts, buf.offsets, buf.perm,
                             buf.inv_perm, buf.active, buf.n_active, buf.y, buf.y_shared, buf.out,
                             buf.layer_workspace)


# ----------------------------------------------------------------------------
# the benchmark's calibration read
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("n,block_bytes,workgroups", [(3, 1 << 20, 3), (3, (1 << 20) + 48, 7),
                                                      (9, 20_054_016, 2304), (2, 4096, 4096),
                                                      (5, 160, 37)])
def test_stream_read_folds_every_piece_of_its_share_once(n, block_bytes, workgroups):
    """moe_measure_stream_read: workgroup w XORs the 16-byte pieces of its
    share (block w / wpb, bytes [per * s, per * s + per) cut at the block's
    end, s = w % wpb, wpb = workgroups / n, per = block_bytes / wpb rounded
    up to 16) into one word; on random blocks every word must equal that
    XOR of the share's 32-bit words, so no piece is skipped or read twice.
    Shapes: ragged blocks, shares past a block's end (empty), one
    workgroup per block, the decode step's nine 19 MB blocks."""
    say(f"stream read n={n} bytes={block_bytes} workgroups={workgroups}")
    rng = np.random.default_rng(block_bytes + workgroups)
    host = rng.integers(0, 2 ** 32, size=(n, block_bytes // 4), dtype=np.uint32)
    dev = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((workgroups,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    moe.moe_measure_stream_read([dev[b].data_ptr() for b in range(n)], block_bytes, workgroups,
                                sink)
    torch.cuda.synchronize()
    wpb = workgroups // n
    per = -(-block_bytes // wpb)
    per = -(-per // 16) * 16
    got = sink.cpu().numpy().view(np.uint32)
    for w in range(wpb * n):
        b, sh = divmod(w, wpb)
        lo, hi = min(per * sh, block_bytes), min(per * sh + per, block_bytes)
        want = np.bitwise_xor.reduce(host[b, lo // 4: hi // 4]) if hi > lo else np.uint32(0)
        assert got[w] == want, f"workgroup {w} (block {b}, share {sh})"
    # entries past wpb * n are not written
    assert np.all(got[wpb * n:] == 0x5A5A5A5A)
