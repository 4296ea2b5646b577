"""GPU checks of the per-layer expert cache (moe_cache_layer_decode).

Every step through a cache smaller than the layer, while misses stream from
pinned host memory on a second stream, is checked three ways:
  * against the float64 oracle: routing bit for bit, gate weights within
    1e-6, the layer output and the shared expert's output within
    2e-3 * rms (the ~19 MB-expert layer through the oracle's per-expert rows);
  * against the reference cache model (oracle/expert_cache.py) fed with the
    oracle's routing: the experts the step fetched, in placement order, and
    the expert each displaced;
  * against the library's own all-resident separate calls, bit for bit (the
    cache must not change a single bit of the result).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import int4_routed_expert_logits_amd as moe
from int4_routed_expert_logits_amd.layer import LayerBuffers, run_layer
from oracle.expert_cache import ExpertCache
from oracle_rows import oracle_sampled

pytestmark = pytest.mark.gpu

DEC = moe.MOE_PATH_DECODE_F32
TOL_DECODE = 2e-3


def rel_err(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref))) / rms


def say(msg):
    print(msg, flush=True)


def packed(sh, blocks_np):
    src = torch.from_numpy(blocks_np).cuda()
    dst = torch.empty_like(src)
    moe.moe_pack_experts(sh, src.shape[0], src, dst)
    return dst


def dev_x(bits):
    if bits.dtype == np.float32:
        return torch.from_numpy(bits).cuda()
    return torch.from_numpy(bits.view(np.int16).copy()).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("cfg,slots,pins,Ts,zipf_bias", [
    (2, 20, (5,), [1, 2, 1, 1, 2, 1, 2, 2, 1, 1, 1, 2], False),
    (3, 24, (), [1, 2, 1, 1, 2, 1, 1, 2, 1, 1], True),
    (4, 16, (0,), [1, 1, 1, 1, 1, 1], True),
])
def test_cached_steps_match_the_oracle_and_the_cache_model(cfg, slots, pins, Ts, zipf_bias):
    say(f"expert cache cfg={cfg} slots={slots} pins={pins} steps={len(Ts)}")
    L = synth.make_layer(cfg)
    sh = moe.shape_of(L.shape)
    bias_np = synth.make_layer(5, experts=[]).bias if zipf_bias else L.bias
    experts = packed(sh, L.experts)
    shared = None if L.shared is None else packed(sh, L.shared[None])[0]
    w_router = torch.from_numpy(L.w_router).cuda()
    bias = None if bias_np is None else torch.from_numpy(bias_np).cuda()
    bb = moe.moe_expert_bytes(sh.d, sh.f, 64)
    host = torch.empty((experts.numel(),), dtype=torch.uint8, pin_memory=True)
    host.copy_(experts.view(-1))
    dev_slots = torch.empty((slots * bb,), dtype=torch.uint8, device="cuda")
    cache = moe.moe_cache_create(sh, slots, dev_slots, host)
    ref = ExpertCache(slots)
    copy_stream = torch.cuda.Stream()
    try:
        for e in pins:
            moe.moe_cache_pin(cache, e)
            ref.pin(e)
        for step, T in enumerate(Ts):
            bits, xf = synth.make_tokens(cfg, T, batch=step)
            x = dev_x(bits)
            a = LayerBuffers.allocate(sh, T, DEC)
            run_layer(x, w_router, bias, experts, shared, a)
            b = LayerBuffers.allocate(sh, T, DEC)
            ws = torch.empty((moe.moe_cache_workspace_bytes(sh, T, slots),), dtype=torch.uint8,
                             device="cuda")
            moe.moe_cache_layer_decode(cache, x, w_router, bias, shared, b.topk_idx, b.topk_w, b.y,
                                       b.y_shared, b.out, ws, copy_stream=copy_stream)
            torch.cuda.synchronize()
            # the oracle
            if cfg == 4:  # 9 experts of ~19 MB: the oracle's rows of this step's tokens
                r = oracle_sampled(L, xf, list(range(T)), bias=bias_np)
                ref_out = np.stack([r["out"][t] for t in range(T)])
                ref_ysh = np.stack([r["y_shared"][t] for t in range(T)])
            else:
                r = oracle.moe_layer(xf, L.w_router, bias_np, L.experts, L.shared, sh.d, sh.f,
                                     sh.n_experts, sh.top_k)
                ref_out, ref_ysh = r["out"], r["y_shared"]
            assert np.array_equal(b.topk_idx.cpu().numpy(), r["topk_idx"]), step
            assert np.max(np.abs(b.topk_w.cpu().numpy() - r["topk_w"])) <= 1e-6, step
            eo = rel_err(b.out.cpu().numpy(), ref_out)
            say(f"  step {step}: T={T} out max|err|/rms = {eo:.2e}")
            assert eo <= TOL_DECODE, step
            if shared is not None:
                assert rel_err(b.y_shared.cpu().numpy()[:T], ref_ysh) <= TOL_DECODE, step
            # the reference cache model, step by step
            _, rf, rev = ref.step(r["topk_idx"].ravel())
            fetched, evicted = moe.moe_cache_last_fetch(cache, sh.n_experts)
            assert fetched == rf, step
            assert evicted == [-1 if rev[e] is None else rev[e] for e in rf], step
            # the library's all-resident calls
            assert torch.equal(a.topk_idx.cpu(), b.topk_idx.cpu()), step
            assert torch.equal(a.topk_w.cpu(), b.topk_w.cpu()), step
            assert torch.equal(a.out.cpu(), b.out.cpu()), step
            if shared is not None:
                assert torch.equal(a.y_shared.cpu(), b.y_shared.cpu()), step
        hits, misses, nbytes = moe.moe_cache_stats(cache)
        assert (hits, misses) == (ref.hits, ref.misses)
        assert nbytes == misses * bb
        assert misses > slots  # the trace did evict
    finally:
        torch.cuda.synchronize()
        moe.moe_cache_destroy(cache)
