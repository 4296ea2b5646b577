"""GPU checks of the per-layer expert cache (moe_cache_layer_decode).

Steps through a cache smaller than the layer must give, bit for bit, the
routing and the layer output of the separate calls with every expert
resident in HBM, while misses stream from pinned host memory on a second
stream; the cache's hit and miss counts must equal the reference model's
(oracle/expert_cache.py) fed with the oracle's own routing of the same
tokens.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import int4_routed_expert_logits_amd as moe
from int4_routed_expert_logits_amd.layer import LayerBuffers, run_layer
from oracle.expert_cache import ExpertCache

pytestmark = pytest.mark.gpu

DEC = moe.MOE_PATH_DECODE_F32


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
def test_cached_steps_equal_the_all_resident_layer(cfg, slots, pins, Ts, zipf_bias):
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
            assert torch.equal(a.topk_idx.cpu(), b.topk_idx.cpu()), step
            assert torch.equal(a.topk_w.cpu(), b.topk_w.cpu()), step
            assert torch.equal(a.out.cpu(), b.out.cpu()), step
            if shared is not None:
                assert torch.equal(a.y_shared.cpu(), b.y_shared.cpu()), step
            idx, _, _ = oracle.route(xf, L.w_router, bias_np, sh.top_k)
            ref.step(idx.ravel())
        hits, misses, nbytes = moe.moe_cache_stats(cache)
        assert (hits, misses) == (ref.hits, ref.misses)
        assert nbytes == misses * bb
        assert misses > slots  # the trace did evict
    finally:
        torch.cuda.synchronize()
        moe.moe_cache_destroy(cache)
