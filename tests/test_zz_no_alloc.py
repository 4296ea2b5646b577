"""GPU check of moe_layer_decode_static, the decode layer whose scratch is the
library's static per-GPU array (no workspace argument, nothing allocated):
through the C ABI, two calls in a row -- the second with a smaller batch --
each equal, bit for bit in every output, to moe_layer_decode with a
workspace of its own on the same inputs."""
import numpy as np
import pytest
import torch

import synth
import int4_routed_expert_logits_amd as moe
from int4_routed_expert_logits_amd.layer import LayerBuffers, run_layer_decode

pytestmark = pytest.mark.gpu

OUTPUTS = ("topk_idx", "topk_w", "counts", "offsets", "perm", "inv_perm", "active", "n_active",
           "y", "y_shared", "out")


def packed(sh, blocks):
    src = torch.from_numpy(np.ascontiguousarray(blocks)).cuda()
    dst = torch.empty_like(src)
    moe.moe_pack_experts(sh, src.shape[0], src, dst)
    return dst


@pytest.mark.parametrize("cfg,Ts", [(6, (8, 3)), (2, (8, 1)), (4, (2, 1))])
def test_static_scratch_call_equals_the_workspace_call(cfg, Ts):
    print(f"moe_layer_decode_static cfg={cfg} T={Ts}", flush=True)
    L = synth.make_layer(cfg)
    sh = moe.shape_of(L.shape)
    experts = packed(sh, L.experts)
    shared = None if L.shared is None else packed(sh, L.shared[None])[0]
    w_router = torch.from_numpy(L.w_router).cuda()
    bias = None if L.bias is None else torch.from_numpy(L.bias).cuda()
    for call, T in enumerate(Ts):
        bits, _ = synth.make_tokens(cfg, T, batch=call + 1)
        x = (torch.from_numpy(bits).cuda() if bits.dtype == np.float32 else
             torch.from_numpy(bits.view(np.int16).copy()).cuda().view(torch.bfloat16))
        a = LayerBuffers.allocate(sh, T, moe.MOE_PATH_DECODE_F32)
        run_layer_decode(x, w_router, bias, experts, shared, a)
        b = LayerBuffers.allocate(sh, T, moe.MOE_PATH_DECODE_F32)
        moe.moe_layer_decode_static(sh, x, w_router, bias, experts, shared, b.topk_idx, b.topk_w,
                                    b.counts, b.offsets, b.perm, b.inv_perm, b.active,
                                    b.n_active, b.y, b.y_shared, b.out)
        torch.cuda.synchronize()
        n = T * sh.top_k
        for name in OUTPUTS:
            ta, tb = getattr(a, name), getattr(b, name)
            if ta is None:
                assert tb is None
                continue
            if name in ("perm", "inv_perm", "y"):
                ta, tb = ta[:n], tb[:n]
            if name == "y_shared":
                ta, tb = ta[:T], tb[:T]
            assert torch.equal(ta.cpu(), tb.cpu()), (call, T, name)
