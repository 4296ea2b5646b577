"""Device buffers for one layer call and the four-call sequence.

Plumbing only: torch allocates the caller-owned device memory the C ABI
expects, and ``run_layer`` issues moe_route_union -> moe_expert_ffn ->
moe_combine on one stream with no host synchronisation in between;
``run_layer_decode`` makes the single moe_layer_decode call instead (decode
batches of at most 8 tokens).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import _binding as B


@dataclasses.dataclass
class LayerBuffers:
    shape: B.Shape
    T: int
    path: int
    topk_idx: torch.Tensor
    topk_w: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    perm: torch.Tensor
    inv_perm: torch.Tensor
    active: torch.Tensor
    n_active: torch.Tensor
    y: torch.Tensor
    y_shared: Optional[torch.Tensor]
    out: torch.Tensor
    workspace: torch.Tensor       # moe_route scratch
    ffn_workspace: torch.Tensor   # moe_expert_ffn scratch (the intermediate h)
    layer_workspace: torch.Tensor  # moe_layer_decode scratch (decode path only)

    @classmethod
    def allocate(cls, shape, T: int, path: int, device="cuda", out_dtype=None):
        sh = B._shape(shape)
        k, E, d = sh.top_k, sh.n_experts, sh.d
        i32 = dict(dtype=torch.int32, device=device)
        ydt = torch.float32 if path == B.MOE_PATH_DECODE_F32 else torch.bfloat16
        odt = out_dtype or ydt
        ws = max(B.moe_route_workspace_bytes(sh, T), 256)
        fws = max(B.moe_ffn_workspace_bytes(sh, T, path), 256)
        lws = max(B.moe_layer_decode_workspace_bytes(sh, T), 256) if path == B.MOE_PATH_DECODE_F32 else 256
        return cls(
            shape=sh, T=T, path=path,
            topk_idx=torch.empty((T, k), **i32),
            topk_w=torch.empty((T, k), dtype=torch.float32, device=device),
            counts=torch.empty((E,), **i32),
            offsets=torch.empty((E + 1,), **i32),
            perm=torch.empty((max(T * k, 1),), **i32),
            inv_perm=torch.empty((max(T * k, 1),), **i32),
            active=torch.empty((E,), **i32),
            n_active=torch.empty((1,), **i32),
            y=torch.empty((max(T * k, 1), d), dtype=ydt, device=device),
            y_shared=torch.empty((max(T, 1), d), dtype=ydt, device=device) if sh.f_shared else None,
            out=torch.empty((T, d), dtype=odt, device=device),
            workspace=torch.empty((ws,), dtype=torch.uint8, device=device),
            ffn_workspace=torch.empty((fws,), dtype=torch.uint8, device=device),
            layer_workspace=torch.empty((lws,), dtype=torch.uint8, device=device),
        )


def run_layer(x, w_router, bias, experts, shared, buf: LayerBuffers, stream=None):
    """All four steps of the layer for the batch x [T, d]: route and union in
    one call (moe_route_union), then the expert FFN and the combine."""
    sh = buf.shape
    B.moe_route_union(sh, x, w_router, bias, buf.topk_idx, buf.topk_w, buf.counts, buf.offsets,
                      buf.perm, buf.inv_perm, buf.active, buf.n_active, buf.workspace, stream)
    B.moe_expert_ffn(sh, x, experts, shared, buf.offsets, buf.perm, buf.active, buf.n_active,
                     buf.path, buf.y, buf.y_shared, buf.ffn_workspace, stream)
    B.moe_combine(sh, buf.y, buf.y_shared, buf.inv_perm, buf.topk_w, buf.out, stream)
    return buf.out


def run_layer_decode(x, w_router, bias, experts, shared, buf: LayerBuffers, stream=None):
    """The same layer for a decode batch of at most 8 tokens in one call
    (moe_layer_decode): four launches, the same outputs as run_layer."""
    B.moe_layer_decode(buf.shape, x, w_router, bias, experts, shared, buf.topk_idx, buf.topk_w,
                       buf.counts, buf.offsets, buf.perm, buf.inv_perm, buf.active, buf.n_active,
                       buf.y, buf.y_shared, buf.out, buf.layer_workspace, stream)
    return buf.out
