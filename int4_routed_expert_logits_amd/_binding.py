"""ctypes binding of libmoe_int4.so: one Python function per C entry point,
with the same name.  Argument marshalling only -- every step of the layer
runs in the library's HIP kernels.  PyTorch supplies device memory and the
current HIP stream.

Loading fails loudly when the library has not been built; there is no other
implementation behind these functions.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_int32, c_size_t, c_void_p, POINTER

LIB_NAME = "libmoe_int4.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_ALIGN = 0, 1, 2, 3, 4
MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 5, 6, 7
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_DTYPE",
                4: "MOE_ERR_ALIGN", 5: "MOE_ERR_UNSUPPORTED", 6: "MOE_ERR_WORKSPACE",
                7: "MOE_ERR_HIP"}
MOE_F32, MOE_BF16 = 0, 1
MOE_PATH_DECODE_F32, MOE_PATH_PREFILL_BF16 = 0, 1
MOE_QUANT_GS64, MOE_QUANT_ROW = 0, 1

# every function include/moe_int4.h declares
EXPORTS = ("moe_expert_bytes", "moe_pack_experts", "moe_quantize", "moe_route_workspace_bytes",
           "moe_route", "moe_union", "moe_route_union", "moe_ffn_workspace_bytes",
           "moe_expert_ffn", "moe_combine", "moe_layer_decode_workspace_bytes",
           "moe_layer_decode", "moe_layer_decode_static", "moe_layer_decode_static_max_bytes",
           "moe_cache_create", "moe_cache_destroy", "moe_cache_pin",
           "moe_cache_plan", "moe_cache_stats", "moe_cache_last_fetch", "moe_cache_unplan_last",
           "moe_cache_workspace_bytes",
           "moe_cache_layer_decode", "moe_status_str", "moe_measure_stream_read")


class Shape(ctypes.Structure):
    """moe_shape: d, f, n_experts, top_k, group, f_shared (all int32)."""
    _fields_ = [("d", c_int32), ("f", c_int32), ("n_experts", c_int32), ("top_k", c_int32),
                ("group", c_int32), ("f_shared", c_int32)]

    def __repr__(self):
        return (f"Shape(d={self.d}, f={self.f}, n_experts={self.n_experts}, top_k={self.top_k}, "
                f"group={self.group}, f_shared={self.f_shared})")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)} ({_status_text(status)})")


_lib = None


def load():
    """Load the shared library (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m int4_routed_expert_logits_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    sp = POINTER(Shape)
    lib.moe_expert_bytes.argtypes = [c_int32, c_int32, c_int32]
    lib.moe_expert_bytes.restype = c_size_t
    lib.moe_route_workspace_bytes.argtypes = [sp, c_int32]
    lib.moe_route_workspace_bytes.restype = c_size_t
    lib.moe_ffn_workspace_bytes.argtypes = [sp, c_int32, c_int32]
    lib.moe_ffn_workspace_bytes.restype = c_size_t
    lib.moe_route.argtypes = [sp, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_void_p, c_size_t, c_void_p]
    lib.moe_route.restype = c_int32
    lib.moe_union.argtypes = [sp, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_void_p, c_void_p]
    lib.moe_union.restype = c_int32
    lib.moe_route_union.argtypes = [sp, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_size_t, c_void_p]
    lib.moe_route_union.restype = c_int32
    lib.moe_expert_ffn.argtypes = [sp, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                   c_void_p, c_size_t, c_void_p]
    lib.moe_expert_ffn.restype = c_int32
    lib.moe_combine.argtypes = [sp, c_int32, c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                c_void_p, c_int32, c_void_p]
    lib.moe_combine.restype = c_int32
    lib.moe_layer_decode_workspace_bytes.argtypes = [sp, c_int32]
    lib.moe_layer_decode_workspace_bytes.restype = c_size_t
    lib.moe_layer_decode.argtypes = ([sp, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                      c_void_p] + [c_void_p] * 11 + [c_int32, c_void_p, c_size_t,
                                                                     c_void_p])
    lib.moe_layer_decode.restype = c_int32
    lib.moe_layer_decode_static.argtypes = ([sp, c_int32, c_void_p, c_int32, c_void_p, c_void_p,
                                             c_void_p, c_void_p] + [c_void_p] * 11 +
                                            [c_int32, c_void_p])
    lib.moe_layer_decode_static.restype = c_int32
    lib.moe_measure_stream_read.argtypes = [c_void_p, c_int32, c_size_t, c_int32, c_void_p,
                                            c_void_p]
    lib.moe_measure_stream_read.restype = c_int32
    lib.moe_layer_decode_static_max_bytes.argtypes = []
    lib.moe_layer_decode_static_max_bytes.restype = c_size_t
    vp = c_void_p
    lib.moe_cache_create.argtypes = [sp, c_int32, vp, vp, POINTER(vp)]
    lib.moe_cache_create.restype = c_int32
    lib.moe_cache_destroy.argtypes = [vp]
    lib.moe_cache_destroy.restype = None
    lib.moe_cache_pin.argtypes = [vp, c_int32, c_int32]
    lib.moe_cache_pin.restype = c_int32
    lib.moe_cache_plan.argtypes = [vp, c_int32, vp, vp, vp, vp, vp]
    lib.moe_cache_plan.restype = c_int32
    lib.moe_cache_stats.argtypes = [vp, vp, vp, vp]
    lib.moe_cache_stats.restype = c_int32
    lib.moe_cache_last_fetch.argtypes = [vp, c_int32, vp, vp, vp]
    lib.moe_cache_last_fetch.restype = c_int32
    lib.moe_cache_unplan_last.argtypes = [vp]
    lib.moe_cache_unplan_last.restype = c_int32
    lib.moe_cache_workspace_bytes.argtypes = [sp, c_int32, c_int32]
    lib.moe_cache_workspace_bytes.restype = c_size_t
    lib.moe_cache_layer_decode.argtypes = [vp, c_int32, vp, c_int32, vp, vp, vp, vp, vp, vp, vp,
                                           vp, c_int32, vp, c_size_t, vp, vp]
    lib.moe_cache_layer_decode.restype = c_int32
    lib.moe_pack_experts.argtypes = [sp, ctypes.c_int64, c_void_p, c_void_p, c_void_p]
    lib.moe_pack_experts.restype = c_int32
    lib.moe_quantize.argtypes = [c_int32, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                 c_void_p]
    lib.moe_quantize.restype = c_int32
    lib.moe_status_str.argtypes = [c_int32]
    lib.moe_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _status_text(status: int) -> str:
    try:
        return load().moe_status_str(status).decode()
    except Exception:  # pragma: no cover - only when the library itself is missing
        return "?"


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

def _ptr(t):
    """Device address of a tensor (None -> NULL).  Raw integers pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _dtype(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)


def _shape(shape):
    if isinstance(shape, Shape):
        return shape
    return Shape(*shape)


# ----------------------------------------------------------------------------
# the C entry points, one to one
# ----------------------------------------------------------------------------

def moe_expert_bytes(d: int, f: int, group: int = 64) -> int:
    return load().moe_expert_bytes(d, f, group)


def moe_pack_experts(shape, n_blocks: int, src, dst, stream=None):
    """Canonical expert blocks (uint8 device tensor) -> packed blocks."""
    sh = _shape(shape)
    _check("moe_pack_experts", load().moe_pack_experts(ctypes.byref(sh), n_blocks, _ptr(src),
                                                       _ptr(dst), _stream(stream)))


def moe_quantize(w, mode, codes, scales, stream=None):
    """w [N, K] bf16/f32 -> codes [N, K/2] uint8 and float16 scales
    ([N, K/64] for MOE_QUANT_GS64, [N] for MOE_QUANT_ROW)."""
    n, k = w.shape
    _check("moe_quantize", load().moe_quantize(n, k, _ptr(w), _dtype(w), mode, _ptr(codes),
                                               _ptr(scales), _stream(stream)))


def moe_route_workspace_bytes(shape, T: int) -> int:
    return load().moe_route_workspace_bytes(ctypes.byref(_shape(shape)), T)


def moe_ffn_workspace_bytes(shape, T: int, path: int) -> int:
    return load().moe_ffn_workspace_bytes(ctypes.byref(_shape(shape)), T, path)


def moe_layer_decode_workspace_bytes(shape, T: int) -> int:
    return load().moe_layer_decode_workspace_bytes(ctypes.byref(_shape(shape)), T)


def moe_status_str(status: int) -> str:
    return load().moe_status_str(status).decode()


def moe_route(shape, x, w_router, bias, topk_idx, topk_w, workspace, stream=None):
    """x [T, d] bf16/f32; writes topk_idx [T, k] int32 and topk_w [T, k] f32."""
    sh = _shape(shape)
    _check("moe_route", load().moe_route(
        ctypes.byref(sh), x.shape[0], _ptr(x), _dtype(x), _ptr(w_router), _ptr(bias),
        _ptr(topk_idx), _ptr(topk_w), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def moe_union(shape, T, topk_idx, counts, offsets, perm, inv_perm, active, n_active, stream=None):
    sh = _shape(shape)
    _check("moe_union", load().moe_union(
        ctypes.byref(sh), T, _ptr(topk_idx), _ptr(counts), _ptr(offsets), _ptr(perm),
        _ptr(inv_perm), _ptr(active), _ptr(n_active), _stream(stream)))


def moe_route_union(shape, x, w_router, bias, topk_idx, topk_w, counts, offsets, perm, inv_perm,
                    active, n_active, workspace, stream=None):
    """moe_route then moe_union in one call (same outputs)."""
    sh = _shape(shape)
    _check("moe_route_union", load().moe_route_union(
        ctypes.byref(sh), x.shape[0], _ptr(x), _dtype(x), _ptr(w_router), _ptr(bias),
        _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv_perm),
        _ptr(active), _ptr(n_active), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_expert_ffn(shape, x, experts, shared, offsets, perm, active, n_active, path, y, y_shared,
                   workspace, stream=None):
    sh = _shape(shape)
    _check("moe_expert_ffn", load().moe_expert_ffn(
        ctypes.byref(sh), x.shape[0], _ptr(x), _dtype(x), _ptr(experts), _ptr(shared),
        _ptr(offsets), _ptr(perm), _ptr(active), _ptr(n_active), path, _ptr(y), _ptr(y_shared),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_combine(shape, y, y_shared, inv_perm, topk_w, out, stream=None):
    sh = _shape(shape)
    _check("moe_combine", load().moe_combine(
        ctypes.byref(sh), out.shape[0], _ptr(y), _ptr(y_shared), _dtype(y), _ptr(inv_perm),
        _ptr(topk_w), _ptr(out), _dtype(out), _stream(stream)))


def moe_layer_decode(shape, x, w_router, bias, experts, shared, topk_idx, topk_w, counts, offsets,
                     perm, inv_perm, active, n_active, y, y_shared, out, workspace, stream=None):
    """The whole layer for a decode batch of T <= 8 tokens (route, union,
    expert FFN, combine): the same outputs as the separate calls."""
    sh = _shape(shape)
    _check("moe_layer_decode", load().moe_layer_decode(
        ctypes.byref(sh), x.shape[0], _ptr(x), _dtype(x), _ptr(w_router), _ptr(bias),
        _ptr(experts), _ptr(shared), _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets),
        _ptr(perm), _ptr(inv_perm), _ptr(active), _ptr(n_active), _ptr(y), _ptr(y_shared),
        _ptr(out), _dtype(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def moe_layer_decode_static_max_bytes() -> int:
    return load().moe_layer_decode_static_max_bytes()


def moe_layer_decode_static(shape, x, w_router, bias, experts, shared, topk_idx, topk_w, counts,
                            offsets, perm, inv_perm, active, n_active, y, y_shared, out,
                            stream=None):
    """moe_layer_decode without a workspace: the library's static per-GPU
    scratch array stands in for it (include/moe_int4_static.h)."""
    sh = _shape(shape)
    _check("moe_layer_decode_static", load().moe_layer_decode_static(
        ctypes.byref(sh), x.shape[0], _ptr(x), _dtype(x), _ptr(w_router), _ptr(bias),
        _ptr(experts), _ptr(shared), _ptr(topk_idx), _ptr(topk_w), _ptr(counts), _ptr(offsets),
        _ptr(perm), _ptr(inv_perm), _ptr(active), _ptr(n_active), _ptr(y), _ptr(y_shared),
        _ptr(out), _dtype(out), _stream(stream)))


def moe_measure_stream_read(block_ptrs, block_bytes: int, workgroups: int, sink, stream=None):
    """Calibration read of the device blocks at block_ptrs (ints) once
    (include/moe_int4_measure.h); sink: a device int32 tensor of at least
    `workgroups` entries."""
    arr = (c_void_p * len(block_ptrs))(*block_ptrs)
    _check("moe_measure_stream_read", load().moe_measure_stream_read(
        arr, len(block_ptrs), block_bytes, workgroups, _ptr(sink), _stream(stream)))


# ----------------------------------------------------------------------------
# per-layer expert cache
# ----------------------------------------------------------------------------

def moe_cache_create(shape, n_slots: int, device_slots=None, host_blocks=None) -> int:
    """Handle of a new cache (device_slots / host_blocks: tensors or None
    for a planning-only cache)."""
    h = c_void_p()
    _check("moe_cache_create", load().moe_cache_create(
        ctypes.byref(_shape(shape)), n_slots, _ptr(device_slots), _ptr(host_blocks),
        ctypes.byref(h)))
    return h.value


def moe_cache_destroy(cache: int):
    load().moe_cache_destroy(cache)


def moe_cache_pin(cache: int, expert: int, pinned: bool = True):
    _check("moe_cache_pin", load().moe_cache_pin(cache, expert, 1 if pinned else 0))


def moe_cache_plan(cache: int, experts):
    """One policy step on a planning-only cache: experts (host ints) ->
    (slot_of per entry, fetched experts in placement order, the expert each
    displaced or -1)."""
    import numpy as np
    e = np.ascontiguousarray(np.asarray(experts, dtype=np.int32))
    n = e.size
    slot_of = np.empty(max(n, 1), np.int32)
    fetched = np.empty(max(n, 1), np.int32)
    evicted = np.empty(max(n, 1), np.int32)
    nf = c_int32(0)
    _check("moe_cache_plan", load().moe_cache_plan(
        cache, n, e.ctypes.data, slot_of.ctypes.data, fetched.ctypes.data, evicted.ctypes.data,
        ctypes.addressof(nf)))
    k = nf.value
    return slot_of[:n].copy(), fetched[:k].copy(), evicted[:k].copy()


def moe_cache_stats(cache: int):
    """(hits, misses, bytes fetched) since creation."""
    h, m, b = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check("moe_cache_stats", load().moe_cache_stats(cache, ctypes.addressof(h),
                                                     ctypes.addressof(m), ctypes.addressof(b)))
    return h.value, m.value, b.value


def moe_cache_last_fetch(cache: int, capacity: int):
    """The latest step's fetched experts in placement order and the expert
    each displaced (-1 for an empty slot): (fetched, evicted) lists."""
    f = (ctypes.c_int32 * max(capacity, 1))()
    e = (ctypes.c_int32 * max(capacity, 1))()
    n = ctypes.c_int32()
    _check("moe_cache_last_fetch", load().moe_cache_last_fetch(
        cache, capacity, ctypes.addressof(f), ctypes.addressof(e), ctypes.addressof(n)))
    return list(f[:n.value]), list(e[:n.value])


def moe_cache_unplan_last(cache: int) -> None:
    """Undo the latest step's placements (its fetched slots become empty)."""
    _check("moe_cache_unplan_last", load().moe_cache_unplan_last(cache))


def moe_cache_workspace_bytes(shape, T: int, n_slots: int) -> int:
    return load().moe_cache_workspace_bytes(ctypes.byref(_shape(shape)), T, n_slots)


def moe_cache_layer_decode(cache: int, x, w_router, bias, shared, topk_idx, topk_w, y, y_shared,
                           out, workspace, stream=None, copy_stream=None):
    """One decode step of the layer through the cache (copies of missing
    experts on copy_stream, overlapped with the resident experts' FFN)."""
    _check("moe_cache_layer_decode", load().moe_cache_layer_decode(
        cache, x.shape[0], _ptr(x), _dtype(x), _ptr(w_router), _ptr(bias), _ptr(shared),
        _ptr(topk_idx), _ptr(topk_w), _ptr(y), _ptr(y_shared), _ptr(out), _dtype(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream),
        _stream(copy_stream) if copy_stream is not None else _stream(stream)))
