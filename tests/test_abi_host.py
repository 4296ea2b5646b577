"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function the headers in include/ declare,
and reject malformed calls before enqueueing anything.  Every call below has
at least one defect, so none of them reaches a kernel launch: they are safe on
a machine with or without a GPU.
"""
import ctypes
import os
import re

import pytest

import int4_routed_expert_logits_amd as moe
from int4_routed_expert_logits_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

P = 1 << 20          # a 256-byte aligned stand-in address (never dereferenced)
MIS = P + 4          # misaligned for 16-byte checks


@pytest.fixture(scope="module")
def lib():
    return moe.load()


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported(lib):
    decl = declared_functions()
    assert decl == sorted(B.EXPORTS)
    for name in decl:
        assert hasattr(lib, name), name
    # and nothing declared is missing from the dynamic symbol table
    handle = ctypes.CDLL(moe.LIB_PATH)
    for name in decl:
        assert ctypes.cast(getattr(handle, name), ctypes.c_void_p).value


def shp(d=512, f=256, E=8, k=2, group=64, fs=0):
    return B.Shape(d, f, E, k, group, fs)


def test_expert_bytes(lib):
    assert lib.moe_expert_bytes(6144, 2048, 64) == 20_054_016
    assert lib.moe_expert_bytes(512, 256, 64) == 208_896
    assert lib.moe_expert_bytes(2048, 1024, 64) == 3_342_336
    assert lib.moe_expert_bytes(2048, 512, 64) == 1_671_168
    # group 32: MXFP4 blocks (one E8M0 byte per 32 codes), the same size
    assert lib.moe_expert_bytes(6144, 2048, 32) == 20_054_016
    assert lib.moe_expert_bytes(6144, 2048, 16) == 0
    assert lib.moe_expert_bytes(100, 2048, 64) == 0


def test_workspace_sizes(lib):
    s = shp(6144, 2048, 256, 8, 64, 2048)
    # float64 partial sums: 8 parts of d per logit for a 2048-token batch, 8 at T = 1
    assert moe.moe_route_workspace_bytes(s, 2048) == 2048 * 256 * 8 * 8
    assert moe.moe_route_workspace_bytes(s, 1) == 256 * 8 * 8
    assert moe.moe_ffn_workspace_bytes(s, 1, moe.MOE_PATH_DECODE_F32) >= (8 + 1) * 2048 * 4
    assert moe.moe_ffn_workspace_bytes(s, 2048, moe.MOE_PATH_PREFILL_BF16) >= 2048 * 9 * 2048 * 2
    for v in (moe.moe_route_workspace_bytes(s, 3), moe.moe_ffn_workspace_bytes(s, 3, 0)):
        assert v % 256 == 0
    assert moe.moe_route_workspace_bytes(shp(group=16), 4) == 0
    assert moe.moe_route_workspace_bytes(shp(group=32), 4) == moe.moe_route_workspace_bytes(shp(), 4)


def test_workspace_sizes_are_zero_for_token_counts_the_calls_reject(lib):
    """T * top_k may reach 2^24: the sizes there are exact (size_t, no 32-bit
    wrap), and one token more, or T < 0, gives 0 from every size function."""
    s = shp(8192, 8192, 1024, 32, 64, 8192)
    T = (1 << 24) // 32
    rows = T * 32 + T  # routed slots plus the shared expert's rows
    # the matrix-core router's parts of d: d / 768, at most 4 for E > 512
    assert moe.moe_route_workspace_bytes(s, T) == T * 1024 * 4 * 8
    assert moe.moe_ffn_workspace_bytes(s, T, moe.MOE_PATH_PREFILL_BF16) >= rows * 8192 * 2 > 2**38
    assert moe.moe_ffn_workspace_bytes(s, T, moe.MOE_PATH_DECODE_F32) > 0
    assert moe.moe_layer_decode_workspace_bytes(s, T) > 0
    for t in (T + 1, -1):
        assert moe.moe_route_workspace_bytes(s, t) == 0
        assert moe.moe_ffn_workspace_bytes(s, t, moe.MOE_PATH_DECODE_F32) == 0
        assert moe.moe_ffn_workspace_bytes(s, t, moe.MOE_PATH_PREFILL_BF16) == 0
        assert moe.moe_layer_decode_workspace_bytes(s, t) == 0
    # the cache's limit is T * top_k <= 1024
    assert moe.moe_cache_workspace_bytes(s, 32, 64) > 0
    assert moe.moe_cache_workspace_bytes(s, 33, 64) == 0
    assert moe.moe_cache_workspace_bytes(s, -1, 64) == 0


def test_status_strings(lib):
    for code in range(8):
        assert moe.moe_status_str(code)
    assert moe.moe_status_str(99) == "unknown status"


@pytest.mark.parametrize("shape,status", [
    (shp(d=0), B.MOE_ERR_SHAPE), (shp(d=96), B.MOE_ERR_SHAPE), (shp(f=-64), B.MOE_ERR_SHAPE),
    (shp(group=16), B.MOE_ERR_UNSUPPORTED), (shp(d=16384), B.MOE_ERR_UNSUPPORTED),
    (shp(E=2048, k=8), B.MOE_ERR_UNSUPPORTED), (shp(E=4, k=5), B.MOE_ERR_SHAPE),
    (shp(E=64, k=33), B.MOE_ERR_UNSUPPORTED), (shp(fs=128), B.MOE_ERR_UNSUPPORTED),
    (shp(k=0), B.MOE_ERR_SHAPE),
])
def test_bad_shapes_are_rejected_by_every_call(lib, shape, status):
    s = ctypes.byref(shape)
    assert lib.moe_route(s, 4, P, 0, P, None, P, P, P, 1 << 20, None) == status
    assert lib.moe_union(s, 4, P, P, P, P, P, P, P, None) == status
    assert lib.moe_expert_ffn(s, 4, P, 0, P, None, P, P, P, P, 0, P, None, P, 1 << 30, None) == status
    assert lib.moe_combine(s, 4, P, None, 0, P, P, P, 0, None) == status
    assert lib.moe_route_union(s, 4, P, 0, P, None, P, P, P, P, P, P, P, P, P, 1 << 20,
                               None) == status
    assert lib.moe_layer_decode(s, 4, P, 0, P, None, P, None, *([P] * 10), None, P, 0, P,
                                1 << 30, None) == status


def test_mxfp4_shapes_only_where_built(lib):
    """group 32 (MXFP4 blocks) is taken by the calls that do not depend on the
    block format and by both paths of moe_expert_ffn, with the int4 workspace
    sizes; the one-call layer and its workspace size refuse it."""
    mx = shp(group=32)
    s = ctypes.byref(mx)
    dec, pre = B.MOE_PATH_DECODE_F32, B.MOE_PATH_PREFILL_BF16
    assert moe.moe_ffn_workspace_bytes(mx, 4, dec) == moe.moe_ffn_workspace_bytes(shp(), 4, dec)
    assert moe.moe_ffn_workspace_bytes(mx, 4, pre) == moe.moe_ffn_workspace_bytes(shp(), 4, pre)
    assert moe.moe_ffn_workspace_bytes(mx, 4, pre) > 0
    assert moe.moe_layer_decode_workspace_bytes(mx, 4) == 0
    assert lib.moe_layer_decode(s, 4, P, 0, P, None, P, None, *([P] * 10), None, P, 0, P,
                                1 << 30, None) == B.MOE_ERR_UNSUPPORTED
    # both paths take it (here stopped by the NULL x, before any launch)
    for path in (dec, pre):
        assert lib.moe_expert_ffn(s, 4, None, 1, P, None, P, P, P, P, path, P, None, P, 1 << 30,
                                  None) == B.MOE_ERR_NULL


def test_null_shape(lib):
    assert lib.moe_route(None, 4, P, 0, P, None, P, P, P, 1 << 20, None) == B.MOE_ERR_NULL


def test_route_argument_checks(lib):
    s = ctypes.byref(shp())
    ws = 4 * 8 * 8
    assert lib.moe_route(s, -1, P, 0, P, None, P, P, P, ws, None) == B.MOE_ERR_SHAPE
    assert lib.moe_route(s, 4, P, 7, P, None, P, P, P, ws, None) == B.MOE_ERR_DTYPE
    assert lib.moe_route(s, 4, None, 0, P, None, P, P, P, ws, None) == B.MOE_ERR_NULL
    assert lib.moe_route(s, 4, P, 0, None, None, P, P, P, ws, None) == B.MOE_ERR_NULL
    assert lib.moe_route(s, 4, P, 0, P, None, P, P, None, ws, None) == B.MOE_ERR_NULL
    assert lib.moe_route(s, 4, MIS, 0, P, None, P, P, P, ws, None) == B.MOE_ERR_ALIGN
    assert lib.moe_route(s, 4, P, 0, P, None, P, P, P + 16, ws, None) == B.MOE_ERR_ALIGN
    assert lib.moe_route(s, 4, P, 0, P, None, P, P, P, ws - 1, None) == B.MOE_ERR_WORKSPACE
    # an empty batch is a no-op
    assert lib.moe_route(s, 0, None, 0, None, None, None, None, None, 0, None) == B.MOE_OK


def test_route_union_argument_checks(lib):
    s = ctypes.byref(shp())
    ws = 4 * 8 * 8

    def call(T=4, x=P, dt=0, w=P, topk_idx=P, counts=P, perm=P, n_active=P, ws_ptr=P, nbytes=ws):
        return lib.moe_route_union(s, T, x, dt, w, None, topk_idx, P, counts, P, perm, P, P,
                                   n_active, ws_ptr, nbytes, None)

    assert call(T=-1) == B.MOE_ERR_SHAPE
    assert call(dt=7) == B.MOE_ERR_DTYPE
    assert call(x=None) == B.MOE_ERR_NULL
    assert call(w=None) == B.MOE_ERR_NULL
    assert call(topk_idx=None) == B.MOE_ERR_NULL
    assert call(counts=None) == B.MOE_ERR_NULL
    assert call(perm=None) == B.MOE_ERR_NULL
    assert call(n_active=None) == B.MOE_ERR_NULL
    assert call(ws_ptr=None) == B.MOE_ERR_NULL
    assert call(x=MIS) == B.MOE_ERR_ALIGN
    assert call(ws_ptr=P + 16) == B.MOE_ERR_ALIGN
    assert call(counts=P + 2) == B.MOE_ERR_ALIGN
    assert call(nbytes=ws - 1) == B.MOE_ERR_WORKSPACE
    assert call(T=1 << 24) == B.MOE_ERR_UNSUPPORTED


def test_layer_decode_argument_checks(lib):
    s = ctypes.byref(shp())
    big = 1 << 30
    ok = dict(T=4, x=P, xdt=0, w=P, bias=None, ex=P, sh=None, idx=P, tw=P, cnt=P, off=P, perm=P,
              inv=P, act=P, na=P, y=P, ys=None, out=P, odt=0, ws=P, wsb=big)

    def call(shape=s, **kw):
        a = dict(ok, **kw)
        return lib.moe_layer_decode(shape, a["T"], a["x"], a["xdt"], a["w"], a["bias"], a["ex"],
                                    a["sh"], a["idx"], a["tw"], a["cnt"], a["off"], a["perm"],
                                    a["inv"], a["act"], a["na"], a["y"], a["ys"], a["out"],
                                    a["odt"], a["ws"], a["wsb"], None)

    assert call(T=-1) == B.MOE_ERR_SHAPE
    assert call(xdt=4) == B.MOE_ERR_DTYPE
    assert call(odt=4) == B.MOE_ERR_DTYPE
    # only small decode batches: at most 8 tokens, 64 slots and 256 experts
    assert call(T=9) == B.MOE_ERR_UNSUPPORTED
    assert call(shape=ctypes.byref(shp(E=64, k=16)), T=5) == B.MOE_ERR_UNSUPPORTED
    assert call(shape=ctypes.byref(shp(E=512, k=8)), T=1) == B.MOE_ERR_UNSUPPORTED
    for name in ("x", "w", "ex", "idx", "tw", "cnt", "off", "perm", "inv", "act", "na", "y",
                 "out", "ws"):
        assert call(**{name: None}) == B.MOE_ERR_NULL, name
    assert call(sh=P) == B.MOE_ERR_NULL            # shared block given but no shared expert
    s2 = ctypes.byref(shp(fs=256))
    assert call(shape=s2, sh=P) == B.MOE_ERR_NULL  # y_shared missing
    assert call(shape=s2, ys=P) == B.MOE_ERR_NULL  # shared block missing
    assert call(x=MIS) == B.MOE_ERR_ALIGN
    assert call(ex=MIS) == B.MOE_ERR_ALIGN
    assert call(y=MIS) == B.MOE_ERR_ALIGN
    assert call(out=MIS) == B.MOE_ERR_ALIGN
    assert call(cnt=P + 2) == B.MOE_ERR_ALIGN
    assert call(ws=P + 64) == B.MOE_ERR_ALIGN
    need = moe.moe_layer_decode_workspace_bytes(shp(), 4)
    assert need == moe.moe_route_workspace_bytes(shp(), 4) + moe.moe_ffn_workspace_bytes(shp(), 4, 0)
    assert call(wsb=need - 1) == B.MOE_ERR_WORKSPACE


def test_quantize_argument_checks(lib):
    q = lambda N=4, K=128, w=P, dt=1, mode=0, c=P, sc=P: lib.moe_quantize(N, K, w, dt, mode, c, sc, None)
    assert q(N=-1) == B.MOE_ERR_SHAPE
    assert q(K=0) == B.MOE_ERR_SHAPE
    assert q(K=96) == B.MOE_ERR_SHAPE
    assert q(K=1 << 17) == B.MOE_ERR_UNSUPPORTED
    assert q(mode=2) == B.MOE_ERR_UNSUPPORTED
    assert q(dt=5) == B.MOE_ERR_DTYPE
    assert q(w=None) == B.MOE_ERR_NULL
    assert q(c=None) == B.MOE_ERR_NULL
    assert q(sc=None) == B.MOE_ERR_NULL
    assert q(w=MIS) == B.MOE_ERR_ALIGN
    assert q(c=P + 2) == B.MOE_ERR_ALIGN
    assert q(sc=P + 1) == B.MOE_ERR_ALIGN
    assert q(N=0, w=None, c=None, sc=None) == B.MOE_OK


def test_pack_argument_checks(lib):
    s = ctypes.byref(shp())
    bb = lib.moe_expert_bytes(512, 256, 64)  # the block of shp()
    assert lib.moe_pack_experts(s, -1, P, P + 4 * bb, None) == B.MOE_ERR_SHAPE
    assert lib.moe_pack_experts(s, 2, None, P, None) == B.MOE_ERR_NULL
    assert lib.moe_pack_experts(s, 2, P, None, None) == B.MOE_ERR_NULL
    assert lib.moe_pack_experts(s, 2, MIS, P + 4 * bb, None) == B.MOE_ERR_ALIGN
    assert lib.moe_pack_experts(s, 2, P, P + 4 * bb + 8, None) == B.MOE_ERR_ALIGN
    # source and destination overlapping by one 16-byte piece, either way round
    assert lib.moe_pack_experts(s, 2, P, P + 2 * bb - 16, None) == B.MOE_ERR_SHAPE
    assert lib.moe_pack_experts(s, 2, P + 2 * bb - 16, P, None) == B.MOE_ERR_SHAPE
    assert lib.moe_pack_experts(ctypes.byref(shp(group=16)), 2, P, P + 4 * bb, None) == \
        B.MOE_ERR_UNSUPPORTED
    assert lib.moe_pack_experts(s, 0, None, None, None) == B.MOE_OK  # nothing to pack


def test_stream_read_argument_checks(lib):
    blocks = (ctypes.c_void_p * 3)(P, P + 4096, P + 8192)
    r = lambda bl=blocks, n=3, bb=4096, wg=12, sink=P: lib.moe_measure_stream_read(
        bl, n, bb, wg, sink, None)
    assert r(bl=None) == B.MOE_ERR_NULL
    assert r(sink=None) == B.MOE_ERR_NULL
    assert r(n=0) == B.MOE_ERR_SHAPE
    assert r(n=65) == B.MOE_ERR_SHAPE
    assert r(bb=0) == B.MOE_ERR_SHAPE
    assert r(bb=4100) == B.MOE_ERR_SHAPE
    assert r(wg=65537) == B.MOE_ERR_SHAPE
    # fewer workgroups than blocks: sink (sized by workgroups) could not hold
    # one word per block
    assert r(wg=2) == B.MOE_ERR_SHAPE
    assert r(bl=(ctypes.c_void_p * 3)(P, None, P)) == B.MOE_ERR_NULL
    assert r(bl=(ctypes.c_void_p * 3)(P, MIS, P)) == B.MOE_ERR_ALIGN
    assert r(sink=P + 2) == B.MOE_ERR_ALIGN


def test_union_argument_checks(lib):
    s = ctypes.byref(shp())
    assert lib.moe_union(s, 4, None, P, P, P, P, P, P, None) == B.MOE_ERR_NULL
    assert lib.moe_union(s, 4, P, None, P, P, P, P, P, None) == B.MOE_ERR_NULL
    assert lib.moe_union(s, 4, P, P, P, P, P, P, None, None) == B.MOE_ERR_NULL
    assert lib.moe_union(s, 4, P + 2, P, P, P, P, P, P, None) == B.MOE_ERR_ALIGN
    assert lib.moe_union(s, -3, P, P, P, P, P, P, P, None) == B.MOE_ERR_SHAPE
    assert lib.moe_union(s, 1 << 24, P, P, P, P, P, P, P, None) == B.MOE_ERR_UNSUPPORTED


def test_ffn_argument_checks(lib):
    s = ctypes.byref(shp())
    big = 1 << 30
    dec, pre = B.MOE_PATH_DECODE_F32, B.MOE_PATH_PREFILL_BF16
    ok_args = dict(x=P, xdt=0, ex=P, sh=None, off=P, perm=P, act=P, na=P, path=dec, y=P, ys=None, ws=P, wsb=big)

    def call(**kw):
        a = dict(ok_args, **kw)
        return lib.moe_expert_ffn(s, 4, a["x"], a["xdt"], a["ex"], a["sh"], a["off"], a["perm"],
                                  a["act"], a["na"], a["path"], a["y"], a["ys"], a["ws"], a["wsb"], None)
    # f32 activations on the bf16 prefill path are rejected, never rounded
    assert call(path=pre, xdt=0) == B.MOE_ERR_DTYPE
    assert call(path=5) == B.MOE_ERR_UNSUPPORTED
    assert call(xdt=3) == B.MOE_ERR_DTYPE
    assert call(x=None) == B.MOE_ERR_NULL
    assert call(ex=None) == B.MOE_ERR_NULL
    assert call(na=None) == B.MOE_ERR_NULL
    assert call(ws=None) == B.MOE_ERR_NULL
    assert call(sh=P) == B.MOE_ERR_NULL            # shared block given but no shared expert
    assert call(ex=MIS) == B.MOE_ERR_ALIGN
    assert call(y=MIS) == B.MOE_ERR_ALIGN
    assert call(ws=P + 64) == B.MOE_ERR_ALIGN
    assert call(wsb=16) == B.MOE_ERR_WORKSPACE
    s2 = ctypes.byref(shp(fs=256))
    assert lib.moe_expert_ffn(s2, 4, P, 0, P, None, P, P, P, P, dec, P, P, P, big, None) == B.MOE_ERR_NULL
    assert lib.moe_expert_ffn(s2, 4, P, 0, P, P, P, P, P, P, dec, P, None, P, big, None) == B.MOE_ERR_NULL
    assert lib.moe_expert_ffn(s, 0, None, 0, None, None, None, None, None, None, dec, None, None, None, 0, None) == B.MOE_OK


def test_combine_argument_checks(lib):
    s = ctypes.byref(shp())
    assert lib.moe_combine(s, 4, P, None, 2, P, P, P, 0, None) == B.MOE_ERR_DTYPE
    assert lib.moe_combine(s, 4, P, None, 0, P, P, P, 9, None) == B.MOE_ERR_DTYPE
    assert lib.moe_combine(s, 4, None, None, 0, P, P, P, 0, None) == B.MOE_ERR_NULL
    assert lib.moe_combine(s, 4, P, P, 0, P, P, P, 0, None) == B.MOE_ERR_NULL   # y_shared without a shared expert
    assert lib.moe_combine(s, 4, P, None, 0, P, P, MIS, 0, None) == B.MOE_ERR_ALIGN
    assert lib.moe_combine(s, 0, None, None, 0, None, None, None, 0, None) == B.MOE_OK


def test_binding_names_match_the_c_entry_points():
    for name in B.EXPORTS:
        assert callable(getattr(moe, name)), name


def test_layer_decode_static_argument_checks(lib):
    """The workspace-free decode layer checks its arguments as
    moe_layer_decode does, before it looks up its static array."""
    s = ctypes.byref(shp())
    ok = dict(T=4, x=P, xdt=0, w=P, bias=None, ex=P, sh=None, idx=P, tw=P, cnt=P, off=P, perm=P,
              inv=P, act=P, na=P, y=P, ys=None, out=P, odt=0)

    def call(shape=s, **kw):
        a = dict(ok, **kw)
        return lib.moe_layer_decode_static(shape, a["T"], a["x"], a["xdt"], a["w"], a["bias"],
                                           a["ex"], a["sh"], a["idx"], a["tw"], a["cnt"], a["off"],
                                           a["perm"], a["inv"], a["act"], a["na"], a["y"], a["ys"],
                                           a["out"], a["odt"], None)

    assert lib.moe_layer_decode_static_max_bytes() == 4 << 20
    assert call(shape=None) == B.MOE_ERR_NULL
    assert call(T=-1) == B.MOE_ERR_SHAPE
    assert call(xdt=4) == B.MOE_ERR_DTYPE
    assert call(T=9) == B.MOE_ERR_UNSUPPORTED
    assert call(shape=ctypes.byref(shp(group=32))) == B.MOE_ERR_UNSUPPORTED
    for name in ("x", "w", "ex", "idx", "tw", "cnt", "perm", "y", "out"):
        assert call(**{name: None}) == B.MOE_ERR_NULL, name
    assert call(x=MIS) == B.MOE_ERR_ALIGN
    # every supported shape fits the array: the largest needs ~2.4 MiB
    big = shp(d=8192, f=8192, E=256, k=8, fs=8192)
    assert moe.moe_layer_decode_workspace_bytes(big, 8) <= lib.moe_layer_decode_static_max_bytes()
