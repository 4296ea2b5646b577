"""The library's expert cache policy against the reference model (CPU only).

moe_cache_plan runs the C++ policy on a planning-only cache (no device
memory, no GPU); every decision -- slot per routing entry, fetched experts in
placement order, the expert each displaced -- must equal the reference
model's, step for step, over long skewed traces with pins.  Also the cache
calls' argument checks, none of which reaches the GPU.
"""
import ctypes

import numpy as np
import pytest

import int4_routed_expert_logits_amd as moe
from int4_routed_expert_logits_amd import _binding as B
from oracle.expert_cache import ExpertCache

P = 1 << 20


def shp(d=512, f=256, E=256, k=8, fs=0):
    return B.Shape(d, f, E, k, 64, fs)


def zipf_steps(rng, E, k, steps, s=1.1):
    """k distinct experts per step, drawn with Zipf(s) popularity over a
    random order of the E experts."""
    order = rng.permutation(E)
    p = 1.0 / np.arange(1, E + 1) ** s
    p /= p.sum()
    for _ in range(steps):
        yield order[rng.choice(E, size=k, replace=False, p=p)]


@pytest.mark.parametrize("E,k,slots,T,pins,seed", [
    (256, 8, 40, 1, (), 0), (256, 8, 64, 1, (3, 100, 200), 1), (64, 8, 12, 1, (0,), 2),
    (256, 8, 80, 4, (7, 9), 3), (8, 2, 2, 1, (), 4), (1024, 8, 300, 2, (1, 2, 3, 500), 5),
])
def test_policy_matches_the_reference_model(E, k, slots, T, pins, seed):
    rng = np.random.default_rng(seed)
    h = moe.moe_cache_create(shp(E=E, k=k), slots)
    ref = ExpertCache(slots)
    try:
        for e in pins:
            moe.moe_cache_pin(h, e)
            ref.pin(e)
        gen = zipf_steps(rng, E, k, 400 * T)
        for step in range(400):
            ids = np.concatenate([next(gen) for _ in range(T)]).astype(np.int32)
            if step == 200 and pins:  # unpin one half-way
                moe.moe_cache_pin(h, pins[0], False)
                ref.pin(pins[0], False)
            slot_of, fetched, evicted = moe.moe_cache_plan(h, ids)
            placed, rf, rev = ref.step(ids)
            assert slot_of.tolist() == [placed[int(e)] for e in ids]
            assert fetched.tolist() == rf
            assert evicted.tolist() == [-1 if rev[e] is None else rev[e] for e in rf]
            # the latest-step record the GPU tests read after a decode step
            assert moe.moe_cache_last_fetch(h, E) == (fetched.tolist(), evicted.tolist())
        hits, misses, nbytes = moe.moe_cache_stats(h)
        assert (hits, misses, nbytes) == (ref.hits, ref.misses, 0)
    finally:
        moe.moe_cache_destroy(h)


def test_a_step_that_cannot_fit_leaves_the_state_unchanged():
    h = moe.moe_cache_create(shp(E=16, k=2), 4)
    try:
        moe.moe_cache_pin(h, 0)
        moe.moe_cache_pin(h, 1)
        moe.moe_cache_plan(h, [0, 1])
        moe.moe_cache_plan(h, [2, 3])
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_cache_plan(h, [0, 4, 5, 6])  # three misses, two evictable slots
        assert ei.value.status == B.MOE_ERR_UNSUPPORTED
        slot_of, fetched, _ = moe.moe_cache_plan(h, [2, 3])
        assert fetched.size == 0  # 2 and 3 still resident
        assert moe.moe_cache_last_fetch(h, 16) == ([], [])
        moe.moe_cache_plan(h, [0, 9])
        assert moe.moe_cache_last_fetch(h, 16) == ([9], [2])  # 2 and 3 tie; lower slot
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_cache_last_fetch(h, 0)  # one entry does not fit in none
        assert ei.value.status == B.MOE_ERR_SHAPE
    finally:
        moe.moe_cache_destroy(h)


def test_undoing_a_step_empties_its_slots_and_keeps_the_rest():
    """What a failed copy leaves behind (moe_cache_layer_decode undoes a step
    whose copies cannot be queued the same way): the step's fetched experts
    lose their slots and their misses, the experts they displaced stay
    evicted, the hits and every other mapping stand, and the next step
    places into the freed slots as into any empty slot."""
    h = moe.moe_cache_create(shp(E=16, k=2), 4)
    ref = ExpertCache(4)
    try:
        for step in ([0, 1], [2, 3], [0, 2]):  # fills the four slots, then two hits
            moe.moe_cache_plan(h, step)
            ref.step(np.array(step))
        assert moe.moe_cache_stats(h) == (2, 4, 0)
        slot_of, fetched, evicted = moe.moe_cache_plan(h, [0, 4, 5])  # 4, 5 evict 1, 3
        assert list(fetched) == [4, 5] and list(evicted) == [1, 3]
        moe.moe_cache_unplan_last(h)
        assert moe.moe_cache_last_fetch(h, 16) == ([], [])
        assert moe.moe_cache_stats(h) == (3, 4, 0)  # the hit on 0 stands, 4 and 5 do not count
        moe.moe_cache_unplan_last(h)  # nothing recorded: no change
        assert moe.moe_cache_stats(h) == (3, 4, 0)
        # 0 and 2 are still resident; 1, 3, 4, 5 are not
        slot_of, fetched, _ = moe.moe_cache_plan(h, [0, 2])
        assert fetched.size == 0 and sorted(slot_of.tolist()) == sorted(set(slot_of.tolist()))
        slot_of, fetched, evicted = moe.moe_cache_plan(h, [1, 3])
        assert list(fetched) == [1, 3] and list(evicted) == [-1, -1]  # the freed slots
        assert moe.moe_cache_stats(h) == (5, 6, 0)
    finally:
        moe.moe_cache_destroy(h)


def test_cache_argument_checks():
    lib = moe.load()
    h = ctypes.c_void_p()
    s = shp()
    assert lib.moe_cache_create(ctypes.byref(s), 40, None, None, None) == B.MOE_ERR_NULL
    assert lib.moe_cache_create(ctypes.byref(s), 7, None, None, ctypes.byref(h)) == B.MOE_ERR_SHAPE
    assert lib.moe_cache_create(ctypes.byref(s), 257, None, None, ctypes.byref(h)) == B.MOE_ERR_SHAPE
    assert lib.moe_cache_create(ctypes.byref(s), 40, P, None, ctypes.byref(h)) == B.MOE_ERR_NULL
    assert lib.moe_cache_create(ctypes.byref(s), 40, P + 16, P, ctypes.byref(h)) == B.MOE_ERR_ALIGN
    assert lib.moe_cache_create(ctypes.byref(shp(d=96)), 40, None, None, ctypes.byref(h)) == B.MOE_ERR_SHAPE
    # a cache over (never dereferenced) stand-in buffers: plan is refused, so
    # its slots can never disagree with what the device holds
    assert lib.moe_cache_create(ctypes.byref(s), 40, P, P, ctypes.byref(h)) == B.MOE_OK
    c = h.value
    try:
        nf = ctypes.c_int32()
        e = (ctypes.c_int32 * 1)(3)
        o = (ctypes.c_int32 * 1)()
        assert lib.moe_cache_plan(c, 1, e, o, o, o, ctypes.byref(nf)) == B.MOE_ERR_UNSUPPORTED
        assert lib.moe_cache_pin(c, 256, 1) == B.MOE_ERR_SHAPE
        assert lib.moe_cache_pin(c, -1, 1) == B.MOE_ERR_SHAPE
        for i in range(32):  # up to n_slots - top_k pins
            assert lib.moe_cache_pin(c, i, 1) == B.MOE_OK
        assert lib.moe_cache_pin(c, 32, 1) == B.MOE_ERR_UNSUPPORTED
        assert lib.moe_cache_pin(c, 0, 0) == B.MOE_OK

        ws = moe.moe_cache_workspace_bytes(s, 1, 40)
        assert ws > 0 and ws % 256 == 0

        def call(T=1, x=P, xdt=1, w=P, sh=None, idx=P, tw=P, y=P, ys=None, out=P, odt=0,
                 wsp=P, wsb=ws):
            return lib.moe_cache_layer_decode(c, T, x, xdt, w, None, sh, idx, tw, y, ys, out, odt,
                                              wsp, wsb, None, None)

        assert call(T=-1) == B.MOE_ERR_SHAPE
        assert call(xdt=5) == B.MOE_ERR_DTYPE
        assert call(odt=5) == B.MOE_ERR_DTYPE
        assert call(T=129) == B.MOE_ERR_UNSUPPORTED  # T * top_k > 1024
        assert call(T=2) == B.MOE_ERR_UNSUPPORTED    # 16 slots needed, 40 - 31 pinned left
        assert lib.moe_cache_pin(c, 1, 0) == B.MOE_OK
        for name in ("x", "w", "idx", "tw", "y", "out", "wsp"):
            assert call(**{name: None}) == B.MOE_ERR_NULL, name
        assert call(sh=P) == B.MOE_ERR_NULL          # no shared expert in this shape
        assert call(x=P + 4) == B.MOE_ERR_ALIGN
        assert call(wsp=P + 64) == B.MOE_ERR_ALIGN
        assert call(wsb=ws - 1) == B.MOE_ERR_WORKSPACE
        assert call(T=0) == B.MOE_OK
    finally:
        moe.moe_cache_destroy(c)
    # a planning-only cache holds no weights
    p = moe.moe_cache_create(s, 40)
    try:
        assert lib.moe_cache_layer_decode(p, 1, P, 1, P, None, None, P, P, P, None, P, 0, P, 1 << 30,
                                          None, None) == B.MOE_ERR_NULL
    finally:
        moe.moe_cache_destroy(p)
