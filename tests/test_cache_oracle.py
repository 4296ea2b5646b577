"""Pins of the expert-cache reference model (CPU only).

The model in oracle/expert_cache.py is checked against a hand-worked trace,
a textbook LRU written differently (an ordered dict, no slots), the classic
LRU closed forms (compulsory misses only when everything fits; every access a
miss on a cyclic trace one longer than the cache), LRU's inclusion property,
and the pinning and same-step rules of its policy.
"""
import collections

import numpy as np
import pytest

from oracle.expert_cache import ExpertCache


def test_hand_worked_trace():
    c = ExpertCache(3)
    # step 1: 5, 2 -> empty slots 0, 1 in ascending id order (2 first)
    placed, fetched, ev = c.step([5, 2])
    assert placed == {2: 0, 5: 1} and fetched == [2, 5] and ev == {2: None, 5: None}
    # step 2: 7 -> the last empty slot
    placed, fetched, ev = c.step([7])
    assert placed == {7: 2} and fetched == [7]
    # step 3: 2 hit, 9 miss -> oldest last use among 5 (step 1) and 7 (step 2): 5 in slot 1
    placed, fetched, ev = c.step([9, 2])
    assert placed == {2: 0, 9: 1} and fetched == [9] and ev == {9: 5}
    # step 4: 4, 6 -> candidates 7 (step 2), 2 (step 3), 9 (step 3): 7 first (slot 2),
    # then the step-3 tie between 2 (slot 0) and 9 (slot 1) goes to the lower slot
    placed, fetched, ev = c.step([6, 4])
    assert placed == {4: 2, 6: 0} and ev == {4: 7, 6: 2}
    assert c.hits == 1 and c.misses == 6


def textbook_lru(capacity, trace):
    """Hit (True) / miss (False) per access of a one-expert-per-step trace."""
    od = collections.OrderedDict()
    out = []
    for e in trace:
        if e in od:
            od.move_to_end(e)
            out.append(True)
        else:
            if len(od) == capacity:
                od.popitem(last=False)
            od[e] = True
            out.append(False)
    return out


@pytest.mark.parametrize("capacity,universe,seed", [(1, 3, 0), (4, 10, 1), (16, 40, 2), (7, 7, 3)])
def test_matches_a_textbook_lru_on_single_expert_steps(capacity, universe, seed):
    rng = np.random.default_rng(seed)
    trace = rng.integers(0, universe, size=2000)
    c = ExpertCache(capacity)
    got = []
    for e in trace:
        _, fetched, _ = c.step([e])
        got.append(not fetched)
    assert got == textbook_lru(capacity, trace)


def test_everything_fits_gives_compulsory_misses_only():
    rng = np.random.default_rng(4)
    c = ExpertCache(64)
    seen = set()
    for _ in range(300):
        step = rng.choice(64, size=8, replace=False)
        _, fetched, ev = c.step(step)
        assert all(v is None for v in ev.values())
        seen.update(int(e) for e in step)
    assert c.misses == len(seen)


def test_cyclic_trace_one_longer_than_the_cache_always_misses():
    c = ExpertCache(5)
    for r in range(10):
        for e in range(6):
            _, fetched, _ = c.step([e])
            assert fetched == [e]
    assert c.hits == 0


def test_inclusion_property_hits_grow_with_capacity():
    rng = np.random.default_rng(5)
    trace = (rng.zipf(1.3, size=3000) % 50).tolist()
    hits = []
    for cap in range(1, 51):
        c = ExpertCache(cap)
        for e in trace:
            c.step([e])
        hits.append(c.hits)
    assert all(a <= b for a, b in zip(hits, hits[1:]))


def test_pinned_experts_stay_and_same_step_experts_are_never_displaced():
    rng = np.random.default_rng(6)
    c = ExpertCache(12)
    pins = {3, 17}
    for e in pins:
        c.pin(e)
    resident_pins = set()
    for _ in range(500):
        step = rng.choice(40, size=8, replace=False).tolist()
        placed, fetched, ev = c.step(step)
        # distinct slots for the step's experts, each holding its expert
        assert len(set(placed.values())) == len(placed)
        assert all(c.slots[i] == e for e, i in placed.items())
        assert not (set(ev.values()) & resident_pins)
        resident_pins |= pins & set(c.slots)
        assert resident_pins <= set(c.slots)
    assert resident_pins == pins
    c.pin(3, False)
    for _ in range(50):
        c.step(rng.choice(np.arange(20, 40), size=8, replace=False).tolist())
    assert 3 not in c.slots and 17 in c.slots


def test_too_many_pins_for_a_step_is_an_error():
    c = ExpertCache(2)
    c.pin(0)
    c.pin(1)
    c.step([0, 1])
    with pytest.raises(RuntimeError):
        c.step([5])
