"""Plain reference model of the per-layer expert cache with pinned experts.

TEST INFRASTRUCTURE ONLY: imported by tests and by the benchmark's checks,
never by the GPU library.  It shares no code with the library's C++ cache;
both are written from the same policy statement below.

Sources (the pages, by title and section):

* zhichai.net, "744亿参数塞进25GB内存：colibrì如何用1300行C代码把不可能变成可能",
  section "为什么 llama.cpp 的 mmap 跟不上" (why mmap falls short): every layer
  keeps its own LRU cache of experts and evicts whole experts (one ~19 MB
  block, never part of one); the hot experts are pinned and take no part in
  LRU eviction.
* yunpan.plus article on Colibrì, section "核心能力一" (capability 1): a
  per-layer LRU plus a pinned hot-store; section "核心能力二" (capability 2):
  a bounded asynchronous I/O pool loads the missing experts while the
  resident ones compute.

Policy (the pages name LRU, whole-expert eviction and pinning; the rest is
this library's reading, listed in the design notes):

  * The cache has n_slots slots; each holds one expert's block or nothing.
  * A step is one layer call: the distinct experts its batch routes to.
    Every expert used by a step gets that step's number as its last use.
  * Experts already in a slot are hits.  The missing ones are placed in
    ascending expert id order, each into
      - the empty slot with the lowest index, if there is one, else
      - the slot whose expert has the oldest last use (ties: lowest slot
        index), among experts that are not pinned and not used by this step.
    The displaced expert is evicted.
  * pin(e) exempts e from eviction while it is resident; it loads nothing.
    unpin(e) makes it evictable again.
  * A step may need at most n_slots - (number of pinned experts) misses
    beyond its hits; the library checks the stronger bound
    n_slots - pinned >= min(E, T * top_k) before it starts.
"""
from __future__ import annotations


class ExpertCache:
    """The cache as a plain list of slots (expert id or None) and a dict of
    last-use step numbers."""

    def __init__(self, n_slots: int):
        self.slots = [None] * n_slots
        self.last_use = {}
        self.pinned = set()
        self.step_no = 0
        self.hits = 0
        self.misses = 0

    def pin(self, e: int, on: bool = True):
        if on:
            self.pinned.add(e)
        else:
            self.pinned.discard(e)

    def slot_of(self, e: int):
        for i, s in enumerate(self.slots):
            if s == e:
                return i
        return None

    def step(self, experts):
        """One step.  Returns (slot_of, fetched, evicted): slot_of maps each
        distinct expert of the step to its slot; fetched lists the experts
        that had to be loaded, in placement order; evicted maps each such
        expert to the expert it displaced (None for an empty slot)."""
        self.step_no += 1
        now = self.step_no
        used = sorted(set(int(e) for e in experts))
        placed = {}
        for e in used:
            i = self.slot_of(e)
            if i is not None:
                placed[e] = i
                self.last_use[e] = now
                self.hits += 1
        fetched, evicted = [], {}
        for e in used:
            if e in placed:
                continue
            empty = [i for i, s in enumerate(self.slots) if s is None]
            if empty:
                victim = empty[0]
            else:
                cands = [(self.last_use[s], i) for i, s in enumerate(self.slots)
                         if s not in self.pinned and self.last_use[s] < now]
                if not cands:
                    raise RuntimeError("no evictable slot: too many pinned or needed experts")
                victim = min(cands)[1]
            evicted[e] = self.slots[victim]
            self.slots[victim] = e
            self.last_use[e] = now
            placed[e] = victim
            fetched.append(e)
            self.misses += 1
        return placed, fetched, evicted
