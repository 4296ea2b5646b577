// Per-layer expert cache in HBM with host-streamed misses (pages: zhichai.net,
// section on why mmap falls short -- each layer keeps an LRU of whole experts
// and pinned hot experts never take part in eviction; yunpan.plus article,
// "capability 1" -- per-layer LRU plus pinned hot-store, and "capability 2" --
// a bounded asynchronous I/O pool loads the missing experts while the
// resident ones compute).
//
// The policy is host logic: a step's distinct experts are hits if a slot
// holds them; the misses, in ascending id order, take the lowest empty slot,
// else the slot whose expert was used least recently (ties to the lower
// slot), skipping pinned experts and experts of the same step.  A decode
// step through the cache is
//
//   router (logits + top-k)  ->  top-k ids to the host (the one host wait)
//   -> plan  ->  misses copied host -> slot on the copy stream
//   -> ids remapped to slots, batch-union over slots
//   -> FFN over the resident experts (+ shared)  ||  the copies
//   -> wait for the copies  ->  FFN over the fetched experts  ->  combine
//
// so the resident experts' weights stream from HBM while PCIe brings the
// missing ones in.  Grouping by slot instead of expert id changes only the
// order of the grouped rows; every token's k expert outputs and their sum
// are the same as without the cache.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <new>
#include <vector>

#include "launch.h"
#include "moe_int4.h"

struct moe_expert_cache {
  moe_shape shape;
  int n_slots = 0;
  size_t block_bytes = 0;
  uint8_t* dev_slots = nullptr;          // caller-owned: n_slots blocks in HBM
  const uint8_t* host_blocks = nullptr;  // caller-owned pinned host memory: E blocks
  std::vector<int32_t> slot_expert;      // expert held by each slot, -1 empty
  std::vector<int32_t> expert_slot;      // slot of each expert, -1 not resident
  std::vector<int64_t> slot_used;        // step of the last use of each slot's expert
  std::vector<uint8_t> pinned;           // per expert
  int n_pinned = 0;
  int64_t step = 0;
  int64_t hits = 0, misses = 0, bytes_fetched = 0;
  // per-step host scratch
  std::vector<uint8_t> mark;
  std::vector<int32_t> distinct;
  // the latest step's fetched experts in placement order and the expert each
  // displaced (-1: an empty slot)
  std::vector<int32_t> last_fetched, last_evicted;
  // pinned staging and the copy event, created on the first decode step
  int32_t* stage = nullptr;
  size_t stage_ints = 0;
  hipEvent_t fetched_ev = nullptr;
};

namespace {

constexpr int kMaxCacheSlots = 1024;  // T * top_k of one cached decode step

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t up256(size_t n) { return (n + 255) / 256 * 256; }

moe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  if (e == hipErrorNotSupported) return MOE_ERR_UNSUPPORTED;
  return MOE_ERR_HIP;
}

// One step of the policy over the n entries of `experts` (ids in [0, E),
// repeats allowed).  Fills slot_of per entry and the fetched experts in
// placement order with the expert each displaced (-1: an empty slot).
// Returns false if a miss finds no evictable slot (the state is then
// unchanged).
bool plan_step(moe_expert_cache* c, int n, const int32_t* experts, int32_t* slot_of,
               int32_t* fetched, int32_t* fetched_slot, int32_t* evicted, int* n_fetched) {
  const int E = c->shape.n_experts;
  for (int i = 0; i < n; ++i) c->mark[experts[i]] = 1;
  c->distinct.clear();
  for (int e = 0; e < E; ++e)
    if (c->mark[e]) {
      c->distinct.push_back(e);
      c->mark[e] = 0;
    }
  // capacity: every miss needs a slot that is empty or holds an unpinned
  // expert outside this step
  int misses = 0, free_slots = 0;
  for (int e : c->distinct) misses += c->expert_slot[e] < 0;
  for (int s = 0; s < c->n_slots; ++s) {
    const int e = c->slot_expert[s];
    if (e < 0) {
      ++free_slots;
      continue;
    }
    if (c->pinned[e]) continue;
    if (std::binary_search(c->distinct.begin(), c->distinct.end(), e)) continue;
    ++free_slots;
  }
  if (misses > free_slots) return false;
  const int64_t now = ++c->step;
  c->last_fetched.clear();
  c->last_evicted.clear();
  for (int e : c->distinct) {
    const int s = c->expert_slot[e];
    if (s >= 0) {
      c->slot_used[s] = now;
      ++c->hits;
    }
  }
  int nf = 0;
  for (int e : c->distinct) {
    if (c->expert_slot[e] >= 0) continue;
    int victim = -1;
    for (int s = 0; s < c->n_slots && victim < 0; ++s)
      if (c->slot_expert[s] < 0) victim = s;
    if (victim < 0) {
      for (int s = 0; s < c->n_slots; ++s) {
        const int o = c->slot_expert[s];
        if (c->pinned[o] || c->slot_used[s] >= now) continue;
        if (victim < 0 || c->slot_used[s] < c->slot_used[victim]) victim = s;
      }
    }
    const int old = c->slot_expert[victim];
    if (old >= 0) c->expert_slot[old] = -1;
    c->slot_expert[victim] = e;
    c->expert_slot[e] = victim;
    c->slot_used[victim] = now;
    ++c->misses;
    if (fetched) fetched[nf] = e;
    if (fetched_slot) fetched_slot[nf] = victim;
    if (evicted) evicted[nf] = old;
    c->last_fetched.push_back(e);
    c->last_evicted.push_back(old);
    ++nf;
  }
  for (int i = 0; i < n; ++i) slot_of[i] = c->expert_slot[experts[i]];
  *n_fetched = nf;
  return true;
}

// Undo the placement of the latest step's fetched experts: their slots
// become empty (whatever part of a block reached a slot is never read as a
// hit), their misses are taken back, and the latest-step record is cleared.
// The experts they displaced stay unmapped (their slots' contents are gone).
void unplace_last(moe_expert_cache* c) {
  for (const int32_t e : c->last_fetched) {
    const int s = c->expert_slot[e];
    if (s < 0) continue;
    c->slot_expert[s] = -1;
    c->slot_used[s] = 0;
    c->expert_slot[e] = -1;
    --c->misses;
  }
  c->last_fetched.clear();
  c->last_evicted.clear();
}

// Device workspace of a cached decode step, in order: router partial sums,
// slot ids [T*k], the grouping over slots (counts [S], offsets [S+1],
// perm [T*k], inv_perm [T*k], active [S], n_active [1]), the two FFN
// expert lists [L] each (L = min(S, T*k)), the FFN's h.
struct CacheWs {
  size_t part, ids, counts, offsets, perm, inv_perm, active, n_active, list_a, list_b, h, total;
};

CacheWs cache_ws(const moe_shape& sh, int T, int S) {
  const int E = sh.n_experts, k = sh.top_k;
  const size_t n = static_cast<size_t>(T) * k;
  const size_t L = std::min<size_t>(S, n);
  CacheWs w{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += up256(bytes);
    return at;
  };
  w.part = take(moe::route_workspace(T, sh.d, E));
  w.ids = take(n * 4);
  w.counts = take(static_cast<size_t>(S) * 4);
  w.offsets = take((static_cast<size_t>(S) + 1) * 4);
  w.perm = take(n * 4);
  w.inv_perm = take(n * 4);
  w.active = take(static_cast<size_t>(S) * 4);
  w.n_active = take(4);
  w.list_a = take(L * 4);
  w.list_b = take(L * 4);
  w.h = take(moe::ffn_decode_workspace(T, k, S, sh.d, sh.f, sh.f_shared != 0));
  w.total = o;
  return w;
}

moe_status check_cache_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_NULL;
  if (s->d <= 0 || s->f <= 0 || s->n_experts <= 0 || s->top_k <= 0 || s->group <= 0 ||
      s->f_shared < 0 || s->top_k > s->n_experts || s->d % 64 || s->f % 64)
    return MOE_ERR_SHAPE;
  if (s->group != 64 || s->d > 8192 || s->f > 8192 || s->n_experts > 1024 || s->top_k > 32 ||
      (s->f_shared != 0 && s->f_shared != s->f))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_cache_create(const moe_shape* shape, int32_t n_slots, uint8_t* device_slots,
                            const uint8_t* host_blocks, moe_expert_cache** cache) {
  if (!cache) return MOE_ERR_NULL;
  moe_status st = check_cache_shape(shape);
  if (st != MOE_OK) return st;
  if (n_slots < shape->top_k || n_slots > shape->n_experts) return MOE_ERR_SHAPE;
  if ((device_slots == nullptr) != (host_blocks == nullptr)) return MOE_ERR_NULL;
  if ((device_slots && !aligned(device_slots, 256)) || (host_blocks && !aligned(host_blocks, 16)))
    return MOE_ERR_ALIGN;
  moe_expert_cache* c = new (std::nothrow) moe_expert_cache();
  if (!c) return MOE_ERR_UNSUPPORTED;
  c->shape = *shape;
  c->n_slots = n_slots;
  c->block_bytes = moe_expert_bytes(shape->d, shape->f, shape->group);
  c->dev_slots = device_slots;
  c->host_blocks = host_blocks;
  c->slot_expert.assign(n_slots, -1);
  c->slot_used.assign(n_slots, 0);
  c->expert_slot.assign(shape->n_experts, -1);
  c->pinned.assign(shape->n_experts, 0);
  c->mark.assign(shape->n_experts, 0);
  c->distinct.reserve(shape->n_experts);
  c->last_fetched.reserve(shape->n_experts);
  c->last_evicted.reserve(shape->n_experts);
  *cache = c;
  return MOE_OK;
}

void moe_cache_destroy(moe_expert_cache* cache) {
  if (!cache) return;
  if (cache->fetched_ev) (void)hipEventDestroy(cache->fetched_ev);
  if (cache->stage) (void)hipHostFree(cache->stage);
  delete cache;
}

moe_status moe_cache_pin(moe_expert_cache* cache, int32_t expert, int32_t pinned) {
  if (!cache) return MOE_ERR_NULL;
  if (expert < 0 || expert >= cache->shape.n_experts) return MOE_ERR_SHAPE;
  const uint8_t v = pinned ? 1 : 0;
  if (v && !cache->pinned[expert] && cache->n_pinned + 1 > cache->n_slots - cache->shape.top_k)
    return MOE_ERR_UNSUPPORTED;  // a step of one token must still find room
  cache->n_pinned += static_cast<int>(v) - static_cast<int>(cache->pinned[expert]);
  cache->pinned[expert] = v;
  return MOE_OK;
}

moe_status moe_cache_plan(moe_expert_cache* cache, int32_t n, const int32_t* experts,
                          int32_t* slot_of, int32_t* fetched, int32_t* evicted,
                          int32_t* n_fetched) {
  if (!cache || !n_fetched) return MOE_ERR_NULL;
  if (cache->dev_slots) return MOE_ERR_UNSUPPORTED;  // planning-only caches
  if (n < 0) return MOE_ERR_SHAPE;
  if (n > 0 && (!experts || !slot_of || !fetched || !evicted)) return MOE_ERR_NULL;
  for (int i = 0; i < n; ++i)
    if (experts[i] < 0 || experts[i] >= cache->shape.n_experts) return MOE_ERR_SHAPE;
  int nf = 0;
  if (!plan_step(cache, n, experts, slot_of, fetched, nullptr, evicted, &nf))
    return MOE_ERR_UNSUPPORTED;
  *n_fetched = nf;
  return MOE_OK;
}

moe_status moe_cache_stats(const moe_expert_cache* cache, int64_t* hits, int64_t* misses,
                           int64_t* bytes_fetched) {
  if (!cache) return MOE_ERR_NULL;
  if (hits) *hits = cache->hits;
  if (misses) *misses = cache->misses;
  if (bytes_fetched) *bytes_fetched = cache->bytes_fetched;
  return MOE_OK;
}

moe_status moe_cache_last_fetch(const moe_expert_cache* cache, int32_t capacity, int32_t* fetched,
                                int32_t* evicted, int32_t* n_fetched) {
  if (!cache || !n_fetched) return MOE_ERR_NULL;
  const int nf = static_cast<int>(cache->last_fetched.size());
  if (capacity < nf) return MOE_ERR_SHAPE;
  if (nf > 0 && (!fetched || !evicted)) return MOE_ERR_NULL;
  for (int i = 0; i < nf; ++i) {
    fetched[i] = cache->last_fetched[i];
    evicted[i] = cache->last_evicted[i];
  }
  *n_fetched = nf;
  return MOE_OK;
}

moe_status moe_cache_unplan_last(moe_expert_cache* cache) {
  if (!cache) return MOE_ERR_NULL;
  unplace_last(cache);
  return MOE_OK;
}

size_t moe_cache_workspace_bytes(const moe_shape* shape, int32_t T, int32_t n_slots) {
  if (check_cache_shape(shape) != MOE_OK || T < 0 || n_slots < 1 ||
      static_cast<int64_t>(T) * shape->top_k > kMaxCacheSlots)
    return 0;
  return cache_ws(*shape, T, n_slots).total;
}

moe_status moe_cache_layer_decode(moe_expert_cache* cache, int32_t T, const void* x,
                                  moe_dtype x_dt, const float* w_router, const float* bias,
                                  const uint8_t* shared, int32_t* topk_idx, float* topk_w,
                                  void* y, void* y_shared, void* out, moe_dtype out_dt,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  void* copy_stream) {
  if (!cache) return MOE_ERR_NULL;
  const moe_shape& sh = cache->shape;
  const int E = sh.n_experts, k = sh.top_k, S = cache->n_slots;
  if (T < 0) return MOE_ERR_SHAPE;
  if (static_cast<int64_t>(T) * k > kMaxCacheSlots) return MOE_ERR_UNSUPPORTED;
  if (x_dt != MOE_F32 && x_dt != MOE_BF16) return MOE_ERR_DTYPE;
  if (out_dt != MOE_F32 && out_dt != MOE_BF16) return MOE_ERR_DTYPE;
  if (T == 0) return MOE_OK;
  if (!cache->dev_slots) return MOE_ERR_NULL;  // a planning-only cache holds no weights
  const int n = T * k;
  if (S - cache->n_pinned < std::min(E, n)) return MOE_ERR_UNSUPPORTED;
  const bool has_shared = sh.f_shared != 0;
  if (!x || !w_router || !topk_idx || !topk_w || !y || !out || !workspace) return MOE_ERR_NULL;
  if (has_shared != (shared != nullptr) || has_shared != (y_shared != nullptr))
    return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_router, 16) || (bias && !aligned(bias, 4)) ||
      (shared && !aligned(shared, 16)) || !aligned(topk_idx, 4) || !aligned(topk_w, 4) ||
      !aligned(y, 16) || (y_shared && !aligned(y_shared, 16)) || !aligned(out, 16) ||
      !aligned(workspace, 256))
    return MOE_ERR_ALIGN;
  const CacheWs w = cache_ws(sh, T, S);
  if (workspace_bytes < w.total) return MOE_ERR_WORKSPACE;
  const size_t L = std::min(S, n);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipStream_t cs = static_cast<hipStream_t>(copy_stream);

  // pinned staging: ids from the device, then slot ids and the two lists
  const size_t need = static_cast<size_t>(kMaxCacheSlots) * 2 + 2 * static_cast<size_t>(S);
  if (!cache->stage) {
    void* p = nullptr;
    if (hipHostMalloc(&p, need * 4, hipHostMallocDefault) != hipSuccess) return MOE_ERR_HIP;
    cache->stage = static_cast<int32_t*>(p);
    cache->stage_ints = need;
  }
  if (!cache->fetched_ev &&
      hipEventCreateWithFlags(&cache->fetched_ev, hipEventDisableTiming) != hipSuccess)
    return MOE_ERR_HIP;
  int32_t* h_ids = cache->stage;                    // [n]
  int32_t* h_up = cache->stage + kMaxCacheSlots;    // slot ids [n], list A [L], list B [L]

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  auto at = [&](size_t off) { return reinterpret_cast<int32_t*>(ws + off); };
  double* part = reinterpret_cast<double*>(ws + w.part);
  hipError_t err = moe::launch_route(T, sh.d, E, k, x, x_dt == MOE_BF16, w_router, bias, part,
                                     topk_idx, topk_w, s);
  if (err == hipSuccess)
    err = hipMemcpyAsync(h_ids, topk_idx, static_cast<size_t>(n) * 4, hipMemcpyDeviceToHost, s);
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  if (err != hipSuccess) return MOE_ERR_HIP;

  // the plan: slot per routing entry, the fetched experts and their slots
  std::vector<int32_t> fetched(std::min(E, n)), fslot(std::min(E, n));
  int nf = 0;
  if (!plan_step(cache, n, h_ids, h_up, fetched.data(), fslot.data(), nullptr, &nf))
    return MOE_ERR_UNSUPPORTED;  // unreachable: the capacity check above covers it
  for (int i = 0; i < nf && err == hipSuccess; ++i) {
    err = hipMemcpyAsync(cache->dev_slots + static_cast<size_t>(fslot[i]) * cache->block_bytes,
                         cache->host_blocks + static_cast<size_t>(fetched[i]) * cache->block_bytes,
                         cache->block_bytes, hipMemcpyHostToDevice, cs);
  }
  if (err == hipSuccess && nf > 0) err = hipEventRecord(cache->fetched_ev, cs);
  if (err != hipSuccess) {
    // a slot whose copy was not queued (or not fenced by the event) must not
    // be taken for its expert later
    unplace_last(cache);
    return MOE_ERR_HIP;
  }
  cache->bytes_fetched += static_cast<int64_t>(nf) * static_cast<int64_t>(cache->block_bytes);
  // list A: the slots of this step's hits, list B: the fetched slots (both
  // ascending, -1 padded)
  int32_t* la = h_up + n;
  int32_t* lb = la + L;
  {
    std::vector<int32_t> hit_slots;
    for (int e : cache->distinct) {
      const int sl = cache->expert_slot[e];
      if (std::find(fslot.begin(), fslot.begin() + nf, sl) == fslot.begin() + nf)
        hit_slots.push_back(sl);
    }
    std::sort(hit_slots.begin(), hit_slots.end());
    std::vector<int32_t> fs(fslot.begin(), fslot.begin() + nf);
    std::sort(fs.begin(), fs.end());
    for (size_t i = 0; i < L; ++i) {
      la[i] = i < hit_slots.size() ? hit_slots[i] : -1;
      lb[i] = i < fs.size() ? fs[i] : -1;
    }
  }
  if (err == hipSuccess)
    err = hipMemcpyAsync(at(w.ids), h_up, static_cast<size_t>(n) * 4, hipMemcpyHostToDevice, s);
  if (err == hipSuccess)
    err = hipMemcpyAsync(at(w.list_a), la, L * 4, hipMemcpyHostToDevice, s);
  if (err == hipSuccess)
    err = hipMemcpyAsync(at(w.list_b), lb, L * 4, hipMemcpyHostToDevice, s);
  if (err == hipSuccess)
    err = moe::launch_union(n, S, at(w.ids), at(w.counts), at(w.offsets), at(w.perm),
                            at(w.inv_perm), at(w.active), at(w.n_active), s);
  moe::FfnProblem p{};
  p.T = T;
  p.d = sh.d;
  p.f = sh.f;
  p.E = S;
  p.k = k;
  p.has_shared = has_shared;
  p.x_bf16 = x_dt == MOE_BF16;
  p.block_bytes = cache->block_bytes;
  p.x = x;
  p.experts = cache->dev_slots;
  p.shared = shared;
  p.offsets = at(w.offsets);
  p.perm = at(w.perm);
  p.active = at(w.list_a);
  p.n_active = at(w.n_active);
  p.y = y;
  p.y_shared = y_shared;
  p.workspace = ws + w.h;
  if (err == hipSuccess) err = moe::launch_ffn_decode(p, s);  // resident experts (+ shared)
  if (err == hipSuccess && nf > 0) {
    err = hipStreamWaitEvent(s, cache->fetched_ev, 0);
    p.has_shared = false;
    p.shared = nullptr;
    p.y_shared = nullptr;
    p.active = at(w.list_b);
    if (err == hipSuccess) err = moe::launch_ffn_decode(p, s);  // fetched experts
  }
  if (err == hipSuccess)
    err = moe::launch_combine(T, sh.d, k, y, y_shared, false, at(w.inv_perm), topk_w, out,
                              out_dt == MOE_BF16, s);
  return hip_status(err);
}

}  // extern "C"
