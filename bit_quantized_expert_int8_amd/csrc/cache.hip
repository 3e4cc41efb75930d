// Per-layer LFU expert cache: host-side policy + copies of missing expert records into HBM slots.
//
// The pages keep 16 expert slots per layer under a least-frequently-used policy and fetch the missing
// experts while the shared expert computes.  Here the slow tier is pinned host memory; each miss is one
// hipMemcpyAsync of a whole expert record on the caller's copy stream, ordered after `wait_event` (the
// last kernel that read this layer's slots and slot ids) and followed by `ready_event`.  Slot ids reach the
// device by one more copy on the same stream, from an entry of a pinned ring the handle owns: the copy
// engine never switches to a kernel between a layer's record copies.  Each ring entry carries an event
// recorded after its copy, and an entry is rewritten only once that event has completed.
#include <string.h>

#include <new>
#include <vector>

#include "common.h"

struct moe_expert_cache {
  struct Layer {
    std::vector<int32_t> expert;   // expert held by each slot, -1 = empty
    std::vector<int64_t> count;    // uses since load
    std::vector<int64_t> last;     // step of last use
    int64_t step = 0;
    uint64_t hits = 0, misses = 0, bytes = 0;
  };
  int32_t n_layers = 0, n_experts = 0, n_slots = 0;
  size_t record_bytes = 0;
  uint32_t flags = 0;
  std::vector<const char*> host_pool;
  std::vector<char*> slot_pool;
  std::vector<Layer> layers;
  int32_t fail_after = -1;
  // pinned staging ring for slot ids (device mode only)
  int32_t* ring = nullptr;          // [kRing][kMaxIds]
  std::vector<hipEvent_t> ring_ev;  // recorded after the copy out of each entry
  std::vector<char> ring_used;
  int ring_pos = 0;
};

namespace moeq4 {
namespace {

constexpr int kMaxIds = 32;
constexpr int kRing = 1024;   // slot-id entries in flight before the host waits for the oldest copy

void release_ring(moe_expert_cache* c) {
  for (size_t i = 0; i < c->ring_ev.size(); ++i) {
    if (c->ring_used[i]) (void)hipEventSynchronize(c->ring_ev[i]);
    (void)hipEventDestroy(c->ring_ev[i]);
  }
  c->ring_ev.clear();
  c->ring_used.clear();
  if (c->ring) (void)hipHostFree(c->ring);
  c->ring = nullptr;
}

// The policy step on a copy of the layer state.  Fills slot_of[i] for each requested id and the list of
// (slot, expert) loads in request order.
void lfu_plan(moe_expert_cache::Layer& L, int n_slots, const int32_t* ids, int n, int32_t* slot_of,
              std::vector<std::pair<int32_t, int32_t>>& loads, int* hits) {
  std::vector<char> pinned(n_slots, 0);
  std::vector<char> resolved(n, 0);
  *hits = 0;
  for (int i = 0; i < n; ++i) {
    for (int s = 0; s < n_slots; ++s) {
      if (L.expert[s] == ids[i]) {
        L.count[s] += 1;
        L.last[s] = L.step;
        pinned[s] = 1;
        slot_of[i] = s;
        resolved[i] = 1;
        ++*hits;
        break;
      }
    }
  }
  for (int i = 0; i < n; ++i) {
    if (resolved[i]) continue;
    int pick = -1;
    for (int s = 0; s < n_slots; ++s)
      if (L.expert[s] < 0) { pick = s; break; }
    if (pick < 0) {
      for (int s = 0; s < n_slots; ++s) {
        if (pinned[s]) continue;
        if (pick < 0 || L.count[s] < L.count[pick] || (L.count[s] == L.count[pick] && L.last[s] < L.last[pick]))
          pick = s;   // ties on (count, last) keep the lower slot index
      }
    }
    L.expert[pick] = ids[i];
    L.count[pick] = 1;
    L.last[pick] = L.step;
    pinned[pick] = 1;
    slot_of[i] = pick;
    loads.emplace_back(pick, ids[i]);
  }
  L.step += 1;
}

}  // namespace
}  // namespace moeq4

using namespace moeq4;

extern "C" moe_status moe_expert_cache_create(int32_t n_layers, int32_t n_experts, int32_t n_slots, size_t record_bytes,
                                              const void* const* host_pool_host, void* const* slot_pool_dev, uint32_t flags,
                                              moe_expert_cache** out) {
  if (!out) return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_create: out is NULL");
  *out = nullptr;
  if (n_layers < 1 || n_experts < 1 || n_slots < 1 || record_bytes == 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_create: n_layers=%d n_experts=%d n_slots=%d record_bytes=%zu", n_layers,
                n_experts, n_slots, record_bytes);
  if (flags & ~MOE_CACHE_HOST_ONLY) return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_create: unknown flags 0x%x", flags);
  if (!host_pool_host || !slot_pool_dev) return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_create: pool array is NULL");
  for (int l = 0; l < n_layers; ++l)
    if (!host_pool_host[l] || !slot_pool_dev[l])
      return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_create: layer %d pool pointer is NULL", l);
  moe_expert_cache* c = new (std::nothrow) moe_expert_cache();
  if (!c) return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_create: out of host memory");
  c->n_layers = n_layers;
  c->n_experts = n_experts;
  c->n_slots = n_slots;
  c->record_bytes = record_bytes;
  c->flags = flags;
  c->host_pool.assign(reinterpret_cast<const char* const*>(host_pool_host),
                      reinterpret_cast<const char* const*>(host_pool_host) + n_layers);
  c->slot_pool.assign(reinterpret_cast<char* const*>(slot_pool_dev), reinterpret_cast<char* const*>(slot_pool_dev) + n_layers);
  c->layers.resize(n_layers);
  for (auto& L : c->layers) {
    L.expert.assign(n_slots, -1);
    L.count.assign(n_slots, 0);
    L.last.assign(n_slots, -1);
  }
  if (!(flags & MOE_CACHE_HOST_ONLY)) {
    hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&c->ring), (size_t)kRing * kMaxIds * sizeof(int32_t),
                                 hipHostMallocDefault);
    if (e != hipSuccess) {
      c->ring = nullptr;
      delete c;
      return fail(MOE_ERR_HIP, "moe_expert_cache_create: hipHostMalloc of the slot-id ring: %s", hipGetErrorString(e));
    }
    c->ring_ev.reserve(kRing);
    for (int i = 0; i < kRing && e == hipSuccess; ++i) {
      hipEvent_t ev = nullptr;
      e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
      if (e == hipSuccess) c->ring_ev.push_back(ev);
    }
    c->ring_used.assign(c->ring_ev.size(), 0);
    if (e != hipSuccess) {
      release_ring(c);
      delete c;
      return fail(MOE_ERR_HIP, "moe_expert_cache_create: hipEventCreate: %s", hipGetErrorString(e));
    }
  }
  *out = c;
  return MOE_OK;
}

extern "C" void moe_expert_cache_destroy(moe_expert_cache* cache) {
  if (!cache) return;
  release_ring(cache);
  delete cache;
}

extern "C" moe_status expert_cache_stage(moe_expert_cache* c, int32_t layer, const int32_t* ids_host, int32_t n,
                                         int32_t* slot_ids_dev, void* copy_stream, void* wait_event, void* ready_event) {
  if (!c || !ids_host || !slot_ids_dev) return fail(MOE_ERR_INVALID_ARG, "expert_cache_stage: NULL pointer");
  if (layer < 0 || layer >= c->n_layers) return fail(MOE_ERR_OUT_OF_RANGE, "expert_cache_stage: layer %d of %d", layer, c->n_layers);
  if (n < 1 || n > c->n_slots || n > kMaxIds)
    return fail(MOE_ERR_CACHE, "expert_cache_stage: %d ids for %d slots (at most min(slots, 32))", n, c->n_slots);
  for (int i = 0; i < n; ++i) {
    if (ids_host[i] < 0 || ids_host[i] >= c->n_experts)
      return fail(MOE_ERR_OUT_OF_RANGE, "expert_cache_stage: id %d outside [0, %d)", ids_host[i], c->n_experts);
    for (int j = 0; j < i; ++j)
      if (ids_host[j] == ids_host[i]) return fail(MOE_ERR_CACHE, "expert_cache_stage: duplicate id %d", ids_host[i]);
  }
  const bool host_only = c->flags & MOE_CACHE_HOST_ONLY;
  hipStream_t cs = as_stream(copy_stream);
  moe_expert_cache::Layer next = c->layers[layer];
  int32_t slot_of[kMaxIds];
  std::vector<std::pair<int32_t, int32_t>> loads;
  int hits = 0;
  lfu_plan(next, c->n_slots, ids_host, n, slot_of, loads, &hits);

  // Every write below (record copies and the slot ids) waits for the last reader of this layer's slots and
  // slot ids, also when every id hits: a caller that runs ahead of the device may stage the next token while
  // the previous token's kernel still reads slot_ids_dev.  An event that has already completed needs no wait
  // on the device.  (A copy that waits on another stream's event still pending when it is enqueued costs the
  // copy engine dearly: streamed decode measured 128 tokens/s with the caller a whole token or more ahead,
  // 146 with the caller waiting on the host for the layer's previous reader before staging, so that no
  // device-side wait is enqueued.)
  if (!host_only && wait_event) {
    const hipEvent_t we = reinterpret_cast<hipEvent_t>(wait_event);
    hipError_t e = hipEventQuery(we);
    if (e == hipErrorNotReady) {
      (void)hipGetLastError();   // a pending event is not an error: do not leave it as the thread's last error
      e = hipStreamWaitEvent(cs, we, 0);
      if (e != hipSuccess) return fail(MOE_ERR_HIP, "expert_cache_stage: hipStreamWaitEvent: %s", hipGetErrorString(e));
    } else if (e != hipSuccess) {
      return fail(MOE_ERR_HIP, "expert_cache_stage: hipEventQuery: %s", hipGetErrorString(e));
    }
  }
  size_t done = 0;
  moe_status st = MOE_OK;
  for (const auto& ld : loads) {
    char* dst = c->slot_pool[layer] + (size_t)ld.first * c->record_bytes;
    const char* src = c->host_pool[layer] + (size_t)ld.second * c->record_bytes;
    if (c->fail_after >= 0 && (int64_t)done == c->fail_after) {
      st = fail(MOE_ERR_HIP, "expert_cache_stage: injected copy failure at copy %zu", done);
      c->fail_after = -1;   // one-shot
      break;
    }
    if (host_only) {
      memcpy(dst, src, c->record_bytes);
    } else {
      hipError_t e = hipMemcpyAsync(dst, src, c->record_bytes, hipMemcpyHostToDevice, cs);
      if (e != hipSuccess) {
        st = fail(MOE_ERR_HIP, "expert_cache_stage: hipMemcpyAsync: %s", hipGetErrorString(e));
        break;
      }
    }
    ++done;
  }
  if (st == MOE_OK) {
    if (host_only) {
      memcpy(slot_ids_dev, slot_of, (size_t)n * sizeof(int32_t));
    } else {
      const int pos = c->ring_pos;
      hipError_t e = hipSuccess;
      if (c->ring_used[pos]) e = hipEventSynchronize(c->ring_ev[pos]);   // the entry's previous copy has run
      int32_t* entry = c->ring + (size_t)pos * kMaxIds;
      if (e == hipSuccess) {
        memcpy(entry, slot_of, (size_t)n * sizeof(int32_t));
        e = hipMemcpyAsync(slot_ids_dev, entry, (size_t)n * sizeof(int32_t), hipMemcpyHostToDevice, cs);
      }
      if (e == hipSuccess) e = hipEventRecord(c->ring_ev[pos], cs);
      if (e != hipSuccess) {
        st = fail(MOE_ERR_HIP, "expert_cache_stage: slot ids: %s", hipGetErrorString(e));
      } else {
        c->ring_used[pos] = 1;
        c->ring_pos = (pos + 1) % (int)c->ring_ev.size();
      }
      if (st == MOE_OK && ready_event) {
        hipError_t e = hipEventRecord(reinterpret_cast<hipEvent_t>(ready_event), cs);
        if (e != hipSuccess) st = fail(MOE_ERR_HIP, "expert_cache_stage: hipEventRecord: %s", hipGetErrorString(e));
      }
    }
  }
  if (st != MOE_OK) {
    // keep the old policy state, but a slot whose copy may already be under way holds nothing usable
    moe_expert_cache::Layer& L = c->layers[layer];
    for (size_t i = 0; i < done; ++i) {
      const int s = loads[i].first;
      L.expert[s] = -1;
      L.count[s] = 0;
      L.last[s] = -1;
    }
    return st;
  }
  next.hits += (uint64_t)hits;
  next.misses += loads.size();
  next.bytes += loads.size() * c->record_bytes;
  c->layers[layer] = std::move(next);
  if (c->fail_after >= 0) c->fail_after = c->fail_after > (int32_t)done ? c->fail_after - (int32_t)done : -1;
  return MOE_OK;
}

extern "C" moe_status moe_expert_cache_stats(const moe_expert_cache* c, int32_t layer, uint64_t* hits, uint64_t* misses,
                                             uint64_t* bytes_copied) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_stats: cache is NULL");
  if (layer < -1 || layer >= c->n_layers) return fail(MOE_ERR_OUT_OF_RANGE, "moe_expert_cache_stats: layer %d", layer);
  uint64_t h = 0, m = 0, b = 0;
  for (int l = 0; l < c->n_layers; ++l) {
    if (layer >= 0 && l != layer) continue;
    h += c->layers[l].hits;
    m += c->layers[l].misses;
    b += c->layers[l].bytes;
  }
  if (hits) *hits = h;
  if (misses) *misses = m;
  if (bytes_copied) *bytes_copied = b;
  return MOE_OK;
}

extern "C" moe_status moe_expert_cache_slots(const moe_expert_cache* c, int32_t layer, int32_t* experts_host) {
  if (!c || !experts_host) return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_slots: NULL pointer");
  if (layer < 0 || layer >= c->n_layers) return fail(MOE_ERR_OUT_OF_RANGE, "moe_expert_cache_slots: layer %d", layer);
  memcpy(experts_host, c->layers[layer].expert.data(), (size_t)c->n_slots * sizeof(int32_t));
  return MOE_OK;
}

extern "C" moe_status moe_expert_cache_inject_copy_failure(moe_expert_cache* c, int32_t after_n_copies) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_inject_copy_failure: cache is NULL");
  if (after_n_copies < -1) return fail(MOE_ERR_INVALID_ARG, "moe_expert_cache_inject_copy_failure: %d", after_n_copies);
  c->fail_after = after_n_copies;
  return MOE_OK;
}
