// The HBM expert-slot cache: host-side LRU over (layer, expert) keys plus the
// stream/event protocol for filling slots from pinned host memory.
//
// Method: host RAM holds every routed expert; one GPU cache is shared by all
// MoE layers; in decode it is an LRU over recently selected experts, hits run
// on the GPU, misses are copied over PCIe (page "FreeToken量子化：MoE推論の
// セットアップガイド", hierarchy and decode paragraphs; bhrtaym-blog page,
// section "MoEバックエンドは4種類から選べる", backend table row "offload").
#include <set>
#include <vector>

#include "common.h"

struct moe_cache {
  int num_slots = 0, num_layers = 0, num_experts = 0;
  size_t slot_bytes = 0;
  uint8_t* pool = nullptr;
  // LRU as an intrusive doubly linked list over keys; head = least recent.
  std::vector<int32_t> key_slot;   // key -> slot or -1
  std::vector<int32_t> slot_key;   // slot -> key or -1
  std::vector<int32_t> prev, next; // per key
  int32_t head = -1, tail = -1;
  std::set<int32_t> free_slots;
  // events (created on first use)
  std::vector<hipEvent_t> reader, filled;
  std::vector<uint8_t> has_reader;
  int device = -1;

  void unlink(int32_t k) {
    int32_t p = prev[k], n = next[k];
    if (p >= 0) next[p] = n; else head = n;
    if (n >= 0) prev[n] = p; else tail = p;
    prev[k] = next[k] = -1;
  }
  void push_mru(int32_t k) {
    prev[k] = tail;
    next[k] = -1;
    if (tail >= 0) next[tail] = k; else head = k;
    tail = k;
  }
  void reset() {
    std::fill(key_slot.begin(), key_slot.end(), -1);
    std::fill(slot_key.begin(), slot_key.end(), -1);
    std::fill(prev.begin(), prev.end(), -1);
    std::fill(next.begin(), next.end(), -1);
    head = tail = -1;
    free_slots.clear();
    for (int s = 0; s < num_slots; ++s) free_slots.insert(s);
  }
};

extern "C" moe_cache* moe_cache_create(int num_slots, size_t slot_bytes, void* slot_pool, int num_layers,
                                       int num_experts) {
  if (num_slots <= 0 || num_layers <= 0 || num_experts <= 0 || slot_bytes == 0 ||
      (long long)num_layers * num_experts > (1LL << 30)) {
    moe::set_error(MOE_EINVAL, "moe_cache_create: bad sizes (slots %d, layers %d, experts %d, slot_bytes %zu)",
                   num_slots, num_layers, num_experts, slot_bytes);
    return nullptr;
  }
  moe_cache* c = new (std::nothrow) moe_cache;
  if (!c) {
    moe::set_error(MOE_ENOMEM, "moe_cache_create: out of host memory");
    return nullptr;
  }
  c->num_slots = num_slots;
  c->num_layers = num_layers;
  c->num_experts = num_experts;
  c->slot_bytes = slot_bytes;
  c->pool = static_cast<uint8_t*>(slot_pool);
  const size_t nk = (size_t)num_layers * num_experts;
  c->key_slot.assign(nk, -1);
  c->prev.assign(nk, -1);
  c->next.assign(nk, -1);
  c->slot_key.assign(num_slots, -1);
  c->has_reader.assign(num_slots, 0);
  c->reset();
  return c;
}

extern "C" void moe_cache_destroy(moe_cache* c) {
  if (!c) return;
  for (hipEvent_t e : c->reader) if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : c->filled) if (e) (void)hipEventDestroy(e);
  delete c;
}

extern "C" moe_status moe_cache_reset(moe_cache* c) {
  MOE_CHECK_ARG(c, "moe_cache_reset: null cache");
  c->reset();
  std::fill(c->has_reader.begin(), c->has_reader.end(), 0);
  return MOE_OK;
}

extern "C" moe_status moe_cache_pin_resident(moe_cache* c, int layer, int s0) {
  MOE_CHECK_ARG(c, "moe_cache_pin_resident: null cache");
  MOE_CHECK_ARG(layer >= 0 && layer < c->num_layers, "moe_cache_pin_resident: layer %d out of range", layer);
  MOE_CHECK_ARG(s0 >= 0 && s0 + c->num_experts <= c->num_slots, "moe_cache_pin_resident: slots [%d, %d) out of range",
                s0, s0 + c->num_experts);
  for (int e = 0; e < c->num_experts; ++e)
    MOE_CHECK_ARG(c->slot_key[s0 + e] < 0 && c->key_slot[(size_t)layer * c->num_experts + e] < 0,
                  "moe_cache_pin_resident: slot %d or key already in use", s0 + e);
  for (int e = 0; e < c->num_experts; ++e) {
    const int32_t k = layer * c->num_experts + e, s = s0 + e;
    c->free_slots.erase(s);
    c->key_slot[k] = s;
    c->slot_key[s] = k;
    c->push_mru(k);
  }
  return MOE_OK;
}

extern "C" moe_status cache_lookup(moe_cache* c, int layer, const int32_t* ids, int n, int32_t* slot, uint8_t* hit,
                                   int32_t* evicted_key) {
  MOE_CHECK_ARG(c, "cache_lookup: null cache");
  MOE_CHECK_ARG(n >= 0 && (n == 0 || (ids && slot && hit && evicted_key)), "cache_lookup: null output");
  MOE_CHECK_ARG(layer >= 0 && layer < c->num_layers, "cache_lookup: layer %d out of range [0, %d)", layer,
                c->num_layers);
  for (int i = 0; i < n; ++i) {
    MOE_CHECK_ARG(ids[i] >= 0 && ids[i] < c->num_experts, "cache_lookup: expert id %d out of range", ids[i]);
    MOE_CHECK_ARG(i == 0 || ids[i] > ids[i - 1], "cache_lookup: ids must be distinct and ascending");
  }
  if (n > c->num_slots)
    return moe::set_error(MOE_ECACHE, "cache_lookup: %d distinct experts in one step > %d slots", n, c->num_slots);
  for (int i = 0; i < n; ++i) {
    const int32_t k = layer * c->num_experts + ids[i];
    int32_t s = c->key_slot[k];
    if (s >= 0) {
      c->unlink(k);
      c->push_mru(k);
      slot[i] = s;
      hit[i] = 1;
      evicted_key[i] = -1;
      continue;
    }
    int32_t victim = -1;
    if (!c->free_slots.empty()) {
      s = *c->free_slots.begin();
      c->free_slots.erase(c->free_slots.begin());
    } else {
      victim = c->head;  // least recently used; never a key of this call since n <= num_slots
      s = c->key_slot[victim];
      c->unlink(victim);
      c->key_slot[victim] = -1;
    }
    c->key_slot[k] = s;
    c->slot_key[s] = k;
    c->push_mru(k);
    slot[i] = s;
    hit[i] = 0;
    evicted_key[i] = victim;
  }
  return MOE_OK;
}

static moe_status ensure_events(moe_cache* c) {
  if (!c->reader.empty()) return MOE_OK;
  MOE_HIP(hipGetDevice(&c->device));
  c->reader.assign(c->num_slots, nullptr);
  c->filled.assign(c->num_slots, nullptr);
  for (int s = 0; s < c->num_slots; ++s) {
    MOE_HIP(hipEventCreateWithFlags(&c->reader[s], hipEventDisableTiming));
    MOE_HIP(hipEventCreateWithFlags(&c->filled[s], hipEventDisableTiming));
  }
  return MOE_OK;
}

extern "C" moe_status cache_fill(moe_cache* c, int layer, int expert, int slot, const void* host_src,
                                 moe_stream_t copy_stream, moe_stream_t compute_stream) {
  MOE_CHECK_ARG(c && host_src, "cache_fill: null pointer");
  MOE_CHECK_ARG(c->pool, "cache_fill: cache has no slot pool");
  MOE_CHECK_ARG(layer >= 0 && layer < c->num_layers && expert >= 0 && expert < c->num_experts,
                "cache_fill: (layer %d, expert %d) out of range", layer, expert);
  MOE_CHECK_ARG(slot >= 0 && slot < c->num_slots, "cache_fill: slot %d out of range", slot);
  MOE_CHECK_ARG(c->key_slot[(size_t)layer * c->num_experts + expert] == slot,
                "cache_fill: (layer %d, expert %d) is not mapped to slot %d", layer, expert, slot);
  moe_status st = ensure_events(c);
  if (st != MOE_OK) return st;
  hipStream_t cs = reinterpret_cast<hipStream_t>(copy_stream);
  hipStream_t ks = reinterpret_cast<hipStream_t>(compute_stream);
  if (c->has_reader[slot]) MOE_HIP(hipStreamWaitEvent(cs, c->reader[slot], 0));
  MOE_HIP(hipMemcpyAsync(c->pool + (size_t)slot * c->slot_bytes, host_src, c->slot_bytes, hipMemcpyHostToDevice, cs));
  MOE_HIP(hipEventRecord(c->filled[slot], cs));
  MOE_HIP(hipStreamWaitEvent(ks, c->filled[slot], 0));
  return MOE_OK;
}

extern "C" moe_status moe_cache_mark_used(moe_cache* c, const int32_t* slots, int n, moe_stream_t compute_stream) {
  MOE_CHECK_ARG(c && (n == 0 || slots), "moe_cache_mark_used: null pointer");
  for (int i = 0; i < n; ++i)
    MOE_CHECK_ARG(slots[i] >= 0 && slots[i] < c->num_slots, "moe_cache_mark_used: slot %d out of range", slots[i]);
  moe_status st = ensure_events(c);
  if (st != MOE_OK) return st;
  hipStream_t ks = reinterpret_cast<hipStream_t>(compute_stream);
  for (int i = 0; i < n; ++i) {
    MOE_HIP(hipEventRecord(c->reader[slots[i]], ks));
    c->has_reader[slots[i]] = 1;
  }
  return MOE_OK;
}
