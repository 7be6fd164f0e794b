// The HBM expert-slot cache: host-side LRU over (layer, expert) keys plus the
// stream/event protocol for filling slots from pinned host memory.
//
// Method: host RAM holds every routed expert; one GPU cache is shared by all
// MoE layers; in decode it is an LRU over recently selected experts, hits run
// on the GPU, misses are copied over PCIe (page "FreeToken量子化：MoE推論の
// セットアップガイド", hierarchy and decode paragraphs; bhrtaym-blog page,
// section "MoEバックエンドは4種類から選べる", backend table row "offload").
#include <string.h>

#include <set>
#include <utility>
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
  // statistics
  long long hits = 0, misses = 0, bytes_filled = 0;
  // per-step scratch of moe_cache_decode_step
  std::vector<int32_t> step_ids, step_slot, step_ev;
  std::vector<uint8_t> step_hit;
  // copies of the last resize, which a fill into a kept slot must follow
  hipEvent_t resized = nullptr;
  int has_resized = 0;
  // last upload from each host slot map: the map is rewritten only after it
  std::vector<std::pair<const void*, hipEvent_t>> map_upload;

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
  for (auto& m : c->map_upload) (void)hipEventDestroy(m.second);
  if (c->resized) (void)hipEventDestroy(c->resized);
  delete c;
}

extern "C" moe_status moe_cache_reset(moe_cache* c) {
  MOE_CHECK_ARG(c, "moe_cache_reset: null cache");
  c->reset();
  std::fill(c->has_reader.begin(), c->has_reader.end(), 0);
  c->hits = c->misses = c->bytes_filled = 0;
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
      ++c->hits;
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
    ++c->misses;
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

// Copy one blob into `slot` on the copy stream once the slot's last readers
// are done; records filled[slot].
static moe_status enqueue_fill(moe_cache* c, int slot, const void* host_src, hipStream_t cs) {
  if (c->has_reader[slot]) MOE_HIP(hipStreamWaitEvent(cs, c->reader[slot], 0));
  if (c->has_resized) MOE_HIP(hipStreamWaitEvent(cs, c->resized, 0));
  MOE_HIP(hipMemcpyAsync(c->pool + (size_t)slot * c->slot_bytes, host_src, c->slot_bytes, hipMemcpyHostToDevice, cs));
  MOE_HIP(hipEventRecord(c->filled[slot], cs));
  c->bytes_filled += (long long)c->slot_bytes;
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
  st = enqueue_fill(c, slot, host_src, cs);
  if (st != MOE_OK) return st;
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

extern "C" moe_status moe_cache_stats(const moe_cache* c, long long* hits, long long* misses, long long* bytes_filled) {
  MOE_CHECK_ARG(c && hits && misses && bytes_filled, "moe_cache_stats: null pointer");
  *hits = c->hits;
  *misses = c->misses;
  *bytes_filled = c->bytes_filled;
  return MOE_OK;
}

// ------------------------------------------------------------ one decode step

// dev_map / host_map layout: int32 slot_of_expert[E], uint8 hit_mask[E], uint8 miss_mask[E].
extern "C" size_t moe_cache_map_bytes(int E) {
  if (E <= 0) return 0;
  return ((size_t)E * 6 + 255) & ~(size_t)255;
}

// The upload of a pinned host map is asynchronous: before the host rewrites a
// map it waits for the last upload from that map (already done in the usual
// case), so steps that do not synchronise the host may share a map.
static moe_status map_before_write(moe_cache* c, const void* host_map, hipEvent_t* ev) {
  for (auto& m : c->map_upload)
    if (m.first == host_map) {
      MOE_HIP(hipEventSynchronize(m.second));
      *ev = m.second;
      return MOE_OK;
    }
  hipEvent_t e = nullptr;
  MOE_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  c->map_upload.emplace_back(host_map, e);
  *ev = e;
  return MOE_OK;
}

extern "C" moe_status moe_cache_decode_step(moe_cache* c, moe_cache_step* s, moe_stream_t copy_stream,
                                            moe_stream_t compute_stream) {
  MOE_CHECK_ARG(c && s, "moe_cache_decode_step: null pointer");
  const moe_ffn_args& f = s->ffn;
  const int E = f.E, T = f.T;
  s->n_experts = 0;
  MOE_CHECK_ARG(c->pool, "moe_cache_decode_step: cache has no slot pool");
  MOE_CHECK_ARG(E == c->num_experts, "moe_cache_decode_step: E=%d but the cache has %d experts per layer", E,
                c->num_experts);
  MOE_CHECK_ARG(s->layer >= 0 && s->layer < c->num_layers, "moe_cache_decode_step: layer %d out of range", s->layer);
  MOE_CHECK_ARG(T >= 0 && f.k >= 1 && f.k <= E, "moe_cache_decode_step: bad T=%d k=%d", T, f.k);
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(s->logits && s->topk_ids && s->host_counts && s->host_map && s->dev_map && s->host_blobs,
                "moe_cache_decode_step: null step buffer");
  MOE_CHECK_ARG(f.y && f.out && f.topk_w && f.inv && f.counts && f.offsets && f.perm,
                "moe_cache_decode_step: ffn.y, out, topk_w, inv, counts, offsets and perm are required");
  MOE_CHECK_ARG(((uintptr_t)s->dev_map & 255) == 0, "moe_cache_decode_step: dev_map must be 256-byte aligned");
  MOE_CHECK_ARG(c->slot_bytes % 256 == 0, "moe_cache_decode_step: slot_bytes %zu is not a multiple of 256",
                c->slot_bytes);
  hipStream_t ks = reinterpret_cast<hipStream_t>(compute_stream);
  hipStream_t cs = reinterpret_cast<hipStream_t>(copy_stream);
  moe_status st = ensure_events(c);
  if (st != MOE_OK) return st;

  // 1-2. routing, then the step's experts on the host
  st = moe_route_permute(s->logits, T, E, f.k, s->renormalize, s->topk_ids, const_cast<float*>(f.topk_w),
                         const_cast<int32_t*>(f.counts), const_cast<int32_t*>(f.offsets), const_cast<int32_t*>(f.perm),
                         const_cast<int32_t*>(f.inv), compute_stream);
  if (st != MOE_OK) return st;
  MOE_HIP(hipMemcpyAsync(s->host_counts, f.counts, sizeof(int32_t) * (size_t)E, hipMemcpyDeviceToHost, ks));
  MOE_HIP(hipStreamSynchronize(ks));
  c->step_ids.clear();
  for (int e = 0; e < E; ++e)
    if (s->host_counts[e] > 0) {
      MOE_CHECK_ARG(s->host_blobs[e], "moe_cache_decode_step: host blob of expert %d is null", e);
      c->step_ids.push_back(e);
    }
  const int n = (int)c->step_ids.size();
  c->step_slot.resize(n);
  c->step_hit.resize(n);
  c->step_ev.resize(n);

  // 3. lookup (the trace)
  st = cache_lookup(c, s->layer, c->step_ids.data(), n, c->step_slot.data(), c->step_hit.data(), c->step_ev.data());
  if (st != MOE_OK) return st;

  // 4. miss fills on the copy stream
  int nh = 0, nm = 0;
  for (int i = 0; i < n; ++i) {
    if (c->step_hit[i]) {
      ++nh;
      continue;
    }
    ++nm;
    st = enqueue_fill(c, c->step_slot[i], s->host_blobs[c->step_ids[i]], cs);
    if (st != MOE_OK) return st;
  }

  // 5. slot map and masks
  const size_t mb = moe_cache_map_bytes(E);
  int32_t* map = static_cast<int32_t*>(s->host_map);
  uint8_t* hm = reinterpret_cast<uint8_t*>(map + E);
  uint8_t* mm = hm + E;
  hipEvent_t up = nullptr;
  st = map_before_write(c, s->host_map, &up);
  if (st != MOE_OK) return st;
  memset(s->host_map, 0, mb);
  for (int i = 0; i < n; ++i) {
    map[c->step_ids[i]] = c->step_slot[i];
    (c->step_hit[i] ? hm : mm)[c->step_ids[i]] = 1;
  }
  MOE_HIP(hipMemcpyAsync(s->dev_map, s->host_map, mb, hipMemcpyHostToDevice, ks));
  MOE_HIP(hipEventRecord(up, ks));
  const int32_t* dmap = static_cast<const int32_t*>(s->dev_map);
  const uint8_t* dhm = reinterpret_cast<const uint8_t*>(dmap + E);
  const uint8_t* dmm = dhm + E;

  // 6. hits now, misses after their fills
  moe_ffn_args a = f;
  a.slot_of_expert = dmap;
  a.slot_pool = c->pool;
  a.slot_stride = c->slot_bytes;
  a.out = nullptr;
  if (nh > 0) {
    a.expert_mask = dhm;
    st = moe_expert_ffn(&a, compute_stream);
    if (st != MOE_OK) return st;
    a.shared_blob = nullptr;  // computed once
  }
  if (nm > 0) {
    for (int i = 0; i < n; ++i)
      if (!c->step_hit[i]) MOE_HIP(hipStreamWaitEvent(ks, c->filled[c->step_slot[i]], 0));
    a.expert_mask = dmm;
    st = moe_expert_ffn(&a, compute_stream);
    if (st != MOE_OK) return st;
  }

  // 7. combine, then the slots' readers
  const float* ysh = f.shared_blob ? f.y + (size_t)T * f.k * f.H : nullptr;
  st = moe_combine(f.y, f.inv, f.topk_w, ysh, T, f.k, f.H, f.out, compute_stream);
  if (st != MOE_OK) return st;
  st = moe_cache_mark_used(c, c->step_slot.data(), n, compute_stream);
  if (st != MOE_OK) return st;

  if (s->trace_expert && s->trace_slot && s->trace_hit && s->trace_evicted)
    for (int i = 0; i < n; ++i) {
      s->trace_expert[i] = c->step_ids[i];
      s->trace_slot[i] = c->step_slot[i];
      s->trace_hit[i] = c->step_hit[i];
      s->trace_evicted[i] = c->step_ev[i];
    }
  s->n_experts = n;
  return MOE_OK;
}

// ------------------------------------------------------------ resize at a safe point

// Blob moves of one launch: source slot of destination slot dst0 + b, passed
// by value (the kernel argument segment holds them; no device buffer).
constexpr int kMoveBatch = 256;
struct SlotMoves {
  int32_t src[kMoveBatch];
};

// Copy blob blockIdx.y of the batch (slot_vecs 16-byte vectors) from its old
// slot to slot dst0 + blockIdx.y; the x blocks stride over the vectors, four
// loads in flight per thread.  HBM-bound: one read and one write per byte.
__global__ __launch_bounds__(256) void k_move_slots(SlotMoves m, int dst0, const uint4* __restrict__ src_pool,
                                                    uint4* __restrict__ dst_pool, uint32_t slot_vecs) {
  const uint4* src = src_pool + (size_t)m.src[blockIdx.y] * slot_vecs;
  uint4* dst = dst_pool + (size_t)(dst0 + blockIdx.y) * slot_vecs;
  const uint32_t step = gridDim.x * 256u;
  for (uint32_t v = blockIdx.x * 256u + threadIdx.x; v < slot_vecs; v += 4 * step) {
    uint4 r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (v + j * step < slot_vecs) r[j] = src[v + j * step];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (v + j * step < slot_vecs) dst[v + j * step] = r[j];
  }
}

extern "C" moe_status moe_cache_resize(moe_cache* c, int num_slots, void* slot_pool, moe_stream_t stream) {
  MOE_CHECK_ARG(c && slot_pool, "moe_cache_resize: null pointer");
  MOE_CHECK_ARG(c->pool, "moe_cache_resize: cache has no slot pool");
  MOE_CHECK_ARG(num_slots > 0, "moe_cache_resize: num_slots %d must be positive", num_slots);
  MOE_CHECK_ARG(((uintptr_t)slot_pool & 255) == 0, "moe_cache_resize: slot_pool must be 256-byte aligned");
  MOE_CHECK_ARG(((uintptr_t)c->pool & 15) == 0 && c->slot_bytes % 16 == 0 && c->slot_bytes / 16 < (1ull << 31),
                "moe_cache_resize: slot size and current pool must be multiples of 16 bytes");
  const uint8_t* np = static_cast<const uint8_t*>(slot_pool);
  const size_t nbytes = (size_t)num_slots * c->slot_bytes, obytes = (size_t)c->num_slots * c->slot_bytes;
  MOE_CHECK_ARG(np + nbytes <= c->pool || c->pool + obytes <= np,
                "moe_cache_resize: the new slot pool overlaps the current one");
  moe_status st = ensure_events(c);
  if (st != MOE_OK) return st;
  if (!c->resized) MOE_HIP(hipEventCreateWithFlags(&c->resized, hipEventDisableTiming));
  // keys from least to most recent; the least recent beyond num_slots are dropped
  std::vector<int32_t> keys;
  for (int32_t k = c->head; k >= 0; k = c->next[k]) keys.push_back(k);
  const int nkeep = std::min<int>((int)keys.size(), num_slots), ndrop = (int)keys.size() - nkeep;
  // the slots' events are reused (a stale record only makes a later wait
  // stricter: readers are reset below, fills are waited for here)
  for (int s = (int)c->filled.size(); s < num_slots; ++s) {
    hipEvent_t f = nullptr, r = nullptr;
    MOE_HIP(hipEventCreateWithFlags(&f, hipEventDisableTiming));
    c->filled.push_back(f);
    MOE_HIP(hipEventCreateWithFlags(&r, hipEventDisableTiming));
    c->reader.push_back(r);
  }
  // the copies start once every kept blob's fill has landed (fills still in
  // flight are waited for; finished ones cost nothing)
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  for (int i = 0; i < nkeep; ++i) {
    hipEvent_t f = c->filled[c->key_slot[keys[ndrop + i]]];
    if (hipEventQuery(f) != hipSuccess) MOE_HIP(hipStreamWaitEvent(hs, f, 0));
  }
  const uint32_t vecs = (uint32_t)(c->slot_bytes / 16);
  const int gx = (int)std::min<uint32_t>(64, (vecs + 1023) / 1024);
  for (int b0 = 0; b0 < nkeep; b0 += kMoveBatch) {
    const int n = std::min(kMoveBatch, nkeep - b0);
    SlotMoves m{};
    for (int b = 0; b < n; ++b) m.src[b] = c->key_slot[keys[ndrop + b0 + b]];
    moe::launch(k_move_slots, dim3(gx, n), dim3(256), 0, hs, m, b0, reinterpret_cast<const uint4*>(c->pool),
                reinterpret_cast<uint4*>(slot_pool), vecs);
    MOE_HIP(hipGetLastError());
  }
  // a later fill into a kept slot (on any stream) must follow the copies
  MOE_HIP(hipEventRecord(c->resized, hs));
  c->has_resized = 1;
  for (int i = 0; i < ndrop; ++i) {
    c->unlink(keys[i]);
    c->key_slot[keys[i]] = -1;
  }
  // events beyond num_slots are kept for a later growth (destroyed with the cache)
  c->num_slots = num_slots;
  c->pool = static_cast<uint8_t*>(slot_pool);
  c->slot_key.assign(num_slots, -1);
  c->has_reader.assign(num_slots, 0);
  for (int i = 0; i < nkeep; ++i) {
    c->key_slot[keys[ndrop + i]] = i;
    c->slot_key[i] = keys[ndrop + i];
  }
  c->free_slots.clear();
  for (int s = nkeep; s < num_slots; ++s) c->free_slots.insert(s);
  return MOE_OK;
}
