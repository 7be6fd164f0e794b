// The HBM expert-slot cache: host-side LRU over (layer, expert) keys plus the
// stream/event protocol for filling slots from pinned host memory.  Host code
// only (the HIP runtime API); the blob moves of a resize are launched through
// launch_move_slots (cache_kernels.hip).
//
// Method: host RAM holds every routed expert; one GPU cache is shared by all
// MoE layers; in decode it is an LRU over recently selected experts, hits run
// on the GPU, misses are copied over PCIe (page "FreeToken量子化：MoE推論の
// セットアップガイド", hierarchy and decode paragraphs; bhrtaym-blog page,
// section "MoEバックエンドは4種類から選べる", backend table row "offload").
// In prefill the next layer's experts are copied while the current layer
// computes (the same page, paragraph on prefill double buffering).
//
// Ordering protocol (one compute stream per cache; fills on copy streams):
//  - write after read: a fill waits for the last readers of its slot.  Each
//    marking of readers records one event from a ring of kRing events on the
//    compute stream; a slot keeps the generation of its last marking.  A
//    ring event is re-recorded only after the host has waited for its
//    previous record, so a slot whose marking is older than kRing needs no
//    wait at all.
//  - read after write: a fill records filled[slot]; the step that first
//    reads the slot makes the compute stream wait for it (pending flag).
//  - a resize copies kept blobs after every fill enqueued so far, through a
//    tail event per copy stream recorded after its last fill.
//  - a decode step on the decode GEMV may copy its misses with a fill kernel
//    on the compute stream instead (pinned blobs read by the shader over
//    PCIe): its miss FFN then follows the fills in stream order, and its hit
//    FFN runs meanwhile on a side stream whose completion the compute stream
//    waits for before the combine.  Such a step starts after the host has
//    seen its counts, which the compute stream published after every earlier
//    step's combine, so no earlier reader or fill of any slot is still
//    running when it enqueues.
#include <string.h>

#include <algorithm>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "host_common.h"

namespace moe {
hipError_t launch_move_slots(const int32_t* src_slots, int n, int dst0, const void* src_pool, void* dst_pool,
                             size_t slot_bytes, hipStream_t s);
hipError_t launch_write_map(const StepMap& m, int E, void* dev_map, hipStream_t s);
hipError_t launch_fill_slots(const FillList& f, const StepMap& m, int E, void* dev_map, void* pool, size_t slot_bytes,
                             hipStream_t s);
bool ffn_takes_gemv(const moe_ffn_args* a);
moe_status expert_ffn_fill(const moe_ffn_args* a, const FillList& f, void* pool, size_t slot_bytes, hipStream_t s);
}

struct moe_cache {
  static constexpr int kRing = 256;
  int num_slots = 0, num_layers = 0, num_experts = 0;
  size_t slot_bytes = 0;
  uint8_t* pool = nullptr;
  // LRU as an intrusive doubly linked list over keys; head = least recent.
  std::vector<int32_t> key_slot;   // key -> slot or -1
  std::vector<int32_t> slot_key;   // slot -> key or -1
  std::vector<int32_t> prev, next; // per key
  int32_t head = -1, tail = -1;
  std::set<int32_t> free_slots;
  // fills: per-slot completion events and pending flags; per copy stream the
  // event recorded after its last fill
  std::vector<hipEvent_t> filled;
  std::vector<uint8_t> fill_pending;
  std::vector<std::pair<hipStream_t, hipEvent_t>> fill_tail;
  // readers: the ring of marking events and each slot's last marking
  std::vector<hipEvent_t> ring;
  long long gen = 0;
  std::vector<long long> reader_gen;  // -1: no reader recorded
  // statistics
  long long hits = 0, misses = 0, bytes_filled = 0;
  // per-step scratch
  std::vector<int32_t> step_ids, step_slot, step_ev;
  std::vector<uint8_t> step_hit;
  // copies of the last resize, which a fill into a kept slot must follow
  hipEvent_t resized = nullptr;
  int has_resized = 0;
  // last upload from each host slot map: the map is rewritten only after it
  std::vector<std::pair<const void*, hipEvent_t>> map_upload;
  // decode-step handoff: a host-mapped flag the GPU publishes each step's
  // sequence number in (publish: -1 not tried yet, 0 unavailable, 1 ready),
  // and the device addresses of the host-count buffers
  int publish = -1;
  uint32_t* flag_host = nullptr;
  uint32_t* flag_dev = nullptr;
  uint32_t seq = 0;
  std::unordered_map<const void*, void*> mapped;  // host address -> device address (null: not mapped)
  // decode steps whose misses a kernel copies on the compute stream: the
  // hits run meanwhile on a side stream with their own slot map, and
  // hit_done joins them back before the combine (copy_engine: 1 forces the
  // copy-engine fills instead)
  int copy_engine = 0;
  hipStream_t side = nullptr;
  hipEvent_t hit_done = nullptr;
  void* side_map = nullptr;
  size_t side_map_bytes = 0;

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
  c->fill_pending.assign(num_slots, 0);
  c->reader_gen.assign(num_slots, -1);
  c->reset();
  return c;
}

extern "C" void moe_cache_destroy(moe_cache* c) {
  if (!c) return;
  for (hipEvent_t e : c->ring) if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : c->filled) if (e) (void)hipEventDestroy(e);
  for (auto& t : c->fill_tail) (void)hipEventDestroy(t.second);
  for (auto& m : c->map_upload) (void)hipEventDestroy(m.second);
  if (c->resized) (void)hipEventDestroy(c->resized);
  if (c->flag_host) (void)hipHostFree(c->flag_host);
  if (c->hit_done) (void)hipEventDestroy(c->hit_done);
  if (c->side) (void)hipStreamDestroy(c->side);
  if (c->side_map) (void)hipFree(c->side_map);
  delete c;
}

extern "C" moe_status moe_cache_reset(moe_cache* c) {
  MOE_CHECK_ARG(c, "moe_cache_reset: null cache");
  c->reset();
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

// ------------------------------------------------------------ the ordering protocol

// Per-slot fill events and the reader ring, created on first use.
// (On a failure the events created so far are released or kept complete:
// the ring is adopted only whole.)
static moe_status ensure_events(moe_cache* c) {
  if (c->ring.empty()) {
    std::vector<hipEvent_t> ring(moe_cache::kRing, nullptr);
    for (auto& e : ring) {
      const hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableTiming);
      if (err != hipSuccess) {
        for (hipEvent_t x : ring) if (x) (void)hipEventDestroy(x);
        return moe::set_error(MOE_EHIP, "hipEventCreateWithFlags failed: %s", hipGetErrorString(err));
      }
    }
    c->ring.swap(ring);
  }
  while ((int)c->filled.size() < c->num_slots) {
    hipEvent_t f = nullptr;
    MOE_HIP(hipEventCreateWithFlags(&f, hipEventDisableTiming));
    c->filled.push_back(f);
  }
  return MOE_OK;
}

// The copy stream waits for the last readers of `slot` (write after read).
static moe_status wait_readers(moe_cache* c, int slot, hipStream_t cs) {
  const long long g = c->reader_gen[slot];
  // the ring entry of generation g is re-recorded at g + kRing, after the
  // host waited for this record: then the readers have finished
  if (g < 0 || c->gen > g + moe_cache::kRing) return MOE_OK;
  MOE_HIP(hipStreamWaitEvent(cs, c->ring[g % moe_cache::kRing], 0));
  return MOE_OK;
}

// Record that slots[0..n) are read by the work enqueued on ks so far.
static moe_status mark_readers(moe_cache* c, const int32_t* slots, int n, hipStream_t ks) {
  if (n == 0) return MOE_OK;
  const long long g = c->gen;
  hipEvent_t e = c->ring[g % moe_cache::kRing];
  if (g >= moe_cache::kRing) MOE_HIP(hipEventSynchronize(e));  // its record of kRing markings ago
  MOE_HIP(hipEventRecord(e, ks));
  for (int i = 0; i < n; ++i) c->reader_gen[slots[i]] = g;
  ++c->gen;
  return MOE_OK;
}

// Copy one blob into `slot` on the copy stream once the slot's last readers
// (and any resize copy) are done; records filled[slot].
static moe_status enqueue_fill(moe_cache* c, int slot, const void* host_src, hipStream_t cs) {
  moe_status st = wait_readers(c, slot, cs);
  if (st != MOE_OK) return st;
  if (c->has_resized) MOE_HIP(hipStreamWaitEvent(cs, c->resized, 0));
  MOE_HIP(hipMemcpyAsync(c->pool + (size_t)slot * c->slot_bytes, host_src, c->slot_bytes, hipMemcpyHostToDevice, cs));
  MOE_HIP(hipEventRecord(c->filled[slot], cs));
  c->fill_pending[slot] = 1;
  c->bytes_filled += (long long)c->slot_bytes;
  return MOE_OK;
}

static moe_status note_fill_tail(moe_cache* c, hipStream_t cs);

// After a fill of the step's lookups failed to enqueue: the misses from
// index i0 on (whose blobs will not arrive) leave the cache and their slots
// become free, so no key maps to a slot without its blob.  Keys they evicted
// stay evicted.
static void drop_unfilled(moe_cache* c, int layer, int i0, int n) {
  for (int i = i0; i < n; ++i) {
    if (c->step_hit[i]) continue;
    const int32_t k = layer * c->num_experts + c->step_ids[i];
    const int32_t s = c->key_slot[k];
    if (s < 0) continue;
    c->unlink(k);
    c->key_slot[k] = -1;
    c->slot_key[s] = -1;
    c->free_slots.insert(s);
  }
}

// Fills of the step's misses (the lookups in step_ids / step_slot /
// step_hit) on cs; on a failure the unfilled misses are dropped.
static moe_status fill_misses(moe_cache* c, int layer, int n, const void* const* host_blobs, hipStream_t cs,
                              int* n_miss) {
  int nm = 0;
  for (int i = 0; i < n; ++i) {
    if (c->step_hit[i]) continue;
    const moe_status st = enqueue_fill(c, c->step_slot[i], host_blobs[c->step_ids[i]], cs);
    if (st != MOE_OK) {
      drop_unfilled(c, layer, i, n);
      return st;
    }
    ++nm;
  }
  *n_miss = nm;
  if (nm > 0) return note_fill_tail(c, cs);
  return MOE_OK;
}

// The compute stream waits for the fill of `slot` if no earlier wait covers it.
static moe_status wait_fill(moe_cache* c, int slot, hipStream_t ks) {
  if (!c->fill_pending[slot]) return MOE_OK;
  MOE_HIP(hipStreamWaitEvent(ks, c->filled[slot], 0));
  c->fill_pending[slot] = 0;
  return MOE_OK;
}

// Records the copy stream's tail event after its latest fills.
static moe_status note_fill_tail(moe_cache* c, hipStream_t cs) {
  for (auto& t : c->fill_tail)
    if (t.first == cs) {
      MOE_HIP(hipEventRecord(t.second, cs));
      return MOE_OK;
    }
  hipEvent_t e = nullptr;
  MOE_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  c->fill_tail.emplace_back(cs, e);
  MOE_HIP(hipEventRecord(e, cs));
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
  st = note_fill_tail(c, cs);
  if (st != MOE_OK) return st;
  return wait_fill(c, slot, ks);
}

extern "C" moe_status moe_cache_use_copy_engine(moe_cache* c, int on) {
  MOE_CHECK_ARG(c, "moe_cache_use_copy_engine: null cache");
  c->copy_engine = on ? 1 : 0;
  return MOE_OK;
}

extern "C" moe_status moe_cache_mark_used(moe_cache* c, const int32_t* slots, int n, moe_stream_t compute_stream) {
  MOE_CHECK_ARG(c && (n == 0 || slots), "moe_cache_mark_used: null pointer");
  for (int i = 0; i < n; ++i)
    MOE_CHECK_ARG(slots[i] >= 0 && slots[i] < c->num_slots, "moe_cache_mark_used: slot %d out of range", slots[i]);
  moe_status st = ensure_events(c);
  if (st != MOE_OK) return st;
  return mark_readers(c, slots, n, reinterpret_cast<hipStream_t>(compute_stream));
}

extern "C" moe_status moe_cache_stats(const moe_cache* c, long long* hits, long long* misses, long long* bytes_filled) {
  MOE_CHECK_ARG(c && hits && misses && bytes_filled, "moe_cache_stats: null pointer");
  *hits = c->hits;
  *misses = c->misses;
  *bytes_filled = c->bytes_filled;
  return MOE_OK;
}

// ------------------------------------------------------------ slot maps

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

// Writes the step's map into host_map (slots and the hit / miss masks of
// step_ids) and uploads it to dev_map on ks.
static moe_status upload_map(moe_cache* c, void* host_map, void* dev_map, int E, int n, hipStream_t ks) {
  hipEvent_t up = nullptr;
  moe_status st = map_before_write(c, host_map, &up);
  if (st != MOE_OK) return st;
  const size_t mb = moe_cache_map_bytes(E);
  int32_t* map = static_cast<int32_t*>(host_map);
  uint8_t* hm = reinterpret_cast<uint8_t*>(map + E);
  uint8_t* mm = hm + E;
  memset(host_map, 0, mb);
  for (int i = 0; i < n; ++i) {
    map[c->step_ids[i]] = c->step_slot[i];
    (c->step_hit[i] ? hm : mm)[c->step_ids[i]] = 1;
  }
  MOE_HIP(hipMemcpyAsync(dev_map, host_map, mb, hipMemcpyHostToDevice, ks));
  MOE_HIP(hipEventRecord(up, ks));
  return MOE_OK;
}

static void copy_trace(const moe_cache* c, int n, int32_t* te, int32_t* ts, uint8_t* th, int32_t* tv) {
  for (int i = 0; i < n; ++i) {
    if (te) te[i] = c->step_ids[i];
    ts[i] = c->step_slot[i];
    th[i] = c->step_hit[i];
    tv[i] = c->step_ev[i];
  }
}

// ------------------------------------------------------------ decode-step handoffs

// The device address of pinned host memory (null if it is not mapped for
// the device; the failed query's error is cleared).
static void* mapped_device_ptr(moe_cache* c, const void* host) {
  const auto it = c->mapped.find(host);
  if (it != c->mapped.end()) return it->second;
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, const_cast<void*>(host), 0) != hipSuccess) {
    (void)hipGetLastError();
    d = nullptr;
  }
  c->mapped.emplace(host, d);
  return d;
}

// The host-mapped, coherent flag of the count handoff (allocated on first
// use; without it the steps copy the counts and synchronise the stream).
static void ensure_flag(moe_cache* c) {
  if (c->publish >= 0) return;
  c->publish = 0;
  void* h = nullptr;
  if (hipHostMalloc(&h, 256, hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess) {
    (void)hipGetLastError();
    return;
  }
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, h, 0) != hipSuccess || !d) {
    (void)hipGetLastError();
    (void)hipHostFree(h);
    return;
  }
  c->flag_host = static_cast<uint32_t*>(h);
  c->flag_dev = static_cast<uint32_t*>(d);
  __atomic_store_n(c->flag_host, 0u, __ATOMIC_RELEASE);
  c->publish = 1;
}

// Waits (polling) until the GPU has published `seq`; checks the stream for
// errors every few thousand polls.
static moe_status wait_flag(moe_cache* c, uint32_t seq, hipStream_t ks, const char* who) {
  for (unsigned long long spin = 1;; ++spin) {
    if (__atomic_load_n(c->flag_host, __ATOMIC_ACQUIRE) == seq) return MOE_OK;
    __builtin_ia32_pause();
    if ((spin & 0xFFF) == 0) {
      const hipError_t q = hipStreamQuery(ks);
      if (q == hipSuccess) {
        if (__atomic_load_n(c->flag_host, __ATOMIC_ACQUIRE) == seq) return MOE_OK;
        return moe::set_error(MOE_EHIP, "%s: the stream finished without publishing the step's counts", who);
      }
      if (q != hipErrorNotReady) return moe::set_error(MOE_EHIP, "%s: %s", who, hipGetErrorString(q));
    }
  }
}

// The step's map (the lookups in step_ids / step_slot / step_hit) into
// dev_map on ks: by a kernel that takes it by value, or for steps with more
// than kStepMapMax experts through host_map.
static void step_map(const moe_cache* c, int n, moe::StepMap* m) {
  m->n = n;
  for (int i = 0; i < n; ++i) {
    m->expert[i] = c->step_ids[i];
    m->slot[i] = c->step_slot[i];
    m->hit[i] = c->step_hit[i];
  }
}
static moe_status write_map(moe_cache* c, void* host_map, void* dev_map, int E, int n, hipStream_t ks) {
  if (n > moe::kStepMapMax) return upload_map(c, host_map, dev_map, E, n, ks);
  moe::StepMap m;
  step_map(c, n, &m);
  const hipError_t e = moe::launch_write_map(m, E, dev_map, ks);
  if (e != hipSuccess) return moe::set_error(MOE_EHIP, "slot map launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

// The step's miss fills as two kernel copy lists: `head` (the blob header
// and the gate/up weights, bytes [0, off_w2)) for the fill kernel and `tail`
// (the down weights to the slot's end) for the copy workgroups of the miss
// FFN's gate/up launch, which copy them while the gate/up runs.  False when
// the fills go through the copy engine instead: the FFN is off the GEMV path
// (the hit and miss launches would share workspace, so they cannot run at
// once), too many experts or misses for the kernel arguments, or a blob that
// is not mapped pinned memory on a 16-byte boundary.
static bool kernel_fill_list(moe_cache* c, const moe_ffn_args& f, const void* const* host_blobs, int n, int nm,
                             moe::FillList* head, moe::FillList* tail) {
  moe::BlobLayout L;
  if (c->copy_engine || nm == 0 || nm > moe::kFillMax || n > moe::kStepMapMax || !moe::ffn_takes_gemv(&f) ||
      c->slot_bytes / 16 >= (1ull << 31) || !moe::layout_of(f.wfmt, f.H, f.I, &L) || L.total > c->slot_bytes)
    return false;
  head->n = 0;
  for (int i = 0; i < n; ++i) {
    if (c->step_hit[i]) continue;
    const void* d = mapped_device_ptr(c, host_blobs[c->step_ids[i]]);
    if (!d || ((uintptr_t)d & 15)) return false;
    head->slot[head->n] = c->step_slot[i];
    head->src[head->n] = static_cast<const uint8_t*>(d);
    ++head->n;
  }
  const uint32_t vecs = (uint32_t)(c->slot_bytes / 16), split = (uint32_t)(L.off_w2 / 16);
  *tail = *head;
  head->off16 = 0;
  head->len16 = split;
  tail->off16 = split;
  tail->len16 = vecs - split;
  return true;
}

// The side stream of the hit FFN, its join event and its slot map (created
// on first use, kept until the cache is destroyed).
static moe_status ensure_side(moe_cache* c) {
  if (!c->side) MOE_HIP(hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking));
  if (!c->hit_done) MOE_HIP(hipEventCreateWithFlags(&c->hit_done, hipEventDisableTiming));
  if (!c->side_map) {
    const size_t mb = moe_cache_map_bytes(c->num_experts);
    MOE_HIP(hipMalloc(&c->side_map, mb));
    c->side_map_bytes = mb;
  }
  return MOE_OK;
}

// ------------------------------------------------------------ one decode step

// A step that returns early after enqueueing its hits on the side stream
// waits for them on the host, so that no later fill overwrites a slot they
// still read (the compute stream never joined them).
struct SideJoin {
  moe_cache* c;
  bool pending;
  ~SideJoin() {
    if (pending && c->side) (void)hipStreamSynchronize(c->side);
  }
};

// One decode step; hy null: every miss copied into the cache.
static moe_status decode_step(moe_cache* c, moe_cache_step* s, moe_hybrid* hy, moe_stream_t copy_stream,
                              moe_stream_t compute_stream, const char* who) {
  MOE_CHECK_ARG(c && s, "%s: null pointer", who);
  const moe_ffn_args& f = s->ffn;
  const int E = f.E, T = f.T;
  s->n_experts = 0;
  MOE_CHECK_ARG(c->pool, "%s: cache has no slot pool", who);
  MOE_CHECK_ARG(E == c->num_experts, "%s: E=%d but the cache has %d experts per layer", who, E, c->num_experts);
  MOE_CHECK_ARG(s->layer >= 0 && s->layer < c->num_layers, "%s: layer %d out of range", who, s->layer);
  MOE_CHECK_ARG(T >= 0 && f.k >= 1 && f.k <= E, "%s: bad T=%d k=%d", who, T, f.k);
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(s->logits && s->topk_ids && s->host_counts && s->host_map && s->dev_map && s->host_blobs,
                "%s: null step buffer", who);
  MOE_CHECK_ARG(f.y && f.out && f.topk_w && f.inv && f.counts && f.offsets && f.perm,
                "%s: ffn.y, out, topk_w, inv, counts, offsets and perm are required", who);
  MOE_CHECK_ARG(((uintptr_t)s->dev_map & 255) == 0, "%s: dev_map must be 256-byte aligned", who);
  MOE_CHECK_ARG(c->slot_bytes % 256 == 0, "%s: slot_bytes %zu is not a multiple of 256", who, c->slot_bytes);
  if (hy)
    MOE_CHECK_ARG(hy->copy_ratio >= 0.f && hy->copy_ratio <= 1.f && hy->threads >= 1 && hy->host_x &&
                      hy->host_perm && hy->host_offsets && hy->host_y,
                  "%s: bad hybrid policy or host buffers", who);
  hipStream_t ks = reinterpret_cast<hipStream_t>(compute_stream);
  hipStream_t cs = reinterpret_cast<hipStream_t>(copy_stream);
  moe_status st = ensure_events(c);
  if (st != MOE_OK) return st;

  // 1-2. routing, then the step's experts on the host (and, for host-run
  // misses, the rows they take)
  ensure_flag(c);
  int32_t* counts_dev = (c->publish == 1 && !hy) ? static_cast<int32_t*>(mapped_device_ptr(c, s->host_counts)) : nullptr;
  if (counts_dev) {
    // the routing writes the counts into the mapped host buffer and then
    // publishes the step's number; the host polls for it
    const uint32_t seq = ++c->seq;
    st = moe::route_permute_publish(s->logits, T, E, f.k, s->renormalize, s->topk_ids, const_cast<float*>(f.topk_w),
                                    const_cast<int32_t*>(f.counts), const_cast<int32_t*>(f.offsets),
                                    const_cast<int32_t*>(f.perm), const_cast<int32_t*>(f.inv), counts_dev, c->flag_dev,
                                    seq, ks);
    if (st != MOE_OK) return st;
    st = wait_flag(c, seq, ks, who);
    if (st != MOE_OK) return st;
  } else {
    st = moe_route_permute(s->logits, T, E, f.k, s->renormalize, s->topk_ids, const_cast<float*>(f.topk_w),
                           const_cast<int32_t*>(f.counts), const_cast<int32_t*>(f.offsets), const_cast<int32_t*>(f.perm),
                           const_cast<int32_t*>(f.inv), compute_stream);
    if (st != MOE_OK) return st;
    MOE_HIP(hipMemcpyAsync(s->host_counts, f.counts, sizeof(int32_t) * (size_t)E, hipMemcpyDeviceToHost, ks));
    if (hy) {
      MOE_HIP(hipMemcpyAsync(hy->host_offsets, f.offsets, sizeof(int32_t) * (size_t)(E + 1), hipMemcpyDeviceToHost, ks));
      MOE_HIP(hipMemcpyAsync(hy->host_perm, f.perm, sizeof(int32_t) * (size_t)T * f.k, hipMemcpyDeviceToHost, ks));
      MOE_HIP(hipMemcpyAsync(hy->host_x, f.x, sizeof(uint16_t) * (size_t)T * f.H, hipMemcpyDeviceToHost, ks));
    }
    MOE_HIP(hipStreamSynchronize(ks));
  }
  std::vector<int32_t> all, host_run;  // the step's experts; those run on the host
  for (int e = 0; e < E; ++e)
    if (s->host_counts[e] > 0) {
      MOE_CHECK_ARG(s->host_blobs[e], "%s: host blob of expert %d is null", who, e);
      all.push_back(e);
    }
  c->step_ids.clear();
  if (hy) {
    int m = 0;
    for (int e : all) m += c->key_slot[(size_t)s->layer * E + e] < 0;
    const int ncopy = (int)(hy->copy_ratio * (float)m + 0.5f);
    int seen = 0;
    for (int e : all) {
      const bool miss = c->key_slot[(size_t)s->layer * E + e] < 0;
      if (miss && seen++ >= ncopy) host_run.push_back(e);
      else c->step_ids.push_back(e);
    }
  } else {
    c->step_ids = all;
  }
  const int n = (int)c->step_ids.size();
  c->step_slot.resize(n);
  c->step_hit.resize(n);
  c->step_ev.resize(n);

  // 3. lookup (the trace)
  st = cache_lookup(c, s->layer, c->step_ids.data(), n, c->step_slot.data(), c->step_hit.data(), c->step_ev.data());
  if (st != MOE_OK) return st;

  // 4-6. miss fills, the slot map and the hit FFN.  With a fill kernel the
  // misses are copied on the compute stream (their FFN follows in stream
  // order) and the hits run meanwhile on the side stream; otherwise the copy
  // engine fills them on the copy stream and the hits run first on the
  // compute stream.
  int nm = 0;
  for (int i = 0; i < n; ++i) nm += !c->step_hit[i];
  const int nh = n - nm;
  moe::FillList fl, fl_tail;
  const bool kfill = kernel_fill_list(c, f, s->host_blobs, n, nm, &fl, &fl_tail);
  const int32_t* dmap = static_cast<const int32_t*>(s->dev_map);
  const uint8_t* dhm = reinterpret_cast<const uint8_t*>(dmap + E);
  const uint8_t* dmm = dhm + E;
  moe_ffn_args a = f;
  a.slot_of_expert = dmap;
  a.slot_pool = c->pool;
  a.slot_stride = c->slot_bytes;
  a.out = nullptr;
  SideJoin join{c, false};
  if (kfill) {
    // The fills first, then the missed experts' FFN: the step's critical
    // path, enqueued before anything else.  Every earlier reader and
    // kernel fill of the slots is behind the host already: this step's counts
    // were published after them on the compute stream, and an earlier step's
    // hits joined it before that step's combine.  A copy-engine fill of a
    // slot that no step has waited for yet is waited for (write after
    // write).  A failure before the fill launch drops the misses.
    moe::StepMap m;
    step_map(c, n, &m);
    for (int i = 0; i < n && st == MOE_OK; ++i)
      if (!c->step_hit[i]) {
        st = wait_readers(c, c->step_slot[i], ks);
        if (st == MOE_OK) st = wait_fill(c, c->step_slot[i], ks);
      }
    if (st == MOE_OK && c->has_resized) {
      const hipError_t e = hipStreamWaitEvent(ks, c->resized, 0);
      if (e != hipSuccess) st = moe::set_error(MOE_EHIP, "%s: %s", who, hipGetErrorString(e));
    }
    if (st == MOE_OK) {
      const hipError_t e = moe::launch_fill_slots(fl, m, E, s->dev_map, c->pool, c->slot_bytes, ks);
      if (e != hipSuccess) st = moe::set_error(MOE_EHIP, "%s: fill launch failed: %s", who, hipGetErrorString(e));
    }
    if (st != MOE_OK) {
      drop_unfilled(c, s->layer, 0, n);
      return st;
    }
    c->bytes_filled += (long long)nm * (long long)c->slot_bytes;
    // the missed experts next (the gate/up launch copies their down weights
    // while it runs); the shared expert goes with the hits when there are any
    moe_ffn_args am = a;
    am.expert_mask = dmm;
    if (nh > 0) am.shared_blob = nullptr;
    st = moe::expert_ffn_fill(&am, fl_tail, c->pool, c->slot_bytes, ks);
    if (st != MOE_OK) {
      drop_unfilled(c, s->layer, 0, n);  // their down weights may never have arrived
      return st;
    }
    // then the hits on the side stream, with their own copy of the map
    if (nh > 0) {
      join.pending = true;
      st = ensure_side(c);
      if (st != MOE_OK) return st;
      const hipError_t e = moe::launch_write_map(m, E, c->side_map, c->side);
      if (e != hipSuccess) return moe::set_error(MOE_EHIP, "%s: slot map launch failed: %s", who, hipGetErrorString(e));
      for (int i = 0; i < n; ++i)
        if (c->step_hit[i] && (st = wait_fill(c, c->step_slot[i], c->side)) != MOE_OK) return st;
      moe_ffn_args ah = a;
      ah.slot_of_expert = static_cast<const int32_t*>(c->side_map);
      ah.expert_mask = static_cast<const uint8_t*>(c->side_map) + 4 * (size_t)E;
      st = moe_expert_ffn(&ah, reinterpret_cast<moe_stream_t>(c->side));
      if (st != MOE_OK) return st;
      MOE_HIP(hipEventRecord(c->hit_done, c->side));
    }
  } else {
    int nq = 0;
    st = fill_misses(c, s->layer, n, s->host_blobs, cs, &nq);
    if (st != MOE_OK) return st;
    st = write_map(c, s->host_map, s->dev_map, E, n, ks);
    if (st != MOE_OK) return st;
    // hits now (after any fill of theirs still pending)
    if (nh > 0 || (nm == 0 && f.shared_blob)) {
      for (int i = 0; i < n; ++i)
        if (c->step_hit[i] && (st = wait_fill(c, c->step_slot[i], ks)) != MOE_OK) return st;
      a.expert_mask = dhm;
      st = moe_expert_ffn(&a, compute_stream);
      if (st != MOE_OK) return st;
      a.shared_blob = nullptr;  // computed once
    }
  }
  // 6b. host-run misses while the GPU works: their rows' outputs into host_y
  // (perm order), then into y
  if (!host_run.empty()) {
    hipEvent_t up = nullptr;
    st = map_before_write(c, hy->host_y, &up);  // the previous upload from host_y has finished
    if (st != MOE_OK) return st;
    std::vector<uint16_t> xg;
    for (int e : host_run) {
      const int p0 = hy->host_offsets[e], cnt = hy->host_offsets[e + 1] - p0;
      xg.resize((size_t)cnt * f.H);
      for (int r = 0; r < cnt; ++r)
        memcpy(&xg[(size_t)r * f.H], hy->host_x + (size_t)(hy->host_perm[p0 + r] / f.k) * f.H, 2 * (size_t)f.H);
      st = moe_cpu_expert_ffn(s->host_blobs[e], xg.data(), cnt, hy->host_y + (size_t)p0 * f.H, hy->threads);
      if (st != MOE_OK) return st;
      MOE_HIP(hipMemcpyAsync(f.y + (size_t)p0 * f.H, hy->host_y + (size_t)p0 * f.H, sizeof(float) * (size_t)cnt * f.H,
                             hipMemcpyHostToDevice, ks));
    }
    MOE_HIP(hipEventRecord(up, ks));
    hy->cpu_experts += (long long)host_run.size();
  }
  // 6c. copy-engine misses after their fills
  if (nm > 0 && !kfill) {
    for (int i = 0; i < n; ++i)
      if (!c->step_hit[i] && (st = wait_fill(c, c->step_slot[i], ks)) != MOE_OK) return st;
    a.expert_mask = dmm;
    st = moe_expert_ffn(&a, compute_stream);
    if (st != MOE_OK) return st;
  }
  if (join.pending) {
    MOE_HIP(hipStreamWaitEvent(ks, c->hit_done, 0));
    join.pending = false;
  }

  // 7. combine, then the slots' readers (one marking for the step)
  const float* ysh = f.shared_blob ? f.y + (size_t)T * f.k * f.H : nullptr;
  st = moe_combine(f.y, f.inv, f.topk_w, ysh, T, f.k, f.H, f.out, compute_stream);
  if (st != MOE_OK) return st;
  st = mark_readers(c, c->step_slot.data(), n, ks);
  if (st != MOE_OK) return st;

  // trace: every expert of the step in ascending id (host-run misses: -1 slot)
  if (s->trace_slot && s->trace_hit && s->trace_evicted) {
    size_t i = 0, j = 0;
    for (int e : all) {
      const bool looked = i < c->step_ids.size() && c->step_ids[i] == e;
      if (s->trace_expert) s->trace_expert[j] = e;
      s->trace_slot[j] = looked ? c->step_slot[i] : -1;
      s->trace_hit[j] = looked ? c->step_hit[i] : 0;
      s->trace_evicted[j] = looked ? c->step_ev[i] : -1;
      i += looked;
      ++j;
    }
  }
  s->n_experts = (int)all.size();
  return MOE_OK;
}

extern "C" moe_status moe_cache_decode_step(moe_cache* c, moe_cache_step* s, moe_stream_t copy_stream,
                                            moe_stream_t compute_stream) {
  return decode_step(c, s, nullptr, copy_stream, compute_stream, "moe_cache_decode_step");
}

extern "C" moe_status moe_cache_decode_step_hybrid(moe_cache* c, moe_cache_step* s, moe_hybrid* hy,
                                                   moe_stream_t copy_stream, moe_stream_t compute_stream) {
  MOE_CHECK_ARG(hy, "moe_cache_decode_step_hybrid: null policy");
  return decode_step(c, s, hy, copy_stream, compute_stream, "moe_cache_decode_step_hybrid");
}

// ------------------------------------------------------------ layer-ahead prefill

extern "C" moe_status moe_cache_prefetch_layer(moe_cache* c, int layer, const void* const* host_blobs,
                                               void* host_map, void* dev_map, int32_t* trace_slot,
                                               uint8_t* trace_hit, int32_t* trace_evicted, moe_stream_t copy_stream,
                                               moe_stream_t compute_stream) {
  MOE_CHECK_ARG(c, "moe_cache_prefetch_layer: null cache");
  MOE_CHECK_ARG(c->pool, "moe_cache_prefetch_layer: cache has no slot pool");
  MOE_CHECK_ARG(layer >= 0 && layer < c->num_layers, "moe_cache_prefetch_layer: layer %d out of range", layer);
  MOE_CHECK_ARG(host_blobs && host_map && dev_map, "moe_cache_prefetch_layer: null pointer");
  MOE_CHECK_ARG(((uintptr_t)dev_map & 255) == 0, "moe_cache_prefetch_layer: dev_map must be 256-byte aligned");
  const int E = c->num_experts;
  for (int e = 0; e < E; ++e) MOE_CHECK_ARG(host_blobs[e], "moe_cache_prefetch_layer: host blob of expert %d is null", e);
  if (E > c->num_slots)
    return moe::set_error(MOE_ECACHE, "moe_cache_prefetch_layer: %d experts of a layer > %d slots", E, c->num_slots);
  moe_status st = ensure_events(c);
  if (st != MOE_OK) return st;
  hipStream_t ks = reinterpret_cast<hipStream_t>(compute_stream);
  hipStream_t cs = reinterpret_cast<hipStream_t>(copy_stream);
  c->step_ids.resize(E);
  for (int e = 0; e < E; ++e) c->step_ids[e] = e;
  c->step_slot.resize(E);
  c->step_hit.resize(E);
  c->step_ev.resize(E);
  st = cache_lookup(c, layer, c->step_ids.data(), E, c->step_slot.data(), c->step_hit.data(), c->step_ev.data());
  if (st != MOE_OK) return st;
  int nm = 0;
  st = fill_misses(c, layer, E, host_blobs, cs, &nm);
  if (st != MOE_OK) return st;
  st = write_map(c, host_map, dev_map, E, E, ks);
  if (st != MOE_OK) return st;
  if (trace_slot && trace_hit && trace_evicted) copy_trace(c, E, nullptr, trace_slot, trace_hit, trace_evicted);
  return MOE_OK;
}

extern "C" moe_status moe_cache_prefill_step(moe_cache* c, moe_cache_prefill* s, moe_stream_t compute_stream) {
  MOE_CHECK_ARG(c && s, "moe_cache_prefill_step: null pointer");
  const moe_ffn_args& f = s->ffn;
  const int E = f.E, T = f.T;
  MOE_CHECK_ARG(c->pool, "moe_cache_prefill_step: cache has no slot pool");
  MOE_CHECK_ARG(E == c->num_experts, "moe_cache_prefill_step: E=%d but the cache has %d experts per layer", E,
                c->num_experts);
  MOE_CHECK_ARG(s->layer >= 0 && s->layer < c->num_layers, "moe_cache_prefill_step: layer %d out of range", s->layer);
  MOE_CHECK_ARG(T >= 0 && f.k >= 1 && f.k <= E, "moe_cache_prefill_step: bad T=%d k=%d", T, f.k);
  MOE_CHECK_ARG(s->logits && s->topk_ids && s->dev_map && f.out && f.topk_w && f.inv && f.counts && f.offsets &&
                    f.perm,
                "moe_cache_prefill_step: logits, topk_ids, dev_map and ffn.out, topk_w, inv, counts, offsets, perm "
                "are required");
  // every expert of the layer must be cached (its prefetch came first);
  // checked before any state changes
  for (int e = 0; e < E; ++e)
    if (c->key_slot[(size_t)s->layer * E + e] < 0)
      return moe::set_error(MOE_ECACHE, "moe_cache_prefill_step: expert (%d, %d) is not cached: prefetch the layer "
                            "first", s->layer, e);
  moe_status st = ensure_events(c);
  if (st != MOE_OK) return st;
  hipStream_t ks = reinterpret_cast<hipStream_t>(compute_stream);
  c->step_ids.resize(E);
  for (int e = 0; e < E; ++e) c->step_ids[e] = e;
  c->step_slot.resize(E);
  c->step_hit.resize(E);
  c->step_ev.resize(E);
  st = cache_lookup(c, s->layer, c->step_ids.data(), E, c->step_slot.data(), c->step_hit.data(), c->step_ev.data());
  if (st != MOE_OK) return st;
  for (int e = 0; e < E; ++e)
    if ((st = wait_fill(c, c->step_slot[e], ks)) != MOE_OK) return st;
  if (T > 0) {
    if ((long long)T * f.k <= 1024) {
      st = moe_route_permute(s->logits, T, E, f.k, s->renormalize, s->topk_ids, const_cast<float*>(f.topk_w),
                             const_cast<int32_t*>(f.counts), const_cast<int32_t*>(f.offsets),
                             const_cast<int32_t*>(f.perm), const_cast<int32_t*>(f.inv), compute_stream);
    } else {
      st = moe_route(s->logits, T, E, f.k, s->renormalize, s->topk_ids, const_cast<float*>(f.topk_w), compute_stream);
      if (st == MOE_OK)
        st = moe_permute(s->topk_ids, T, f.k, E, const_cast<int32_t*>(f.counts), const_cast<int32_t*>(f.offsets),
                         const_cast<int32_t*>(f.perm), const_cast<int32_t*>(f.inv), compute_stream);
    }
    if (st != MOE_OK) return st;
    moe_ffn_args a = f;
    a.slot_of_expert = static_cast<const int32_t*>(s->dev_map);
    a.slot_pool = c->pool;
    a.slot_stride = c->slot_bytes;
    a.expert_mask = nullptr;
    st = moe_expert_ffn(&a, compute_stream);
    if (st != MOE_OK) return st;
  }
  st = mark_readers(c, c->step_slot.data(), E, ks);
  if (st != MOE_OK) return st;
  if (s->trace_slot && s->trace_hit && s->trace_evicted)
    copy_trace(c, E, nullptr, s->trace_slot, s->trace_hit, s->trace_evicted);
  return MOE_OK;
}

// ------------------------------------------------------------ resize at a safe point

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
  // the copies start after every fill enqueued so far: one wait per copy
  // stream, and one on the last marking of readers, which followed every
  // fill kernel and side-stream hit FFN of the decode steps
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  for (auto& t : c->fill_tail) MOE_HIP(hipStreamWaitEvent(hs, t.second, 0));
  if (c->gen > 0) MOE_HIP(hipStreamWaitEvent(hs, c->ring[(c->gen - 1) % moe_cache::kRing], 0));
  std::vector<int32_t> src(nkeep);
  for (int i = 0; i < nkeep; ++i) src[i] = c->key_slot[keys[ndrop + i]];
  const hipError_t e = moe::launch_move_slots(src.data(), nkeep, 0, c->pool, slot_pool, c->slot_bytes, hs);
  if (e != hipSuccess) return moe::set_error(MOE_EHIP, "moe_cache_resize: copy launch failed: %s", hipGetErrorString(e));
  // a later fill into a kept slot (on any stream) must follow the copies
  MOE_HIP(hipEventRecord(c->resized, hs));
  c->has_resized = 1;
  for (int i = 0; i < ndrop; ++i) {
    c->unlink(keys[i]);
    c->key_slot[keys[i]] = -1;
  }
  c->num_slots = num_slots;
  c->pool = static_cast<uint8_t*>(slot_pool);
  c->slot_key.assign(num_slots, -1);
  // the new slots were written by the copies on `stream` (ordered before later
  // steps, which run on it); their readers start afresh
  c->fill_pending.assign(num_slots, 0);
  c->reader_gen.assign(num_slots, -1);
  for (int i = 0; i < nkeep; ++i) {
    c->key_slot[keys[ndrop + i]] = i;
    c->slot_key[i] = keys[ndrop + i];
  }
  c->free_slots.clear();
  for (int s = nkeep; s < num_slots; ++s) c->free_slots.insert(s);
  return ensure_events(c);
}
