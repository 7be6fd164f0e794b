// A recording stand-in, for CPU tests only, of the HIP runtime calls made by
// the expert cache's host code (cache.cpp) and of the library calls it makes
// (routing, expert FFN, combine, slot moves).  Never part of the library.
//
// "Device memory" is host memory that the test registers.  Every operation
// executes at once, in host order, and is also placed on a happens-before
// relation: each stream carries a vector clock, advanced by its operations,
// recorded into events and joined at stream waits (and into the host's clock
// at synchronisations).  Against it every write of a cache slot (a fill, a
// resize move) and every read of one (the blobs an FFN call uses) is checked:
//   WAR  - a write must follow every earlier read of its slot;
//   WAW  - and the slot's previous write;
//   RAW  - a read must follow the last write of its slot;
//   map  - a host buffer is re-sent only after the host saw its last copy finish.
// Copies must stay inside registered regions, and the FFN stand-in checks
// that each slot it reads holds the blob of the (layer, expert) it wants
// (the test writes a marker into every blob).  Failures can be injected
// into the n-th call of a kind.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <memory>
#include <vector>

#include "../../fp4_expert_ffn_amd/csrc/host_common.h"

struct ihipStream_t {
  int id;
};
struct ihipEvent_t {
  std::vector<int> vc;
};

namespace {
constexpr int kMaxStreams = 16;
constexpr int kTagOffset = 200;  // (layer, expert) tag of a test blob, inside its header padding
typedef std::vector<int> VC;

struct Op {
  int sid = -1;
  VC vc;
};
bool hb(const Op& a, const VC& b) { return a.sid < 0 || a.vc[a.sid] <= b[a.sid]; }

struct SlotState {
  Op last_write;
  std::vector<Op> reads;  // since the last write
};

struct Region {
  uintptr_t base;
  size_t bytes;
  int device;  // 0: host memory the host never rewrites, 1: device memory, 2: host memory the host rewrites
};

VC g_vc[kMaxStreams];
VC g_host(kMaxStreams, 0);
int g_nstreams = 1;
std::vector<Region> g_regions;
std::map<uintptr_t, SlotState> g_slots;  // by slot start address
std::map<uintptr_t, Op> g_host_src;      // last H2D copy from each host address
uintptr_t g_pool = 0;
size_t g_slot_bytes = 0;
int g_num_slots = 0;
int g_layer = 0;
std::vector<int32_t> g_next_counts;
long long g_hazards = 0, g_bad = 0, g_ops = 0;
int g_fail_kind = -1, g_fail_at = -1, g_calls[8];

void hazard(const char* what, long long a, long long b) {
  if (g_hazards++ < 10) fprintf(stderr, "hazard: %s (%lld, %lld)\n", what, a, b);
}
void bad(const char* what, long long a, long long b) {
  if (g_bad++ < 10) fprintf(stderr, "bad: %s (%lld, %lld)\n", what, a, b);
}
int sid_of(hipStream_t s) { return s ? s->id : 0; }
// An operation enqueued after the host has seen other work finish (a
// synchronisation, or the count flag the stream publishes) runs after that
// work: the stream's clock joins the host's.
Op tick(hipStream_t s) {
  const int id = sid_of(s);
  if (g_vc[id].empty()) g_vc[id].assign(kMaxStreams, 0);
  for (int i = 0; i < kMaxStreams; ++i) g_vc[id][i] = std::max(g_vc[id][i], g_host[i]);
  ++g_vc[id][id];
  ++g_ops;
  Op o;
  o.sid = id;
  o.vc = g_vc[id];
  return o;
}
bool inject(int kind) { return ++g_calls[kind] == g_fail_at && kind == g_fail_kind; }
const Region* region_of(uintptr_t p, size_t n) {
  for (const Region& r : g_regions)
    if (p >= r.base && p + n <= r.base + r.bytes) return &r;
  return nullptr;
}
void slot_write(uintptr_t addr, const Op& w) {
  SlotState& st = g_slots[addr];
  for (const Op& r : st.reads)
    if (!hb(r, w.vc)) hazard("WAR: a slot write does not follow an earlier read", (long long)addr, r.sid);
  if (!hb(st.last_write, w.vc)) hazard("WAW: a slot write does not follow the previous one", (long long)addr, 0);
  st.reads.clear();
  st.last_write = w;
}
void slot_read(uintptr_t addr, const Op& r) {
  SlotState& st = g_slots[addr];
  if (!hb(st.last_write, r.vc)) hazard("RAW: a slot read does not follow its last write", (long long)addr, r.sid);
  st.reads.push_back(r);
}
// slot start address of a pool byte address, or 0 when outside the current pool
uintptr_t slot_addr(uintptr_t p) {
  if (!g_pool || p < g_pool || p >= g_pool + (uintptr_t)g_num_slots * g_slot_bytes) return 0;
  return g_pool + (p - g_pool) / g_slot_bytes * g_slot_bytes;
}
}  // namespace

// ------------------------------------------------------------ test controls
extern "C" {
hipStream_t stub_stream_create() {
  static std::vector<std::unique_ptr<ihipStream_t>> streams;
  if (g_nstreams >= kMaxStreams) {
    fprintf(stderr, "stub: more than %d streams\n", kMaxStreams);
    abort();
  }
  streams.emplace_back(new ihipStream_t{g_nstreams++});
  ihipStream_t* s = streams.back().get();
  g_vc[s->id].assign(kMaxStreams, 0);
  return s;
}
void stub_region(const void* p, size_t bytes, int device) { g_regions.push_back({(uintptr_t)p, bytes, device}); }
void stub_pool(const void* p, size_t slot_bytes, int n) {
  g_pool = (uintptr_t)p;
  g_slot_bytes = slot_bytes;
  g_num_slots = n;
}
void stub_layer(int l) { g_layer = l; }
void stub_counts(const int32_t* c, int E) { g_next_counts.assign(c, c + E); }
void stub_fail(int kind, int nth) {
  g_fail_kind = kind;
  g_fail_at = nth;
  memset(g_calls, 0, sizeof g_calls);
}
long long stub_hazards() { return g_hazards; }
long long stub_bad() { return g_bad; }
}

// ------------------------------------------------------------ HIP runtime
extern "C" {
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "injected failure"; }

hipError_t hipEventCreate(hipEvent_t* e) {
  if (inject(1)) return hipErrorOutOfMemory;
  *e = new ihipEvent_t{VC(kMaxStreams, 0)};
  return hipSuccess;
}
hipError_t hipEventElapsedTime(float* ms, hipEvent_t, hipEvent_t) {
  *ms = 1.0f;
  return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
  if (inject(1)) return hipErrorOutOfMemory;
  *e = new ihipEvent_t{VC(kMaxStreams, 0)};
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t e) {
  delete e;
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t s) {
  if (inject(2)) return hipErrorInvalidValue;
  const int id = sid_of(s);
  if (g_vc[id].empty()) g_vc[id].assign(kMaxStreams, 0);
  e->vc = g_vc[id];
  return hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t e) {
  for (int i = 0; i < kMaxStreams; ++i) g_host[i] = std::max(g_host[i], e->vc[i]);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t s) {
  const int id = sid_of(s);
  if (!g_vc[id].empty())
    for (int i = 0; i < kMaxStreams; ++i) g_host[i] = std::max(g_host[i], g_vc[id][i]);
  return hipSuccess;
}
hipError_t hipStreamWaitEvent(hipStream_t s, hipEvent_t e, unsigned int) {
  if (inject(3)) return hipErrorInvalidValue;
  const int id = sid_of(s);
  if (g_vc[id].empty()) g_vc[id].assign(kMaxStreams, 0);
  for (int i = 0; i < kMaxStreams; ++i) g_vc[id][i] = std::max(g_vc[id][i], e->vc[i]);
  return hipSuccess;
}
hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned int) {
  *s = stub_stream_create();
  return hipSuccess;
}
hipError_t hipStreamDestroy(hipStream_t) { return hipSuccess; }
// device memory the library allocates itself (registered as device memory)
hipError_t hipMalloc(void** p, size_t n) {
  static std::vector<std::unique_ptr<std::vector<uint8_t>>> bufs;
  bufs.emplace_back(new std::vector<uint8_t>(n + 256));
  *p = (void*)(((uintptr_t)bufs.back()->data() + 255) & ~(uintptr_t)255);
  g_regions.push_back({(uintptr_t)*p, n, 1});
  return hipSuccess;
}
hipError_t hipFree(void*) { return hipSuccess; }
hipError_t hipGetLastError() { return hipSuccess; }
hipError_t hipStreamQuery(hipStream_t) { return hipSuccess; }
hipError_t hipHostMalloc(void** p, size_t n, unsigned int) {
  static std::vector<std::unique_ptr<std::vector<uint8_t>>> bufs;
  bufs.emplace_back(new std::vector<uint8_t>(n + 256));
  *p = (void*)(((uintptr_t)bufs.back()->data() + 255) & ~(uintptr_t)255);
  g_regions.push_back({(uintptr_t)*p, n, 2});
  return hipSuccess;
}
hipError_t hipHostFree(void*) { return hipSuccess; }
// host memory the test registered (or hipHostMalloc gave) is "mapped": same address
hipError_t hipHostGetDevicePointer(void** d, void* h, unsigned int) {
  const Region* r = region_of((uintptr_t)h, 1);
  if (!r || r->device == 1) return hipErrorInvalidValue;
  *d = h;
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind kind, hipStream_t s) {
  if (inject(0)) return hipErrorOutOfMemory;
  const Region* rd = region_of((uintptr_t)dst, n);
  const Region* rs = region_of((uintptr_t)src, n);
  if (!rd || !rs) {
    bad("copy outside the registered memory", (long long)(uintptr_t)dst, (long long)n);
    return hipSuccess;
  }
  if (kind == hipMemcpyHostToDevice && (rd->device != 1 || rs->device == 1)) bad("H2D copy direction", 0, 0);
  if (kind == hipMemcpyDeviceToHost && (rd->device == 1 || rs->device != 1)) bad("D2H copy direction", 0, 0);
  const Op o = tick(s);
  if (kind == hipMemcpyHostToDevice && rs->device == 2) {
    auto it = g_host_src.find((uintptr_t)src);
    // the host rewrote this buffer since its last copy: it must have seen that copy finish
    if (it != g_host_src.end() && !hb(it->second, g_host)) hazard("map: host buffer re-sent before its last copy", 0, 0);
    g_host_src[(uintptr_t)src] = o;
  }
  if (const uintptr_t a = slot_addr((uintptr_t)dst)) {
    if ((uintptr_t)dst != a || n != g_slot_bytes) bad("fill not covering exactly one slot", (long long)n, 0);
    slot_write(a, o);
  }
  memcpy(dst, src, n);
  return hipSuccess;
}
}

// ------------------------------------------------------------ library stand-ins
namespace {
void route_counts(int E, int32_t* counts, int32_t* offsets, int32_t* perm) {
  int run = 0;
  for (int e = 0; e < E; ++e) {
    counts[e] = e < (int)g_next_counts.size() ? g_next_counts[e] : 0;
    offsets[e] = run;
    run += counts[e];
  }
  offsets[E] = run;
  if (perm)
    for (int p = 0; p < run; ++p) perm[p] = p;  // flat index p: token p / k
}
}  // namespace

extern "C" moe_status moe_route_permute(const float*, int, int E, int, int, int32_t*, float*, int32_t* counts,
                                        int32_t* offsets, int32_t* perm, int32_t*, moe_stream_t stream) {
  tick(reinterpret_cast<hipStream_t>(stream));
  route_counts(E, counts, offsets, perm);
  return MOE_OK;
}
extern "C" moe_status moe_route(const float*, int, int, int, int, int32_t*, float*, moe_stream_t stream) {
  tick(reinterpret_cast<hipStream_t>(stream));
  return MOE_OK;
}
extern "C" moe_status moe_permute(const int32_t*, int, int, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                                  int32_t*, moe_stream_t stream) {
  tick(reinterpret_cast<hipStream_t>(stream));
  route_counts(E, counts, offsets, perm);
  return MOE_OK;
}
extern "C" moe_status moe_combine(const float*, const int32_t*, const float*, const float*, int, int, int, uint16_t*,
                                  moe_stream_t stream) {
  tick(reinterpret_cast<hipStream_t>(stream));
  return MOE_OK;
}
// Reads the blob of every expert with rows (and enabled by the mask): its
// slot must be in the pool, ordered after its fill, and hold the blob of
// (current layer, expert), both in its header and among its down weights.
namespace {
void ffn_reads(const moe_ffn_args* a, const Op& o) {
  moe::BlobLayout Ly;
  if (!moe::layout_of(a->wfmt, a->H, a->I, &Ly)) bad("FFN blob layout", a->H, a->I);
  for (int e = 0; e < a->E; ++e) {
    if (a->counts[e] <= 0 || (a->expert_mask && !a->expert_mask[e])) continue;
    const int slot = a->slot_of_expert[e];
    const uintptr_t addr = (uintptr_t)a->slot_pool + (uintptr_t)slot * a->slot_stride;
    if (slot < 0 || (uintptr_t)a->slot_pool != g_pool || slot >= g_num_slots || a->slot_stride != g_slot_bytes) {
      bad("FFN slot outside the pool", slot, e);
      continue;
    }
    slot_read(addr, o);
    int32_t tag[2], tag2[2];  // in the blob header's padding, and among the down weights
    memcpy(tag, reinterpret_cast<const void*>(addr + kTagOffset), sizeof tag);
    memcpy(tag2, reinterpret_cast<const void*>(addr + Ly.off_w2 + 16), sizeof tag2);
    if (tag[0] != g_layer || tag[1] != e) bad("slot holds another blob", tag[0] * 100000LL + tag[1], g_layer * 100000LL + e);
    if (tag2[0] != g_layer || tag2[1] != e) bad("slot holds another blob's down weights", tag2[0], tag2[1]);
  }
}
}  // namespace

extern "C" moe_status moe_expert_ffn(const moe_ffn_args* a, moe_stream_t stream) {
  const Op o = tick(reinterpret_cast<hipStream_t>(stream));
  ffn_reads(a, o);
  return MOE_OK;
}

namespace moe {
// copies of blob ranges into slots by a kernel (the fill kernel, or the copy
// workgroups of a gate/up launch)
static void copy_parts(const FillList& f, void* pool, size_t slot_bytes, const Op& o) {
  if (f.n < 1 || f.n > kFillMax) bad("fill list size", f.n, 0);
  if ((uint64_t)f.off16 + f.len16 > slot_bytes / 16) bad("fill range outside the slot", f.off16, f.len16);
  for (int i = 0; i < f.n; ++i) {
    const uintptr_t to = (uintptr_t)pool + (uintptr_t)f.slot[i] * slot_bytes;
    const Region* rs = region_of((uintptr_t)f.src[i], slot_bytes);
    if (!rs || rs->device == 1 || ((uintptr_t)f.src[i] & 15)) {
      bad("fill source not in host memory", f.slot[i], 0);
      continue;
    }
    if (slot_addr(to) != to || slot_bytes != g_slot_bytes || (uintptr_t)pool != g_pool) {
      bad("fill destination not a slot of the pool", f.slot[i], 0);
      continue;
    }
    slot_write(to, o);
    memcpy(reinterpret_cast<void*>(to + 16 * (size_t)f.off16), f.src[i] + 16 * (size_t)f.off16, 16 * (size_t)f.len16);
  }
}
// the count handoff: the stream writes the counts to host memory and the flag,
// which the host has then observed (its clock joins the stream's)
hipError_t launch_publish_counts(const int32_t* counts, int E, int32_t* host_counts, uint32_t* flag, uint32_t seq,
                                 hipStream_t s) {
  const Op o = tick(s);
  memcpy(host_counts, counts, sizeof(int32_t) * (size_t)E);
  __atomic_store_n(flag, seq, __ATOMIC_RELEASE);
  for (int i = 0; i < kMaxStreams; ++i) g_host[i] = std::max(g_host[i], o.vc[i]);
  return hipSuccess;
}
// routing with the handoff folded in: one stream operation that writes the
// routing outputs, then the host copy of the counts and the flag
moe_status route_permute_publish(const float*, int, int E, int, int, int32_t*, float*, int32_t* counts,
                                 int32_t* offsets, int32_t* perm, int32_t*, int32_t* host_counts, uint32_t* flag,
                                 uint32_t seq, hipStream_t s) {
  const Op o = tick(s);
  route_counts(E, counts, offsets, perm);
  memcpy(host_counts, counts, sizeof(int32_t) * (size_t)E);
  __atomic_store_n(flag, seq, __ATOMIC_RELEASE);
  for (int i = 0; i < kMaxStreams; ++i) g_host[i] = std::max(g_host[i], o.vc[i]);
  return MOE_OK;
}
hipError_t launch_write_map(const StepMap& m, int E, void* dev_map, hipStream_t s) {
  tick(s);
  if (!region_of((uintptr_t)dev_map, 6 * (size_t)E)) bad("slot map outside the registered memory", E, 0);
  int32_t* slot = static_cast<int32_t*>(dev_map);
  uint8_t* hit = static_cast<uint8_t*>(dev_map) + 4 * E;
  memset(dev_map, 0, 6 * (size_t)E);
  for (int i = 0; i < m.n; ++i) {
    slot[m.expert[i]] = m.slot[i];
    (m.hit[i] ? hit : hit + E)[m.expert[i]] = 1;
  }
  return hipSuccess;
}
// the fill kernel: writes the map like launch_write_map, then copies each
// listed host blob (host memory, slot_bytes long) into its slot (kind 4 fails)
hipError_t launch_fill_slots(const FillList& f, const StepMap& m, int E, void* dev_map, void* pool, size_t slot_bytes,
                             hipStream_t s) {
  if (inject(4)) return hipErrorLaunchFailure;
  const Op o = tick(s);
  if (E > 0) {  // E == 0: no map (a plain copy)
    if (!region_of((uintptr_t)dev_map, 6 * (size_t)E)) bad("slot map outside the registered memory", E, 0);
    int32_t* slot = static_cast<int32_t*>(dev_map);
    uint8_t* hit = static_cast<uint8_t*>(dev_map) + 4 * E;
    memset(dev_map, 0, 6 * (size_t)E);
    for (int i = 0; i < m.n; ++i) {
      slot[m.expert[i]] = m.slot[i];
      (m.hit[i] ? hit : hit + E)[m.expert[i]] = 1;
    }
  }
  copy_parts(f, pool, slot_bytes, o);
  return hipSuccess;
}
// the FFN whose gate/up launch copies the rest of the blobs: one operation
// that writes the listed ranges and reads the masked experts' blobs (which
// must hold both parts by then)
moe_status expert_ffn_fill(const moe_ffn_args* a, const FillList& f, void* pool, size_t slot_bytes, hipStream_t s) {
  if (inject(4)) return MOE_EHIP;
  const Op o = tick(s);
  copy_parts(f, pool, slot_bytes, o);
  ffn_reads(a, o);
  return MOE_OK;
}
bool ffn_takes_gemv(const moe_ffn_args* a) { return (long long)a->T * a->k < 512 && a->amode != MOE_ACT_MXFP4; }
hipError_t launch_move_slots(const int32_t* src_slots, int n, int dst0, const void* src_pool, void* dst_pool,
                             size_t slot_bytes, hipStream_t s) {
  const Op o = tick(s);
  for (int i = 0; i < n; ++i) {
    const uintptr_t from = (uintptr_t)src_pool + (uintptr_t)src_slots[i] * slot_bytes;
    const uintptr_t to = (uintptr_t)dst_pool + (uintptr_t)(dst0 + i) * slot_bytes;
    if (!region_of(from, slot_bytes) || !region_of(to, slot_bytes)) {
      bad("move outside the registered memory", src_slots[i], dst0 + i);
      continue;
    }
    slot_read(from, o);
    slot_write(to, o);
    memcpy(reinterpret_cast<void*>(to), reinterpret_cast<const void*>(from), slot_bytes);
  }
  return hipSuccess;
}
}  // namespace moe
