// Scenarios for the CPU test of the expert cache: cache.cpp and host.cpp
// linked against the recording HIP stand-in (hip_stub.cpp); built with g++
// and the address and undefined-behaviour sanitizers.
//
// usage:
//   cache_harness decode L E k T C steps seed [step:slots ...]   decode stream (optional resizes)
//   cache_harness prefill L E C passes seed                      layer-ahead prefill passes
//   cache_harness fault KIND NTH L E k T C steps seed            decode stream, the NTH call of KIND fails
//                                                                (0 copy, 1 event create, 2 event record, 3 stream wait,
//                                                                4 fill-kernel launch)
// HARNESS_COPY_ENGINE=1 in the environment: decode steps fill through the
// copy engine (moe_cache_use_copy_engine), else through the fill kernel.
//   cache_harness hybrid RATIO L E k T C steps seed              decode stream, hybrid miss policy
// stdout, one line per call:
//   D <layer> <status> e:h:s:v ...   a decode step's records
//   P <layer> <status> h:s:v ...     a prefetch's lookups of experts 0..E-1
//   S <layer> <status> h:s:v ...     a prefill step's lookups
//   R <slots> <status>               a resize
//   END hazards <n> bad <n>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <memory>
#include <vector>

#include "../../fp4_expert_ffn_amd/csrc/host_common.h"

extern "C" {
hipStream_t stub_stream_create();
void stub_region(const void* p, size_t bytes, int device);
void stub_pool(const void* p, size_t slot_bytes, int n);
void stub_layer(int l);
void stub_counts(const int32_t* c, int E);
void stub_fail(int kind, int nth);
long long stub_hazards();
long long stub_bad();
}

namespace {
uint64_t g_rng = 88172645463325252ull;
uint32_t rnd() {  // xorshift64
  g_rng ^= g_rng << 13;
  g_rng ^= g_rng >> 7;
  g_rng ^= g_rng << 17;
  return (uint32_t)(g_rng >> 11);
}
// k distinct experts, popularity falling with the id's rank (skewed draws)
void draw(int E, int k, std::vector<int>& out) {
  out.clear();
  while ((int)out.size() < k) {
    const uint32_t r = rnd() % (uint32_t)E, r2 = rnd() % (uint32_t)E;
    const int e = (int)std::min(r, r2);  // smaller ids more likely
    bool dup = false;
    for (int x : out) dup |= x == e;
    if (!dup) out.push_back(e);
  }
}
std::vector<std::unique_ptr<std::vector<uint8_t>>> g_buffers;  // every buffer of the run
std::vector<uint8_t>* keep(size_t n) {
  g_buffers.emplace_back(new std::vector<uint8_t>(n + 256));
  return g_buffers.back().get();
}
// 256-aligned buffer registered with the stand-in
void* buffer(size_t n, int device) {
  std::vector<uint8_t>* v = keep(n);
  uintptr_t p = ((uintptr_t)v->data() + 255) & ~(uintptr_t)255;
  stub_region((void*)p, n, device);
  return (void*)p;
}

constexpr int kH = 128, kI = 128;  // blob shape: valid MXFP4 blobs, so the host FFN can run them
constexpr int kTagOffset = 200;

struct World {
  int L, E, k, T, C;
  size_t slot = (moe_blob_bytes(MOE_FMT_MXFP4, kH, kI) + 255) / 256 * 256;
  std::vector<void*> blob_ptr;  // L * E host blobs, tagged (layer, expert)
  void* pool;
  int32_t *counts, *offsets, *perm, *inv, *ids, *host_counts, *host_perm, *host_offsets;
  uint16_t* host_x;
  float* host_y;
  float *topk_w, *y, *logits;
  uint16_t *out, *x;
  std::vector<void*> host_map, dev_map;  // per layer
  hipStream_t ks, cs;
  moe_cache* c;

  World(int L_, int E_, int k_, int T_, int C_) : L(L_), E(E_), k(k_), T(T_), C(C_) {
    uint8_t* bank = (uint8_t*)buffer(slot * L * E, 0);
    for (int l = 0; l < L; ++l)
      for (int e = 0; e < E; ++e) {
        uint8_t* b = bank + slot * ((size_t)l * E + e);
        memset(b, (l * 31 + e) & 127, slot);  // codes; scales below 2^0
        moe::BlobHeader hdr{};
        moe::BlobLayout Ly;
        moe::layout_of(MOE_FMT_MXFP4, kH, kI, &Ly);
        hdr.magic = moe::kBlobMagic;
        hdr.fmt = MOE_FMT_MXFP4; hdr.H = kH; hdr.I = kI;
        hdr.g[0] = hdr.g[1] = hdr.g[2] = 1.f;
        hdr.off_w13 = Ly.off_w13; hdr.off_s13 = Ly.off_s13; hdr.off_w2 = Ly.off_w2; hdr.off_s2 = Ly.off_s2;
        hdr.total = Ly.total;
        memcpy(b, &hdr, sizeof hdr);
        const int32_t tag[2] = {l, e};
        memcpy(b + kTagOffset, tag, sizeof tag);
        memcpy(b + Ly.off_w2 + 16, tag, sizeof tag);  // a second tag among the down weights
        blob_ptr.push_back(b);
      }
    pool = buffer(slot * C, 1);
    stub_pool(pool, slot, C);
    counts = (int32_t*)buffer(4 * E, 1);
    offsets = (int32_t*)buffer(4 * (E + 1), 1);
    perm = (int32_t*)buffer(4 * T * k, 1);
    inv = (int32_t*)buffer(4 * T * k, 1);
    ids = (int32_t*)buffer(4 * T * k, 1);
    host_counts = (int32_t*)buffer(4 * E, 2);
    topk_w = (float*)buffer(4 * T * k, 1);
    y = (float*)buffer(4 * T * k * kH, 1);
    logits = (float*)buffer(4 * T * E, 1);
    out = (uint16_t*)buffer(2 * T * kH, 1);
    x = (uint16_t*)buffer(2 * T * kH, 1);
    host_x = (uint16_t*)buffer(2 * T * kH, 2);
    host_perm = (int32_t*)buffer(4 * T * k, 2);
    host_offsets = (int32_t*)buffer(4 * (E + 1), 2);
    host_y = (float*)buffer(4 * T * k * kH, 2);
    for (int l = 0; l < L; ++l) {
      host_map.push_back(buffer(moe_cache_map_bytes(E), 2));
      dev_map.push_back(buffer(moe_cache_map_bytes(E), 1));
    }
    ks = stub_stream_create();
    cs = stub_stream_create();
    c = moe_cache_create(C, slot, pool, L, E);
  }
  moe_ffn_args ffn() const {
    moe_ffn_args a{};
    a.T = T; a.k = k; a.E = E; a.H = kH; a.I = kI; a.wfmt = MOE_FMT_MXFP4; a.amode = MOE_ACT_BF16;
    a.x = x; a.counts = counts; a.offsets = offsets; a.perm = perm; a.inv = inv; a.topk_w = topk_w;
    a.y = y; a.out = out;
    return a;
  }
};

void print_recs(char tag, int layer, int st, int n, const int32_t* e, const uint8_t* h, const int32_t* s,
                const int32_t* v) {
  printf("%c %d %d", tag, layer, st);
  for (int i = 0; i < n; ++i) {
    if (e) printf(" %d:%d:%d:%d", e[i], h[i], s[i], v[i]);
    else printf(" %d:%d:%d", h[i], s[i], v[i]);
  }
  printf("\n");
}

int decode(int argc, char** argv, int fail_kind, int fail_nth, float ratio = -1.f) {
  const int L = atoi(argv[0]), E = atoi(argv[1]), k = atoi(argv[2]), T = atoi(argv[3]), C = atoi(argv[4]);
  const int steps = atoi(argv[5]);
  g_rng ^= (uint64_t)atoll(argv[6]) * 0x9E3779B97F4A7C15ull;
  std::map<int, int> resize_at;
  for (int i = 7; i < argc; ++i) {
    int st = 0, n = 0;
    if (sscanf(argv[i], "%d:%d", &st, &n) == 2) resize_at[st] = n;
  }
  World w(L, E, k, T, C);
  const char* ce = getenv("HARNESS_COPY_ENGINE");
  if (ce && atoi(ce)) moe_cache_use_copy_engine(w.c, 1);
  if (fail_kind >= 0) stub_fail(fail_kind, fail_nth);
  moe_hybrid hy{ratio, 2, w.host_x, w.host_perm, w.host_offsets, w.host_y, 0};
  std::vector<std::vector<int>> prev(L);
  std::vector<int> sel;
  std::vector<int32_t> te(E), ts(E), tv(E), cnt(E);
  std::vector<uint8_t> th(E);
  for (int step = 0; step < steps; ++step) {
    auto r = resize_at.find(step);
    if (r != resize_at.end()) {
      void* np = buffer(w.slot * r->second, 1);
      const moe_status st = moe_cache_resize(w.c, r->second, np, reinterpret_cast<moe_stream_t>(w.ks));
      if (st == MOE_OK) stub_pool(np, w.slot, r->second);
      printf("R %d %d\n", r->second, (int)st);
    }
    const int l = step % L;
    std::fill(cnt.begin(), cnt.end(), 0);
    for (int t = 0; t < T; ++t) {
      if (!prev[l].empty() && rnd() % 10 < 6) sel = prev[l];
      else draw(E, k, sel);
      prev[l] = sel;
      for (int e : sel) ++cnt[e];
    }
    stub_counts(cnt.data(), E);
    stub_layer(l);
    moe_cache_step s{};
    s.layer = l;
    s.logits = w.logits;
    s.renormalize = 1;
    s.topk_ids = w.ids;
    s.host_counts = w.host_counts;
    s.host_map = w.host_map[0];
    s.dev_map = w.dev_map[0];
    s.host_blobs = (const void* const*)&w.blob_ptr[(size_t)l * E];
    s.ffn = w.ffn();
    s.trace_expert = te.data(); s.trace_slot = ts.data(); s.trace_hit = th.data(); s.trace_evicted = tv.data();
    const moe_status st =
        ratio < 0.f ? moe_cache_decode_step(w.c, &s, reinterpret_cast<moe_stream_t>(w.cs),
                                            reinterpret_cast<moe_stream_t>(w.ks))
                    : moe_cache_decode_step_hybrid(w.c, &s, &hy, reinterpret_cast<moe_stream_t>(w.cs),
                                                   reinterpret_cast<moe_stream_t>(w.ks));
    print_recs('D', l, (int)st, st == MOE_OK ? s.n_experts : 0, te.data(), th.data(), ts.data(), tv.data());
  }
  moe_cache_destroy(w.c);
  printf("END hazards %lld bad %lld\n", stub_hazards(), stub_bad());
  return 0;
}

int prefill(char** argv) {
  const int L = atoi(argv[0]), E = atoi(argv[1]), C = atoi(argv[2]), passes = atoi(argv[3]);
  g_rng ^= (uint64_t)atoll(argv[4]) * 0x9E3779B97F4A7C15ull;
  const int k = 2, T = 64;
  World w(L, E, k, T, C);
  std::vector<int32_t> ts(E), tv(E), cnt(E);
  std::vector<uint8_t> th(E);
  auto prefetch = [&](int l) {
    const moe_status st = moe_cache_prefetch_layer(w.c, l, (const void* const*)&w.blob_ptr[(size_t)l * E],
                                                   w.host_map[l], w.dev_map[l], ts.data(), th.data(), tv.data(),
                                                   reinterpret_cast<moe_stream_t>(w.cs),
                                                   reinterpret_cast<moe_stream_t>(w.ks));
    print_recs('P', l, (int)st, st == MOE_OK ? E : 0, nullptr, th.data(), ts.data(), tv.data());
  };
  for (int p = 0; p < passes; ++p) {
    prefetch(0);
    for (int l = 0; l < L; ++l) {
      for (int e = 0; e < E; ++e) cnt[e] = (int)(rnd() % 5);  // some experts get no rows
      stub_counts(cnt.data(), E);
      stub_layer(l);
      moe_cache_prefill s{};
      s.layer = l;
      s.logits = w.logits;
      s.renormalize = 1;
      s.topk_ids = w.ids;
      s.dev_map = w.dev_map[l];
      s.ffn = w.ffn();
      s.ffn.y = nullptr;
      s.trace_slot = ts.data(); s.trace_hit = th.data(); s.trace_evicted = tv.data();
      const moe_status st = moe_cache_prefill_step(w.c, &s, reinterpret_cast<moe_stream_t>(w.ks));
      print_recs('S', l, (int)st, st == MOE_OK ? E : 0, nullptr, th.data(), ts.data(), tv.data());
      if (l + 1 < L) prefetch(l + 1);
    }
  }
  // a step of a layer that is not cached (the last prefetch evicted layer
  // L - 3 with 2E slots): MOE_ECACHE, cache unchanged
  {
    const int l = L - 3;
    stub_layer(l);
    moe_cache_prefill s{};
    s.layer = l; s.logits = w.logits; s.topk_ids = w.ids; s.dev_map = w.dev_map[l]; s.ffn = w.ffn();
    s.trace_slot = ts.data(); s.trace_hit = th.data(); s.trace_evicted = tv.data();
    long long h0, m0, b0, h1, m1, b1;
    moe_cache_stats(w.c, &h0, &m0, &b0);
    const moe_status st = moe_cache_prefill_step(w.c, &s, reinterpret_cast<moe_stream_t>(w.ks));
    moe_cache_stats(w.c, &h1, &m1, &b1);
    printf("U %d %d %d\n", l, (int)st, (int)(h0 == h1 && m0 == m1 && b0 == b1));
  }
  moe_cache_destroy(w.c);
  printf("END hazards %lld bad %lld\n", stub_hazards(), stub_bad());
  return 0;
}
}  // namespace

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  if (!strcmp(argv[1], "decode") && argc >= 9) return decode(argc - 2, argv + 2, -1, -1);
  if (!strcmp(argv[1], "prefill") && argc == 7 && atoi(argv[2]) >= 3) return prefill(argv + 2);
  if (!strcmp(argv[1], "fault") && argc == 11) return decode(7, argv + 4, atoi(argv[2]), atoi(argv[3]));
  if (!strcmp(argv[1], "hybrid") && argc == 10) return decode(7, argv + 3, -1, -1, (float)atof(argv[2]));
  return 2;
}
