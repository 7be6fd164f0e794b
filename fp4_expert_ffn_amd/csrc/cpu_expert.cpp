// The host side of the hybrid miss policy: a CPU expert FFN over a packed
// blob, a persistent thread pool for it, and the one-time bandwidth
// calibration that sets the share of misses copied over PCIe.
//
// Method: on a cache miss in decode the runtime either copies the expert
// over PCIe or runs it on the CPU, by the host-memory and PCIe bandwidths
// it measured on the machine (page "FreeToken量子化：MoE推論のセットアップ
// ガイド", decode paragraph and the paragraph on the bandwidth-adaptive
// policy; bhrtaym-blog page, section "MoEバックエンドは4種類から選べる",
// backend table rows "cpu" and "hybrid" and the note on the one-time
// bandwidth calibration).
//
// The host kernel reads the same prepacked blob the GPU slots hold: tiles of
// 16 rows x KT values, lane l holding row l % 16 and K-chunk l / 16; it
// decodes each lane chunk to fp32 and takes its dot product with the token
// rows (fp32 accumulation), so every tile is read once per call whatever the
// token count.  Work is split by row groups across the pool's threads.
#include <string.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "host_common.h"

namespace moe {
hipError_t launch_fill_slots(const FillList& f, const StepMap& m, int E, void* dev_map, void* pool, size_t slot_bytes,
                             hipStream_t s);
}

namespace {

// ---------------------------------------------------------------- thread pool
// Workers wait for a generation change, run fn(worker) and count down.
class Pool {
 public:
  void run(int nthreads, const std::function<void(int, int)>& fn) {
    std::unique_lock<std::mutex> lock(call_mu_);  // one call at a time
    ensure(nthreads - 1);
    {
      std::lock_guard<std::mutex> l(mu_);
      fn_ = &fn;
      active_ = nthreads - 1;
      pending_ = nthreads - 1;
      ++gen_;
    }
    cv_.notify_all();
    fn(0, nthreads);
    std::unique_lock<std::mutex> l(mu_);
    done_.wait(l, [&] { return pending_ == 0; });
    fn_ = nullptr;
  }
  ~Pool() {
    {
      std::lock_guard<std::mutex> l(mu_);
      stop_ = true;
      ++gen_;
    }
    cv_.notify_all();
    for (auto& t : threads_) t.join();
  }

 private:
  void ensure(int n) {
    while ((int)threads_.size() < n) {
      const int id = (int)threads_.size() + 1;
      threads_.emplace_back([this, id] { loop(id); });
    }
  }
  void loop(int id) {
    long long seen = 0;
    for (;;) {
      const std::function<void(int, int)>* fn;
      int n;
      {
        std::unique_lock<std::mutex> l(mu_);
        cv_.wait(l, [&] { return stop_ || gen_ != seen; });
        if (stop_) return;
        seen = gen_;
        if (id > active_) continue;
        fn = fn_;
        n = active_ + 1;
      }
      (*fn)(id, n);
      std::lock_guard<std::mutex> l(mu_);
      if (--pending_ == 0) done_.notify_one();
    }
  }
  std::mutex call_mu_, mu_;
  std::condition_variable cv_, done_;
  std::vector<std::thread> threads_;
  const std::function<void(int, int)>* fn_ = nullptr;
  int active_ = 0, pending_ = 0;
  long long gen_ = 0;
  bool stop_ = false;
};

Pool& pool() {
  static Pool p;
  return p;
}

// ---------------------------------------------------------------- decoding
const float kE2M1[16] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f, -0.f, -0.5f, -1.f, -1.5f, -2.f, -3.f, -4.f, -6.f};

float e4m3(uint8_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  float v = e == 0 ? std::ldexp((float)m, -9) : std::ldexp(1.f + m / 8.f, e - 7);
  if (e == 15 && m == 7) v = NAN;
  return (c & 0x80) ? -v : v;
}
float e8m0(uint8_t c) { return c == 255 ? NAN : std::ldexp(1.f, (int)c - 127); }
float bf16f(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// Values of lane chunk `lane` of tile `t` of a section (codes at w, scales
// at s) into out[0..cv): cv = 32 (E2M1), 16 (FP8) or 8 (BF16) values.
int decode_chunk(int fmt, const uint8_t* w, const uint8_t* s, size_t t, int lane, float* out) {
  const uint8_t* q = w + t * moe::kTileBytes + (size_t)lane * 16;
  switch (fmt) {
    case MOE_FMT_MXFP4: {
      const float sc = e8m0(s[t * 64 + lane]);
      for (int i = 0; i < 16; ++i) {
        out[2 * i] = kE2M1[q[i] & 15] * sc;
        out[2 * i + 1] = kE2M1[q[i] >> 4] * sc;
      }
      return 32;
    }
    case MOE_FMT_NVFP4: {
      const float s0 = e4m3(s[t * 128 + 2 * lane]), s1 = e4m3(s[t * 128 + 2 * lane + 1]);
      for (int i = 0; i < 16; ++i) {
        const float sc = i < 8 ? s0 : s1;
        out[2 * i] = kE2M1[q[i] & 15] * sc;
        out[2 * i + 1] = kE2M1[q[i] >> 4] * sc;
      }
      return 32;
    }
    case MOE_FMT_FP8:
      for (int i = 0; i < 16; ++i) out[i] = e4m3(q[i]);
      return 16;
    default: {
      uint16_t b[8];
      memcpy(b, q, 16);
      for (int i = 0; i < 8; ++i) out[i] = bf16f(b[i]);
      return 8;
    }
  }
}

// acc[t][r] (t < n, r < 16 * ngroups) += sum_k W[row][k] x[t][k] over the
// row groups [g0, g1) of a section with nk K-tiles of kt values each.
void section_dot(int fmt, const uint8_t* w, const uint8_t* s, int nk, int kt, int g0, int g1, const float* x, int K,
                 int n, float* acc, int acc_stride) {
  float v[32];
  for (int g = g0; g < g1; ++g)
    for (int k = 0; k < nk; ++k) {
      const size_t t = (size_t)g * nk + k;
      for (int lane = 0; lane < 64; ++lane) {
        const int cv = decode_chunk(fmt, w, s, t, lane, v);
        const int row = g * 16 + (lane & 15), k0 = k * kt + (lane >> 4) * cv;
        for (int tok = 0; tok < n; ++tok) {
          const float* xr = x + (size_t)tok * K + k0;
          float d = 0.f;
          for (int i = 0; i < cv; ++i) d += v[i] * xr[i];
          acc[(size_t)tok * acc_stride + row] += d;
        }
      }
    }
}

}  // namespace

extern "C" moe_status moe_cpu_expert_ffn(const void* blob, const uint16_t* x, int n, float* y, int threads) {
  MOE_CHECK_ARG(blob && (n == 0 || (x && y)) && n >= 0, "moe_cpu_expert_ffn: null pointer or negative n");
  MOE_CHECK_ARG(threads >= 1 && threads <= 256, "moe_cpu_expert_ffn: threads %d out of [1, 256]", threads);
  const moe::BlobHeader* h = static_cast<const moe::BlobHeader*>(blob);
  MOE_CHECK_ARG(h->magic == moe::kBlobMagic, "moe_cpu_expert_ffn: not a blob (magic %08x)", h->magic);
  moe::BlobLayout L;
  MOE_CHECK_ARG(moe::layout_of(h->fmt, h->H, h->I, &L), "moe_cpu_expert_ffn: bad blob header");
  if (n == 0) return MOE_OK;
  const int fmt = h->fmt, H = h->H, I = h->I, kt = moe::k_per_tile(fmt);
  const uint8_t* b = static_cast<const uint8_t*>(blob);
  std::vector<float> xf((size_t)n * H), gu((size_t)n * 2 * I, 0.f), hf((size_t)n * I), yf((size_t)n * H, 0.f);
  for (size_t i = 0; i < xf.size(); ++i) xf[i] = bf16f(x[i]);
  const float gg = h->g[0], gup = h->g[1], gd = h->g[2];
  // gate/up: W13 row groups (2 I / 16; even gate, odd up), K = H; acc rows in W13 order
  const int g13 = 2 * I / 16, g2 = H / 16;
  pool().run(threads, [&](int id, int nt) {
    const int a = (int)((long long)g13 * id / nt), e = (int)((long long)g13 * (id + 1) / nt);
    section_dot(fmt, b + L.off_w13, b + L.off_s13, H / kt, kt, a, e, xf.data(), H, n, gu.data(), 2 * I);
  });
  // SwiGLU: W13 row 32 p + r is gate row 16 p + r (r < 16), else up row 16 p + r - 16
  for (int t = 0; t < n; ++t)
    for (int i = 0; i < I; ++i) {
      const int p = i / 16, r = i % 16;
      const float g = gu[(size_t)t * 2 * I + 32 * p + r] * gg, u = gu[(size_t)t * 2 * I + 32 * p + 16 + r] * gup;
      hf[(size_t)t * I + i] = g / (1.f + std::exp(-g)) * u;
    }
  pool().run(threads, [&](int id, int nt) {
    const int a = (int)((long long)g2 * id / nt), e = (int)((long long)g2 * (id + 1) / nt);
    section_dot(fmt, b + L.off_w2, b + L.off_s2, I / kt, kt, a, e, hf.data(), I, n, yf.data(), H);
  });
  for (size_t i = 0; i < yf.size(); ++i) y[i] = yf[i] * gd;
  return MOE_OK;
}

extern "C" moe_status moe_calibrate_bw(const void* host_blob, void* dev_buf, int reps, int threads,
                                       moe_stream_t copy_stream, moe_bw_calib* out) {
  MOE_CHECK_ARG(host_blob && dev_buf && out && reps >= 1, "moe_calibrate_bw: bad arguments");
  const moe::BlobHeader* h = static_cast<const moe::BlobHeader*>(host_blob);
  MOE_CHECK_ARG(h->magic == moe::kBlobMagic, "moe_calibrate_bw: not a blob");
  const size_t bytes = (size_t)h->total;
  hipStream_t cs = reinterpret_cast<hipStream_t>(copy_stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  MOE_HIP(hipEventCreate(&e0));
  MOE_HIP(hipEventCreate(&e1));
  // host -> device: reps copies of the blob from pinned memory, after one
  // untimed, by the path the decode steps take: the fill kernel when the blob
  // is mapped pinned memory on a 16-byte boundary, else the copy engine
  void* mapped = nullptr;
  if (hipHostGetDevicePointer(&mapped, const_cast<void*>(host_blob), 0) != hipSuccess) {
    (void)hipGetLastError();
    mapped = nullptr;
  }
  const bool kernel = mapped && ((uintptr_t)mapped & 15) == 0 && ((uintptr_t)dev_buf & 15) == 0 && bytes % 16 == 0 &&
                      bytes / 16 < (1ull << 31);
  moe::FillList fl{};
  moe::StepMap none{};
  if (kernel) {
    fl.n = 1;
    fl.off16 = 0;
    fl.len16 = (uint32_t)(bytes / 16);
    fl.slot[0] = 0;
    fl.src[0] = static_cast<const uint8_t*>(mapped);
  }
  auto copy_once = [&]() {
    return kernel ? moe::launch_fill_slots(fl, none, 0, nullptr, dev_buf, bytes, cs)
                  : hipMemcpyAsync(dev_buf, host_blob, bytes, hipMemcpyHostToDevice, cs);
  };
  hipError_t err = copy_once();
  if (err == hipSuccess) err = hipEventRecord(e0, cs);
  for (int i = 0; i < reps && err == hipSuccess; ++i) err = copy_once();
  if (err == hipSuccess) err = hipEventRecord(e1, cs);
  if (err == hipSuccess) err = hipEventSynchronize(e1);
  float ms = 0.f;
  if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (err != hipSuccess) return moe::set_error(MOE_EHIP, "moe_calibrate_bw: copy timing failed: %s", hipGetErrorString(err));
  // host: the CPU expert FFN on one token row, reps times after one untimed
  std::vector<uint16_t> x((size_t)h->H, 0x3F80);  // 1.0
  std::vector<float> y((size_t)h->H);
  moe_status st = moe_cpu_expert_ffn(host_blob, x.data(), 1, y.data(), threads);
  if (st != MOE_OK) return st;
  const auto t0 = std::chrono::steady_clock::now();
  for (int i = 0; i < reps; ++i) moe_cpu_expert_ffn(host_blob, x.data(), 1, y.data(), threads);
  const double cpu_us = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count() / reps;
  out->copy_us = ms * 1e3 / reps;
  out->cpu_us = cpu_us;
  out->h2d_gbs = bytes / (out->copy_us * 1e3);
  out->host_gbs = bytes / (cpu_us * 1e3);
  // misses split so that the copies of a share r and the host's run of the
  // rest take equal time: r copy_us = (1 - r) cpu_us
  out->copy_ratio = (float)(cpu_us / (cpu_us + out->copy_us));
  return MOE_OK;
}
