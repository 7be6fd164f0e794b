// Internal header of libmoe (not installed).  gfx950 only.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/moe.h"

// ---------------------------------------------------------------- errors
namespace moe {
moe_status set_error(moe_status st, const char* fmt, ...);
inline moe_status ok() { return MOE_OK; }
}  // namespace moe

#define MOE_CHECK_ARG(cond, ...)                                  \
  do {                                                            \
    if (!(cond)) return moe::set_error(MOE_EINVAL, __VA_ARGS__);  \
  } while (0)

#define MOE_HIP(call)                                                                          \
  do {                                                                                         \
    hipError_t e_ = (call);                                                                    \
    if (e_ != hipSuccess)                                                                      \
      return moe::set_error(MOE_EHIP, "%s failed: %s", #call, hipGetErrorString(e_));          \
  } while (0)

// Launch check: picks up launch-configuration errors and earlier asynchronous faults.
#define MOE_LAUNCHED()                                                                         \
  do {                                                                                         \
    hipError_t e_ = hipGetLastError();                                                         \
    if (e_ != hipSuccess)                                                                      \
      return moe::set_error(MOE_EHIP, "kernel launch failed: %s", hipGetErrorString(e_));      \
  } while (0)

// ---------------------------------------------------------------- blob layout
//
// Blob = 256-byte header, then four sections, each 256-byte aligned:
//   W13 codes, W13 scales, W2 codes, W2 scales.
// W13 holds gate and up interleaved by 16-row groups: row-group rg = 2p is
// gate rows [16p, 16p+16), rg = 2p+1 is up rows [16p, 16p+16).  W2 is down.
//
// Every section is a sequence of 1 KiB tiles, ordered (row-group, K-tile)
// with K fastest.  A tile covers 16 rows x KT columns, KT = 128 for the 4-bit
// formats and 32 for BF16, and lists 64 lanes' 16-byte fragments in lane
// order: lane l holds row (l % 16) and the K-chunk (l / 16) of the tile
// (32 E2M1 codes, or 8 bf16 values).  This is the operand layout of the
// gfx950 16x16x128 (FP4) and 16x16x32 (BF16) MFMA B-fragments, and it makes
// every wave-wide 16-byte load one contiguous 1 KiB transaction.
//
// Scale tiles follow the same order: MXFP4 64 B per tile (lane l: the E8M0
// of its 32 values), NVFP4 128 B per tile (lane l: bytes 2l, 2l+1 = the two
// E4M3 scales of its 32 values).
namespace moe {

constexpr uint32_t kBlobMagic = 0x42454F4Du;  // "MOEB"
constexpr int kHeaderBytes = 256;
constexpr int kTileBytes = 1024;

struct BlobHeader {
  uint32_t magic;
  uint32_t version;
  int32_t fmt, H, I;
  float g[3];  // NVFP4 per-tensor multipliers (gate, up, down); 1 otherwise
  uint64_t off_w13, off_s13, off_w2, off_s2, total;
  uint8_t pad[kHeaderBytes - 4 * 2 - 4 * 3 - 4 * 3 - 8 * 5];
};
static_assert(sizeof(BlobHeader) == kHeaderBytes, "header size");

__host__ __device__ inline int k_per_tile(int fmt) { return fmt == MOE_FMT_BF16 ? 32 : 128; }
__host__ __device__ inline int scale_bytes_per_tile(int fmt) {
  return fmt == MOE_FMT_MXFP4 ? 64 : (fmt == MOE_FMT_NVFP4 ? 128 : 0);
}
inline uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

struct BlobLayout {
  uint64_t off_w13, off_s13, off_w2, off_s2, total;
  int tiles13, tiles2;  // tile counts
};

inline bool layout_of(int fmt, int H, int I, BlobLayout* L) {
  if (fmt != MOE_FMT_BF16 && fmt != MOE_FMT_MXFP4 && fmt != MOE_FMT_NVFP4) return false;
  if (H <= 0 || I <= 0 || H % 128 || I % 128) return false;
  const int kt = k_per_tile(fmt), sb = scale_bytes_per_tile(fmt);
  L->tiles13 = (2 * I / 16) * (H / kt);
  L->tiles2 = (H / 16) * (I / kt);
  uint64_t o = kHeaderBytes;
  L->off_w13 = o; o = align256(o + (uint64_t)L->tiles13 * kTileBytes);
  L->off_s13 = o; o = align256(o + (uint64_t)L->tiles13 * sb);
  L->off_w2 = o;  o = align256(o + (uint64_t)L->tiles2 * kTileBytes);
  L->off_s2 = o;  o = align256(o + (uint64_t)L->tiles2 * sb);
  L->total = o;
  return true;
}

// Device-side view of one expert blob.
struct BlobView {
  const uint8_t* w13;
  const uint8_t* s13;
  const uint8_t* w2;
  const uint8_t* s2;
  float g_gate, g_up, g_down;
};

__device__ inline BlobView blob_view(const uint8_t* b, const BlobLayout& L) {
  const BlobHeader* h = reinterpret_cast<const BlobHeader*>(b);
  BlobView v;
  v.w13 = b + L.off_w13;
  v.s13 = b + L.off_s13;
  v.w2 = b + L.off_w2;
  v.s2 = b + L.off_s2;
  v.g_gate = h->g[0];
  v.g_up = h->g[1];
  v.g_down = h->g[2];
  return v;
}

// ---------------------------------------------------------------- launch tracing
// moe_expert_ffn_traced hands caller-created events to every kernel launch of
// one call through this per-thread hook: launch i records events 2i and 2i+1
// at the kernel's own start and end (hipExtLaunchKernelGGL).
struct LaunchTrace {
  void* const* events;  // hipEvent_t
  int n, used;
};
extern thread_local LaunchTrace* g_launch_trace;

template <typename F, typename... Args>
inline void launch(F kernel, dim3 grid, dim3 block, size_t shmem, hipStream_t s, Args... args) {
  LaunchTrace* t = g_launch_trace;
  if (t && t->used + 2 <= t->n) {
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)shmem, s, static_cast<hipEvent_t>(t->events[t->used]),
                          static_cast<hipEvent_t>(t->events[t->used + 1]), 0u, args...);
    t->used += 2;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
  }
}

// ---------------------------------------------------------------- numerics helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

// SwiGLU gate factor z * sigmoid(z) from the hardware exp2 and reciprocal
// (each within 1 ulp); -inf -> -0, +inf -> +inf.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

// E4M3FN code -> float (positive scales only are produced; sign kept for generality).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = (e == 0) ? (float)m * 0.001953125f /* 2^-9 */
                       : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

// E8M0 code -> float 2^(c-127) (c = 255 is NaN; c = 0 is the fp32 subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
  if (c == 0) return __uint_as_float(0x00400000u);
  if (c == 255) return __uint_as_float(0x7FC00000u);
  return __uint_as_float(c << 23);
}

}  // namespace moe
