// Internal header of libmoe (not installed).  gfx950 only.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "host_common.h"

namespace moe {

// Copies vectors [f.off16, f.off16 + f.len16) of every blob of f from host
// memory into its slot (slot_vecs 16-byte vectors a slot of pool): workgroup
// w of nw takes every nw-th 256-vector chunk of each blob in turn, two loads
// in flight per thread.  With nw = kCopyWgs that is 128 KiB in flight, which
// keeps the host link at its read rate (about 51 GB/s on MI355X) without a
// deep backlog: host-memory reads of other work (command packets, kernel
// arguments, a concurrent kernel's launch) then wait about 2 us behind it
// instead of about 13 us with 1 MiB in flight.
constexpr int kCopyWgs = 16;
__device__ __forceinline__ void copy_blob_list(const FillList& f, uint4* __restrict__ pool, uint32_t slot_vecs, int w,
                                               int nw) {
  const uint32_t n = f.len16, step = (uint32_t)nw * 256u;
  for (int b = 0; b < f.n; ++b) {
    const uint4* src = reinterpret_cast<const uint4*>(f.src[b]) + f.off16;
    uint4* dst = pool + (size_t)f.slot[b] * slot_vecs + f.off16;
    uint32_t v = (uint32_t)w * 256u + threadIdx.x;
    for (; v + step < n; v += 2 * step) {  // named registers: no stack array
      const uint4 r0 = src[v], r1 = src[v + step];
      dst[v] = r0;
      dst[v + step] = r1;
    }
    if (v < n) dst[v] = src[v];
  }
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
  return __builtin_bit_cast(uint16_t, (__bf16)f);  // v_cvt_pk_bf16_f32: round to nearest even
}

// Two fp32 values as packed bf16 (a in the low half), round to nearest even:
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  typedef float v2f __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2bf));
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
  // selects, not branches: this runs once per weight tile in the decode loops
  const uint32_t n = c << 23;
  const uint32_t u = c == 0u ? 0x00400000u : n;
  return __uint_as_float(c == 255u ? 0x7FC00000u : u);
}

}  // namespace moe
