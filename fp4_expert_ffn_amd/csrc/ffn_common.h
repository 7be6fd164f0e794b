// Shared device helpers for the expert-FFN kernels (GEMV and MFMA paths).
#pragma once
#include "common.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// Everything a FFN kernel needs to find its expert, its rows and its weights.
struct FfnParams {
  int T, k, E, H, I, fmt;
  const uint16_t* x;           // [T, H] bf16
  const int32_t* counts;       // [E]
  const int32_t* offsets;      // [E+1]
  const int32_t* perm;         // [T*k]
  const int32_t* inv;          // [T*k] perm inverse (inv[perm[p]] = p); null: derive into inv_ws
  int32_t* inv_ws;             // [T*k] workspace for the derived inverse
  const int32_t* slot_of_expert;
  const uint8_t* slot_pool;
  size_t slot_stride;
  const uint8_t* shared_blob;  // nullable
  const uint8_t* mask;         // nullable [E]
  BlobLayout L;
  int umax;                    // routed active-expert indices covered by the grid
};

// Workspace buffers of the matrix-core path.
struct MfmaBufs {
  const uint8_t* xq;   // FP4 gate/up A operand: [T][H/2] codes
  const uint8_t* xs;   //                        [T][H/32] E8M0
  uint8_t* hq;         // FP4 SwiGLU output: [R][I/2] codes
  uint8_t* hs;         //                    [R][I/32] E8M0
  uint16_t* hb;        // BF16 SwiGLU output: [R][I]
  float* y;            // expert outputs: [R][H] fp32, perm order
  uint16_t* yb;        // if set, the expert outputs go here instead, as bf16
};

// Arguments of the decode (GEMV) launches beyond FfnParams.
struct GemvArgs {
  uint16_t* h;     // [R][I] bf16 SwiGLU output
  float* y;        // [R][H] fp32 expert outputs
  float* trash;    // 1 MiB of scratch: stores of padding rows land here
  int ng, nd;      // gate/up and down column chunks per expert
  int rbs1, rbs2;  // rows per row block (<= 16) of the two launches
  int na;          // active-expert capacity of the LDS table
  int act_off;     // LDS byte offset of the staged operand rows
  int yflat;       // 1: y rows in flat order t * k + j (T*k <= 1024 only), 0: perm order
  int ncu;         // > 0: the grid is two workgroups per CU on ncu CUs (items dealt per CU)
  // routing folded into the gate/up launch (logits non-null): every workgroup
  // routes the call's few tokens itself; workgroup 0 writes topk ids /
  // weights and the counts, offsets, permutation and its inverse (P's
  // pointers) for the down projection and the combine
  const float* logits;
  int renorm;
  int32_t* ids_out;
  float* w_out;
  // blob copies riding along a gate/up launch without folded routing
  // (copy_wgs > 0): the last copy_wgs workgroups copy vectors [copy.off16,
  // copy.off16 + copy.len16) of each listed blob from host memory into its
  // slot of copy_pool (copy_slot_vecs vectors a slot; copy_blob_list); the
  // others run the GEMV
  int copy_wgs;
  uint32_t copy_slot_vecs;
  uint4* copy_pool;
  FillList copy;
};

// One unit of expert work: an expert (or the shared expert) and its rows.
struct Job {
  const uint8_t* blob;
  int rows;    // number of rows
  int p0;      // first row index in the perm-ordered h / y buffers
  int shared;  // 1 for the shared expert (row r is token r)
};

// Resolve active-expert index `a` (ascending expert id among experts with
// rows and an enabled mask; a == umax is the shared expert).  Must be called
// by every thread of the workgroup (uses LDS and a barrier).  rows == 0 means
// "nothing to do".
__device__ inline Job resolve_job(const FfnParams& P, int a) {
  __shared__ int s_e;
  Job j;
  j.blob = nullptr;
  j.rows = 0;
  j.p0 = 0;
  j.shared = 0;
  if (a == P.umax) {
    if (P.shared_blob) {
      j.blob = P.shared_blob;
      j.rows = P.T;
      j.p0 = P.T * P.k;
      j.shared = 1;
    }
    return j;  // uniform across the workgroup: no barrier needed
  }
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int found = -1, seen = 0;
    for (int base = 0; base < P.E && found < 0; base += 64) {
      const int e = base + lane;
      bool act = false;
      if (e < P.E) act = P.counts[e] > 0 && (P.mask == nullptr || P.mask[e] != 0);
      const uint64_t b = __ballot(act);
      const int n = __popcll(b);
      if (a < seen + n) {
        // the (a - seen)-th set bit of b
        uint64_t bb = b;
        for (int i = 0; i < a - seen; ++i) bb &= bb - 1;
        found = base + __ffsll((unsigned long long)bb) - 1;
      }
      seen += n;
    }
    if (lane == 0) s_e = found;
  }
  __syncthreads();
  const int e = s_e;
  if (e >= 0) {
    j.rows = P.counts[e];
    j.p0 = P.offsets[e];
    j.blob = P.slot_pool + (size_t)P.slot_of_expert[e] * P.slot_stride;
  }
  return j;
}

__device__ __forceinline__ int job_token(const FfnParams& P, const Job& j, int r) {
  return j.shared ? r : P.perm[j.p0 + r] / P.k;
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }

// 32 E2M1 codes (16 bytes) -> 16 packed bf16 pairs (exact; scale applied later).
__device__ __forceinline__ void fp4x32_to_bf16(const uint4 c, bf16x2_t out[16]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    out[4 * d + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], 1.0f, 0);
    out[4 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], 1.0f, 1);
    out[4 * d + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], 1.0f, 2);
    out[4 * d + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], 1.0f, 3);
  }
}

// 32 E2M1 codes -> 32 floats (exact).
__device__ __forceinline__ void fp4x32_to_f32(const uint4 c, float out[32]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 0);
    f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 1);
    f32x2_t c2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 2);
    f32x2_t d2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 3);
    out[8 * d + 0] = a.x; out[8 * d + 1] = a.y;
    out[8 * d + 2] = b.x; out[8 * d + 3] = b.y;
    out[8 * d + 4] = c2.x; out[8 * d + 5] = c2.y;
    out[8 * d + 6] = d2.x; out[8 * d + 7] = d2.y;
  }
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), c, false);
}

__device__ __forceinline__ uint4 ldg16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads() it
// does not wait for outstanding global loads (weight prefetches stay in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------------------------ MXFP4 encoding
// floor(log2|v|) of a finite nonzero fp32 value (exact, from the bits).
__device__ __forceinline__ int ilog2_f32(float v) {
  const uint32_t u = __float_as_uint(v) & 0x7FFFFFFFu;
  const int e = (int)(u >> 23);
  const int sub = (31 - __clz(u)) - 149;  // subnormal: u * 2^-149
  return e ? e - 127 : sub;               // a select, not a branch
}

// |q| -> E2M1 magnitude code, round to nearest even, saturate at 6: the
// boundaries (ties to the even code: <= at 0.25, 1.25, 2.5, 5; < at 0.75,
// 1.75, 3.5) are nested, so the code is the number of them a lies above,
// counted without branches (a NaN lies above none and gets 7).
__device__ __forceinline__ uint32_t e2m1_mag_rne(float a) {
  return (uint32_t)!(a <= 0.25f) + (uint32_t)!(a < 0.75f) + (uint32_t)!(a <= 1.25f) + (uint32_t)!(a < 1.75f) +
         (uint32_t)!(a <= 2.5f) + (uint32_t)!(a < 3.5f) + (uint32_t)!(a <= 5.0f);
}

// Encode 32 fp32 values as MXFP4: 16 packed bytes (element 2i low nibble) + E8M0.
__device__ __forceinline__ void mxfp4_encode32(const float* v, uint4& q, uint32_t& s) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int ex = amax != 0.f ? min(127, max(-127, ilog2_f32(amax) - 2)) : 0;
  s = (uint32_t)(ex + 127);
  // 2^-ex as an exact fp32 (normal for ex in [-127, 126]; subnormal 2^-127 for ex = 127)
  const float inv = ex == 127 ? __uint_as_float(0x00400000u) : __uint_as_float((uint32_t)(127 - ex) << 23);
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float qv = v[i] * inv;
    const uint32_t code = e2m1_mag_rne(fabsf(qv)) | ((__float_as_uint(v[i]) >> 28) & 8u);
    w[i >> 3] |= code << (4 * (i & 7));
  }
  q = make_uint4(w[0], w[1], w[2], w[3]);
}

// Barrier that orders LDS only: waits for this wave's LDS operations, not
// for its global loads.  (A fenced barrier also waits for every global
// load while direct-to-LDS loads are outstanding.)
__device__ __forceinline__ void lds_sync() {
  // gfx9 s_waitcnt: vmcnt 63 (no wait), expcnt 7 (no wait), lgkmcnt 0
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace moe
