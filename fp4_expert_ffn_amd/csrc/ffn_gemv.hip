// Decode path of the expert FFN: a dequantising GEMV that streams each
// touched expert's packed weights from HBM exactly once per call.
//
// Method: cache hits execute on the GPU (page "FreeToken量子化：MoE推論の
// セットアップガイド", decode paragraph); the expert is a SwiGLU FFN over
// MXFP4 / NVFP4 / BF16 weights (this library's reading; formats named on the
// same page, third paragraph).
//
// Work split (wave64, 256-thread workgroups):
//   gate/up: one workgroup per (active expert, 16-row pair group of gate and
//            up rows); the four waves split the K-tiles of H; each lane owns
//            row (lane % 16) and K-chunk (lane / 16) of every tile, so a
//            wave-wide 16-byte load is one contiguous 1 KiB tile.  Block
//            scales are applied to per-block partial dots (fp32), the NVFP4
//            per-tensor multiplier after the reduction.  h = silu(g) * u, fp32.
//   down:    one workgroup per (active expert, 64 output rows); each wave owns
//            16 rows over all K-tiles of I.  h is staged in LDS as fp32.
// Activations: x stays bf16 (bf16 x bf16 products are exact in fp32 via
// v_dot2_f32_bf16); h stays fp32 (v_fma_f32 against exact fp4->f32 weights).
#include "ffn_common.h"

namespace moe {

template <int FMT>
struct Fmt;
template <>
struct Fmt<MOE_FMT_BF16> {
  static constexpr int KT = 32, EPL = 8, SB = 0;
};
template <>
struct Fmt<MOE_FMT_MXFP4> {
  static constexpr int KT = 128, EPL = 32, SB = 64;
};
template <>
struct Fmt<MOE_FMT_NVFP4> {
  static constexpr int KT = 128, EPL = 32, SB = 128;
};

// Partial dot of one lane's fragment (EPL weights) with EPL bf16 activations.
// xs: EPL/2 packed bf16 pairs.  Returns the scaled partial (block scales applied).
template <int FMT>
__device__ __forceinline__ float frag_dot_bf16(const uint4 wq, uint32_t sc, const uint32_t* xs);

template <>
__device__ __forceinline__ float frag_dot_bf16<MOE_FMT_BF16>(const uint4 wq, uint32_t, const uint32_t* xs) {
  float a = 0.f;
  a = dot2_bf16(wq.x, xs[0], a);
  a = dot2_bf16(wq.y, xs[1], a);
  a = dot2_bf16(wq.z, xs[2], a);
  a = dot2_bf16(wq.w, xs[3], a);
  return a;
}

template <>
__device__ __forceinline__ float frag_dot_bf16<MOE_FMT_MXFP4>(const uint4 wq, uint32_t sc, const uint32_t* xs) {
  bf16x2_t w[16];
  fp4x32_to_bf16(wq, w);
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) a = __builtin_amdgcn_fdot2_f32_bf16(w[i], as_bf16x2(xs[i]), a, false);
  return a * e8m0_to_f32(sc & 0xFFu);
}

template <>
__device__ __forceinline__ float frag_dot_bf16<MOE_FMT_NVFP4>(const uint4 wq, uint32_t sc, const uint32_t* xs) {
  bf16x2_t w[16];
  fp4x32_to_bf16(wq, w);
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a0 = __builtin_amdgcn_fdot2_f32_bf16(w[i], as_bf16x2(xs[i]), a0, false);
#pragma unroll
  for (int i = 8; i < 16; ++i) a1 = __builtin_amdgcn_fdot2_f32_bf16(w[i], as_bf16x2(xs[i]), a1, false);
  return a0 * e4m3_to_f32(sc & 0xFFu) + a1 * e4m3_to_f32((sc >> 8) & 0xFFu);
}

template <int FMT>
__device__ __forceinline__ uint32_t load_scale(const uint8_t* s_tiles, size_t tile, int lane) {
  if constexpr (FMT == MOE_FMT_MXFP4) return s_tiles[tile * 64 + lane];
  if constexpr (FMT == MOE_FMT_NVFP4) return *reinterpret_cast<const uint16_t*>(s_tiles + tile * 128 + 2 * lane);
  return 0u;
}

// ---------------------------------------------------------------- gate / up

template <int FMT, int RB>
__global__ __launch_bounds__(256) void k_gemv_gateup(FfnParams P, float* __restrict__ hbuf) {
  using F = Fmt<FMT>;
  const Job job = resolve_job(P, blockIdx.y);
  if (job.rows == 0) return;
  extern __shared__ __align__(16) uint8_t lds[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds);                    // [RB][H]
  float* red = reinterpret_cast<float*>(lds + (size_t)RB * P.H * 2);  // [4 waves][RB][16][2]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = P.H, I = P.I, nk = H / F::KT;
  const int pair = blockIdx.x;  // rows [16*pair, 16*pair+16) of gate and of up
  const BlobView bv = blob_view(job.blob, P.L);
  const size_t tile_g0 = (size_t)(2 * pair) * nk, tile_u0 = (size_t)(2 * pair + 1) * nk;
  const int kchunk = (lane >> 4) * F::EPL;  // element offset of this lane's chunk within a tile

  for (int r0 = 0; r0 < job.rows; r0 += RB) {
    const int nr = min(RB, job.rows - r0);
    // stage x rows (bf16) for this chunk of rows
    for (int i = tid * 8; i < nr * H; i += 256 * 8) {
      const int r = i / H, c = i % H;
      const int t = job_token(P, job, r0 + r);
      *reinterpret_cast<uint4*>(xs + (size_t)r * H + c) = *reinterpret_cast<const uint4*>(P.x + (size_t)t * H + c);
    }
    __syncthreads();
    float ag[RB], au[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) ag[r] = au[r] = 0.f;
    for (int kt = wave; kt < nk; kt += 4) {
      const uint4 wg = ldg16(bv.w13 + (tile_g0 + kt) * kTileBytes + lane * 16);
      const uint4 wu = ldg16(bv.w13 + (tile_u0 + kt) * kTileBytes + lane * 16);
      const uint32_t sg = load_scale<FMT>(bv.s13, tile_g0 + kt, lane);
      const uint32_t su = load_scale<FMT>(bv.s13, tile_u0 + kt, lane);
      const int col = kt * F::KT + kchunk;
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if (r < nr) {
          uint32_t xv[F::EPL / 2];
          const uint4* xp = reinterpret_cast<const uint4*>(xs + (size_t)r * H + col);
#pragma unroll
          for (int q = 0; q < F::EPL / 8; ++q) {
            const uint4 v = xp[q];
            xv[4 * q + 0] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
          }
          ag[r] += frag_dot_bf16<FMT>(wg, sg, xv);
          au[r] += frag_dot_bf16<FMT>(wu, su, xv);
        }
      }
    }
    // reduce the 4 K-chunks of a row (lanes l, l^16, l^32, l^48) then across waves
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      float g = ag[r], u = au[r];
      g += __shfl_xor(g, 16);
      u += __shfl_xor(u, 16);
      g += __shfl_xor(g, 32);
      u += __shfl_xor(u, 32);
      if (lane < 16) {
        red[((wave * RB + r) * 16 + lane) * 2 + 0] = g;
        red[((wave * RB + r) * 16 + lane) * 2 + 1] = u;
      }
    }
    __syncthreads();
    if (tid < 16 * nr) {
      const int i = tid & 15, r = tid >> 4;
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        g += red[((w * RB + r) * 16 + i) * 2 + 0];
        u += red[((w * RB + r) * 16 + i) * 2 + 1];
      }
      g *= bv.g_gate;
      u *= bv.g_up;
      hbuf[(size_t)(job.p0 + r0 + r) * I + 16 * pair + i] = silu_f32(g) * u;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- down

template <int FMT>
__device__ __forceinline__ void frag_dot_f32_rows(const uint4 wq, uint32_t sc, const float* hrow, float& acc);

template <>
__device__ __forceinline__ void frag_dot_f32_rows<MOE_FMT_BF16>(const uint4 wq, uint32_t, const float* h,
                                                                float& acc) {
  const uint32_t w[4] = {wq.x, wq.y, wq.z, wq.w};
  const float4 h0 = reinterpret_cast<const float4*>(h)[0], h1 = reinterpret_cast<const float4*>(h)[1];
  const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a = fmaf(__uint_as_float(w[i] << 16), hv[2 * i], a);
    a = fmaf(__uint_as_float(w[i] & 0xFFFF0000u), hv[2 * i + 1], a);
  }
  acc += a;
}

template <>
__device__ __forceinline__ void frag_dot_f32_rows<MOE_FMT_MXFP4>(const uint4 wq, uint32_t sc, const float* h,
                                                                 float& acc) {
  float w[32];
  fp4x32_to_f32(wq, w);
  float a = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float4 hv = reinterpret_cast<const float4*>(h)[q];
    a = fmaf(w[4 * q + 0], hv.x, a);
    a = fmaf(w[4 * q + 1], hv.y, a);
    a = fmaf(w[4 * q + 2], hv.z, a);
    a = fmaf(w[4 * q + 3], hv.w, a);
  }
  acc += a * e8m0_to_f32(sc & 0xFFu);
}

template <>
__device__ __forceinline__ void frag_dot_f32_rows<MOE_FMT_NVFP4>(const uint4 wq, uint32_t sc, const float* h,
                                                                 float& acc) {
  float w[32];
  fp4x32_to_f32(wq, w);
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 hv = reinterpret_cast<const float4*>(h)[q];
    a0 = fmaf(w[4 * q + 0], hv.x, a0);
    a0 = fmaf(w[4 * q + 1], hv.y, a0);
    a0 = fmaf(w[4 * q + 2], hv.z, a0);
    a0 = fmaf(w[4 * q + 3], hv.w, a0);
  }
#pragma unroll
  for (int q = 4; q < 8; ++q) {
    const float4 hv = reinterpret_cast<const float4*>(h)[q];
    a1 = fmaf(w[4 * q + 0], hv.x, a1);
    a1 = fmaf(w[4 * q + 1], hv.y, a1);
    a1 = fmaf(w[4 * q + 2], hv.z, a1);
    a1 = fmaf(w[4 * q + 3], hv.w, a1);
  }
  acc += a0 * e4m3_to_f32(sc & 0xFFu) + a1 * e4m3_to_f32((sc >> 8) & 0xFFu);
}

template <int FMT, int RB>
__global__ __launch_bounds__(256) void k_gemv_down(FfnParams P, const float* __restrict__ hbuf,
                                                   float* __restrict__ ybuf) {
  using F = Fmt<FMT>;
  const Job job = resolve_job(P, blockIdx.y);
  if (job.rows == 0) return;
  extern __shared__ __align__(16) uint8_t lds[];
  float* hs = reinterpret_cast<float*>(lds);  // [RB][I]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = P.H, I = P.I, nk = I / F::KT;
  const int rg = blockIdx.x * 4 + wave;  // 16-row group of W_down = output columns [16 rg, 16 rg + 16)
  const BlobView bv = blob_view(job.blob, P.L);
  const size_t tile0 = (size_t)rg * nk;
  const int kchunk = (lane >> 4) * F::EPL;

  for (int r0 = 0; r0 < job.rows; r0 += RB) {
    const int nr = min(RB, job.rows - r0);
    for (int i = tid * 4; i < nr * I; i += 256 * 4) {
      const int r = i / I, c = i % I;
      *reinterpret_cast<float4*>(hs + (size_t)r * I + c) =
          *reinterpret_cast<const float4*>(hbuf + (size_t)(job.p0 + r0 + r) * I + c);
    }
    __syncthreads();
    float acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r] = 0.f;
    for (int kt = 0; kt < nk; ++kt) {
      const uint4 wq = ldg16(bv.w2 + (tile0 + kt) * kTileBytes + lane * 16);
      const uint32_t sc = load_scale<FMT>(bv.s2, tile0 + kt, lane);
      const int col = kt * F::KT + kchunk;
#pragma unroll
      for (int r = 0; r < RB; ++r)
        if (r < nr) frag_dot_f32_rows<FMT>(wq, sc, hs + (size_t)r * I + col, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      float v = acc[r];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (lane < 16 && r < nr) ybuf[(size_t)(job.p0 + r0 + r) * H + 16 * rg + lane] = v * bv.g_down;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- launchers

template <int FMT, int RB>
static hipError_t launch_gemv_fmt(const FfnParams& P, float* h, float* y, hipStream_t s) {
  const dim3 grid_gu(P.I / 16, P.umax + 1), grid_dn(P.H / 64, P.umax + 1);
  const size_t lds_gu = (size_t)RB * P.H * 2 + 4 * RB * 16 * 2 * sizeof(float);
  const size_t lds_dn = (size_t)RB * P.I * sizeof(float);
  hipLaunchKernelGGL((k_gemv_gateup<FMT, RB>), grid_gu, dim3(256), lds_gu, s, P, h);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemv_down<FMT, RB>), grid_dn, dim3(256), lds_dn, s, P, (const float*)h, y);
  return hipGetLastError();
}

// Rows per LDS chunk: keep the x / h staging under 64 KiB.
hipError_t launch_gemv(const FfnParams& P, float* h, float* y, hipStream_t s) {
  const bool big = (size_t)8 * P.H * 2 > 48 * 1024 || (size_t)8 * P.I * 4 > 48 * 1024;
  switch (P.fmt) {
    case MOE_FMT_BF16:
      return big ? launch_gemv_fmt<MOE_FMT_BF16, 2>(P, h, y, s) : launch_gemv_fmt<MOE_FMT_BF16, 8>(P, h, y, s);
    case MOE_FMT_MXFP4:
      return big ? launch_gemv_fmt<MOE_FMT_MXFP4, 2>(P, h, y, s) : launch_gemv_fmt<MOE_FMT_MXFP4, 8>(P, h, y, s);
    case MOE_FMT_NVFP4:
      return big ? launch_gemv_fmt<MOE_FMT_NVFP4, 2>(P, h, y, s) : launch_gemv_fmt<MOE_FMT_NVFP4, 8>(P, h, y, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
