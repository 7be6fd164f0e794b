// Top-k routing of one logits row by one wave64 (gfx950): the k largest
// logits (ties to the lower expert id, NaN below every number), in
// descending order, and their softmax weights.
//
// Method: a routing network selects a subset of experts for every token at
// every step (page "FreeToken qwen：ローカルQwen MoEセットアップガイド", third
// paragraph; page "FreeToken量子化：MoE推論のセットアップガイド", second
// paragraph).  The selection rule and the softmax over the selected logits
// (renormalised, or over all E) are this library's reading.
#pragma once
#include "common.h"
#include "wave.h"

namespace moe {

constexpr int kRouteMaxK = 16;

// Order-preserving map of an fp32 logit to uint32: larger value -> larger key;
// -0 is folded onto +0; every NaN maps to 0, below -inf (0x007FFFFF).
__device__ __forceinline__ uint32_t rank_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;  // NaN
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;             // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// exp(v - m) for the softmax numerators: NaN contributes 0, the top value 1.
__device__ __forceinline__ float unnorm(float v, float m) {
  if (v != v) return 0.f;
  if (v == m) return 1.f;
  return expf(v - m);
}

// Lane l holds experts l + 64 i (i < NPER, NPER * 64 >= E).  Selection: k
// rounds of a wave-wide max over 64-bit keys (rank key << 32 | (0xFFFF - id)),
// so a larger logit wins and equal logits go to the lower id; the owner of
// each winner removes it.  Round r's winner is output position r.
// Writes ids[pos], w[pos] for pos in [0, k) (global or LDS pointers).
template <int NPER>
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int E, int k, int renorm, int32_t* ids,
                                          float* wout) {
  const int lane = threadIdx.x & 63;
  uint32_t rk[NPER];
  float val[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + 64 * i;
    val[i] = 0.f;
    rk[i] = 0u;
    if (e < E) {
      val[i] = row[e];
      rk[i] = rank_bits(val[i]) + 1u;  // 0 marks "no key"; NaN -> 1, below every number
    }
  }
  uint32_t selmask = 0;
  int pos[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) pos[i] = 0;
  int id0 = 0;  // the largest logit's expert (wave-uniform)
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const uint64_t key = ((uint64_t)rk[i] << 32) | (uint32_t)(0xFFFF - (lane + 64 * i));
      if (rk[i] != 0u && !((selmask >> i) & 1u)) best = max_u64(best, key);
    }
    const uint64_t win = wave_max_u64(best);
    const int id = 0xFFFF - (int)(win & 0xFFFFu);
    if (r == 0) id0 = id;
#pragma unroll
    for (int i = 0; i < NPER; ++i)
      if (lane + 64 * i == id) {
        selmask |= 1u << i;
        pos[i] = r;
      }
  }
  // the top logit m, from the lane that holds it, and the softmax weights
  float tv = 0.f;
#pragma unroll
  for (int i = 0; i < NPER; ++i)
    if (i == (id0 >> 6)) tv = val[i];
  const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tv), id0 & 63));
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const bool sel = (selmask >> i) & 1u;
    if (renorm ? sel : lane + 64 * i < E) part += unnorm(val[i], top);
  }
  const float den = wave_sum(part);
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    if ((selmask >> i) & 1u) {
      ids[pos[i]] = lane + 64 * i;
      wout[pos[i]] = den > 0.f ? unnorm(val[i], top) / den : 1.0f / (float)k;
    }
  }
}

}  // namespace moe
