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

// Lane l holds experts l + 64 i (i < NPER, NPER * 64 >= E), each as a 32-bit
// rank key (0: no expert).  Selection in k rounds: round r takes the largest
// remaining key (a wave-wide maximum: DPP row steps, then the cross-row
// permlane swaps) and, of the keys equal to it, the one with the lowest
// expert id (the lowest slot i holding one, then the lowest lane); that key
// is output position r and leaves the remaining set.  The k keys are thus
// the k largest in the order (key descending, id ascending), in that order.
// Then the softmax over them (renormalised) or over all E.
// Writes ids[pos], w[pos] for pos in [0, k) (global or LDS pointers).
//
// The logits of one row as the selection holds them: lane l, experts
// l + 64 i (0 past E).  Separate from the selection so that a wave can load
// several rows before it selects in any of them.
template <int NPER>
__device__ __forceinline__ void wave_topk_load(const float* __restrict__ row, int E, float (&val)[NPER]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + 64 * i;
    val[i] = e < E ? row[e] : 0.f;
  }
}

template <int NPER>
__device__ __forceinline__ void wave_topk_select(const float (&val)[NPER], int E, int k, int renorm, int32_t* ids,
                                                 float* wout) {
  const int lane = threadIdx.x & 63;
  uint32_t rk[NPER];  // remaining keys (0: none, or taken)
  bool sel[NPER];
  int pos[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    rk[i] = lane + 64 * i < E ? rank_bits(val[i]) + 1u : 0u;  // NaN -> 1, below every number
    sel[i] = false;
    pos[i] = 0;
  }
  float top = 0.f;  // the logit at position 0
  for (int r = 0; r < k; ++r) {
    uint32_t lm = rk[0];
#pragma unroll
    for (int i = 1; i < NPER; ++i) lm = max(lm, rk[i]);
    const uint32_t m = wave_max_u32(lm);
    if (m == 0u) break;  // fewer than k keys (not reached: k <= E)
    // slot ws and lane wl of the key taken: the lowest slot holding m, its
    // lowest lane (wave-uniform selects, no branches)
    uint64_t bs[NPER];
#pragma unroll
    for (int i = 0; i < NPER; ++i) bs[i] = __ballot(rk[i] == m);
    int ws = NPER - 1;
    uint64_t bw = bs[NPER - 1];
#pragma unroll
    for (int i = NPER - 2; i >= 0; --i) {
      ws = bs[i] ? i : ws;
      bw = bs[i] ? bs[i] : bw;
    }
    const int wl = __builtin_ctzll(bw);
    if (r == 0) {
      float v = val[0];
#pragma unroll
      for (int i = 1; i < NPER; ++i) v = i == ws ? val[i] : v;
      top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), wl));
    }
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const bool hit = i == ws && lane == wl;
      sel[i] = sel[i] || hit;
      pos[i] = hit ? r : pos[i];
      rk[i] = hit ? 0u : rk[i];
    }
  }
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < NPER; ++i)
    if (renorm ? sel[i] : lane + 64 * i < E) part += unnorm(val[i], top);
  const float den = wave_sum(part);
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    if (sel[i]) {
      ids[pos[i]] = lane + 64 * i;
      wout[pos[i]] = den > 0.f ? unnorm(val[i], top) / den : 1.0f / (float)k;
    }
  }
}

template <int NPER>
__device__ __forceinline__ void wave_topk(const float* __restrict__ row, int E, int k, int renorm, int32_t* ids,
                                          float* wout) {
  float val[NPER];
  wave_topk_load<NPER>(row, E, val);
  wave_topk_select<NPER>(val, E, k, renorm, ids, wout);
}

}  // namespace moe
