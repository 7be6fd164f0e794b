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

// Rank of this lane among the set lanes of a wave-uniform mask m below it.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Lane l holds experts l + 64 i (i < NPER, NPER * 64 >= E), each as a 32-bit
// rank key (0: no expert).  Selection:
//  1. the k-th largest key value thr, counted with multiplicity, by a binary
//     radix walk from the top bit: at bit b the keys that match the bits
//     above b chosen so far and have bit b set are counted with ballots; if
//     they are at least the number still needed, bit b of thr is set, else
//     they are all selected and taken off the count;
//  2. every key above thr is selected, and of the keys equal to thr the ones
//     with the lowest expert ids, as many as are still needed;
//  3. a selected key's output position is the number of selected keys that
//     rank above it (larger key, or equal key and lower id), found by one
//     pass over the selected keys with readlane.
// All counts are ballots and scalar arithmetic: no cross-lane reduction
// sits on the critical path except the softmax denominator.
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
  // 1. threshold (wave-uniform)
  uint32_t thr = 0u;
  int need = k;
#pragma unroll 4
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = thr | (1u << b);
    const uint32_t hi = ~0u << b;
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NPER; ++i) cnt += (int)__popcll(__ballot((rk[i] & hi) == cand));
    if (cnt >= need) thr = cand;
    else need -= cnt;
  }
  // 2. selection: `need` keys equal to thr remain to be taken, lowest ids first
  bool sel[NPER];
  uint64_t selm[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const bool eq = rk[i] == thr && rk[i] != 0u;
    const uint64_t eqm = __ballot(eq);
    sel[i] = (rk[i] > thr) || (eq && lanes_below(eqm) < need);
    selm[i] = __ballot(sel[i]);
    need = max(0, need - (int)__popcll(eqm));  // __popcll is unsigned: keep the difference signed
  }
  // 3. output positions
  int pos[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) pos[i] = 0;
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    uint64_t m = selm[j];
    while (m) {
      const int src = __builtin_ctzll(m);
      m &= m - 1;
      const uint32_t ks = (uint32_t)__builtin_amdgcn_readlane((int)rk[j], src);
      const int id = 64 * j + src;
#pragma unroll
      for (int i = 0; i < NPER; ++i) pos[i] += (ks > rk[i] || (ks == rk[i] && id < lane + 64 * i)) ? 1 : 0;
    }
  }
  // the top logit m (position 0), from the lane that holds it, and the softmax weights
  float top = 0.f;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const uint64_t b = __ballot(sel[i] && pos[i] == 0);
    if (b) top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(val[i]), __builtin_ctzll(b)));
  }
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < NPER; ++i)
    if (renorm ? sel[i] : lane + 64 * i < E) part += unnorm(val[i], top);
  const float den = wave_sum(part);
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    if (sel[i] && pos[i] < k) {  // exactly k keys are selected; the bound keeps every store in the row
      ids[pos[i]] = lane + 64 * i;
      wout[pos[i]] = den > 0.f ? unnorm(val[i], top) / den : 1.0f / (float)k;
    }
  }
}

}  // namespace moe
