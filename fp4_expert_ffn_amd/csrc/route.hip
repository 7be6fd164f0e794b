// Router logits, top-k routing with softmax weights, and the token->expert
// permutation (gfx950, wave64).
//
// Method: a routing network selects a subset of experts for every token at
// every step (page "FreeToken qwen：ローカルQwen MoEセットアップガイド", third
// paragraph; page "FreeToken量子化：MoE推論のセットアップガイド", second
// paragraph).  The selection rule (fp32 logit keys, ties to the lower id, NaN
// lowest) and the softmax over the selected logits are this library's reading.
#include <algorithm>

#include "common.h"
#include "topk.h"
#include "wave.h"

namespace {

using namespace moe;

// ------------------------------------------------------------------ router logits

// Small T: one workgroup per expert, 256 threads split H; tokens in registers.
constexpr int kRouterGemvMaxT = 16;

template <int TM>  // token capacity (T <= TM)
__global__ __launch_bounds__(256) void k_router_gemv(const uint16_t* __restrict__ x, const float* __restrict__ w,
                                                     int T, int H, int E, float* __restrict__ out) {
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float acc[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) acc[t] = 0.f;
  const float* wr = w + (size_t)e * H;
  if ((H & 3) == 0) {
    // rows 16-byte (weights) and 8-byte (x) aligned: 4 values per thread and
    // chunk, kU chunks' loads issued before any of them is used
    constexpr int kU = TM >= 16 ? 2 : TM >= 4 ? 4 : 8;
    for (int h0 = 0; h0 < H; h0 += 1024 * kU) {
      float4 wv[kU];
      uint2 xv[kU][TM];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int h = min(h0 + u * 1024 + tid * 4, H - 4);  // past the end: a valid chunk, weight 0 below
        wv[u] = *reinterpret_cast<const float4*>(wr + h);
#pragma unroll
        for (int t = 0; t < TM; ++t)
          xv[u][t] = *reinterpret_cast<const uint2*>(x + (size_t)min(t, T - 1) * H + h);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (h0 + u * 1024 + tid * 4 >= H) wv[u] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int t = 0; t < TM; ++t) {
          acc[t] = fmaf(__uint_as_float(xv[u][t].x << 16), wv[u].x, acc[t]);
          acc[t] = fmaf(__uint_as_float(xv[u][t].x & 0xFFFF0000u), wv[u].y, acc[t]);
          acc[t] = fmaf(__uint_as_float(xv[u][t].y << 16), wv[u].z, acc[t]);
          acc[t] = fmaf(__uint_as_float(xv[u][t].y & 0xFFFF0000u), wv[u].w, acc[t]);
        }
      }
    }
  } else {
    for (int h = tid; h < H; h += 256) {
      const float wv = wr[h];
#pragma unroll
      for (int t = 0; t < TM; ++t) acc[t] = fmaf(bf16_to_f32(x[(size_t)min(t, T - 1) * H + h]), wv, acc[t]);
    }
  }
  __shared__ float red[4][TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    if (t < T) {
      const float v = wave_sum(acc[t]);
      if (lane == 0) red[wave][t] = v;
    }
  }
  __syncthreads();
  if (tid < T) out[(size_t)tid * E + e] = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
}

// Large T: LDS-tiled fp32 GEMM, 64 tokens x 64 experts per workgroup, K step 32.
__global__ __launch_bounds__(256) void k_router_tiled(const uint16_t* __restrict__ x, const float* __restrict__ w,
                                                      int T, int H, int E, float* __restrict__ out) {
  constexpr int BT = 64, BE = 64, BK = 32;
  __shared__ float xs[BK][BT + 4];
  __shared__ float ws[BK][BE + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int t0 = blockIdx.y * BT, e0 = blockIdx.x * BE;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < H; k0 += BK) {
    for (int i = tid; i < BT * BK; i += 256) {
      const int r = i / BK, c = i % BK, t = t0 + r, h = k0 + c;
      xs[c][r] = (t < T && h < H) ? bf16_to_f32(x[(size_t)t * H + h]) : 0.f;
    }
    for (int i = tid; i < BE * BK; i += 256) {
      const int r = i / BK, c = i % BK, e = e0 + r, h = k0 + c;
      ws[c][r] = (e < E && h < H) ? w[(size_t)e * H + h] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = ws[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) out[(size_t)t * E + e] = acc[i][j];
    }
  }
}

// Large T, H % 32 == 0: the bf16 matrix cores with the weights split into
// three bf16 parts (w = hi + lo + lo2 exactly: each part takes the next 8
// significant bits by truncation), each part's products summed in its own
// fp32 accumulator, the three sums added at the end.  x is bf16, so every
// product is exact; the error stays within fp32 summation of H terms per
// part (plus two final additions).  One wave: 32 tokens x 16 experts, the
// operands read straight from global memory (x rows and W rows, 64 bytes per
// 16-lane group per K-step of 32).
typedef __bf16 rbf16x8_t __attribute__((ext_vector_type(8)));
typedef float rf32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned ru32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void split3(const float4& a, const float4& b, rbf16x8_t& hi, rbf16x8_t& lo,
                                       rbf16x8_t& lo2) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  ru32x4_t h, l, l2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t ph = 0, pl = 0, pl2 = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float x0 = v[2 * i + j];
      const uint32_t u0 = __float_as_uint(x0) & 0xFFFF0000u;          // hi: top 16 bits
      const float r1 = x0 - __uint_as_float(u0);                        // exact
      const uint32_t u1 = __float_as_uint(r1) & 0xFFFF0000u;
      const float r2 = r1 - __uint_as_float(u1);                        // exact, <= 8 significant bits
      const uint32_t u2 = __float_as_uint(r2) & 0xFFFF0000u;            // == r2
      ph |= (u0 >> 16) << (16 * j);
      pl |= (u1 >> 16) << (16 * j);
      pl2 |= (u2 >> 16) << (16 * j);
    }
    h[i] = ph; l[i] = pl; l2[i] = pl2;
  }
  hi = __builtin_bit_cast(rbf16x8_t, h);
  lo = __builtin_bit_cast(rbf16x8_t, l);
  lo2 = __builtin_bit_cast(rbf16x8_t, l2);
}

__global__ __launch_bounds__(64) void k_router_mfma(const uint16_t* __restrict__ x, const float* __restrict__ w,
                                                    int T, int H, int E, float* __restrict__ out) {
  const int lane = threadIdx.x;
  const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 32;
  const int r = lane & 15, kc = (lane >> 4) * 8;
  // rows past T or E re-read the last one (results not stored)
  const uint16_t* xa = x + (size_t)min(t0 + r, T - 1) * H + kc;
  const uint16_t* xb = x + (size_t)min(t0 + 16 + r, T - 1) * H + kc;
  const float* wp = w + (size_t)min(e0 + r, E - 1) * H + kc;
  rf32x4_t acc[2][3];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int p = 0; p < 3; ++p) acc[i][p] = rf32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < H; k0 += 32) {
    const rbf16x8_t a0 = __builtin_bit_cast(rbf16x8_t, *reinterpret_cast<const ru32x4_t*>(xa + k0));
    const rbf16x8_t a1 = __builtin_bit_cast(rbf16x8_t, *reinterpret_cast<const ru32x4_t*>(xb + k0));
    const float4 w0 = *reinterpret_cast<const float4*>(wp + k0), w1 = *reinterpret_cast<const float4*>(wp + k0 + 4);
    rbf16x8_t b[3];
    split3(w0, w1, b[0], b[1], b[2]);
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      acc[0][p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b[p], acc[0][p], 0, 0, 0);
      acc[1][p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b[p], acc[1][p], 0, 0, 0);
    }
  }
  // lane l: expert e0 + l % 16, tokens 4 (l / 16) + v of each 16-token tile
  const int e = e0 + r;
  if (e >= E) return;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = t0 + 16 * i + 4 * (lane >> 4) + v;
      if (t < T) out[(size_t)t * E + e] = (acc[i][0][v] + acc[i][1][v]) + acc[i][2][v];
    }
}

// ------------------------------------------------------------------ top-k + softmax (wave_topk: topk.h)

template <int NPER>
__global__ __launch_bounds__(256) void k_route(const float* __restrict__ logits, int T, int E, int k, int renorm,
                                               int32_t* __restrict__ ids, float* __restrict__ wts) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  wave_topk<NPER>(logits + (size_t)t * E, E, k, renorm, ids + (size_t)t * k, wts + (size_t)t * k);
}

// ------------------------------------------------------------------ permutation
// One workgroup places a chunk of blockDim.x flat indices [c0, c0 + blockDim.x):
// from the histogram of all ids (tot) and of the ids before its chunk
// (before), it scans the totals and places its chunk: position = offsets[e] +
// (# of e before the chunk) + (# of e in earlier waves of the chunk) + (rank
// within the wave).  `ids` may point to global memory or to LDS.  LDS:
// E * (2 + waves) ints.
constexpr int kPermChunk = 1024;
constexpr int kPermWaves = kPermChunk / 64;

// Clears the LDS counters (tot, before, per-wave counts).
__device__ void permute_clear(int E, int32_t* sm) {
  const int nt = blockDim.x, nw = nt >> 6;
  for (int i = threadIdx.x; i < E * (2 + nw); i += nt) sm[i] = 0;
  __syncthreads();
}

// tot and before by counting every id (small N: one workgroup does all).
__device__ void permute_count(const int32_t* ids, int N, int E, int c0, int32_t* sm) {
  int32_t* tot = sm;
  int32_t* before = sm + E;
  for (int f = threadIdx.x; f < N; f += blockDim.x) {
    const int e = ids[f];
    if (e >= 0 && e < E) {
      atomicAdd(&tot[e], 1);
      if (f < c0) atomicAdd(&before[e], 1);
    }
  }
  __syncthreads();
}

// Scan, counts/offsets (chunk 0), and the placement of the chunk (inv too if
// `inv` is set).  tot and before must be complete.
__device__ void permute_place(const int32_t* ids, int N, int E, int c0, int32_t* sm, int32_t* __restrict__ counts,
                              int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int32_t wsum[kPermWaves];
  const int nt = blockDim.x;
  int32_t* tot = sm;                   // [E]
  int32_t* before = sm + E;            // [E]
  int32_t* wcnt = sm + 2 * E;          // [nw][E]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  {
    // exclusive scan of the totals: thread t owns experts [t*per, t*per + per);
    // a wave scan with shuffles, then the totals of the earlier waves
    const int per = (E + nt - 1) / nt;
    int run = 0;
    for (int i = 0; i < per; ++i) {
      const int e = tid * per + i;
      if (e < E) run += tot[e];
    }
    int incl = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o);
      if (lane >= o) incl += u;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int prefix = 0;
    for (int w = 0; w < wave; ++w) prefix += wsum[w];
    int base = prefix + incl - run;
    for (int i = 0; i < per; ++i) {
      const int e = tid * per + i;
      if (e < E) {
        if (c0 == 0) {
          counts[e] = tot[e];
          offsets[e] = base;
        }
        before[e] += base;
        base += tot[e];
      }
    }
    if (c0 == 0 && tid == nt - 1) offsets[E] = prefix + incl;
  }
  // rank within the wave: wave-level match of equal ids
  const int f = c0 + tid;
  const int e = f < N ? ids[f] : -1;
  const bool valid = e >= 0 && e < E;
  uint64_t todo = __ballot(valid);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rank = 0, cnt = 0;
  bool leader = false;
  while (todo) {
    const int src = __ffsll((unsigned long long)todo) - 1;
    const int key = __builtin_amdgcn_readlane(e, src);
    const uint64_t m = __ballot(valid && e == key);
    if (valid && e == key) {
      rank = __popcll(m & lt);
      cnt = __popcll(m);
      leader = lane == src;
    }
    todo &= ~m;
  }
  __syncthreads();  // before[] final
  if (leader) wcnt[wave * E + e] = cnt;
  __syncthreads();
  if (valid) {
    int pos = before[e] + rank;
    for (int w = 0; w < wave; ++w) pos += wcnt[w * E + e];
    perm[pos] = f;
    if (inv) inv[f] = pos;
  }
}

__device__ void permute_chunk(const int32_t* ids, int N, int E, int c0, int32_t* sm, int32_t* __restrict__ counts,
                              int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  permute_clear(E, sm);
  permute_count(ids, N, E, c0, sm);
  permute_place(ids, N, E, c0, sm, counts, offsets, perm, inv);
}

__global__ __launch_bounds__(1024) void k_permute(const int32_t* __restrict__ ids, int N, int E,
                                                  int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  extern __shared__ int32_t sm[];
  permute_chunk(ids, N, E, blockIdx.x * kPermChunk, sm, counts, offsets, perm, inv);
}

// Large N, E <= 256: one workgroup per expert compacts the flat indices of
// that expert in order.  Chunk j of 1024 indices is read coalesced (thread t
// takes index 1024 j + t); a ballot per (chunk, wave) counts the matches, a
// workgroup scan of those counts in index order gives each match its
// position (+ its rank among the wave's matches), and the count of (valid)
// ids below e is the expert's offset.  Both stores of a (chunk, wave) then go
// to consecutive positions and consecutive indices.  Every id is read by
// every workgroup (E * N * 4 bytes, from L2), which is why E is bounded.
constexpr int kPermExpertMaxE = 256;
constexpr int kPermExpertMaxChunks = 32;  // N <= 32768: the ids of a thread fit in registers

__global__ __launch_bounds__(1024) void k_perm_expert(const int32_t* __restrict__ ids, int N, int E,
                                                      int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int32_t cnt[kPermExpertMaxChunks * 16];  // [chunk][wave], then its exclusive scan
  __shared__ int32_t wlt[16], wsum[16];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nj = (N + 1023) >> 10;
  // every id of this thread's chunks, loaded at once (one memory latency)
  int v[kPermExpertMaxChunks];
#pragma unroll
  for (int j = 0; j < kPermExpertMaxChunks; ++j) {
    const int f = (j << 10) + tid;
    v[j] = (j < nj && f < N) ? ids[f] : -1;
  }
  int lt = 0;
#pragma unroll
  for (int j = 0; j < kPermExpertMaxChunks; ++j) {
    if (j < nj) {
      const uint64_t m = __ballot(v[j] == e);
      if (lane == 0) cnt[j * 16 + wave] = __popcll(m);
      lt += (v[j] >= 0) & (v[j] < e);
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) lt += __shfl_xor(lt, o);
  if (lane == 0) wlt[wave] = lt;
  __syncthreads();
  // exclusive scan of cnt[0 .. 16 nj): thread t owns entries 2t, 2t + 1
  const int n = nj * 16;
  const int c0 = 2 * tid < n ? cnt[2 * tid] : 0, c1 = 2 * tid + 1 < n ? cnt[2 * tid + 1] : 0;
  int inc = c0 + c1;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(inc, o);
    if (lane >= o) inc += u;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int pre = 0, total = 0, off = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    if (w < wave) pre += wsum[w];
    total += wsum[w];
    off += wlt[w];
  }
  const int ex = pre + inc - c0 - c1;
  __syncthreads();  // every count read before the scan overwrites them
  if (2 * tid < n) cnt[2 * tid] = ex;
  if (2 * tid + 1 < n) cnt[2 * tid + 1] = ex + c0;
  __syncthreads();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int j = 0; j < kPermExpertMaxChunks; ++j) {
    if (j < nj) {
      const uint64_t m = __ballot(v[j] == e);
      if (v[j] == e) {
        const int f = (j << 10) + tid;
        const int pos = off + cnt[j * 16 + wave] + __popcll(m & below);
        perm[pos] = f;
        inv[f] = pos;
      }
    }
  }
  if (tid == 0) {
    counts[e] = total;
    offsets[e] = off;
    if (e == E - 1) offsets[E] = off + total;
  }
}

// Routing and permutation of a small batch (T*k <= 1024) in one workgroup of
// at least T*k threads (one wave per token for the top-k, up to 16 waves).
template <int NPER>
__global__ __launch_bounds__(1024) void k_route_permute(const float* __restrict__ logits, int T, int E, int k,
                                                        int renorm, int32_t* __restrict__ ids, float* __restrict__ wts,
                                                        int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  extern __shared__ int32_t sm[];
  __shared__ int32_t ids_s[kPermChunk];
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __shared__ float w_s[kPermChunk];
  for (int t = wave; t < T; t += nw)
    wave_topk<NPER>(logits + (size_t)t * E, E, k, renorm, ids_s + t * k, w_s + t * k);
  __syncthreads();
  for (int f = threadIdx.x; f < T * k; f += blockDim.x) {
    ids[f] = ids_s[f];
    wts[f] = w_s[f];
  }
  permute_chunk(ids_s, T * k, E, 0, sm, counts, offsets, perm, inv);
}

// Batches of at most 64 tokens.  The k experts of one token are distinct, so
// the flat indices routed to expert e are ordered by token, and the stable
// position of (t, e) is offsets[e] + (number of earlier tokens routed to e).
// Each expert keeps a 64-bit mask of its tokens in LDS, set by the token's
// wave right after its top-k: counts are popcounts, the rank within an
// expert is the popcount of the mask below t.  Every wave scans the counts
// itself (no barrier between the scan and the placement), then places its
// own tokens.  LDS: E 64-bit masks + E ints per wave.
//
// host_counts (null: none): a host-mapped copy of the counts, after which
// the kernel publishes `seq` in the host-mapped *flag with a release at
// system scope, once every output of the kernel is written: a host that sees
// the flag may enqueue work on any stream that reads them.
template <int NPER>
__global__ __launch_bounds__(1024) void k_route_permute_small(const float* __restrict__ logits, int T, int E, int k,
                                                              int renorm, int32_t* __restrict__ ids,
                                                              float* __restrict__ wts, int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                                              int32_t* __restrict__ host_counts, uint32_t* flag,
                                                              uint32_t seq) {
  extern __shared__ uint64_t tmask[];  // [E], then int off[nw][E]
  __shared__ int32_t ids_s[64 * kRouteMaxK];
  __shared__ float w_s[64 * kRouteMaxK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  int32_t* off = reinterpret_cast<int32_t*>(tmask + E) + wave * E;
  for (int e = tid; e < E; e += blockDim.x) tmask[e] = 0ull;
  __syncthreads();
  for (int t = wave; t < T; t += nw) {
    wave_topk<NPER>(logits + (size_t)t * E, E, k, renorm, ids_s + t * k, w_s + t * k);
    if (lane < k) {  // the wave reads back its own LDS writes (in order)
      const int e = ids_s[t * k + lane];
      ids[t * k + lane] = e;
      wts[t * k + lane] = w_s[t * k + lane];
      atomicOr(reinterpret_cast<unsigned long long*>(&tmask[e]), 1ull << t);
    }
  }
  __syncthreads();
  // exclusive scan of the counts: lane l owns experts [l * per, l * per + per)
  const int per = (E + 63) / 64;
  int run = 0;
  for (int i = 0; i < per; ++i) {
    const int e = lane * per + i;
    if (e < E) run += __popcll(tmask[e]);
  }
  int incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  int base = incl - run;
  for (int i = 0; i < per; ++i) {
    const int e = lane * per + i;
    if (e < E) {
      const int c = __popcll(tmask[e]);
      off[e] = base;
      if (wave == 0) {
        counts[e] = c;
        offsets[e] = base;
        if (host_counts) host_counts[e] = c;
      }
      base += c;
    }
  }
  if (wave == 0 && lane == 63) offsets[E] = incl;
  for (int t = wave; t < T; t += nw) {
    if (lane < k) {
      const int f = t * k + lane;
      const int e = ids_s[f];
      const int pos = off[e] + (int)__popcll(tmask[e] & ((1ull << t) - 1ull));
      if (pos < T * k) {  // always true for a valid routing; keeps every store inside perm
        perm[pos] = f;
        inv[f] = pos;
      }
    }
  }
  if (host_counts) {
    __threadfence_system();
    __syncthreads();
    if (tid == 0) __hip_atomic_store(flag, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

// Threads of the one-workgroup routing + permutation: a wave per token (up to
// 16) and at least one thread per flat index.
static int route_permute_threads(int T, int k) {
  const int by_tok = 64 * std::min(T, kPermWaves);
  const int by_idx = (T * k + 63) / 64 * 64;
  return std::max(64, std::min(kPermChunk, std::max(by_tok, by_idx)));
}

// Kernels with more than 64 KiB of dynamic LDS must opt in once per process.
moe_status set_lds_limits() {
  static bool done = false;
  if (!done) {
    MOE_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(k_permute), hipFuncAttributeMaxDynamicSharedMemorySize,
                                120 * 1024));
    const void* fns[] = {reinterpret_cast<const void*>(k_route_permute<1>),
                         reinterpret_cast<const void*>(k_route_permute<2>),
                         reinterpret_cast<const void*>(k_route_permute<4>),
                         reinterpret_cast<const void*>(k_route_permute<16>)};
    const void* fns_small[] = {reinterpret_cast<const void*>(k_route_permute_small<1>),
                               reinterpret_cast<const void*>(k_route_permute_small<2>),
                               reinterpret_cast<const void*>(k_route_permute_small<4>),
                               reinterpret_cast<const void*>(k_route_permute_small<16>)};
    for (const void* f : fns) MOE_HIP(hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 120 * 1024));
    for (const void* f : fns_small)
      MOE_HIP(hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 120 * 1024));
    done = true;
  }
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_router_logits(const uint16_t* x, const float* w_router, int T, int H, int E, float* logits,
                                        moe_stream_t stream) {
  MOE_CHECK_ARG(T >= 0 && H >= 1 && E >= 1, "moe_router_logits: bad sizes T=%d H=%d E=%d", T, H, E);
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(x && w_router && logits, "moe_router_logits: null pointer");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T <= kRouterGemvMaxT) {
    if (T == 1) hipLaunchKernelGGL(k_router_gemv<1>, dim3(E), dim3(256), 0, s, x, w_router, T, H, E, logits);
    else if (T <= 4) hipLaunchKernelGGL(k_router_gemv<4>, dim3(E), dim3(256), 0, s, x, w_router, T, H, E, logits);
    else hipLaunchKernelGGL(k_router_gemv<16>, dim3(E), dim3(256), 0, s, x, w_router, T, H, E, logits);
  } else if (H % 32 == 0 && ((uintptr_t)x & 15) == 0 && ((uintptr_t)w_router & 15) == 0) {
    hipLaunchKernelGGL(k_router_mfma, dim3((E + 15) / 16, (T + 31) / 32), dim3(64), 0, s, x, w_router, T, H, E, logits);
  } else {
    hipLaunchKernelGGL(k_router_tiled, dim3((E + 63) / 64, (T + 63) / 64), dim3(256), 0, s, x, w_router, T, H, E,
                       logits);
  }
  MOE_LAUNCHED();
  return MOE_OK;
}

extern "C" moe_status moe_route(const float* logits, int T, int E, int k, int renormalize, int32_t* topk_ids,
                                float* topk_w, moe_stream_t stream) {
  MOE_CHECK_ARG(T >= 0 && E >= 1 && E <= 1024, "moe_route: bad sizes T=%d E=%d (E <= 1024)", T, E);
  MOE_CHECK_ARG(k >= 1 && k <= E && k <= kRouteMaxK, "moe_route: k=%d must be in [1, min(E, 16)]", k);
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(logits && topk_ids && topk_w, "moe_route: null pointer");
  const dim3 g((T + 3) / 4);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int rn = renormalize ? 1 : 0;
  if (E <= 64) hipLaunchKernelGGL(k_route<1>, g, dim3(256), 0, st, logits, T, E, k, rn, topk_ids, topk_w);
  else if (E <= 128) hipLaunchKernelGGL(k_route<2>, g, dim3(256), 0, st, logits, T, E, k, rn, topk_ids, topk_w);
  else if (E <= 256) hipLaunchKernelGGL(k_route<4>, g, dim3(256), 0, st, logits, T, E, k, rn, topk_ids, topk_w);
  else hipLaunchKernelGGL(k_route<16>, g, dim3(256), 0, st, logits, T, E, k, rn, topk_ids, topk_w);
  MOE_LAUNCHED();
  return MOE_OK;
}

extern "C" moe_status moe_permute(const int32_t* topk_ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                                  int32_t* perm, int32_t* inv, moe_stream_t stream) {
  MOE_CHECK_ARG(T >= 0 && k >= 1 && E >= 1 && E <= 1024, "moe_permute: bad sizes T=%d k=%d E=%d", T, k, E);
  const long long N = (long long)T * k;
  MOE_CHECK_ARG(N <= (1 << 17), "moe_permute: T*k = %lld exceeds 131072", N);
  MOE_CHECK_ARG(counts && offsets && (N == 0 || (topk_ids && perm && inv)), "moe_permute: null pointer");
  const int blocks = N == 0 ? 1 : (int)((N + kPermChunk - 1) / kPermChunk);
  const size_t lds = sizeof(int32_t) * (size_t)E * (2 + kPermWaves);
  moe_status st = set_lds_limits();
  if (st != MOE_OK) return st;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (blocks > 1 && E <= kPermExpertMaxE && blocks <= kPermExpertMaxChunks) {
    hipLaunchKernelGGL(k_perm_expert, dim3(E), dim3(1024), 0, hs, topk_ids, (int)N, E, counts, offsets, perm, inv);
  } else {
    hipLaunchKernelGGL(k_permute, dim3(blocks), dim3(kPermChunk), lds, hs, topk_ids, (int)N, E, counts, offsets,
                       perm, inv);
  }
  MOE_LAUNCHED();
  return MOE_OK;
}

extern "C" moe_status moe_route_permute(const float* logits, int T, int E, int k, int renormalize, int32_t* topk_ids,
                                        float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                        moe_stream_t stream) {
  MOE_CHECK_ARG(T >= 0 && E >= 1 && E <= 1024, "moe_route_permute: bad sizes T=%d E=%d (E <= 1024)", T, E);
  MOE_CHECK_ARG(k >= 1 && k <= E && k <= kRouteMaxK, "moe_route_permute: k=%d must be in [1, min(E, 16)]", k);
  MOE_CHECK_ARG(counts && offsets, "moe_route_permute: null pointer");
  if ((long long)T * k > kPermChunk) {
    moe_status st = moe_route(logits, T, E, k, renormalize, topk_ids, topk_w, stream);
    if (st != MOE_OK) return st;
    return moe_permute(topk_ids, T, k, E, counts, offsets, perm, inv, stream);
  }
  MOE_CHECK_ARG(T == 0 || (logits && topk_ids && topk_w && perm && inv), "moe_route_permute: null pointer");
  moe_status st = set_lds_limits();
  if (st != MOE_OK) return st;
  const int nt = route_permute_threads(T, k);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const int rn = renormalize ? 1 : 0;
  if (T >= 1 && T <= 64) {
    const int ntw = 64 * std::min(T, kPermWaves);  // a wave per token, up to 16
    const size_t lds = sizeof(uint64_t) * (size_t)E + sizeof(int32_t) * (size_t)E * (ntw / 64);
#define MOE_RPS(N) hipLaunchKernelGGL(k_route_permute_small<N>, dim3(1), dim3(ntw), lds, hs, logits, T, E, k, rn, \
                                      topk_ids, topk_w, counts, offsets, perm, inv, nullptr, nullptr, 0u)
    if (E <= 64) MOE_RPS(1);
    else if (E <= 128) MOE_RPS(2);
    else if (E <= 256) MOE_RPS(4);
    else MOE_RPS(16);
#undef MOE_RPS
  } else {
    const size_t lds = sizeof(int32_t) * (size_t)E * (2 + nt / 64);
#define MOE_RP(N) hipLaunchKernelGGL(k_route_permute<N>, dim3(1), dim3(nt), lds, hs, logits, T, E, k, rn, \
                                     topk_ids, topk_w, counts, offsets, perm, inv)
    if (E <= 64) MOE_RP(1);
    else if (E <= 128) MOE_RP(2);
    else if (E <= 256) MOE_RP(4);
    else MOE_RP(16);
#undef MOE_RP
  }
  MOE_LAUNCHED();
  return MOE_OK;
}

// moe_route_permute, then the counts copied into host_counts (host-mapped)
// and `seq` published in the host-mapped *flag (release at system scope)
// after every routing output is written.  Steps of up to 64 tokens do all of
// it in the one routing kernel; larger ones add the publishing kernel.
moe_status moe::route_permute_publish(const float* logits, int T, int E, int k, int renormalize, int32_t* topk_ids,
                                      float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                      int32_t* host_counts, uint32_t* flag, uint32_t seq, hipStream_t hs) {
  MOE_CHECK_ARG(host_counts && flag, "route_permute_publish: null host pointer");
  if (!(T >= 1 && T <= 64 && (long long)T * k <= kPermChunk && E >= 1 && E <= 1024 && k >= 1 && k <= E &&
        k <= kRouteMaxK)) {
    moe_status st = moe_route_permute(logits, T, E, k, renormalize, topk_ids, topk_w, counts, offsets, perm, inv,
                                      reinterpret_cast<moe_stream_t>(hs));
    if (st != MOE_OK) return st;
    const hipError_t e = launch_publish_counts(counts, E, host_counts, flag, seq, hs);
    if (e != hipSuccess) return set_error(MOE_EHIP, "count handoff launch failed: %s", hipGetErrorString(e));
    return MOE_OK;
  }
  MOE_CHECK_ARG(logits && topk_ids && topk_w && counts && offsets && perm && inv,
                "route_permute_publish: null pointer");
  moe_status st = set_lds_limits();
  if (st != MOE_OK) return st;
  const int rn = renormalize ? 1 : 0;
  const int ntw = 64 * std::min(T, kPermWaves);
  const size_t lds = sizeof(uint64_t) * (size_t)E + sizeof(int32_t) * (size_t)E * (ntw / 64);
#define MOE_RPS(N) hipLaunchKernelGGL(k_route_permute_small<N>, dim3(1), dim3(ntw), lds, hs, logits, T, E, k, rn, \
                                      topk_ids, topk_w, counts, offsets, perm, inv, host_counts, flag, seq)
  if (E <= 64) MOE_RPS(1);
  else if (E <= 128) MOE_RPS(2);
  else if (E <= 256) MOE_RPS(4);
  else MOE_RPS(16);
#undef MOE_RPS
  MOE_LAUNCHED();
  return MOE_OK;
}
