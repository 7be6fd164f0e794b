// Decode path of the expert FFN: a dequantising GEMV that streams every
// touched expert's packed weights from HBM once.
//
// Method: cache hits execute on the GPU (page "FreeToken量子化：MoE推論の
// セットアップガイド", decode paragraph); the expert is a SwiGLU FFN over
// MXFP4 / NVFP4 / BF16 weights (this library's reading; formats named on the
// same page, third paragraph).
//
// Two launches, neither waits for another workgroup:
//   k_gemv_gateup: work items (row block of up to 16 rows of one expert, 32
//     intermediate rows); the four waves split the K-tiles of H; h =
//     silu(g) * u is written as bf16.
//   k_gemv_down: work items (row block, 64 output columns); y in fp32.  For
//     small batches the last item of each column chunk (a per-chunk counter)
//     also performs the weighted combine of that chunk for every token, with
//     y exchanged through agent-scope (cross-XCD coherent) accesses.
// Every workgroup first compacts the active experts from the per-expert row
// counts, then walks the items with a grid stride, so the grid never carries
// workgroups for experts that received no row.
//
// Inner product: the weight tiles are decoded exactly to bf16 (E2M1 times
// its block scale) in registers and fed with up to 16 token rows to
// v_mfma_f32_16x16x32_bf16, fp32 accumulation.  The kernels remain an HBM
// stream of the packed weights; the matrix cores only replace the VALU
// dot products (with dot2 the per-row VALU work, not HBM, set the speed).
// Lane l loads row (l % 16), K-chunk (l / 16) of each 1 KiB tile, so one
// wave-wide 16-byte load is one contiguous tile.
#include "ffn_common.h"
#include "wave.h"

namespace moe {

template <int FMT>
struct Fmt;
template <>
struct Fmt<MOE_FMT_BF16> {
  static constexpr int KT = 32, SPT = 1;  // K per tile, 16x16x32 MFMA steps per tile
};
template <>
struct Fmt<MOE_FMT_MXFP4> {
  static constexpr int KT = 128, SPT = 4;
};
template <>
struct Fmt<MOE_FMT_NVFP4> {
  static constexpr int KT = 128, SPT = 4;
};

template <int FMT>
__device__ __forceinline__ uint32_t load_scale(const uint8_t* s_tiles, size_t tile, int lane) {
  if constexpr (FMT == MOE_FMT_MXFP4) return s_tiles[tile * 64 + lane];
  if constexpr (FMT == MOE_FMT_NVFP4) return *reinterpret_cast<const uint16_t*>(s_tiles + tile * 128 + 2 * lane);
  return 0u;
}

// B operand of MFMA step s (8 bf16) from a lane's tile fragment, block scale
// applied (exact: E2M1 x E8M0 and E2M1 x E4M3 both fit bf16).  For the 4-bit
// formats step s takes the lane's values 8s..8s+7 (its 32 values cover 4 steps).
template <int FMT, int S>
__device__ __forceinline__ bf16x8_t bfrag(const uint4 q, uint32_t sc) {
  if constexpr (FMT == MOE_FMT_BF16) {
    return __builtin_bit_cast(bf16x8_t, q);
  } else {
    const uint32_t d = S == 0 ? q.x : S == 1 ? q.y : S == 2 ? q.z : q.w;
    if constexpr (FMT == MOE_FMT_MXFP4) {
      const float f = e8m0_to_f32(sc & 0xFFu);  // power of two: applied exactly by the conversion
      const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, f, 0);
      const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, f, 1);
      const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, f, 2);
      const bf16x2_t e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, f, 3);
      return bf16x8_t{a.x, a.y, b.x, b.y, c.x, c.y, e.x, e.y};
    } else {
      // E4M3 scale of the 16-value block holding values 8S..8S+7
      const float f = __builtin_amdgcn_cvt_f32_fp8((int)sc, S / 2);
      bf16x8_t r;
      const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0);
      const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1);
      const f32x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2);
      const f32x2_t e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3);
      r[0] = (__bf16)(a.x * f); r[1] = (__bf16)(a.y * f);
      r[2] = (__bf16)(b.x * f); r[3] = (__bf16)(b.y * f);
      r[4] = (__bf16)(c.x * f); r[5] = (__bf16)(c.y * f);
      r[6] = (__bf16)(e.x * f); r[7] = (__bf16)(e.y * f);
      return r;
    }
  }
}

constexpr int kRing = 4;  // K-tiles of weight loads in flight per wave

template <int FMT>
__device__ __forceinline__ void tiles4_load(const uint8_t* __restrict__ wsec, const uint8_t* __restrict__ ssec, int rg0,
                                            int nk, int kt, uint4 (&q)[4], uint32_t (&sc)[4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const size_t tile = (size_t)(rg0 + j) * nk + kt;
    q[j] = ldg16(wsec + tile * kTileBytes + lane * 16);
    sc[j] = load_scale<FMT>(ssec, tile, lane);
  }
}

// Issue this wave's first kRing K-tiles (kt = wave, wave + 4, ...) of the 4
// row-groups [rg0, rg0+4).
template <int FMT>
__device__ __forceinline__ void mfma4_first(const uint8_t* __restrict__ wsec, const uint8_t* __restrict__ ssec,
                                            int rg0, int nk, uint4 (&buf)[kRing][4], uint32_t (&bsc)[kRing][4]) {
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kRing; ++i)
    if (wave + 4 * i < nk) tiles4_load<FMT>(wsec, ssec, rg0, nk, wave + 4 * i, buf[i], bsc[i]);
}

// D[m][n] += sum over this wave's K-tiles of A[m][k] W[n][k] for the 16 rows
// m of the A operand and the 64 weight rows n of row-groups [rg0, rg0+4):
// one v_mfma_f32_16x16x32_bf16 per (row-group, 32 K).  A row m (lane % 16)
// is read from LDS at arow[m] (nullptr: a zero row).  Within a 128-K tile
// of a 4-bit format the contraction index is permuted identically in A and
// B so that step s uses each lane's own values 8s..8s+7 (lane group g covers
// K 32g..32g+31 of the tile).  acc[j]: lane l holds D[4 (l/16) + v][16 j + l % 16].
template <int FMT>
__device__ __forceinline__ void mfma4_run(const uint8_t* __restrict__ wsec, const uint8_t* __restrict__ ssec, int rg0,
                                          int nk, uint4 (&buf)[kRing][4], uint32_t (&bsc)[kRing][4],
                                          const uint16_t* arow, f32x4_t (&acc)[4]) {
  using F = Fmt<FMT>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int kt0 = wave; kt0 < nk; kt0 += 4 * kRing) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      const int kt = kt0 + 4 * i;
      if (kt < nk) {
        const uint4 q[4] = {buf[i][0], buf[i][1], buf[i][2], buf[i][3]};
        const uint32_t sc[4] = {bsc[i][0], bsc[i][1], bsc[i][2], bsc[i][3]};
        if (kt + 4 * kRing < nk) tiles4_load<FMT>(wsec, ssec, rg0, nk, kt + 4 * kRing, buf[i], bsc[i]);
#pragma unroll
        for (int s = 0; s < F::SPT; ++s) {
          const int col = kt * F::KT + (F::SPT == 4 ? 32 * g + 8 * s : 8 * g);
          const uint4 av = arow ? *reinterpret_cast<const uint4*>(arow + col) : make_uint4(0, 0, 0, 0);
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            bf16x8_t b;
            if (s == 0) b = bfrag<FMT, 0>(q[j], sc[j]);
            else if (s == 1) b = bfrag<FMT, 1>(q[j], sc[j]);
            else if (s == 2) b = bfrag<FMT, 2>(q[j], sc[j]);
            else b = bfrag<FMT, 3>(q[j], sc[j]);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
          }
        }
      }
    }
  }
}

// The active experts of a call, compacted in LDS by every workgroup with one
// round of global loads: active expert a (ascending expert id among experts
// with rows and an enabled mask; the shared expert last) has rows cnt[a],
// first perm-order row p0[a], slot slot[a] (-1: shared) and row blocks of
// `rbs` rows numbered [rb[a], rb[a+1]).  tok[p] caches perm[p] / k.
constexpr int kTokCache = 1024;
struct ActiveLds {
  int cnt[kMaxActive], p0[kMaxActive], slot[kMaxActive], rb[kMaxActive + 1];
  int tok[kTokCache];
  int n;
};

__device__ inline void build_active(const FfnParams& P, int rbs, ActiveLds& A) {
  const int tid = threadIdx.x;
  const int N = P.T * P.k;
  if (N <= kTokCache)
    for (int p = tid; p < N; p += 256) A.tok[p] = P.perm[p] / P.k;
  if (tid < 64) {
    int seen = 0, rbrun = 0;
    const uint64_t lt = (tid == 0) ? 0ull : (~0ull >> (64 - tid));
    for (int base = 0; base < P.E; base += 64) {
      const int e = base + tid;
      int c = 0, off = 0, sl = 0;
      if (e < P.E) {
        c = P.counts[e];
        off = P.offsets[e];
        sl = P.slot_of_expert[e];
        if (P.mask != nullptr && P.mask[e] == 0) c = 0;
      }
      const uint64_t b = __ballot(c > 0);
      const int at = seen + __popcll(b & lt);
      int nb = (c + rbs - 1) / rbs;  // inclusive scan of row blocks
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(nb, o);
        if (tid >= o) nb += u;
      }
      if (c > 0) {
        A.cnt[at] = c;
        A.p0[at] = off;
        A.slot[at] = sl;
        A.rb[at + 1] = rbrun + nb;
      }
      rbrun += __shfl(nb, 63);
      seen += __popcll(b);
    }
    if (tid == 0) {
      A.rb[0] = 0;
      int n = seen;
      if (P.shared_blob) {
        A.cnt[n] = P.T;
        A.p0[n] = P.T * P.k;
        A.slot[n] = -1;
        A.rb[n + 1] = rbrun + (P.T + rbs - 1) / rbs;
        ++n;
      }
      A.n = n;
    }
  }
  __syncthreads();
}

// Work item of one row block: which expert, which rows.
struct RowBlock {
  const uint8_t* blob;
  int p0;      // perm-order index of the expert's first row
  int r0;      // first row of the block within the expert
  int nr;      // rows in the block (<= 16)
  int shared;
};

__device__ inline RowBlock row_block(const FfnParams& P, const ActiveLds& A, int rbs, int rb) {
  int lo = 0, hi = A.n - 1;  // active expert a with rb[a] <= rb < rb[a+1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (A.rb[mid] <= rb) lo = mid; else hi = mid - 1;
  }
  RowBlock b;
  b.r0 = (rb - A.rb[lo]) * rbs;
  b.nr = min(rbs, A.cnt[lo] - b.r0);
  b.p0 = A.p0[lo];
  b.shared = A.slot[lo] < 0;
  b.blob = b.shared ? P.shared_blob : P.slot_pool + (size_t)A.slot[lo] * P.slot_stride;
  return b;
}

__device__ __forceinline__ int row_token(const FfnParams& P, const ActiveLds& A, const RowBlock& b, int r) {
  if (b.shared) return b.r0 + r;
  const int p = b.p0 + b.r0 + r;
  return P.T * P.k <= kTokCache ? A.tok[p] : P.perm[p] / P.k;
}

struct GemvArgs {
  uint16_t* h;          // [R][I] bf16
  float* y;             // [R][H] fp32
  GemvSync* sync;
  const float* topk_w;  // fused combine (nullable)
  const int32_t* inv;
  uint16_t* out;
  int ng, nd;           // gate/up and down column chunks per expert
  int rbs1, rbs2;       // rows per row block (<= 16) of the two launches
  int x_all;            // 1: every token's x row is staged once per workgroup
  int x_bytes;          // LDS bytes of those rows (16-byte multiple)
};

// Sum the four waves' partial 16 x 64 outputs: red[j][m][n] (floats, LDS).
__device__ __forceinline__ void reduce_waves(const f32x4_t (&acc)[4], float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // red layout [wave][j][m][n] (4 x 4 x 16 x 16)
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[((wave * 4 + j) * 16 + 4 * (lane >> 4) + v) * 16 + (lane & 15)] = acc[j][v];
  __syncthreads();
}

__device__ __forceinline__ float red_sum(const float* red, int j, int m, int n) {
  return red[((0 * 4 + j) * 16 + m) * 16 + n] + red[((1 * 4 + j) * 16 + m) * 16 + n] +
         red[((2 * 4 + j) * 16 + m) * 16 + n] + red[((3 * 4 + j) * 16 + m) * 16 + n];
}

constexpr int kRedFloats = 4 * 4 * 16 * 16;

// Gate/up + SwiGLU.  Items (row block, chunk of 32 intermediate rows), chunk
// fastest; workgroup b takes items b, b + grid, ...
template <int FMT>
__global__ __launch_bounds__(256) void k_gemv_gateup(FfnParams P, GemvArgs G) {
  using F = Fmt<FMT>;
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ ActiveLds A;
  const int tid = threadIdx.x, lane = tid & 63;
  const int H = P.H, I = P.I, nk = H / F::KT, Hp = H + 8, rbs = G.rbs1;
  // act: [rows][H + 8] bf16.  red (the cross-wave sums) follows the rows of
  // every token, or else reuses the rows of the item once the MFMAs are done.
  uint16_t* act = reinterpret_cast<uint16_t*>(lds);
  float* red = reinterpret_cast<float*>(lds + (G.x_all ? G.x_bytes : 0));
  build_active(P, rbs, A);
  if (G.x_all) {
    for (int i = tid * 8; i < P.T * H; i += 256 * 8) {
      const int t = i / H, c = i % H;
      *reinterpret_cast<uint4*>(act + (size_t)t * Hp + c) = *reinterpret_cast<const uint4*>(P.x + (size_t)t * H + c);
    }
    __syncthreads();
  }
  const int items = A.rb[A.n] * G.ng;
#pragma unroll 1
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int chunk = it % G.ng, rb = it / G.ng;
    const RowBlock blk = row_block(P, A, rbs, rb);
    const BlobView bv = blob_view(blk.blob, P.L);
    const int rg0 = 4 * chunk;  // row-groups g_{2c}, u_{2c}, g_{2c+1}, u_{2c+1}
    uint4 buf[kRing][4];
    uint32_t bsc[kRing][4];
    mfma4_first<FMT>(bv.w13, bv.s13, rg0, nk, buf, bsc);
    if (!G.x_all) {
      for (int i = tid * 8; i < blk.nr * H; i += 256 * 8) {
        const int r = i / H, c = i % H;
        *reinterpret_cast<uint4*>(act + (size_t)r * Hp + c) =
            *reinterpret_cast<const uint4*>(P.x + (size_t)row_token(P, A, blk, r) * H + c);
      }
      __syncthreads();
    }
    const int m = lane & 15;
    const uint16_t* arow = nullptr;
    if (m < blk.nr) arow = act + (size_t)(G.x_all ? row_token(P, A, blk, m) : m) * Hp;
    f32x4_t acc[4];
    mfma4_run<FMT>(bv.w13, bv.s13, rg0, nk, buf, bsc, arow, acc);
    if (!G.x_all) __syncthreads();  // red overwrites the item's rows
    reduce_waves(acc, red);
    for (int idx = tid; idx < 2 * 16 * 16; idx += 256) {  // (pair, row, column)
      const int n = idx & 15, mm = (idx >> 4) & 15, pp = idx >> 8;
      if (mm < blk.nr) {
        const float g = red_sum(red, 2 * pp, mm, n) * bv.g_gate, u = red_sum(red, 2 * pp + 1, mm, n) * bv.g_up;
        G.h[(size_t)(blk.p0 + blk.r0 + mm) * I + 32 * chunk + 16 * pp + n] = f32_to_bf16_rne(silu_f32(g) * u);
      }
    }
    __syncthreads();
  }
}

// Down projection.  Items (row block, chunk of 64 output columns).  With a
// fused combine, the last item of a column chunk (over all row blocks) sums
// that chunk for every token; y is then exchanged through agent-scope
// (cross-XCD coherent) accesses and a per-chunk counter.
template <int FMT>
__global__ __launch_bounds__(256) void k_gemv_down(FfnParams P, GemvArgs G) {
  using F = Fmt<FMT>;
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ ActiveLds A;
  __shared__ int s_flag;
  const int tid = threadIdx.x, lane = tid & 63;
  const int H = P.H, I = P.I, nk = I / F::KT, Ip = I + 8, rbs = G.rbs2;
  uint16_t* act = reinterpret_cast<uint16_t*>(lds);  // [rows][I + 8] bf16
  float* red = reinterpret_cast<float*>(lds);        // reuses act after the MFMAs
  build_active(P, rbs, A);
  const int nrb = A.rb[A.n];
  const int items = nrb * G.nd;
  const bool fuse = G.out != nullptr;
#pragma unroll 1
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int chunk = it % G.nd, rb = it / G.nd;
    const RowBlock blk = row_block(P, A, rbs, rb);
    const BlobView bv = blob_view(blk.blob, P.L);
    const int rg0 = 4 * chunk;  // output columns [64 chunk, 64 chunk + 64)
    uint4 buf[kRing][4];
    uint32_t bsc[kRing][4];
    mfma4_first<FMT>(bv.w2, bv.s2, rg0, nk, buf, bsc);
    for (int i = tid * 8; i < blk.nr * I; i += 256 * 8) {
      const int r = i / I, c = i % I;
      *reinterpret_cast<uint4*>(act + (size_t)r * Ip + c) =
          *reinterpret_cast<const uint4*>(G.h + (size_t)(blk.p0 + blk.r0 + r) * I + c);
    }
    __syncthreads();
    const int m = lane & 15;
    const uint16_t* arow = m < blk.nr ? act + (size_t)m * Ip : nullptr;
    f32x4_t acc[4];
    mfma4_run<FMT>(bv.w2, bv.s2, rg0, nk, buf, bsc, arow, acc);
    __syncthreads();  // red overwrites the item's rows
    reduce_waves(acc, red);
    for (int idx = tid; idx < 4 * 16 * 16; idx += 256) {  // (row group, row, column)
      const int n = idx & 15, mm = (idx >> 4) & 15, j = idx >> 8;
      if (mm < blk.nr) {
        const float v = red_sum(red, j, mm, n) * bv.g_down;
        float* dst = G.y + (size_t)(blk.p0 + blk.r0 + mm) * H + 64 * chunk + 16 * j + n;
        if (fuse) __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else *dst = v;
      }
    }
    if (fuse) {
      __builtin_amdgcn_s_waitcnt(0);  // this thread's y stores have completed
      __syncthreads();
      if (tid == 0) {
        const unsigned q = __hip_atomic_fetch_add(&G.sync->dn_done[chunk], 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        s_flag = q == (unsigned)nrb - 1;
      }
      __syncthreads();
      if (s_flag) {
        // Last row block of this 64-column chunk: combine it for every token.
        const int T = P.T, k = P.k;
        const float* ysh = P.shared_blob ? G.y + (size_t)T * k * H : nullptr;
        for (int idx = tid; idx < T * 64; idx += 256) {
          const int t = idx >> 6, c = 64 * chunk + (idx & 63);
          float sum = 0.f;
          for (int j = 0; j < k; ++j)
            sum = fmaf(G.topk_w[(size_t)t * k + j],
                       __hip_atomic_load(G.y + (size_t)G.inv[(size_t)t * k + j] * H + c, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT),
                       sum);
          if (ysh) sum += __hip_atomic_load(ysh + (size_t)t * H + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          G.out[(size_t)t * H + c] = f32_to_bf16_rne(sum);
        }
        if (tid == 0) __hip_atomic_store(&G.sync->dn_done[chunk], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- launcher

static int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    n = cus;
  }
  return n;
}

// Dynamic LDS per workgroup: with the static part (about 21 KB) two
// workgroups fit one CU's 160 KB.
constexpr size_t kDynLds = 58 * 1024;
constexpr size_t kRedBytes = (size_t)kRedFloats * 4;

template <int FMT>
static hipError_t launch_fmt(const FfnParams& P, GemvArgs G, hipStream_t s) {
  const size_t rowb1 = (size_t)(P.H + 8) * 2, rowb2 = (size_t)(P.I + 8) * 2;
  G.rbs1 = (int)std::min<size_t>(16, kDynLds / rowb1);
  G.rbs2 = (int)std::min<size_t>(16, kDynLds / rowb2);
  G.x_bytes = (int)(((size_t)P.T * rowb1 + 15) / 16 * 16);
  G.x_all = (size_t)G.x_bytes + kRedBytes <= kDynLds ? 1 : 0;
  const size_t lds1 = G.x_all ? (size_t)G.x_bytes + kRedBytes : std::max(kRedBytes, G.rbs1 * rowb1);
  const size_t lds2 = std::max(kRedBytes, G.rbs2 * rowb2);
  // Row blocks: at most ceil(T*k / rbs) + min(E, T*k) routed, plus the shared expert's.
  auto nrb = [&](int rbs) {
    const long long rows = (long long)P.T * P.k;
    long long n = (rows + rbs - 1) / rbs + std::min<long long>(P.E, rows);
    if (P.shared_blob) n += (P.T + rbs - 1) / rbs;
    return n;
  };
  const long long cap = 2ll * cu_count();
  const int g1 = (int)std::min<long long>(nrb(G.rbs1) * G.ng, cap);
  const int g2 = (int)std::min<long long>(nrb(G.rbs2) * G.nd, cap);
  hipLaunchKernelGGL((k_gemv_gateup<FMT>), dim3(g1), dim3(256), lds1, s, P, G);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemv_down<FMT>), dim3(g2), dim3(256), lds2, s, P, G);
  return hipGetLastError();
}

static hipError_t set_gemv_lds_limits() {
  static bool done = false;
  if (!done) {
    const void* fns[] = {
        reinterpret_cast<const void*>(k_gemv_gateup<MOE_FMT_BF16>), reinterpret_cast<const void*>(k_gemv_down<MOE_FMT_BF16>),
        reinterpret_cast<const void*>(k_gemv_gateup<MOE_FMT_MXFP4>), reinterpret_cast<const void*>(k_gemv_down<MOE_FMT_MXFP4>),
        reinterpret_cast<const void*>(k_gemv_gateup<MOE_FMT_NVFP4>), reinterpret_cast<const void*>(k_gemv_down<MOE_FMT_NVFP4>)};
    for (const void* f : fns) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDynLds);
      if (e != hipSuccess) return e;
    }
    done = true;
  }
  return hipSuccess;
}

hipError_t launch_gemv(const FfnParams& P, const GemvArgs& G, hipStream_t s) {
  hipError_t e = set_gemv_lds_limits();
  if (e != hipSuccess) return e;
  switch (P.fmt) {
    case MOE_FMT_BF16: return launch_fmt<MOE_FMT_BF16>(P, G, s);
    case MOE_FMT_MXFP4: return launch_fmt<MOE_FMT_MXFP4>(P, G, s);
    case MOE_FMT_NVFP4: return launch_fmt<MOE_FMT_NVFP4>(P, G, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
