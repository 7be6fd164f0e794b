// Decode path of the expert FFN: a dequantising GEMV that streams every
// touched expert's packed weights from HBM once.
//
// Method: cache hits execute on the GPU (page "FreeToken量子化：MoE推論の
// セットアップガイド", decode paragraph); the expert is a SwiGLU FFN over
// MXFP4 / NVFP4 / BF16 weights (this library's reading; formats named on the
// same page, third paragraph).
//
// Two launches of one kernel template (k_gemv), neither waits for another
// workgroup: gate/up + SwiGLU (h in bf16), then the down projection (y in
// fp32; for small batches it also performs the weighted combine).  Every
// workgroup first compacts the active experts from the per-expert row
// counts, so the grid never carries work for experts without rows.
//
// Inner product: the weight tiles are decoded exactly (E2M1 times its block
// scale; bf16 for MXFP4 and BF16 weights, fp16 for NVFP4) in registers and
// fed with up to 16 token rows to the 16x16x32 matrix-core instruction of
// that type, fp32 accumulation.  The kernels remain an HBM
// stream of the packed weights; the matrix cores only replace the VALU
// dot products (with dot2 the per-row VALU work, not HBM, set the speed).
// Lane l loads row (l % 16), K-chunk (l / 16) of each 1 KiB tile, so one
// wave-wide 16-byte load is one contiguous tile.
#include "ffn_common.h"
#include "wave.h"

namespace moe {

template <int FMT>
struct Fmt;
// KT: K per tile; SPT: 16x16x32 MFMA steps per tile; F16: operands in fp16
// (NVFP4) rather than bf16.
template <>
struct Fmt<MOE_FMT_BF16> {
  static constexpr int KT = 32, SPT = 1;
  static constexpr bool F16 = false;
  using V = bf16x8_t;
};
template <>
struct Fmt<MOE_FMT_MXFP4> {
  static constexpr int KT = 128, SPT = 4;
  static constexpr bool F16 = false;
  using V = bf16x8_t;
};
template <>
struct Fmt<MOE_FMT_NVFP4> {
  static constexpr int KT = 128, SPT = 4;
  static constexpr bool F16 = true;
  using V = f16x8_t;
};

template <int FMT>
__device__ __forceinline__ f32x4_t mma(typename Fmt<FMT>::V a, typename Fmt<FMT>::V b, f32x4_t c) {
  if constexpr (Fmt<FMT>::F16) return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Scale bytes per tile and per lane of each format (none for BF16).
template <int FMT>
constexpr int kScaleTileBytes = FMT == MOE_FMT_MXFP4 ? 64 : FMT == MOE_FMT_NVFP4 ? 128 : 0;
template <int FMT>
constexpr int kScaleLaneBytes = FMT == MOE_FMT_MXFP4 ? 1 : FMT == MOE_FMT_NVFP4 ? 2 : 0;

// A lane's scale bytes of one tile (p already offset to the lane).
template <int FMT>
__device__ __forceinline__ uint32_t load_scale_at(const uint8_t* p) {
  if constexpr (FMT == MOE_FMT_MXFP4) return *p;
  if constexpr (FMT == MOE_FMT_NVFP4) return *reinterpret_cast<const uint16_t*>(p);
  return 0u;
}

// B operand of MFMA step s (8 values) from a lane's tile fragment, block
// scale applied exactly: E2M1 x E8M0 in bf16 (the conversion applies the
// power of two); E2M1 x E4M3 in fp16, where the product (at most 5
// significant bits, magnitude in [2^-10, 2688]) is exact, so one packed
// fp16 multiply applies the scale.  For the 4-bit formats step s takes the
// lane's values 8s..8s+7 (its 32 values cover 4 steps).
template <int FMT, int S>
__device__ __forceinline__ typename Fmt<FMT>::V bfrag(const uint4 q, uint32_t sc) {
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
      // E4M3 scale of the 16-value block holding values 8S..8S+7 (exact in fp16)
      const _Float16 f = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)sc, S / 2);
      const f16x2_t ff = {f, f};
      const f16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0) * ff;
      const f16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1) * ff;
      const f16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2) * ff;
      const f16x2_t e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3) * ff;
      return f16x8_t{a.x, a.y, b.x, b.y, c.x, c.y, e.x, e.y};
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
  if (tid >= 64) {
    if (N <= kTokCache)
      for (int p = tid - 64; p < N; p += 192) A.tok[p] = P.perm[p] / P.k;
  } else {
    // every load first (one round trip), then the compaction
    constexpr int kPer = 1024 / 64;
    int c[kPer], off[kPer], sl[kPer], mk[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = 64 * i + tid;
      c[i] = 0;
      off[i] = 0;
      sl[i] = 0;
      mk[i] = 1;
      if (e < P.E) {
        c[i] = P.counts[e];
        off[i] = P.offsets[e];
        sl[i] = P.slot_of_expert[e];
        if (P.mask != nullptr) mk[i] = P.mask[e];
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (mk[i] == 0) c[i] = 0;
    int seen = 0, rbrun = 0;
    const uint64_t lt = (tid == 0) ? 0ull : (~0ull >> (64 - tid));
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (64 * i >= P.E) break;
      const uint64_t b = __ballot(c[i] > 0);
      const int at = seen + __popcll(b & lt);
      int nb = (c[i] + rbs - 1) / rbs;  // inclusive scan of row blocks
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(nb, o);
        if (tid >= o) nb += u;
      }
      if (c[i] > 0) {
        A.cnt[at] = c[i];
        A.p0[at] = off[i];
        A.slot[at] = sl[i];
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
  lds_barrier();
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
  int ng, nd;           // gate/up and down column chunks per expert
  int rbs1, rbs2;       // rows per row block (<= 16) of the two launches
  int x_all;            // 1: every token's x row is staged once per workgroup
  int x_bytes;          // LDS bytes of those rows (16-byte multiple)
  float* trash;         // 1 MiB of scratch: stores of padding rows land here
};

constexpr int kMaxStagedRows = 256;

// Copy nr rows of K bf16 values (row r at rowptr(r)) into LDS with row stride
// Kp.  For the fp16 operand path the rows are then rewritten in place as
// fp16 of value * 2^-pexp[r], with pexp[r] >= 0 the smallest shift that keeps
// the row's largest magnitude below 2^15 (inside fp16's range; the output
// rows are multiplied back by 2^pexp[r]).  bf16 -> fp16 is then exact for
// every value of magnitude >= 2^-14 * 2^pexp[r]; smaller ones round at
// 2^-24 * 2^pexp[r], far below the row's largest product.  Ends with a barrier.
template <bool F16, class RowPtr>
__device__ __forceinline__ void stage_rows(uint16_t* act, int Kp, int K, int nr, RowPtr rowptr, int* pexp,
                                           unsigned* rmax) {
  const int tid = threadIdx.x;
  if constexpr (F16) {
    for (int r = tid; r < nr; r += 256) rmax[r] = 0u;
    lds_barrier();
  }
  for (int i = tid * 8; i < nr * K; i += 256 * 8) {
    const int r = i / K, c = i % K;
    const uint4 v = *reinterpret_cast<const uint4*>(rowptr(r) + c);
    *reinterpret_cast<uint4*>(act + (size_t)r * Kp + c) = v;
    if constexpr (F16) {
      uint32_t m = max(max(v.x & 0x7FFFu, v.x >> 16 & 0x7FFFu), max(v.y & 0x7FFFu, v.y >> 16 & 0x7FFFu));
      m = max(m, max(max(v.z & 0x7FFFu, v.z >> 16 & 0x7FFFu), max(v.w & 0x7FFFu, v.w >> 16 & 0x7FFFu)));
      atomicMax(&rmax[r], m);  // |bf16| bit patterns order like the magnitudes
    }
  }
  lds_barrier();
  if constexpr (F16) {
    for (int r = tid; r < nr; r += 256) {
      const int E = (int)(rmax[r] >> 7);  // biased exponent of the row's largest |value|: it is < 2^(E-126)
      pexp[r] = (E == 0xFF) ? 0 : max(0, E - 141);
    }
    lds_barrier();
    for (int i = tid * 8; i < nr * K; i += 256 * 8) {
      const int r = i / K, c = i % K;
      uint4* p = reinterpret_cast<uint4*>(act + (size_t)r * Kp + c);
      const uint4 v = *p;
      const float sc = __uint_as_float((uint32_t)(127 - pexp[r]) << 23);
      auto cv = [&](uint32_t w) -> uint32_t {
        const f16x2_t h = {(_Float16)(bf16_to_f32((uint16_t)w) * sc), (_Float16)(bf16_to_f32((uint16_t)(w >> 16)) * sc)};
        return __builtin_bit_cast(uint32_t, h);
      };
      *p = make_uint4(cv(v.x), cv(v.y), cv(v.z), cv(v.w));
    }
    lds_barrier();
  }
}

// 2^p as a float (0 <= p < 128)
__device__ __forceinline__ float pow2i(int p) { return __uint_as_float((uint32_t)(127 + p) << 23); }

// A float the compiler cannot see is uniform: loads from `p + opaque_zero()`
// are vector-memory loads, ordered with the weight loads, rather than scalar
// loads (whose counter the LDS reads share).
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

constexpr int kTrashSlots = 256;         // 4 KiB scratch slots (workgroup index modulo this)

// One projection of the decode path.
//   DOWN = false: gate/up + SwiGLU.  Item (row block, c) covers intermediate
//     rows [32c, 32c + 32): wave w streams row group 4c + w of W13 (waves 0
//     and 2 gate, 1 and 3 up); the up waves hand their 16 x 16 outputs to the
//     gate waves through LDS, which write h = silu(g) * u as bf16.
//   DOWN = true: down projection.  Item (row block, c) covers output columns
//     [64c, 64c + 64): wave w streams row group 4c + w of W2 and writes its 16
//     columns of y (fp32).
// Items are numbered with c fastest; workgroup b takes the contiguous range
// [b*items/grid, (b+1)*items/grid), so consecutive items mostly share a row
// block and its staged operand rows.  Each wave runs all K-tiles of its row
// group itself (no cross-wave reduction), in sub-items of SUB K-tiles (SUB
// divides K / KT); the loads of the next sub-item are in flight while the
// current one computes, also across items.
template <int FMT, bool DOWN, int SUB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemv(FfnParams P, GemvArgs G) {
  using F = Fmt<FMT>;
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ ActiveLds A;
  __shared__ int s_pexp[DOWN ? 16 : kMaxStagedRows];
  __shared__ unsigned s_rmax[DOWN ? 16 : kMaxStagedRows];
  __shared__ float s_u[2][16][17];
  __shared__ float s_g[2];  // per-tensor multipliers of the staged row block's expert
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, m = lane & 15, grp = lane >> 4;
  const int H = P.H, I = P.I;
  const int K = DOWN ? I : H, Kp = K + 8, nk = K / F::KT;
  const int rbs = DOWN ? G.rbs2 : G.rbs1, nchunk = DOWN ? G.nd : G.ng;
  const bool x_all = !DOWN && G.x_all;
  uint16_t* act = reinterpret_cast<uint16_t*>(lds);  // [rows][K + 8] operand rows
  build_active(P, rbs, A);
  const int nrb = A.rb[A.n];
  const int items = nrb * nchunk;
  const int i0 = (int)((long long)items * blockIdx.x / gridDim.x);
  const int i1 = (int)((long long)items * (blockIdx.x + 1) / gridDim.x);
  const int nsub = nk / SUB;  // SUB divides nk: every sub-item loads exactly SUB tiles
  const int nS = (i1 - i0) * nsub;
  const size_t off_w = DOWN ? P.L.off_w2 : P.L.off_w13, off_s = DOWN ? P.L.off_s2 : P.L.off_s13;

  // Loads and stores are unconditional and fixed in number per sub-item (the
  // compiler then counts them exactly and waits only for the bank in use).
  auto issue = [&](int ss, uint4 (&q)[SUB], uint32_t (&sc)[SUB]) {
    const int it = i0 + ss / nsub, sub = ss % nsub;
    const RowBlock blk = row_block(P, A, rbs, it / nchunk);
    const int rg = 4 * (it % nchunk) + wave, kt0 = sub * SUB;
    // 32-bit tile index (a blob holds far fewer than 2^31 tiles); per-tile
    // addresses are then constant offsets from two base pointers, so no
    // 64-bit arithmetic sits between the loads.
    const uint32_t t0 = (uint32_t)rg * (uint32_t)nk + (uint32_t)kt0;
    const uint8_t* wp = blk.blob + off_w + ((size_t)t0 << 10) + lane * 16;
    const uint8_t* sp = blk.blob + off_s + (size_t)t0 * kScaleTileBytes<FMT> + lane * kScaleLaneBytes<FMT>;
#pragma unroll
    for (int j = 0; j < SUB; ++j) {
      q[j] = ldg16(wp + j * kTileBytes);
      sc[j] = load_scale_at<FMT>(sp + j * kScaleTileBytes<FMT>);
    }
  };

  int staged = -1;
  // On a new row block: its expert's per-tensor multipliers, and its operand
  // rows (all T token rows once, if they fit).  The multipliers' load is in
  // flight together with the rows'.
  auto prepare = [&](int ss) {
    const int rb = (i0 + ss / nsub) / nchunk;
    if (rb == staged) return;  // uniform: every wave walks the same sub-items
    const RowBlock blk = row_block(P, A, rbs, rb);
    float gv = 0.f;
    if (tid < (DOWN ? 1 : 2)) gv = reinterpret_cast<const BlobHeader*>(blk.blob)->g[DOWN ? 2 : tid];
    lds_barrier();  // the previous block's rows and multipliers are no longer read
    if (x_all) {
      if (staged < 0)
        stage_rows<F::F16>(act, Kp, K, P.T, [&](int t) { return P.x + (size_t)t * H; }, s_pexp, s_rmax);
    } else if constexpr (DOWN) {
      stage_rows<F::F16>(act, Kp, K, blk.nr, [&](int r) { return G.h + (size_t)(blk.p0 + blk.r0 + r) * I; }, s_pexp,
                         s_rmax);
    } else {
      stage_rows<F::F16>(act, Kp, K, blk.nr, [&](int r) { return P.x + (size_t)row_token(P, A, blk, r) * H; },
                         s_pexp, s_rmax);
    }
    if (tid < (DOWN ? 1 : 2)) s_g[tid] = gv;
    lds_barrier();
    staged = rb;
  };

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  // The epilogue runs after every sub-item (uniform code: no branch around
  // memory operations inside the pipelined loop); before an item's last
  // sub-item its stores go to a scratch area, as do rows past the block and
  // the up waves' h.
  // this workgroup's own 4 KiB of scratch (distinct lines: no store contention)
  float* trash = G.trash + (size_t)(blockIdx.x % kTrashSlots) * 1024;
  auto body = [&](int ss, const uint4 (&q)[SUB], const uint32_t (&sc)[SUB]) {
    const int it = i0 + ss / nsub, sub = ss % nsub;
    const int chunk = it % nchunk;
    const bool last = sub == nsub - 1;
    const RowBlock blk = row_block(P, A, rbs, it / nchunk);
    if (sub == 0) acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // x_all implies T*k <= kTokCache: tokens come from LDS (no global load
    // may sit inside the pipelined loop body)
    auto tok = [&](int r) { return blk.shared ? blk.r0 + r : A.tok[blk.p0 + blk.r0 + r]; };
    const uint16_t* arow = nullptr;
    if (m < blk.nr) arow = act + (size_t)(x_all ? tok(m) : m) * Kp;
#pragma unroll
    for (int j = 0; j < SUB; ++j) {
      const int kt = sub * SUB + j;
#pragma unroll
      for (int st = 0; st < F::SPT; ++st) {
        const int col = kt * F::KT + (F::SPT == 4 ? 32 * grp + 8 * st : 8 * grp);
        const uint4 av = arow ? *reinterpret_cast<const uint4*>(arow + col) : make_uint4(0, 0, 0, 0);
        typename F::V b;
        if constexpr (F::SPT == 4) {
          b = st == 0 ? bfrag<FMT, 0>(q[j], sc[j]) : st == 1 ? bfrag<FMT, 1>(q[j], sc[j])
            : st == 2 ? bfrag<FMT, 2>(q[j], sc[j]) : bfrag<FMT, 3>(q[j], sc[j]);
        } else {
          b = bfrag<FMT, 0>(q[j], sc[j]);
        }
        acc = mma<FMT>(__builtin_bit_cast(typename F::V, av), b, acc);
      }
    }
    // Lane: rows 4 (lane / 16) + v of the block, column lane % 16 of this
    // wave's 16 output rows of the weight; per-tensor multiplier of those
    // rows: gate (even waves) / up (odd) / down.
    const float g = s_g[DOWN ? 0 : (wave & 1)];
    float val[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = 4 * grp + v;
      float sc2 = g;
      if constexpr (F::F16) sc2 *= pow2i(s_pexp[r < blk.nr ? (x_all ? tok(r) : r) : 0]);
      val[v] = acc[v] * sc2;
    }
    if constexpr (DOWN) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 4 * grp + v;
        float* dst = (last && r < blk.nr) ? G.y + (size_t)(blk.p0 + blk.r0 + r) * H + 64 * chunk + 16 * wave + m
                                          : trash + (r * 4 + wave) * 16 + m;
        *dst = val[v];
      }
    } else {
      if (wave & 1)
#pragma unroll
        for (int v = 0; v < 4; ++v) s_u[wave >> 1][4 * grp + v][m] = val[v];
      lds_barrier();
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 4 * grp + v;
        const float hv = silu_f32(val[v]) * s_u[wave >> 1][r][m];
        uint16_t* dst = (last && r < blk.nr && !(wave & 1))
                            ? G.h + (size_t)(blk.p0 + blk.r0 + r) * I + 32 * chunk + 16 * (wave >> 1) + m
                            : reinterpret_cast<uint16_t*>(trash) + (r * 4 + wave) * 16 + m;
        *dst = f32_to_bf16_rne(hv);
      }
      lds_barrier();
    }
  };

  // Software pipeline: the loads of sub-item ss + 1 are issued before
  // sub-item ss computes and are consumed in the next iteration (a
  // loop-carried bank, so the compiler keeps them in flight).  The issue is
  // unconditional (the last iteration re-reads its own sub-item, from cache).
  uint4 cq[SUB], nq[SUB];
  uint32_t cs[SUB], ns[SUB];
  if (nS > 0) issue(0, cq, cs);
#pragma unroll 1
  for (int ss = 0; ss < nS; ++ss) {
    prepare(ss);
    issue(min(ss + 1, nS - 1), nq, ns);
    __builtin_amdgcn_sched_barrier(0);
    body(ss, cq, cs);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < SUB; ++j) {
      cq[j] = nq[j];
      cs[j] = ns[j];
    }
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

// Resident workgroups of 256 threads per CU for a kernel and its dynamic LDS
// (at least 1), memoised.
static int blocks_per_cu(const void* fn, size_t lds) {
  static const void* fns[16];
  static size_t ldss[16];
  static int vals[16];
  static int n = 0;
  for (int i = 0; i < n; ++i)
    if (fns[i] == fn && ldss[i] == lds) return vals[i];
  int b = 1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, fn, 256, lds) != hipSuccess || b < 1) b = 1;
  if (n < 16) {
    fns[n] = fn;
    ldss[n] = lds;
    vals[n] = b;
    ++n;
  }
  return b;
}

// Dynamic LDS per workgroup: with the static part (at most 25 KB) two
// workgroups fit one CU's 160 KB.
constexpr size_t kDynLds = 55 * 1024;

typedef void (*GemvKernel)(FfnParams, GemvArgs);

// Sub-item size: the largest of 16 (only when it is all of K), 8, 6, 4, 2, 1
// K-tiles dividing nk.
template <int FMT, bool DOWN>
static GemvKernel gemv_kernel(int nk) {
  if (nk == 16) return k_gemv<FMT, DOWN, 16>;
  if (nk % 8 == 0) return k_gemv<FMT, DOWN, 8>;
  if (nk % 6 == 0) return k_gemv<FMT, DOWN, 6>;
  if (nk % 4 == 0) return k_gemv<FMT, DOWN, 4>;
  if (nk % 2 == 0) return k_gemv<FMT, DOWN, 2>;
  return k_gemv<FMT, DOWN, 1>;
}

template <int FMT>
static hipError_t launch_fmt(const FfnParams& P, GemvArgs G, hipStream_t s) {
  const size_t rowb1 = (size_t)(P.H + 8) * 2, rowb2 = (size_t)(P.I + 8) * 2;
  G.rbs1 = (int)std::min<size_t>(16, kDynLds / rowb1);
  G.rbs2 = (int)std::min<size_t>(16, kDynLds / rowb2);
  G.x_bytes = (int)(((size_t)P.T * rowb1 + 15) / 16 * 16);
  G.x_all = ((size_t)G.x_bytes <= kDynLds && P.T <= kMaxStagedRows && P.T * P.k <= kTokCache) ? 1 : 0;
  const size_t lds1 = G.x_all ? (size_t)G.x_bytes : G.rbs1 * rowb1;
  const size_t lds2 = G.rbs2 * rowb2;
  // Row blocks: at most ceil(T*k / rbs) + min(E, T*k) routed, plus the shared expert's.
  auto nrb = [&](int rbs) {
    const long long rows = (long long)P.T * P.k;
    long long n = (rows + rbs - 1) / rbs + std::min<long long>(P.E, rows);
    if (P.shared_blob) n += (P.T + rbs - 1) / rbs;
    return n;
  };
  const auto k1 = gemv_kernel<FMT, false>(P.H / Fmt<FMT>::KT);
  const auto k2 = gemv_kernel<FMT, true>(P.I / Fmt<FMT>::KT);
  const long long cap1 = (long long)blocks_per_cu(reinterpret_cast<const void*>(k1), lds1) * cu_count();
  const long long cap2 = (long long)blocks_per_cu(reinterpret_cast<const void*>(k2), lds2) * cu_count();
  const int g1 = (int)std::max<long long>(1, std::min<long long>(nrb(G.rbs1) * G.ng, cap1));
  const int g2 = (int)std::max<long long>(1, std::min<long long>(nrb(G.rbs2) * G.nd, cap2));
  launch(k1, dim3(g1), dim3(256), lds1, s, P, G);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch(k2, dim3(g2), dim3(256), lds2, s, P, G);
  e = hipGetLastError();
  return e;
}

template <int FMT, bool DOWN>
static hipError_t set_lds_limit_all() {
  const GemvKernel ks[] = {k_gemv<FMT, DOWN, 16>, k_gemv<FMT, DOWN, 8>, k_gemv<FMT, DOWN, 6>, k_gemv<FMT, DOWN, 4>,
                           k_gemv<FMT, DOWN, 2>, k_gemv<FMT, DOWN, 1>};
  for (GemvKernel f : ks) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(f), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)kDynLds);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

static hipError_t set_gemv_lds_limits() {
  static bool done = false;
  if (!done) {
    hipError_t e;
    if ((e = set_lds_limit_all<MOE_FMT_BF16, false>()) != hipSuccess) return e;
    if ((e = set_lds_limit_all<MOE_FMT_BF16, true>()) != hipSuccess) return e;
    if ((e = set_lds_limit_all<MOE_FMT_MXFP4, false>()) != hipSuccess) return e;
    if ((e = set_lds_limit_all<MOE_FMT_MXFP4, true>()) != hipSuccess) return e;
    if ((e = set_lds_limit_all<MOE_FMT_NVFP4, false>()) != hipSuccess) return e;
    if ((e = set_lds_limit_all<MOE_FMT_NVFP4, true>()) != hipSuccess) return e;
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
