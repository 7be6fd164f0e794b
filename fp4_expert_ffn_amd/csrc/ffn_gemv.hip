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
// fp32; when only the combined output is wanted, y rows are written in token
// order t * k + j, so the combine kernel after it needs no row index).  Every
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
#include <type_traits>

#include "ffn_common.h"
#include "topk.h"
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
template <>
struct Fmt<MOE_FMT_FP8> {
  static constexpr int KT = 64, SPT = 2;
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

// A lane's scale bytes of one tile (p already offset to the lane), kept in
// their loaded width: widening them right after the load would make the
// compiler wait for it there.
template <int FMT>
using ScaleT = typename std::conditional<FMT == MOE_FMT_NVFP4, uint16_t, uint8_t>::type;
template <int FMT>
__device__ __forceinline__ ScaleT<FMT> load_scale_at(const uint8_t* p) {
  if constexpr (FMT == MOE_FMT_MXFP4) return *p;
  if constexpr (FMT == MOE_FMT_NVFP4) return *reinterpret_cast<const uint16_t*>(p);
  return 0;
}

// B operand of MFMA step s (8 values) from a lane's tile fragment, block
// scale applied exactly: E2M1 x E8M0 in bf16 (the conversion applies the
// power of two); E2M1 x E4M3 in fp16, where the product (at most 5
// significant bits, magnitude in [2^-10, 2688]) is exact, so one packed
// fp16 multiply applies the scale; E4M3 (FP8) in fp16 as it is.  For the
// 4-bit formats step s takes the lane's values 8s..8s+7 (its 32 values
// cover 4 steps), for FP8 its 16 values cover 2 steps.
template <int FMT, int S>
__device__ __forceinline__ typename Fmt<FMT>::V bfrag(const uint4 q, uint32_t sc) {
  if constexpr (FMT == MOE_FMT_BF16) {
    return __builtin_bit_cast(bf16x8_t, q);
  } else if constexpr (FMT == MOE_FMT_FP8) {
    const uint32_t lo = S == 0 ? q.x : q.z, hi = S == 0 ? q.y : q.w;
    const f16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
    const f16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
    const f16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
    const f16x2_t e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
    return f16x8_t{a.x, a.y, b.x, b.y, c.x, c.y, e.x, e.y};
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
// `rbs` rows numbered [rb[a], rb[a+1]).  flat[p] caches perm[p] and tok[p]
// perm[p] / k when T*k <= kTokCache.  The arrays live in dynamic LDS, sized
// for na active experts (min(E, T*k) routed, plus the shared one).
constexpr int kTokCache = 1024;
struct ActiveLds {
  int *cnt, *p0, *slot, *rb, *tok, *flat;
  int* n;
};

__host__ __device__ inline size_t active_lds_bytes(int na, int ntok) {
  return (size_t)(4 * na + 2 + 2 * ntok) * sizeof(int);
}

// ntok: T*k if it is at most kTokCache, else 0
__device__ inline ActiveLds active_view(uint8_t* base, int na, int ntok) {
  int* b = reinterpret_cast<int*>(base);
  ActiveLds A;
  A.n = b;
  A.cnt = b + 1;
  A.p0 = A.cnt + na;
  A.slot = A.p0 + na;
  A.rb = A.slot + na;  // na + 1 entries
  A.tok = A.rb + na + 1;
  A.flat = A.tok + ntok;
  return A;
}

template <int KPER>
__device__ inline void build_active(const FfnParams& P, int rbs, const ActiveLds& A) {
  const int tid = threadIdx.x;
  const int N = P.T * P.k;
  if (tid >= 64) {
    if (N <= kTokCache)
      for (int p = tid - 64; p < N; p += 192) {
        const int f = P.perm[p];
        A.flat[p] = f;
        A.tok[p] = f / P.k;
      }
  } else {
    // every load first (one round trip), then the compaction
    constexpr int kPer = KPER;
    int c[kPer], off[kPer], sl[kPer], mk[kPer];
    // unconditional loads (indices clamped to E - 1), so they all issue
    // before the first wait; lanes past E are zeroed afterwards
    // (without a mask, the byte loads read the counts and are ignored)
    const bool has_mask = P.mask != nullptr;
    const uint8_t* mask = has_mask ? P.mask : reinterpret_cast<const uint8_t*>(P.counts);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = min(64 * i + tid, P.E - 1);
      c[i] = P.counts[e];
      off[i] = P.offsets[e];
      sl[i] = P.slot_of_expert[e];
      mk[i] = mask[has_mask ? e : 0];
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if ((has_mask && mk[i] == 0) || 64 * i + tid >= P.E) c[i] = 0;
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
      *A.n = n;
    }
  }
  lds_barrier();
}

// The routing of a call of at most kRouteFoldRows tokens (T * k <= 64),
// computed by every workgroup of the gate/up launch in place of reading it:
// wave t selects token t's experts (wave_topk, the routing kernels' own
// selection), then the stable counting sort of the T * k pairs by expert
// (rank = pairs with a lower expert id + pairs of the same expert and a
// lower flat index) fills the active-expert table.  Each expert's rows fit
// one row block (count <= T <= rbs).  Workgroup 0 also writes the routing
// outputs for the later launches: ids, weights, counts (all E), offsets
// (E + 1), perm and inv.  No expert mask.
constexpr int kRouteFoldRows = 4;

template <int NPER>
__device__ inline void route_active(const FfnParams& P, const GemvArgs& G, const ActiveLds& A) {
  __shared__ int32_t s_ids[64], s_rank[64], s_lower[64];
  __shared__ float s_w[64];
  __shared__ int32_t s_slot[256];
  __shared__ uint8_t s_first[64];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int T = P.T, k = P.k, E = P.E, N = T * k;
  for (int e = tid; e < E; e += 256) s_slot[e] = P.slot_of_expert[e];
  if (wave < T) wave_topk<NPER>(G.logits + (size_t)wave * E, E, k, G.renorm, s_ids + wave * k, s_w + wave * k);
  __syncthreads();
  if (tid < N) {
    const int e = s_ids[tid];
    int lower = 0, same_before = 0;
    for (int g = 0; g < N; ++g) {
      const int eg = s_ids[g];
      lower += eg < e;
      same_before += (eg == e) & (g < tid);
    }
    s_rank[tid] = lower + same_before;
    s_lower[tid] = lower;
    s_first[tid] = same_before == 0;
  }
  __syncthreads();
  if (tid < N) {
    A.flat[s_rank[tid]] = tid;
    A.tok[s_rank[tid]] = tid / k;
    if (s_first[tid]) {
      const int e = s_ids[tid];
      int a = 0, cnt = 0;
      for (int g = 0; g < N; ++g) {
        a += s_first[g] && s_ids[g] < e;
        cnt += s_ids[g] == e;
      }
      A.cnt[a] = cnt;
      A.p0[a] = s_lower[tid];
      A.slot[a] = s_slot[e];
      A.rb[a + 1] = a + 1;
    }
  }
  if (tid == 0) {
    int n = 0;
    for (int g = 0; g < N; ++g) n += s_first[g];
    A.rb[0] = 0;
    if (P.shared_blob) {
      A.cnt[n] = T;
      A.p0[n] = N;
      A.slot[n] = -1;
      A.rb[n + 1] = n + 1;
      ++n;
    }
    *A.n = n;
  }
  if (blockIdx.x == 0) {
    int32_t* counts = const_cast<int32_t*>(P.counts);
    int32_t* offsets = const_cast<int32_t*>(P.offsets);
    for (int e = tid; e <= E; e += 256) {
      int below = 0, at = 0;
      for (int g = 0; g < N; ++g) {
        below += s_ids[g] < e;
        at += s_ids[g] == e;
      }
      offsets[e] = below;
      if (e < E) counts[e] = at;
    }
    if (tid < N) {
      G.ids_out[tid] = s_ids[tid];
      G.w_out[tid] = s_w[tid];
      const_cast<int32_t*>(P.perm)[s_rank[tid]] = tid;
      const_cast<int32_t*>(P.inv)[tid] = s_rank[tid];
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
  int lo = 0, hi = *A.n - 1;  // active expert a with rb[a] <= rb < rb[a+1]
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

// Operand rows in LDS: nr rows of K bf16 (or fp16) values, each followed by
// one 16-byte pad, so 16-byte piece j of row r sits at slot r * (K/8 + 1) + j.
// The 16 rows that one A-fragment read touches then fall 16 bytes apart in
// the bank space (no conflicts), and a fragment's address is a per-lane base
// plus a compile-time offset.  The rows arrive by direct global->LDS loads
// (no registers), which write 64 consecutive slots per wave instruction (a
// pad slot receives a copy of its row's last piece); a last partial
// instruction spills into kRowSlack bytes past the rows.
constexpr int kRowSlack = 1024;

__host__ __device__ constexpr size_t row_bytes(int K) { return (size_t)K * 2 + 16; }

template <class Src>
__device__ __forceinline__ void dma_rows(uint8_t* act, const uint16_t* base, int K, int nr, Src src) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int spr = K / 8 + 1, total = nr * spr;  // slots per row, slots
  const int nch = (total + 63) >> 6;
  for (int c = wave; c < nch; c += 4) {
    const int p = min(c * 64 + lane, total - 1);  // lanes past the rows re-read the last piece (into the slack)
    const int r = p / spr, j = min(p % spr, spr - 2);
    __builtin_amdgcn_global_load_lds(base + (size_t)src(r) * K + j * 8,
                                     (__attribute__((address_space(3))) void*)(act + c * 1024), 16, 0, 0);
  }
}

__device__ __forceinline__ uint32_t bf16x8_absmax_bits(const uint4 v) {
  uint32_t m = max(max(v.x & 0x7FFFu, v.x >> 16 & 0x7FFFu), max(v.y & 0x7FFFu, v.y >> 16 & 0x7FFFu));
  return max(m, max(max(v.z & 0x7FFFu, v.z >> 16 & 0x7FFFu), max(v.w & 0x7FFFu, v.w >> 16 & 0x7FFFu)));
}

// bf16 values of one 16-byte piece (8 values) as fp16 times sc = 2^-p: the
// power of two is applied exactly in fp32, then one rounding to fp16.
__device__ __forceinline__ uint4 bf16x8_to_f16x8(const uint4 v, float sc) {
  auto cv = [&](uint32_t w) -> uint32_t {
    const f32x2_t f = {__uint_as_float(w << 16) * sc, __uint_as_float(w & 0xFFFF0000u) * sc};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
  };
  return make_uint4(cv(v.x), cv(v.y), cv(v.z), cv(v.w));
}

// After every wave's rows have landed (and a barrier): for the fp16 operand
// path the rows are rewritten in place as fp16 of value * 2^-pexp[r].  A row
// whose largest magnitude lies in [2^-10, 2^16) converts as it is: pexp[r] =
// 0, one pass.  A row holding a larger value (or inf / NaN), or a piece below
// 2^-10, is marked in *big by the pass; if its largest magnitude (from its
// global copy src(r)) is outside [2^-10, 2^16) it is converted again with the
// shift pexp[r] (in [-126, 127]) that puts that magnitude in [2^14, 2^15)
// (the output rows are multiplied back by 2^pexp[r]).  bf16 -> fp16 is exact
// for every value of magnitude >= 2^-14 * 2^pexp[r]; smaller ones round at
// 2^-24 * 2^pexp[r], far below the row's largest product (at most 2^-14 of
// it).  The piece order does not matter for the pass.  For fp16, ends with a
// barrier; bf16 rows need nothing more.  *big is zero on entry and on return.
template <bool F16, class Src>
__device__ __forceinline__ void finish_rows(uint8_t* act, int K, int nr, int* pexp, int* big, Src src) {
  if constexpr (F16) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, ppr = K / 8, spr = ppr + 1;
    const int total = nr * spr;  // pad slots hold copies of real pieces: converted alike
    if (tid < nr) pexp[tid] = 0;
    for (int p = tid; p < total; p += 256) {
      uint4* q = reinterpret_cast<uint4*>(act) + p;
      const uint4 v = *q;
      // |value| >= 2^16, inf or NaN; or a piece below 2^-10, whose row may
      // lie below fp16's normal range (decided from the whole row below)
      const uint32_t am = bf16x8_absmax_bits(v);
      if (am >= 0x4780u || am < 0x3A80u) atomicOr(big, 1 << (p / spr));
      *q = bf16x8_to_f16x8(v, 1.0f);
    }
    lds_barrier();
    const int bm = *big;
    if (bm != 0) {
      for (int r = wave; r < nr; r += 4) {
        if (!((bm >> r) & 1)) continue;
        const uint4* g = reinterpret_cast<const uint4*>(src(r));
        uint32_t mx = 0;
        for (int j = lane; j < ppr; j += 64) mx = max(mx, bf16x8_absmax_bits(g[j]));
        mx = wave_max_u32(mx);
        const int E = (int)(mx >> 7);  // biased exponent of the row's largest |value|: it is < 2^(E-126)
        // rows in [2^-10, 2^16) stay as converted; others are shifted so that
        // their largest |value| lies in [2^14, 2^15) (up by at most 2^126)
        if (E != 0xFF && E >= 0x75 && E < 0x8F) continue;
        const int pe = (E == 0xFF) ? 0 : max(-126, E - 141);
        if (lane == 0) pexp[r] = pe;
        const float sc = __uint_as_float((uint32_t)(127 - pe) << 23);
        uint4* row = reinterpret_cast<uint4*>(act) + (size_t)r * spr;
        for (int j = lane; j < ppr; j += 64) row[j] = bf16x8_to_f16x8(g[j], sc);
      }
      lds_barrier();
      if (tid == 0) *big = 0;
    }
  }
}

// Wait until at most `after` vector-memory operations are outstanding, then
// barrier: the direct-to-LDS row loads of every wave have landed and are
// visible, while the last `after` loads issued behind them stay in flight.
// (The compiler does not order its own waits after these row loads; and a
// fenced barrier would wait for every load.)
template <int AFTER>
__device__ __forceinline__ void rows_landed() {
  static_assert(AFTER >= 0 && AFTER <= 63, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt [3:0] and [15:14], expcnt [6:4] (7: no wait), lgkmcnt [11:8]
  constexpr int enc = (AFTER & 15) | ((AFTER >> 4) << 14) | (7 << 4) | (0 << 8);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(enc);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 2^p as a float (-126 <= p < 128)
__device__ __forceinline__ float pow2i(int p) { return __uint_as_float((uint32_t)(127 + p) << 23); }

constexpr int kTrashSlots = 256;         // 4 KiB scratch slots (workgroup index modulo this)

// One projection of the decode path.
//   DOWN = false: gate/up + SwiGLU.  Item (row block, c) covers intermediate
//     rows [32c, 32c + 32): wave w streams row group 4c + w of W13 (waves 0
//     and 2 gate, 1 and 3 up); the up waves hand their 16 x 16 outputs to the
//     gate waves through LDS, which write h = silu(g) * u as bf16.
//   DOWN = true: down projection.  Item (row block, c) covers output columns
//     [64c, 64c + 64): wave w streams row group 4c + w of W2 and writes its 16
//     columns of y (fp32).
// The items (row block major) are dealt to the workgroups in contiguous,
// equal ranges, so every workgroup (and every CU) streams the same number of
// weight tiles, give or take one item.  A range splits into tasks at row
// block boundaries; a task stages its operand rows once, so each row is read
// by the few workgroups of its expert, not by all of them.  With XALL (the
// gate/up projection of at most kXallMaxT tokens) every token row of x is
// staged once, in token order, by the first task, and later tasks stage
// nothing.  Each wave runs all K-tiles of its row group itself (no
// cross-wave reduction), in sub-items of SUB K-tiles (SUB divides K / KT).
//
// Memory pipeline: two register banks of weight tiles (plus the item's
// per-tensor multiplier) alternate, and the loop is unrolled by two so each
// bank keeps fixed registers: the loads of sub-item ss + 1 are in flight
// while sub-item ss computes.  The operand rows are loaded before the first
// weights and written to LDS while those are in flight.  Inside a sub-item
// the operand fragments of the next K-tile are read from LDS while the
// current one's matrix instructions run.
constexpr int kXallMaxT = 4;

template <int FMT, bool DOWN, int SUB, bool XALL, bool ROUTE = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemv(FfnParams P, GemvArgs G) {
  using F = Fmt<FMT>;
  static_assert(!(XALL && DOWN), "the down projection stages its rows per task");
  static_assert(!ROUTE || XALL, "the folded routing goes with every token row staged");
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int s_pexp[16];
  __shared__ float s_u[2][16][17];
  __shared__ int s_rows[16];
  __shared__ int s_big;  // rows of the staged block that overflow fp16 (finish_rows)
  // workgroups of the GEMV (the copy workgroups come after them)
  int ngemv = (int)gridDim.x;
  if constexpr (!DOWN && !ROUTE) {
    ngemv -= G.copy_wgs;
    if ((int)blockIdx.x >= ngemv) {
      copy_blob_list(G.copy, G.copy_pool, G.copy_slot_vecs, (int)blockIdx.x - ngemv, G.copy_wgs);
      return;
    }
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, m = lane & 15, grp = lane >> 4;
  if (tid == 0) s_big = 0;  // visible after the table's barrier
  const int H = P.H, I = P.I;
  const int K = DOWN ? I : H, nk = K / F::KT;
  const int rbs = DOWN ? G.rbs2 : G.rbs1, nchunk = DOWN ? G.nd : G.ng;
  const ActiveLds A = active_view(lds, G.na, P.T * P.k <= kTokCache ? P.T * P.k : 0);
  uint8_t* act = lds + G.act_off;  // operand rows (swizzled) + slack
  if constexpr (ROUTE) {
    // the token rows do not depend on the routing: staged while it runs
    dma_rows(act, P.x, K, P.T, [](int r) { return r; });
    if (P.E <= 128) route_active<2>(P, G, A);
    else route_active<4>(P, G, A);
  } else if (P.E <= 128) {
    build_active<2>(P, rbs, A);
  } else if (P.E <= 256) {
    build_active<4>(P, rbs, A);
  } else {
    build_active<16>(P, rbs, A);
  }
  const int nrb = A.rb[*A.n];
  // this workgroup's items: [i_beg, i_end) of nrb * nchunk, row block major.
  // With two workgroups per CU (workgroups b and b + ncu share a CU), each
  // CU gets an equal contiguous range, split between its two workgroups, so
  // CU loads differ by at most one item.
  const long long nitems = (long long)nrb * nchunk;
  long long i_beg, i_end;
  if (G.ncu > 0) {
    const int cu = blockIdx.x % G.ncu, half = blockIdx.x / G.ncu;
    const long long c0 = nitems * cu / G.ncu, c1 = nitems * (cu + 1) / G.ncu, mid = c0 + (c1 - c0 + 1) / 2;
    i_beg = half ? mid : c0;
    i_end = half ? c1 : mid;
  } else {
    i_beg = nitems * blockIdx.x / ngemv;
    i_end = nitems * (blockIdx.x + 1) / ngemv;
  }
  const int nsub = nk / SUB;  // SUB divides nk: every sub-item loads exactly SUB tiles
  const size_t off_w = DOWN ? P.L.off_w2 : P.L.off_w13, off_s = DOWN ? P.L.off_s2 : P.L.off_s13;
  // per-tensor multiplier of this wave's rows: gate (even waves) / up (odd) / down
  const int gsel = DOWN ? 2 : (wave & 1);
  const uint16_t* rbase = DOWN ? G.h : P.x;
  // this workgroup's own 4 KiB of scratch (distinct lines: no store contention)
  float* trash = G.trash + (size_t)(blockIdx.x % kTrashSlots) * 1024;

  struct Bank {
    uint4 q[SUB];
    ScaleT<FMT> sc[SUB];
  };
  // Vector-memory loads of one bank: SUB tiles and SUB scale loads (4-bit
  // formats; 64 or 128 bytes apart, never merged).
  constexpr int kBankLoads = SUB + (kScaleTileBytes<FMT> ? SUB : 0);

  // XALL: every token row of x, in token order, before the first task (whose
  // first weights then go out behind them)
  if (XALL && !ROUTE && i_beg < i_end) dma_rows(act, P.x, K, P.T, [](int r) { return r; });
  bool first = true;
#pragma unroll 1
  for (long long it = i_beg; it < i_end;) {
    const int rbi = (int)(it / nchunk);
    const int c0 = (int)(it % nchunk), c1 = (int)std::min<long long>(nchunk, c0 + (i_end - it));
    it += c1 - c0;
    const RowBlock blk = row_block(P, A, rbs, rbi);
    const int nS = (c1 - c0) * nsub;
    const uint8_t* wbase = blk.blob + off_w;
    const uint8_t* sbase = blk.blob + off_s;

    // Loads are unconditional and fixed in number per sub-item (the compiler
    // then counts them exactly and waits only for the bank in use).
    auto issue = [&](int ss, Bank& b) {
      const int chunk = c0 + ss / nsub, sub = ss % nsub;
      const int rg = 4 * chunk + wave, kt0 = sub * SUB;
      // 32-bit tile index (a blob holds far fewer than 2^31 tiles); per-tile
      // addresses are then constant offsets from two base pointers, so no
      // 64-bit arithmetic sits between the loads.
      const uint32_t t0 = (uint32_t)rg * (uint32_t)nk + (uint32_t)kt0;
      const uint8_t* wp = wbase + ((size_t)t0 << 10) + lane * 16;
      const uint8_t* sp = sbase + (size_t)t0 * kScaleTileBytes<FMT> + lane * kScaleLaneBytes<FMT>;
      // exactly kBankLoads loads: the row wait below counts them
#pragma unroll
      for (int j = 0; j < SUB; ++j) b.sc[j] = load_scale_at<FMT>(sp + j * kScaleTileBytes<FMT>);
#pragma unroll
      for (int j = 0; j < SUB; ++j) b.q[j] = ldg16(wp + j * kTileBytes);
    };

    Bank b0, b1;
    // the per-tensor multiplier of this wave's rows, loaded once per task
    // ahead of the rows (so the row wait below covers it too)
    const float gmul = reinterpret_cast<const BlobHeader*>(blk.blob)->g[gsel];
    asm volatile("" ::: "memory");
    if constexpr (!XALL) {
      // operand rows of the block (token rows of x, or rows of h), loaded
      // ahead of the first weights; the table's barrier also ends the
      // previous task
      lds_barrier();
      if (tid < blk.nr) s_rows[tid] = DOWN ? blk.p0 + blk.r0 + tid : row_token(P, A, blk, tid);
      lds_barrier();
      dma_rows(act, rbase, K, blk.nr, [&](int r) { return s_rows[r]; });
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    issue(0, b0);  // behind the rows: waiting for the rows leaves all of its loads in flight
    __builtin_amdgcn_sched_barrier(0);
    if (!XALL || first) {
      rows_landed<kBankLoads>();
      finish_rows<F::F16>(act, K, XALL ? P.T : blk.nr, s_pexp, &s_big,
                          [&](int r) { return rbase + (size_t)(XALL ? r : s_rows[r]) * K; });
    }
    first = false;

    // this lane's A row: row m of the block (rows past the block read its
    // last row; their outputs are discarded), as an LDS row index
    const int am = min(m, blk.nr - 1);
    const int arow_i = XALL ? row_token(P, A, blk, am) : am;
    // this lane's fragment base: K-group grp of its row (values 32 grp + 8 st
    // of each 128-value K-tile, or 8 grp of each 32-value one)
    const uint8_t* abase = act + (size_t)arow_i * row_bytes(K) + (F::KT / 2) * grp;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    // The epilogue runs after every sub-item (uniform code: no branch around
    // memory operations inside the pipelined loop); before an item's last
    // sub-item its stores go to a scratch area, as do rows past the block and
    // the up waves' h.
    auto body = [&](int ss, const Bank& b) {
      const int chunk = c0 + ss / nsub, sub = ss % nsub;
      const bool last = sub == nsub - 1;
      if (sub == 0) acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // Operand fragment of MFMA step u of the sub-item (K-tile u / SPT),
      // read from LDS two steps ahead of its use (a ring of three).
      constexpr int NU = SUB * F::SPT;
      auto read_a = [&](int u) {
        const int kt = sub * SUB + u / F::SPT, st = u % F::SPT;
        return *reinterpret_cast<const uint4*>(abase + kt * (F::KT * 2) + 16 * st);
      };
      uint4 ar[3];
      ar[0] = read_a(0);
      if (NU > 1) ar[1] = read_a(1);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        if (u + 2 < NU) ar[(u + 2) % 3] = read_a(u + 2);
        const int j = u / F::SPT, st = u % F::SPT;
        typename F::V bv;
        if constexpr (F::SPT == 4) {
          bv = st == 0 ? bfrag<FMT, 0>(b.q[j], b.sc[j]) : st == 1 ? bfrag<FMT, 1>(b.q[j], b.sc[j])
             : st == 2 ? bfrag<FMT, 2>(b.q[j], b.sc[j]) : bfrag<FMT, 3>(b.q[j], b.sc[j]);
        } else if constexpr (F::SPT == 2) {
          bv = st == 0 ? bfrag<FMT, 0>(b.q[j], b.sc[j]) : bfrag<FMT, 1>(b.q[j], b.sc[j]);
        } else {
          bv = bfrag<FMT, 0>(b.q[j], b.sc[j]);
        }
        acc = mma<FMT>(__builtin_bit_cast(typename F::V, ar[u % 3]), bv, acc);
        if (st == F::SPT - 1) {
          // one K-tile at a time (the compiler would otherwise hoist the
          // decode and the LDS reads of the whole sub-item)
          asm volatile("" ::: "memory");
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // Lane: rows 4 (lane / 16) + v of the block, column lane % 16 of this
      // wave's 16 output rows of the weight.
      auto scaled = [&](float (&val)[4]) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = 4 * grp + v;
          float sc2 = gmul;
          if constexpr (F::F16) {
            const int rr = min(r, blk.nr - 1);
            sc2 *= pow2i(s_pexp[XALL ? row_token(P, A, blk, rr) : rr]);
          }
          val[v] = acc[v] * sc2;
        }
      };
      if constexpr (DOWN) {
        float val[4];
        scaled(val);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = 4 * grp + v;
          // y row: perm order, or flat order (t * k + j) for the combine
          // (shared rows T*k + t either way)
          const int p = blk.p0 + blk.r0 + min(r, blk.nr - 1);
          const int yrow = (G.yflat && !blk.shared) ? A.flat[p] : p;
          float* dst = (last && r < blk.nr) ? G.y + (size_t)yrow * H + 64 * chunk + 16 * wave + m
                                            : trash + (r * 4 + wave) * 16 + m;
          *dst = val[v];
        }
      } else {
        // SwiGLU on an item's last sub-item only (a workgroup-uniform
        // branch); the stores are issued on every sub-item all the same, to
        // the scratch area before the last one.
        float hv[4] = {0.f, 0.f, 0.f, 0.f};
        if (last) {
          float val[4];
          scaled(val);
          if (wave & 1)
#pragma unroll
            for (int v = 0; v < 4; ++v) s_u[wave >> 1][4 * grp + v][m] = val[v];
          lds_barrier();
#pragma unroll
          for (int v = 0; v < 4; ++v) hv[v] = silu_fast(val[v]) * s_u[wave >> 1][4 * grp + v][m];
          lds_barrier();
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = 4 * grp + v;
          uint16_t* dst = (last && r < blk.nr && !(wave & 1))
                              ? G.h + (size_t)(blk.p0 + blk.r0 + r) * I + 32 * chunk + 16 * (wave >> 1) + m
                              : reinterpret_cast<uint16_t*>(trash) + (r * 4 + wave) * 16 + m;
          *dst = f32_to_bf16_rne(hv[v]);
        }
      }
    };

    // Two banks, loop unrolled by two: sub-items ss (bank b0) and ss + 1 (b1)
    // per trip, with ss + 2 loading into b0 during ss + 1.  The last one or
    // two sub-items run after the loop and issue nothing past the end.
    int ss = 0;
#pragma unroll 1
    for (; ss + 2 < nS; ss += 2) {
      issue(ss + 1, b1);
      __builtin_amdgcn_sched_barrier(0);
      body(ss, b0);
      __builtin_amdgcn_sched_barrier(0);
      issue(ss + 2, b0);
      __builtin_amdgcn_sched_barrier(0);
      body(ss + 1, b1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (ss + 1 < nS) {
      issue(ss + 1, b1);
      __builtin_amdgcn_sched_barrier(0);
      body(ss, b0);
      __builtin_amdgcn_sched_barrier(0);
      body(ss + 1, b1);
    } else {
      body(ss, b0);
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
  constexpr int kMemo = 64;
  static const void* fns[kMemo];
  static size_t ldss[kMemo];
  static int vals[kMemo];
  static int n = 0;
  for (int i = 0; i < n; ++i)
    if (fns[i] == fn && ldss[i] == lds) return vals[i];
  int b = 1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, fn, 256, lds) != hipSuccess || b < 1) b = 1;
  if (n < kMemo) {
    fns[n] = fn;
    ldss[n] = lds;
    vals[n] = b;
    ++n;
  }
  return b;
}

// Dynamic LDS per workgroup: with the static part (under 5 KB) two
// workgroups fit one CU's 160 KB.
constexpr size_t kDynLds = 75 * 1024;

typedef void (*GemvKernel)(FfnParams, GemvArgs);

// Sub-item size: the largest of 16 (only when it is all of K, and not for
// NVFP4, whose decode needs more registers), 8, 6, 4, 2, 1 K-tiles dividing nk.
template <int FMT>
constexpr int kSubMax = (FMT == MOE_FMT_NVFP4 || FMT == MOE_FMT_FP8) ? 8 : 16;

template <int FMT, bool DOWN, bool XALL>
static GemvKernel gemv_kernel(int nk) {
  if (nk == 16) return k_gemv<FMT, DOWN, kSubMax<FMT>, XALL>;
  if (nk % 8 == 0) return k_gemv<FMT, DOWN, 8, XALL>;
  if (nk % 6 == 0) return k_gemv<FMT, DOWN, 6, XALL>;
  if (nk % 4 == 0) return k_gemv<FMT, DOWN, 4, XALL>;
  if (nk % 2 == 0) return k_gemv<FMT, DOWN, 2, XALL>;
  return k_gemv<FMT, DOWN, 1, XALL>;
}

template <int FMT>
static GemvKernel gemv_route_kernel(int nk) {
  if (nk == 16) return k_gemv<FMT, false, kSubMax<FMT>, true, true>;
  if (nk % 8 == 0) return k_gemv<FMT, false, 8, true, true>;
  if (nk % 6 == 0) return k_gemv<FMT, false, 6, true, true>;
  if (nk % 4 == 0) return k_gemv<FMT, false, 4, true, true>;
  if (nk % 2 == 0) return k_gemv<FMT, false, 2, true, true>;
  return k_gemv<FMT, false, 1, true, true>;
}

template <int FMT>
static hipError_t launch_fmt(const FfnParams& P, GemvArgs G, hipStream_t s) {
  const long long rows = (long long)P.T * P.k;
  G.na = (int)std::min<long long>(P.E, rows) + (P.shared_blob ? 1 : 0);
  const int ntok = rows <= kTokCache ? (int)rows : 0;
  G.act_off = (int)((active_lds_bytes(G.na, ntok) + 15) / 16 * 16);
  const size_t avail = kDynLds - (size_t)G.act_off;
  // Rows per row block: at most 16, within the LDS left.
  auto block_rows = [&](int K) {
    const size_t by_lds = (avail - kRowSlack) / row_bytes(K);
    return (int)std::max<size_t>(1, std::min<size_t>(16, by_lds));
  };
  G.rbs1 = block_rows(P.H);
  G.rbs2 = block_rows(P.I);
  // Small batches stage every token row of x once per workgroup (it fits the
  // LDS of one row block, and the token table is cached).
  const bool xall = P.T <= kXallMaxT && P.T <= G.rbs1 && ntok > 0;
  const size_t lds1 = G.act_off + (size_t)(xall ? P.T : G.rbs1) * row_bytes(P.H) + kRowSlack;
  const size_t lds2 = G.act_off + (size_t)G.rbs2 * row_bytes(P.I) + kRowSlack;
  // Row blocks: at most ceil(T*k / rbs) + min(E, T*k) routed, plus the shared expert's.
  auto nrb = [&](int rbs) {
    long long n = (rows + rbs - 1) / rbs + std::min<long long>(P.E, rows);
    if (P.shared_blob) n += (P.T + rbs - 1) / rbs;
    return n;
  };
  const bool route = G.logits != nullptr;  // the caller checked gemv_route_fits
  if ((route && !xall) || (route && G.copy_wgs > 0)) return hipErrorInvalidValue;
  const auto k1 = route ? gemv_route_kernel<FMT>(P.H / Fmt<FMT>::KT)
                  : xall ? gemv_kernel<FMT, false, true>(P.H / Fmt<FMT>::KT)
                         : gemv_kernel<FMT, false, false>(P.H / Fmt<FMT>::KT);
  const auto k2 = gemv_kernel<FMT, true, false>(P.I / Fmt<FMT>::KT);
  // The kernels are built for two resident workgroups per CU (their register
  // budget); more would start late, after the first ones finish.
  const long long cap1 = (long long)std::min(2, blocks_per_cu(reinterpret_cast<const void*>(k1), lds1)) * cu_count();
  const long long cap2 = (long long)std::min(2, blocks_per_cu(reinterpret_cast<const void*>(k2), lds2)) * cu_count();
  const int g1 = (int)std::max<long long>(1, std::min<long long>(nrb(G.rbs1) * G.ng, cap1));
  const int g2 = (int)std::max<long long>(1, std::min<long long>(nrb(G.rbs2) * G.nd, cap2));
  // a full grid of two workgroups per CU deals its items per CU
  G.ncu = g1 == 2 * cu_count() ? cu_count() : 0;
  launch(k1, dim3(g1 + G.copy_wgs), dim3(256), lds1, s, P, G);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  G.copy_wgs = 0;
  G.ncu = g2 == 2 * cu_count() ? cu_count() : 0;
  launch(k2, dim3(g2), dim3(256), lds2, s, P, G);
  e = hipGetLastError();
  return e;
}

template <int FMT, bool DOWN, bool XALL, bool ROUTE = false>
static hipError_t set_lds_limit_all() {
  const GemvKernel ks[] = {k_gemv<FMT, DOWN, kSubMax<FMT>, XALL, ROUTE>, k_gemv<FMT, DOWN, 8, XALL, ROUTE>,
                           k_gemv<FMT, DOWN, 6, XALL, ROUTE>, k_gemv<FMT, DOWN, 4, XALL, ROUTE>,
                           k_gemv<FMT, DOWN, 2, XALL, ROUTE>, k_gemv<FMT, DOWN, 1, XALL, ROUTE>};
  for (GemvKernel f : ks) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(f), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)kDynLds);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int FMT>
static hipError_t set_lds_limits_fmt() {
  hipError_t e;
  if ((e = set_lds_limit_all<FMT, false, false>()) != hipSuccess) return e;
  if ((e = set_lds_limit_all<FMT, false, true>()) != hipSuccess) return e;
  if ((e = set_lds_limit_all<FMT, false, true, true>()) != hipSuccess) return e;
  return set_lds_limit_all<FMT, true, false>();
}

static hipError_t set_gemv_lds_limits() {
  static bool done = false;
  if (!done) {
    hipError_t e;
    if ((e = set_lds_limits_fmt<MOE_FMT_BF16>()) != hipSuccess) return e;
    if ((e = set_lds_limits_fmt<MOE_FMT_MXFP4>()) != hipSuccess) return e;
    if ((e = set_lds_limits_fmt<MOE_FMT_NVFP4>()) != hipSuccess) return e;
    if ((e = set_lds_limits_fmt<MOE_FMT_FP8>()) != hipSuccess) return e;
    done = true;
  }
  return hipSuccess;
}

// Whether a call can take the gate/up launch with the routing folded in.
bool gemv_route_fits(const FfnParams& P) {
  // every token row staged in LDS beside the tables (the launcher's XALL condition holds with room to spare)
  return P.T >= 1 && P.T <= kRouteFoldRows && P.T * P.k <= 64 && P.E <= 256 && P.mask == nullptr &&
         (size_t)P.T * row_bytes(P.H) + kRowSlack + 16384 <= kDynLds;
}

hipError_t launch_gemv(const FfnParams& P, const GemvArgs& G, hipStream_t s) {
  hipError_t e = set_gemv_lds_limits();
  if (e != hipSuccess) return e;
  switch (P.fmt) {
    case MOE_FMT_BF16: return launch_fmt<MOE_FMT_BF16>(P, G, s);
    case MOE_FMT_MXFP4: return launch_fmt<MOE_FMT_MXFP4>(P, G, s);
    case MOE_FMT_NVFP4: return launch_fmt<MOE_FMT_NVFP4>(P, G, s);
    case MOE_FMT_FP8: return launch_fmt<MOE_FMT_FP8>(P, G, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
