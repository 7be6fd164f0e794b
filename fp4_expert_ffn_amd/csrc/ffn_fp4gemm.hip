// Prefill path, FP4: a persistent grouped GEMM on the block-scaled FP4 matrix
// cores (v_mfma_scale_f32_16x16x128_f8f6f4, both operands E2M1 with one E8M0
// scale per 32 K-values per row), for the gate/up projection (+ SwiGLU and
// the MXFP4 encoding of its output) and the down projection.
//
// Method: the expert FFN of a sparse MoE layer (pages as for the GEMV path);
// the activation precision (x and the SwiGLU output MXFP4-encoded per row per
// 32 values) is this library's reading of a 4-bit-weight GEMM on FP4 matrix
// cores.
//
// Design for gfx950:
//  - One workgroup of 8 waves per CU, looping over a contiguous range of
//    output tiles of 128 rows x 256 columns (XCD x takes the x-th eighth of
//    the tile list, so an expert's tiles share one L2).  Waves form a 2 x 4
//    grid of 64 x 64 blocks (4 x 4 MFMA tiles each).
//  - K advances 256 values (two 128-wide K-tiles) per step.  A step's
//    operands (A 16 KiB, B 32 KiB, their scales 3 KiB) arrive by direct
//    global->LDS loads into a ring of NS stage buffers, issued NS - 1 steps
//    ahead across tile boundaries: no registers hold loads in flight, so the
//    prefetch depth is set by LDS (3 x 51 KiB).
//  - Every wave issues a fixed number of loads per step, so "stage s has
//    landed" is an s_waitcnt vmcnt with a compile-time count; one LDS-only
//    barrier per step then publishes the stage and frees the previous one.
//  - Each tile's expert, rows and column block come from descriptors built
//    in LDS at the start, and the gate/up tiles' token rows from perm
//    entries loaded (also directly into LDS) one tile ahead: the loop issues
//    no global loads besides the ring.
//  - The gate/up epilogue forms SwiGLU in registers (each wave holds matching
//    gate and up columns) and MXFP4-encodes each row's 32 values with
//    cross-lane (DPP) maxima: no LDS, so the ring keeps streaming.
#include <type_traits>

#include "ffn_common.h"
#include "wave.h"

namespace moe {

// ---------------------------------------------------------------- the GEMM

enum { kG_GateUp = 0, kG_Down = 1 };

constexpr int kGBM = 128, kGBN = 256;
constexpr int kGA = 128 * 128;           // A: 128 rows x 128 bytes (256 FP4 values)
constexpr int kGB = 16 * 2 * 1024;       // B: 16 row groups x 2 K-tiles x 1 KiB
constexpr int kGSA = 128 * 8;            // A scales: 8 E8M0 per row
constexpr int kGSB = 16 * 2 * 64;        // B scales: 32 scale tiles of 64 bytes
constexpr int kGStage = kGA + kGB + kGSA + kGSB;
constexpr int kGStages = 3;
constexpr int kGMaxTiles = 64;           // tiles per workgroup (descriptors in LDS)

// The stage ring: three LDS buffers; the step loop is unrolled by three so
// each step's buffers are known at compile time.
__shared__ __align__(16) uint8_t g_stage0[kGStage];
__shared__ __align__(16) uint8_t g_stage1[kGStage];
__shared__ __align__(16) uint8_t g_stage2[kGStage];

struct TileDesc {
  int slot;  // expert blob slot; -1: the shared expert
  int row0;  // first row (permutation order) of the tile
  int rows;  // valid rows (<= 128)
  int nt;    // 256-column block
};

// Direct global->LDS loads (lane l's 16 or 4 bytes land at dst + 16 l or
// dst + 4 l; dst must be wave-uniform), written as inline assembly: the
// compiler then does not treat every later LDS read as a possible reader of
// these loads (it would wait for all of them), and the pipeline's explicit
// vmcnt waits order them instead.  They write no registers, and any wait the
// compiler computes for its own loads only becomes more conservative.  One
// wait state separates the M0 write from the load that reads it.  (The
// compiler uses M0 nowhere else in these kernels; a CPU test checks that.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ uint32_t lds_off(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)p;
}
__device__ __forceinline__ void dma16(const void* src, uint8_t* dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src),
               "s"(__builtin_amdgcn_readfirstlane(lds_off(dst)))
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* src, uint8_t* dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src),
               "s"(__builtin_amdgcn_readfirstlane(lds_off(dst)))
               : "memory", "m0");
}

#pragma clang diagnostic pop

// Wait until at most N vector-memory operations of this wave are
// outstanding (gfx9 s_waitcnt: vmcnt [3:0] and [15:14]; expcnt, lgkmcnt not waited).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  constexpr int enc = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(enc);
  asm volatile("" ::: "memory");
}

// max over the 16 lanes of a DPP row (lanes 16r .. 16r + 15), in every lane
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppRowMirror>(v));
  return v;
}

template <int I>
__device__ __forceinline__ uint8_t* stage_buf() {
  if constexpr (I == 0) return g_stage0;
  else if constexpr (I == 1) return g_stage1;
  else return g_stage2;
}

template <int MODE>
__global__ __launch_bounds__(512) void k_fp4_gemm(FfnParams P, MfmaBufs B) {
  __shared__ TileDesc desc[kGMaxTiles];
  // gate/up: perm entries of the rows of tiles q (slot q % 2) and q + 1 (the
  // other slot, loaded while tile q streams); the A row of a routed tile's
  // row r is token plist[...] / k of the token-order activations
  __shared__ int32_t plist[2][kGBM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 2, wn = wave & 3;
  const int K = MODE == kG_GateUp ? P.H : P.I;
  const int NT = (MODE == kG_GateUp ? 2 * P.I : P.H) / kGBN;
  const int nk_w = K / 128;  // weight K-tiles per row group
  const int nsteps = (K + 255) / 256;
  const bool half_tail = (K % 256) != 0;  // the last step holds one K-tile
  const uint32_t arow = K / 2, asrow = K / 32;

  // ---- the tile list: experts in id order, each expert's row tiles, each
  // row tile's column blocks (fastest); the shared expert's tiles last.
  int* pre = reinterpret_cast<int*>(g_stage0);  // [E + 1], in the (still idle) stage area
  const int E = P.E;
  if (tid < 64) {
    int run = 0;
    for (int base = 0; base < E; base += 64) {
      const int e = base + tid;
      int t = 0;
      if (e < E) {
        const int c = P.counts[e];
        if (c > 0 && (P.mask == nullptr || P.mask[e] != 0)) t = ((c + kGBM - 1) / kGBM) * NT;
      }
      int v = t;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o);
        if (tid >= o) v += u;
      }
      if (e < E) pre[e + 1] = run + v;
      run += __shfl(v, 63);
    }
    if (tid == 0) pre[0] = 0;
  }
  lds_barrier();
  const int routed = pre[E];
  const int total = routed + (P.shared_blob ? ((P.T + kGBM - 1) / kGBM) * NT : 0);
  const int G = gridDim.x, b = blockIdx.x;
  const int r = (b % 8) * (G / 8) + b / 8;  // XCD b % 8 takes the (b % 8)-th eighth of the list
  const int L0 = (int)((long long)total * r / G), L1 = (int)((long long)total * (r + 1) / G);
  const int ntile = L1 - L0;  // <= kGMaxTiles (checked by the launcher)
  for (int q = tid; q < ntile; q += 512) {
    const int L = L0 + q;
    TileDesc d;
    if (L >= routed) {
      const int local = L - routed;
      const int m0 = (local / NT) * kGBM;
      d.slot = -1;
      d.row0 = P.T * P.k + m0;
      d.rows = min(kGBM, P.T - m0);
      d.nt = local % NT;
    } else {
      int lo = 0, hi = E - 1;  // expert e with pre[e] <= L < pre[e + 1]
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= L) lo = mid; else hi = mid - 1;
      }
      const int local = L - pre[lo];
      const int m0 = (local / NT) * kGBM;
      d.slot = P.slot_of_expert[lo];
      d.row0 = P.offsets[lo] + m0;
      d.rows = min(kGBM, P.counts[lo] - m0);
      d.nt = local % NT;
    }
    desc[q] = d;
  }
  lds_barrier();
  if (ntile == 0) return;
  if (MODE == kG_GateUp && tid < kGBM && desc[0].slot >= 0)
    plist[0][tid] = P.perm[desc[0].row0 + min(tid, desc[0].rows - 1)];
  lds_barrier();
  const int nsteps_total = ntile * nsteps;

  const uint8_t* abase = MODE == kG_GateUp ? B.xq : B.hq;
  const uint8_t* asbase = MODE == kG_GateUp ? B.xs : B.hs;
  const size_t off_w = MODE == kG_GateUp ? P.L.off_w13 : P.L.off_w2;
  const size_t off_s = MODE == kG_GateUp ? P.L.off_s13 : P.L.off_s2;

  // Loads of global step s into stage buffer `buf`: waves 0-3 issue 8 (A 2,
  // B 4, A scales 1, B scales 1), waves 4-7 issue 7 (no A scales).
  // Issue-side tile state: the byte offsets of this lane's loads for K-step
  // 0 of the tile being issued, recomputed at each tile's first step (the
  // steps only add K offsets).
  const int seg0 = (lane & 7) ^ (lane >> 3);  // logical A segment this lane loads
  uint32_t a_off[2], as_off = 0, b_off[4], bs_off;
  const uint8_t* blob = nullptr;
  // row of the A operand (and its scales) for row r of tile q
  auto a_row = [&](int q, const TileDesc& d, int r) __attribute__((always_inline)) -> uint32_t {
    const int rr = min(r, d.rows - 1);  // rows past the tile re-read its last row
    if (MODE == kG_Down) return d.row0 + rr;
    if (d.slot < 0) return d.row0 - P.T * P.k + rr;  // the shared expert: token rows
    return (uint32_t)plist[q & 1][rr] / (uint32_t)P.k;
  };
  auto tile_state = [&](int q) __attribute__((always_inline)) {
    const TileDesc d = desc[q];
#pragma unroll
    for (int i = 0; i < 2; ++i) a_off[i] = a_row(q, d, 8 * (2 * wave + i) + (lane >> 3)) * arow + seg0 * 16;
    if (wave < 4) as_off = a_row(q, d, 32 * wave + (lane >> 1)) * asrow + (lane & 1) * 4;
    blob = d.slot < 0 ? P.shared_blob : P.slot_pool + (size_t)d.slot * P.slot_stride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qq = 4 * wave + i;
      b_off[i] = ((uint32_t)(d.nt * 16 + (qq >> 1)) * nk_w + (qq & 1)) * kTileBytes + lane * 16;
    }
    bs_off = ((uint32_t)(d.nt * 16 + 2 * wave + (lane >> 5)) * nk_w + ((lane >> 4) & 1)) * 64 + (lane & 15) * 4;
  };
  auto issue = [&](int s, uint8_t* st) __attribute__((always_inline)) {
    const int q = s / nsteps, ks = s - q * nsteps;
    if (ks == 0) {
      tile_state(q);
      // gate/up: the next tile's perm entries, ahead of that tile's first
      // loads by nsteps >= 2 steps (in the other slot, whose last reader was
      // the issue of this tile's state)
      if (MODE == kG_GateUp && wave < 2 && q + 1 < ntile) {
        const TileDesc dn = desc[q + 1];
        if (dn.slot >= 0) {
          const int r = min(64 * wave + lane, dn.rows - 1);
          dma4(P.perm + dn.row0 + r, reinterpret_cast<uint8_t*>(&plist[(q + 1) & 1][64 * wave]));
        }
      }
    }
    // A tail step (K % 256 == 128) holds one K-tile: its second K-tile's
    // loads re-read the first's (never used).
    const bool tail = half_tail && ks == nsteps - 1;
    // A: chunk c = 2 wave + i holds rows 8c .. 8c + 7; lane l writes physical
    // segment l % 8 of row 8c + l / 8, which holds logical segment
    // (l % 8) ^ (l / 8) (the swizzle that makes fragment reads conflict-free).
    const uint32_t a_k = ks * 128 - ((tail && seg0 >= 4) ? 64 : 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(abase + a_off[i] + a_k, st + (2 * wave + i) * 1024);
    // B: tile qq = 4 wave + i is row group nt * 16 + qq / 2, K-tile 2 ks + qq % 2
    const uint8_t* wt = blob + off_w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t kk = 2 * ks * kTileBytes - ((tail && (i & 1)) ? kTileBytes : 0);
      dma16(wt + b_off[i] + kk, st + kGA + (4 * wave + i) * 1024);
    }
    // A scales (waves 0-3): row 32 wave + l / 2, dword l % 2 of its 8 step bytes
    if (wave < 4) dma4(asbase + as_off + ks * 8 - ((tail && (lane & 1)) ? 4 : 0), st + kGA + kGB + wave * 256);
    // B scales: scale tile (row group nt * 16 + 2 wave + l / 32, K-tile
    // 2 ks + (l / 16) % 2), dword l % 16; in LDS at (2 ntl + kt) * 64
    dma4(blob + off_s + bs_off + 2 * ks * 64 - ((tail && ((lane >> 4) & 1)) ? 64 : 0),
         st + kGA + kGB + kGSA + wave * 256);
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int s, const uint8_t* st) __attribute__((always_inline)) {
    const bool tail = half_tail && (s % nsteps) == nsteps - 1;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      if (kt == 1 && tail) break;
      i32x8_t a[4], bb[4];
      int sa[4], sb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (4 * wm + i) * 16 + (lane & 15), seg = kt * 4 + (lane >> 4);
        const uint4 u = *reinterpret_cast<const uint4*>(st + row * 128 + ((seg ^ (row & 7)) << 4));
        a[i] = i32x8_t{(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
        sa[i] = st[kGA + kGB + row * 8 + kt * 4 + (lane >> 4)];
        const int qq = (4 * wn + i) * 2 + kt;
        const uint4 v = *reinterpret_cast<const uint4*>(st + kGA + qq * 1024 + lane * 16);
        bb[i] = i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        sb[i] = st[kGA + kGB + kGSA + qq * 64 + lane];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], bb[j], acc[i][j], 4, 4, 0, sa[i], 0,
                                                                        sb[j]);
    }
  };

  // Lane l of MFMA tile (i, j) holds column l % 16 and rows 4 (l / 16) + v.
  auto epilogue = [&](int q) __attribute__((always_inline)) {
    const TileDesc d = desc[q];
    const int col = lane & 15;
    if constexpr (MODE == kG_Down) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = (4 * wm + i) * 16 + 4 * (lane >> 4) + v;
          if (m < d.rows) {
            const size_t o = (size_t)(d.row0 + m) * P.H + d.nt * kGBN + (4 * wn) * 16 + col;
            if (B.yb) {
#pragma unroll
              for (int j = 0; j < 4; ++j) B.yb[o + 16 * j] = f32_to_bf16_rne(acc[i][j][v]);
            } else {
#pragma unroll
              for (int j = 0; j < 4; ++j) B.y[o + 16 * j] = acc[i][j][v];
            }
          }
        }
    } else {
      // W13 row groups alternate gate / up, so MFMA columns j = 0, 1 and 2, 3
      // are (gate, up) of two 16-column pairs: 32 SwiGLU columns per row, one
      // MXFP4 block, starting at intermediate column d.nt * 128 + 32 wn.
      const int cb = d.nt * 128 + 32 * wn;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float h0 = silu_f32(acc[i][0][v]) * acc[i][1][v];
          const float h1 = silu_f32(acc[i][2][v]) * acc[i][3][v];
          const float amax = row16_max(fmaxf(fabsf(h0), fabsf(h1)));
          int ex = 0;
          if (amax != 0.f) ex = min(127, max(-127, ilog2_f32(amax) - 2));
          const float inv = ex == 127 ? __uint_as_float(0x00400000u) : __uint_as_float((uint32_t)(127 - ex) << 23);
          const uint32_t c0 = e2m1_mag_rne(fabsf(h0 * inv)) | ((__float_as_uint(h0) >> 28) & 8u);
          const uint32_t c1 = e2m1_mag_rne(fabsf(h1 * inv)) | ((__float_as_uint(h1) >> 28) & 8u);
          // bytes of the row: byte b = codes of columns 2b (low nibble) and
          // 2b + 1; lane 14 of each 16-lane row gathers bytes 0-7 (pair 0)
          // and 8-15 (pair 1) by DPP row shifts and stores all 16
          uint32_t ba = c0 | (dpp_u32<kDppQuadXor1>(c0) << 4), bb = c1 | (dpp_u32<kDppQuadXor1>(c1) << 4);
          ba = dpp_u32<kDppRowShr2>(ba) | (ba << 8);     // lanes 4j + 2: bytes 2j, 2j + 1
          bb = dpp_u32<kDppRowShr2>(bb) | (bb << 8);
          ba = dpp_u32<kDppRowShr4>(ba) | (ba << 16);    // lanes 8j + 6: bytes 4j .. 4j + 3
          bb = dpp_u32<kDppRowShr4>(bb) | (bb << 16);
          const uint32_t la = dpp_u32<kDppRowShr8>(ba), lb = dpp_u32<kDppRowShr8>(bb);  // lane 14: bytes 0-3
          const int m = (4 * wm + i) * 16 + 4 * (lane >> 4) + v;
          if (m < d.rows) {
            const size_t p = (size_t)(d.row0 + m);
            if (col == 14) *reinterpret_cast<uint4*>(B.hq + p * (P.I / 2) + cb / 2) = make_uint4(la, ba, lb, bb);
            if (col == 0) B.hs[p * (P.I / 32) + cb / 32] = (uint8_t)(ex + 127);
          }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };

  // ---- the pipeline: steps 0 .. NS-2 in flight before the first; step s
  // waits for its own loads (the NS - 2 later steps' loads stay in flight),
  // barriers, refills the buffer step s - 1 used with step s + NS - 1 (past
  // the end: the last step again, never read), and computes.
  const int last = nsteps_total - 1;
  issue(0, stage_buf<0>());
  issue(min(1, last), stage_buf<1>());
  auto step = [&](int s, auto bufc) __attribute__((always_inline)) {
    constexpr int I = decltype(bufc)::value;
    if (wave < 4) wait_vm<(kGStages - 2) * 8>();
    else wait_vm<(kGStages - 2) * 7>();
    lds_sync();
    issue(min(s + kGStages - 1, last), stage_buf<(I + kGStages - 1) % kGStages>());
    compute(s, stage_buf<I>());
    if ((s % nsteps) == nsteps - 1) epilogue(s / nsteps);
  };
  int s = 0;
  for (; s + 3 <= nsteps_total; s += 3) {
    step(s, std::integral_constant<int, 0>{});
    step(s + 1, std::integral_constant<int, 1>{});
    step(s + 2, std::integral_constant<int, 2>{});
  }
  if (s < nsteps_total) step(s, std::integral_constant<int, 0>{});
  if (s + 1 < nsteps_total) step(s + 1, std::integral_constant<int, 1>{});
  wait_vm<0>();  // no load into this workgroup's LDS outlives it
}

// Upper bound on the tiles of one launch.
static long long fp4_max_tiles(const FfnParams& P, int NT) {
  const long long rows = (long long)P.T * P.k;
  long long mt = (rows + kGBM - 1) / kGBM + std::min<long long>(P.E, rows);
  if (P.shared_blob) mt += (P.T + kGBM - 1) / kGBM;
  return mt * NT;
}

static int cu_count_fp4() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    n = cus;
  }
  return n;
}

// Whether a projection of N output columns can run here (else the caller
// uses the 128 x 128 kernel).
bool fp4_gemm_fits(const FfnParams& P, int N, int K, bool gateup) {
  if (N % kGBN != 0) return false;
  if (gateup && (K + 255) / 256 < 2) return false;  // the perm entries arrive a tile ahead
  const int G = cu_count_fp4() / 8 * 8;
  if (G < 8) return false;
  const long long per = (fp4_max_tiles(P, N / kGBN) + G - 1) / G + 1;
  return per <= kGMaxTiles && (size_t)(P.E + 1) * 4 <= (size_t)kGStages * kGStage;
}

hipError_t launch_fp4_gemm(const FfnParams& P, const MfmaBufs& B, bool down, hipStream_t s) {
  const int G = cu_count_fp4() / 8 * 8;
  if (down) launch(k_fp4_gemm<kG_Down>, dim3(G), dim3(512), 0, s, P, B);
  else launch(k_fp4_gemm<kG_GateUp>, dim3(G), dim3(512), 0, s, P, B);
  return hipGetLastError();
}

}  // namespace moe
