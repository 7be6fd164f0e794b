// Prefill path: persistent grouped GEMMs for the gate/up projection (+
// SwiGLU) and the down projection, in two forms:
//  - k_fp4_gemm: MXFP4 weights x MXFP4 activations on the block-scaled FP4
//    matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4, both operands E2M1
//    with one E8M0 scale per 32 K-values per row); the gate/up epilogue
//    MXFP4-encodes its SwiGLU output for the down projection;
//  - k_bf16_gemm: BF16 weights x bf16 activations on
//    v_mfma_f32_16x16x32_bf16; h is stored as bf16.
//
// Method: the expert FFN of a sparse MoE layer (pages as for the GEMV path);
// the activation precision of the FP4 form (x and the SwiGLU output
// MXFP4-encoded per row per 32 values) is this library's reading of a
// 4-bit-weight GEMM on FP4 matrix cores.
//
// Design for gfx950 (both forms; the FP4 form's differences are listed at
// its kernel):
//  - A persistent grid loops over output tiles of 128 rows x N columns.
//    XCD x takes the x-th eighth of the tile list (an expert's tiles share
//    one L2) and deals it round-robin to its workgroups, so they work on
//    neighbouring tiles, which share a weight block, at the same time.
//  - The BF16 form: one workgroup of 4 waves per CU, tiles 128 x 512; wave w
//    computes all 128 rows x columns 128 w .. 128 w + 127: 8 x 8 MFMA tiles,
//    256 accumulators (the AGPRs), so every LDS fragment feeds 8 MFMAs.
//  - K advances one blob K-tile per step.  A step's operands arrive by
//    direct global->LDS loads into a ring of three stage buffers, issued
//    three steps ahead across tile boundaries: no registers hold loads in
//    flight.
//  - Fragments are double-buffered in registers: step s's MFMAs run on
//    fragments read during step s - 1, while step s + 1's fragments are read
//    between them; the loads of step s + 3 (into the buffer step s's
//    fragments came from) go out between the MFMA groups too, so LDS latency
//    and waits for texture-unit slots overlap matrix-core work.
//  - Every wave issues a fixed number of loads per step, so "stage s has
//    landed" is an s_waitcnt vmcnt with a compile-time count; one LDS-only
//    barrier per step publishes the stage and frees the one read before.
//  - Each tile's expert, rows and column block come from descriptors built
//    in LDS at the start: the loop issues no global loads besides the ring.
//  - The weights are the MFMA's first operand, so a lane's accumulator holds
//    four consecutive output columns of one row.
//  - Epilogues stage their output in LDS and store whole row segments: a
//    store instruction that touches 16 rows costs the texture-address unit
//    about as much as four contiguous ones.
#include <type_traits>

#include "ffn_common.h"
#include "wave.h"

namespace moe {

// ---------------------------------------------------------------- the GEMM

// down: bf16 expert outputs (yb) or fp32 (y)
enum { kG_GateUp = 0, kG_Down = 1, kG_DownF32 = 2 };

// the BF16 form
constexpr int kGBM = 128, kGBN = 512;
constexpr int kGA = 128 * 64;            // A: 128 rows x 64 bytes (32 bf16 values)
constexpr int kGB = 32 * 1024;           // B: 32 row groups x one 1 KiB tile
constexpr int kGStage = kGA + kGB;
constexpr int kGStages = 3;
// epilogue staging: four waves x 16 rows x 256 B (down) or x 128 B (h)
constexpr int kGStaging = 4 * 4096;
constexpr int kGMaxTiles = 64;           // tiles per workgroup (descriptors in LDS)
constexpr int kGThreads = 256;

// The stage ring (indexed at run time: every fragment read is a per-lane
// base plus the stage's offset plus an immediate) and the staging area.
__shared__ __align__(16) uint8_t g_ring[kGStages * kGStage];
__shared__ __align__(16) uint8_t g_stg[kGStaging];

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
// dst: LDS byte address
__device__ __forceinline__ void dma16(const void* src, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src),
               "s"(__builtin_amdgcn_readfirstlane(dst))
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* src, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src),
               "s"(__builtin_amdgcn_readfirstlane(dst))
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

// Two E2M1 codes (a in bits 3:0, b in bits 7:4) of a / 2^e and b / 2^e,
// where 2^e is the normal fp32 `scale` (the conversion uses its exponent
// alone): round to nearest even, saturate at +-6.
__device__ __forceinline__ uint32_t e2m1_pair(float a, float b, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, scale, 0) & 0xFFu;
}

// BF16 weights x bf16 activations on v_mfma_f32_16x16x32_bf16: K-tiles of
// 32 values, 64 bytes per A row and 1 KiB per weight row group per step, no
// scales; A operands row-major: x token rows gathered through the
// permutation, h in permutation order.
template <int MODE>
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_bf16_gemm(FfnParams P, MfmaBufs B) {
  __shared__ TileDesc desc[kGMaxTiles];
  // wave-uniform values in scalar registers (the compiler cannot prove it)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = MODE == kG_GateUp ? P.H : P.I;
  const int NT = (MODE == kG_GateUp ? 2 * P.I : P.H) / kGBN;
  constexpr int kKT = 32;     // K values per step (one blob K-tile)
  const int nsteps = K / kKT;
  // rows of the A operands (routed rows, then shared rows)
  const uint32_t rtot = P.T * P.k + (P.shared_blob ? P.T : 0);
  // A operand bytes between consecutive K-tiles of one row, and between rows
  const size_t a_kstride = 64;
  const uint32_t a_rowbytes = (uint32_t)K * 2;
  // constant loads per step and wave (the vmcnt bookkeeping)
  constexpr int kLoads = 10;

  // ---- the tile list: experts in id order, each expert's column blocks,
  // each column block's row tiles (fastest); the shared expert's tiles last.
  int* pre = reinterpret_cast<int*>(g_ring);  // [E + 1], in the (still idle) stage area
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
  // XCD x (workgroups b with b % 8 == x) takes the x-th eighth of the list
  // and deals it round-robin to its workgroups: at any time they work on
  // neighbouring tiles, which share an expert's weight block (row tiles are
  // the fastest index) in that XCD's L2.
  const int G = gridDim.x, b = blockIdx.x, per_xcd = G / 8, x = b % 8, w = b / 8;
  const int X0 = (int)((long long)total * x / 8), X1 = (int)((long long)total * (x + 1) / 8);
  const int ntile = X1 - X0 > w ? (X1 - X0 - w + per_xcd - 1) / per_xcd : 0;  // <= kGMaxTiles (launcher)
  for (int q = tid; q < ntile; q += kGThreads) {
    const int L = X0 + w + q * per_xcd;
    TileDesc d;
    if (L >= routed) {
      const int local = L - routed, nrt = (P.T + kGBM - 1) / kGBM;
      const int m0 = (local % nrt) * kGBM;
      d.slot = -1;
      d.row0 = P.T * P.k + m0;
      d.rows = min(kGBM, P.T - m0);
      d.nt = local / nrt;
    } else {
      int lo = 0, hi = E - 1;  // expert e with pre[e] <= L < pre[e + 1]
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= L) lo = mid; else hi = mid - 1;
      }
      const int local = L - pre[lo], nrt = (P.counts[lo] + kGBM - 1) / kGBM;
      const int m0 = (local % nrt) * kGBM;
      d.slot = P.slot_of_expert[lo];
      d.row0 = P.offsets[lo] + m0;
      d.rows = min(kGBM, P.counts[lo] - m0);
      d.nt = local / nrt;
    }
    desc[q] = d;
  }
  lds_barrier();
  if (ntile == 0) return;
  const int nsteps_total = ntile * nsteps;

  const uint8_t* abase = MODE == kG_GateUp ? reinterpret_cast<const uint8_t*>(P.x)
                                           : reinterpret_cast<const uint8_t*>(B.hb);
  static_assert(MODE == kG_GateUp || MODE == kG_Down || MODE == kG_DownF32, "mode");
  const size_t off_w = MODE == kG_GateUp ? P.L.off_w13 : P.L.off_w2;
  const uint32_t wstride = (uint32_t)nsteps * kTileBytes;  // weight bytes per row group

  auto uniform_desc = [&](int q) __attribute__((always_inline)) -> TileDesc {
    TileDesc d;
    d.slot = __builtin_amdgcn_readfirstlane(desc[q].slot);
    d.row0 = __builtin_amdgcn_readfirstlane(desc[q].row0);
    d.rows = __builtin_amdgcn_readfirstlane(desc[q].rows);
    d.nt = __builtin_amdgcn_readfirstlane(desc[q].nt);
    return d;
  };

  // Loads of one step (K-tile ks of a tile) into a stage buffer, 10 slots:
  //   1-2: A chunk 2 wave + J - 1 (rows 16 c .. 16 c + 15, 1 KiB)
  //   3-10: B row group nt * 32 + 8 wave + J - 3
  // A chunk c: lane l writes physical segment l % 4 of row 16 c + l / 4,
  // which holds logical segment (l % 4) ^ (l / 16) (row bits 3:2), the
  // swizzle that makes fragment reads conflict-free.
  const int aseg = (lane & 3) ^ (lane >> 4);
  // issue-side tile state, refreshed at each tile's first K-tile
  uint32_t a_off[2];
  const uint8_t* wt = nullptr;   // this wave's first B row group of the tile
  int iss_ks = 0;
  uint32_t iss_st = 0;
  // the A row of row rr of a tile (rows past the tile re-read its last row):
  // its permutation-order row, or for gate/up the token of that row
  auto a_row = [&](const TileDesc& d, int rr) __attribute__((always_inline)) -> uint32_t {
    const uint32_t r = d.row0 + min(rr, d.rows - 1);
    if constexpr (MODE == kG_GateUp) {
      if (r >= (uint32_t)(P.T * P.k)) return r - P.T * P.k;  // the shared expert: token rows
      return (uint32_t)P.perm[r] / (uint32_t)P.k;
    }
    return r;
  };
  auto issue_begin = [&](int s, const uint8_t* stp) __attribute__((always_inline)) {
    iss_st = lds_off(stp);
    const int q = s / nsteps;
    iss_ks = s - q * nsteps;
    if (iss_ks == 0) {
      const TileDesc d = uniform_desc(q);
#pragma unroll
      for (int u = 0; u < 2; ++u) a_off[u] = a_row(d, 16 * (2 * wave + u) + (lane >> 2)) * a_rowbytes + aseg * 16;
      const uint8_t* blob = d.slot < 0 ? P.shared_blob : P.slot_pool + (size_t)d.slot * P.slot_stride;
      const uint32_t g0 = (uint32_t)(d.nt * 32 + 8 * wave);
      wt = blob + off_w + (size_t)g0 * wstride;
    }
  };
  auto issue_slot = [&](auto jc) __attribute__((always_inline)) {
    constexpr int J = decltype(jc)::value;
    if constexpr (J >= 1 && J < 3) {
      dma16(abase + a_off[J - 1] + iss_ks * a_kstride, iss_st + (2 * wave + J - 1) * 1024);
    } else if constexpr (J >= 3 && J < 11) {
      dma16(wt + (size_t)(J - 3) * wstride + (size_t)iss_ks * kTileBytes + lane * 16,
            iss_st + kGA + (8 * wave + J - 3) * 1024);
    }
  };
  auto issue_all = [&](int s, const uint8_t* stp) __attribute__((always_inline)) {
    issue_begin(s, stp);
    issue_slot(std::integral_constant<int, 0>{});
    issue_slot(std::integral_constant<int, 1>{});
    issue_slot(std::integral_constant<int, 2>{});
    issue_slot(std::integral_constant<int, 3>{});
    issue_slot(std::integral_constant<int, 4>{});
    issue_slot(std::integral_constant<int, 5>{});
    issue_slot(std::integral_constant<int, 6>{});
    issue_slot(std::integral_constant<int, 7>{});
    issue_slot(std::integral_constant<int, 8>{});
    issue_slot(std::integral_constant<int, 9>{});
    issue_slot(std::integral_constant<int, 10>{});
    issue_slot(std::integral_constant<int, 11>{});
    issue_slot(std::integral_constant<int, 12>{});
  };

  // acc[i][j]: output rows 16 i + (l % 16), columns 128 wave + 16 j + 4 (l / 16) + v
  // (the weights are the MFMA's row operand)
  // (a tile's first K-tile starts the sums from zero: no accumulator is ever
  // written by a plain move, which keeps them in the AGPRs)
  f32x4_t acc[8][8];

  // Fragment set: A (rows 16 i + l % 16, K-chunk l / 16) and B (row group
  // 8 wave + j) operands, for one step.
  u32x4_t fa0[8], fb0[8], fa1[8], fb1[8];
  // fragment u (A row tile u and B row group u) of stage buffer st: per-lane
  // byte offsets, to which u adds only constants (A row 16 u + l % 16 keeps
  // the swizzle bits of row l % 16)
  const int seg = lane >> 4;
  const uint32_t a_rd = (lane & 15) * 64 + ((seg ^ (((lane & 15) >> 2) & 3)) << 4);
  const uint32_t b_rd = kGA + (8 * wave) * 1024 + lane * 16;
  auto read_frag = [&](const uint8_t* st, int u, u32x4_t* fa, u32x4_t* fb) __attribute__((always_inline)) {
    fa[u] = *reinterpret_cast<const u32x4_t*>(st + a_rd + u * 1024);
    fb[u] = *reinterpret_cast<const u32x4_t*>(st + b_rd + u * 1024);
  };

  // Epilogue of tile q (reads the accumulators); a tile of at most 64 rows
  // (full false) skips row blocks 4-7.
  bool full = true;
  auto epilogue = [&](int q) __attribute__((always_inline)) {
    const TileDesc d = uniform_desc(q);
    const int t16 = lane & 15, g = lane >> 4;
    if constexpr (MODE == kG_Down) {
      {
        // per 16-row block: the wave's 16 x 128 bf16 outputs through its own
        // 4 KiB of the staging area (16-byte granules XOR-swizzled by row),
        // then stores of 4 rows x 256 contiguous bytes
        uint8_t* ws = g_stg + wave * 4096;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
        if (i >= 4 && !full) break;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t lo = bf16x2_rne(acc[i][j][0], acc[i][j][1]);
            const uint32_t hi = bf16x2_rne(acc[i][j][2], acc[i][j][3]);
            const int gr = 2 * j + (g >> 1);  // 16-byte granule of columns 16 j + 4 g
            *reinterpret_cast<uint2*>(ws + t16 * 256 + ((gr ^ t16) << 4) + (g & 1) * 8) = make_uint2(lo, hi);
          }
#pragma unroll
          for (int pr = 0; pr < 4; ++pr) {
            const int rr = 4 * pr + (lane >> 4), gr = lane & 15;
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ws + rr * 256 + ((gr ^ rr) << 4));
            const int m = 16 * i + rr;
            if (m < d.rows)
              *reinterpret_cast<u32x4_t*>(B.yb + (size_t)(d.row0 + m) * P.H + d.nt * kGBN + 128 * wave + gr * 8) = v;
          }
        }
      }
    } else if constexpr (MODE == kG_DownF32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i >= 4 && !full) break;
        const int m = 16 * i + t16;
        if (m < d.rows) {
          const size_t o = (size_t)(d.row0 + m) * P.H + d.nt * kGBN + 128 * wave + 4 * g;
#pragma unroll
          for (int j = 0; j < 8; ++j) *reinterpret_cast<f32x4_t*>(B.y + o + 16 * j) = acc[i][j];
        }
      }
    } else {
      // h = bf16(silu(gate) * up) for SwiGLU columns d.nt * 256 + 64 wave
      // + 16 p + 4 g + v (MFMA tiles j = 2p gate, 2p + 1 up), row-major
      // [R][I]: per 16-row block through the wave's own 2 KiB of staging,
      // then stores of 8 rows x 128 contiguous bytes
      uint8_t* ws = g_stg + wave * 4096;
      const int cb = d.nt * 256 + 64 * wave;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i >= 4 && !full) break;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          uint32_t w2[2];
#pragma unroll
          for (int v = 0; v < 2; ++v) {
            const float h0 = silu_fast(acc[i][2 * p][2 * v]) * acc[i][2 * p + 1][2 * v];
            const float h1 = silu_fast(acc[i][2 * p][2 * v + 1]) * acc[i][2 * p + 1][2 * v + 1];
            w2[v] = bf16x2_rne(h0, h1);
          }
          // row t16, 16-byte granule 2p + g / 2 of the row's 128 bytes, XOR-swizzled by row
          const int gr = 2 * p + (g >> 1);
          *reinterpret_cast<uint2*>(ws + t16 * 128 + (((gr ^ t16) & 7) << 4) + (g & 1) * 8) = make_uint2(w2[0], w2[1]);
        }
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const int rr = 8 * pr + (lane >> 3), gr = lane & 7;
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ws + rr * 128 + (((gr ^ rr) & 7) << 4));
          const int m = 16 * i + rr;
          if (m < d.rows)
            *reinterpret_cast<u32x4_t*>(B.hb + (size_t)(d.row0 + m) * P.I + cb + gr * 8) = v;
        }
      }
    }
  };

  // ---- the pipeline.  Prologue: stages 0-2 issued, stage 0's fragments read.
  // Step s: wait for stage s + 1 (stage s + 2 stays in flight), barrier
  // (stage s + 1 published; stage s's buffer, read during step s - 1, free),
  // then 8 groups of 8 MFMAs on step s's fragments, each followed by the
  // reads of one fragment of stage s + 1 and one or two loads of stage s + 3
  // into stage s's buffer (past the end: the last stage again, never read).
  const int last = nsteps_total - 1;
  issue_all(0, g_ring);
  issue_all(min(1, last), g_ring + kGStage);
  issue_all(min(2, last), g_ring + 2 * kGStage);
  wait_vm<2 * kLoads>();
  lds_sync();
#pragma unroll
  for (int u = 0; u < 8; ++u) read_frag(g_ring, u, fa0, fb0);

  int cur = 0, s = 0;  // global step and the stage buffer it reads
  auto step = [&](auto zc, auto pc, u32x4_t* fa, u32x4_t* fb, u32x4_t* na, u32x4_t* nb)
      __attribute__((always_inline)) {
    constexpr bool first = decltype(zc)::value;     // a tile's first K-tile
    constexpr bool prefetch = decltype(pc)::value;  // read the next step's fragments
    wait_vm<kLoads>();
    lds_sync();
    const int nxt = cur == kGStages - 1 ? 0 : cur + 1;
    const uint8_t* stn = g_ring + nxt * kGStage;
    issue_begin(min(s + kGStages, last), g_ring + cur * kGStage);
    issue_slot(std::integral_constant<int, 0>{});
    auto group = [&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fb[j]),
                                                             __builtin_bit_cast(bf16x8_t, fa[i]),
                                                             first ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[i][j], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (prefetch) read_frag(stn, j, na, nb);
      if constexpr (j < 4) {
        issue_slot(std::integral_constant<int, 2 * j + 1>{});
        issue_slot(std::integral_constant<int, 2 * j + 2>{});
      } else {
        issue_slot(std::integral_constant<int, j + 5>{});
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    group(std::integral_constant<int, 0>{});
    group(std::integral_constant<int, 1>{});
    group(std::integral_constant<int, 2>{});
    group(std::integral_constant<int, 3>{});
    group(std::integral_constant<int, 4>{});
    group(std::integral_constant<int, 5>{});
    group(std::integral_constant<int, 6>{});
    group(std::integral_constant<int, 7>{});
    // The step's MFMAs stay in the step: without a use here the compiler
    // sinks side-effect-free MFMAs whose results are next read in a later
    // block (a tile's first step into the next one, its last step into the
    // epilogue), and they lose their place between the loads.
#pragma unroll
    for (int i = 0; i < 8; ++i)
      asm volatile("" ::"a"(acc[i][0]), "a"(acc[i][1]), "a"(acc[i][2]), "a"(acc[i][3]), "a"(acc[i][4]),
                   "a"(acc[i][5]), "a"(acc[i][6]), "a"(acc[i][7]));
    cur = nxt;
    ++s;
  };
  // nsteps is even (checked by the launcher): a tile's steps alternate
  // between the two fragment sets, starting with set 0.  The last step of a
  // tile reads no fragments: the epilogue runs with only the accumulators
  // live, and the next tile's first fragments are read after it.
  const std::true_type yes;
  const std::false_type no;
  // A tile of at most 64 rows skips the epilogue work of its empty row
  // blocks 4-7.  (Its matrix instructions for them still run: a branch
  // around them splits the accumulator updates, and the kernel then spills.)
  for (int q = 0; q < ntile; ++q) {
    full = __builtin_amdgcn_readfirstlane(desc[q].rows) > 64;
    step(yes, yes, fa0, fb0, fa1, fb1);
    for (int ks = 1; ks < nsteps - 1; ks += 2) {
      step(no, yes, fa1, fb1, fa0, fb0);
      step(no, yes, fa0, fb0, fa1, fb1);
    }
    step(no, no, fa1, fb1, fa0, fb0);
    epilogue(q);
    if (q + 1 < ntile) {
#pragma unroll
      for (int u = 0; u < 8; ++u) read_frag(g_ring + cur * kGStage, u, fa0, fb0);
    }
  }
  wait_vm<0>();  // no load into this workgroup's LDS outlives it
}

// ------------------------------------------------- the FP4 GEMM, two per CU
// The FP4 projections run on a narrower form of the kernel above, sized so
// that two workgroups share a CU: the FP4 matrix instruction issues at about
// twice the rate with two waves per SIMD as with one.
//  - Both A operands are MXFP4 rows in permutation order (routed rows, then
//    the shared expert's token rows; R in all), stored K-tile-major: codes
//    [K/128][R][64 B], scales [K/128][R][4 B].  x arrives so from the row
//    quantiser; the gate/up epilogue writes its SwiGLU output so.  Every
//    direct load of an A operand or its scales then reads contiguous memory.
//  - The gate/up epilogue encodes SwiGLU outputs to E2M1 in pairs with
//    v_cvt_scalef32_pk_fp4_f32 (round to nearest even, saturating at 6, as
//    the MXFP4 encoding here requires) after a 4-lane maximum per 32-column
//    block.
//  - Tiles of 128 rows x 256 columns; wave w computes all 128 rows x columns
//    64 w .. 64 w + 63: 8 x 4 MFMA tiles, 128 accumulators, which leaves
//    the other 128 of a wave's 256 registers (two waves per SIMD) for
//    operands and addresses.
//  - A step's operands (A 8 KiB, B 16 KiB, scales 1.5 KiB) arrive in a ring
//    of three 25.5 KiB stages, three steps ahead, as above.  A workgroup
//    holds 77.3 KiB of LDS, so two fit the CU's 160 KiB; the epilogue stages
//    its output in the stage buffer of the tile's last step, whose loads are
//    deferred until the epilogue is done.
//  - An A fragment is read right after the MFMAs that consume its
//    predecessor (one register set; the next step's fragment replaces the
//    current one), B fragments are double-buffered: 80 operand registers.
//  - Gate/up: wave w's four weight row groups are (gate, up, gate, up) of
//    SwiGLU columns 32 w .. 32 w + 31 of the tile's 128, one MXFP4 block,
//    and the tile's SwiGLU output is one K-tile of the down projection.
constexpr int kHBN = 256;
constexpr int kHA = 128 * 64;
constexpr int kHB = 16 * 1024;
constexpr int kHSA = 128 * 4;
constexpr int kHSB = 16 * 64;
constexpr int kHStage = kHA + kHB + kHSA + kHSB;
constexpr int kHStages = 3;
constexpr int kHMaxTiles = 48;
static_assert(kHStage >= kGBM * 64 + kGBM * 4 && kHStage >= 4 * 2048, "epilogue staging fits a stage");

__shared__ __align__(16) uint8_t h_ring[kHStages * kHStage];

template <int MODE>
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_fp4_gemm(FfnParams P, MfmaBufs B) {
  __shared__ TileDesc desc[kHMaxTiles];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = MODE == kG_GateUp ? P.H : P.I;
  const int NT = (MODE == kG_GateUp ? 2 * P.I : P.H) / kHBN;
  const int nsteps = K / 128;  // even (launcher)
  const uint32_t rtot = P.T * P.k + (P.shared_blob ? P.T : 0);
  const size_t a_kstride = (size_t)rtot * 64, as_kstride = (size_t)rtot * 4;
  // loads per step and wave: waves 0-1 also load the A scales
  constexpr int kLoadsHi = 8, kLoadsLo = 7;

  // ---- the tile list (as above, 256-column blocks)
  int* pre = reinterpret_cast<int*>(h_ring);
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
  const int G = gridDim.x, b = blockIdx.x, per_xcd = G / 8, x = b % 8, w = b / 8;
  const int X0 = (int)((long long)total * x / 8), X1 = (int)((long long)total * (x + 1) / 8);
  const int ntile = X1 - X0 > w ? (X1 - X0 - w + per_xcd - 1) / per_xcd : 0;  // <= kHMaxTiles (launcher)
  for (int q = tid; q < ntile; q += kGThreads) {
    const int L = X0 + w + q * per_xcd;
    TileDesc d;
    if (L >= routed) {
      const int local = L - routed, nrt = (P.T + kGBM - 1) / kGBM;
      const int m0 = (local % nrt) * kGBM;
      d.slot = -1;
      d.row0 = P.T * P.k + m0;
      d.rows = min(kGBM, P.T - m0);
      d.nt = local / nrt;
    } else {
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= L) lo = mid; else hi = mid - 1;
      }
      const int local = L - pre[lo], nrt = (P.counts[lo] + kGBM - 1) / kGBM;
      const int m0 = (local % nrt) * kGBM;
      d.slot = P.slot_of_expert[lo];
      d.row0 = P.offsets[lo] + m0;
      d.rows = min(kGBM, P.counts[lo] - m0);
      d.nt = local / nrt;
    }
    desc[q] = d;
  }
  lds_barrier();
  if (ntile == 0) return;
  const int nsteps_total = ntile * nsteps;

  const uint8_t* abase = MODE == kG_GateUp ? B.xq : B.hq;
  const uint8_t* asbase = MODE == kG_GateUp ? B.xs : B.hs;
  const size_t off_w = MODE == kG_GateUp ? P.L.off_w13 : P.L.off_w2;
  const size_t off_s = MODE == kG_GateUp ? P.L.off_s13 : P.L.off_s2;
  const uint32_t wstride = (uint32_t)nsteps * kTileBytes;

  auto uniform_desc = [&](int q) __attribute__((always_inline)) -> TileDesc {
    TileDesc d;
    d.slot = __builtin_amdgcn_readfirstlane(desc[q].slot);
    d.row0 = __builtin_amdgcn_readfirstlane(desc[q].row0);
    d.rows = __builtin_amdgcn_readfirstlane(desc[q].rows);
    d.nt = __builtin_amdgcn_readfirstlane(desc[q].nt);
    return d;
  };

  // Loads of one step into a stage buffer, 8 slots:
  //   0: A scales (waves 0-1): row 64 wave + l, the dword of K-tile ks
  //   1-2: A chunk 2 wave + J - 1 (rows 16 c .. 16 c + 15, 1 KiB, swizzled as above)
  //   3-6: B row group nt * 16 + 4 wave + J - 3
  //   7: B scale tiles of row groups nt * 16 + 4 wave + l / 16
  const int aseg = (lane & 3) ^ (lane >> 4);
  uint32_t a_off[2], as_off = 0;
  const uint8_t* wt = nullptr;
  const uint8_t* wst = nullptr;
  int iss_ks = 0;
  uint32_t iss_st = 0;
  auto a_row = [&](const TileDesc& d, int rr) __attribute__((always_inline)) -> uint32_t {
    return (uint32_t)(d.row0 + min(rr, d.rows - 1));
  };
  auto issue_begin = [&](int s, const uint8_t* stp) __attribute__((always_inline)) {
    iss_st = lds_off(stp);
    const int q = s / nsteps;
    iss_ks = s - q * nsteps;
    if (iss_ks == 0) {
      const TileDesc d = uniform_desc(q);
#pragma unroll
      for (int u = 0; u < 2; ++u) a_off[u] = a_row(d, 16 * (2 * wave + u) + (lane >> 2)) * 64u + aseg * 16;
      if (wave < 2) as_off = a_row(d, 64 * wave + lane) * 4u;
      const uint8_t* blob = d.slot < 0 ? P.shared_blob : P.slot_pool + (size_t)d.slot * P.slot_stride;
      const uint32_t g0 = (uint32_t)(d.nt * 16 + 4 * wave);
      wt = blob + off_w + (size_t)g0 * wstride;
      wst = blob + off_s + (size_t)g0 * nsteps * 64;
    }
  };
  auto issue_slot = [&](auto jc) __attribute__((always_inline)) {
    constexpr int J = decltype(jc)::value;
    if constexpr (J == 0) {
      if (wave < 2) dma4(asbase + as_off + iss_ks * as_kstride, iss_st + kHA + kHB + wave * 256);
    } else if constexpr (J < 3) {
      dma16(abase + a_off[J - 1] + iss_ks * a_kstride, iss_st + (2 * wave + J - 1) * 1024);
    } else if constexpr (J < 7) {
      dma16(wt + (size_t)(J - 3) * wstride + (size_t)iss_ks * kTileBytes + lane * 16,
            iss_st + kHA + (4 * wave + J - 3) * 1024);
    } else {
      dma4(wst + ((size_t)(lane >> 4) * nsteps + iss_ks) * 64 + (lane & 15) * 4,
           iss_st + kHA + kHB + kHSA + wave * 256);
    }
  };
  auto issue_all = [&](int s, const uint8_t* stp) __attribute__((always_inline)) {
    issue_begin(s, stp);
    issue_slot(std::integral_constant<int, 0>{});
    issue_slot(std::integral_constant<int, 1>{});
    issue_slot(std::integral_constant<int, 2>{});
    issue_slot(std::integral_constant<int, 3>{});
    issue_slot(std::integral_constant<int, 4>{});
    issue_slot(std::integral_constant<int, 5>{});
    issue_slot(std::integral_constant<int, 6>{});
    issue_slot(std::integral_constant<int, 7>{});
  };

  // acc[i][j]: output rows 16 i + (l % 16), columns 64 wave + 16 j + 4 (l / 16) + v
  f32x4_t acc[8][4];
  // A fragments (rows 16 i + l % 16, K-chunk l / 16) and their scale bytes:
  // one set; B fragments (row group 4 wave + j): two
  u32x4_t fa[8], fb0[4], fb1[4];
  int sa[8], sb0[4], sb1[4];
  const int seg = lane >> 4;
  const uint32_t a_rd = (lane & 15) * 64 + ((seg ^ (((lane & 15) >> 2) & 3)) << 4);
  const uint32_t sa_rd = kHA + kHB + (lane & 15) * 4 + seg;
  const uint32_t b_rd = kHA + (4 * wave) * 1024 + lane * 16;
  const uint32_t sb_rd = kHA + kHB + kHSA + (4 * wave) * 64 + lane;
  auto read_a = [&](const uint8_t* st, int i) __attribute__((always_inline)) {
    fa[i] = *reinterpret_cast<const u32x4_t*>(st + a_rd + i * 1024);
    sa[i] = st[sa_rd + i * 64];
  };
  auto read_b = [&](const uint8_t* st, int j, u32x4_t* fb, int* sb) __attribute__((always_inline)) {
    fb[j] = *reinterpret_cast<const u32x4_t*>(st + b_rd + j * 1024);
    sb[j] = st[sb_rd + j * 64];
  };

  bool full = true;
  // Epilogue of tile q through the staging buffer stg (a free stage buffer).
  auto epilogue = [&](int q, uint8_t* stg) __attribute__((always_inline)) {
    const TileDesc d = uniform_desc(q);
    // The lane id through an empty asm: the epilogue's lane-dependent
    // offsets are then computed here, per tile, instead of being hoisted
    // out of the tile loop, where they would hold registers (and spill)
    // across the matrix loop.
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int t16 = lane & 15, g = lane >> 4;
    if constexpr (MODE == kG_Down) {
      // per 16-row block: the wave's 16 x 64 bf16 outputs through its own
      // 2 KiB (16-byte granules XOR-swizzled by row), then stores of 8 rows x
      // 128 contiguous bytes
      uint8_t* ws = stg + wave * 2048;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i >= 4 && !full) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo = bf16x2_rne(acc[i][j][0], acc[i][j][1]);
          const uint32_t hi = bf16x2_rne(acc[i][j][2], acc[i][j][3]);
          const int gr = 2 * j + (g >> 1);  // 16-byte granule of columns 16 j + 4 g
          *reinterpret_cast<uint2*>(ws + t16 * 128 + (((gr ^ t16) & 7) << 4) + (g & 1) * 8) = make_uint2(lo, hi);
        }
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const int rr = 8 * pr + (lane >> 3), gr = lane & 7;
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ws + rr * 128 + (((gr ^ rr) & 7) << 4));
          const int m = 16 * i + rr;
          if (m < d.rows)
            *reinterpret_cast<u32x4_t*>(B.yb + (size_t)(d.row0 + m) * P.H + d.nt * kHBN + 64 * wave + gr * 8) = v;
        }
      }
    } else if constexpr (MODE == kG_DownF32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i >= 4 && !full) break;
        const int m = 16 * i + t16;
        if (m < d.rows) {
          const size_t o = (size_t)(d.row0 + m) * P.H + d.nt * kHBN + 64 * wave + 4 * g;
#pragma unroll
          for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4_t*>(B.y + o + 16 * j) = acc[i][j];
        }
      }
    } else {
      // Lane l holds SwiGLU columns 4 (l / 16) + v and 16 + 4 (l / 16) + v of
      // the wave's block (MFMA tiles 0, 1: gate, up of the first 16; 2, 3 of
      // the next 16): the block's 32 values of a row sit in lanes l % 16 +
      // 16 g, g = 0..3.  Staging: codes [128 rows][64 B], then scales [128][4 B].
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i >= 4 && !full) break;
        const int m = 16 * i + t16;
        float h[8];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          h[v] = silu_fast(acc[i][0][v]) * acc[i][1][v];
          h[4 + v] = silu_fast(acc[i][2][v]) * acc[i][3][v];
        }
        float amax = 0.f;
#pragma unroll
        for (int v = 0; v < 8; ++v) amax = fmaxf(amax, fabsf(h[v]));
        amax = max_rows4(amax);
        const int ex = amax != 0.f ? min(127, max(-127, ilog2_f32(amax) - 2)) : 0;
        // The block scale 2^ex as a normal fp32; for ex = -127 (every |h| <
        // 2^-124) the scale 2^-126 with doubled values gives the same
        // quotient, h / 2^-127 = 2h / 2^-126 (doubling such small values is
        // exact).
        const float sc = __uint_as_float((uint32_t)(max(ex, -126) + 127) << 23);
        if (ex == -127) {
#pragma unroll
          for (int v = 0; v < 8; ++v) h[v] *= 2.0f;
        }
        const uint32_t lo = e2m1_pair(h[0], h[1], sc) | (e2m1_pair(h[2], h[3], sc) << 8);
        const uint32_t hi = e2m1_pair(h[4], h[5], sc) | (e2m1_pair(h[6], h[7], sc) << 8);
        // (row m = 16 i + t16: a per-lane base plus a constant per i)
        uint8_t* dst = stg + t16 * 64 + 16 * wave + 2 * g + i * 1024;
        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)lo;
        *reinterpret_cast<uint16_t*>(dst + 8) = (uint16_t)hi;
        if (g == 0) stg[kGBM * 64 + t16 * 4 + wave + i * 64] = (uint8_t)(ex + 127);
      }
      lds_sync();
      // down K-tile nt of the tile's rows: 16 rows x 64 B (1 KiB contiguous)
      // per store, the scales 64 rows x 4 B per store
      // (row 16 c + l / 4, bytes 16 (l % 4): byte 1024 c + 16 l of the chunk run)
      uint8_t* hq = B.hq + ((size_t)d.nt * rtot + d.row0) * 64 + lane * 16;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c = 2 * wave + u, row = 16 * c + (lane >> 2);
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + c * 1024 + lane * 16);
        if (row < d.rows) *reinterpret_cast<u32x4_t*>(hq + c * 1024) = v;
      }
      if (wave < 2) {
        const int row = 64 * wave + lane;
        const uint32_t v = *reinterpret_cast<const uint32_t*>(stg + kGBM * 64 + row * 4);
        if (row < d.rows) *reinterpret_cast<uint32_t*>(B.hs + ((size_t)d.nt * rtot + d.row0 + row) * 4) = v;
      }
    }
  };

  // ---- the pipeline (as above).  Step s: wait for stage s + 1, barrier,
  // then 8 groups of 4 MFMAs (A row tile i against the wave's 4 B
  // fragments), each followed by the read of A fragment i (and every other
  // group a B fragment) of stage s + 1 and one load of stage s + 3 into
  // stage s's buffer.  A tile's last step reads nothing and defers its loads
  // until the epilogue has used that buffer.
  const int last = nsteps_total - 1;
  issue_all(0, h_ring);
  issue_all(min(1, last), h_ring + kHStage);
  issue_all(min(2, last), h_ring + 2 * kHStage);
  if (wave < 2) wait_vm<2 * kLoadsHi>();
  else wait_vm<2 * kLoadsLo>();
  lds_sync();
#pragma unroll
  for (int i = 0; i < 8; ++i) read_a(h_ring, i);
#pragma unroll
  for (int j = 0; j < 4; ++j) read_b(h_ring, j, fb0, sb0);

  int cur = 0, s = 0;
  auto step = [&](auto zc, auto pc, u32x4_t* fb, int* sb, u32x4_t* nb, int* nsb) __attribute__((always_inline)) {
    constexpr bool first = decltype(zc)::value;     // a tile's first K-tile
    constexpr bool prefetch = decltype(pc)::value;  // not the tile's last K-tile
    if (wave < 2) wait_vm<kLoadsHi>();
    else wait_vm<kLoadsLo>();
    lds_sync();
    const int nxt = cur == kHStages - 1 ? 0 : cur + 1;
    const uint8_t* stn = h_ring + nxt * kHStage;
    if constexpr (prefetch) {
      issue_begin(min(s + kHStages, last), h_ring + cur * kHStage);
      issue_slot(std::integral_constant<int, 0>{});
    }
    auto group = [&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            i32x8_t{(int)fb[j].x, (int)fb[j].y, (int)fb[j].z, (int)fb[j].w, 0, 0, 0, 0},
            i32x8_t{(int)fa[i].x, (int)fa[i].y, (int)fa[i].z, (int)fa[i].w, 0, 0, 0, 0},
            first ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[i][j], 4, 4, 0, sb[j], 0, sa[i]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (prefetch) {
        read_a(stn, i);
        if constexpr (i % 2 == 0) read_b(stn, i / 2, nb, nsb);
        if constexpr (i < 7) issue_slot(std::integral_constant<int, i + 1>{});
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    group(std::integral_constant<int, 0>{});
    group(std::integral_constant<int, 1>{});
    group(std::integral_constant<int, 2>{});
    group(std::integral_constant<int, 3>{});
    group(std::integral_constant<int, 4>{});
    group(std::integral_constant<int, 5>{});
    group(std::integral_constant<int, 6>{});
    group(std::integral_constant<int, 7>{});
#pragma unroll
    for (int i = 0; i < 8; ++i)
      asm volatile("" ::"a"(acc[i][0]), "a"(acc[i][1]), "a"(acc[i][2]), "a"(acc[i][3]));
    cur = nxt;
    ++s;
  };
  const std::true_type yes;
  const std::false_type no;
  for (int q = 0; q < ntile; ++q) {
    full = __builtin_amdgcn_readfirstlane(desc[q].rows) > 64;
    step(yes, yes, fb0, sb0, fb1, sb1);
    for (int ks = 1; ks < nsteps - 1; ks += 2) {
      step(no, yes, fb1, sb1, fb0, sb0);
      step(no, yes, fb0, sb0, fb1, sb1);
    }
    const int lst = cur;  // the last step's buffer: its fragments are in registers
    step(no, no, fb1, sb1, fb0, sb0);
    epilogue(q, h_ring + lst * kHStage);
    if (q + 1 < ntile) {
      lds_sync();  // every wave is done with the staging buffer
      issue_all(min(s - 1 + kHStages, last), h_ring + lst * kHStage);
#pragma unroll
      for (int i = 0; i < 8; ++i) read_a(h_ring + cur * kHStage, i);
#pragma unroll
      for (int j = 0; j < 4; ++j) read_b(h_ring + cur * kHStage, j, fb0, sb0);
    }
  }
  wait_vm<0>();
}

// Upper bound on the tiles of one launch.
static long long fp4_max_tiles(const FfnParams& P, int NT) {
  const long long rows = (long long)P.T * P.k;
  long long mt = (rows + kGBM - 1) / kGBM + std::min<long long>(P.E, rows);
  if (P.shared_blob) mt += (P.T + kGBM - 1) / kGBM;
  return mt * NT;
}

// Persistent grid: one workgroup per CU, a multiple of the 8 XCDs.
static int fp4_grid() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    n = cus / 8 * 8;
  }
  return n;
}

// Two workgroups per CU for the FP4 form.
static int fp4_grid2() { return 2 * fp4_grid(); }

// Whether an FP4 projection of N output columns over K can run on the
// persistent kernel (else the caller uses the 128 x 128 kernel).
bool fp4_gemm_fits(const FfnParams& P, int N, int K, bool /*gateup*/) {
  if (N % kHBN != 0 || K % 256 != 0) return false;  // an even number of K-tiles
  const int G = fp4_grid2();
  if (G < 8) return false;
  const long long per = (fp4_max_tiles(P, N / kHBN) + G - 1) / G + 2;
  return per <= kHMaxTiles && (size_t)(P.E + 1) * 4 <= (size_t)kHStages * kHStage;
}

// The same for BF16 weights (K-tiles of 32: K % 64 == 0 keeps their count even).
bool bf16_gemm_fits(const FfnParams& P, int N, int K) {
  if (N % kGBN != 0 || K % 64 != 0) return false;
  const int G = fp4_grid();
  if (G < 8) return false;
  const long long per = (fp4_max_tiles(P, N / kGBN) + G - 1) / G + 2;
  return per <= kGMaxTiles && (size_t)(P.E + 1) * 4 <= (size_t)kGStages * kGStage;
}

hipError_t launch_fp4_gemm(const FfnParams& P, const MfmaBufs& B, bool down, hipStream_t s) {
  const int G = fp4_grid2();
  if (down && B.yb) launch(k_fp4_gemm<kG_Down>, dim3(G), dim3(kGThreads), 0, s, P, B);
  else if (down) launch(k_fp4_gemm<kG_DownF32>, dim3(G), dim3(kGThreads), 0, s, P, B);
  else launch(k_fp4_gemm<kG_GateUp>, dim3(G), dim3(kGThreads), 0, s, P, B);
  return hipGetLastError();
}

// The BF16-weight projections on the same persistent kernel.
hipError_t launch_bf16_gemm(const FfnParams& P, const MfmaBufs& B, bool down, hipStream_t s) {
  const int G = fp4_grid();
  if (down && B.yb) launch(k_bf16_gemm<kG_Down>, dim3(G), dim3(kGThreads), 0, s, P, B);
  else if (down) launch(k_bf16_gemm<kG_DownF32>, dim3(G), dim3(kGThreads), 0, s, P, B);
  else launch(k_bf16_gemm<kG_GateUp>, dim3(G), dim3(kGThreads), 0, s, P, B);
  return hipGetLastError();
}

}  // namespace moe
