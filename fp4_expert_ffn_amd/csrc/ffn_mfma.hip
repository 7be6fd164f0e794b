// Prefill path of the expert FFN: a grouped GEMM over (expert, 128-row tile,
// 128-column tile) work items on the gfx950 matrix cores.
//
//   FP4 : v_mfma_scale_f32_16x16x128_f8f6f4 with both operands E2M1 and one
//         E8M0 scale per 32 K-values per row (MXFP4 weights x MXFP4 activations;
//         x and the SwiGLU output are MXFP4-encoded per row, blocks of 32).
//   BF16: v_mfma_f32_16x16x32_bf16 (BF16 weights x bf16 activations; the
//         SwiGLU output is rounded to bf16 before the down projection).
//
// Method: the expert FFN of a sparse MoE layer (pages as for the GEMV path);
// the activation precision of the FP4 path is this library's reading of a
// 4-bit-weight GEMM on FP4 matrix cores.
//
// Workgroup: 256 threads = 4 waves in a 2x2 grid, each wave 64 rows x 64 cols
// (4x4 MFMA 16x16 tiles).  K-steps of 256 (FP4) or 64 (BF16), i.e. 128 bytes
// of every operand row, are staged global -> registers -> LDS
// (double-buffered) with the next steps' loads in flight during the current
// step's MFMAs.  Tiles are listed expert by expert, row tile by row tile,
// column tile fastest, and each XCD takes a contiguous range of the list:
// the workgroups running at once on an XCD then share one row tile's
// operand rows and their expert's weights in its L2.
#include <algorithm>

#include "ffn_common.h"
#include "mfma_addr.h"
#include "wave.h"

namespace moe {

constexpr int kBM = 128, kBN = 128;

// ---------------------------------------------------------------- activation quantiser

// x [rows, cols] bf16 -> q [rows, cols/2], s [rows, cols/32]; one thread per 32-block.
__global__ __launch_bounds__(256) void k_quant_mxfp4(const uint16_t* __restrict__ x, int rows, int cols,
                                                     uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const long long b = (long long)blockIdx.x * 256 + threadIdx.x;
  const int nb = cols / 32;
  if (b >= (long long)rows * nb) return;
  const long long r = b / nb;
  const int c = (int)(b % nb);
  const uint4* src = reinterpret_cast<const uint4*>(x + r * cols + c * 32);
  float v[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = src[i];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
  uint4 qq;
  uint32_t ss;
  mxfp4_encode32(v, qq, ss);
  *reinterpret_cast<uint4*>(q + r * (cols / 2) + c * 16) = qq;
  s[r * nb + c] = (uint8_t)ss;
}

// The inverse of the permutation: inv[perm[p]] = p.
__global__ __launch_bounds__(256) void k_invert(const int32_t* __restrict__ perm, int n, int32_t* __restrict__ inv) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p < n) inv[perm[p]] = p;
}

// x -> MXFP4 for the persistent FP4 GEMM, in its A-operand layout: one wave
// per token, one 32-value block per lane, written to the token's k routed
// rows (inv) and, with a shared expert, to row T*k + t, K-tile-major:
// q [cols/128][R][64 B] (block c at byte 16 (c % 4) of K-tile c / 4),
// s [cols/128][R][4 B] (byte c % 4).  The scale dword of a K-tile is
// gathered from its four lanes by DPP.
__global__ __launch_bounds__(256) void k_quant_rows(const uint16_t* __restrict__ x, int T, int cols, int k,
                                                    const int32_t* __restrict__ inv, int shared, uint32_t rtot,
                                                    uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  // Workgroup b runs on XCD b % 8, and each XCD takes a contiguous eighth of
  // the tokens: an expert's neighbouring rows (tokens close in order) are then
  // written through one L2, which merges their 64-byte code and 4-byte scale
  // pieces into whole lines.  The grid is 8 * ceil(T / 32) workgroups.
  const int per = (int)gridDim.x / 8, b = blockIdx.x;
  const int t = ((b % 8) * per + b / 8) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int nb = cols / 32;  // a multiple of 4
  // the token's destination rows, one per lane (k <= 16), loaded once ahead
  // of x: the stores below take them by lane broadcast, so a wave waits for
  // one memory latency here instead of one per destination row
  const uint32_t dst_row =
      lane < k ? (uint32_t)inv[(size_t)t * k + lane] : (lane == k ? (uint32_t)(T * k + t) : 0u);
  for (int c0 = 0; c0 < nb; c0 += 64) {
    const int c = c0 + lane;
    float v[32];
    if (c < nb) {
      const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * cols + c * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 u = src[i];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
          v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = 0.f;
    }
    uint4 qq;
    uint32_t ss;
    mxfp4_encode32(v, qq, ss);
    // quad_perm broadcasts of lanes 4m + 0..3
    const uint32_t sd = dpp_u32<0x00>(ss) | (dpp_u32<0x55>(ss) << 8) | (dpp_u32<0xAA>(ss) << 16) |
                        (dpp_u32<0xFF>(ss) << 24);
    if (c < nb) {
      const size_t kt = (size_t)(c >> 2) * rtot;
      for (int j = 0; j < k + shared; ++j) {
        const uint32_t row = (uint32_t)__builtin_amdgcn_readlane((int)dst_row, j);
        *reinterpret_cast<uint4*>(q + (kt + row) * 64 + (c & 3) * 16) = qq;
        if ((c & 3) == 0) *reinterpret_cast<uint32_t*>(s + (kt + row) * 4) = sd;
      }
    }
  }
}

hipError_t launch_quant_mxfp4(const uint16_t* x, int rows, int cols, uint8_t* q, uint8_t* s, hipStream_t st) {
  const long long n = (long long)rows * (cols / 32);
  if (n == 0) return hipSuccess;
  launch(k_quant_mxfp4, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, x, rows, cols, q, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------- tile scheduling

struct TileJob {
  const uint8_t* blob;
  int rows;    // valid rows in this tile (0: no work)
  int p0;      // perm-order row index of the tile's first row
  int shared;
  int m0;      // first row of the tile within the expert
  int nt;      // column tile
};

// Every thread of the workgroup must call this (LDS + barriers).
__device__ inline TileJob find_tile(const FfnParams& P, int NT) {
  __shared__ int pre[1024 + 2];
  __shared__ int s_info[4];
  TileJob tj{};
  const int tid = threadIdx.x;
  const int E = P.E;
  if (tid < 64) {
    int run = 0;
    for (int base = 0; base < E; base += 64) {
      const int e = base + tid;
      int t = 0;
      if (e < E) {
        const int c = P.counts[e];
        if (c > 0 && (P.mask == nullptr || P.mask[e] != 0)) t = ((c + kBM - 1) / kBM) * NT;
      }
      // inclusive wave scan
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
  __syncthreads();
  const int routed = pre[E];
  const int shared_tiles = P.shared_blob ? ((P.T + kBM - 1) / kBM) * NT : 0;
  const int total = routed + shared_tiles;
  // XCD-aware order: workgroup b runs on XCD b % 8; give each XCD a contiguous range.
  const int per = (total + 7) / 8;
  const int b = blockIdx.x;
  const int L = (b % 8) * per + b / 8;
  if (b / 8 >= per || L >= total) return tj;  // rows == 0
  if (L >= routed) {
    const int local = L - routed;
    tj.blob = P.shared_blob;
    tj.shared = 1;
    tj.nt = local % NT;
    tj.m0 = (local / NT) * kBM;
    tj.p0 = P.T * P.k;
    tj.rows = min(kBM, P.T - tj.m0);
    return tj;
  }
  // binary search: expert e with pre[e] <= L < pre[e+1]
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= L) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int c = P.counts[e], local = L - pre[e];
  tj.blob = P.slot_pool + (size_t)P.slot_of_expert[e] * P.slot_stride;
  tj.nt = local % NT;
  tj.m0 = (local / NT) * kBM;
  tj.p0 = P.offsets[e];
  tj.rows = min(kBM, c - tj.m0);
  (void)s_info;
  return tj;
}

// ---------------------------------------------------------------- the grouped GEMM

enum { kGateUp = 0, kDown = 1 };

// Weights decoded to bf16 as they are stored to LDS (bf16 activations, the
// bf16 MFMA): E2M1 times its block scale (NVFP4: E4M3, MXFP4: E8M0) or an
// E4M3 value (FP8) has at most 6 significant bits and a magnitude inside
// bf16's range, so each decoded weight is exact; NVFP4 and FP8 per-tensor
// multipliers scale the fp32 sums in the epilogue.
__device__ __forceinline__ uint32_t bf16_pair_scaled(float a, float b, float sc) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a * sc, b * sc}, bf16x2_t));
}

// 8 bf16 values (16 bytes) of E2M1 codes `d` (8 nibbles, element 2i low) times sc.
__device__ __forceinline__ uint4 e2m1x8_to_bf16(uint32_t d, float sc) {
  const f32x2_t v[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3)};
  return make_uint4(bf16_pair_scaled(v[0].x, v[0].y, sc), bf16_pair_scaled(v[1].x, v[1].y, sc),
                    bf16_pair_scaled(v[2].x, v[2].y, sc), bf16_pair_scaled(v[3].x, v[3].y, sc));
}

// 8 bf16 values of 8 E4M3 codes (two dwords), exact.
__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true)));
}

// WQ: with FP4 false, the weight format: MOE_FMT_BF16 (copied), or NVFP4,
// MXFP4 or FP8 (decoded to bf16 at the LDS store).
template <bool FP4, int MODE, int D, int WQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_mfma_ffn(FfnParams P, MfmaBufs B) {
  constexpr bool DEC = !FP4 && WQ != MOE_FMT_BF16;  // weights decoded at the LDS store
  constexpr bool Q4 = DEC && WQ != MOE_FMT_FP8;     // E2M1 weights with block scales
  const int K = MODE == kGateUp ? P.H : P.I;
  const int NT = MODE == kGateUp ? (2 * P.I) / kBN : P.H / kBN;
  const TileJob tj = find_tile(P, NT);
  if (tj.rows == 0) return;

  // One K-step = 128 bytes of every operand row (FP4: K = 256, two 128-wide
  // K-tiles; BF16: K = 64, two 32-wide K-tiles): 16 KiB per operand.
  constexpr int KSTEP = FP4 ? 256 : 64;
  constexpr int kStage = 16384;
  // A rows are kept row-major with a 16-byte pad (144-byte stride): the
  // fragment reads (16 rows at once) then hit 16 distinct bank groups.
  constexpr int kArow = 144, kAbytes = 128 * kArow;
  constexpr int kBoff = kAbytes, kSoff = kAbytes + kStage;
  constexpr int kBuf = kAbytes + kStage + (FP4 ? 2048 : 0);  // A, B (+ A and B scale bytes)
  __shared__ __align__(16) uint8_t lds[2 * kBuf];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const uint8_t* wt = tj.blob + (MODE == kGateUp ? P.L.off_w13 : P.L.off_w2);
  const uint8_t* st = tj.blob + (MODE == kGateUp ? P.L.off_s13 : P.L.off_s2);
  const int nk_w = K / (FP4 ? 128 : k_per_tile(WQ));  // weight K-tiles per row-group
  const int rg0 = tj.nt * 8;              // first 16-row group of the column tile

  // Operand A: thread t stages 16-byte segment t % 8 of rows t / 8 + 32 i
  // (i < 4), so a wave reads eight whole 128-byte row segments per load.
  // Rows past the tile are clamped for the address and zeroed after the load.
  // 32-bit byte offsets from one base pointer (the launcher bounds every
  // operand buffer below 4 GiB) keep the per-stage address state small; the
  // offsets come from mfma_addr.h.
  const uint8_t* abase = MODE == kGateUp ? (FP4 ? B.xq : reinterpret_cast<const uint8_t*>(P.x))
                                         : (FP4 ? B.hq : reinterpret_cast<const uint8_t*>(B.hb));
  const uint32_t arow_bytes = FP4 ? K / 2 : K * 2;
  uint32_t aoff[4];
  uint32_t avalid = 0;  // bit i: row (tid / 8) + 32 i is inside the tile
  const int seg = tid & 7;
  // the buffer row of tile row r: the token (gate/up) or the permutation-order row (down)
  auto src_row_of = [&](int r) -> uint32_t {
    if (MODE == kGateUp) return tj.shared ? tj.m0 + r : P.perm[tj.p0 + tj.m0 + r] / P.k;
    return tj.p0 + tj.m0 + r;
  };
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (tid >> 3) + 32 * i;
    if (row < tj.rows) avalid |= 1u << i;
    aoff[i] = mfma_a_base(src_row_of(row < tj.rows ? row : 0), arow_bytes, tid);
  }
  // FP4 A scales: 8 bytes (the step's eight 32-blocks) of row tid / 2, half tid % 2.
  const uint8_t* asbase = MODE == kGateUp ? B.xs : B.hs;
  uint32_t as_off = 0, askeep = 0;
  if (FP4) {
    const int row = tid >> 1;
    askeep = row < tj.rows ? 0xFFFFFFFFu : 0u;
    as_off = mfma_sa_base(src_row_of(row < tj.rows ? row : 0), (uint32_t)K / 32, tid);
  }
  // Operand B: chunk c = t + 256 i is lane c % 64 of weight tile (row group
  // rg0 + c / 128, K-tile (c / 64) % 2 of the step); LDS holds it at c * 16.
  // FP4 B scales: dword t of the step's 16 scale tiles (64 bytes each).
  const uint32_t bs_off = mfma_sb_base(rg0, nk_w, tid);

  struct Stage {
    uint4 a[4], b[4];
    uint32_t sa, sb;
  };
  // per-tensor multipliers of the decoded formats (gate, up, down)
  float gq = 1.f, uq = 1.f, dq = 1.f;
  if constexpr (DEC) {
    const BlobHeader* hd = reinterpret_cast<const BlobHeader*>(tj.blob);
    gq = hd->g[0];
    uq = hd->g[1];
    dq = hd->g[2];
  }
  const int nsteps = (K + KSTEP - 1) / KSTEP;
  // FP4 with K % 256 == 128: the last step holds one K-tile; its second
  // half re-reads the first half's addresses (in bounds, finite) and is
  // stored as zeros.
  const bool half_tail = FP4 && (K % KSTEP) != 0;
  auto load_stage = [&](int ks, Stage& S) {
    const bool tail = half_tail && ks == nsteps - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      S.a[i] = *reinterpret_cast<const uint4*>(abase + mfma_step_off(aoff[i], ks, 128u, mfma_a_back(tid, tail)));
      if constexpr (!DEC)
        S.b[i] = *reinterpret_cast<const uint4*>(
            wt + mfma_step_off(mfma_b_base(rg0, nk_w, tid, i), ks, 2u * kTileBytes, mfma_b_back(tid, tail)));
    }
    if constexpr (Q4) {
      S.b[0] = *reinterpret_cast<const uint4*>(wt + mfma_q4_b_off(rg0, nk_w, tid, ks));
      constexpr uint32_t lsb = WQ == MOE_FMT_NVFP4 ? 2 : 1;
      const uint8_t* sp = st + mfma_q4_s_off(rg0, nk_w, tid, ks, lsb);
      S.sb = WQ == MOE_FMT_NVFP4 ? (uint32_t)*reinterpret_cast<const uint16_t*>(sp) : (uint32_t)*sp;
    } else if constexpr (DEC) {
#pragma unroll
      for (int i = 0; i < 2; ++i) S.b[i] = *reinterpret_cast<const uint4*>(wt + mfma_f8_b_off(rg0, nk_w, tid, i, ks));
    }
    if (FP4) {
      S.sa = *reinterpret_cast<const uint32_t*>(asbase + mfma_step_off(as_off, ks, 8u, mfma_sa_back(tid, tail)));
      S.sb = *reinterpret_cast<const uint32_t*>(st + mfma_step_off(bs_off, ks, 128u, mfma_sb_back(tid, tail)));
    }
  };
  auto store_stage = [&](const Stage& S, uint8_t* buf, int ks) {
    const uint32_t lk = 0xFFFFFFFFu;
    const bool tail = half_tail && ks == nsteps - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t k = (0u - ((avalid >> i) & 1u)) & lk & ((tail && seg >= 4) ? 0u : 0xFFFFFFFFu);  // bit masks
      *reinterpret_cast<uint4*>(buf + ((tid >> 3) + 32 * i) * kArow + seg * 16) =
          make_uint4(S.a[i].x & k, S.a[i].y & k, S.a[i].z & k, S.a[i].w & k);
      if constexpr (!DEC) reinterpret_cast<uint4*>(buf + kBoff)[tid + 256 * i] = S.b[i];
    }
    // decoded weights, in the bf16 layout: chunk (row group g, K-tile kt of
    // the step, lane l) at index (2 g + kt) * 64 + l, lane l = row l % 16,
    // values 8 (l / 16) .. + 8 of the 32-value K-tile
    uint4* bl = reinterpret_cast<uint4*>(buf + kBoff);
    if constexpr (Q4) {
      // tile lane 32 (ks % 2) + tid % 32: row r, values 32 j .. 32 j + 31 of the step
      const int g = tid >> 5, r = tid & 15, j = (tid >> 4) & 1;
      float s0, s1;
      if constexpr (WQ == MOE_FMT_NVFP4) {
        s0 = __builtin_amdgcn_cvt_f32_fp8((int)S.sb, 0);  // E4M3 of values 0..15
        s1 = __builtin_amdgcn_cvt_f32_fp8((int)S.sb, 1);  // and 16..31
      } else {
        s0 = s1 = e8m0_to_f32(S.sb);
      }
      bl[(2 * g + j) * 64 + r] = e2m1x8_to_bf16(S.b[0].x, s0);
      bl[(2 * g + j) * 64 + r + 16] = e2m1x8_to_bf16(S.b[0].y, s0);
      bl[(2 * g + j) * 64 + r + 32] = e2m1x8_to_bf16(S.b[0].z, s1);
      bl[(2 * g + j) * 64 + r + 48] = e2m1x8_to_bf16(S.b[0].w, s1);
    } else if constexpr (DEC) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        // chunk tid + 256 i: row group c / 64, tile lane l = c % 64: row l % 16,
        // values 16 (l / 16) .. + 16 = K-tile l / 32, chunks 2 ((l / 16) % 2) and + 1
        const int c = tid + 256 * i, g = c >> 6, l = c & 63, r = l & 15, kt = l >> 5, q = 2 * ((l >> 4) & 1);
        bl[(2 * g + kt) * 64 + r + 16 * q] = e4m3x8_to_bf16(S.b[i].x, S.b[i].y);
        bl[(2 * g + kt) * 64 + r + 16 * (q + 1)] = e4m3x8_to_bf16(S.b[i].z, S.b[i].w);
      }
    }
    if (FP4) {
      const uint32_t k = askeep & lk & ((tail && (tid & 1)) ? 0u : 0xFFFFFFFFu);
      reinterpret_cast<uint32_t*>(buf + kSoff)[tid] = (S.sa & k) | (0x7F7F7F7Fu & ~k);
      reinterpret_cast<uint32_t*>(buf + kSoff + 1024)[tid] = S.sb;
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // A fragment of 16-row tile mt: lane l reads row mt*16 + l%16, bytes
  // [kt*64 + (l/16)*16, +16) of the step (FP4: K-tile kt, 32-block l/16;
  // BF16: 32-wide K-tile kt, 8 values l/16).
  auto a_frag = [&](const uint8_t* buf, int mt, int kt) {
    return *reinterpret_cast<const uint4*>(buf + (mt * 16 + (lane & 15)) * kArow + kt * 64 + (lane >> 4) * 16);
  };
  auto compute = [&](const uint8_t* buf) {
    const uint4* Bs = reinterpret_cast<const uint4*>(buf + kBoff);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      if (FP4) {
        i32x8_t a[4], b[4];
        int sa[4], sb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int mt = 4 * wm + i, nt = 4 * wn + i;
          const uint4 u = a_frag(buf, mt, kt);
          a[i] = i32x8_t{(int)u.x, (int)u.y, (int)u.z, (int)u.w, 0, 0, 0, 0};
          sa[i] = buf[kSoff + (mt * 16 + (lane & 15)) * 8 + kt * 4 + (lane >> 4)];
          const uint4 v = Bs[(nt * 2 + kt) * 64 + lane];
          b[i] = i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
          sb[i] = buf[kSoff + 1024 + (nt * 2 + kt) * 64 + lane];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], b[j], acc[i][j], 4, 4, 0, sa[i], 0,
                                                                          sb[j]);
      } else {
        bf16x8_t a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[i] = __builtin_bit_cast(bf16x8_t, a_frag(buf, 4 * wm + i, kt));
          b[i] = __builtin_bit_cast(bf16x8_t, Bs[((4 * wn + i) * 2 + kt) * 64 + lane]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    }
  };

  // Pipeline of D register stages: while step ks is stored to one LDS buffer
  // and computed, steps ks+1 .. ks+D-1 are loading.  The stage loop is
  // unrolled by D so every stage has fixed registers (no copies, which would
  // force the loads to land early) and its body has no branch around memory
  // operations (loads past the end re-read the last K-step).  The remaining
  // nsteps % D steps run after the loop.  The other LDS buffer still serves
  // the waves finishing step ks-1, so one barrier per step suffices, and it
  // orders LDS only: the global loads stay in flight across it.
  Stage S[D];
#pragma unroll
  for (int d = 0; d + 1 < D; ++d) {  // issued in stage order (the wait counter is in order)
    load_stage(min(d, nsteps - 1), S[d]);
    __builtin_amdgcn_sched_barrier(0);
  }
  auto step = [&](int ks, Stage& cur, Stage& next) {
    load_stage(min(ks + D - 1, nsteps - 1), next);
    __builtin_amdgcn_sched_barrier(0);
    uint8_t* buf = lds + (ks & 1) * kBuf;
    store_stage(cur, buf, ks);
    lds_barrier();
    compute(buf);
    // Pin this step's products here: otherwise the compiler may sink the
    // matrix instructions past later steps' barriers and loads.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(acc[i][j]));
    __builtin_amdgcn_sched_barrier(0);
  };
  int ks0 = 0;
#pragma unroll 1
  for (; ks0 + D <= nsteps; ks0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) step(ks0 + d, S[d], S[(d + D - 1) % D]);
  }
#pragma unroll
  for (int d = 0; d + 1 < D; ++d)
    if (ks0 + d < nsteps) step(ks0 + d, S[d], S[(d + D - 1) % D]);
  lds_barrier();  // the epilogue reuses the LDS

  // ------------------------------------------------------------ epilogues
  const int col = lane & 15, rq = (lane >> 4) * 4;
  if (MODE == kDown) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = (4 * wm + i) * 16 + rq + v;
        if (row < tj.rows) {
          const size_t o = ((size_t)tj.p0 + tj.m0 + row) * P.H + tj.nt * kBN + (4 * wn) * 16 + col;
          if (B.yb) {
#pragma unroll
            for (int j = 0; j < 4; ++j) B.yb[o + 16 * j] = f32_to_bf16_rne(acc[i][j][v] * dq);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) B.y[o + 16 * j] = acc[i][j][v] * dq;
          }
        }
      }
    return;
  }
  // gate/up: column tile holds 4 (gate, up) pairs of 16 rows: pair q = 4 nt + 2 wn + jj
  float* ht = reinterpret_cast<float*>(lds);  // [128][64] fp32 (aliases the staging buffers)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = (4 * wm + i) * 16 + rq + v;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const float g = acc[i][2 * jj][v] * gq, u = acc[i][2 * jj + 1][v] * uq;
        ht[row * 64 + (2 * wn + jj) * 16 + col] = silu_f32(g) * u;
      }
    }
  lds_barrier();
  const int row = tid >> 1, blk = tid & 1;  // 128 rows x 2 blocks of 32 columns
  if (row < tj.rows) {
    const size_t p = (size_t)tj.p0 + tj.m0 + row;
    const float* hv = ht + row * 64 + blk * 32;
    const int c0 = tj.nt * 64 + blk * 32;  // intermediate column of the block
    if (FP4) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = hv[i];
      uint4 q;
      uint32_t s;
      mxfp4_encode32(v, q, s);
      *reinterpret_cast<uint4*>(B.hq + p * (P.I / 2) + c0 / 2) = q;
      B.hs[p * (P.I / 32) + c0 / 32] = (uint8_t)s;
    } else {
      uint16_t* dst = B.hb + p * P.I + c0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w[j] = bf16x2_rne(hv[8 * q + 2 * j], hv[8 * q + 2 * j + 1]);
        reinterpret_cast<uint4*>(dst)[q] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }
}

// Upper bound on the number of work tiles of one launch.
static int max_tiles(const FfnParams& P, int NT) {
  const long long rows = (long long)P.T * P.k;
  long long mt = (rows + kBM - 1) / kBM + std::min<long long>(P.E, rows);
  if (P.shared_blob) mt += (P.T + kBM - 1) / kBM;
  long long g = mt * NT;
  g = (g + 7) / 8 * 8;
  return (int)g;
}

typedef void (*MfmaKernel)(FfnParams, MfmaBufs);

// Pipeline depth: 2 register stages for FP4 (its operands and scales leave
// no room for a third) and the decoded formats, 3 for BF16 when the K-steps
// divide by 3.
template <bool FP4, int MODE, int WQ = MOE_FMT_BF16>
static MfmaKernel mfma_kernel(int nsteps) {
  if constexpr (!FP4 && WQ == MOE_FMT_BF16)
    if (nsteps % 3 == 0) return k_mfma_ffn<FP4, MODE, 3, WQ>;
  return k_mfma_ffn<FP4, MODE, 2, WQ>;
}

bool fp4_gemm_fits(const FfnParams& P, int N, int K, bool gateup);
hipError_t launch_fp4_gemm(const FfnParams& P, const MfmaBufs& B, bool down, hipStream_t s);
bool bf16_gemm_fits(const FfnParams& P, int N, int K);
hipError_t launch_bf16_gemm(const FfnParams& P, const MfmaBufs& B, bool down, hipStream_t s);

// Both projections run on the persistent 128 x 512 kernel where the shapes
// allow (column counts multiples of 512; FP4: K a multiple of 256), else both
// on the 128 x 128 one (on the FP4 path the two store x and the SwiGLU output
// in different layouts).  FP4: x MXFP4-encoded first (per token, into its
// destination rows for the persistent kernel).
bool fp4_persistent(const FfnParams& P) {
  return fp4_gemm_fits(P, 2 * P.I, P.H, true) && fp4_gemm_fits(P, P.H, P.I, false);
}

// Copies the MXFP4 encoding of x (which = 0) or of the SwiGLU output (1) left
// in the workspace by an FP4 call into canonical layout: q [R][K/2], s [R][K/32]
// with row p = permutation-order row p (token perm[p] / k), rows T*k.. the
// shared expert's tokens.  One thread per 16 code bytes (and 4 scale bytes)
// of a row.  persistent: the workspace holds [K/128][R][64 B] and
// [K/128][R][4 B]; else x is token-ordered [T][K/2], [T][K/32] and h is
// already canonical.
__global__ __launch_bounds__(256) void k_fp4_codes_canon(const uint8_t* __restrict__ wq,
                                                         const uint8_t* __restrict__ ws, int persistent, int is_x,
                                                         const int32_t* __restrict__ perm, int T, int k, int R,
                                                         int K, uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const int chunks = K / 32;  // 16 code bytes and 1 scale byte per 32 values
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  if (g >= (long long)R * chunks) return;
  const int r = (int)(g / chunks), c = (int)(g % chunks);
  long long src_q, src_s;
  if (persistent) {
    const int kt = c >> 2, j = c & 3;
    src_q = ((long long)kt * R + r) * 64 + j * 16;
    src_s = ((long long)kt * R + r) * 4 + j;
  } else {
    const int row = (is_x && r < T * k) ? perm[r] / k : (is_x ? r - T * k : r);
    src_q = (long long)row * (K / 2) + c * 16;
    src_s = (long long)row * (K / 32) + c;
  }
  *reinterpret_cast<uint4*>(q + (size_t)r * (K / 2) + c * 16) = *reinterpret_cast<const uint4*>(wq + src_q);
  s[(size_t)r * (K / 32) + c] = ws[src_s];
}

hipError_t launch_fp4_codes_canon(const FfnParams& P, const MfmaBufs& B, int which, uint8_t* q, uint8_t* s,
                                  hipStream_t st) {
  const int R = P.T * P.k + (P.shared_blob ? P.T : 0), K = which == 0 ? P.H : P.I;
  const long long n = (long long)R * (K / 32);
  if (n == 0) return hipSuccess;
  launch(k_fp4_codes_canon, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, which == 0 ? B.xq : B.hq,
         which == 0 ? B.xs : B.hs, fp4_persistent(P) ? 1 : 0, which == 0 ? 1 : 0, P.perm, P.T, P.k, R, K, q, s);
  return hipGetLastError();
}

hipError_t launch_mfma(const FfnParams& P, bool fp4, const MfmaBufs& B, hipStream_t s) {
  hipError_t e;
  if (fp4) {
    if (fp4_persistent(P)) {
      const int n = P.T * P.k;
      const uint32_t rtot = (uint32_t)n + (P.shared_blob ? P.T : 0);
      const int32_t* inv = P.inv;
      if (!inv) {
        launch(k_invert, dim3((n + 255) / 256), dim3(256), 0, s, P.perm, n, P.inv_ws);
        inv = P.inv_ws;
      }
      launch(k_quant_rows, dim3(8 * ((P.T + 31) / 32)), dim3(256), 0, s, P.x, P.T, P.H, P.k, inv, P.shared_blob ? 1 : 0, rtot,
             const_cast<uint8_t*>(B.xq), const_cast<uint8_t*>(B.xs));
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      e = launch_fp4_gemm(P, B, false, s);
      if (e != hipSuccess) return e;
      return launch_fp4_gemm(P, B, true, s);
    }
    e = launch_quant_mxfp4(P.x, P.T, P.H, const_cast<uint8_t*>(B.xq), const_cast<uint8_t*>(B.xs), s);
    if (e != hipSuccess) return e;
    launch(mfma_kernel<true, kGateUp>((P.H + 255) / 256), dim3(max_tiles(P, (2 * P.I) / kBN)), dim3(256), 0, s, P, B);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch(mfma_kernel<true, kDown>((P.I + 255) / 256), dim3(max_tiles(P, P.H / kBN)), dim3(256), 0, s, P, B);
    return hipGetLastError();
  }
  if (P.fmt != MOE_FMT_BF16) {
    // NVFP4, MXFP4 or FP8 weights with bf16 activations: decoded at the LDS store
    const int nt_gu = (2 * P.I) / kBN, nt_dn = P.H / kBN;
    MfmaKernel gu, dn;
    if (P.fmt == MOE_FMT_NVFP4) {
      gu = mfma_kernel<false, kGateUp, MOE_FMT_NVFP4>(P.H / 64);
      dn = mfma_kernel<false, kDown, MOE_FMT_NVFP4>(P.I / 64);
    } else if (P.fmt == MOE_FMT_MXFP4) {
      gu = mfma_kernel<false, kGateUp, MOE_FMT_MXFP4>(P.H / 64);
      dn = mfma_kernel<false, kDown, MOE_FMT_MXFP4>(P.I / 64);
    } else {
      gu = mfma_kernel<false, kGateUp, MOE_FMT_FP8>(P.H / 64);
      dn = mfma_kernel<false, kDown, MOE_FMT_FP8>(P.I / 64);
    }
    launch(gu, dim3(max_tiles(P, nt_gu)), dim3(256), 0, s, P, B);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch(dn, dim3(max_tiles(P, nt_dn)), dim3(256), 0, s, P, B);
    return hipGetLastError();
  }
  if (bf16_gemm_fits(P, 2 * P.I, P.H) && bf16_gemm_fits(P, P.H, P.I)) {
    e = launch_bf16_gemm(P, B, false, s);
    if (e != hipSuccess) return e;
    return launch_bf16_gemm(P, B, true, s);
  }
  const int nt_gu = (2 * P.I) / kBN, nt_dn = P.H / kBN;
  launch(mfma_kernel<false, kGateUp>(P.H / 64), dim3(max_tiles(P, nt_gu)), dim3(256), 0, s, P, B);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch(mfma_kernel<false, kDown>(P.I / 64), dim3(max_tiles(P, nt_dn)), dim3(256), 0, s, P, B);
  return hipGetLastError();
}

}  // namespace moe
