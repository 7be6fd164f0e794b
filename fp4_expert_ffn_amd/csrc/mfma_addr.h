// Byte offsets of the stage loads of the 128 x 128 grouped GEMM (k_mfma_ffn).
// Host and device code: the kernel forms its addresses with these functions,
// and a CPU test enumerates every offset they give for the layer shapes the
// kernel accepts and checks it against the size of the buffer it indexes.
//
// A K-step covers 128 bytes of every operand row: FP4 K = 256 (two 128-value
// K-tiles), BF16 K = 64 (two 32-value K-tiles).  When an FP4 projection has
// K % 256 == 128 its last step holds one K-tile; the loads of its second
// half re-read the first half's bytes (in bounds, finite) and are stored to
// LDS as zeros.  Every offset is formed in 32-bit unsigned arithmetic and
// only then added to its base pointer: a step offset is never negative, so
// it never wraps (the buffers indexed are far below 4 GiB).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Offset of step ks from a thread's step-0 offset `base`: `per_step` bytes a
// step, less `back` bytes when the load re-reads the previous half K-step.
__host__ __device__ inline uint32_t mfma_step_off(uint32_t base, int ks, uint32_t per_step, uint32_t back) {
  return base + (uint32_t)ks * per_step - back;
}

// ---- operand A (x or the SwiGLU output, row-major rows of arow_bytes)
// Thread tid loads 16-byte segment tid % 8 of the step's 128 bytes of tile
// rows tid / 8 + 32 i; `src_row` is the buffer row that tile row maps to.
__host__ __device__ inline uint32_t mfma_a_base(uint32_t src_row, uint32_t arow_bytes, int tid) {
  return src_row * arow_bytes + (uint32_t)(tid & 7) * 16u;
}
// The half-K tail re-reads the first 64 bytes for segments 4..7.
__host__ __device__ inline uint32_t mfma_a_back(int tid, bool tail) { return (tail && (tid & 7) >= 4) ? 64u : 0u; }

// ---- operand B (weights: 1 KiB tiles ordered (row group, K-tile), nk_w
// K-tiles per row group).  Chunk c = tid + 256 i of a step is lane c % 64 of
// the tile of row group rg0 + c / 128 and step-local K-tile (c / 64) % 2.
__host__ __device__ inline uint32_t mfma_b_base(int rg0, int nk_w, int tid, int i) {
  const uint32_t rg = (uint32_t)(rg0 + (tid >> 7) + 2 * i);
  return (rg * (uint32_t)nk_w + (uint32_t)((tid >> 6) & 1)) * 1024u + (uint32_t)(tid & 63) * 16u;
}
// The half-K tail re-reads the step's first K-tile for chunks of the second.
__host__ __device__ inline uint32_t mfma_b_back(int tid, bool tail) {
  return (tail && ((tid >> 6) & 1)) ? 1024u : 0u;
}

// ---- FP4 scales.  A: the step's 8 E8M0 bytes of tile row tid / 2, half
// tid % 2, from a row of srow_bytes scale bytes (one per 32 values).
__host__ __device__ inline uint32_t mfma_sa_base(uint32_t src_row, uint32_t srow_bytes, int tid) {
  return src_row * srow_bytes + (uint32_t)(tid & 1) * 4u;
}
__host__ __device__ inline uint32_t mfma_sa_back(int tid, bool tail) { return (tail && (tid & 1)) ? 4u : 0u; }
// B: dword tid % 16 of the 64-byte scale tile of row group rg0 + tid / 32 and
// step-local K-tile (tid / 16) % 2.
__host__ __device__ inline uint32_t mfma_sb_base(int rg0, int nk_w, int tid) {
  const uint32_t rg = (uint32_t)(rg0 + (tid >> 5));
  return (rg * (uint32_t)nk_w + (uint32_t)((tid >> 4) & 1)) * 64u + (uint32_t)(tid & 15) * 4u;
}
__host__ __device__ inline uint32_t mfma_sb_back(int tid, bool tail) {
  return (tail && ((tid >> 4) & 1)) ? 64u : 0u;
}

// ---- weights decoded to bf16 as they are stored to LDS (bf16 activations).
// A K-step covers 64 values.  E2M1 tiles (NVFP4, MXFP4) hold 128 values, so
// a step reads half of a tile of each of the column tile's 8 row groups:
// thread tid takes lane 32 (ks % 2) + tid % 32 of the tile of row group
// rg0 + tid / 32, 16 bytes (32 values), and its scale bytes (lane_sb each:
// 2 for NVFP4, 1 for MXFP4).
__host__ __device__ inline uint32_t mfma_q4_tile(int rg0, int nk_w, int tid, int ks) {
  return (uint32_t)(rg0 + (tid >> 5)) * (uint32_t)nk_w + (uint32_t)(ks >> 1);
}
__host__ __device__ inline uint32_t mfma_q4_lane(int tid, int ks) { return 32u * (uint32_t)(ks & 1) + (uint32_t)(tid & 31); }
__host__ __device__ inline uint32_t mfma_q4_b_off(int rg0, int nk_w, int tid, int ks) {
  return mfma_q4_tile(rg0, nk_w, tid, ks) * 1024u + mfma_q4_lane(tid, ks) * 16u;
}
__host__ __device__ inline uint32_t mfma_q4_s_off(int rg0, int nk_w, int tid, int ks, uint32_t lane_sb) {
  return mfma_q4_tile(rg0, nk_w, tid, ks) * 64u * lane_sb + mfma_q4_lane(tid, ks) * lane_sb;
}
// FP8 tiles hold 64 values: a step reads the whole tile of each row group,
// chunk c = tid + 256 i (i < 2) being lane c % 64 of row group rg0 + c / 64.
__host__ __device__ inline uint32_t mfma_f8_b_off(int rg0, int nk_w, int tid, int i, int ks) {
  const uint32_t c = (uint32_t)tid + 256u * (uint32_t)i;
  return ((uint32_t)(rg0 + (int)(c >> 6)) * (uint32_t)nk_w + (uint32_t)ks) * 1024u + (c & 63u) * 16u;
}

}  // namespace moe
