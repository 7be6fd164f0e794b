// Device side of the expert-slot cache: the blob moves of a resize.
//
// Method: resizing the expert cache at runtime at scheduler safe points
// (page "FreeToken量子化：MoE推論のセットアップガイド", paragraph on the
// cache resize); the kept blobs move device to device, so a resize costs no
// PCIe traffic (this library's reading).
#include <algorithm>

#include "common.h"

namespace moe {

// Blob moves of one launch: source slot of destination slot dst0 + b, passed
// by value (the kernel argument segment holds them; no device buffer).
constexpr int kMoveBatch = 256;
struct SlotMoves {
  int32_t src[kMoveBatch];
};

// Copy blob blockIdx.y of the batch (slot_vecs 16-byte vectors) from its old
// slot to slot dst0 + blockIdx.y; the x blocks stride over the vectors, four
// loads in flight per thread.  HBM-bound: one read and one write per byte.
__global__ __launch_bounds__(256) void k_move_slots(SlotMoves m, int dst0, const uint4* __restrict__ src_pool,
                                                    uint4* __restrict__ dst_pool, uint32_t slot_vecs) {
  const uint4* src = src_pool + (size_t)m.src[blockIdx.y] * slot_vecs;
  uint4* dst = dst_pool + (size_t)(dst0 + blockIdx.y) * slot_vecs;
  const uint32_t step = gridDim.x * 256u;
  for (uint32_t v = blockIdx.x * 256u + threadIdx.x; v < slot_vecs; v += 4 * step) {
    uint4 r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (v + j * step < slot_vecs) r[j] = src[v + j * step];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (v + j * step < slot_vecs) dst[v + j * step] = r[j];
  }
}

// Moves blobs src_slots[0..n) of src_pool to slots dst0, dst0 + 1, ... of
// dst_pool (slot_bytes a multiple of 16, below 2^35), one launch per 256.
hipError_t launch_move_slots(const int32_t* src_slots, int n, int dst0, const void* src_pool, void* dst_pool,
                             size_t slot_bytes, hipStream_t s) {
  const uint32_t vecs = (uint32_t)(slot_bytes / 16);
  const int gx = (int)std::min<uint32_t>(64, (vecs + 1023) / 1024);
  for (int b0 = 0; b0 < n; b0 += kMoveBatch) {
    const int nb = std::min(kMoveBatch, n - b0);
    SlotMoves m{};
    for (int b = 0; b < nb; ++b) m.src[b] = src_slots[b0 + b];
    launch(k_move_slots, dim3(gx, nb), dim3(256), 0, s, m, dst0 + b0, reinterpret_cast<const uint4*>(src_pool),
           reinterpret_cast<uint4*>(dst_pool), vecs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
