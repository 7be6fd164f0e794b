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

// ---------------------------------------------------------------- decode-step handoffs

// Copies the step's per-expert row counts into a host-mapped buffer, then
// publishes `seq` in the host-mapped flag (release at system scope): the host
// waits for the flag by polling instead of a copy and a stream
// synchronisation.
__global__ __launch_bounds__(256) void k_publish_counts(const int32_t* __restrict__ counts, int E,
                                                        int32_t* __restrict__ host_counts, uint32_t* flag,
                                                        uint32_t seq) {
  for (int e = threadIdx.x; e < E; e += 256) host_counts[e] = counts[e];
  __threadfence_system();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(flag, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

hipError_t launch_publish_counts(const int32_t* counts, int E, int32_t* host_counts_dev, uint32_t* flag_dev,
                                 uint32_t seq, hipStream_t s) {
  launch(k_publish_counts, dim3(1), dim3(256), 0, s, counts, E, host_counts_dev, flag_dev, seq);
  return hipGetLastError();
}

// The step's slot map, passed by value: map layout int32 slot[E], uint8
// hit[E], uint8 miss[E]; experts outside the step get slot 0 and no mask.
// One workgroup of 256 threads.
__device__ __forceinline__ void write_step_map(const StepMap& m, int E, uint8_t* __restrict__ map) {
  int32_t* slot = reinterpret_cast<int32_t*>(map);
  uint8_t* hit = map + 4 * E;
  uint8_t* miss = hit + E;
  for (int e = threadIdx.x; e < E; e += 256) {
    slot[e] = 0;
    hit[e] = 0;
    miss[e] = 0;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < m.n; i += 256) {
    const int e = m.expert[i];
    slot[e] = m.slot[i];
    (m.hit[i] ? hit : miss)[e] = 1;
  }
}

__global__ __launch_bounds__(256) void k_write_map(StepMap m, int E, uint8_t* __restrict__ map) {
  write_step_map(m, E, map);
}

hipError_t launch_write_map(const StepMap& m, int E, void* dev_map, hipStream_t s) {
  launch(k_write_map, dim3(1), dim3(256), 0, s, m, E, static_cast<uint8_t*>(dev_map));
  return hipGetLastError();
}

// Miss fills of a decode step read straight from pinned host memory (PCIe
// reads issued by the shader, no copy engine), so the step's miss FFN follows
// them on the same stream with no cross-queue handoff.  Workgroups below
// kCopyWgs copy vectors [f.off16, f.off16 + f.len16) of every blob of the
// list into its slot (of slot_vecs 16-byte vectors; copy_blob_list), and
// workgroup kCopyWgs writes the step's map.  PCIe-bound.
__global__ __launch_bounds__(256) void k_fill_slots(FillList f, StepMap m, int E, uint8_t* __restrict__ map,
                                                    uint4* __restrict__ pool, uint32_t slot_vecs) {
  if (blockIdx.x == kCopyWgs) {
    write_step_map(m, E, map);
    return;
  }
  copy_blob_list(f, pool, slot_vecs, blockIdx.x, kCopyWgs);
}

// f.n in [1, kFillMax]; slot_bytes a multiple of 16, below 2^35; the range
// inside the slot (f.off16 + f.len16 <= slot_bytes / 16, checked by the caller).
hipError_t launch_fill_slots(const FillList& f, const StepMap& m, int E, void* dev_map, void* pool, size_t slot_bytes,
                             hipStream_t s) {
  launch(k_fill_slots, dim3(kCopyWgs + 1), dim3(256), 0, s, f, m, E, static_cast<uint8_t*>(dev_map),
         static_cast<uint4*>(pool), (uint32_t)(slot_bytes / 16));
  return hipGetLastError();
}

}  // namespace moe
