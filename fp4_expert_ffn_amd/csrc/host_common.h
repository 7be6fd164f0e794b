// Internal header of libmoe (not installed): the host-only part (errors,
// blob layout), usable from plain C++ against the HIP runtime API.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

// ---------------------------------------------------------------- errors
namespace moe {
moe_status set_error(moe_status st, const char* fmt, ...);
inline moe_status ok() { return MOE_OK; }
}  // namespace moe

#define MOE_CHECK_ARG(cond, ...)                                  \
  do {                                                            \
    if (!(cond)) return moe::set_error(MOE_EINVAL, __VA_ARGS__);  \
  } while (0)

#define MOE_HIP(call)                                                                          \
  do {                                                                                         \
    hipError_t e_ = (call);                                                                    \
    if (e_ != hipSuccess)                                                                      \
      return moe::set_error(MOE_EHIP, "%s failed: %s", #call, hipGetErrorString(e_));          \
  } while (0)

// Launch check: picks up launch-configuration errors and earlier asynchronous faults.
#define MOE_LAUNCHED()                                                                         \
  do {                                                                                         \
    hipError_t e_ = hipGetLastError();                                                         \
    if (e_ != hipSuccess)                                                                      \
      return moe::set_error(MOE_EHIP, "kernel launch failed: %s", hipGetErrorString(e_));      \
  } while (0)

// ---------------------------------------------------------------- blob layout
//
// Blob = 256-byte header, then four sections, each 256-byte aligned:
//   W13 codes, W13 scales, W2 codes, W2 scales.
// W13 holds gate and up interleaved by 16-row groups: row-group rg = 2p is
// gate rows [16p, 16p+16), rg = 2p+1 is up rows [16p, 16p+16).  W2 is down.
//
// Every section is a sequence of 1 KiB tiles, ordered (row-group, K-tile)
// with K fastest.  A tile covers 16 rows x KT columns, KT = 128 for the 4-bit
// formats, 64 for FP8 and 32 for BF16, and lists 64 lanes' 16-byte fragments in lane
// order: lane l holds row (l % 16) and the K-chunk (l / 16) of the tile
// (32 E2M1 codes, 16 E4M3 codes, or 8 bf16 values).  This is the operand layout of the
// gfx950 16x16x128 (FP4) and 16x16x32 (BF16) MFMA B-fragments, and it makes
// every wave-wide 16-byte load one contiguous 1 KiB transaction.
//
// Scale tiles follow the same order: MXFP4 64 B per tile (lane l: the E8M0
// of its 32 values), NVFP4 128 B per tile (lane l: bytes 2l, 2l+1 = the two
// E4M3 scales of its 32 values).
namespace moe {

constexpr uint32_t kBlobMagic = 0x42454F4Du;  // "MOEB"
constexpr int kHeaderBytes = 256;
constexpr int kTileBytes = 1024;

struct BlobHeader {
  uint32_t magic;
  uint32_t version;
  int32_t fmt, H, I;
  float g[3];  // NVFP4 per-tensor multipliers (gate, up, down); 1 otherwise
  uint64_t off_w13, off_s13, off_w2, off_s2, total;
  uint8_t pad[kHeaderBytes - 4 * 2 - 4 * 3 - 4 * 3 - 8 * 5];
};
static_assert(sizeof(BlobHeader) == kHeaderBytes, "header size");

__host__ __device__ inline int k_per_tile(int fmt) {
  return fmt == MOE_FMT_BF16 ? 32 : (fmt == MOE_FMT_FP8 ? 64 : 128);
}
__host__ __device__ inline int scale_bytes_per_tile(int fmt) {
  return fmt == MOE_FMT_MXFP4 ? 64 : (fmt == MOE_FMT_NVFP4 ? 128 : 0);
}
inline uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

struct BlobLayout {
  uint64_t off_w13, off_s13, off_w2, off_s2, total;
  int tiles13, tiles2;  // tile counts
};

inline bool layout_of(int fmt, int H, int I, BlobLayout* L) {
  if (fmt != MOE_FMT_BF16 && fmt != MOE_FMT_MXFP4 && fmt != MOE_FMT_NVFP4 && fmt != MOE_FMT_FP8) return false;
  if (H <= 0 || I <= 0 || H % 128 || I % 128) return false;
  const int kt = k_per_tile(fmt), sb = scale_bytes_per_tile(fmt);
  L->tiles13 = (2 * I / 16) * (H / kt);
  L->tiles2 = (H / 16) * (I / kt);
  uint64_t o = kHeaderBytes;
  L->off_w13 = o; o = align256(o + (uint64_t)L->tiles13 * kTileBytes);
  L->off_s13 = o; o = align256(o + (uint64_t)L->tiles13 * sb);
  L->off_w2 = o;  o = align256(o + (uint64_t)L->tiles2 * kTileBytes);
  L->off_s2 = o;  o = align256(o + (uint64_t)L->tiles2 * sb);
  L->total = o;
  return true;
}

// The slot map of one decode step, passed to a kernel by value (the kernel
// argument segment holds it; no host buffer).
constexpr int kStepMapMax = 256;
struct StepMap {
  int32_t n;
  int32_t expert[kStepMapMax];
  int32_t slot[kStepMapMax];
  uint8_t hit[kStepMapMax];
};

// The blobs a decode step copies from pinned host memory into its miss
// slots, passed by value: src[i] is the device address of the host blob
// (16-byte aligned, slot_bytes long), slot[i] its slot; the 16-byte vectors
// [off16, off16 + len16) of each blob are copied.
constexpr int kFillMax = 64;
struct FillList {
  int32_t n;
  uint32_t off16, len16;
  int32_t slot[kFillMax];
  const uint8_t* src[kFillMax];
};

// The count handoff of a cache decode step: counts[0..E) copied into the
// host-mapped host_counts, then `seq` stored in the host-mapped *flag with a
// release at system scope (cache_kernels.hip).
hipError_t launch_publish_counts(const int32_t* counts, int E, int32_t* host_counts, uint32_t* flag, uint32_t seq,
                                 hipStream_t s);
// moe_route_permute followed by that handoff, issued once every routing
// output is written (route.hip).
moe_status route_permute_publish(const float* logits, int T, int E, int k, int renormalize, int32_t* topk_ids,
                                 float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                 int32_t* host_counts, uint32_t* flag, uint32_t seq, hipStream_t s);

}  // namespace moe
