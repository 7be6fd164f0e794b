// Host-side pieces of libmoe: error strings, blob sizes and prepacking.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "host_common.h"

namespace moe {
static thread_local char g_err[512] = "";

moe_status set_error(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}
}  // namespace moe

extern "C" const char* moe_last_error(void) { return moe::g_err; }
extern "C" const char* moe_version(void) { return "libmoe 0.1 gfx950"; }

extern "C" size_t moe_blob_bytes(int fmt, int H, int I) {
  moe::BlobLayout L;
  return moe::layout_of(fmt, H, I, &L) ? (size_t)L.total : 0;
}

namespace {

// Copy one projection [rows, cols] into tiles of 16 rows x kt columns.
// rg_map(rg) gives (source row-group index within `src`) for destination
// row-group rg; for W13 the caller interleaves gate and up.
void pack_codes_tile(const uint8_t* src_row0, size_t src_row_bytes, int kt_idx, int fmt, uint8_t* tile) {
  const int kt = moe::k_per_tile(fmt);
  for (int l = 0; l < 64; ++l) {
    const int r = l % 16, kb = l / 16;
    const uint8_t* s;
    if (fmt == MOE_FMT_BF16)
      s = src_row0 + (size_t)r * src_row_bytes + ((size_t)kt_idx * kt + kb * 8) * 2;
    else if (fmt == MOE_FMT_FP8)
      s = src_row0 + (size_t)r * src_row_bytes + (size_t)kt_idx * kt + kb * 16;
    else
      s = src_row0 + (size_t)r * src_row_bytes + ((size_t)kt_idx * kt + kb * 32) / 2;
    memcpy(tile + l * 16, s, 16);
  }
}

void pack_scale_tile(const uint8_t* s_row0, size_t s_row_bytes, int kt_idx, int fmt, uint8_t* tile) {
  for (int l = 0; l < 64; ++l) {
    const int r = l % 16, kb = l / 16;
    const uint8_t* s = s_row0 + (size_t)r * s_row_bytes;
    if (fmt == MOE_FMT_MXFP4) {
      tile[l] = s[kt_idx * 4 + kb];
    } else {
      tile[2 * l] = s[kt_idx * 8 + kb * 2];
      tile[2 * l + 1] = s[kt_idx * 8 + kb * 2 + 1];
    }
  }
}

}  // namespace

extern "C" moe_status moe_prepack_expert(const moe_expert_canonical* src, void* blob_out, size_t blob_bytes) {
  MOE_CHECK_ARG(src && blob_out, "moe_prepack_expert: null pointer");
  moe::BlobLayout L;
  MOE_CHECK_ARG(moe::layout_of(src->fmt, src->H, src->I, &L),
                "moe_prepack_expert: unsupported fmt %d / H %d / I %d (H, I must be multiples of 128)",
                src->fmt, src->H, src->I);
  MOE_CHECK_ARG(blob_bytes >= L.total, "moe_prepack_expert: blob_bytes %zu < %llu", blob_bytes,
                (unsigned long long)L.total);
  const int fmt = src->fmt, H = src->H, I = src->I, kt = moe::k_per_tile(fmt);
  const bool fp4 = fmt == MOE_FMT_MXFP4 || fmt == MOE_FMT_NVFP4;  // block scales present
  MOE_CHECK_ARG(src->gate_q && src->up_q && src->down_q, "moe_prepack_expert: null weight tensor");
  MOE_CHECK_ARG(!fp4 || (src->gate_s && src->up_s && src->down_s), "moe_prepack_expert: null scale tensor");

  uint8_t* b = static_cast<uint8_t*>(blob_out);
  memset(b, 0, L.total);
  moe::BlobHeader* h = reinterpret_cast<moe::BlobHeader*>(b);
  h->magic = moe::kBlobMagic;
  h->version = 1;
  h->fmt = fmt;
  h->H = H;
  h->I = I;
  const bool nv = fmt == MOE_FMT_NVFP4 || fmt == MOE_FMT_FP8;  // per-tensor multipliers
  h->g[0] = nv ? src->gate_g : 1.0f;
  h->g[1] = nv ? src->up_g : 1.0f;
  h->g[2] = nv ? src->down_g : 1.0f;
  h->off_w13 = L.off_w13;
  h->off_s13 = L.off_s13;
  h->off_w2 = L.off_w2;
  h->off_s2 = L.off_s2;
  h->total = L.total;

  // bytes per row of the canonical code / scale tensors
  auto row_bytes = [&](int cols) -> size_t {
    return fp4 ? (size_t)cols / 2 : (fmt == MOE_FMT_FP8 ? (size_t)cols : (size_t)cols * 2);
  };
  auto srow_bytes = [&](int cols) -> size_t { return fmt == MOE_FMT_MXFP4 ? (size_t)cols / 32 : (size_t)cols / 16; };
  const int sb = moe::scale_bytes_per_tile(fmt);

  // W13: interleaved 16-row groups of gate and up, K = H
  const int nk13 = H / kt;
  for (int rg = 0; rg < 2 * I / 16; ++rg) {
    const int p = rg / 2;
    const uint8_t* q = static_cast<const uint8_t*>((rg & 1) ? src->up_q : src->gate_q);
    const uint8_t* s = (rg & 1) ? src->up_s : src->gate_s;
    for (int k = 0; k < nk13; ++k) {
      const size_t t = (size_t)rg * nk13 + k;
      pack_codes_tile(q + (size_t)16 * p * row_bytes(H), row_bytes(H), k, fmt, b + L.off_w13 + t * moe::kTileBytes);
      if (fp4) pack_scale_tile(s + (size_t)16 * p * srow_bytes(H), srow_bytes(H), k, fmt, b + L.off_s13 + t * sb);
    }
  }
  // W2: down [H, I], K = I
  const int nk2 = I / kt;
  const uint8_t* q2 = static_cast<const uint8_t*>(src->down_q);
  for (int rg = 0; rg < H / 16; ++rg) {
    for (int k = 0; k < nk2; ++k) {
      const size_t t = (size_t)rg * nk2 + k;
      pack_codes_tile(q2 + (size_t)16 * rg * row_bytes(I), row_bytes(I), k, fmt, b + L.off_w2 + t * moe::kTileBytes);
      if (fp4) pack_scale_tile(src->down_s + (size_t)16 * rg * srow_bytes(I), srow_bytes(I), k, fmt, b + L.off_s2 + t * sb);
    }
  }
  return MOE_OK;
}
