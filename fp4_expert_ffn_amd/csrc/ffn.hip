// moe_expert_ffn dispatcher, the weighted combine, and the debug dequantiser.
//
// Method: the combine weights each routed expert's output by its routing
// weight and sums them back in token order (the sparse activation of page
// "FreeToken量子化：MoE推論のセットアップガイド", second paragraph: every token
// passes through a few experts); the shared expert, when present, is added
// with weight 1 (this library's reading).
#include <algorithm>
#include <mutex>

#include "ffn_common.h"

namespace moe {
hipError_t launch_gemv(const FfnParams& P, const GemvArgs& G, hipStream_t s);
bool gemv_route_fits(const FfnParams& P);
bool ffn_takes_gemv(const moe_ffn_args* a);
moe_status expert_ffn_fill(const moe_ffn_args* a, const FillList& f, void* pool, size_t slot_bytes, hipStream_t s);
hipError_t launch_mfma(const FfnParams& P, bool fp4, const MfmaBufs& B, hipStream_t s);
hipError_t launch_quant_mxfp4(const uint16_t* x, int rows, int cols, uint8_t* q, uint8_t* s, hipStream_t st);
hipError_t launch_fp4_codes_canon(const FfnParams& P, const MfmaBufs& B, int which, uint8_t* q, uint8_t* s,
                                  hipStream_t st);
}  // namespace moe

namespace {
using namespace moe;

// Row count at or above which bf16-activation calls take the bf16 MFMA
// grouped GEMM (BF16 weights as they are; NVFP4, MXFP4 and FP8 weights
// decoded to bf16 on the way into LDS).
constexpr long long kMfmaMinRows = 512;
// Largest H and I of the GEMV path (one bf16 row of x or h per LDS stage).
constexpr int kGemvMaxK = 28672;

enum Path { kPathGemv, kPathMfmaFp4, kPathMfmaBf16 };

Path choose_path(const moe_ffn_args* a) {
  if (a->amode == MOE_ACT_MXFP4) return kPathMfmaFp4;
  if ((long long)a->T * a->k >= kMfmaMinRows) return kPathMfmaBf16;
  return kPathGemv;
}

struct WsLayout {
  size_t trash, h, y, xq, xs, hq, hs, hb, inv, total;
};

size_t al(size_t v) { return (v + 255) & ~size_t(255); }

bool internal_bf16_y(const moe_ffn_args* a) { return !a->y && a->out && choose_path(a) != kPathGemv; }

WsLayout ws_layout(const moe_ffn_args* a) {
  const size_t R = (size_t)a->T * a->k + (a->shared_blob ? a->T : 0);
  WsLayout w{};
  size_t o = 0;
  w.trash = o; o = al(o + (1 << 20));  // 256 slots of 4 KiB
  const Path p = choose_path(a);
  if (p == kPathGemv) {
    w.h = o; o = al(o + R * a->I * 2);
  } else if (p == kPathMfmaFp4) {
    // x encoded per token row (128 x 128 kernel) or per routed + shared row
    // (persistent kernel): room for the larger
    w.xq = o; o = al(o + R * a->H / 2);
    w.xs = o; o = al(o + R * a->H / 32);
    w.inv = o; o = al(o + (size_t)a->T * a->k * 4);
    w.hq = o; o = al(o + R * a->I / 2);
    w.hs = o; o = al(o + R * a->I / 32);
  } else {
    w.hb = o; o = al(o + R * a->I * 2);
  }
  // Internal expert outputs: bf16 on the matrix-core paths when only the
  // combined output is wanted (halves the y round trip), else fp32.
  w.y = o;
  if (!a->y) o = al(o + R * a->H * (internal_bf16_y(a) ? 2 : sizeof(float)));
  w.total = o;
  return w;
}

moe_status check_args(const moe_ffn_args* a) {
  MOE_CHECK_ARG(a, "moe_expert_ffn: null args");
  MOE_CHECK_ARG(a->T >= 0 && a->k >= 1 && a->k <= 16 && a->E >= 1 && a->E <= 1024,
                "moe_expert_ffn: bad sizes T=%d k=%d E=%d", a->T, a->k, a->E);
  MOE_CHECK_ARG(a->H > 0 && a->I > 0 && a->H % 128 == 0 && a->I % 128 == 0,
                "moe_expert_ffn: H=%d and I=%d must be positive multiples of 128", a->H, a->I);
  MOE_CHECK_ARG(a->wfmt == MOE_FMT_BF16 || a->wfmt == MOE_FMT_MXFP4 || a->wfmt == MOE_FMT_NVFP4 ||
                    a->wfmt == MOE_FMT_FP8,
                "moe_expert_ffn: bad weight format %d", a->wfmt);
  MOE_CHECK_ARG(a->amode == MOE_ACT_BF16 || a->amode == MOE_ACT_MXFP4, "moe_expert_ffn: bad amode %d", a->amode);
  if (a->amode == MOE_ACT_MXFP4 && a->wfmt != MOE_FMT_MXFP4)
    return set_error(MOE_EUNSUPPORTED, "moe_expert_ffn: MXFP4 activations need MXFP4 weights (got format %d)",
                     a->wfmt);
  MOE_CHECK_ARG((long long)a->T * a->k <= (1 << 17), "moe_expert_ffn: T*k exceeds 131072");
  MOE_CHECK_ARG(choose_path(a) != kPathGemv || (a->H <= kGemvMaxK && a->I <= kGemvMaxK),
                "moe_expert_ffn: H=%d, I=%d: the bf16-activation path stages one row of up to %d values in LDS",
                a->H, a->I, kGemvMaxK);
  MOE_CHECK_ARG(a->slot_stride % 256 == 0 && a->slot_stride >= moe_blob_bytes(a->wfmt, a->H, a->I),
                "moe_expert_ffn: slot_stride %zu must be a multiple of 256 and >= blob bytes %zu", a->slot_stride,
                moe_blob_bytes(a->wfmt, a->H, a->I));
  if (a->T == 0) return MOE_OK;
  MOE_CHECK_ARG(a->x && a->counts && a->offsets && a->perm && a->slot_of_expert && a->slot_pool,
                "moe_expert_ffn: null input pointer");
  MOE_CHECK_ARG(!a->out || (a->topk_w && a->inv), "moe_expert_ffn: out needs topk_w and inv");
  MOE_CHECK_ARG(!(a->out && a->expert_mask), "moe_expert_ffn: with expert_mask set, run moe_combine separately");
  // The matrix-core kernels address their operand rows (x, the SwiGLU
  // output, their MXFP4 encodings) with 32-bit byte offsets.
  if (choose_path(a) != kPathGemv) {
    const long long R = (long long)a->T * a->k + (a->shared_blob ? a->T : 0);
    MOE_CHECK_ARG(R * 2 * std::max(a->H, a->I) < (1LL << 32),
                  "moe_expert_ffn: %lld rows of H=%d / I=%d bf16 values exceed 4 GiB", R, a->H, a->I);
  }
  const WsLayout w = ws_layout(a);
  if (a->workspace_bytes < w.total || (w.total && !a->workspace))
    return set_error(MOE_ENOMEM, "moe_expert_ffn: workspace %zu bytes < %zu needed", a->workspace_bytes, w.total);
  MOE_CHECK_ARG(((uintptr_t)a->workspace & 255) == 0 && ((uintptr_t)a->slot_pool & 255) == 0 &&
                    ((uintptr_t)a->x & 15) == 0 && (!a->y || ((uintptr_t)a->y & 15) == 0) &&
                    (!a->shared_blob || ((uintptr_t)a->shared_blob & 255) == 0),
                "moe_expert_ffn: misaligned pointer (workspace/slot_pool/shared_blob need 256 B, x/y 16 B)");
  return MOE_OK;
}

// Eight expert outputs starting at p (fp32 or bf16) as floats.
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// out[t, c..c+8) = bf16( sum_j w[t,j] * y[inv[t*k+j], c..] (+ y[T*k + t, c..]) ),
// or with inv null (y rows already in flat order) y[t*k+j].
// KMAX >= k: the row indices and weights are loaded first, then every y row
// (branch-free: slots past k re-read row k-1 with weight 0), so the loads
// overlap instead of forming k dependent round trips; flat rows need no
// index load at all.
template <typename YT, int KMAX>
__global__ __launch_bounds__(128) void k_combine(const YT* __restrict__ y, const int32_t* __restrict__ inv,
                                                 const float* __restrict__ w, const YT* __restrict__ ysh, int T,
                                                 int k, int H, uint16_t* __restrict__ out) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 128 + threadIdx.x) * 8;
  if (c >= H) return;
  int row[KMAX];
  float wj[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int jj = min(j, k - 1);
    row[j] = inv ? inv[(size_t)t * k + jj] : t * k + jj;
    wj[j] = w[(size_t)t * k + jj];
  }
  float v[KMAX][8];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) load8(y + (size_t)row[j] * H + c, v[j]);
  float vs[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (ysh) load8(ysh + (size_t)t * H + c, vs);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const float ww = j < k ? wj[j] : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(ww, v[j][i], acc[i]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] += vs[i];
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = bf16x2_rne(acc[2 * i], acc[2 * i + 1]);
  *reinterpret_cast<uint4*>(out + (size_t)t * H + c) = make_uint4(o[0], o[1], o[2], o[3]);
}

template <typename YT>
hipError_t launch_combine(const YT* y, const int32_t* inv, const float* w, const YT* ysh, int T, int k, int H,
                          uint16_t* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 g((H / 8 + 127) / 128, T);
  if (k <= 2) launch(k_combine<YT, 2>, g, dim3(128), 0, s, y, inv, w, ysh, T, k, H, out);
  else if (k <= 4) launch(k_combine<YT, 4>, g, dim3(128), 0, s, y, inv, w, ysh, T, k, H, out);
  else if (k <= 8) launch(k_combine<YT, 8>, g, dim3(128), 0, s, y, inv, w, ysh, T, k, H, out);
  else launch(k_combine<YT, 16>, g, dim3(128), 0, s, y, inv, w, ysh, T, k, H, out);
  return hipGetLastError();
}

// Debug dequantiser: one thread per (tile, lane) fragment.
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ blob, BlobLayout L, int fmt, int which,
                                                 int H, int I, float* __restrict__ out) {
  const BlobView bv = blob_view(blob, L);
  const bool down = which == 2;
  const int rows = down ? H : I, cols = down ? I : H;
  const int KT = k_per_tile(fmt), nk = cols / KT;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long nfrag = (long long)(rows / 16) * nk * 64;
  if (gid >= nfrag) return;
  const int lane = (int)(gid & 63);
  const long long tl = gid >> 6;
  const int kt = (int)(tl % nk), grp = (int)(tl / nk);
  const int rg = down ? grp : 2 * grp + which;  // interleaved gate/up groups
  const size_t tile = (size_t)rg * nk + kt;
  const uint8_t* wsrc = (down ? bv.w2 : bv.w13) + tile * kTileBytes + lane * 16;
  const uint8_t* ssrc = down ? bv.s2 : bv.s13;
  const int row = grp * 16 + (lane & 15);
  const uint4 q = *reinterpret_cast<const uint4*>(wsrc);
  float* o = out + (size_t)row * cols;
  if (fmt == MOE_FMT_BF16) {
    const int c0 = kt * 32 + (lane >> 4) * 8;
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    for (int i = 0; i < 4; ++i) {
      o[c0 + 2 * i] = __uint_as_float(w[i] << 16);
      o[c0 + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    return;
  }
  if (fmt == MOE_FMT_FP8) {
    const int c0 = kt * 64 + (lane >> 4) * 16;
    const float g = which == 0 ? bv.g_gate : (which == 1 ? bv.g_up : bv.g_down);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    for (int i = 0; i < 4; ++i) {
      o[c0 + 4 * i + 0] = __builtin_amdgcn_cvt_f32_fp8((int)w[i], 0) * g;
      o[c0 + 4 * i + 1] = __builtin_amdgcn_cvt_f32_fp8((int)w[i], 1) * g;
      o[c0 + 4 * i + 2] = __builtin_amdgcn_cvt_f32_fp8((int)w[i], 2) * g;
      o[c0 + 4 * i + 3] = __builtin_amdgcn_cvt_f32_fp8((int)w[i], 3) * g;
    }
    return;
  }
  const int c0 = kt * 128 + (lane >> 4) * 32;
  float v[32];
  fp4x32_to_f32(q, v);
  if (fmt == MOE_FMT_MXFP4) {
    const float s = e8m0_to_f32(ssrc[tile * 64 + lane]);
    for (int i = 0; i < 32; ++i) o[c0 + i] = v[i] * s;
  } else {
    const float g = which == 0 ? bv.g_gate : (which == 1 ? bv.g_up : bv.g_down);
    const float s0 = e4m3_to_f32(ssrc[tile * 128 + 2 * lane]), s1 = e4m3_to_f32(ssrc[tile * 128 + 2 * lane + 1]);
    for (int i = 0; i < 32; ++i) o[c0 + i] = (v[i] * (i < 16 ? s0 : s1)) * g;
  }
}

}  // namespace

// Whether moe_expert_ffn runs `a` on the decode GEMV, whose launches write
// only the h and y rows of their masked experts' permutation positions (so
// two calls with disjoint masks may run at once on one workspace and y).
bool moe::ffn_takes_gemv(const moe_ffn_args* a) { return choose_path(a) == kPathGemv; }

extern "C" size_t moe_expert_ffn_workspace_size(const moe_ffn_args* a) {
  if (!a) return 0;
  return ws_layout(a).total;
}

namespace {
FfnParams params_of(const moe_ffn_args* a) {
  FfnParams P{};
  P.T = a->T; P.k = a->k; P.E = a->E; P.H = a->H; P.I = a->I; P.fmt = a->wfmt;
  P.x = a->x; P.counts = a->counts; P.offsets = a->offsets; P.perm = a->perm; P.inv = a->inv;
  P.slot_of_expert = a->slot_of_expert;
  P.slot_pool = static_cast<const uint8_t*>(a->slot_pool);
  P.slot_stride = a->slot_stride;
  P.shared_blob = static_cast<const uint8_t*>(a->shared_blob);
  P.mask = a->expert_mask;
  layout_of(a->wfmt, a->H, a->I, &P.L);
  P.umax = (int)std::min<long long>(a->E, (long long)a->T * a->k);
  return P;
}
}  // namespace

// Routing folded into the expert FFN's first launch (moe_layer).
struct RouteFold {
  const float* logits;
  int renorm;
  int32_t* ids;
};

// Blob copies for the gate/up launch of a GEMV-path call (GemvArgs::copy).
struct CopyReq {
  const FillList* f;
  void* pool;
  size_t slot_bytes;
};

static moe_status run_ffn(const moe_ffn_args* a, hipStream_t s, const RouteFold* rf, const CopyReq* cp = nullptr) {
  FfnParams P = params_of(a);

  const WsLayout w = ws_layout(a);
  uint8_t* ws = static_cast<uint8_t*>(a->workspace);
  float* y = a->y ? a->y : reinterpret_cast<float*>(ws + w.y);
  hipError_t e;
  const Path path = choose_path(a);
  if (path == kPathGemv) {
    GemvArgs G{};
    G.h = reinterpret_cast<uint16_t*>(ws + w.h);
    G.y = y;
    G.trash = reinterpret_cast<float*>(ws + w.trash);
    G.ng = a->I / 32;
    G.nd = a->H / 64;
    // an internal y read only by the combine below: written in flat order,
    // so the combine needs no row-index load
    G.yflat = (!a->y && a->out && (long long)a->T * a->k <= 1024) ? 1 : 0;
    if (rf) {
      G.logits = rf->logits;
      G.renorm = rf->renorm;
      G.ids_out = rf->ids;
      G.w_out = const_cast<float*>(a->topk_w);
    }
    if (cp) {
      G.copy = *cp->f;
      G.copy_wgs = kCopyWgs;
      G.copy_pool = static_cast<uint4*>(cp->pool);
      G.copy_slot_vecs = (uint32_t)(cp->slot_bytes / 16);
    }
    e = launch_gemv(P, G, s);
  } else {
    MfmaBufs B{};
    B.y = y;
    if (internal_bf16_y(a)) B.yb = reinterpret_cast<uint16_t*>(ws + w.y);
    if (path == kPathMfmaFp4) {
      B.xq = ws + w.xq; B.xs = ws + w.xs; B.hq = ws + w.hq; B.hs = ws + w.hs;
      P.inv_ws = reinterpret_cast<int32_t*>(ws + w.inv);
    } else {
      B.hb = reinterpret_cast<uint16_t*>(ws + w.hb);
    }
    e = launch_mfma(P, path == kPathMfmaFp4, B, s);
  }
  if (e != hipSuccess) return set_error(MOE_EHIP, "moe_expert_ffn: launch failed: %s", hipGetErrorString(e));
  if (a->out && internal_bf16_y(a)) {
    const uint16_t* yb = reinterpret_cast<const uint16_t*>(ws + w.y);
    const uint16_t* ysh = a->shared_blob ? yb + (size_t)a->T * a->k * a->H : nullptr;
    e = launch_combine(yb, a->inv, a->topk_w, ysh, a->T, a->k, a->H, a->out, s);
    if (e != hipSuccess) return set_error(MOE_EHIP, "moe_expert_ffn: combine launch failed: %s", hipGetErrorString(e));
  } else if (a->out) {
    const float* ysh = a->shared_blob ? y + (size_t)a->T * a->k * a->H : nullptr;
    const bool yflat = path == kPathGemv && !a->y && (long long)a->T * a->k <= 1024;
    e = launch_combine(y, yflat ? nullptr : a->inv, a->topk_w, ysh, a->T, a->k, a->H, a->out, s);
    if (e != hipSuccess) return set_error(MOE_EHIP, "moe_expert_ffn: combine launch failed: %s", hipGetErrorString(e));
  }
  return MOE_OK;
}

extern "C" moe_status moe_expert_ffn(const moe_ffn_args* a, moe_stream_t stream) {
  moe_status st = check_args(a);
  if (st != MOE_OK || a->T == 0) return st;
  return run_ffn(a, reinterpret_cast<hipStream_t>(stream), nullptr);
}

// moe_expert_ffn on the decode GEMV whose gate/up launch also copies part of
// some blobs from host memory into their slots (f: 1 to kFillMax blobs, the
// range inside slot_bytes, slot_bytes a multiple of 16 below 2^35).  The
// copies land before the down launch starts; none may touch a slot the call
// reads in that range.
moe_status moe::expert_ffn_fill(const moe_ffn_args* a, const FillList& f, void* pool, size_t slot_bytes,
                                hipStream_t s) {
  moe_status st = check_args(a);
  if (st != MOE_OK) return st;
  MOE_CHECK_ARG(a->T > 0 && choose_path(a) == kPathGemv, "expert_ffn_fill: the call must take the decode GEMV");
  MOE_CHECK_ARG(f.n >= 1 && f.n <= kFillMax && pool && slot_bytes % 16 == 0 && slot_bytes / 16 < (1ull << 31) &&
                    (uint64_t)f.off16 + f.len16 <= slot_bytes / 16,
                "expert_ffn_fill: bad copy list");
  const CopyReq cp{&f, pool, slot_bytes};
  return run_ffn(a, s, nullptr, &cp);
}

extern "C" moe_status moe_layer(const moe_layer_args* la, moe_stream_t stream) {
  MOE_CHECK_ARG(la, "moe_layer: null args");
  const moe_ffn_args* a = &la->ffn;
  moe_status st = check_args(a);
  if (st != MOE_OK) return st;
  MOE_CHECK_ARG(a->out && !a->expert_mask, "moe_layer: out is required and expert_mask must be null");
  MOE_CHECK_ARG(a->k <= a->E, "moe_layer: k=%d > E=%d", a->k, a->E);
  if (a->T == 0) return MOE_OK;
  MOE_CHECK_ARG(la->logits && la->topk_ids, "moe_layer: logits and topk_ids are required");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (choose_path(a) == kPathGemv && gemv_route_fits(params_of(a))) {
    const RouteFold rf{la->logits, la->renormalize ? 1 : 0, la->topk_ids};
    return run_ffn(a, s, &rf);
  }
  if ((long long)a->T * a->k <= 1024)
    st = moe_route_permute(la->logits, a->T, a->E, a->k, la->renormalize, la->topk_ids, const_cast<float*>(a->topk_w),
                           const_cast<int32_t*>(a->counts), const_cast<int32_t*>(a->offsets),
                           const_cast<int32_t*>(a->perm), const_cast<int32_t*>(a->inv), stream);
  else {
    st = moe_route(la->logits, a->T, a->E, a->k, la->renormalize, la->topk_ids, const_cast<float*>(a->topk_w), stream);
    if (st == MOE_OK)
      st = moe_permute(la->topk_ids, a->T, a->k, a->E, const_cast<int32_t*>(a->counts), const_cast<int32_t*>(a->offsets),
                       const_cast<int32_t*>(a->perm), const_cast<int32_t*>(a->inv), stream);
  }
  if (st != MOE_OK) return st;
  return run_ffn(a, s, nullptr);
}

extern "C" moe_status moe_debug_fp4_codes(const moe_ffn_args* a, int which, uint8_t* q, uint8_t* s,
                                          moe_stream_t stream) {
  moe_status st = check_args(a);
  if (st != MOE_OK) return st;
  MOE_CHECK_ARG(a->amode == MOE_ACT_MXFP4, "moe_debug_fp4_codes: the call has no MXFP4 activations");
  MOE_CHECK_ARG(which == 0 || which == 1, "moe_debug_fp4_codes: which must be 0 (x) or 1 (SwiGLU output)");
  if (a->T == 0) return MOE_OK;
  MOE_CHECK_ARG(q && s && ((uintptr_t)q & 15) == 0, "moe_debug_fp4_codes: q (16-byte aligned) and s are required");
  const FfnParams P = params_of(a);
  const WsLayout w = ws_layout(a);
  uint8_t* ws = static_cast<uint8_t*>(a->workspace);
  MfmaBufs B{};
  B.xq = ws + w.xq; B.xs = ws + w.xs; B.hq = ws + w.hq; B.hs = ws + w.hs;
  hipError_t e = launch_fp4_codes_canon(P, B, which, q, s, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return set_error(MOE_EHIP, "moe_debug_fp4_codes: launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

// ------------------------------------------------- allocation-free entry point
// The workspace of moe_expert_ffn_noalloc: a static device array, one copy
// per GPU, held until the process ends.  In host code `scratch` names a
// host-side stand-in; its device address on each GPU comes from
// hipGetSymbolAddress, taken once per device on the first call there.
// Nothing in it needs clearing: every kernel reads only workspace bytes the
// same call wrote first.
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch` on each device

moe_status scratch_address(void** out) {
  int dev = -1;
  MOE_HIP(hipGetDevice(&dev));
  MOE_CHECK_ARG(dev >= 0 && dev < kMaxDevices, "moe_expert_ffn_noalloc: device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    MOE_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    MOE_CHECK_ARG(ptr && ((uintptr_t)ptr & 255) == 0, "moe_expert_ffn_noalloc: bad scratch address %p", ptr);
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}
}  // namespace

extern "C" moe_status moe_expert_ffn_noalloc(const moe_ffn_args* a, moe_stream_t stream) {
  MOE_CHECK_ARG(a, "moe_expert_ffn_noalloc: null args");
  moe_ffn_args b = *a;
  const size_t need = moe_expert_ffn_workspace_size(&b);
  if (need > kNoallocScratchBytes)
    return set_error(MOE_ENOMEM, "moe_expert_ffn_noalloc: the call needs %zu bytes of workspace, more than the "
                     "%zu of static scratch (use moe_expert_ffn with a workspace)", need, kNoallocScratchBytes);
  void* ptr = nullptr;
  moe_status st = scratch_address(&ptr);
  if (st != MOE_OK) return st;
  b.workspace = ptr;
  b.workspace_bytes = kNoallocScratchBytes;
  return moe_expert_ffn(&b, stream);
}

thread_local LaunchTrace* moe::g_launch_trace = nullptr;

extern "C" moe_status moe_expert_ffn_traced(const moe_ffn_args* a, moe_stream_t stream, void* const* events,
                                            int n_events, int* n_recorded) {
  MOE_CHECK_ARG(n_events >= 0 && (n_events == 0 || events) && n_recorded, "moe_expert_ffn_traced: bad event list");
  LaunchTrace t{events, n_events, 0};
  g_launch_trace = &t;
  const moe_status st = moe_expert_ffn(a, stream);
  g_launch_trace = nullptr;
  *n_recorded = t.used;
  return st;
}

extern "C" moe_status moe_layer_traced(const moe_layer_args* a, moe_stream_t stream, void* const* events,
                                       int n_events, int* n_recorded) {
  MOE_CHECK_ARG(n_events >= 0 && (n_events == 0 || events) && n_recorded, "moe_layer_traced: bad event list");
  LaunchTrace t{events, n_events, 0};
  g_launch_trace = &t;
  const moe_status st = moe_layer(a, stream);
  g_launch_trace = nullptr;
  *n_recorded = t.used;
  return st;
}

extern "C" moe_status moe_combine(const float* y, const int32_t* inv, const float* topk_w, const float* y_shared, int T,
                                  int k, int H, uint16_t* out, moe_stream_t stream) {
  MOE_CHECK_ARG(T >= 0 && k >= 1 && H > 0 && H % 8 == 0, "moe_combine: bad sizes T=%d k=%d H=%d (H %% 8 == 0)", T, k, H);
  if (T == 0) return MOE_OK;
  MOE_CHECK_ARG(y && inv && topk_w && out, "moe_combine: null pointer");
  MOE_CHECK_ARG(((uintptr_t)y & 15) == 0 && ((uintptr_t)out & 15) == 0 && (!y_shared || ((uintptr_t)y_shared & 15) == 0),
                "moe_combine: y, y_shared and out must be 16-byte aligned");
  hipError_t e = launch_combine(y, inv, topk_w, y_shared, T, k, H, out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return set_error(MOE_EHIP, "moe_combine: launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

extern "C" moe_status moe_quantize_mxfp4(const uint16_t* x, int rows, int cols, uint8_t* q, uint8_t* s,
                                         moe_stream_t stream) {
  MOE_CHECK_ARG(rows >= 0 && cols > 0 && cols % 32 == 0, "moe_quantize_mxfp4: bad sizes rows=%d cols=%d", rows, cols);
  if (rows == 0) return MOE_OK;
  MOE_CHECK_ARG(x && q && s, "moe_quantize_mxfp4: null pointer");
  MOE_CHECK_ARG(((uintptr_t)x & 15) == 0 && ((uintptr_t)q & 15) == 0, "moe_quantize_mxfp4: x and q need 16-byte alignment");
  hipError_t e = launch_quant_mxfp4(x, rows, cols, q, s, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return set_error(MOE_EHIP, "moe_quantize_mxfp4: launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

extern "C" moe_status moe_dequant_blob(const void* blob, int which, float* out, moe_stream_t stream) {
  MOE_CHECK_ARG(blob && out && which >= 0 && which <= 2, "moe_dequant_blob: bad arguments");
  // The header lives in device memory; read it back synchronously (debug entry only).
  BlobHeader h;
  MOE_HIP(hipMemcpy(&h, blob, sizeof h, hipMemcpyDeviceToHost));
  MOE_CHECK_ARG(h.magic == kBlobMagic, "moe_dequant_blob: not a blob (magic %08x)", h.magic);
  BlobLayout L;
  MOE_CHECK_ARG(layout_of(h.fmt, h.H, h.I, &L), "moe_dequant_blob: bad header");
  const int rows = which == 2 ? h.H : h.I, cols = which == 2 ? h.I : h.H;
  const long long nfrag = (long long)(rows / 16) * (cols / k_per_tile(h.fmt)) * 64;
  hipLaunchKernelGGL(k_dequant, dim3((unsigned)((nfrag + 255) / 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const uint8_t*>(blob), L, h.fmt, which, h.H,
                     h.I, out);
  MOE_LAUNCHED();
  return MOE_OK;
}
