/*
 * libmoe — the sparse MoE layer of an expert-offloading inference engine,
 * written for AMD Instinct MI355X (gfx950).  C ABI: plain pointers and sizes.
 *
 * The method (FreeToken, as described on five web pages):
 *   - a routing network picks a few experts for every token at every step
 *     [page "FreeToken qwen：ローカルQwen MoEセットアップガイド", 3rd paragraph;
 *      page "FreeToken量子化：MoE推論のセットアップガイド", 2nd paragraph];
 *   - host RAM holds every routed expert and the GPU keeps one expert cache
 *     shared by all MoE layers; in decode the cache is an LRU over recently
 *     selected experts, a hit runs on the GPU and a miss is brought over PCIe
 *     [page "FreeToken量子化：...", paragraphs on the two-tier expert memory
 *      hierarchy and on decode; bhrtaym-blog page, section
 *      "MoEバックエンドは4種類から選べる", backend table, row "offload"];
 *   - expert weights come as MXFP4, NVFP4 or BF16 checkpoints
 *     [page "FreeToken量子化：...", 3rd paragraph; page "VRAM高騰時代の救世主? ...",
 *      section "FreeTokenとは何か", bullet on formats].
 * The pages give no layer-level API and no formulas; the calls below follow
 * their statement of the problem and the standard definitions (top-k softmax
 * router, SwiGLU expert, OCP MX / OFP8 formats).
 *
 * Conventions (all calls):
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns
 *     every buffer.  No call allocates device memory except
 *     moe_cache_create (host metadata and HIP events only).
 *   - bf16 tensors are passed as uint16_t bit patterns; row-major.
 *   - Every call returns moe_status.  Only host-visible arguments are
 *     validated; device contents (ids out of range, ...) are not.  On a
 *     non-OK status nothing was enqueued and moe_last_error() describes the
 *     problem.  Asynchronous HIP failures surface as MOE_EHIP on a later call.
 *   - Calls taking a hipStream_t only enqueue work on that stream (no host
 *     synchronisation) unless stated otherwise.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* moe_stream_t; /* == hipStream_t */

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,        /* bad dimension, null pointer, bad enum          */
  MOE_EUNSUPPORTED = 2,  /* valid but unsupported combination               */
  MOE_EHIP = 3,          /* a HIP runtime call failed                       */
  MOE_ENOMEM = 4,        /* workspace too small / host allocation failed     */
  MOE_ECACHE = 5         /* a step needs more distinct experts than slots    */
} moe_status;

typedef enum { MOE_FMT_BF16 = 0, MOE_FMT_MXFP4 = 1, MOE_FMT_NVFP4 = 2, MOE_FMT_FP8 = 3 } moe_wfmt;
typedef enum { MOE_ACT_BF16 = 0, MOE_ACT_MXFP4 = 1 } moe_amode;

/* Thread-local description of the last non-OK status of this thread. */
const char* moe_last_error(void);
const char* moe_version(void);

/* ------------------------------------------------------------------ routing */

/* Router logits: logits[t,e] = sum_h x[t,h] * w_router[e,h], fp32 accumulation.
 * [page "FreeToken qwen：...", 3rd paragraph: a routing network selects a
 *  subset of experts per step.]
 * x: [T,H] bf16; w_router: [E,H] fp32; logits: [T,E] fp32.
 * Requires T >= 0, H >= 1, 1 <= E. */
moe_status moe_router_logits(const uint16_t* x, const float* w_router, int T, int H, int E,
                             float* logits, moe_stream_t stream);

/* Top-k routing with softmax weights.
 * [pages as for moe_router_logits; the selection rule is this library's
 *  reading: keys are the fp32 logits, larger first, ties to the lower expert
 *  id, NaN below -inf; ids of a row are written in rank order.]
 * renormalize=1: w_j = exp(l_j - m) / sum over the k selected (m = top logit);
 * renormalize=0: the softmax over all E experts, at the selected ids.
 * exp(l - m) is taken as 1 where l == m and 0 where l is NaN; a row whose
 * weights would all be 0 gets 1/k each.
 * logits: [T,E] fp32; topk_ids: [T,k] int32; topk_w: [T,k] fp32.
 * Requires 1 <= k <= min(E, 16), E <= 1024, T >= 0. */
moe_status moe_route(const float* logits, int T, int E, int k, int renormalize,
                     int32_t* topk_ids, float* topk_w, moe_stream_t stream);

/* Token -> expert permutation: a stable counting sort of the T*k flat
 * indices f = t*k + j by expert id (ties in ascending f), so that the rows
 * every expert processes are contiguous.
 * [page "FreeToken量子化：MoE推論のセットアップガイド", 2nd paragraph: each
 *  token passes through only a few of the experts, so the work of a step is
 *  grouped per expert; the stable order is this library's reading.]
 * counts: [E]; offsets: [E+1] (exclusive scan, offsets[E] = T*k);
 * perm: [T*k] (perm[p] = flat index at sorted position p);
 * inv: [T*k] (inv[perm[p]] = p).  topk_ids values must lie in [0, E).
 * Requires E <= 1024, T*k <= 2^24. */
moe_status moe_permute(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* inv, moe_stream_t stream);

/* moe_route followed by moe_permute, in a single launch when T*k <= 1024
 * (decode batches): one workgroup selects the experts of every token and
 * sorts the (token, slot) pairs without a round trip through a second launch.
 * Same arguments, results and requirements as the two calls. */
moe_status moe_route_permute(const float* logits, int T, int E, int k, int renormalize, int32_t* topk_ids,
                             float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                             moe_stream_t stream);

/* ------------------------------------------------------------- expert FFN */

/* Prepacked expert ("slot blob") layout, shared by the host bank and the HBM
 * slots: a 256-byte header, then gate/up and down weights and scales in the
 * tile order the kernels stream.  See moe_blob_bytes / moe_prepack_expert. */
typedef struct {
  int32_t fmt;            /* moe_wfmt                                         */
  int32_t H, I;           /* hidden, intermediate; both multiples of 128      */
  /* canonical row-major tensors (host): gate, up [I,H]; down [H,I]
   *   BF16 : w_* = uint16 bf16 bits [rows, cols]
   *   MXFP4: q_* = E2M1 codes [rows, cols/2] (element 2i in the low nibble),
   *          s_* = E8M0 codes [rows, cols/32]
   *   NVFP4: q_* as MXFP4, s_* = E4M3FN codes [rows, cols/16],
   *          g_* = per-tensor dequant multiplier (w = E2M1 * E4M3 * g)
   *   FP8  : q_* = E4M3FN codes [rows, cols], s_* unused,
   *          g_* = per-tensor dequant multiplier (w = E4M3 * g)            */
  const void* gate_q; const uint8_t* gate_s; float gate_g;
  const void* up_q;   const uint8_t* up_s;   float up_g;
  const void* down_q; const uint8_t* down_s; float down_g;
} moe_expert_canonical;

/* Bytes of one expert blob for (fmt, H, I); 0 if the shape is unsupported.
 * [page "FreeToken量子化：...", 3rd paragraph: MXFP4, NVFP4 and BF16 expert
 *  checkpoints; bhrtaym-blog page, section on models and quantisation
 *  formats: MXFP4, NVFP4, FP8 and BF16; paragraph on the two-tier expert memory hierarchy: every
 *  routed expert is held in host RAM and copied whole into a GPU cache slot,
 *  so one expert is one fixed-size blob.]  H and I must be multiples of 128
 *  (this library's tile width; every shape the pages name satisfies it). */
size_t moe_blob_bytes(int fmt, int H, int I);

/* Host-side prepack of one expert into blob_out (host, >= moe_blob_bytes).
 * A bijection of the canonical tensors (round-trip tested).
 * [pages as for moe_blob_bytes: the blob is what host RAM holds and what a
 *  cache fill copies; the tile order inside it is this library's.]
 * Returns MOE_EINVAL for a null pointer, a bad format or shape, or
 * blob_bytes < moe_blob_bytes(fmt, H, I). */
moe_status moe_prepack_expert(const moe_expert_canonical* src, void* blob_out, size_t blob_bytes);

/* Arguments of one expert-FFN call (SwiGLU: y = W_down (silu(W_gate x) * (W_up x))).
 * [page "FreeToken量子化：...", decode paragraph: cached experts execute on the
 *  GPU; the expert form is this library's reading (SwiGLU, no bias).] */
typedef struct {
  int T, k, E, H, I;            /* tokens, top-k, routed experts, hidden, intermediate */
  int wfmt;                     /* moe_wfmt of every blob (routed and shared)            */
  int amode;                    /* MOE_ACT_BF16: activations stay bf16 / fp32.
                                   MOE_ACT_MXFP4 (wfmt MXFP4 only): x and the SwiGLU output
                                   are MXFP4-encoded per row per 32 values and the products
                                   run on the block-scaled FP4 matrix cores.             */
  const uint16_t* x;            /* [T,H] bf16                                            */
  const int32_t* counts;        /* [E]    from moe_permute                               */
  const int32_t* offsets;       /* [E+1]  from moe_permute                               */
  const int32_t* perm;          /* [T*k]  from moe_permute                               */
  const int32_t* slot_of_expert;/* [E]    slot index of each routed expert's blob        */
  const void* slot_pool;        /* base of the slots; blob of expert e at
                                   slot_pool + slot_of_expert[e] * slot_stride           */
  size_t slot_stride;           /* bytes, >= moe_blob_bytes, multiple of 256             */
  const void* shared_blob;      /* nullable: always-on shared expert (same fmt, H, I),
                                   weight 1, added after the routed sum                  */
  const uint8_t* expert_mask;   /* nullable: [E]; if set only experts with mask[e] != 0
                                   run (lets hits run while misses are still copying);
                                   out must then be null (combine with moe_combine)      */
  float* y;                     /* nullable: [T*k (+T if shared)][H] fp32 expert outputs
                                   in perm order (shared rows last).  If null, y lives in
                                   the workspace (as bf16 on the matrix-core paths when
                                   out is set: the combine then reads bf16 values).      */
  const float* topk_w;          /* nullable with out: [T,k] routing weights              */
  const int32_t* inv;           /* nullable with out: [T*k] from moe_permute             */
  uint16_t* out;                /* nullable: [T,H] bf16; if set, the combine runs too    */
  void* workspace;              /* device scratch, >= moe_expert_ffn_workspace_size, 256-byte
                                   aligned; no contents carry over between calls.  Calls
                                   that share a workspace must not overlap.                */
  size_t workspace_bytes;
} moe_ffn_args;

/* Bytes of device workspace a call with these dimensions needs. */
size_t moe_expert_ffn_workspace_size(const moe_ffn_args* a);

/* Grouped expert FFN over every expert with at least one row (and the shared
 * expert).  Small batches run a dequantising GEMV that streams each touched
 * expert's weights once; large batches run a grouped GEMM on the matrix cores
 * (bf16 MFMA for BF16 weights, block-scaled FP4 MFMA for MXFP4 with amode
 * MXFP4).  Requires H, I multiples of 128 (this library's tile width; the
 * formats themselves need multiples of 32), 1 <= k <= 16, E <= 1024, T*k <=
 * 131072, and on the matrix-core paths R * max(H, I) * 2 < 2^32 bytes
 * (R = T*k, +T with a shared expert).
 * Errors: MOE_EINVAL (sizes, null or misaligned pointers), MOE_EUNSUPPORTED
 * (MXFP4 activations with other weights), MOE_ENOMEM (workspace too small),
 * MOE_EHIP (a launch failed); nothing is enqueued on an error. */
moe_status moe_expert_ffn(const moe_ffn_args* a, moe_stream_t stream);

/* One whole layer call: routing (moe_route + moe_permute), the expert FFN and
 * the combine, with results equal to moe_route_permute(logits, ...)
 * followed by moe_expert_ffn(&ffn), in as few launches as the batch
 * allows: for decode batches of up to 4 tokens (T*k <= 64, E <= 256, the
 * bf16-activation path) the routing runs inside the gate/up launch, which
 * saves the routing kernel and its boundary.
 * [pages as for moe_route and moe_expert_ffn.]
 * ffn.counts, offsets, perm, inv and topk_w are outputs here (written by
 * the call); ffn.out is required, ffn.expert_mask must be null.  logits:
 * [T,E] fp32; topk_ids: [T,k] output. */
typedef struct {
  const float* logits;
  int renormalize;
  int32_t* topk_ids;
  moe_ffn_args ffn;
} moe_layer_args;
moe_status moe_layer(const moe_layer_args* a, moe_stream_t stream);

/* moe_layer timing its expert-FFN launches as moe_expert_ffn_traced does
 * (a separate routing kernel, when one runs, records no events); with the
 * routing folded in, launch 0 is the gate/up launch that routes. */
moe_status moe_layer_traced(const moe_layer_args* a, moe_stream_t stream, void* const* events, int n_events,
                            int* n_recorded);

/* moe_expert_ffn without a caller workspace and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  a->workspace and
 * a->workspace_bytes are ignored: the kernels use a static device scratch
 * array of 32 MiB (one per GPU, held until the process ends; its address is
 * looked up on the first call on each device).  Calls whose
 * moe_expert_ffn_workspace_size exceeds 32 MiB return MOE_ENOMEM before any
 * device work (decode batches need a few MiB; large prefills do not fit).
 * Every call on a GPU shares that GPU's scratch: calls that overlap on one
 * GPU (on different streams, or from several host threads) race and must be
 * ordered by the caller.  Otherwise as moe_expert_ffn. */
moe_status moe_expert_ffn_noalloc(const moe_ffn_args* a, moe_stream_t stream);

/* moe_expert_ffn, timing each of its kernel launches with caller-created HIP
 * events (hipEvent_t, passed as void*): launch i records events[2i] and
 * events[2i + 1] at the kernel's own start and end (hipExtLaunchKernelGGL),
 * for as many launches as n_events covers; *n_recorded (host) receives the
 * number of events recorded.  Launch order: BF16-activation GEMV path:
 * gate/up, down[, combine]; FP4 matrix-core path: activation quantiser,
 * gate/up, down[, combine]; BF16 matrix-core path: gate/up, down[, combine].
 * For measuring one kernel of the layer; not for stream capture. */
moe_status moe_expert_ffn_traced(const moe_ffn_args* a, moe_stream_t stream, void* const* events, int n_events,
                                 int* n_recorded);

/* Weighted combine back to token order:
 * out[t,:] = bf16( sum_{j=0..k-1} topk_w[t,j] * y[inv[t*k+j],:]  (+ y_shared[t,:]) ).
 * [page "FreeToken量子化：MoE推論のセットアップガイド", 2nd paragraph: a token's
 *  output is made from the few experts it passed through; page "FreeToken
 *  qwen：...", 3rd paragraph: the router's choice per step.  Weighting by the
 *  routing weights, j ascending, the shared expert added last with weight 1,
 *  and bf16 rounding are this library's reading.]
 * y: [T*k][H] fp32 in perm order; y_shared: nullable [T][H] fp32. */
moe_status moe_combine(const float* y, const int32_t* inv, const float* topk_w, const float* y_shared,
                       int T, int k, int H, uint16_t* out, moe_stream_t stream);

/* MXFP4 encoding of bf16 activations, per row per 32 values (the activation
 * quantiser of the FP4 matrix-core path): shared exponent floor(log2 amax)-2
 * (E8M0, 127 for an all-zero block), elements round-to-nearest-even on the
 * E2M1 grid, saturating at 6, sign from the input.
 * x: [rows, cols] bf16; q: [rows, cols/2] bytes (element 2i low nibble);
 * s: [rows, cols/32] E8M0.  cols % 32 == 0. */
moe_status moe_quantize_mxfp4(const uint16_t* x, int rows, int cols, uint8_t* q, uint8_t* s,
                              moe_stream_t stream);

/* Debug: the MXFP4 encodings an FP4 matrix-core call (amode MXFP4) left in
 * its workspace, copied to canonical layout, for the bit-exact tests of the
 * activation quantiser.  Enqueue on the call's stream after moe_expert_ffn
 * with the same arguments, before the workspace is reused.
 * which = 0: x, which = 1: the SwiGLU output h.  q: [R][K/2] bytes (element
 * 2i in the low nibble, 16-byte aligned), s: [R][K/32] E8M0, K = H (x) or I
 * (h), R = T*k (+T with a shared expert); row p is permutation-order row p
 * (token perm[p] / k), rows T*k.. are the shared expert's tokens 0..T-1. */
moe_status moe_debug_fp4_codes(const moe_ffn_args* a, int which, uint8_t* q, uint8_t* s, moe_stream_t stream);

/* Debug: dequantise projection `which` (0 gate, 1 up, 2 down) of a device blob
 * into out [rows, cols] fp32 (canonical order).  Used by the bit-exact tests. */
moe_status moe_dequant_blob(const void* blob, int which, float* out, moe_stream_t stream);

/* ------------------------------------------------------- expert-slot cache */

/* The HBM expert cache: num_slots slots of slot_bytes each, in a device
 * buffer owned by the caller, shared by num_layers layers of num_experts
 * experts.  Keys are (layer, expert) = layer*num_experts + expert.
 * [page "FreeToken量子化：...", hierarchy and decode paragraphs; bhrtaym-blog
 *  page, backend table row "offload".]  The cache holds host metadata and
 * HIP events only.  One cache per host thread.  Returns NULL on bad
 * arguments (see moe_last_error). */
typedef struct moe_cache moe_cache;
moe_cache* moe_cache_create(int num_slots, size_t slot_bytes, void* slot_pool, int num_layers,
                            int num_experts);
void moe_cache_destroy(moe_cache* c);

/* Look up the distinct, ascending expert ids (host) of one step of `layer`.
 * [page "FreeToken量子化：...", decode paragraph: the cache is an LRU over
 *  the recently selected experts of all layers, a hit runs on the GPU, a
 *  miss is brought in; bhrtaym-blog page, backend table row "offload".  The
 *  key, the lookup order and the slot choice are this library's reading.]
 * Host-only and synchronous.  For each id: slot[i] (host), hit[i] (host,
 * 1/0) and evicted_key[i] (host, the key whose slot a miss took, -1 if the
 * slot was free or on a hit).  Every access makes its key most recent; a miss
 * takes the lowest free slot, else evicts the least recently used key.  Keys
 * of this call are never evicted by it.  n > num_slots returns MOE_ECACHE
 * and leaves the state unchanged; unsorted / duplicate / out-of-range ids
 * return MOE_EINVAL and leave the state unchanged. */
moe_status cache_lookup(moe_cache* c, int layer, const int32_t* ids, int n, int32_t* slot,
                        uint8_t* hit, int32_t* evicted_key);

/* Fill `slot` with the blob of (layer, expert) from pinned host memory.
 * [page "FreeToken量子化：...", decode paragraph: a miss is copied over PCIe
 *  from host RAM into the GPU cache; paragraph on double buffering: the copy
 *  of some experts overlaps the computation of others.]
 * Enqueues on copy_stream: wait until every compute-stream use of the slot
 * recorded by moe_cache_mark_used has finished (write-after-read guard), then
 * hipMemcpyAsync host->device of slot_bytes, then an event; then makes
 * compute_stream wait on that event (read-after-write guard).  Compute work
 * enqueued on compute_stream before this call may overlap the copy.
 * host_src must be pinned (hipHostMalloc) and hold slot_bytes bytes. */
moe_status cache_fill(moe_cache* c, int layer, int expert, int slot, const void* host_src,
                      moe_stream_t copy_stream, moe_stream_t compute_stream);

/* Record on compute_stream that slots[0..n) (host) are read by the work
 * enqueued so far; a later cache_fill of one of them waits for that work. */
moe_status moe_cache_mark_used(moe_cache* c, const int32_t* slots, int n, moe_stream_t compute_stream);

/* Decode steps copy their misses through the copy engine (on != 0) even
 * where the fill kernel of moe_cache_decode_step could (on == 0, the
 * default).  Both orders give the same results and trace. */
moe_status moe_cache_use_copy_engine(moe_cache* c, int on);

/* Hits, misses and bytes copied by cache_fill since creation or reset (host). */
moe_status moe_cache_stats(const moe_cache* c, long long* hits, long long* misses, long long* bytes_filled);

/* One decode step of one MoE layer through the expert cache: routing, slot
 * lookup, miss fills and the expert FFN with its combine.
 * [page "FreeToken量子化：...", decode paragraph: the router picks experts,
 *  hits run on the GPU at once, misses come over PCIe into LRU slots shared
 *  by all layers; page "...", hierarchy paragraph: double buffering lets the
 *  transfer of some experts overlap the computation of others.]
 * The call enqueues, in this order:
 *   1. moe_route_permute(logits) into ffn.topk_w / ffn.counts / ffn.offsets /
 *      ffn.perm / ffn.inv and topk_ids, on compute_stream;
 *   2. a copy of counts to host_counts, and waits for it (the host must
 *      know the step's experts: this is the step's one host synchronisation);
 *   3. cache_lookup of the experts with rows, in ascending id (the trace);
 *   4-6. the miss fills, the slot map and the two FFN calls, in one of two
 *      orders.  Fill kernel (the FFN takes the decode GEMV, at most 64 misses
 *      and 256 experts, every miss blob mapped pinned memory on a 16-byte
 *      boundary, and moe_cache_use_copy_engine not set): one kernel on
 *      compute_stream copies the header and gate/up weights of every miss
 *      blob from host memory into its slot and writes dev_map, then the FFN
 *      over the missed experts follows, its gate/up launch copying the down
 *      weights while it runs; meanwhile the FFN over the hit experts (and
 *      the shared expert) runs on a stream the cache owns, with its own copy
 *      of the map, and compute_stream waits for it before the combine.  A
 *      failure after the lookups leaves no key mapped to a slot whose blob
 *      did not arrive.  Copy engine (otherwise): for every miss a fill
 *      from host_blobs[expert] on copy_stream (after the slot's previous
 *      readers), the slot map and masks host_map -> dev_map, the FFN over the
 *      hit experts (overlapping the fills), a wait on each miss's fill, then
 *      the FFN over the missed experts;
 *   7. moe_combine into ffn.out, and moe_cache_mark_used of the step's slots.
 * ffn.slot_of_expert, ffn.expert_mask are set by the call; ffn.y is
 * required; ffn.out, topk_w, inv receive the combine.  host_counts and
 * host_map are pinned (hipHostMalloc) host buffers of 4E and
 * moe_cache_map_bytes(E) bytes, dev_map a device buffer of that size;
 * host_counts and dev_map may be reused by a later step on the same
 * compute_stream, and a step waits for the previous upload from its host_map
 * before rewriting it.  The trace
 * arrays (host, capacity E) receive the step's n_experts records. */
typedef struct {
  int layer;
  const float* logits;          /* [T,E] fp32 router logits of the step             */
  int renormalize;
  int32_t* topk_ids;            /* [T,k] device                                     */
  int32_t* host_counts;         /* pinned host [E]                                  */
  void* host_map;               /* pinned host, moe_cache_map_bytes(E)              */
  void* dev_map;                /* device, moe_cache_map_bytes(E), 256-byte aligned */
  const void* const* host_blobs;/* host [E]: pinned blob of each expert of `layer`  */
  moe_ffn_args ffn;
  int32_t* trace_expert;        /* host [E] (nullable together)                     */
  int32_t* trace_slot;
  uint8_t* trace_hit;
  int32_t* trace_evicted;
  int n_experts;                /* out: distinct experts of the step                */
} moe_cache_step;

size_t moe_cache_map_bytes(int E);
moe_status moe_cache_decode_step(moe_cache* c, moe_cache_step* s, moe_stream_t copy_stream,
                                 moe_stream_t compute_stream);

/* ------------------------------------------------- layer-ahead prefill
 * [page "FreeToken量子化：MoE推論のセットアップガイド", paragraph on prefill:
 *  the experts of the next layer are copied over PCIe while the current
 *  layer computes, double buffering whole layers.]  A prefill batch routes
 * its tokens to nearly every expert, so a layer's step needs all of its
 * experts: moe_cache_prefetch_layer(l + 1) is called right after
 * moe_cache_prefill_step(l), and its copies overlap that step's compute.  A
 * cache of 2E slots holds the layer computing and the layer arriving.
 * Neither call synchronises the host.  All steps of a cache run on one
 * compute stream. */

/* Look up every expert of `layer` in ascending id (misses take the lowest
 * free slot, else evict the least recently used key), fill each miss from
 * host_blobs[e] (pinned, slot_bytes each) on copy_stream after its slot's
 * last readers, and upload the layer's slot map (moe_cache_map_bytes(E):
 * int32 slot of every expert first) from host_map (pinned; rewritten only
 * after its previous upload) to dev_map (device, 256-byte aligned) on
 * compute_stream.  trace_slot / trace_hit / trace_evicted (host [E],
 * nullable together) receive the lookups of experts 0..E-1.  Returns
 * MOE_ECACHE (cache unchanged) if E > num_slots. */
moe_status moe_cache_prefetch_layer(moe_cache* c, int layer, const void* const* host_blobs, void* host_map,
                                    void* dev_map, int32_t* trace_slot, uint8_t* trace_hit, int32_t* trace_evicted,
                                    moe_stream_t copy_stream, moe_stream_t compute_stream);

/* One prefill step of a layer whose experts were prefetched. */
typedef struct {
  int layer;
  const float* logits;          /* [T,E] fp32 router logits                          */
  int renormalize;
  int32_t* topk_ids;            /* [T,k] device                                      */
  const void* dev_map;          /* the layer's map from moe_cache_prefetch_layer     */
  moe_ffn_args ffn;             /* T, k, E, H, I, wfmt, amode, x, counts, offsets,
                                   perm, inv, topk_w, out (required), y (nullable),
                                   shared_blob, workspace; slot_of_expert, slot_pool,
                                   slot_stride and expert_mask are set by the call    */
  int32_t* trace_slot;          /* host [E] (nullable together): the lookups         */
  uint8_t* trace_hit;
  int32_t* trace_evicted;
} moe_cache_prefill;

/* Looks up every expert of s->layer (all hits, ascending id: the step's
 * trace), makes compute_stream wait for the layer's fills, then enqueues
 * routing, permutation, the expert FFN and the combine into ffn.out on
 * compute_stream, and records the layer's slots as read by them.  Returns
 * MOE_ECACHE with the cache unchanged if an expert of the layer is not
 * cached (its prefetch did not run, or a later one evicted it). */
moe_status moe_cache_prefill_step(moe_cache* c, moe_cache_prefill* s, moe_stream_t compute_stream);

/* ------------------------------------------------- hybrid miss policy
 * [page "FreeToken量子化：MoE推論のセットアップガイド", decode paragraph: a
 *  miss is either brought over PCIe into the cache or executed on the CPU,
 *  by the host-memory and PCIe bandwidths measured on the machine; paragraph
 *  on the bandwidth-adaptive policy; bhrtaym-blog page, section
 *  "MoEバックエンドは4種類から選べる": backend rows "cpu" (misses computed on
 *  the CPU, not fetched) and "hybrid" (part of the misses copied, the rest
 *  computed on the CPU, overlapped), and the one-time bandwidth calibration
 *  run before hybrid is used.] */

/* The expert FFN of one blob on the host: y[t,:] = W_down (silu(W_gate x_t) *
 * (W_up x_t)) for the n bf16 rows x [n,H] (host), y [n,H] fp32 (host); fp32
 * accumulation, per-tensor multipliers applied to the sums, `threads` host
 * threads (a pool kept until the process ends).  blob: host memory holding
 * a prepacked blob (any format).  Synchronous; no GPU work. */
moe_status moe_cpu_expert_ffn(const void* blob, const uint16_t* x, int n, float* y, int threads);

/* Result of the one-time bandwidth calibration. */
typedef struct {
  double copy_us;    /* one blob, pinned host -> device                          */
  double cpu_us;     /* moe_cpu_expert_ffn of that blob on one token row          */
  double h2d_gbs;    /* blob bytes / copy_us                                      */
  double host_gbs;   /* blob bytes / cpu_us: the host kernel's weight stream rate  */
  float copy_ratio;  /* share of a step's misses to copy: cpu_us / (cpu_us + copy_us),
                        which makes the copies and the host's run take equal time */
} moe_bw_calib;

/* Times `reps` copies of host_blob (pinned, a prepacked blob) into dev_buf
 * (device, at least the blob's size) on copy_stream, and `reps` runs of
 * moe_cpu_expert_ffn on it with `threads` threads; synchronises the host.
 * The copies take the path of moe_cache_decode_step's misses: the fill
 * kernel when host_blob is mapped pinned memory and both pointers are on
 * 16-byte boundaries, else the copy engine. */
moe_status moe_calibrate_bw(const void* host_blob, void* dev_buf, int reps, int threads, moe_stream_t copy_stream,
                            moe_bw_calib* out);

/* Host buffers and policy of moe_cache_decode_step_hybrid. */
typedef struct {
  float copy_ratio;       /* in [0, 1]: of a step's m misses, the first
                             floor(copy_ratio * m + 0.5) in ascending id are
                             copied into the cache; the rest run on the host and
                             are not cached (1: every miss copied; 0: none)      */
  int threads;            /* host threads of moe_cpu_expert_ffn                  */
  uint16_t* host_x;       /* pinned [T,H]: the step's token rows                 */
  int32_t* host_perm;     /* pinned [T*k]                                        */
  int32_t* host_offsets;  /* pinned [E+1]                                        */
  float* host_y;          /* pinned [T*k][H]: expert outputs of host-run experts  */
  long long cpu_experts;  /* in/out: incremented by the experts run on the host   */
} moe_hybrid;

/* moe_cache_decode_step with the hybrid miss policy: the step's routing,
 * counts, offsets, permutation and token rows come to the host (its one
 * synchronisation); hits and the looked-up misses are handled as in
 * moe_cache_decode_step (lookups in ascending id, fills on copy_stream, the
 * FFN on the GPU); each miss past the copied share runs on the host, after
 * the GPU's hit FFN is enqueued, and its outputs are copied into ffn.y
 * before the combine.  The trace lists every expert of the step in
 * ascending id; a host-run miss has hit 0, slot -1 and evicted key -1 and
 * leaves the cache unchanged.  s->host_blobs must point to prepacked blobs
 * the host can read. */
moe_status moe_cache_decode_step_hybrid(moe_cache* c, moe_cache_step* s, moe_hybrid* hy, moe_stream_t copy_stream,
                                        moe_stream_t compute_stream);

/* Resize the cache at a safe point (between layer calls, no step in flight).
 * [page "FreeToken量子化：MoE推論のセットアップガイド", paragraph on resizing
 *  the expert cache at runtime at scheduler safe points.]
 * The cache moves to num_slots slots in slot_pool (same slot size, 256-byte
 * aligned, not overlapping the current pool).  It keeps the min(num_slots,
 * cached) most recently used keys, packed into slots 0, 1, ... from least to
 * most recent with their recency order unchanged, and drops the rest; later
 * misses take the free slots above them, lowest first.  The kept blobs are
 * copied device to device on `stream` (one kernel per 256 blobs) after every
 * fill enqueued so far has landed.  Later steps must run on `stream` or be ordered after it
 * by the caller; later fills wait for the copies themselves.  The caller may
 * release the old pool once the copies and every earlier reader of it have
 * finished (e.g. after synchronising `stream` when all steps ran on it).  The
 * slot size and the current pool must be multiples of 16 bytes.  Returns
 * MOE_EINVAL for bad arguments (cache unchanged). */
moe_status moe_cache_resize(moe_cache* c, int num_slots, void* slot_pool, moe_stream_t stream);

/* Reset the cache to the empty state (host metadata only). */
moe_status moe_cache_reset(moe_cache* c);

/* Pre-fill bookkeeping for a fully resident layer: key (layer, e) -> slot s0 + e
 * for e in [0, num_experts); no copy is made (the caller placed the blobs). */
moe_status moe_cache_pin_resident(moe_cache* c, int layer, int s0);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
