"""ctypes binding of libmoe.so: argument marshalling only.

Every function has the name of the C entry point it wraps and forwards to it;
device tensors are passed as ``data_ptr()`` values, the stream defaults to
torch's current HIP stream.  All arithmetic happens in the library's kernels.
A missing library is an error (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EHIP, MOE_ENOMEM, MOE_ECACHE = range(6)
FMT = {"bf16": 0, "mxfp4": 1, "nvfp4": 2, "fp8": 3}
AMODE = {"bf16": 0, "mxfp4": 1}
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_EINVAL", 2: "MOE_EUNSUPPORTED", 3: "MOE_EHIP", 4: "MOE_ENOMEM", 5: "MOE_ECACHE"}


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class FfnArgs(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int), ("k", ctypes.c_int), ("E", ctypes.c_int), ("H", ctypes.c_int), ("I", ctypes.c_int),
        ("wfmt", ctypes.c_int), ("amode", ctypes.c_int),
        ("x", ctypes.c_void_p), ("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p), ("perm", ctypes.c_void_p),
        ("slot_of_expert", ctypes.c_void_p), ("slot_pool", ctypes.c_void_p), ("slot_stride", ctypes.c_size_t),
        ("shared_blob", ctypes.c_void_p), ("expert_mask", ctypes.c_void_p),
        ("y", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("inv", ctypes.c_void_p), ("out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class LayerArgs(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("renormalize", ctypes.c_int), ("topk_ids", ctypes.c_void_p),
                ("ffn", FfnArgs)]


class CacheStep(ctypes.Structure):
    _fields_ = [
        ("layer", ctypes.c_int), ("logits", ctypes.c_void_p), ("renormalize", ctypes.c_int),
        ("topk_ids", ctypes.c_void_p), ("host_counts", ctypes.c_void_p), ("host_map", ctypes.c_void_p),
        ("dev_map", ctypes.c_void_p), ("host_blobs", ctypes.c_void_p), ("ffn", FfnArgs),
        ("trace_expert", ctypes.c_void_p), ("trace_slot", ctypes.c_void_p), ("trace_hit", ctypes.c_void_p),
        ("trace_evicted", ctypes.c_void_p), ("n_experts", ctypes.c_int),
    ]


class CachePrefill(ctypes.Structure):
    _fields_ = [
        ("layer", ctypes.c_int), ("logits", ctypes.c_void_p), ("renormalize", ctypes.c_int),
        ("topk_ids", ctypes.c_void_p), ("dev_map", ctypes.c_void_p), ("ffn", FfnArgs),
        ("trace_slot", ctypes.c_void_p), ("trace_hit", ctypes.c_void_p), ("trace_evicted", ctypes.c_void_p),
    ]


class BwCalib(ctypes.Structure):
    _fields_ = [("copy_us", ctypes.c_double), ("cpu_us", ctypes.c_double), ("h2d_gbs", ctypes.c_double),
                ("host_gbs", ctypes.c_double), ("copy_ratio", ctypes.c_float)]


class Hybrid(ctypes.Structure):
    _fields_ = [("copy_ratio", ctypes.c_float), ("threads", ctypes.c_int), ("host_x", ctypes.c_void_p),
                ("host_perm", ctypes.c_void_p), ("host_offsets", ctypes.c_void_p), ("host_y", ctypes.c_void_p),
                ("cpu_experts", ctypes.c_longlong)]


class ExpertCanonical(ctypes.Structure):
    _fields_ = [
        ("fmt", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
        ("gate_q", ctypes.c_void_p), ("gate_s", ctypes.c_void_p), ("gate_g", ctypes.c_float),
        ("up_q", ctypes.c_void_p), ("up_s", ctypes.c_void_p), ("up_g", ctypes.c_float),
        ("down_q", ctypes.c_void_p), ("down_s", ctypes.c_void_p), ("down_g", ctypes.c_float),
    ]


# name -> (restype, argtypes); the exported C ABI (include/moe.h)
_vp, _i, _sz, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
SIGNATURES = {
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_version": (ctypes.c_char_p, []),
    "moe_router_logits": (_i, [_vp, _vp, _i, _i, _i, _vp, _vp]),
    "moe_route": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp]),
    "moe_permute": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp]),
    "moe_route_permute": (_i, [_vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_blob_bytes": (_sz, [_i, _i, _i]),
    "moe_prepack_expert": (_i, [ctypes.POINTER(ExpertCanonical), _vp, _sz]),
    "moe_expert_ffn_workspace_size": (_sz, [ctypes.POINTER(FfnArgs)]),
    "moe_expert_ffn": (_i, [ctypes.POINTER(FfnArgs), _vp]),
    "moe_expert_ffn_noalloc": (_i, [ctypes.POINTER(FfnArgs), _vp]),
    "moe_layer": (_i, [ctypes.POINTER(LayerArgs), _vp]),
    "moe_layer_traced": (_i, [ctypes.POINTER(LayerArgs), _vp, _vp, _i, _vp]),
    "moe_expert_ffn_traced": (_i, [ctypes.POINTER(FfnArgs), _vp, _vp, _i, _vp]),
    "moe_combine": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _vp, _vp]),
    "moe_quantize_mxfp4": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
    "moe_dequant_blob": (_i, [_vp, _i, _vp, _vp]),
    "moe_debug_fp4_codes": (_i, [ctypes.POINTER(FfnArgs), _i, _vp, _vp, _vp]),
    "moe_cache_create": (_vp, [_i, _sz, _vp, _i, _i]),
    "moe_cache_destroy": (None, [_vp]),
    "cache_lookup": (_i, [_vp, _i, _vp, _i, _vp, _vp, _vp]),
    "cache_fill": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp]),
    "moe_cache_mark_used": (_i, [_vp, _vp, _i, _vp]),
    "moe_cache_reset": (_i, [_vp]),
    "moe_cache_use_copy_engine": (_i, [_vp, _i]),
    "moe_cache_pin_resident": (_i, [_vp, _i, _i]),
    "moe_cache_stats": (_i, [_vp, _vp, _vp, _vp]),
    "moe_cache_map_bytes": (_sz, [_i]),
    "moe_cache_decode_step": (_i, [_vp, ctypes.POINTER(CacheStep), _vp, _vp]),
    "moe_cache_resize": (_i, [_vp, _i, _vp, _vp]),
    "moe_cache_prefetch_layer": (_i, [_vp, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_cache_prefill_step": (_i, [_vp, ctypes.POINTER(CachePrefill), _vp]),
    "moe_cpu_expert_ffn": (_i, [_vp, _vp, _i, _vp, _i]),
    "moe_calibrate_bw": (_i, [_vp, _vp, _i, _i, _vp, ctypes.POINTER(BwCalib)]),
    "moe_cache_decode_step_hybrid": (_i, [_vp, ctypes.POINTER(CacheStep), ctypes.POINTER(Hybrid), _vp, _vp]),
}

_lib = None


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(python -m fp4_expert_ffn_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(st: int, what: str):
    if st != MOE_OK:
        raise MoeError(st, f"{what}: {lib().moe_last_error().decode()}")


def ptr(t) -> int | None:
    """Device/host address of a torch tensor, numpy array, int or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def stream_handle(stream=None) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_version() -> str:
    return lib().moe_version().decode()


def moe_router_logits(x, w_router, T, H, E, logits, stream=None):
    _check(lib().moe_router_logits(ptr(x), ptr(w_router), T, H, E, ptr(logits), stream_handle(stream)),
           "moe_router_logits")


def moe_route(logits, T, E, k, renormalize, topk_ids, topk_w, stream=None):
    _check(lib().moe_route(ptr(logits), T, E, k, int(renormalize), ptr(topk_ids), ptr(topk_w), stream_handle(stream)),
           "moe_route")


def moe_permute(topk_ids, T, k, E, counts, offsets, perm, inv, stream=None):
    _check(lib().moe_permute(ptr(topk_ids), T, k, E, ptr(counts), ptr(offsets), ptr(perm), ptr(inv),
                             stream_handle(stream)), "moe_permute")


def moe_route_permute(logits, T, E, k, renormalize, topk_ids, topk_w, counts, offsets, perm, inv, stream=None):
    _check(lib().moe_route_permute(ptr(logits), T, E, k, int(renormalize), ptr(topk_ids), ptr(topk_w), ptr(counts),
                                   ptr(offsets), ptr(perm), ptr(inv), stream_handle(stream)), "moe_route_permute")


def moe_blob_bytes(fmt, H, I) -> int:
    return int(lib().moe_blob_bytes(FMT.get(fmt, fmt), H, I))


def moe_prepack_expert(fmt, H, I, gate, up, down) -> np.ndarray:
    """gate/up/down: (codes_or_bf16, scales_or_None, g) numpy arrays in canonical layout.

    Returns the blob as a host uint8 array."""
    f = FMT.get(fmt, fmt)
    keep = []

    def arr(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        keep.append(a)
        return a.ctypes.data

    c = ExpertCanonical(f, H, I,
                        arr(gate[0]), arr(gate[1]), float(gate[2]),
                        arr(up[0]), arr(up[1]), float(up[2]),
                        arr(down[0]), arr(down[1]), float(down[2]))
    n = moe_blob_bytes(f, H, I)
    out = np.empty(max(n, 1), np.uint8)
    _check(lib().moe_prepack_expert(ctypes.byref(c), out.ctypes.data, n), "moe_prepack_expert")
    return out


def ffn_args(**kw) -> FfnArgs:
    a = FfnArgs()
    for name, _ in FfnArgs._fields_:
        if name in kw:
            v = kw.pop(name)
            if name == "wfmt":
                v = FMT.get(v, v)
            elif name == "amode":
                v = AMODE.get(v, v)
            elif name in ("T", "k", "E", "H", "I", "slot_stride", "workspace_bytes"):
                v = int(v)
            else:
                v = ptr(v)
            setattr(a, name, v)
    if kw:
        raise TypeError(f"unknown moe_ffn_args fields: {sorted(kw)}")
    return a


def moe_expert_ffn_workspace_size(args: FfnArgs) -> int:
    return int(lib().moe_expert_ffn_workspace_size(ctypes.byref(args)))


def moe_expert_ffn(args: FfnArgs, stream=None):
    _check(lib().moe_expert_ffn(ctypes.byref(args), stream_handle(stream)), "moe_expert_ffn")


def moe_layer(args: LayerArgs, stream=None):
    """Routing, expert FFN and combine of one layer call (args.ffn.out required)."""
    _check(lib().moe_layer(ctypes.byref(args), stream_handle(stream)), "moe_layer")


def moe_layer_traced(args: LayerArgs, events, stream=None) -> int:
    arr = (ctypes.c_void_p * max(len(events), 1))(*[e.cuda_event for e in events])
    n = ctypes.c_int(0)
    _check(lib().moe_layer_traced(ctypes.byref(args), stream_handle(stream), arr, len(events), ctypes.byref(n)),
           "moe_layer_traced")
    return n.value


def moe_expert_ffn_noalloc(args: FfnArgs, stream=None):
    """moe_expert_ffn on the library's static device scratch (args.workspace is ignored)."""
    _check(lib().moe_expert_ffn_noalloc(ctypes.byref(args), stream_handle(stream)), "moe_expert_ffn_noalloc")


def moe_expert_ffn_traced(args: FfnArgs, events, stream=None) -> int:
    """moe_expert_ffn recording the given events (torch.cuda.Event, already
    created) around its kernel launches; returns how many were recorded."""
    arr = (ctypes.c_void_p * max(len(events), 1))(*[e.cuda_event for e in events])
    n = ctypes.c_int(0)
    _check(lib().moe_expert_ffn_traced(ctypes.byref(args), stream_handle(stream), arr, len(events), ctypes.byref(n)),
           "moe_expert_ffn_traced")
    return n.value


def moe_combine(y, inv, topk_w, y_shared, T, k, H, out, stream=None):
    _check(lib().moe_combine(ptr(y), ptr(inv), ptr(topk_w), ptr(y_shared), T, k, H, ptr(out), stream_handle(stream)),
           "moe_combine")


def moe_quantize_mxfp4(x, rows, cols, q, s, stream=None):
    _check(lib().moe_quantize_mxfp4(ptr(x), rows, cols, ptr(q), ptr(s), stream_handle(stream)), "moe_quantize_mxfp4")


def moe_debug_fp4_codes(args: FfnArgs, which, q, s, stream=None):
    _check(lib().moe_debug_fp4_codes(ctypes.byref(args), int(which), ptr(q), ptr(s), stream_handle(stream)),
           "moe_debug_fp4_codes")


def moe_dequant_blob(blob, which, out, stream=None):
    _check(lib().moe_dequant_blob(ptr(blob), which, ptr(out), stream_handle(stream)), "moe_dequant_blob")


class Cache:
    """Owner of a moe_cache handle (host LRU metadata + HIP events)."""

    def __init__(self, num_slots, slot_bytes, slot_pool, num_layers, num_experts):
        h = lib().moe_cache_create(num_slots, slot_bytes, ptr(slot_pool), num_layers, num_experts)
        if not h:
            raise MoeError(MOE_EINVAL, moe_last_error())
        self.handle = h
        self.num_slots = num_slots

    def close(self):
        if self.handle:
            lib().moe_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_cache_create(num_slots, slot_bytes, slot_pool, num_layers, num_experts) -> Cache:
    return Cache(num_slots, slot_bytes, slot_pool, num_layers, num_experts)


def moe_cache_destroy(cache: Cache):
    cache.close()


def cache_lookup(cache: Cache, layer: int, ids):
    """ids: distinct ascending expert ids.  Returns (slot, hit, evicted_key) numpy arrays."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n = ids.size
    slot = np.empty(n, np.int32)
    hit = np.empty(n, np.uint8)
    ev = np.empty(n, np.int32)
    _check(lib().cache_lookup(cache.handle, layer, ids.ctypes.data, n, slot.ctypes.data, hit.ctypes.data,
                              ev.ctypes.data), "cache_lookup")
    return slot, hit, ev


def cache_fill(cache: Cache, layer, expert, slot, host_src, copy_stream=None, compute_stream=None):
    _check(lib().cache_fill(cache.handle, layer, expert, slot, ptr(host_src), stream_handle(copy_stream),
                            stream_handle(compute_stream)), "cache_fill")


def moe_cache_mark_used(cache: Cache, slots, stream=None):
    s = np.ascontiguousarray(slots, dtype=np.int32)
    _check(lib().moe_cache_mark_used(cache.handle, s.ctypes.data, s.size, stream_handle(stream)),
           "moe_cache_mark_used")


def moe_cache_reset(cache: Cache):
    _check(lib().moe_cache_reset(cache.handle), "moe_cache_reset")


def moe_cache_use_copy_engine(cache: Cache, on: bool):
    _check(lib().moe_cache_use_copy_engine(cache.handle, 1 if on else 0), "moe_cache_use_copy_engine")


def moe_cache_pin_resident(cache: Cache, layer, s0):
    _check(lib().moe_cache_pin_resident(cache.handle, layer, s0), "moe_cache_pin_resident")


def moe_cache_stats(cache: Cache):
    """(hits, misses, bytes_filled) since creation or reset."""
    v = (ctypes.c_longlong * 3)()
    _check(lib().moe_cache_stats(cache.handle, ctypes.byref(v, 0), ctypes.byref(v, 8), ctypes.byref(v, 16)),
           "moe_cache_stats")
    return int(v[0]), int(v[1]), int(v[2])


def moe_cache_map_bytes(E: int) -> int:
    return int(lib().moe_cache_map_bytes(E))


def moe_cache_decode_step(cache: Cache, step: CacheStep, copy_stream=None, compute_stream=None):
    _check(lib().moe_cache_decode_step(cache.handle, ctypes.byref(step), stream_handle(copy_stream),
                                       stream_handle(compute_stream)), "moe_cache_decode_step")


def moe_cache_resize(cache: Cache, num_slots: int, slot_pool, stream=None):
    _check(lib().moe_cache_resize(cache.handle, int(num_slots), ptr(slot_pool), stream_handle(stream)),
           "moe_cache_resize")


def moe_cache_prefetch_layer(cache: Cache, layer, host_blobs, host_map, dev_map, trace=None, copy_stream=None,
                             compute_stream=None):
    """host_blobs: ctypes array of E pinned blob addresses; trace: None or
    (slot int32 [E], hit uint8 [E], evicted int32 [E]) numpy arrays."""
    t = (None, None, None) if trace is None else tuple(a.ctypes.data for a in trace)
    _check(lib().moe_cache_prefetch_layer(cache.handle, int(layer), ctypes.cast(host_blobs, ctypes.c_void_p),
                                          ptr(host_map), ptr(dev_map), *t, stream_handle(copy_stream),
                                          stream_handle(compute_stream)), "moe_cache_prefetch_layer")


def moe_cache_prefill_step(cache: Cache, step: CachePrefill, compute_stream=None):
    _check(lib().moe_cache_prefill_step(cache.handle, ctypes.byref(step), stream_handle(compute_stream)),
           "moe_cache_prefill_step")


def moe_cpu_expert_ffn(blob, x, n, y, threads=1):
    """blob, x (bf16 bits [n,H]), y (fp32 [n,H]): host arrays."""
    _check(lib().moe_cpu_expert_ffn(ptr(blob), ptr(x), int(n), ptr(y), int(threads)), "moe_cpu_expert_ffn")


def moe_calibrate_bw(host_blob, dev_buf, reps=8, threads=1, copy_stream=None) -> BwCalib:
    out = BwCalib()
    _check(lib().moe_calibrate_bw(ptr(host_blob), ptr(dev_buf), int(reps), int(threads), stream_handle(copy_stream),
                                  ctypes.byref(out)), "moe_calibrate_bw")
    return out


def moe_cache_decode_step_hybrid(cache: Cache, step: CacheStep, hybrid: Hybrid, copy_stream=None, compute_stream=None):
    _check(lib().moe_cache_decode_step_hybrid(cache.handle, ctypes.byref(step), ctypes.byref(hybrid),
                                              stream_handle(copy_stream), stream_handle(compute_stream)),
           "moe_cache_decode_step_hybrid")
