"""CPU tests of libmoe: it loads, exports every declared symbol, and its
host-only parts (blob layout, prepack, LRU cache bookkeeping, argument
checks) behave as documented.  No GPU calls."""
import os
import re

import numpy as np
import pytest

import synth
from oracle.lru import SlotLRU
from tests.conftest import ROOT

lib_mod = pytest.importorskip("fp4_expert_ffn_amd._lib")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lib_mod.LIB_PATH):
        from fp4_expert_ffn_amd import build
        build.build()
    return lib_mod


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)
    return sorted({n for n in names if n.startswith(("moe_", "cache_")) and n not in ("moe_stream_t",)})


def test_exports_every_declared_symbol(L):
    lib = L.lib()
    declared = _declared_functions()
    assert len(declared) >= 19
    for n in declared:
        assert hasattr(lib, n), n
    assert set(declared) == set(L.SIGNATURES), set(declared) ^ set(L.SIGNATURES)


def test_blob_bytes(L):
    # 4.5 bits/param (NVFP4), 4.25 (MXFP4), 16 (BF16) plus header and 256 B section padding
    for fmt, bits in (("nvfp4", 4.5), ("mxfp4", 4.25), ("bf16", 16), ("fp8", 8)):
        n = L.moe_blob_bytes(fmt, 2048, 768)
        assert abs(n - (256 + 3 * 2048 * 768 * bits / 8)) < 4 * 256
    assert L.moe_blob_bytes("mxfp4", 100, 128) == 0 and L.moe_blob_bytes(7, 128, 128) == 0


def _tile_codes(q, rows, cols, fmt):
    """Independent numpy statement of the documented tile order: [row-group][K-tile][lane][16 B]."""
    kt = {"bf16": 32, "fp8": 64}.get(fmt, 128)
    raw = q.view(np.uint8).reshape(rows, -1)
    bpr = raw.shape[1]
    out = []
    for rg in range(rows // 16):
        for k in range(cols // kt):
            for lane in range(64):
                r, kb = rg * 16 + lane % 16, lane // 16
                if fmt == "bf16":
                    b0 = (k * kt + kb * 8) * 2
                elif fmt == "fp8":
                    b0 = k * kt + kb * 16
                else:
                    b0 = (k * kt + kb * 32) // 2
                out.append(raw[r, b0:b0 + 16])
    return np.concatenate(out), bpr


@pytest.mark.parametrize("fmt", synth.FMTS)
def test_prepack_layout(L, fmt):
    H, I = 256, 128
    ex = synth.expert(fmt, H, I, config=60, expert_id=1)
    from fp4_expert_ffn_amd.layer import blob_of
    blob = blob_of(ex)
    assert blob.size == L.moe_blob_bytes(fmt, H, I)
    hdr = blob[:256]
    assert hdr[:4].tobytes() == b"MOEB"
    fmt_id, h, i = np.frombuffer(hdr[8:20].tobytes(), np.int32)
    assert (fmt_id, h, i) == (L.FMT[fmt], H, I)
    g = np.frombuffer(hdr[20:32].tobytes(), np.float32)
    off = np.frombuffer(hdr[32:72].tobytes(), np.uint64)
    if fmt in ("nvfp4", "fp8"):
        assert list(g) == [np.float32(ex.gate.g), np.float32(ex.up.g), np.float32(ex.down.g)]
    else:
        assert list(g) == [1.0, 1.0, 1.0]
    # W13 = interleaved 16-row groups of gate and up
    src = lambda p: p.w if fmt == "bf16" else p.q
    gate, _ = _tile_codes(src(ex.gate), I, H, fmt)
    up, _ = _tile_codes(src(ex.up), I, H, fmt)
    kt = {"bf16": 32, "fp8": 64}.get(fmt, 128)
    per_group = (H // kt) * 1024
    inter = np.concatenate([np.concatenate([gate[p * per_group:(p + 1) * per_group], up[p * per_group:(p + 1) * per_group]])
                            for p in range(I // 16)])
    assert np.array_equal(blob[off[0]:off[0] + inter.size], inter)
    down, _ = _tile_codes(src(ex.down), H, I, fmt)
    assert np.array_equal(blob[off[2]:off[2] + down.size], down)
    if fmt == "mxfp4":
        s = ex.down.s
        want = np.array([s[rg * 16 + l % 16, k * 4 + l // 16] for rg in range(H // 16) for k in range(I // 128)
                         for l in range(64)], np.uint8)
        assert np.array_equal(blob[off[3]:off[3] + want.size], want)
    if fmt == "nvfp4":
        s = ex.gate.s
        want = []
        for p in range(I // 16):
            for k in range(H // 128):
                for l in range(64):
                    r = p * 16 + l % 16
                    want += [s[r, k * 8 + (l // 16) * 2], s[r, k * 8 + (l // 16) * 2 + 1]]
        # the scale section interleaves gate and up groups like the codes; check the gate groups
        gate_tiles = np.array(want, np.uint8).reshape(I // 16, -1)
        blob_s = blob[off[1]:off[1] + 2 * gate_tiles.size].reshape(I // 16, 2, -1)[:, 0, :]
        assert np.array_equal(blob_s, gate_tiles)


def test_prepack_rejects_bad_shapes(L):
    ex = synth.expert("mxfp4", 256, 128, config=60, expert_id=2)
    with pytest.raises(L.MoeError) as e:
        L.moe_prepack_expert("mxfp4", 200, 128, (ex.gate.q, ex.gate.s, 1), (ex.up.q, ex.up.s, 1),
                             (ex.down.q, ex.down.s, 1))
    assert e.value.status == L.MOE_EINVAL and "multiples of 128" in str(e.value)


def test_cache_trace_matches_oracle_lru(L):
    rng = np.random.default_rng(11)
    layers, E, C = 4, 32, 24
    p = np.arange(1, E + 1, dtype=float) ** -1.1
    p /= p.sum()
    c = L.moe_cache_create(C, 1 << 20, 0, layers, E)
    ref = SlotLRU(C)
    for step in range(300):
        for layer in range(layers):
            ids = np.unique(rng.choice(E, 8, replace=False, p=p)).astype(np.int32)
            slot, hit, ev = L.cache_lookup(c, layer, ids)
            want = ref.lookup(layer, ids.tolist())
            for i, (e, h, s, v) in enumerate(want):
                assert (hit[i] == int(h)) and slot[i] == s, (step, layer, e)
                assert ev[i] == (-1 if v is None else v[0] * E + v[1])
    c.close()


def test_cache_errors_leave_state_unchanged(L):
    c = L.moe_cache_create(3, 4096, 0, 2, 8)
    L.cache_lookup(c, 0, [1, 2])
    for bad, status in (([3, 2], L.MOE_EINVAL), ([1, 1], L.MOE_EINVAL), ([9], L.MOE_EINVAL),
                        ([0, 3, 4, 5], L.MOE_ECACHE)):
        with pytest.raises(L.MoeError) as e:
            L.cache_lookup(c, 0, bad)
        assert e.value.status == status
    with pytest.raises(L.MoeError):
        L.cache_lookup(c, 2, [0])
    slot, hit, ev = L.cache_lookup(c, 0, [1, 2])
    assert hit.tolist() == [1, 1] and slot.tolist() == [0, 1]
    # pin_resident refuses slots already in use
    with pytest.raises(L.MoeError):
        L.moe_cache_pin_resident(c, 1, 0)
    L.moe_cache_reset(c)
    slot, hit, ev = L.cache_lookup(c, 0, [1])
    assert hit.tolist() == [0] and slot.tolist() == [0]
    c.close()


def test_cache_create_rejects_bad_sizes(L):
    with pytest.raises(L.MoeError):
        L.moe_cache_create(0, 4096, 0, 1, 8)


def test_pin_resident(L):
    c = L.moe_cache_create(16, 4096, 0, 2, 8)
    L.moe_cache_pin_resident(c, 1, 8)
    slot, hit, ev = L.cache_lookup(c, 1, np.arange(8))
    assert hit.all() and slot.tolist() == list(range(8, 16))
    slot, hit, ev = L.cache_lookup(c, 0, [3])
    assert not hit[0] and slot[0] == 0
    c.close()


def test_matrix_core_operands_must_fit_32_bit_offsets(L):
    """The matrix-core kernels address x and the SwiGLU output with 32-bit
    byte offsets: a call whose rows of max(H, I) bf16 values reach 4 GiB is
    rejected before any device call (fake addresses)."""
    H, I = 28672, 128
    stride = (L.moe_blob_bytes("mxfp4", H, I) + 255) // 256 * 256
    a = L.ffn_args(T=16384, k=8, E=8, H=H, I=I, wfmt="mxfp4", amode="mxfp4", x=0x10000, counts=0x20000,
                   offsets=0x30000, perm=0x40000, slot_of_expert=0x50000, slot_pool=0x100000, slot_stride=stride,
                   topk_w=0x60000, inv=0x70000, out=0x80000, workspace=0x1000000, workspace_bytes=1 << 40)
    with pytest.raises(L.MoeError, match="exceed 4 GiB"):
        L.moe_expert_ffn(a, 0)


def test_cache_resize_rejects_bad_arguments(L):
    """Argument errors return before any device call (fake pool addresses) and leave the cache unchanged."""
    c = L.moe_cache_create(4, 1024, 0x100000, 2, 8)
    for n, pool in [(0, 0x200000), (4, 0), (4, 0x200010), (4, 0x100400), (8, 0x0FF000)]:
        with pytest.raises(L.MoeError):
            L.moe_cache_resize(c, n, pool, 0)
    slot, hit, ev = L.cache_lookup(c, 0, [1, 2, 3, 4])
    assert list(slot) == [0, 1, 2, 3] and not any(hit)
    c.close()


def test_noalloc_refuses_calls_beyond_its_scratch(L):
    """moe_expert_ffn_noalloc checks the call's workspace need against its
    32 MiB static scratch before any device call (fake addresses): a
    4096-token FP4 prefill needs far more and gets MOE_ENOMEM."""
    H, I = 2048, 768
    stride = (L.moe_blob_bytes("mxfp4", H, I) + 255) // 256 * 256
    a = L.ffn_args(T=4096, k=8, E=128, H=H, I=I, wfmt="mxfp4", amode="mxfp4", x=0x10000, counts=0x20000,
                   offsets=0x30000, perm=0x40000, slot_of_expert=0x50000, slot_pool=0x100000, slot_stride=stride,
                   topk_w=0x60000, inv=0x70000, out=0x80000)
    assert L.moe_expert_ffn_workspace_size(a) > 32 << 20
    with pytest.raises(L.MoeError, match="static scratch") as e:
        L.moe_expert_ffn_noalloc(a, 0)
    assert e.value.status == L.MOE_ENOMEM


@pytest.mark.parametrize("fmt", synth.FMTS)
@pytest.mark.parametrize("n", [1, 5])
def test_cpu_expert_ffn_matches_the_oracle(L, fmt, n):
    """The host expert FFN of the hybrid miss policy, on the prepacked blob,
    against the oracle's float64 SwiGLU expert on the same rows: fp32
    accumulation over K = 512 keeps max |cpu - oracle| / max |oracle| under
    1e-5, for every weight format and with several threads."""
    import oracle
    from fp4_expert_ffn_amd.layer import blob_of
    H, I = 512, 256
    ex = synth.expert(fmt, H, I, config=61, expert_id=2)
    x = synth.activations(n, H, 61, n)
    y = np.empty((n, H), np.float32)
    L.moe_cpu_expert_ffn(blob_of(ex), x, n, y, threads=3)
    ref = oracle.moe.expert_forward(ex, x)
    assert oracle.moe.relative_error(y, ref) <= 1e-5
