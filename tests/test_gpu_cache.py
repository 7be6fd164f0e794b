"""The expert-slot cache on the GPU through the C ABI: slot fills from pinned
host memory, and decode streams over several layers whose experts live in a
pinned host bank behind an LRU cache with few slots (many misses and
evictions).  The hit / miss / slot / eviction trace of every step must equal
the oracle's LRU simulation exactly; each step's output must match the oracle
layer within max |gpu - oracle| / max |oracle| <= 1e-2."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import DEV, DequantCache, need_gpu, say, torch

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    import fp4_expert_ffn_amd  # noqa: F401


def _pinned_blob(ex, stride):
    from fp4_expert_ffn_amd.layer import blob_of
    b = blob_of(ex)
    t = torch.zeros(stride, dtype=torch.uint8, pin_memory=True)
    t[:b.size].copy_(torch.from_numpy(b))
    return t


def test_cache_fill_copies_the_blob_into_its_slot():
    import fp4_expert_ffn_amd as F
    ex = synth.expert("nvfp4", 256, 128, config=85, expert_id=3)
    stride = (F.moe_blob_bytes("nvfp4", 256, 128) + 255) // 256 * 256
    pool = torch.zeros(4 * stride, dtype=torch.uint8, device=DEV)
    c = F.moe_cache_create(4, stride, pool, 1, 8)
    src = _pinned_blob(ex, stride)
    for e in (3, 5):
        slot, hit, ev = F.cache_lookup(c, 0, [e])
        say(f"cache_fill expert {e} -> slot {slot[0]}")
        copy = torch.cuda.Stream()
        F.cache_fill(c, 0, e, int(slot[0]), src, copy, torch.cuda.current_stream())
        F.moe_cache_mark_used(c, slot)
        torch.cuda.synchronize()
        got = pool[int(slot[0]) * stride:(int(slot[0]) + 1) * stride].cpu()
        assert torch.equal(got, src)
    assert F.moe_cache_stats(c) == (0, 2, 2 * stride)
    c.close()


def test_calibration_copies_the_blob():
    """moe_calibrate_bw times the decode steps' miss copy (the fill kernel on
    a pinned blob) and the host expert FFN: the device buffer then holds the
    blob byte for byte, and the figures are positive with a copy share in
    (0, 1)."""
    import fp4_expert_ffn_amd as F
    ex = synth.expert("nvfp4", 256, 128, config=85, expert_id=1)
    nbytes = F.moe_blob_bytes("nvfp4", 256, 128)
    stride = (nbytes + 255) // 256 * 256
    src = _pinned_blob(ex, stride)
    dst = torch.zeros(stride, dtype=torch.uint8, device=DEV)
    say("moe_calibrate_bw on one NVFP4 blob (hidden 256, inter 128)")
    cal = F.moe_calibrate_bw(src, dst, reps=3, threads=2)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes].cpu(), src[:nbytes])
    assert cal.copy_us > 0 and cal.cpu_us > 0 and cal.h2d_gbs > 0 and 0 < cal.copy_ratio < 1


def _run_stream(*, layers, E, k, H, I, tokens, slots, make_expert, check_steps=None, config=86, resize_at=None,
                routing_seed=None, blob_key=None, copy_ratio=None, copy_engine=False, raw=False):
    """Decode `tokens` single-token steps through `layers` layers; returns the
    number of steps checked against the oracle.  blob_key(l, e) names the
    pinned blob of an expert (experts with equal keys share one host copy;
    make_expert must give them equal weights).  raw: steps through
    CachedDecoder.step_raw (inputs by device address) instead of step."""
    from fp4_expert_ffn_amd.layer import CachedDecoder, to_numpy_bf16
    import fp4_expert_ffn_amd as F
    stride = (F.moe_blob_bytes("nvfp4", H, I) + 255) // 256 * 256
    bank = {}
    blob_key = blob_key or (lambda l, e: (l, e))

    def host_blob(l, e):
        key = blob_key(l, e)
        if key not in bank:
            bank[key] = _pinned_blob(make_expert(l, e), stride)
        return bank[key]

    dec = CachedDecoder(num_layers=layers, num_experts=E, k=k, H=H, I=I, fmt="nvfp4", num_slots=slots,
                        host_blob=host_blob, device=DEV, copy_ratio=copy_ratio, host_threads=4,
                        copy_engine=copy_engine)
    seed = config if routing_seed is None else routing_seed
    logits = synth.stream_routing(tokens, layers, E, seed=seed)
    xs = np.stack([np.stack([synth.stream_activations(t, l, H, seed=seed)[0] for l in range(layers)])
                   for t in range(tokens)])
    lg_d = torch.from_numpy(logits).to(DEV)
    x_d = torch.from_numpy(xs.view(np.int16)).to(DEV)
    lru = oracle.lru.SlotLRU(slots)
    wts = {l: DequantCache(lambda e, l=l: make_expert(l, e), cap=E) for l in range(layers)}
    checked = 0
    misses = 0
    for t in range(tokens):
        if resize_at and t in resize_at:
            say(f"    resize to {resize_at[t]} slots before token {t}")
            dec.resize(resize_at[t])
            lru.resize(resize_at[t])
        for l in range(layers):
            if raw:
                i = t * layers + l
                n = dec.step_raw(l, x_d.data_ptr() + 2 * H * i, lg_d.data_ptr() + 4 * E * i,
                                 torch.cuda.current_stream().cuda_stream)
                out = dec.out[:1]
                te, ts, th, tv = (a[:n].copy() for a in dec.trace)
            else:
                out, (te, ts, th, tv) = dec.step(l, x_d[t, l:l + 1], lg_d[t, l:l + 1])
            ids, w = oracle.moe.route(logits[t, l:l + 1], k)
            want = _policy_lookup(lru, l, sorted(set(ids[0].tolist())), copy_ratio)
            assert te.tolist() == [r[0] for r in want], (t, l)
            assert th.tolist() == [int(r[1]) for r in want], (t, l)
            assert ts.tolist() == [r[2] for r in want], (t, l)
            assert tv.tolist() == [-1 if r[3] is None else r[3][0] * E + r[3][1] for r in want], (t, l)
            misses += int(np.sum((th == 0) & (ts >= 0)))
            if check_steps is None or (t, l) in check_steps:
                torch.cuda.synchronize()
                got = synth.bf16_bits_to_f32(to_numpy_bf16(out))
                ref = oracle.moe.token_output(0, xs[t, l:l + 1], ids[0], w[0], wts[l])
                err = oracle.moe.relative_error(got[0], ref)
                assert err <= TOL, (t, l, err)
                checked += 1
    torch.cuda.synchronize()
    hits, m, nbytes = dec.stats()
    assert m == misses and nbytes == misses * stride
    # the cached blobs are byte-equal to their host copies (up to 32 of them)
    cached = [(l, e) for l in range(layers) for e in range(E) if (l, e) in lru][:32]
    for l, e in cached:
        sl = lru.slot_of((l, e))
        assert torch.equal(dec.pool[sl * stride:(sl + 1) * stride].cpu(), host_blob(l, e)), (l, e, sl)
    say(f"    {tokens} tokens x {layers} layers: {hits} hits, {m} misses, {checked} outputs checked")
    dec.close()
    return checked


def _policy_lookup(lru, layer, ids, copy_ratio):
    """The oracle LRU's records of one step under the hybrid miss policy: of
    the step's m misses, the first floor(r m + 1/2) in ascending id (r and
    the product in float32, as the library takes them) are looked up (and
    cached); the others run on the host: (expert, False, -1, None), cache
    unchanged.  copy_ratio None: every expert looked up."""
    if copy_ratio is None:
        return lru.lookup(layer, ids)
    misses = [e for e in ids if (layer, e) not in lru]
    ncopy = int(np.float32(copy_ratio) * np.float32(len(misses)) + np.float32(0.5))
    host = set(misses[ncopy:])
    recs = {r[0]: r for r in lru.lookup(layer, [e for e in ids if e not in host])}
    return [recs[e] if e in recs else (e, False, -1, None) for e in ids]


@pytest.mark.parametrize("copy_engine", [False, True])
def test_cached_stream_small_every_step(copy_engine):
    """16 experts per layer, top-4, 10 slots for 3 layers: most steps miss and
    evict.  Misses copied by the fill kernel (hits on the side stream) or by
    the copy engine."""
    say(f"cached stream: 3 layers x 16 NVFP4 experts (hidden 256, inter 256), 10 slots, 20 tokens, "
        f"copy engine {copy_engine}")

    def make(l, e):
        return synth.expert("nvfp4", 256, 256, config=86, layer=l, expert_id=e)

    _run_stream(layers=3, E=16, k=4, H=256, I=256, tokens=20, slots=10, make_expert=make, copy_engine=copy_engine)


@pytest.mark.parametrize("copy_ratio", [0.5, 0.0])
def test_cached_stream_hybrid_policy(copy_ratio):
    """The hybrid miss policy: a share of each step's misses copied into the
    cache, the rest run on the host (copy_ratio 0: the cpu backend, every
    miss on the host and nothing cached after the first lookups).  Every
    step's trace equals the oracle LRU under the same split and every output
    matches the oracle layer."""
    say(f"cached stream, hybrid policy (copy ratio {copy_ratio}): 3 layers x 16 NVFP4 experts, 10 slots, 20 tokens")

    def make(l, e):
        return synth.expert("nvfp4", 256, 256, config=92, layer=l, expert_id=e)

    _run_stream(layers=3, E=16, k=4, H=256, I=256, tokens=20, slots=10, make_expert=make, config=92,
                copy_ratio=copy_ratio, raw=True)


@pytest.mark.parametrize("T,copy_engine", [(4, False), (4, True), (80, False)])
def test_cached_stream_batched_steps(T, copy_engine):
    """Decode steps of several tokens through the cache (3 layers x 16 NVFP4
    experts, top-4, 16 slots): up to 16 distinct experts a step, so a step
    has many misses in one fill list and hits on the side stream at once;
    steps of 80 tokens publish their counts through the separate handoff
    kernel (the routing kernel folds it in up to 64 tokens).  Every step's
    trace equals the oracle LRU's and every token's output matches the
    oracle layer."""
    from fp4_expert_ffn_amd.layer import CachedDecoder, to_numpy_bf16
    import fp4_expert_ffn_amd as F
    L_, E, k, H, I, slots, steps = 3, 16, 4, 256, 256, 16, 12
    say(f"cached stream, {T}-token steps: {L_} layers x {E} NVFP4 experts, {slots} slots, {steps} steps, "
        f"copy engine {copy_engine}")

    def make(l, e):
        return synth.expert("nvfp4", H, I, config=93, layer=l, expert_id=e)

    stride = (F.moe_blob_bytes("nvfp4", H, I) + 255) // 256 * 256
    bank = {(l, e): _pinned_blob(make(l, e), stride) for l in range(L_) for e in range(E)}
    dec = CachedDecoder(num_layers=L_, num_experts=E, k=k, H=H, I=I, fmt="nvfp4", num_slots=slots,
                        host_blob=lambda l, e: bank[(l, e)], max_tokens=T, device=DEV, copy_engine=copy_engine)
    rng = np.random.default_rng(93)
    lru = oracle.lru.SlotLRU(slots)
    wts = {l: DequantCache(lambda e, l=l: make(l, e), cap=E) for l in range(L_)}
    for step in range(steps):
        l = step % L_
        logits = rng.standard_normal((T, E)).astype(np.float32)
        xb = synth.activations(T, H, 93, 1, step)
        out, (te, ts, th, tv) = dec.step(l, torch.from_numpy(xb.view(np.int16)).to(DEV),
                                         torch.from_numpy(logits).to(DEV))
        ids, w = oracle.moe.route(logits, k)
        want = lru.lookup(l, sorted(set(ids.ravel().tolist())))
        assert te.tolist() == [r[0] for r in want], step
        assert th.tolist() == [int(r[1]) for r in want], step
        assert ts.tolist() == [r[2] for r in want], step
        assert tv.tolist() == [-1 if r[3] is None else r[3][0] * E + r[3][1] for r in want], step
        torch.cuda.synchronize()
        got = synth.bf16_bits_to_f32(to_numpy_bf16(out))
        for t in range(T):
            ref = oracle.moe.token_output(t, xb, ids[t], w[t], wts[l])
            err = oracle.moe.relative_error(got[t], ref)
            assert err <= TOL, (step, t, err)
    dec.close()


def test_cached_stream_with_resizes():
    """The 16-expert stream with the cache shrunk from 10 to 5 slots, then grown
    to 14, between steps: the traces after each resize (which keys stayed, in
    which slots) equal the oracle LRU's, and every output matches the oracle."""
    say("cached stream with resizes: 3 layers x 16 NVFP4 experts, 10 -> 5 -> 14 slots, 24 tokens")

    def make(l, e):
        return synth.expert("nvfp4", 256, 256, config=90, layer=l, expert_id=e)

    _run_stream(layers=3, E=16, k=4, H=256, I=256, tokens=24, slots=10, make_expert=make, config=90,
                resize_at={8: 5, 16: 14})


def test_cached_stream_a3b_shape():
    """A3B-like layers (hidden 2048, 128 NVFP4 experts, top-8, inter 768), 2 layers,
    24 slots: the trace of every step, the output of sampled steps."""
    say("cached stream: 2 A3B-like layers, 24 slots, 12 tokens")
    gen = {}

    def make(l, e):
        if (l, e) not in gen:
            gen[(l, e)] = synth.expert("nvfp4", 2048, 768, config=87, layer=l, expert_id=e)
        return gen[(l, e)]

    rng = np.random.default_rng(0)
    steps = {(int(t), int(l)) for t, l in zip(rng.integers(0, 12, 6), rng.integers(0, 2, 6))} | {(11, 1)}
    n = _run_stream(layers=2, E=128, k=8, H=2048, I=768, tokens=12, slots=24, make_expert=make,
                    check_steps=steps, config=87, raw=True)
    assert n == len(steps)


@pytest.mark.slow
def test_cached_stream_full_size_trace():
    """The cached decode stream at its real size: 48 A3B-like NVFP4 layers
    (128 experts, top-8), 2048 HBM slots shared by all layers under LRU, 512
    single-token steps from a cold cache with the stream's own routing
    (Zipf(1.1), 0.6 repeat of the previous token's experts).  Every one of
    the 24,576 steps' hit / miss / slot / eviction records equals the oracle
    LRU's; sampled outputs match the oracle layer.  The LRU trace depends on
    the routing only, so the layers share expert weights in pairs (one pinned
    copy per (layer % 2, expert)) to keep the host bank small."""
    say("cached stream at full size: 48 layers x 128 NVFP4 experts, 2048 slots, 512 tokens (trace of every step)")
    gen = {}

    def make(l, e):
        key = (l % 2, e)
        if key not in gen:
            gen[key] = synth.expert("nvfp4", 2048, 768, config=4, layer=key[0], expert_id=e)
        return gen[key]

    steps = {(0, 0), (1, 47), (63, 5), (200, 30), (511, 47), (511, 0), (300, 17), (64, 1)}
    n = _run_stream(layers=48, E=128, k=8, H=2048, I=768, tokens=512, slots=2048, make_expert=make,
                    check_steps=steps, config=4, routing_seed=0, blob_key=lambda l, e: (l % 2, e))
    assert n == len(steps)


# Prefill through the cache one layer ahead (every expert of layer l + 1
# copied while layer l computes).


def _trace_of(want, E):
    return ([r[0] for r in want], [int(r[1]) for r in want], [r[2] for r in want],
            [-1 if r[3] is None else r[3][0] * E + r[3][1] for r in want])


@pytest.mark.parametrize("fmt,amode,T,E,k,H,I", [
    ("mxfp4", "mxfp4", 300, 8, 2, 256, 128),
    ("nvfp4", "bf16", 77, 16, 4, 256, 256),
])
def test_cached_prefill_layer_ahead(fmt, amode, T, E, k, H, I):
    """Two prefill passes over 3 layers through a 2E-slot cache, each layer's
    experts copied while the previous layer computes: the lookups equal the
    oracle's LRU (the prefetch of layer l + 1 evicts layer l - 1, never l),
    every step hits, and each layer's output matches the oracle layer."""
    from fp4_expert_ffn_amd.layer import CachedPrefill, to_numpy_bf16
    import fp4_expert_ffn_amd as F
    layers, config = 3, 88
    say(f"cached prefill {fmt}/{amode}: {layers} layers x {E} experts, T={T} k={k} H={H} I={I}, {2 * E} slots")
    stride = (F.moe_blob_bytes(fmt, H, I) + 255) // 256 * 256
    experts = {(l, e): synth.expert(fmt, H, I, config=config, layer=l, expert_id=e)
               for l in range(layers) for e in range(E)}
    pf = CachedPrefill(num_layers=layers, num_experts=E, k=k, H=H, I=I, fmt=fmt, amode=amode, max_tokens=T,
                       host_blob=lambda l, e: _pinned_blob(experts[(l, e)], stride), device=DEV)
    lru = oracle.lru.SlotLRU(2 * E)
    want_misses = 0
    for rnd in range(2):
        xs = [synth.activations(T, H, config, rnd, l) for l in range(layers)]
        lg = [synth.rng(config, rnd, l, 1).standard_normal((T, E), dtype=np.float32) for l in range(layers)]
        x_d = [torch.from_numpy(x.view(np.int16)).to(DEV) for x in xs]
        lg_d = [torch.from_numpy(a).to(DEV) for a in lg]
        outs = [torch.empty((T, H), dtype=torch.int16, device=DEV) for _ in range(layers)]
        traces = pf.run(x_d, lg_d, outs)
        torch.cuda.synchronize()
        for l in range(layers):
            want_misses += sum(not r[1] for r in lru.lookup(l, range(E)))   # the prefetch
            want = lru.lookup(l, range(E))          # the step: all hits
            assert all(r[1] for r in want)
            got = tuple(t.tolist() for t in traces[l])
            assert got == _trace_of(want, E), (rnd, l)
            ref = oracle.moe.layer(xs[l], [experts[(l, e)] for e in range(E)], k, logits=lg[l], amode=amode)
            if l == layers - 1:                      # the ids buffer holds the last layer's routing
                assert np.array_equal(pf.ids[:T].cpu().numpy(), ref["ids"])
            err = oracle.moe.relative_error(synth.bf16_bits_to_f32(to_numpy_bf16(outs[l])), ref["out"])
            say(f"    pass {rnd} layer {l}: rel err {err:.3e}")
            assert err <= TOL, (rnd, l, err)
    hits, misses, nbytes = pf.stats()
    # 3 layers through 2 layers' slots: every prefetch misses
    assert misses == want_misses == 6 * E and nbytes == misses * stride, (hits, misses)
    pf.close()


def test_cached_prefill_step_needs_the_prefetch():
    """A step whose layer was not prefetched fails with MOE_ECACHE and leaves the cache unchanged."""
    from fp4_expert_ffn_amd.layer import CachedPrefill
    import fp4_expert_ffn_amd as F
    H, I, E, k, T = 256, 128, 8, 2, 16
    stride = (F.moe_blob_bytes("mxfp4", H, I) + 255) // 256 * 256
    ex = synth.expert("mxfp4", H, I, config=89)
    blob = _pinned_blob(ex, stride)
    pf = CachedPrefill(num_layers=2, num_experts=E, k=k, H=H, I=I, fmt="mxfp4", max_tokens=T,
                       host_blob=lambda l, e: blob, device=DEV)
    x = torch.zeros((T, H), dtype=torch.int16, device=DEV)
    lg = torch.zeros((T, E), dtype=torch.float32, device=DEV)
    out = torch.empty((T, H), dtype=torch.int16, device=DEV)
    pf.prefetch(0)
    with pytest.raises(F.MoeError, match="not cached"):
        pf.layer_step(1, x, lg, out)
    torch.cuda.synchronize()
    assert pf.stats() == (0, E, E * stride)
    pf.close()
