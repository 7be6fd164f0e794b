"""Host-only tests of the expert cache's stream and event protocol.

cache.cpp and host.cpp are built with g++ and the address and
undefined-behaviour sanitizers against a recording stand-in of the HIP
runtime calls they make and of the library calls they enqueue
(tests/cpu/hip_stub.cpp: no GPU, no HIP library).  The stand-in executes
every copy at once and keeps a happens-before relation over streams, events
and host synchronisations, and checks every cache-slot write (fill, resize
move) and read (an FFN call's blobs) against it: a fill after the slot's last
readers, a read after the slot's last fill, each slot holding the blob of the
expert its reader wants, no copy outside registered memory, a pinned map
re-sent only after the host saw its last copy finish.

Scenarios (tests/cpu/cache_harness.cpp): decode streams with many evictions
and with resizes, the layer-ahead prefill passes, and failures injected into
the n-th copy, event creation, event record or stream wait.  The lookups
every scenario prints are compared with the oracle LRU (oracle.lru.SlotLRU)."""
import os
import subprocess

import pytest

from oracle.lru import SlotLRU
from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "fp4_expert_ffn_amd", "csrc")
CPU = os.path.join(ROOT, "tests", "cpu")
MOE_OK, MOE_EHIP, MOE_ECACHE = 0, 3, 5


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("cache") / "cache_harness")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined",
           os.path.join(CSRC, "cache.cpp"), os.path.join(CSRC, "host.cpp"), os.path.join(CSRC, "cpu_expert.cpp"),
           os.path.join(CPU, "hip_stub.cpp"), os.path.join(CPU, "cache_harness.cpp"), "-o", exe, "-pthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(f"build failed:\n{r.stderr}")
    return exe


def run(exe, *args, copy_engine=False):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1",
               HARNESS_COPY_ENGINE="1" if copy_engine else "0")
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = r.stdout.split("\n")
    end = [ln for ln in lines if ln.startswith("END")]
    assert end == ["END hazards 0 bad 0"], (end, r.stderr[-3000:])
    return [ln.split() for ln in lines if ln and not ln.startswith("END")]


def _ev(v, E):
    return -1 if v is None else v[0] * E + v[1]


@pytest.mark.parametrize("L,E,k,T,C,steps,seed,resizes", [
    (3, 16, 4, 1, 10, 300, 1, []),         # most steps miss and evict
    (4, 32, 8, 3, 40, 400, 2, []),
    (2, 128, 8, 16, 80, 200, 3, []),       # 16-token steps, up to ~60 experts a step
    (3, 16, 4, 2, 10, 300, 4, ["100:8", "200:14"]),  # shrink, then grow
])
@pytest.mark.parametrize("copy_engine", [False, True])
def test_decode_stream_protocol_and_trace(harness, L, E, k, T, C, steps, seed, resizes, copy_engine):
    """Decode streams, misses filled by the fill kernel on the compute stream
    (hits on the side stream) or by the copy engine: the lookups equal the
    oracle LRU's and the stand-in sees no ordering hazard."""
    out = run(harness, "decode", L, E, k, T, C, steps, seed, *resizes, copy_engine=copy_engine)
    lru = SlotLRU(C)
    n = 0
    for ln in out:
        if ln[0] == "R":
            assert int(ln[2]) == MOE_OK
            lru.resize(int(ln[1]))
            continue
        assert ln[0] == "D" and int(ln[2]) == MOE_OK, ln
        layer = int(ln[1])
        recs = [tuple(map(int, r.split(":"))) for r in ln[3:]]
        want = lru.lookup(layer, [r[0] for r in recs])
        assert [(r[1], r[2], r[3]) for r in recs] == [(int(h), s, _ev(v, E)) for _, h, s, v in want], (n, layer)
        n += 1
    assert n == steps


@pytest.mark.parametrize("L,E,passes,seed", [(3, 8, 2, 1), (5, 16, 3, 2)])
def test_layer_ahead_prefill_protocol_and_trace(harness, L, E, passes, seed):
    """Each layer's experts are prefetched while the previous layer's step is
    in flight, into 2E slots: every prefetch and step lookup equals the
    oracle LRU's (the prefetch of layer l + 1 evicts layer l - 1, never l),
    every step hits, and a step of an evicted layer fails with MOE_ECACHE
    leaving the statistics unchanged."""
    out = run(harness, "prefill", L, E, 2 * E, passes, seed)
    lru = SlotLRU(2 * E)
    for ln in out:
        if ln[0] == "U":
            assert int(ln[2]) == MOE_ECACHE and ln[3] == "1"
            assert not any((int(ln[1]), e) in lru for e in range(E))
            continue
        layer, status = int(ln[1]), int(ln[2])
        assert status == MOE_OK, ln
        recs = [tuple(map(int, r.split(":"))) for r in ln[3:]]
        want = lru.lookup(layer, range(E))
        assert recs == [(int(h), s, _ev(v, E)) for _, h, s, v in want], ln[:3]
        if ln[0] == "S":
            assert all(r[0] == 1 for r in recs)


@pytest.mark.parametrize("copy_engine,kind", [(True, 0), (True, 1), (True, 2), (True, 3),
                                              (False, 1), (False, 2), (False, 3), (False, 4)])
@pytest.mark.parametrize("nth", [1, 2, 5, 9])
def test_injected_failures_leave_a_consistent_cache(harness, kind, nth, copy_engine):
    """The n-th copy (0), event creation (1), event record (2), stream wait
    (3) or fill-kernel launch (4) fails: that step returns MOE_EHIP, every
    later step succeeds, no ordering hazard appears, and no step ever reads a
    slot that does not hold the blob it wants (a miss whose fill never
    started leaves the cache).  Copy-engine fills, or the fill kernel with
    the hits on the side stream."""
    out = run(harness, "fault", kind, nth, 3, 16, 4, 2, 10, 60, nth, copy_engine=copy_engine)
    st = [int(ln[2]) for ln in out]
    assert st.count(MOE_EHIP) == 1 and all(s == MOE_OK for s in st if s != MOE_EHIP), st


@pytest.mark.parametrize("ratio", ["0.5", "0", "1"])
@pytest.mark.parametrize("copy_engine", [False, True])
def test_hybrid_policy_protocol_and_trace(harness, ratio, copy_engine):
    """The hybrid miss policy on the CPU harness (real host expert FFN on
    the blobs): the copied share of each step's misses is looked up as by
    the oracle LRU, the rest are reported as host-run (slot -1) and leave the
    cache unchanged; the host's expert outputs are copied to the device
    before the combine and its staging buffer is rewritten only after its
    previous copy finished (no hazard)."""
    import numpy as np
    E = 16
    out = run(harness, "hybrid", ratio, 3, E, 4, 2, 10, 200, 6, copy_engine=copy_engine)
    lru = SlotLRU(10)
    r = np.float32(float(ratio))
    for ln in out:
        assert ln[0] == "D" and int(ln[2]) == MOE_OK, ln
        layer = int(ln[1])
        recs = [tuple(map(int, x.split(":"))) for x in ln[3:]]
        ids = [x[0] for x in recs]
        misses = [e for e in ids if (layer, e) not in lru]
        ncopy = int(r * np.float32(len(misses)) + np.float32(0.5))
        host = set(misses[ncopy:])
        want = {w[0]: w for w in lru.lookup(layer, [e for e in ids if e not in host])}
        for e, h, s_, v in recs:
            if e in host:
                assert (h, s_, v) == (0, -1, -1)
            else:
                _, wh, ws, wv = want[e]
                assert (h, s_, v) == (int(wh), ws, _ev(wv, E))
