"""Per-kernel parity on the GPU through the C ABI: dequantisation, activation
quantiser, router logits, routing, permutation and combine."""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import DEV, need_gpu, say, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    import fp4_expert_ffn_amd  # noqa: F401  (fails loudly if libmoe.so is missing)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("fmt", synth.FMTS)
@pytest.mark.parametrize("H,I", [(256, 128), (2048, 768)])
def test_dequant_bitexact(fmt, H, I):
    from fp4_expert_ffn_amd import moe_dequant_blob
    from fp4_expert_ffn_amd.layer import blob_of
    ex = synth.expert(fmt, H, I, config=70, expert_id=5)
    blob = _dev(blob_of(ex))
    for which, p in enumerate(ex.projs()):
        say(f"dequant {fmt} H={H} I={I} proj={which}")
        out = torch.empty((p.rows, p.cols), dtype=torch.float32, device=DEV)
        moe_dequant_blob(blob, which, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        want = oracle.formats.dequant(p, fmt).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (fmt, which)


def _quant_cases():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 256)).astype(np.float32) * rng.uniform(1e-3, 1e3, (64, 1)).astype(np.float32)
    x[0] = 0.0                                          # all-zero blocks
    x[1, :32] = np.float32(1e-40)                       # subnormal block
    x[2, :32] = np.array([6, 5, 3.5, 2.5, 1.75, 1.25, 0.75, 0.25] * 4, np.float32)  # exact ties at scale 1
    x[3, :32] = -x[2, :32]
    x[4, :32] = np.float32(3.0e38)                       # near the top of the range
    x[5, :32] = -0.0
    x[6, 5] = 7.9                                        # saturating element
    x[7] *= np.float32(2.0**-124) / np.abs(x[7]).max()   # shared exponents -127..-128 clamped, mixed codes
    x[8] *= np.float32(2.0**-120) / np.abs(x[8]).max()   # normal fp32 values, exponents near the bottom
    return synth.f32_to_bf16_bits(x)


def test_quantize_mxfp4_bitexact():
    from fp4_expert_ffn_amd import moe_quantize_mxfp4
    xb = _quant_cases()
    rows, cols = xb.shape
    x = _dev(xb.view(np.int16))
    q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=DEV)
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=DEV)
    say("quantize mxfp4", xb.shape)
    moe_quantize_mxfp4(x, rows, cols, q, s)
    torch.cuda.synchronize()
    codes, scales = oracle.quant.quantize_mxfp4_rows(synth.bf16_bits_to_f32(xb))
    assert np.array_equal(s.cpu().numpy(), scales)
    assert np.array_equal(q.cpu().numpy(), oracle.quant.pack_codes(codes))


def _route_gpu(logits, k, renorm=True):
    from fp4_expert_ffn_amd import moe_route
    T, E = logits.shape
    lg = _dev(logits.astype(np.float32))
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    moe_route(lg, T, E, k, renorm, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def _check_route(logits, k, renorm=True):
    ids, w = _route_gpu(logits, k, renorm)
    rid, rw = oracle.moe.route(logits, k, renorm)
    assert np.array_equal(ids, rid)
    np.testing.assert_allclose(w, rw, rtol=2e-6, atol=1e-7)


def test_route_tie_rows(golden):
    for r in golden("route_ties.txt"):
        k, vals, _ = [p.strip() for p in r.split("|")]
        row = np.array([[float(v) for v in vals.split(",")]], np.float32)
        say("route tie row", r)
        _check_route(row, int(k))


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (1, 128, 8), (37, 128, 8), (300, 256, 8), (64, 1024, 16), (5, 3, 3),
                                   (33, 64, 1)])
def test_route_random(T, E, k):
    rng = np.random.default_rng(T * E + k)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[::3, ::5] = np.round(lg[::3, ::5])  # ties
    if T > 4:
        lg[1, :] = 0.0
        lg[2, ::2] = -0.0
        lg[3, 7 % E] = np.nan
        lg[4, :] = -np.inf
    say(f"route T={T} E={E} k={k}")
    _check_route(lg, k)
    _check_route(lg, k, renorm=False)


def test_route_zipf_workloads():
    for T in (1, 4, 16):
        _check_route(synth.decode_batch(T)["logits"], 8)
    say("route prefill 4096 (masked experts)")
    _check_route(synth.prefill_batch(4096)["logits"], 8)


@pytest.mark.parametrize("T,H,E", [(16, 256, 8), (1, 7168, 256), (2, 2048, 128), (40, 7168, 256), (130, 384, 24),
                                   (2048, 7168, 256), (77, 200, 10), (3, 202, 12), (9, 1000, 64), (4, 9000, 7)])
def test_router_logits_error_bound(T, H, E):
    from fp4_expert_ffn_amd import moe_router_logits
    x = synth.activations(T, H, 71, T, H)
    w = synth.router_weight(E, H, 72, E)
    out = torch.empty((T, E), dtype=torch.float32, device=DEV)
    say(f"router logits T={T} H={H} E={E}")
    moe_router_logits(_dev(x.view(np.int16)), _dev(w), T, H, E, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = oracle.moe.router_logits(x, w)
    # fp32 accumulation of H exact products: |err| <= gamma_H * sum |x||w|  (Higham, gamma_n = n u / (1 - n u)).
    # The matrix-core path splits w = hi + lo + lo2 (bf16 parts by truncation, |hi| + |lo| + |lo2| <=
    # (1 + 2^-7 + 2^-15) |w|), sums each part over H in fp32 and adds the three sums: gamma_{H+2} * (1 + 2^-6)
    # * sum |x||w| bounds both methods.
    u = 2.0 ** -24
    n = H + 2
    gamma = n * u / (1 - n * u) * (1 + 2.0 ** -6)
    bound = gamma * (np.abs(synth.bf16_bits_to_f32(x)).astype(np.float64) @ np.abs(w.astype(np.float64)).T)
    assert np.all(np.abs(got - ref) <= bound + 1e-30)


def _permute_gpu(ids, E):
    from fp4_expert_ffn_amd import moe_permute
    T, k = ids.shape
    N = T * k
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    perm = torch.empty(max(N, 1), dtype=torch.int32, device=DEV)
    inv = torch.empty(max(N, 1), dtype=torch.int32, device=DEV)
    moe_permute(_dev(ids) if N else None, T, k, E, counts, offsets, perm, inv)
    torch.cuda.synchronize()
    return counts.cpu().numpy(), offsets.cpu().numpy(), perm.cpu().numpy()[:N], inv.cpu().numpy()[:N]


@pytest.mark.parametrize("T,k,E", [(16, 2, 8), (1, 8, 128), (4, 8, 128), (16, 8, 128), (37, 8, 128), (129, 8, 1024),
                                   (300, 1, 1), (2048, 8, 256), (1100, 8, 512), (350, 3, 3), (1000, 8, 1024),
                                   (1500, 7, 200), (129, 8, 64)])
def test_permute_bitexact(T, k, E):
    rng = np.random.default_rng(T + k + E)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    say(f"permute T={T} k={k} E={E}")
    got = _permute_gpu(ids, E)
    want = oracle.moe.permute(ids, E)
    for g, w in zip(got, want):
        assert np.array_equal(g, w)


def test_permute_prefill_zipf_full_size():
    lg = synth.prefill_batch(4096)["logits"]
    ids, _ = oracle.moe.route(lg, 8)
    say("permute 4096 x 8 Zipf")
    got = _permute_gpu(ids, 128)
    want = oracle.moe.permute(ids, 128)
    for g, w in zip(got, want):
        assert np.array_equal(g, w)
    assert np.sum(want[0] == 0) == 8  # the masked experts receive no token


@pytest.mark.parametrize("T,E,k", [(1, 128, 8), (4, 128, 8), (16, 128, 8), (16, 8, 2), (64, 1024, 16), (128, 128, 8),
                                   (200, 256, 8), (0, 32, 4), (64, 128, 8), (33, 64, 16), (5, 3, 3), (40, 300, 4),
                                   (17, 256, 8), (64, 8, 8), (65, 128, 8), (2, 1000, 16)])
def test_route_permute_fused(T, E, k):
    """moe_route_permute (one launch when T*k <= 1024, two otherwise) equals the oracle."""
    from fp4_expert_ffn_amd import moe_route_permute
    rng = np.random.default_rng(T * 7 + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if T > 2:
        lg[1, :] = 0.0
        lg[2, 3 % E] = np.nan
    if T > 4:
        lg[3, :] = -np.inf
        lg[4, ::2] = np.round(lg[4, ::2])  # ties
    N = T * k
    ids = torch.empty((max(T, 1), k), dtype=torch.int32, device=DEV)
    w = torch.empty((max(T, 1), k), dtype=torch.float32, device=DEV)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    perm = torch.empty(max(N, 1), dtype=torch.int32, device=DEV)
    inv = torch.empty(max(N, 1), dtype=torch.int32, device=DEV)
    say(f"route+permute T={T} E={E} k={k}")
    moe_route_permute(_dev(lg) if T else None, T, E, k, True, ids, w, counts, offsets, perm, inv)
    torch.cuda.synchronize()
    rid, rw = oracle.moe.route(lg, k) if T else (np.zeros((0, k), np.int32), np.zeros((0, k), np.float32))
    c, o, p, iv = oracle.moe.permute(rid, E)
    if T:
        assert np.array_equal(ids.cpu().numpy(), rid)
        np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=2e-6, atol=1e-7)
    assert np.array_equal(counts.cpu().numpy(), c) and np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(perm.cpu().numpy()[:N], p) and np.array_equal(inv.cpu().numpy()[:N], iv)


def test_permute_empty():
    say("permute empty")
    counts, offsets, perm, inv = _permute_gpu(np.zeros((0, 4), np.int32), 16)
    assert not counts.any() and not offsets.any()


def test_combine_matches_formula():
    from fp4_expert_ffn_amd import moe_combine
    rng = np.random.default_rng(5)
    T, k, H = 37, 8, 1024
    y = rng.standard_normal((T * k, H)).astype(np.float32)
    perm = rng.permutation(T * k).astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(T * k)
    w = rng.random((T, k)).astype(np.float32)
    sh = rng.standard_normal((T, H)).astype(np.float32)
    out = torch.empty((T, H), dtype=torch.int16, device=DEV)
    say("combine")
    moe_combine(_dev(y), _dev(inv), _dev(w), _dev(sh), T, k, H, out)
    torch.cuda.synchronize()
    got = synth.bf16_bits_to_f32(out.cpu().numpy().view(np.uint16))
    ref, _ = oracle.moe.combine(y.astype(np.float64), inv, w, sh.astype(np.float64))
    assert oracle.moe.relative_error(got, ref) <= 2 ** -8
