"""Whole-layer parity on the GPU through the C ABI, at small sizes (every path,
several tiles, ragged tails, edge cases) and at the workloads' full sizes
(sampled tokens checked against the oracle one by one).

Tolerance: max |gpu - oracle| / max |oracle| <= 1e-2 over the checked outputs;
routing ids and the permutation bit-exact."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import DEV, DequantCache, need_gpu, out_f32, resident_layer, sample_tokens, say, torch

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    import fp4_expert_ffn_amd  # noqa: F401


def _x(bits):
    from fp4_expert_ffn_amd.layer import bf16_tensor
    return bf16_tensor(bits, DEV)


def _full_check(layer, x_bits, experts, k, logits, shared=None, amode="bf16"):
    T = x_bits.shape[0]
    ids = layer.ids[:T].cpu().numpy()
    ref = oracle.moe.layer(x_bits, experts, k, logits=logits, shared=shared, amode=amode)
    assert np.array_equal(ids, ref["ids"])
    assert np.array_equal(layer.perm[:T * k].cpu().numpy(), ref["perm"])
    err = oracle.moe.relative_error(out_f32(layer, T), ref["out"])
    say(f"    rel err {err:.3e}")
    assert err <= TOL
    return err


def test_tiny_layer():
    L = synth.tiny_layer()
    layer = resident_layer(L["experts"], k=L["k"], T=L["T"])
    say("tiny layer (hidden 256, 8 MXFP4 experts, top-2, 16 tokens)")
    layer.forward(_x(L["x"]), w_router=torch.from_numpy(L["w_router"]).to(DEV))
    torch.cuda.synchronize()
    logits = layer.logits[:L["T"]].cpu().numpy()
    _full_check(layer, L["x"], L["experts"], L["k"], logits)


SMALL = [  # fmt, amode, T, E, k, H, I, shared
    ("nvfp4", "bf16", 37, 16, 4, 256, 256, False),
    ("mxfp4", "bf16", 37, 16, 4, 256, 384, True),
    ("bf16", "bf16", 21, 16, 4, 384, 256, False),
    ("bf16", "bf16", 300, 8, 2, 256, 384, True),     # bf16 MFMA path (600 rows)
    ("mxfp4", "mxfp4", 300, 8, 2, 256, 384, False),  # FP4 MFMA path, several row tiles + ragged tails
    ("mxfp4", "mxfp4", 97, 6, 3, 512, 256, True),
    ("mxfp4", "bf16", 600, 8, 1, 256, 128, False),   # GEMV path at a prefill-like row count
    ("nvfp4", "bf16", 1, 1, 1, 128, 128, False),     # one expert, top-1
]


@pytest.mark.parametrize("fmt,amode,T,E,k,H,I,shared", SMALL)
def test_small_layers_every_path(fmt, amode, T, E, k, H, I, shared):
    experts = [synth.expert(fmt, H, I, config=80, expert_id=e) for e in range(E)]
    sh = synth.expert(fmt, H, I, config=80, expert_id=synth.SHARED_EXPERT) if shared else None
    x = synth.activations(T, H, 80, T, E)
    logits = np.random.default_rng(T + E).standard_normal((T, E)).astype(np.float32)
    if E > 4:
        logits[:, 1] = -1e4  # one expert with no rows
    layer = resident_layer(experts, k=k, T=T, shared=sh, amode=amode)
    say(f"small layer {fmt}/{amode} T={T} E={E} k={k} H={H} I={I} shared={shared}")
    layer.forward(_x(x), logits=torch.from_numpy(logits).to(DEV))
    torch.cuda.synchronize()
    _full_check(layer, x, experts, k, logits, shared=sh, amode=amode)


@pytest.mark.parametrize("fmt,rows", [("nvfp4", "all"), ("mxfp4", "all"), ("nvfp4", "some")])
def test_large_magnitude_activations(fmt, rows):
    """|x| up to about 2^21 (beyond fp16's range) in every token row, or in
    two of them: the NVFP4 path stages operand rows in fp16 with a per-row
    power-of-two shift, taken again from the row's global copy for the rows
    that overflow."""
    T, E, k, H, I = 5, 8, 2, 256, 256
    experts = [synth.expert(fmt, H, I, config=83, expert_id=e) for e in range(E)]
    scale = np.full((T, 1), 2.0 ** 19, np.float32)
    if rows == "some":
        scale[[0, 2, 4]] = 1.0
    x = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(synth.activations(T, H, 83)) * scale)
    logits = np.random.default_rng(9).standard_normal((T, E)).astype(np.float32)
    layer = resident_layer(experts, k=k, T=T)
    say(f"large-magnitude activations {fmt}, {rows} rows")
    layer.forward(_x(x), logits=torch.from_numpy(logits).to(DEV))
    torch.cuda.synchronize()
    _full_check(layer, x, experts, k, logits)


def test_zero_tokens_is_a_no_op():
    experts = [synth.expert("nvfp4", 128, 128, config=81, expert_id=e) for e in range(4)]
    layer = resident_layer(experts, k=2, T=4)
    x = _x(synth.activations(4, 128, 81))
    layer.forward(x[:0], logits=torch.zeros((0, 4), device=DEV))
    torch.cuda.synchronize()


def test_expert_mask_splits_the_work():
    fmt, T, E, k, H, I = "nvfp4", 8, 16, 4, 256, 256
    experts = [synth.expert(fmt, H, I, config=82, expert_id=e) for e in range(E)]
    x = synth.activations(T, H, 82)
    logits = np.random.default_rng(2).standard_normal((T, E)).astype(np.float32)
    layer = resident_layer(experts, k=k, T=T)
    xd = _x(x)
    layer.route(T, logits=torch.from_numpy(logits).to(DEV))
    mask_a = torch.from_numpy((np.arange(E) % 2).astype(np.uint8)).to(DEV)
    mask_b = 1 - mask_a
    say("expert mask: odd experts, then even experts, then combine")
    layer.ffn(T, xd, args=layer.args(T, xd, out=False, mask=mask_a))
    layer.ffn(T, xd, args=layer.args(T, xd, out=False, mask=mask_b))
    from fp4_expert_ffn_amd import moe_combine
    moe_combine(layer.y, layer.inv, layer.w, None, T, k, H, layer.out)
    torch.cuda.synchronize()
    _full_check(layer, x, experts, k, logits)


# ------------------------------------------------------------------ full-size workloads

@pytest.fixture(scope="module")
def a3b_nvfp4():
    return synth.a3b_experts("nvfp4", config=1)


@pytest.mark.parametrize("T", [1, 4, 16])
def test_decode_a3b_nvfp4(a3b_nvfp4, T):
    b = synth.decode_batch(T)
    layer = resident_layer(a3b_nvfp4, k=8, T=T)
    say(f"decode A3B NVFP4 T={T}")
    layer.forward(_x(b["x"]), logits=torch.from_numpy(b["logits"]).to(DEV))
    torch.cuda.synchronize()
    _full_check(layer, b["x"], a3b_nvfp4, 8, b["logits"])


def _sampled_check(layer, b, make_expert, k, amode, shared=None, n_random=10):
    T = b["x"].shape[0]
    ids = layer.ids[:T].cpu().numpy()
    w = layer.w[:T].cpu().numpy()
    rid, rw = oracle.moe.route(b["logits"] if "logits" in b else layer.logits[:T].cpu().numpy(), k)
    assert np.array_equal(ids, rid)
    np.testing.assert_allclose(w, rw, rtol=2e-6, atol=1e-7)
    counts, offsets, perm, inv = oracle.moe.permute(rid, layer.E)
    assert np.array_equal(layer.perm[:T * k].cpu().numpy(), perm)
    assert np.array_equal(layer.counts.cpu().numpy(), counts)
    out = out_f32(layer, T)
    assert np.all(np.isfinite(out))
    toks = sample_tokens(perm, offsets, k, T, n_random, seed=T)
    wts = DequantCache(make_expert)
    sw = oracle.moe.dequant_expert(shared) if shared is not None else None
    ref = np.stack([oracle.moe.token_output(t, b["x"], rid[t], rw[t], wts, shared_weights=sw, amode=amode)
                    for t in toks])
    err = oracle.moe.relative_error(out[toks], ref)
    say(f"    {len(toks)} sampled tokens, rel err {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("fmt,amode", [("bf16", "bf16"), ("mxfp4", "mxfp4")])
def test_prefill_a3b(fmt, amode):
    b = synth.prefill_batch(4096)
    experts = synth.a3b_experts(fmt, config=2)
    layer = resident_layer(experts, k=8, T=4096, amode=amode)
    say(f"prefill A3B T=4096 {fmt} weights, {amode} activations")
    layer.forward(_x(b["x"]), logits=torch.from_numpy(b["logits"]).to(DEV))
    torch.cuda.synchronize()
    _sampled_check(layer, b, lambda e: experts[e], 8, amode)


@pytest.fixture(scope="module")
def large_layer():
    say("generating the large-expert layer (256 + 1 MXFP4 experts, hidden 7168, intermediate 2048)")
    experts = [synth.large_expert(e) for e in range(256)]
    shared = synth.large_expert(synth.SHARED_EXPERT)
    return experts, shared


@pytest.mark.slow
@pytest.mark.parametrize("T,amode", [(1, "bf16"), (2048, "mxfp4")])
def test_large_expert_layer(large_layer, T, amode):
    experts, shared = large_layer
    b = synth.large_batch(T)
    layer = resident_layer(experts, k=8, T=T, shared=shared, amode=amode)
    say(f"large-expert layer T={T} ({amode} activations)")
    layer.forward(_x(b["x"]), w_router=torch.from_numpy(b["w_router"]).to(DEV))
    torch.cuda.synchronize()
    _sampled_check(layer, b, lambda e: experts[e], 8, amode, shared=shared, n_random=6)
    del layer
    torch.cuda.empty_cache()
