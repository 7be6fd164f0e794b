"""Whole-layer parity on the GPU through the C ABI, at small sizes (every path,
several tiles, ragged tails, edge cases) and at the workloads' full sizes (the
whole [T, H] output against the oracle's grouped evaluation).

Tolerance: max |gpu - oracle| / max |oracle| <= 1e-2 over the whole output;
routing ids, weights' selection and the permutation bit-exact.  On the FP4
path (MXFP4 x MXFP4) the encoding of x is bit-exact and at most 1e-3 of the
SwiGLU output's encoded values may differ from the oracle's (a value within
rounding of an E2M1 boundary); its deviation from the bf16-activation oracle
is printed, not graded."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (DEV, fp4_code_report, gpu_fp4_codes, grouped_reference, need_gpu, out_f32, resident_layer, say,
                            torch)

pytestmark = pytest.mark.gpu
TOL = 1e-2
H_CODE_TOL = 1e-3


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
    if amode == "mxfp4":
        h_ref = {}
        oracle.moe.layer_outputs(x_bits, ref["ids"], ref["w"], len(experts),
                                 lambda e: oracle.moe.dequant_expert(experts[e]),
                                 shared_weights=oracle.moe.dequant_expert(shared) if shared is not None else None,
                                 amode=amode, h_codes=h_ref)
        frac = fp4_code_report(layer, T, layer.state.last_x, x_bits, ref["perm"], k, h_ref, shared=shared is not None)
        assert frac <= H_CODE_TOL
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
    ("mxfp4", "mxfp4", 300, 8, 2, 256, 768, True),   # persistent FP4 GEMM: 6 gate/up column blocks, down K 6 steps
    ("mxfp4", "bf16", 600, 8, 1, 256, 128, False),   # GEMV path at a prefill-like row count
    ("nvfp4", "bf16", 1, 1, 1, 128, 128, False),     # one expert, top-1
    ("mxfp4", "mxfp4", 300, 8, 2, 256, 128, False),  # 128 x 128 FP4 kernel, down K = 128: half K-step at step 0
    ("mxfp4", "mxfp4", 77, 8, 2, 128, 256, True),    # 128 x 128 FP4 kernel, gate/up K = 128
    ("mxfp4", "mxfp4", 40, 4, 2, 128, 128, True),    # both projections K = 128
    ("fp8", "bf16", 37, 16, 4, 256, 384, True),      # FP8 on the GEMV
    ("fp8", "bf16", 13, 8, 2, 384, 128, False),
    ("fp8", "bf16", 600, 8, 1, 256, 128, False),     # FP8 decoded to bf16 on the matrix cores
    ("nvfp4", "bf16", 300, 8, 2, 256, 384, True),    # NVFP4 decoded to bf16 on the matrix cores
    ("nvfp4", "bf16", 700, 16, 1, 384, 256, False),
    ("fp8", "bf16", 257, 6, 3, 512, 256, True),
    ("mxfp4", "bf16", 3, 64, 8, 256, 256, True),     # routing folded into the gate/up launch (T <= 4)
    ("bf16", "bf16", 4, 256, 8, 256, 128, False),
    ("fp8", "bf16", 2, 16, 4, 384, 256, True),
    ("nvfp4", "bf16", 4, 128, 16, 256, 128, False),  # T * k = 64
    ("nvfp4", "bf16", 16, 128, 8, 256, 256, True),   # T * k = 128: routing kernel, then the GEMV launches
    ("mxfp4", "bf16", 11, 256, 8, 512, 384, False),  # E = 256; down K-tiles 3 (sub-items of 1)
    ("bf16", "bf16", 16, 32, 8, 256, 256, True),
    ("fp8", "bf16", 9, 64, 8, 384, 768, True),       # gate/up K-tiles 6 (sub-items of 2), down 12
    ("mxfp4", "bf16", 5, 8, 8, 256, 128, False),     # k = E: every expert in every token
    ("nvfp4", "bf16", 7, 16, 8, 128, 256, True),     # one gate/up K-tile
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


def test_fp4_tiny_swiglu_blocks():
    """x scaled by 2^-61, so that many 32-value blocks of the SwiGLU output lie
    below 2^-124 and take the smallest block scale (E8M0 code 0, 2^-127): the
    persistent FP4 kernel's encodings of them match the oracle's, as does the
    (tiny) output."""
    fmt, amode, T, E, k, H, I = "mxfp4", "mxfp4", 300, 8, 2, 256, 768
    experts = [synth.expert(fmt, H, I, config=80, expert_id=e) for e in range(E)]
    x = synth.activations(T, H, 80, T, E)
    # an exact power-of-two scaling of the bf16 values (no underflow at 2^-61)
    x = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(x) * np.float32(2.0 ** -61))
    logits = np.random.default_rng(7).standard_normal((T, E)).astype(np.float32)
    layer = resident_layer(experts, k=k, T=T, amode=amode)
    say(f"tiny SwiGLU blocks: {fmt}/{amode} T={T} E={E} k={k} H={H} I={I}, x * 2^-61")
    layer.forward(_x(x), logits=torch.from_numpy(logits).to(DEV))
    torch.cuda.synchronize()
    _, hs = gpu_fp4_codes(layer, T, layer.state.last_x, 1)
    frac0 = float(np.mean(hs == 0))
    say(f"    blocks with scale 2^-127: {frac0:.2f}")
    assert frac0 > 0.05, "the inputs no longer reach the smallest block scale"
    _full_check(layer, x, experts, k, logits, amode=amode)


@pytest.mark.parametrize("fmt,rows", [("nvfp4", "all"), ("mxfp4", "all"), ("nvfp4", "some"), ("fp8", "some")])
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


@pytest.mark.parametrize("fmt,T,rows", [("nvfp4", 1, "all"), ("nvfp4", 4, "all"), ("nvfp4", 16, "some"),
                                         ("fp8", 16, "all")])
def test_tiny_activation_rows(fmt, T, rows):
    """Token rows whose largest |x| is about 2^-55 (fp16's subnormal range ends
    at 2^-24): the NVFP4 / FP8 decode path stages operand rows in fp16, so such
    rows are taken again from their global copy with a power-of-two up-shift.
    Checked per token row, each against its own largest output."""
    E, k, H, I = 8, 2, 256, 256
    experts = [synth.expert(fmt, H, I, config=84, expert_id=e) for e in range(E)]
    scale = np.full((T, 1), 2.0 ** -57, np.float32)
    if rows == "some":
        scale[[0, 2, 4]] = 1.0
    x = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(synth.activations(T, H, 84)) * scale)
    logits = np.random.default_rng(11).standard_normal((T, E)).astype(np.float32)
    layer = resident_layer(experts, k=k, T=T)
    say(f"tiny activation rows {fmt} T={T}, {rows} rows")
    layer.forward(_x(x), logits=torch.from_numpy(logits).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.moe.layer(x, experts, k, logits=logits)
    assert np.array_equal(layer.ids[:T].cpu().numpy(), ref["ids"])
    out = out_f32(layer, T)
    worst = max(oracle.moe.relative_error(out[t], ref["out"][t]) for t in range(T))
    say(f"    worst per-row rel err {worst:.3e}")
    assert worst <= TOL


@pytest.mark.parametrize("T", [1, 4, 16])
def test_folded_routing_edge_rows(T):
    """moe_layer's routing (folded into the gate/up launch for T <= 4, the
    routing kernel above) on rows with ties, -inf and NaN logits: ids,
    weights, counts, offsets, perm and inv against the oracle's route and
    permute (ids and the permutation bit-exact), and the output against the
    oracle layer."""
    fmt, E, k, H, I = "nvfp4", 128, 8, 256, 256
    experts = [synth.expert(fmt, H, I, config=93, expert_id=e) for e in range(E)]
    rng = np.random.default_rng(T)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[0, [5, 9, 17, 40, 41, 100, 120, 127]] = 3.0                 # an 8-way tie at the top
    logits[0, [60, 61]] = 3.0                                          # ... and beyond it
    if T > 1:
        logits[1, :] = -np.inf
        logits[1, [7, 8, 90]] = [0.5, np.nan, 0.5]
        logits[2, :] = 1.0                                             # all equal
        logits[3, 10:20] = np.nan
    if T > 4:
        logits[5, :] = 0.0                                             # all zero (+0 and -0)
        logits[5, 1::2] = -0.0
        logits[9, [3, 4]] = np.inf                                     # two +inf
        logits[T - 1] = logits[0]                                      # the first row again
    x = synth.activations(T, H, 93, T)
    layer = resident_layer(experts, k=k, T=T)
    say(f"folded routing, edge rows, T={T}")
    layer.forward(_x(x), logits=torch.from_numpy(logits).to(DEV))
    torch.cuda.synchronize()
    rid, rw = oracle.moe.route(logits, k)
    counts, offsets, perm, inv = oracle.moe.permute(rid, E)
    assert np.array_equal(layer.ids[:T].cpu().numpy(), rid)
    np.testing.assert_allclose(layer.w[:T].cpu().numpy(), rw, rtol=2e-6, atol=1e-7)
    assert np.array_equal(layer.counts.cpu().numpy(), counts)
    assert np.array_equal(layer.offsets.cpu().numpy(), offsets)
    assert np.array_equal(layer.perm[:T * k].cpu().numpy(), perm)
    assert np.array_equal(layer.inv[:T * k].cpu().numpy(), inv)
    ref = oracle.moe.layer(x, experts, k, logits=logits)
    err = oracle.moe.relative_error(out_f32(layer, T), ref["out"])
    say(f"    rel err {err:.3e}")
    assert err <= TOL


def test_layer_replays_over_a_dirty_workspace():
    """A moe_layer call reads no workspace byte it has not written itself:
    graph replays of one call, with the whole workspace overwritten by
    garbage between them, and eager calls after that give the first call's
    output bit for bit (the sums run in a fixed order, so the result is
    deterministic)."""
    fmt, E, k, H, I, T = "nvfp4", 128, 8, 256, 256, 16
    experts = [synth.expert(fmt, H, I, config=95, expert_id=e) for e in range(E)]
    sh = synth.expert(fmt, H, I, config=95, expert_id=synth.SHARED_EXPERT)
    x = synth.activations(T, H, 95, T, E)
    logits = np.random.default_rng(95).standard_normal((T, E)).astype(np.float32)
    layer = resident_layer(experts, k=k, T=T, shared=sh)
    xs, lg = _x(x), torch.from_numpy(logits).to(DEV)
    say("moe_layer: graph replays over a dirty workspace")
    layer.forward(xs, logits=lg)
    torch.cuda.synchronize()
    _full_check(layer, x, experts, k, logits, shared=sh)
    st = layer.state
    first = st.out[:T].clone()
    la = st.layer_args(T, xs, lg)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        st.call(T, xs, logits=lg, la=la)
    torch.cuda.synchronize()
    for i, junk in enumerate((0xFF, 0x5A, 0x01)):
        st._ws.fill_(junk)
        st.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.out[:T], first), f"replay {i}"
    st._ws.fill_(0x7F)
    layer.forward(xs, logits=lg)
    torch.cuda.synchronize()
    assert torch.equal(st.out[:T], first)


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


@pytest.mark.parametrize("H,I,shared", [(256, 128, False), (128, 256, True)])
def test_fp4_expert_outputs_in_fp32(H, I, shared):
    """MXFP4 activations on the 128 x 128 kernel (a projection with K = 128:
    its only K-step is the half tail) writing fp32 expert outputs in
    permutation order: every row of y against the oracle's, then
    moe_combine."""
    fmt, T, E, k = "mxfp4", 300, 8, 2
    experts = [synth.expert(fmt, H, I, config=84, expert_id=e) for e in range(E)]
    sh = synth.expert(fmt, H, I, config=84, expert_id=synth.SHARED_EXPERT) if shared else None
    x = synth.activations(T, H, 84, H, I)
    logits = np.random.default_rng(H + I).standard_normal((T, E)).astype(np.float32)
    layer = resident_layer(experts, k=k, T=T, shared=sh, amode="mxfp4")
    xd = _x(x)
    say(f"FP4 expert outputs in fp32: T={T} E={E} k={k} H={H} I={I} shared={shared}")
    layer.route(T, logits=torch.from_numpy(logits).to(DEV))
    layer.ffn(T, xd, args=layer.args(T, xd, out=False))
    from fp4_expert_ffn_amd import moe_combine
    R = T * k
    ysh = layer.y[R:] if shared else None
    moe_combine(layer.y, layer.inv, layer.w, ysh, T, k, H, layer.out)
    torch.cuda.synchronize()
    ref = oracle.moe.layer(x, experts, k, logits=logits, shared=sh, amode="mxfp4")
    y = layer.y[:R].cpu().numpy()
    err_y = oracle.moe.relative_error(y, ref["y_perm"])
    err_s = oracle.moe.relative_error(layer.y[R:R + T].cpu().numpy(), ref["y_shared"]) if shared else 0.0
    err = oracle.moe.relative_error(out_f32(layer, T), ref["out"])
    say(f"    y rel err {err_y:.3e}, shared {err_s:.3e}, combined {err:.3e}")
    assert err_y <= TOL and err_s <= TOL and err <= TOL


# ------------------------------------------------------------------ full-size workloads

@pytest.fixture(scope="module")
def a3b_nvfp4():
    return synth.a3b_experts("nvfp4", config=1)


@pytest.mark.parametrize("T", [1, 16])
def test_decode_a3b_fp8(T):
    experts = synth.a3b_experts("fp8", config=1)
    b = synth.decode_batch(T)
    layer = resident_layer(experts, k=8, T=T)
    say(f"decode A3B FP8 T={T}")
    layer.forward(_x(b["x"]), logits=torch.from_numpy(b["logits"]).to(DEV))
    torch.cuda.synchronize()
    _full_check(layer, b["x"], experts, 8, b["logits"])


@pytest.mark.parametrize("T", [1, 4, 16])
def test_decode_a3b_nvfp4(a3b_nvfp4, T):
    b = synth.decode_batch(T)
    layer = resident_layer(a3b_nvfp4, k=8, T=T)
    say(f"decode A3B NVFP4 T={T}")
    layer.forward(_x(b["x"]), logits=torch.from_numpy(b["logits"]).to(DEV))
    torch.cuda.synchronize()
    _full_check(layer, b["x"], a3b_nvfp4, 8, b["logits"])


def _whole_check(layer, b, make_expert, k, amode, shared=None, logits=None, bf16_deviation=False):
    """The whole [T, H] output against the oracle's grouped evaluation of the
    same routing (routing, weights and permutation checked first); on the FP4
    path also the R15 encodings, and optionally the deviation from the
    bf16-activation oracle (printed)."""
    T = b["x"].shape[0]
    ids = layer.ids[:T].cpu().numpy()
    w = layer.w[:T].cpu().numpy()
    lg = logits if logits is not None else layer.logits[:T].cpu().numpy()
    rid, rw = oracle.moe.route(lg, k)
    assert np.array_equal(ids, rid)
    np.testing.assert_allclose(w, rw, rtol=2e-6, atol=1e-7)
    counts, offsets, perm, inv = oracle.moe.permute(rid, layer.E)
    assert np.array_equal(layer.perm[:T * k].cpu().numpy(), perm)
    assert np.array_equal(layer.counts.cpu().numpy(), counts)
    out = out_f32(layer, T)
    h_ref = {} if amode == "mxfp4" else None
    ref = grouped_reference(b["x"], rid, rw, layer.E, make_expert, shared=shared, amode=amode, h_codes=h_ref)
    err = oracle.moe.relative_error(out, ref)
    say(f"    whole output [{T}, {out.shape[1]}]: rel err {err:.3e}")
    assert err <= TOL
    if amode == "mxfp4":
        frac = fp4_code_report(layer, T, layer.state.last_x, b["x"], perm, k, h_ref, shared=shared is not None)
        assert frac <= H_CODE_TOL
        if bf16_deviation:
            ref16 = grouped_reference(b["x"], rid, rw, layer.E, make_expert, shared=shared, amode="bf16")
            say(f"    deviation from the bf16-activation oracle (reported, not graded): "
                f"{oracle.moe.relative_error(out, ref16):.3e}")


@pytest.mark.parametrize("fmt,amode", [("bf16", "bf16"), ("mxfp4", "mxfp4"), ("nvfp4", "bf16"), ("fp8", "bf16")])
def test_prefill_a3b(fmt, amode):
    b = synth.prefill_batch(4096)
    experts = synth.a3b_experts(fmt, config=2)
    layer = resident_layer(experts, k=8, T=4096, amode=amode)
    say(f"prefill A3B T=4096 {fmt} weights, {amode} activations")
    layer.forward(_x(b["x"]), logits=torch.from_numpy(b["logits"]).to(DEV))
    torch.cuda.synchronize()
    _whole_check(layer, b, lambda e: experts[e], 8, amode, logits=b["logits"], bf16_deviation=amode == "mxfp4")


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
    _whole_check(layer, b, lambda e: experts[e], 8, amode, shared=shared)
    del layer
    torch.cuda.empty_cache()
