"""The allocation-free entry point, moe_expert_ffn_noalloc, through the C ABI.

Two calls in a row on one layer, the second with a smaller batch, each
compared with moe_expert_ffn (caller workspace) on the same inputs and
routing: the same kernels run, so the outputs must be bit-identical; each is
also checked against the oracle (max |gpu - oracle| / max |oracle| <= 1e-2).
Covers the decode GEMV path (NVFP4) and the FP4 matrix-core path (MXFP4
activations)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import DEV, need_gpu, out_f32, resident_layer, say, torch

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.mark.parametrize("fmt,amode,E,k,H,I,sizes", [
    ("nvfp4", "bf16", 32, 8, 2048, 768, (16, 3)),
    ("mxfp4", "mxfp4", 8, 2, 256, 256, (97, 40)),
])
def test_noalloc_matches_the_workspace_entry_point(fmt, amode, E, k, H, I, sizes):
    need_gpu()
    import fp4_expert_ffn_amd as F
    from fp4_expert_ffn_amd.layer import bf16_tensor
    experts = [synth.expert(fmt, H, I, config=91, expert_id=e) for e in range(E)]
    layer = resident_layer(experts, k=k, T=max(sizes), amode=amode)
    for T in sizes:
        say(f"noalloc {fmt}/{amode}: T={T} E={E} k={k} H={H} I={I}")
        x = synth.activations(T, H, 91, T, E)
        logits = np.random.default_rng(T).standard_normal((T, E)).astype(np.float32)
        xd = bf16_tensor(x, DEV)
        layer.route(T, logits=torch.from_numpy(logits).to(DEV))
        a = layer.args(T, xd)
        F.moe_expert_ffn(a)
        torch.cuda.synchronize()
        want = layer.out[:T].clone()
        layer.out.fill_(0x7FC0)  # bf16 NaN: every output must be rewritten
        F.moe_expert_ffn_noalloc(a)
        torch.cuda.synchronize()
        assert torch.equal(layer.out[:T], want)
        ref = oracle.moe.layer(x, experts, k, logits=logits, amode=amode)
        assert np.array_equal(layer.ids[:T].cpu().numpy(), ref["ids"])
        err = oracle.moe.relative_error(out_f32(layer, T), ref["out"])
        say(f"    bit-identical to moe_expert_ffn; rel err vs oracle {err:.3e}")
        assert err <= TOL
