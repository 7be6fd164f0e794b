"""Static checks on the compiled decode kernel (CPU only: hipcc cross-compiles
gfx950 assembly).

The decode GEMV waits for its direct-to-LDS operand rows with an explicit
`s_waitcnt vmcnt(N)` that counts the weight loads issued behind them (the
vector-memory counter completes in order, so N later loads outstanding means
the rows have landed).  That is only correct if the compiled code issues
exactly N vector-memory loads behind the rows before the wait (the bank
between two scheduling barriers, nothing else); this test checks it for every
instantiation, so a compiler that merges or splits those loads fails here
instead of racing on the GPU."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def gemv_asm(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "gemv.s"
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
           os.path.join(ROOT, "fp4_expert_ffn_amd", "csrc", "ffn_gemv.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _row_waits(body):
    """(N, loads) for every explicit row wait: an `s_waitcnt vmcnt(N)` directly
    followed by `s_barrier`, with the number of vector-memory loads issued in
    the block between the two scheduling barriers that precede it (the bank
    issued behind the rows)."""
    lines = [ln.strip() for ln in body.split("\n")]
    code = [(i, t) for i, t in enumerate(lines) if t and not t.startswith(";;")]
    out = []
    for n, (i, t) in enumerate(code[:-1]):
        if not (t.startswith("s_waitcnt") and "vmcnt(" in t and code[n + 1][1] == "s_barrier"):
            continue
        wait = int(t.split("vmcnt(")[1].split(")")[0])
        marks = [j for j in range(i) if lines[j].startswith("; sched_barrier")]
        assert len(marks) >= 2, "row wait without the bank's scheduling barriers"
        lo, hi = marks[-2], marks[-1]
        between = lines[hi + 1:i]
        assert not any(x.startswith(("global_", "buffer_", "flat_", "scratch_")) for x in between), between
        loads = sum(1 for x in lines[lo + 1:hi] if x.startswith(("global_load", "buffer_load", "flat_load")))
        out.append((wait, loads))
    return out


def test_row_wait_counts_the_loads_behind_the_rows(gemv_asm):
    names = re.findall(r"^(_ZN3moe6k_gemvILi(\d)ELb(\d)ELi(\d+)ELb(\d)ELb(\d)EEE\w+):", gemv_asm, re.M)
    # 4 formats x (gate/up, gate/up with every token row staged, the same
    # with the routing folded in, down) x 6 sub-item sizes, less NVFP4's and
    # FP8's 16 (their largest is 8)
    assert len(names) == 88, len(names)
    for full, fmt, _down, sub, _xall, route in names:
        fmt, sub = int(fmt), int(sub)
        body = gemv_asm[gemv_asm.index(full + ":"):gemv_asm.index(".Lfunc_end", gemv_asm.index(full + ":"))]
        k = body.find("global_load_lds_dwordx4")
        assert k > 0, full
        if route == "1":
            # the token rows go out first; the folded routing's first barrier
            # waits for every load (they have landed before any use)
            lines = [ln.strip() for ln in body[k:].split("\n") if ln.strip() and not ln.strip().startswith(";")]
            b = lines.index("s_barrier")
            assert lines[b - 1].startswith("s_waitcnt") and "vmcnt(0)" in lines[b - 1], (full, lines[b - 1])
            continue
        waits = _row_waits(body[k:])
        assert waits, full
        # tiles and scales (the 4-bit formats) of the bank issued behind the rows
        expected = sub + (sub if fmt in (1, 2) else 0)
        for wait, loads in waits:
            assert wait == expected and loads == expected, (full, loads, wait, expected)


@pytest.fixture(scope="module")
def fp4gemm_asm(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "fp4gemm.s"
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
           os.path.join(ROOT, "fp4_expert_ffn_amd", "csrc", "ffn_fp4gemm.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def test_prefill_gemm_owns_m0(fp4gemm_asm):
    """The prefill GEMM's direct-to-LDS loads set M0 in inline assembly; that is
    only sound while the compiler itself neither reads nor writes M0 in the
    kernel: every mention must be one of those `s_mov_b32 m0` + load pairs."""
    names = re.findall(r"^(_ZN3moe1[01]k_(?:fp4|bf16)_gemm\w+):", fp4gemm_asm, re.M)
    # {FP4, BF16} x {gate/up, down (bf16 out), down (fp32 out)}
    assert len(names) == 6, names
    for full in names:
        i = fp4gemm_asm.index(full + ":")
        body = fp4gemm_asm[i:fp4gemm_asm.index(".Lfunc_end", i)]
        lines = [ln.strip() for ln in body.split("\n") if ln.strip() and not ln.strip().startswith(";")]
        n = 0
        for k, ln in enumerate(lines):
            if re.search(r"\bm0\b", ln):
                assert ln.startswith("s_mov_b32 m0,") and lines[k + 1] == "s_nop 0" and \
                    lines[k + 2].startswith("global_load_lds"), (full, ln)
                n += 1
        assert n >= 8, (full, n)
