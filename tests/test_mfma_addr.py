"""CPU check of the 128 x 128 grouped GEMM's stage-load addresses.

The kernel forms the byte offset of every stage load with the host+device
functions of ``csrc/mfma_addr.h``.  This test compiles that header into a
host program and enumerates, for the shapes the kernel accepts (including a
half K-step tail at the first step, K = 128, and at a later one, K = 384),
every offset each thread forms for x or the SwiGLU output, the weights and
both scale operands: each must index the intended row, K-tile and lane, and
stay inside its buffer.  The same enumeration through a formula that casts
the step offset to 32 bits after subtracting the tail's step-back (a wrap to
about 4 GiB when the tail is step 0) must report violations, which shows the
check sees that mistake."""
import os
import subprocess

import pytest

from tests.conftest import ROOT

SRC = os.path.join(ROOT, "tests", "cpu", "mfma_addr_check.cpp")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("addr") / "mfma_addr_check")
    cmd = ["/opt/rocm/bin/hipcc", "-x", "hip", "--offload-host-only", "-O1", "-std=c++17", SRC, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(f"build failed:\n{r.stderr}")
    return exe


def _run(exe, fp4, gateup, H, I, rows):
    r = subprocess.run([exe, str(int(fp4)), str(int(gateup)), str(H), str(I), str(rows)], capture_output=True,
                       text=True, check=True)
    _, bad, _, wrapped = r.stdout.split()
    return int(bad), int(wrapped), r.stderr


SHAPES = [  # H, I, rows of the A operand
    (256, 128, 300), (128, 256, 37), (128, 128, 5), (256, 384, 600), (512, 256, 97),
    (2048, 768, 4096), (7168, 2048, 2048 * 9),
]


@pytest.mark.parametrize("H,I,rows", SHAPES)
@pytest.mark.parametrize("fp4", [True, False])
@pytest.mark.parametrize("gateup", [True, False])
def test_every_stage_load_in_bounds(checker, fp4, gateup, H, I, rows):
    bad, wrapped, err = _run(checker, fp4, gateup, H, I, rows)
    assert bad == 0, err
    K = H if gateup else I
    if fp4 and K == 128:
        # the half K-step tail is step 0: the wrapping formula leaves the buffer
        assert wrapped > 0
    else:
        assert wrapped == 0
