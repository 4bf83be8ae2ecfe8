"""dllm_step from plain C: tests/c/step_from_c (built by __graft_entry__.build() with gcc against the
in-tree libdllm.so and the HIP runtime, no Python or PyTorch in it) runs a closed-form case on the
GPU and checks every output itself; see tests/c/step_from_c.c."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "step_from_c")


def test_step_from_plain_c():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(EXE), "tests/c/step_from_c is not built: run __graft_entry__.build()"
    print("running tests/c/step_from_c", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok:"), r.stdout
