"""Host-side check of the one-launch batch-1 step's load schedule: compiles
tests/step_schedule_check.cpp (which includes the kernel's own schedule header,
decode_step_amd/csrc/qd_step_sched.h) for the host and runs it over the 0.5B
shape at the positions the tests and the benchmark use, plus edge positions, a
q/k-norm case and a small shape. No GPU is touched.

It checks that every DMA lane of every workgroup reads inside the tensor its
block belongs to, that every matrix byte of a layer (and of the lm_head) is
loaded exactly once, that each needed KV page is loaded, and that the compute
waves' ring cursor agrees with the loader's at every phase."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("sched") / "step_schedule_check")
    cmd = [HIPCC, "-std=c++17", "-O2", "-x", "hip", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "decode_step_amd", "csrc"), os.path.join(ROOT, "tests", "step_schedule_check.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def test_step_schedule_is_in_bounds_and_complete(checker):
    r = subprocess.run([checker], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]
    assert r.stdout.strip().endswith("ok")
