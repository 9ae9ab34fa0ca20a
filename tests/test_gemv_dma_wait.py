"""Generated-code check of the batch-1 GEMV (qd_gemv.hip): the kernel stages its
activation and norm gain in LDS by DMA (global_load_lds_dwordx4) and then issues
every weight load of the tile before waiting, so its wait before the first LDS
barrier is a partial one, s_waitcnt vmcnt(N) with N = the weight loads still
allowed in flight. Vector memory operations retire in issue order, so a DMA has
landed once a wait vmcnt(N) follows it with at least N vector memory
instructions issued after it. This test compiles qd_gemv.hip for gfx950 to
assembly and checks, for every gemv1_kernel instantiation, that each DMA before
the first s_barrier is covered that way (a barrier reached with a DMA still in
flight would let another wave read LDS the DMA has not written). No GPU."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
VMEM = re.compile(r"^\s*(global_|buffer_|scratch_|flat_)\w*")
WAIT = re.compile(r"^\s*s_waitcnt\b(.*)$")


def _vmcnt(args: str):
    m = re.search(r"vmcnt\((\d+)\)", args)
    return int(m.group(1)) if m else None


@pytest.fixture(scope="module")
def gemv_asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "gemv.s")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(ROOT, "decode_step_amd", "csrc"), "--cuda-device-only", "-S",
           os.path.join(ROOT, "decode_step_amd", "csrc", "qd_gemv.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return open(out).read()


def _functions(asm: str):
    """(name, lines) of every gemv1_kernel instantiation, in text order."""
    out, cur, name = [], None, None
    for line in asm.split("\n"):
        m = re.match(r"^(_Z\w*gemv1_kernel\w*):", line)
        if m:
            name, cur = m.group(1), []
            continue
        if cur is not None:
            if line.startswith(".Lfunc_end"):
                out.append((name, cur))
                cur = None
            else:
                cur.append(line)
    return out


def _check(funcs):
    checked = 0
    for name, lines in funcs:
        pending = []      # vector memory ops issued after each uncovered DMA
        for line in lines:
            code = line.split(";")[0]
            if re.match(r"^\s*s_barrier\b", code):
                assert not pending, f"{name}: a DMA may still be in flight at the first s_barrier"
                break
            w = WAIT.match(code)
            if w is not None:
                n = _vmcnt(w.group(1))
                if n is not None:
                    pending = [c for c in pending if c < n]
                continue
            if VMEM.match(code):
                pending = [c + 1 for c in pending]
                if "global_load_lds" in code:
                    pending.append(0)
                    checked += 1
        else:
            raise AssertionError(f"{name}: no s_barrier found")
    return checked


def test_the_check_rejects_an_uncovered_dma():
    """The checker itself: a wait that leaves the DMA among the loads still in
    flight, or no wait at all, fails; a covering wait passes."""
    dma = "\tglobal_load_lds_dwordx4 v0, s[0:1]"
    loads = ["\tglobal_load_dwordx4 v[4:7], v1, s[2:3]"] * 3
    bad1 = [dma] + loads + ["\ts_waitcnt vmcnt(4)", "\ts_barrier"]
    bad2 = [dma] + loads + ["\ts_barrier"]
    good = [dma] + loads + ["\ts_waitcnt vmcnt(3)", "\ts_barrier"]
    for lines in (bad1, bad2):
        with pytest.raises(AssertionError):
            _check([("f", lines)])
    assert _check([("f", good)]) == 1


def test_every_dma_lands_before_the_first_barrier(gemv_asm):
    funcs = _functions(gemv_asm)
    assert len(funcs) >= 20
    assert _check(funcs) > 0
