"""qd_decode_step_noalloc, the workspace-free decode step over the library's
static device scratch, against qd_decode_step on the same inputs: two calls in
a row, the second over a smaller input (fewer sequences, shorter context)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from tests._gpu_setup import canaries_intact, dev_i32, guarded, make_case, rel_err
from workloads import shapes as S

pytestmark = pytest.mark.gpu


def _step(case, ctx, tokens, noalloc):
    B, V, D = len(ctx), case.shape.vocab, case.shape.hidden
    full, logits = guarded(B * V)
    nxt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    xo = torch.empty(B, D, device="cuda")
    fn = case.runner.step_noalloc if noalloc else case.runner.step
    fn(ctx, dev_i32(ctx), tokens=dev_i32(tokens), logits=logits, next_tokens=nxt, x_out=xo)
    torch.cuda.synchronize()
    assert canaries_intact(full, B * V)
    return logits.view(B, V).cpu().numpy(), nxt.cpu().numpy(), xo.cpu().numpy()


def test_noalloc_matches_the_workspace_step():
    shape = replace(S.QWEN2_0P5B, n_layers=2, vocab=4096)
    case = make_case(shape, [300, 37, 150, 90], seed=3, random_order=True)
    rng = np.random.default_rng(11)
    # first call: four sequences; residual K ranges meet through float atomics at
    # batch > 1, so two runs agree to 1e-5 of the largest logit, not bitwise
    ctx4 = np.array([300, 37, 150, 90], dtype=np.int32)
    tok4 = rng.integers(0, shape.vocab, size=4).astype(np.int32)
    ref_l, ref_n, ref_x = _step(case, ctx4, tok4, noalloc=False)
    got_l, got_n, got_x = _step(case, ctx4, tok4, noalloc=True)
    print(f"batch 4: logits rel diff {rel_err(got_l, ref_l):.2e}, x_out {rel_err(got_x, ref_x):.2e}")
    assert rel_err(got_l, ref_l) <= 1e-5 and rel_err(got_x, ref_x) <= 1e-5
    assert np.array_equal(got_n, ref_n)
    # second call, smaller: one sequence at a shorter position; batch 1 is bitwise repeatable
    ctx1 = np.array([21], dtype=np.int32)
    tok1 = rng.integers(0, shape.vocab, size=1).astype(np.int32)
    ref_l, ref_n, ref_x = _step(case, ctx1, tok1, noalloc=False)
    k_ref = [t.clone() for t in case.kv.k]
    v_ref = [t.clone() for t in case.kv.v]
    got_l, got_n, got_x = _step(case, ctx1, tok1, noalloc=True)
    assert np.array_equal(got_l, ref_l) and np.array_equal(got_x, ref_x)
    assert np.array_equal(got_n, ref_n)
    for a, b in zip(k_ref + v_ref, list(case.kv.k) + list(case.kv.v)):
        assert torch.equal(a, b)
