"""Bitwise repeatability of batched decode steps with QD_DETERMINISTIC=1: the
residual products (o_proj, down) at batch 2..16 take one K range per output block
instead of adding K ranges with float atomics, so two runs of the same step give
the same bits (batch 1 always does). Parity with the fp64 oracle as for every
decode step: 2e-3 of the largest value (bf16 weights and KV), tokens identical.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle.qwen2 import OracleWeights, decode_step
from workloads import shapes as S
from workloads import synth
from tests._gpu_setup import make_case, dev_i32, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _step(case, ctx, tok):
    sh = case.shape
    B = len(ctx)
    logits = torch.full((B, sh.vocab), float("nan"), device="cuda")
    nxt = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    x_out = torch.full((B, sh.hidden), float("nan"), device="cuda")
    case.runner.step(ctx, dev_i32(ctx), tokens=dev_i32(tok), logits=logits, next_tokens=nxt, x_out=x_out)
    torch.cuda.synchronize()
    return logits.cpu(), nxt.cpu(), x_out.cpu()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("shape_name,ctx_list", [
    ("small", [5, 40, 0, 17, 300]),
    ("qwen2-0.5b", [128, 900, 4096, 33, 700, 2048, 1500, 64, 1000, 3000, 257, 511, 2500, 800, 1200, 4000]),
])
def test_batched_step_is_bitwise_repeatable(shape_name, ctx_list, monkeypatch):
    shape = (S.ModelShape(n_layers=2, hidden=136, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=264, vocab=1000)
             if shape_name == "small" else replace(S.QWEN2_0P5B, n_layers=4))
    monkeypatch.setenv("QD_DETERMINISTIC", "1")
    ctx = np.array(ctx_list, np.int32)
    B = len(ctx)
    case = make_case(shape, ctx, seed=19 + B, random_order=True)
    tok = synth.make_tokens(B, shape.vocab, seed=19 + B)
    print(f"deterministic {shape_name} batch {B}", flush=True)
    runs = [_step(case, ctx, tok) for _ in range(3)]
    for lg, nx, xo in runs[1:]:
        assert torch.equal(lg, runs[0][0]) and torch.equal(nx, runs[0][1]) and torch.equal(xo, runs[0][2])
    ref = decode_step(shape, OracleWeights(shape, case.host_w), case.k_host, case.v_host, case.kv.block_table,
                      ctx, tokens=tok)
    err = rel_err(runs[0][0].numpy(), ref.logits)
    print(f"  logits rel err {err:.3e}", flush=True)
    assert err <= 2e-3
    assert rel_err(runs[0][2].numpy(), ref.x_out) <= 2e-3
    assert runs[0][1].tolist() == list(ref.next_tokens)
