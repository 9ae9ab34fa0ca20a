"""GPU parity of the batch-1 residual product by head slices (the o_proj of a
context wider than 1024 values, over several attention splits: each workgroup
merges one head's splits and adds its slice of the product into the residual
with float atomics, so no merge launch runs), against the fp64 oracle, and
against the same step with the merge launch (QD_O_HEADS=0) and with
QD_DETERMINISTIC=1 (the merge launch again, bitwise repeatable).

Shapes: head_dim 128 with q/k norm and no biases (the 8B-class layer, scaled
down: 16 query heads, 4 KV heads, a multiple of 8 heads, so the workgroups of a
head share an XCD), and head_dim 64 with biases and 20 query heads (not a
multiple of 8: the plain workgroup order). Positions: short contexts take one
query head per workgroup on the vector-ALU attention with long splits (288 keys
at head_dim 128, 576 at 64): 499 (two splits), 576 (a last split holding only
the new token); long ones the matrix-core attention, at most 32 splits where
the chunk allows: 1999 (32 splits of 64 keys), 4095 (32 of 128) and 9000 (36 of
256, the longest chunk: the kernel's 64-split form).
Bound: 2e-3 of the largest value (bf16 weights and KV), identical greedy tokens,
stored K/V within one bf16 step of the oracle's; the two forms of the product
agree to 1e-5 (float32 rounding of a different order of additions).
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from decode_step_amd import qd as Q
from oracle.qwen2 import OracleWeights, decode_step
from workloads import shapes as S
from workloads import synth
from tests._gpu_setup import make_case, dev_i32, rel_err, kv_matches

pytestmark = pytest.mark.gpu

SHAPES = {
    "hd128_qknorm": S.ModelShape(n_layers=2, hidden=512, n_q_heads=16, n_kv_heads=4, head_dim=128, ffn=1024,
                                 vocab=2048, qkv_bias=False, qk_norm=True, tied=False),
    "hd64_bias": S.ModelShape(n_layers=2, hidden=640, n_q_heads=20, n_kv_heads=4, head_dim=64, ffn=1024,
                              vocab=2048),
}
CASES = [("hd128_qknorm", p) for p in (499, 576, 1999, 9000)] + [("hd64_bias", p) for p in (576, 4095, 9000)]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _step(case, p, tok):
    sh = case.shape
    logits = torch.full((1, sh.vocab), float("nan"), device="cuda")
    nxt = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    layer_out = torch.full((sh.n_layers, 1, sh.hidden), float("nan"), device="cuda")
    pos = np.array([p], np.int32)
    case.runner.step(pos, dev_i32(pos), tokens=dev_i32(tok), logits=logits, next_tokens=nxt, layer_out=layer_out)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), int(nxt.cpu()[0]), layer_out.cpu().numpy()


@pytest.mark.timeout(300)
@pytest.mark.parametrize("shape_name,p", CASES)
def test_o_proj_by_head_slices(shape_name, p, monkeypatch):
    sh = SHAPES[shape_name]
    monkeypatch.delenv("QD_O_HEADS", raising=False)
    monkeypatch.delenv("QD_DETERMINISTIC", raising=False)
    case = make_case(sh, np.array([p], np.int32), seed=300 + p, extra=2)
    plan = Q.qd_decode_plan(case.runner.cfg, 1, p + 1)
    assert plan.merge_in_o_proj == 2 and 1 < plan.splits <= 64, (plan.merge_in_o_proj, plan.splits)
    tok = synth.make_tokens(1, sh.vocab, seed=300 + p)
    print(f"o_proj by head slices: {shape_name} p={p} splits={plan.splits}", flush=True)
    logits, nxt, layer_out = _step(case, p, tok)
    ref = decode_step(sh, OracleWeights(sh, case.host_w), case.k_host, case.v_host, case.kv.block_table,
                      np.array([p]), tokens=tok)
    err = rel_err(logits, ref.logits)
    print(f"  logits rel err {err:.3e}", flush=True)
    assert err <= 2e-3
    for l in range(sh.n_layers):
        assert rel_err(layer_out[l], ref.layer_out[l]) <= 2e-3, l
    assert nxt == int(ref.next_tokens[0])
    for l in range(sh.n_layers):
        assert kv_matches(case.kv.k[l], case.k_host[l]) and kv_matches(case.kv.v[l], case.v_host[l]), l

    # the merge launch and the row-block GEMV: the same result to float32 rounding
    monkeypatch.setenv("QD_O_HEADS", "0")
    assert Q.qd_decode_plan(case.runner.cfg, 1, p + 1).merge_in_o_proj == 0
    print(f"  merge launch", flush=True)
    logits2, nxt2, layer_out2 = _step(case, p, tok)
    assert rel_err(logits2, ref.logits) <= 2e-3
    assert rel_err(layer_out2, layer_out.astype(np.float64)) <= 1e-5
    assert nxt2 == nxt

    # QD_DETERMINISTIC=1 keeps the merge launch: two runs bitwise equal
    monkeypatch.delenv("QD_O_HEADS")
    monkeypatch.setenv("QD_DETERMINISTIC", "1")
    assert Q.qd_decode_plan(case.runner.cfg, 1, p + 1).merge_in_o_proj == 0
    print(f"  deterministic", flush=True)
    a = _step(case, p, tok)
    b = _step(case, p, tok)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[2], b[2]) and a[1] == b[1]
    assert np.array_equal(a[0], logits2) and np.array_equal(a[2], layer_out2)


@pytest.mark.timeout(300)
def test_o_proj_by_head_slices_graph_replay(monkeypatch):
    """The head-sliced step captured in a HIP graph and replayed several times, with
    eager work and synchronisations in between: every replay matches the eager
    result to float32 rounding (the slices' atomic additions may come in another
    order) with the same token."""
    monkeypatch.delenv("QD_O_HEADS", raising=False)
    monkeypatch.delenv("QD_DETERMINISTIC", raising=False)
    sh = SHAPES["hd128_qknorm"]
    p = 1999
    case = make_case(sh, np.array([p], np.int32), seed=77, extra=2)
    assert Q.qd_decode_plan(case.runner.cfg, 1, p + 1).merge_in_o_proj == 2
    ctx = np.array([p], np.int32)
    pos = dev_i32(ctx)
    tok = dev_i32(synth.make_tokens(1, sh.vocab, seed=77))
    logits = torch.empty(1, sh.vocab, device="cuda")
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")

    def step():
        case.runner.step(ctx, pos, tokens=tok, logits=logits, next_tokens=nxt, stream=torch.cuda.current_stream())

    step()
    torch.cuda.synchronize()
    ref_logits, ref_next = logits.clone(), nxt.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        logits.fill_(float("nan"))
        nxt.fill_(-1)
        junk = torch.randn(1000, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        print(f"replay {i}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert not torch.isnan(logits).any(), i
        assert rel_err(logits.cpu().numpy(), ref_logits.cpu().numpy().astype(np.float64)) <= 1e-5, i
        assert torch.equal(nxt, ref_next), i
    del junk
