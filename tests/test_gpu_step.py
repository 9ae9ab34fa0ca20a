"""GPU parity of the batch-1 one-launch step kernel (qd_decode_step with
QD_STEP_KERNEL=1, through the C ABI) against the fp64 CPU oracle.

The step kernel computes the same forward as the per-op launch path (the
pre-norm Qwen2 block, the new token's K/V stored before it attends, split
attention merged by the online-softmax rule), so it is held to the same bars:
max |gpu - ref| / max |ref| <= 2e-3 for bf16 weights and KV, identical greedy
token ids, and the appended K/V within one bf16 step of the oracle's. Each test
also checks, through the library's launch timing, that the step kernel ran
(an ineligible call falls back to the per-op path silently).

Shapes: the 0.5B layer width with 2 and 4 layers and a narrow vocabulary at
positions 0, 15, 16, 300 and 2000 (one to 32 pages per split, ragged last
split, positions on both sides of a page boundary), a q/k-norm variant without
q/k/v bias, the hidden-state entry (x_in in, x_out out, no lm_head), and the
full 24-layer 0.5B step at past 512 with 8 greedy steps.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from decode_step_amd import qd as Q
from oracle.qwen2 import OracleWeights, decode_step
from workloads import shapes as S
from workloads import synth
from tests._gpu_setup import make_case, dev_i32, rel_err, kv_matches, check_argmax_tie

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _step_kernel_on(monkeypatch):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    monkeypatch.setenv("QD_STEP_KERNEL", "1")
    Q.qd_profile_enable(1 << Q.QD_K_STEP)
    yield
    Q.qd_profile_enable(0)
    Q.qd_profile_reset()


def _step_launches() -> int:
    n, _ = Q.qd_profile_read(Q.QD_K_STEP)
    return n


def _cache_matches(case):
    return all(kv_matches(dev, host) for l in range(case.shape.n_layers)
               for dev, host in ((case.kv.k[l], case.k_host[l]), (case.kv.v[l], case.v_host[l])))


def _check_one(shape, pos, seed=0, tol=2e-3):
    ctx = np.array([pos], np.int32)
    case = make_case(shape, ctx, seed=seed, random_order=True)
    tok = synth.make_tokens(1, shape.vocab, seed=seed + 7, name="tok")
    logits = torch.full((1, shape.vocab), float("nan"), device="cuda")
    nxt = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    layer_out = torch.full((shape.n_layers, 1, shape.hidden), float("nan"), device="cuda")
    x_out = torch.full((1, shape.hidden), float("nan"), device="cuda")
    before = _step_launches()
    case.runner.step(ctx, dev_i32(ctx), tokens=dev_i32(tok), logits=logits, next_tokens=nxt, x_out=x_out,
                     layer_out=layer_out)
    torch.cuda.synchronize()
    assert _step_launches() == before + 1, "the step kernel did not run"
    ow = OracleWeights(shape, case.host_w, cache_layers=True)
    ref = decode_step(shape, ow, case.k_host, case.v_host, case.kv.block_table, ctx, tokens=tok)
    e = rel_err(logits.cpu().numpy(), ref.logits)
    print(f"layers {shape.n_layers} pos {pos}: logits rel err {e:.3e}")
    assert e <= tol
    for l in range(shape.n_layers):
        assert rel_err(layer_out[l].cpu().numpy(), ref.layer_out[l]) <= tol, l
    assert rel_err(x_out.cpu().numpy(), ref.layer_out[-1]) <= tol
    assert int(nxt.cpu()[0]) == int(ref.next_tokens[0])
    assert _cache_matches(case)


NARROW = replace(S.QWEN2_0P5B, n_layers=2, vocab=4096)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("pos", [0, 15, 16, 300, 2000])
def test_step_kernel_two_layers(pos):
    _check_one(NARROW, pos, seed=pos)


@pytest.mark.timeout(300)
def test_step_kernel_four_layers_qk_norm_no_bias():
    sh = replace(S.QWEN2_0P5B, n_layers=4, vocab=4096, qkv_bias=False, qk_norm=True)
    _check_one(sh, 517, seed=3)


@pytest.mark.timeout(300)
def test_step_kernel_hidden_state_in_and_out():
    sh = replace(S.QWEN2_0P5B, n_layers=2, vocab=4096)
    ctx = np.array([129], np.int32)
    case = make_case(sh, ctx, seed=5)
    x_in = synth.make_x(1, sh.hidden, seed=5, device="cuda")
    x_out = torch.full((1, sh.hidden), float("nan"), device="cuda")
    before = _step_launches()
    case.runner.step(ctx, dev_i32(ctx), x_in=x_in, x_out=x_out)
    torch.cuda.synchronize()
    assert _step_launches() == before + 1
    ow = OracleWeights(sh, case.host_w, cache_layers=True)
    ref = decode_step(sh, ow, case.k_host, case.v_host, case.kv.block_table, ctx,
                      x_in=x_in.cpu().numpy().astype(np.float64), with_logits=False)
    assert rel_err(x_out.cpu().numpy(), ref.layer_out[-1]) <= 2e-3
    assert _cache_matches(case)


@pytest.mark.timeout(300)
def test_step_kernel_matches_per_op_path(monkeypatch):
    """Both batch-1 paths on the same inputs (two copies of one seeded case): each
    within the bf16 bar of the other, and the same token."""
    sh = replace(S.QWEN2_0P5B, n_layers=3, vocab=8192)
    ctx = np.array([700], np.int32)
    outs = []
    for flag in ("1", "0"):
        monkeypatch.setenv("QD_STEP_KERNEL", flag)
        case = make_case(sh, ctx, seed=11)
        tok = synth.make_tokens(1, sh.vocab, seed=12, name="tok")
        lg = torch.empty(1, sh.vocab, device="cuda")
        nx = torch.empty(1, dtype=torch.int32, device="cuda")
        case.runner.step(ctx, dev_i32(ctx), tokens=dev_i32(tok), logits=lg, next_tokens=nx)
        torch.cuda.synchronize()
        outs.append((lg.cpu().numpy(), int(nx.cpu()[0])))
        del case
    assert rel_err(outs[0][0], outs[1][0]) <= 2e-3
    assert outs[0][1] == outs[1][1]


@pytest.mark.timeout(900)
def test_step_kernel_qwen2_0p5b_past512_greedy():
    wl = S.QWEN2_0P5B_B1_PAST512
    sh = wl.shape
    steps = 8
    ctx = np.array([wl.past], np.int32)
    case = make_case(sh, ctx, seed=wl.seed, extra=steps + 1)
    tok0 = synth.make_tokens(1, sh.vocab, seed=wl.seed, name="tok0")
    ow = OracleWeights(sh, case.host_w, cache_layers=True)
    pos = ctx.copy()
    tok_d = dev_i32(tok0)
    ref_tok = tok0
    gpu_tokens, ref_tokens, worst = [], [], 0.0
    before = _step_launches()
    for step in range(steps):
        lg = torch.empty(1, sh.vocab, device="cuda")
        nx = torch.empty(1, dtype=torch.int32, device="cuda")
        lo = torch.empty(sh.n_layers, 1, sh.hidden, device="cuda") if step == 0 else None
        case.runner.step(pos, dev_i32(pos), tokens=tok_d, logits=lg, next_tokens=nx, layer_out=lo)
        r = decode_step(sh, ow, case.k_host, case.v_host, case.kv.block_table, pos, tokens=ref_tok)
        torch.cuda.synchronize()
        worst = max(worst, rel_err(lg.cpu().numpy(), r.logits))
        if lo is not None:
            for l in range(sh.n_layers):
                assert rel_err(lo[l].cpu().numpy(), r.layer_out[l]) <= 2e-3, l
        gpu_tokens.append(int(nx.cpu()[0]))
        ref_tokens.append(int(r.next_tokens[0]))
        tok_d = nx
        ref_tok = np.array(ref_tokens[-1:], np.int32)
        pos = pos + 1
    print(f"step kernel, {steps} greedy steps: worst logits rel err {worst:.3e}; tokens {gpu_tokens}")
    assert _step_launches() == before + steps
    assert gpu_tokens == ref_tokens
    assert worst <= 2e-3
    assert _cache_matches(case)


@pytest.mark.timeout(300)
def test_step_kernel_argmax_tie_takes_the_lower_index():
    sh = replace(S.QWEN2_0P5B, n_layers=2, vocab=5000)
    ctx = np.array([40], np.int32)
    case = make_case(sh, ctx, seed=23)
    before = _step_launches()
    check_argmax_tie(case, ctx, synth.make_tokens(1, sh.vocab, seed=24, name="tie"))
    assert _step_launches() == before + 3
