"""GPU parity of the int8 weight path (nanoinfer page, phase 6: per-output-channel
symmetric int8, half away from zero, norms and biases unquantized) against the
oracle.

* qd_quantize_rows_int8: codes and scales bit-exact against oracle.quant on
  random bf16 and float32 matrices, including planted ties.
* qd_decode_step with w_dtype = QD_I8 at batch 1 and at batches of 2..16 (the
  batched projections on the vector ALUs): the GPU runs the int8 codes with their
  row scales; the oracle runs the same codes dequantized (the page's "simulated
  INT8", the same function). Tolerance 2e-3 max rel err per tensor, as for bf16
  weights (the KV cache is bf16 on both sides; what differs is float32
  accumulation against float64); greedy tokens identical.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle.numerics import f32_to_bf16_bits
from oracle.quant import quantize_rows_int8, quantized_model
from oracle.qwen2 import OracleWeights, decode_step
from workloads import shapes as S
from workloads import synth
from tests._gpu_setup import make_case, dev_i32, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


SMALL_I8 = S.ModelShape(n_layers=2, hidden=144, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=272,
                        vocab=1000, w_dtype="i8")


def _quantize_on_gpu(host: np.ndarray):
    from decode_step_amd.runner import quantize_int8
    if host.dtype == np.uint16:
        t = torch.from_numpy(host.view(np.int16).copy()).view(torch.bfloat16).cuda()
    else:
        t = torch.from_numpy(host.copy()).cuda()
    q, s = quantize_int8(t)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantizer_bit_exact(dtype):
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((300, 272)) * 0.02).astype(np.float32)
    # planted ties: rows with max 127 * 2^-7 and elements at (k + 1/2) * 2^-7, exact
    # in float32 and bf16, whose quotients land exactly on halves
    for r in range(0, 300, 37):
        w[r, :] = (rng.integers(-126, 126, 272) + 0.5) * 2.0 ** -7
        w[r, 5] = 127 * 2.0 ** -7
    w[11] = 0.0                                         # a zero row
    w[12, 3] = 1e-3                                     # a row with one nonzero
    w[12, np.arange(272) != 3] = 0.0
    host = f32_to_bf16_bits(w) if dtype == "bf16" else w
    qg, sg = _quantize_on_gpu(host)
    qo, so = quantize_rows_int8(host)
    assert np.array_equal(sg, so)
    assert np.array_equal(qg, qo), np.argwhere(qg != qo)[:5]


def _run(case, pos, tok):
    sh = case.shape
    B = len(pos)
    logits = torch.full((B, sh.vocab), float("nan"), device="cuda")
    nxt = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    layer_out = torch.full((sh.n_layers, B, sh.hidden), float("nan"), device="cuda")
    case.runner.step(np.asarray(pos, np.int32), dev_i32(pos), tokens=dev_i32(tok), logits=logits,
                     next_tokens=nxt, layer_out=layer_out)
    torch.cuda.synchronize()
    return logits, nxt, layer_out


def _int8_case(shape, ctx, seed, extra=4):
    from decode_step_amd.runner import DecodeRunner, quantize_weights_int8
    case = make_case(shape, ctx, seed=seed, extra=extra, random_order=True)
    wq = quantize_weights_int8(case.w)
    torch.cuda.synchronize()
    case.runner = DecodeRunner(shape, wq, case.kv.k, case.kv.v, case.kv.block_table, max_batch=len(ctx),
                               max_ctx=int(np.max(ctx)) + extra + 1)
    deq, codes = quantized_model(case.host_w)
    # the codes the GPU runs are the oracle's codes
    for l in range(shape.n_layers):
        q, s = codes["layers"][l]["w_down"]
        assert np.array_equal(wq["layers"][l]["w_down"].cpu().numpy(), q)
        assert np.array_equal(wq["layers"][l]["s_down"].cpu().numpy(), s)
    assert np.array_equal(wq["embed"].cpu().numpy(), codes["embed"][0])
    case.w_q = wq
    return case, deq


@pytest.mark.parametrize("ctx0", [0, 37, 130])
def test_small_int8_decode_step(ctx0):
    ctx = np.array([ctx0], np.int32)
    case, deq = _int8_case(SMALL_I8, ctx, seed=41 + ctx0)
    tok = synth.make_tokens(1, SMALL_I8.vocab, seed=41 + ctx0)
    logits, nxt, layer_out = _run(case, ctx, tok)
    ow = OracleWeights(SMALL_I8, deq, cache_layers=True)
    ref = decode_step(SMALL_I8, ow, case.k_host, case.v_host, case.kv.block_table, ctx, tokens=tok)
    assert rel_err(logits.cpu().numpy(), ref.logits) <= 2e-3
    assert rel_err(layer_out.cpu().numpy(), ref.layer_out) <= 2e-3
    assert int(nxt.cpu()[0]) == int(ref.next_tokens[0])


def _cache_matches(case):
    from tests._gpu_setup import kv_matches
    return all(kv_matches(dev, host) for l in range(case.shape.n_layers)
               for dev, host in ((case.kv.k[l], case.k_host[l]), (case.kv.v[l], case.v_host[l])))


@pytest.mark.parametrize("ctx_list", [[5, 9], [0, 17, 64, 130, 33], [3 * b + 1 for b in range(16)]])
def test_small_int8_batched_decode_step(ctx_list):
    """Batches of 2..16 with ragged positions (0, on and around page edges): every
    layer's output and the logits within 2e-3, tokens identical, the new K/V stored
    within one bf16 step of the oracle's."""
    ctx = np.array(ctx_list, np.int32)
    B = len(ctx)
    case, deq = _int8_case(SMALL_I8, ctx, seed=60 + B)
    tok = synth.make_tokens(B, SMALL_I8.vocab, seed=60 + B)
    print(f"int8 batch {B} ctx {ctx_list}", flush=True)
    logits, nxt, layer_out = _run(case, ctx, tok)
    ow = OracleWeights(SMALL_I8, deq, cache_layers=True)
    ref = decode_step(SMALL_I8, ow, case.k_host, case.v_host, case.kv.block_table, ctx, tokens=tok)
    assert rel_err(logits.cpu().numpy(), ref.logits) <= 2e-3
    for l in range(SMALL_I8.n_layers):
        assert rel_err(layer_out[l].cpu().numpy(), ref.layer_out[l]) <= 2e-3, l
    assert list(nxt.cpu().numpy()) == list(ref.next_tokens)
    assert _cache_matches(case)


def test_int8_rejects_missing_scales():
    from decode_step_amd import qd as Q
    ctx = np.array([5, 9], np.int32)
    case, _ = _int8_case(SMALL_I8, ctx, seed=3)
    case.runner.layers[1].s_up = None
    st = case.runner.step(ctx, dev_i32(ctx), tokens=dev_i32([1, 2]), raise_on_error=False)
    assert st == Q.QD_EINVAL


@pytest.mark.timeout(600)
def test_qwen2_0p5b_int8_b1_past512_greedy():
    wl = S.QWEN2_0P5B_INT8_B1_PAST512
    sh = wl.shape
    ctx = np.array([wl.past], np.int32)
    case, deq = _int8_case(sh, ctx, seed=wl.seed, extra=wl.greedy_steps + 1)
    del case.w   # the bf16 draw is no longer needed on the device
    tok = synth.make_tokens(1, sh.vocab, seed=wl.seed, name="tok0")
    ow = OracleWeights(sh, deq, cache_layers=True)
    pos = ctx.copy()
    worst = 0.0
    for step in range(wl.greedy_steps):
        logits, nxt, layer_out = _run(case, pos, tok)
        ref = decode_step(sh, ow, case.k_host, case.v_host, case.kv.block_table, pos, tokens=tok)
        worst = max(worst, rel_err(logits.cpu().numpy(), ref.logits))
        if step == 0:
            for l in range(sh.n_layers):
                assert rel_err(layer_out[l].cpu().numpy(), ref.layer_out[l]) <= 2e-3, l
        assert int(nxt.cpu()[0]) == int(ref.next_tokens[0]), step
        tok = ref.next_tokens.astype(np.int32)
        pos = pos + 1
    print(f"int8 greedy: worst logits rel err {worst:.3e}")
    assert worst <= 2e-3


@pytest.mark.timeout(600)
def test_qwen2_0p5b_int8_batch4_paged():
    """The 0.5B shape with int8 rows at batch 4 over a random paged block table
    (contexts 100..700): logits and every layer's output within 2e-3, tokens
    identical, over 3 greedy steps."""
    sh = S.QWEN2_0P5B_INT8_B1_PAST512.shape
    ctx = np.array([100, 371, 700, 512], np.int32)
    case, deq = _int8_case(sh, ctx, seed=77, extra=4)
    del case.w
    tok = synth.make_tokens(4, sh.vocab, seed=77)
    ow = OracleWeights(sh, deq, cache_layers=True)
    pos = ctx.copy()
    for step in range(3):
        print(f"int8 0.5B batch 4 step {step}", flush=True)
        logits, nxt, layer_out = _run(case, pos, tok)
        ref = decode_step(sh, ow, case.k_host, case.v_host, case.kv.block_table, pos, tokens=tok)
        err = rel_err(logits.cpu().numpy(), ref.logits)
        print(f"  logits rel err {err:.3e}", flush=True)
        assert err <= 2e-3
        if step == 0:
            for l in range(sh.n_layers):
                assert rel_err(layer_out[l].cpu().numpy(), ref.layer_out[l]) <= 2e-3, l
        assert list(nxt.cpu().numpy()) == list(ref.next_tokens), step
        tok = ref.next_tokens.astype(np.int32)
        pos = pos + 1
