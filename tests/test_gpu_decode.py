"""GPU parity of the decode step (qd_decode_step through the C ABI) against the
fp64 CPU oracle, on the same seeded inputs.

Tolerances (max |gpu - ref| / max |ref| per tensor): 1e-4 for the fp32 block,
2e-3 for bf16 weights/KV; greedy token ids identical. Shapes: a small ragged
model (several GEMV tiles plus a ragged tail, positions on and around page
boundaries, position 0), the fp32 Qwen2 block at past 16, the full 24-layer
0.5B step at past 512 with a 32-step greedy run, batch 16 with per-sequence
context in [128, 4096] over a random paged block table, and the 8B-class shape
with per-head q/k RMSNorm at past 4096.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from decode_step_amd import qd as Q
from oracle.qwen2 import OracleWeights, decode_step
from workloads import shapes as S
from workloads import synth
from tests._gpu_setup import make_case, dev_i32, rel_err, guarded, canaries_intact, kv_matches, check_argmax_tie

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


SMALL = S.ModelShape(n_layers=2, hidden=136, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=264,
                     vocab=1000)


def _run_step(case, pos, tokens=None, x_in=None, want_layers=True):
    sh = case.shape
    B = len(pos)
    logits = torch.full((B, sh.vocab), float("nan"), device="cuda")
    nxt = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    layer_out = torch.full((sh.n_layers, B, sh.hidden), float("nan"), device="cuda") if want_layers else None
    x_out = torch.full((B, sh.hidden), float("nan"), device="cuda")
    tok_d = dev_i32(tokens) if tokens is not None else None
    case.runner.step(np.asarray(pos, np.int32), dev_i32(pos), tokens=tok_d, x_in=x_in,
                     logits=logits if x_in is None else None, next_tokens=nxt if x_in is None else None,
                     x_out=x_out, layer_out=layer_out)
    torch.cuda.synchronize()
    return logits, nxt, x_out, layer_out


def _oracle(case, pos, tokens=None, x_in=None, with_logits=True, cache_layers=True):
    ow = OracleWeights(case.shape, case.host_w, cache_layers=cache_layers)
    return decode_step(case.shape, ow, case.k_host, case.v_host, case.kv.block_table,
                       np.asarray(pos), tokens=tokens, x_in=x_in, with_logits=with_logits)


def _cache_matches(case):
    return all(kv_matches(dev, host) for l in range(case.shape.n_layers)
               for dev, host in ((case.kv.k[l], case.k_host[l]), (case.kv.v[l], case.v_host[l])))


# ---------------------------------------------------------------- small ragged model

@pytest.mark.parametrize("w_dtype,kv_dtype,tol", [("bf16", "bf16", 2e-3), ("f32", "f32", 1e-4),
                                                  ("bf16", "f32", 2e-3)])
def test_small_ragged_batch(w_dtype, kv_dtype, tol):
    shape = replace(SMALL, w_dtype=w_dtype, kv_dtype=kv_dtype)
    ctx = np.array([0, 15, 16, 17, 100, 255, 33], np.int32)
    case = make_case(shape, ctx, seed=11, random_order=True)
    tok = synth.make_tokens(len(ctx), shape.vocab, seed=11)
    logits, nxt, x_out, layer_out = _run_step(case, ctx, tokens=tok)
    ref = _oracle(case, ctx, tokens=tok)
    assert rel_err(logits.cpu().numpy(), ref.logits) <= tol
    assert rel_err(layer_out.cpu().numpy(), ref.layer_out) <= tol
    assert rel_err(x_out.cpu().numpy(), ref.x_out) <= tol
    assert list(nxt.cpu().numpy()) == list(ref.next_tokens)
    assert _cache_matches(case)


@pytest.mark.parametrize("batch", [2, 5, 16])
def test_batched_projections_chunked_k_wide_vocab(batch):
    """Batched decode (B > 1, bf16 weights) runs its projections on the matrix cores.
    hidden 1032 and ffn 2056 are not multiples of 32 and exceed one staged K chunk
    (2 and 3 chunks); vocab 40003 takes the wide (128-row) lm_head tiling with a
    ragged last tile; B = 5 leaves MFMA columns empty."""
    shape = replace(SMALL, n_layers=2, hidden=1032, ffn=2056, vocab=40003, n_q_heads=6,
                    n_kv_heads=2, head_dim=64)
    ctx = np.array([(37 * b + 5) % 300 for b in range(batch)], np.int32)
    case = make_case(shape, ctx, seed=31 + batch, random_order=True)
    tok = synth.make_tokens(batch, shape.vocab, seed=31 + batch)
    logits, nxt, x_out, layer_out = _run_step(case, ctx, tokens=tok)
    ref = _oracle(case, ctx, tokens=tok)
    assert rel_err(logits.cpu().numpy(), ref.logits) <= 2e-3
    assert rel_err(layer_out.cpu().numpy(), ref.layer_out) <= 2e-3
    assert rel_err(x_out.cpu().numpy(), ref.x_out) <= 2e-3
    assert list(nxt.cpu().numpy()) == list(ref.next_tokens)
    assert _cache_matches(case)


@pytest.mark.parametrize("batch", [5, 16])
def test_batched_multi_block_gate_up_and_grouped_down(batch):
    """ffn 4200 gives 263 row blocks of gate|up, more than the chip has CUs: two
    blocks per workgroup with the activation staged once (the last workgroup holds
    one block, the last block 8 rows); down (K = 4200, a ragged last k-step) takes
    groups of two row blocks over 16 K ranges."""
    shape = replace(SMALL, n_layers=2, hidden=256, ffn=4200, vocab=3001, n_q_heads=4,
                    n_kv_heads=2, head_dim=64)
    ctx = np.array([(53 * b + 7) % 400 for b in range(batch)], np.int32)
    case = make_case(shape, ctx, seed=71 + batch, random_order=True)
    tok = synth.make_tokens(batch, shape.vocab, seed=71 + batch)
    logits, nxt, x_out, layer_out = _run_step(case, ctx, tokens=tok)
    ref = _oracle(case, ctx, tokens=tok)
    assert rel_err(logits.cpu().numpy(), ref.logits) <= 2e-3
    assert rel_err(layer_out.cpu().numpy(), ref.layer_out) <= 2e-3
    assert rel_err(x_out.cpu().numpy(), ref.x_out) <= 2e-3
    assert list(nxt.cpu().numpy()) == list(ref.next_tokens)
    assert _cache_matches(case)


def test_small_qk_norm_no_bias_untied():
    shape = replace(SMALL, qkv_bias=False, qk_norm=True, tied=False, n_q_heads=8, n_kv_heads=2,
                    head_dim=128)
    ctx = np.array([3, 64, 130], np.int32)
    case = make_case(shape, ctx, seed=12, random_order=True)
    tok = synth.make_tokens(len(ctx), shape.vocab, seed=12)
    logits, nxt, _, layer_out = _run_step(case, ctx, tokens=tok)
    ref = _oracle(case, ctx, tokens=tok)
    assert rel_err(logits.cpu().numpy(), ref.logits) <= 2e-3
    assert rel_err(layer_out.cpu().numpy(), ref.layer_out) <= 2e-3
    assert list(nxt.cpu().numpy()) == list(ref.next_tokens)


def test_batched_three_block_gate_up_full_lds():
    """hidden 1024 and ffn 8200 at batch 4: gate|up takes 32-33 rows per workgroup
    (three MFMA blocks, the third mostly masked), eight k-steps per wave, and
    66 KB of LDS for the staged activation (past the default 64 KB)."""
    shape = replace(SMALL, hidden=1024, ffn=8200, vocab=2003, n_q_heads=8, n_kv_heads=2, head_dim=128)
    ctx = np.array([5, 300, 77, 1000], np.int32)
    case = make_case(shape, ctx, seed=91, random_order=True)
    tok = synth.make_tokens(len(ctx), shape.vocab, seed=91)
    logits, nxt, x_out, layer_out = _run_step(case, ctx, tokens=tok)
    ref = _oracle(case, ctx, tokens=tok)
    assert rel_err(logits.cpu().numpy(), ref.logits) <= 2e-3
    assert rel_err(layer_out.cpu().numpy(), ref.layer_out) <= 2e-3
    assert rel_err(x_out.cpu().numpy(), ref.x_out) <= 2e-3
    assert list(nxt.cpu().numpy()) == list(ref.next_tokens)
    assert _cache_matches(case)


@pytest.mark.parametrize("qkv_bias,qk_norm", [(False, True), (True, False)])
def test_batched_partial_qkv_head_dim_128(qkv_bias, qk_norm):
    """hidden 512 at batch 8 with a context past 1000: q|k|v runs as K-range
    partial products that the matrix-core attention kernel (head_dim 128) sums,
    scales by the RMSNorm factor and biases (or not) before the q/k norm and RoPE.
    The host plan confirms that path (at batch 6 and 512 keys the step takes one
    query head per workgroup on the other kernel instead)."""
    shape = replace(SMALL, hidden=512, ffn=1024, qkv_bias=qkv_bias, qk_norm=qk_norm, tied=not qk_norm,
                    n_q_heads=8, n_kv_heads=2, head_dim=128)
    ctx = np.array([0, 3, 64, 130, 511, 17, 1001, 700], np.int32)
    case = make_case(shape, ctx, seed=13, random_order=True)
    plan = Q.qd_decode_plan(case.runner.cfg, len(ctx), int(ctx.max()) + 1)
    assert plan.matrix_core_attention == 1 and plan.qkv_partials > 1
    tok = synth.make_tokens(len(ctx), shape.vocab, seed=13)
    logits, nxt, x_out, layer_out = _run_step(case, ctx, tokens=tok)
    ref = _oracle(case, ctx, tokens=tok)
    assert rel_err(logits.cpu().numpy(), ref.logits) <= 2e-3
    assert rel_err(layer_out.cpu().numpy(), ref.layer_out) <= 2e-3
    assert rel_err(x_out.cpu().numpy(), ref.x_out) <= 2e-3
    assert list(nxt.cpu().numpy()) == list(ref.next_tokens)
    assert _cache_matches(case)


def test_position_zero_returns_v():
    """One cached token (the new one): attention output is the stored v exactly, so the
    block output equals the oracle's to fp32 rounding of the GEMVs."""
    shape = replace(SMALL, n_layers=1, w_dtype="f32", kv_dtype="f32")
    case = make_case(shape, np.array([0]), seed=3)
    x = synth.make_x(1, shape.hidden, seed=3, device="cuda")
    _, _, x_out, _ = _run_step(case, [0], x_in=x)
    ref = _oracle(case, [0], x_in=synth.to_host_bits(x), with_logits=False)
    assert rel_err(x_out.cpu().numpy(), ref.x_out) <= 1e-5


@pytest.mark.parametrize("ctx_list", [[40], [40, 7]])
def test_outputs_guarded_and_deterministic(ctx_list):
    """Same position twice: idempotent. Batch 1 is bitwise deterministic (no float
    atomics on its path); batches of 2..16 add the K ranges of the residual
    projections with float atomics, so only the order of those few additions may
    vary: the two runs agree to float32 rounding (1e-5 of the largest logit, the
    last-bit differences of the residual grown over the layers)."""
    shape = SMALL
    ctx = np.array(ctx_list, np.int32)
    B = len(ctx)
    case = make_case(shape, ctx, seed=5, random_order=True)
    tok = dev_i32(synth.make_tokens(B, shape.vocab, seed=5))
    n = B * shape.vocab
    outs = []
    for _ in range(2):
        full, view = guarded(n)
        nxt = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        case.runner.step(ctx, dev_i32(ctx), tokens=tok, logits=view.view(B, shape.vocab), next_tokens=nxt)
        torch.cuda.synchronize()
        assert canaries_intact(full, n)
        assert not torch.isnan(view).any()
        outs.append((view.cpu().clone(), nxt.cpu().clone()))
    assert torch.equal(outs[0][1], outs[1][1])
    if B == 1:
        assert torch.equal(outs[0][0], outs[1][0])
    else:
        assert rel_err(outs[0][0].numpy(), outs[1][0].numpy().astype(np.float64)) <= 1e-5


def _guard(t, pad, sentinel):
    """t's values inside a larger buffer whose first and last pad elements hold the
    sentinel; returns (full, view shaped like t)."""
    n = t.numel()
    full = torch.full((n + 2 * pad,), sentinel, dtype=t.dtype, device=t.device)
    full[pad:pad + n].copy_(t.reshape(-1))
    return full, full[pad:pad + n].view(t.shape)


def _guard_intact(full, n, pad, sentinel):
    f = full.cpu()
    return bool(torch.all(f[:pad] == sentinel)) and bool(torch.all(f[pad + n:] == sentinel))


@pytest.mark.parametrize("kv_dtype,ctx_list", [("bf16", [40]), ("bf16", [40, 7, 300]), ("f32", [33, 16])])
def test_writes_stay_inside_outputs_and_pools(kv_dtype, ctx_list):
    """Canaries on both sides of logits, next_tokens, x_out, layer_out and of every
    layer's K and V page pool: a step writes none of them, every output element is
    written, and the pools then equal the oracle's (which holds the new rows only)."""
    from decode_step_amd.runner import DecodeRunner
    shape = replace(SMALL, kv_dtype=kv_dtype)
    ctx = np.array(ctx_list, np.int32)
    B, pad = len(ctx), 2048
    w = synth.make_weights(shape, seed=29, device="cuda")
    kv = synth.make_kv(shape, ctx, extra=4, seed=29, device="cuda", random_order=True)
    sent = 1024.0
    kg = [_guard(t, pad, sent) for t in kv.k]
    vg = [_guard(t, pad, sent) for t in kv.v]
    runner = DecodeRunner(shape, w, [v for _, v in kg], [v for _, v in vg], kv.block_table, max_batch=B,
                          max_ctx=int(ctx.max()) + 5)
    k_host = [synth.to_host_bits(v).copy() for _, v in kg]
    v_host = [synth.to_host_bits(v).copy() for _, v in vg]
    tok = synth.make_tokens(B, shape.vocab, seed=29)
    lg_full, lg = guarded(B * shape.vocab)
    xo_full, xo = guarded(B * shape.hidden)
    lo_full, lo = guarded(shape.n_layers * B * shape.hidden)
    nx_full = torch.full((B + 2 * pad,), 777, dtype=torch.int32, device="cuda")
    nx = nx_full[pad:pad + B]
    nx.fill_(-1)
    runner.step(ctx, dev_i32(ctx), tokens=dev_i32(tok), logits=lg.view(B, shape.vocab), next_tokens=nx,
                x_out=xo.view(B, shape.hidden), layer_out=lo.view(shape.n_layers, B, shape.hidden))
    torch.cuda.synchronize()
    assert canaries_intact(lg_full, B * shape.vocab) and canaries_intact(xo_full, B * shape.hidden)
    assert canaries_intact(lo_full, shape.n_layers * B * shape.hidden)
    nf = nx_full.cpu()
    assert bool(torch.all(nf[:pad] == 777)) and bool(torch.all(nf[pad + B:] == 777))
    for full, view in kg + vg:
        assert _guard_intact(full, view.numel(), pad, sent)
    assert not torch.isnan(lg).any() and not torch.isnan(xo).any() and not torch.isnan(lo).any()
    ow = OracleWeights(shape, synth.weights_to_host(w), cache_layers=True)
    ref = decode_step(shape, ow, k_host, v_host, kv.block_table, ctx, tokens=tok)
    assert rel_err(lg.cpu().numpy().reshape(B, -1), ref.logits) <= 2e-3
    assert list(nx.cpu().numpy()) == list(ref.next_tokens)
    assert all(kv_matches(view, host) for (_, view), host in zip(kg + vg, k_host + v_host))


@pytest.mark.parametrize("ctx_list", [[70], [70, 3, 129]])
def test_graph_replay_matches_eager(ctx_list):
    """One decode step captured in a HIP graph and replayed several times, with eager
    work and synchronisations in between: every replay equals the eager result
    (bitwise at batch 1; to float32 rounding where float atomics add the residual
    projections' K ranges), with the same tokens."""
    shape = SMALL
    ctx = np.array(ctx_list, np.int32)
    B = len(ctx)
    case = make_case(shape, ctx, seed=21, random_order=True)
    tok = dev_i32(synth.make_tokens(B, shape.vocab, seed=21))
    pos = dev_i32(ctx)
    logits = torch.empty(B, shape.vocab, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")

    def step():
        case.runner.step(ctx, pos, tokens=tok, logits=logits, next_tokens=nxt,
                         stream=torch.cuda.current_stream())

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
        g.replay()
        torch.cuda.synchronize()
        if B == 1:
            assert torch.equal(logits, ref_logits), i
        else:
            assert not torch.isnan(logits).any(), i
            assert rel_err(logits.cpu().numpy(), ref_logits.cpu().numpy().astype(np.float64)) <= 1e-5, i
        assert torch.equal(nxt, ref_next), i
    del junk


def test_kv_append_matches_oracle_rounding():
    from oracle.numerics import store_kv
    shape = replace(SMALL, n_layers=1)
    ctx = np.array([5, 31, 200], np.int32)
    case = make_case(shape, ctx, seed=9, random_order=True)
    k = torch.randn(3, shape.n_kv_heads, shape.head_dim, device="cuda")
    v = torch.randn(3, shape.n_kv_heads, shape.head_dim, device="cuda")
    case.runner.kv_append(0, ctx, dev_i32(ctx), k, v)
    torch.cuda.synchronize()
    kg = synth.to_host_bits(case.kv.k[0])
    vg = synth.to_host_bits(case.kv.v[0])
    kh, vh = k.cpu().numpy(), v.cpu().numpy()
    bt = case.kv.block_table
    for b, p in enumerate(ctx):
        pg, sl = bt[b, p // 16], p % 16
        assert np.array_equal(kg[pg, :, sl, :], store_kv(kh[b], "bf16"))
        assert np.array_equal(vg[pg, :, sl, :], store_kv(vh[b], "bf16"))


# ---------------------------------------------------------------- full-size workloads

@pytest.mark.timeout(300)
def test_qwen2_block_f32_past16():
    wl = S.QWEN2_BLOCK_F32_PAST16
    ctx = np.array([wl.past], np.int32)
    case = make_case(wl.shape, ctx, seed=wl.seed)
    x = synth.make_x(1, wl.shape.hidden, seed=wl.seed, device="cuda")
    _, _, x_out, layer_out = _run_step(case, ctx, x_in=x)
    ref = _oracle(case, ctx, x_in=synth.to_host_bits(x), with_logits=False)
    assert rel_err(x_out.cpu().numpy(), ref.x_out) <= 1e-4
    assert _cache_matches(case)


@pytest.mark.timeout(600)
def test_qwen2_0p5b_b1_past512_and_32_greedy_steps():
    wl = S.QWEN2_0P5B_B1_PAST512
    sh = wl.shape
    ctx = np.array([wl.past], np.int32)
    case = make_case(sh, ctx, seed=wl.seed, extra=wl.greedy_steps + 1)
    tok0 = synth.make_tokens(1, sh.vocab, seed=wl.seed, name="tok0")
    # step 1: full comparison of logits and every layer's output
    logits, nxt, _, layer_out = _run_step(case, ctx, tokens=tok0)
    ow = OracleWeights(sh, case.host_w, cache_layers=True)
    ref = decode_step(sh, ow, case.k_host, case.v_host, case.kv.block_table, ctx, tokens=tok0)
    assert rel_err(logits.cpu().numpy(), ref.logits) <= 2e-3
    for l in range(sh.n_layers):
        assert rel_err(layer_out[l].cpu().numpy(), ref.layer_out[l]) <= 2e-3, l
    gpu_tokens, ref_tokens = [int(nxt.cpu()[0])], [int(ref.next_tokens[0])]
    # steps 2..32: each side feeds back its own argmax
    pos = ctx.copy()
    tok_d = nxt.clone()
    lg = torch.empty(1, sh.vocab, device="cuda")
    worst = 0.0
    for step in range(1, wl.greedy_steps):
        pos = pos + 1
        nxt_d = torch.empty(1, dtype=torch.int32, device="cuda")
        case.runner.step(pos, dev_i32(pos), tokens=tok_d, logits=lg, next_tokens=nxt_d)
        r = decode_step(sh, ow, case.k_host, case.v_host, case.kv.block_table, pos,
                        tokens=np.array(ref_tokens[-1:], np.int32))
        torch.cuda.synchronize()
        worst = max(worst, rel_err(lg.cpu().numpy(), r.logits))
        gpu_tokens.append(int(nxt_d.cpu()[0]))
        ref_tokens.append(int(r.next_tokens[0]))
        tok_d = nxt_d
    print(f"32-step greedy: worst logits rel err {worst:.3e}; tokens {gpu_tokens}")
    assert gpu_tokens == ref_tokens
    assert worst <= 2e-3


@pytest.mark.timeout(600)
def test_qwen2_0p5b_b16_paged_random_ctx():
    wl = S.QWEN2_0P5B_B16_PAGED
    sh = wl.shape
    ctx = synth.make_ctx(wl.batch, None, wl.ctx_range, wl.seed)
    case = make_case(sh, ctx, seed=wl.seed, extra=wl.greedy_steps + 1, random_order=True)
    tok = synth.make_tokens(wl.batch, sh.vocab, seed=wl.seed)
    logits, nxt, _, layer_out = _run_step(case, ctx, tokens=tok)
    ow = OracleWeights(sh, case.host_w, cache_layers=True)
    ref = decode_step(sh, ow, case.k_host, case.v_host, case.kv.block_table, ctx, tokens=tok)
    assert rel_err(logits.cpu().numpy(), ref.logits) <= 2e-3
    assert rel_err(layer_out.cpu().numpy(), ref.layer_out) <= 2e-3
    assert list(nxt.cpu().numpy()) == list(ref.next_tokens)
    # a few greedy steps for all 16 sequences
    pos, tok_d, ref_tok = ctx.copy(), nxt.clone(), ref.next_tokens.copy()
    for _ in range(wl.greedy_steps - 1):
        pos = pos + 1
        nd = torch.empty(wl.batch, dtype=torch.int32, device="cuda")
        case.runner.step(pos, dev_i32(pos), tokens=tok_d, next_tokens=nd)
        r = decode_step(sh, ow, case.k_host, case.v_host, case.kv.block_table, pos, tokens=ref_tok)
        torch.cuda.synchronize()
        assert list(nd.cpu().numpy()) == list(r.next_tokens)
        tok_d, ref_tok = nd, r.next_tokens
    # every K/V the steps appended (4 per sequence, pages in random order)
    assert _cache_matches(case)


@pytest.mark.timeout(900)
def test_qwen_8b_qknorm_b1_past4096():
    wl = S.QWEN_8B_B1_PAST4096
    sh = wl.shape
    ctx = np.array([wl.past], np.int32)
    case = make_case(sh, ctx, seed=wl.seed, extra=2)
    tok = synth.make_tokens(1, sh.vocab, seed=wl.seed, name="tok0")
    logits, nxt, _, layer_out = _run_step(case, ctx, tokens=tok)
    ref = _oracle(case, ctx, tokens=tok, cache_layers=False)
    assert rel_err(logits.cpu().numpy(), ref.logits) <= 2e-3
    assert rel_err(layer_out.cpu().numpy(), ref.layer_out) <= 2e-3
    assert int(nxt.cpu()[0]) == int(ref.next_tokens[0])
    assert _cache_matches(case)


# ---------------------------------------------------------------- argmax ties


def test_argmax_tie_takes_the_lower_index():
    ctx = np.array([33], np.int32)
    case = make_case(SMALL, ctx, seed=21)
    check_argmax_tie(case, ctx, synth.make_tokens(1, SMALL.vocab, seed=22, name="tie"))
