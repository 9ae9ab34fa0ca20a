"""GPU parity of the batch-1 decode step whose q|k|v projection runs inside the
attention launch (the attention covers the cached positions, and the residual
product adds the new token as one more split), against the fp64 oracle, and of
the same step with the projection launch kept (QD_FUSED_QKV=0).

Shape: the Qwen2-0.5B layer (hidden 896, 14 query heads, 2 KV heads, head_dim
64, q|k|v biases), two layers, a 4096-token vocabulary. Positions: an empty past
(p = 0, the context is the new token's v), one key, and both sides of the
144-token split edges (p = 143, 144, 145, 288, 431, 576: a last split that ends
exactly at the new token, or one that holds no cached key and exits), up to 600.
Bound: 2e-3 of the largest value (bf16 weights and KV), identical greedy tokens,
stored K/V within one bf16 step of the oracle's.
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

SHAPE = replace(S.QWEN2_0P5B, n_layers=2, vocab=4096)
POSITIONS = [0, 1, 143, 144, 145, 288, 431, 576, 600]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def case():
    return make_case(SHAPE, np.array([600], np.int32), seed=11, extra=4)


def _launch_counts(fn):
    """(projection launches, attention launches) of one call of fn()."""
    mask = (1 << Q.QD_K_QKV) | (1 << Q.QD_K_ATTN)
    Q.qd_profile_reset()
    Q.qd_profile_enable(mask)
    try:
        fn()
        torch.cuda.synchronize()
        return Q.qd_profile_read(Q.QD_K_QKV)[0], Q.qd_profile_read(Q.QD_K_ATTN)[0]
    finally:
        Q.qd_profile_enable(0)
        Q.qd_profile_reset()


def _step(case, p, tok):
    sh = case.shape
    logits = torch.full((1, sh.vocab), float("nan"), device="cuda")
    nxt = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    layer_out = torch.full((sh.n_layers, 1, sh.hidden), float("nan"), device="cuda")
    pos = np.array([p], np.int32)
    counts = _launch_counts(lambda: case.runner.step(pos, dev_i32(pos), tokens=dev_i32(tok), logits=logits,
                                                     next_tokens=nxt, layer_out=layer_out))
    return logits.cpu().numpy(), int(nxt.cpu()[0]), layer_out.cpu().numpy(), counts


@pytest.mark.timeout(300)
@pytest.mark.parametrize("p", POSITIONS)
def test_fused_projection_matches_oracle(case, p, monkeypatch):
    sh = case.shape
    monkeypatch.delenv("QD_FUSED_QKV", raising=False)
    assert Q.qd_decode_plan(case.runner.cfg, 1, p + 1).fused_qkv == 1
    tok = synth.make_tokens(1, sh.vocab, seed=100 + p)
    print(f"fused q|k|v at p={p}", flush=True)
    logits, nxt, layer_out, (n_qkv, n_attn) = _step(case, p, tok)
    assert (n_qkv, n_attn) == (0, sh.n_layers)
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

    # the same step with the projection launch: the cache slot at p is rewritten by
    # the other path (its own rounding), the oracle's step stays the reference
    monkeypatch.setenv("QD_FUSED_QKV", "0")
    assert Q.qd_decode_plan(case.runner.cfg, 1, p + 1).fused_qkv == 0
    print(f"projection launch at p={p}", flush=True)
    logits2, nxt2, layer_out2, (n_qkv, n_attn) = _step(case, p, tok)
    assert (n_qkv, n_attn) == (sh.n_layers, sh.n_layers)
    assert rel_err(logits2, ref.logits) <= 2e-3
    for l in range(sh.n_layers):
        assert rel_err(layer_out2[l], ref.layer_out[l]) <= 2e-3, l
    assert nxt2 == nxt
