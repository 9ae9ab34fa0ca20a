"""Whole-forward pins for the oracle (CPU only).

The strongest pin is the transformers library's own Qwen2 (biases on q/k/v,
tied embeddings) and Qwen3 (per-head q/k RMSNorm, no bias, untied head) models,
run in float64 on tiny shapes with the same weights: the nanoinfer page used
that library as its oracle (phase 3). Planted mistakes in the oracle (wrong RoPE
pairing, GQA tiling, a dropped bias, a dropped residual, position 0 instead of
the cached length) must each break that agreement.

Also: cached decode equals an uncached pass (nanoinfer page, phase 4), paged
equals contiguous, batched equals single, and the parameter census and KV bytes
the pages print (tests/golden/qwen2_0p5b_counts.json).
"""
import json
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle.qwen2 as oq
from oracle.qwen2 import OracleWeights, decode_step, prefill_block
from workloads import shapes as S
from workloads import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / np.max(np.abs(np.asarray(b))))


# ------------------------------------------------------------------ transformers pins

def _hf_model(shape, w):
    if shape.qk_norm:
        from transformers import Qwen3Config, Qwen3ForCausalLM
        cfg = Qwen3Config(vocab_size=shape.vocab, hidden_size=shape.hidden,
                          intermediate_size=shape.ffn, num_hidden_layers=shape.n_layers,
                          num_attention_heads=shape.n_q_heads,
                          num_key_value_heads=shape.n_kv_heads, head_dim=shape.head_dim,
                          max_position_embeddings=4096, rope_theta=shape.rope_theta,
                          rms_norm_eps=shape.rms_eps, tie_word_embeddings=shape.tied,
                          attention_bias=shape.qkv_bias)
        cfg._attn_implementation = "eager"
        m = Qwen3ForCausalLM(cfg)
    else:
        from transformers import Qwen2Config, Qwen2ForCausalLM
        cfg = Qwen2Config(vocab_size=shape.vocab, hidden_size=shape.hidden,
                          intermediate_size=shape.ffn, num_hidden_layers=shape.n_layers,
                          num_attention_heads=shape.n_q_heads,
                          num_key_value_heads=shape.n_kv_heads, max_position_embeddings=4096,
                          rope_theta=shape.rope_theta, rms_norm_eps=shape.rms_eps,
                          tie_word_embeddings=shape.tied)
        cfg._attn_implementation = "eager"
        m = Qwen2ForCausalLM(cfg)
    m = m.double().eval()
    f = lambda t: torch.nn.Parameter(t.double().clone())
    with torch.no_grad():
        m.model.embed_tokens.weight = f(w["embed"])
        m.model.norm.weight = f(w["final_norm"])
        m.lm_head.weight = m.model.embed_tokens.weight if shape.tied else f(w["lm_head"])
        for l, L in enumerate(w["layers"]):
            layer = m.model.layers[l]
            a = layer.self_attn
            layer.input_layernorm.weight = f(L["attn_norm"])
            layer.post_attention_layernorm.weight = f(L["mlp_norm"])
            a.q_proj.weight, a.k_proj.weight, a.v_proj.weight = f(L["wq"]), f(L["wk"]), f(L["wv"])
            a.o_proj.weight = f(L["wo"])
            if shape.qkv_bias:
                a.q_proj.bias, a.k_proj.bias, a.v_proj.bias = f(L["bq"]), f(L["bk"]), f(L["bv"])
            if shape.qk_norm:
                a.q_norm.weight, a.k_norm.weight = f(L["q_norm"]), f(L["k_norm"])
            layer.mlp.gate_proj.weight = f(L["w_gate"])
            layer.mlp.up_proj.weight = f(L["w_up"])
            layer.mlp.down_proj.weight = f(L["w_down"])
    return m


def _oracle_token_by_token(shape, host, tokens):
    """Decode the sequence one token at a time from an empty cache; logits per position."""
    ctx = np.array([0])
    kv = synth.make_kv(shape, ctx, extra=len(tokens), fill="zeros")
    kp = [synth.to_host_bits(t) for t in kv.k]
    vp = [synth.to_host_bits(t) for t in kv.v]
    ow = OracleWeights(shape, host)
    out = []
    for t, tok in enumerate(tokens):
        r = decode_step(shape, ow, kp, vp, kv.block_table, np.array([t]), tokens=np.array([tok]))
        out.append(r.logits[0])
    return np.stack(out)


SHAPE_Q2 = S.tiny_shape(w_dtype="f32", kv_dtype="f32", rms_eps=1e-2)   # eps large enough to pin its placement
SHAPE_Q3 = S.tiny_shape(w_dtype="f32", kv_dtype="f32", qkv_bias=False, qk_norm=True, tied=False,
                        n_q_heads=6, n_kv_heads=2, head_dim=16)
TOKENS = [5, 17, 199, 0, 42, 42, 101, 7, 63, 150, 3, 88, 12, 190, 77, 31, 2, 9, 160, 45]


def _pair(shape, seed=3):
    w = synth.make_weights(shape, seed=seed, w_std=0.25)
    host = synth.weights_to_host(w)
    with torch.no_grad():
        ref = _hf_model(shape, w)(torch.tensor([TOKENS])).logits[0].numpy()
    return host, ref


@pytest.fixture(scope="module")
def qwen2_pair():
    return _pair(SHAPE_Q2)


@pytest.fixture(scope="module")
def qwen3_pair():
    return _pair(SHAPE_Q3)


def test_matches_transformers_qwen2(qwen2_pair):
    host, ref = qwen2_pair
    got = _oracle_token_by_token(SHAPE_Q2, host, TOKENS)
    assert _rel(got, ref) < 2e-6
    assert list(got.argmax(-1)) == list(ref.argmax(-1))


def test_matches_transformers_qwen3_qk_norm(qwen3_pair):
    host, ref = qwen3_pair
    got = _oracle_token_by_token(SHAPE_Q3, host, TOKENS)
    assert _rel(got, ref) < 2e-6


def _tile_attention(q, K, V, group):
    Hq = q.shape[0]
    Hkv = K.shape[1]
    out = np.empty_like(q)
    for h in range(Hq):
        g = h % Hkv
        out[h] = oq.softmax((K[:, g] @ q[h]) / np.sqrt(q.shape[1])) @ V[:, g]
    return out


MUTATIONS = {
    "rope_interleaved": lambda mp: mp.setattr(oq, "rope", oq.rope_interleaved),
    "rope_sign": lambda mp: mp.setattr(oq, "rope", _rope_neg),
    "gqa_tile": lambda mp: mp.setattr(oq, "attention_heads", _tile_attention),
    "no_score_scale": lambda mp: mp.setattr(oq, "attention_heads", lambda q, K, V, g: _orig_attn(q * np.sqrt(q.shape[1]), K, V, g)),
    "silu_as_sigmoid": lambda mp: mp.setattr(oq, "silu", oq.sigmoid),
    "eps_outside_sqrt": lambda mp: mp.setattr(oq, "rms_norm", lambda x, g, e: np.asarray(x) / (np.sqrt(np.mean(np.square(x), -1, keepdims=True)) + e) * g),
    "linear_drops_bias": lambda mp: mp.setattr(oq, "linear", lambda w, x, b=None: _orig_linear(w, x, None)),
}
_orig_attn = oq.attention_heads
_orig_linear = oq.linear
_orig_rope = oq.rope


def _rope_neg(u, p, th):
    return _orig_rope(u, -p, th)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_break_the_pin(qwen2_pair, monkeypatch, name):
    host, ref = qwen2_pair
    MUTATIONS[name](monkeypatch)
    got = _oracle_token_by_token(SHAPE_Q2, host, TOKENS)
    assert _rel(got, ref) > 1e-4, name


def test_position_zero_instead_of_cache_length_differs():
    shape = SHAPE_Q2
    host = synth.weights_to_host(synth.make_weights(shape, seed=5, w_std=0.25))
    ctx = np.array([9])
    kv = synth.make_kv(shape, ctx, extra=4, seed=5)
    ow = OracleWeights(shape, host)

    def run(p):
        kp = [synth.to_host_bits(t).copy() for t in kv.k]
        vp = [synth.to_host_bits(t).copy() for t in kv.v]
        return decode_step(shape, ow, kp, vp, kv.block_table, np.array([p]),
                           tokens=np.array([11])).logits

    good, bad = run(9), run(0)
    assert np.all(np.isfinite(bad))
    assert _rel(bad, good) > 1e-3


# ------------------------------------------------------------------ structural identities

def test_cached_decode_equals_uncached_prefill():
    shape = replace(S.tiny_shape(w_dtype="f32", kv_dtype="f32"), n_layers=1)
    host = synth.weights_to_host(synth.make_weights(shape, seed=9, w_std=0.25, with_embed=False))
    N = 21
    X = synth.to_host_bits(synth.make_x(N, shape.hidden, seed=9))
    ow = OracleWeights(shape, host)
    kv = synth.make_kv(shape, np.array([0]), extra=N, fill="zeros")
    kp, vp = synth.to_host_bits(kv.k[0]).copy(), synth.to_host_bits(kv.v[0]).copy()
    full = prefill_block(shape, ow.layer(0), kp, vp, kv.block_table[0], 0, X)
    kp2 = [synth.to_host_bits(kv.k[0]).copy()]
    vp2 = [synth.to_host_bits(kv.v[0]).copy()]
    rows = []
    for t in range(N):
        r = decode_step(shape, ow, kp2, vp2, kv.block_table, np.array([t]), x_in=X[t:t + 1],
                        with_logits=False)
        rows.append(r.x_out[0])
    assert _rel(np.stack(rows), full) < 1e-6
    # same K in the cache after either path (prefill rounds its matrix-product operand to f32)
    assert _rel(kp2[0], kp) < 1e-6


def test_chunked_prefill_equals_one_shot():
    shape = replace(S.tiny_shape(w_dtype="f32", kv_dtype="f32"), n_layers=1)
    host = synth.weights_to_host(synth.make_weights(shape, seed=2, w_std=0.25, with_embed=False))
    N = 37
    X = synth.to_host_bits(synth.make_x(N, shape.hidden, seed=2))
    W = OracleWeights(shape, host).layer(0)
    kv = synth.make_kv(shape, np.array([0]), extra=N, fill="zeros")
    one = prefill_block(shape, W, synth.to_host_bits(kv.k[0]).copy(),
                        synth.to_host_bits(kv.v[0]).copy(), kv.block_table[0], 0, X)
    kp, vp = synth.to_host_bits(kv.k[0]).copy(), synth.to_host_bits(kv.v[0]).copy()
    parts = []
    for a, b in [(0, 5), (5, 6), (6, 20), (20, 37)]:
        parts.append(prefill_block(shape, W, kp, vp, kv.block_table[0], a, X[a:b]))
    assert _rel(np.concatenate(parts), one) < 1e-12


def test_paged_equals_contiguous():
    shape = S.tiny_shape()
    host = synth.weights_to_host(synth.make_weights(shape, seed=4))
    ctx = np.array([40, 3, 77])
    kv = synth.make_kv(shape, ctx, extra=2, seed=4, random_order=False)
    ow = OracleWeights(shape, host)
    # build a permuted pool with the same logical contents
    perm = np.random.default_rng(0).permutation(kv.num_pages)
    table2 = np.where(kv.block_table >= 0, perm[np.maximum(kv.block_table, 0)], -1).astype(np.int32)
    kc = [synth.to_host_bits(t).copy() for t in kv.k]
    vc = [synth.to_host_bits(t).copy() for t in kv.v]
    kpg, vpg = [], []
    for a, b in zip(kc, vc):
        pa, pb = np.empty_like(a), np.empty_like(b)
        pa[perm], pb[perm] = a, b
        kpg.append(pa)
        vpg.append(pb)
    tok = np.array([1, 2, 3])
    r1 = decode_step(shape, ow, kc, vc, kv.block_table, ctx, tokens=tok)
    r2 = decode_step(shape, ow, kpg, vpg, table2, ctx, tokens=tok)
    assert np.array_equal(r1.logits, r2.logits)
    assert np.array_equal(r1.layer_out, r2.layer_out)


def test_batched_equals_single():
    shape = S.tiny_shape()
    host = synth.weights_to_host(synth.make_weights(shape, seed=6))
    ctx = np.array([40, 3, 77])
    kv = synth.make_kv(shape, ctx, extra=2, seed=6, random_order=True)
    ow = OracleWeights(shape, host)
    tok = np.array([10, 20, 30])
    kp = [synth.to_host_bits(t).copy() for t in kv.k]
    vp = [synth.to_host_bits(t).copy() for t in kv.v]
    rb = decode_step(shape, ow, kp, vp, kv.block_table, ctx, tokens=tok)
    for b in range(3):
        kp1 = [synth.to_host_bits(t).copy() for t in kv.k]
        vp1 = [synth.to_host_bits(t).copy() for t in kv.v]
        r1 = decode_step(shape, ow, kp1, vp1, kv.block_table[b:b + 1], ctx[b:b + 1],
                         tokens=tok[b:b + 1])
        assert np.allclose(r1.logits[0], rb.logits[b], rtol=0, atol=1e-12 * np.abs(rb.logits).max())
        assert r1.next_tokens[0] == rb.next_tokens[b]


def test_decode_is_idempotent_at_a_position():
    shape = S.tiny_shape()
    host = synth.weights_to_host(synth.make_weights(shape, seed=8))
    ctx = np.array([30])
    kv = synth.make_kv(shape, ctx, extra=2, seed=8)
    ow = OracleWeights(shape, host)
    kp = [synth.to_host_bits(t).copy() for t in kv.k]
    vp = [synth.to_host_bits(t).copy() for t in kv.v]
    r1 = decode_step(shape, ow, kp, vp, kv.block_table, ctx, tokens=np.array([4]))
    snap = [a.copy() for a in kp]
    r2 = decode_step(shape, ow, kp, vp, kv.block_table, ctx, tokens=np.array([4]))
    assert np.array_equal(r1.logits, r2.logits)
    assert all(np.array_equal(a, b) for a, b in zip(snap, kp))


def test_fused_norm_into_gemv_and_concat_qkv():
    shape = S.QWEN2_0P5B
    rng = np.random.default_rng(0)
    D = shape.hidden
    x = rng.standard_normal(D)
    g = 1 + 0.02 * rng.standard_normal(D)
    Wq = 0.02 * rng.standard_normal((shape.q_dim, D))
    Wk = 0.02 * rng.standard_normal((shape.kv_dim, D))
    Wv = 0.02 * rng.standard_normal((shape.kv_dim, D))
    unfused = np.concatenate([oq.linear(W, oq.rms_norm(x, g, 1e-6)) for W in (Wq, Wk, Wv)])
    r = 1.0 / np.sqrt(np.sum(x * x) / D + 1e-6)
    fused = r * oq.linear(np.concatenate([Wq, Wk, Wv]), g * x)
    assert _rel(fused, unfused) < 1e-13


# ------------------------------------------------------------------ page-printed counts

def test_parameter_census_and_kv_bytes_match_the_pages():
    gold = json.load(open(os.path.join(GOLDEN, "qwen2_0p5b_counts.json")))
    c = S.QWEN2_0P5B.param_counts()
    assert c["total"] == gold["params_total"]
    assert c["embeddings"] == gold["params_embeddings"]
    assert c["mlp"] == gold["params_mlp"]
    assert c["attention"] == gold["params_attention"]
    assert c["norms"] == gold["params_norms"]
    sh = S.QWEN2_0P5B
    kv_f32 = sh.n_layers * 2 * sh.n_kv_heads * sh.head_dim * 4
    assert kv_f32 == gold["kv_bytes_per_token_f32"] == gold["fused_bytes_past_coeff"]
    assert sh.n_layers * 2 * sh.n_q_heads * sh.head_dim * 4 == gold["kv_bytes_per_token_f32_without_gqa"]
    # weights read once in fp32 plus the logits write sit within 4 KB of the page's constant term
    const = c["total"] * 4 + sh.vocab * 4
    assert 0 <= gold["fused_bytes_const"] - const < 4096
    seq, past = 1, 17
    total = 5376 * past * seq + 5376 * seq * seq + 24576 * past + 2644488 * seq + gold["fused_bytes_const"]
    assert round(total / 1e9, 4) == gold["fused_bytes_seq1_past17_gb"]


# ------------------------------------------------------------------ prefill bf16 operand rounding

def _bf16_exact(a) -> bool:
    """Every value is a bf16 number: float32-exact with the low 16 bits of its
    float32 pattern zero (read off the bits, not through the oracle's rounding)."""
    a = np.asarray(a, dtype=np.float64)
    f = a.astype(np.float32)
    return bool(np.all(f.astype(np.float64) == a) and np.all((f.view(np.uint32) & 0xFFFF) == 0))


def _prefill_case(w_dtype, seed=4, N=9, start=3):
    shape = replace(S.tiny_shape(w_dtype="bf16", kv_dtype="bf16"), n_layers=1)
    host = synth.weights_to_host(synth.make_weights(shape, seed=seed, w_std=0.25, with_embed=False))
    W = OracleWeights(shape, host).layer(0)
    kv = synth.make_kv(shape, np.array([start]), extra=N, seed=seed)
    X = synth.to_host_bits(synth.make_x(N, shape.hidden, seed=seed))
    run_shape = replace(shape, w_dtype=w_dtype)
    kp, vp = synth.to_host_bits(kv.k[0]).copy(), synth.to_host_bits(kv.v[0]).copy()
    return prefill_block(run_shape, W, kp, vp, kv.block_table[0], start, X, return_operands=True)


def test_prefill_bf16_operands_are_rounded_to_nearest():
    """The bf16 prefill rounds exactly the four activation operands of its matrix
    products (normed input, attention context, second normed input, SwiGLU output)
    to bf16, each to the nearest bf16 of the value the float32 form computes."""
    _, ob = _prefill_case("bf16")
    _, of = _prefill_case("f32")
    for name in ("n", "ctx", "n2", "h"):
        assert _bf16_exact(ob[name]), name
        assert not _bf16_exact(of[name]), name
    # the first operand has no rounded input upstream: nearest bf16 of the float32 form
    ulp_half = np.ldexp(1.0, np.frexp(np.abs(of["n"]))[1] - 9)
    assert np.all(np.abs(ob["n"] - of["n"]) <= ulp_half * (1 + 1e-6))
    # later operands inherit the first rounding: within a few bf16 steps of the float32 form
    for name in ("ctx", "n2", "h"):
        assert _rel(ob[name], of[name]) < 2e-2, name


def test_prefill_q_and_residual_are_not_rounded():
    """q after RoPE and the residual stream stay unrounded in the bf16 prefill."""
    _, ob = _prefill_case("bf16")
    assert not _bf16_exact(ob["q"])
    assert not _bf16_exact(ob["x_mid"])


def test_prefill_rounding_pin_catches_a_dropped_rounding(monkeypatch):
    """Planted mistake: with the bf16 rounding replaced by the float32 one, the
    operand check above fails."""
    monkeypatch.setattr(oq, "round_bf16", oq.round_f32)
    _, ob = _prefill_case("bf16")
    assert not _bf16_exact(ob["n"])


def test_prefill_bf16_branch_equals_f32_branch_on_bf16_exact_data():
    """On a block whose operands are bf16 numbers before any rounding (x of
    entries +-2^-3 with eps 0, so the normed input is +-g exactly; one token at
    position 0, so the context is the stored v; o_proj and up rows zero, so the
    second normed input is +-g_mlp and the SwiGLU output 0), the bf16 and float32
    branches agree exactly."""
    shape = replace(S.tiny_shape(w_dtype="bf16", kv_dtype="bf16"), n_layers=1, rms_eps=0.0)
    host = synth.weights_to_host(synth.make_weights(shape, seed=6, w_std=0.25, with_embed=False))
    W = dict(OracleWeights(shape, host).layer(0))
    W["wo"] = np.zeros_like(W["wo"])
    W["w_up"] = np.zeros_like(W["w_up"])
    rng = np.random.default_rng(6)
    X = np.where(rng.random((1, shape.hidden)) < 0.5, -0.125, 0.125)
    outs = []
    for wd in ("bf16", "f32"):
        kv = synth.make_kv(shape, np.array([0]), extra=1, fill="zeros")
        kp, vp = synth.to_host_bits(kv.k[0]).copy(), synth.to_host_bits(kv.v[0]).copy()
        out, ops = prefill_block(replace(shape, w_dtype=wd), W, kp, vp, kv.block_table[0], 0, X,
                                 return_operands=True)
        for name in ("n", "ctx", "n2", "h"):
            assert _bf16_exact(ops[name]), (wd, name)
        outs.append((out, ops))
    assert np.array_equal(outs[0][0], outs[1][0])
    for name in ("n", "ctx", "n2", "h", "q"):
        assert np.array_equal(outs[0][1][name], outs[1][1][name]), name
