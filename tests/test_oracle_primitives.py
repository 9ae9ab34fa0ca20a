"""Pins for the oracle's primitives against closed forms, invariants, exact brute
force and library special cases (CPU only).

Sources: RMSNorm, SiLU, RoPE half-split, GQA repeat, causal j <= i (nanoinfer
page, phase 3); sigmoid select (nanoinfer page, phase 7); online softmax and the
split merge as monoids (Tang page, section 2.2 and Table 1).
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle.qwen2 import (rms_norm, linear, silu, sigmoid, rope, rope_interleaved, softmax,
                          attention_heads, attention_online, attention_split_merge, argmax_first)

RNG = np.random.default_rng(1234)


# ------------------------------------------------------------------ RMSNorm

@pytest.mark.parametrize("D", [1, 8, 896])
def test_rmsnorm_constant_vector(D):
    c, eps = 0.37, 1e-6
    g = 1.0 + 0.02 * RNG.standard_normal(D)
    n = rms_norm(np.full(D, c), g, eps)
    assert np.allclose(n, g * c / math.sqrt(c * c + eps), rtol=1e-15, atol=0)


def test_rmsnorm_one_hot():
    D, a, j, eps = 64, 3.0, 17, 1e-6
    g = 1.0 + 0.02 * RNG.standard_normal(D)
    x = np.zeros(D)
    x[j] = a
    n = rms_norm(x, g, eps)
    assert n[j] == pytest.approx(g[j] * a / math.sqrt(a * a / D + eps), rel=1e-15)
    assert np.count_nonzero(n) == 1


def test_rmsnorm_eps_inside_sqrt():
    # x = 0 gives 0; tiny x is damped by eps (eps inside the square root, not added to the rms)
    D, eps = 16, 1e-6
    x = np.full(D, 1e-4)
    n = rms_norm(x, np.ones(D), eps)
    assert n[0] == pytest.approx(1e-4 / math.sqrt(1e-8 + eps), rel=1e-14)


def test_rmsnorm_matches_torch():
    x = RNG.standard_normal((5, 96))
    g = 1.0 + 0.02 * RNG.standard_normal(96)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps=1e-6)
    assert np.allclose(rms_norm(x, g, 1e-6), ref.numpy(), rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------------ GEMV vs brute force

@pytest.mark.parametrize("out_f,in_f", [(3, 5), (7, 2), (13, 11)])
def test_linear_matches_integer_brute_force(out_f, in_f):
    W = RNG.integers(-8, 9, size=(out_f, in_f))
    x = RNG.integers(-8, 9, size=in_f)
    b = RNG.integers(-8, 9, size=out_f)
    want = [sum(int(W[o, i]) * int(x[i]) for i in range(in_f)) + int(b[o]) for o in range(out_f)]
    got = linear(W.astype(np.float64), x.astype(np.float64), b.astype(np.float64))
    assert got.shape == (out_f,)
    assert [int(v) for v in got] == want


def test_linear_rows():
    W = RNG.integers(-4, 5, size=(6, 4)).astype(np.float64)
    X = RNG.integers(-4, 5, size=(3, 4)).astype(np.float64)
    got = linear(W, X)
    for r in range(3):
        for o in range(6):
            assert got[r, o] == sum(W[o, i] * X[r, i] for i in range(4))


# ------------------------------------------------------------------ SiLU

def test_sigmoid_symmetry_and_silu_zero():
    z = np.concatenate([RNG.standard_normal(1000) * 10, [0.0, 800.0, -800.0]])
    assert np.allclose(sigmoid(z) + sigmoid(-z), 1.0, rtol=0, atol=1e-15)
    assert silu(np.array([0.0]))[0] == 0.0
    assert np.all(np.isfinite(silu(z)))


def test_silu_matches_library():
    z = RNG.standard_normal(5000) * 6
    assert np.allclose(silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)
    assert silu(np.array([-800.0]))[0] == pytest.approx(0.0, abs=1e-300)


# ------------------------------------------------------------------ RoPE

def test_rope_position_zero_is_identity():
    u = RNG.standard_normal((3, 64))
    assert np.array_equal(rope(u, 0, 1e6), u)


@pytest.mark.parametrize("hd,pos", [(64, 1), (64, 511), (128, 4096)])
def test_rope_preserves_pair_norms(hd, pos):
    u = RNG.standard_normal(hd)
    r = rope(u, pos, 1e6)
    h = hd // 2
    assert np.allclose(u[:h] ** 2 + u[h:] ** 2, r[:h] ** 2 + r[h:] ** 2, rtol=1e-13)


def test_rope_relative_position():
    q, k = RNG.standard_normal(64), RNG.standard_normal(64)
    d1 = rope(q, 100, 1e6) @ rope(k, 90, 1e6)
    d2 = rope(q, 1010, 1e6) @ rope(k, 1000, 1e6)
    assert d1 == pytest.approx(d2, rel=1e-11)
    d3 = rope(q, 1011, 1e6) @ rope(k, 1000, 1e6)
    assert abs(d3 - d1) > 1e-6


def test_rope_hand_worked_hd4():
    # hd = 4: pairs (0, 2) and (1, 3); angles p * theta^0 and p * theta^(-1/2)
    p, theta = 3, 1e6
    a0, a1 = p * 1.0, p * theta ** -0.5
    e0 = np.array([1.0, 0, 0, 0])
    e2 = np.array([0, 0, 1.0, 0])
    e1 = np.array([0, 1.0, 0, 0])
    assert np.allclose(rope(e0, p, theta), [math.cos(a0), 0, math.sin(a0), 0], atol=1e-16)
    assert np.allclose(rope(e2, p, theta), [-math.sin(a0), 0, math.cos(a0), 0], atol=1e-16)
    assert np.allclose(rope(e1, p, theta), [0, math.cos(a1), 0, math.sin(a1)], atol=1e-16)


def test_rope_conventions_differ_and_stay_finite():
    u = RNG.standard_normal(64)
    a, b = rope(u, 37, 1e6), rope_interleaved(u, 37, 1e6)
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b))
    assert np.max(np.abs(a - b)) > 1e-2
    assert np.linalg.norm(a) == pytest.approx(np.linalg.norm(b), rel=1e-12)


# ------------------------------------------------------------------ softmax / attention

def test_softmax_rows_sum_to_one_and_shift_invariance():
    s = RNG.standard_normal((7, 513)) * 5
    p = softmax(s)
    assert np.allclose(p.sum(-1), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(softmax(s + 123.0), p, rtol=1e-12, atol=0)
    assert np.allclose(p, scipy.special.softmax(s, axis=-1), rtol=1e-13, atol=0)


def test_one_token_attention_returns_v_exactly():
    q = RNG.standard_normal((14, 64))
    K = RNG.standard_normal((1, 2, 64))
    V = RNG.standard_normal((1, 2, 64))
    out = attention_heads(q, K, V, 7)
    for h in range(14):
        assert np.array_equal(out[h], V[0, h // 7])


def test_identical_keys_average_values():
    q = RNG.standard_normal((4, 16))
    K = np.repeat(RNG.standard_normal((1, 2, 16)), 9, axis=0)
    V = RNG.standard_normal((9, 2, 16))
    out = attention_heads(q, K, V, 2)
    for h in range(4):
        assert np.allclose(out[h], V[:, h // 2].mean(0), rtol=1e-13)


def test_gqa_repeats_not_tiles():
    Hq, Hkv, T, hd = 14, 2, 5, 8
    q = RNG.standard_normal((Hq, hd))
    K = RNG.standard_normal((T, Hkv, hd))
    V = np.zeros((T, Hkv, hd))
    for g in range(Hkv):
        V[:, g, :] = g + 1.0
    out = attention_heads(q, K, V, Hq // Hkv)
    assert [int(round(out[h, 0])) for h in range(Hq)] == [1] * 7 + [2] * 7


def test_attention_matches_torch_sdpa_with_repeated_kv():
    Hq, Hkv, T, hd = 8, 2, 33, 16
    q = RNG.standard_normal((Hq, hd))
    K = RNG.standard_normal((T, Hkv, hd))
    V = RNG.standard_normal((T, Hkv, hd))
    grp = Hq // Hkv
    Kr = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(grp, dim=0)   # [Hq, T, hd]
    Vr = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(grp, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, :], Kr, Vr)[:, 0, :]
    assert np.allclose(attention_heads(q, K, V, grp), ref.numpy(), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("T", [1, 2, 17, 300])
def test_online_equals_two_pass(T):
    q = RNG.standard_normal(64) * 2
    K = RNG.standard_normal((T, 64))
    V = RNG.standard_normal((T, 64))
    two = attention_heads(q[None], K[:, None, :], V[:, None, :], 1)[0]
    assert np.allclose(attention_online(q, K, V), two, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("T,chunk", [(1, 16), (16, 16), (17, 16), (513, 64), (4097, 256)])
def test_split_merge_equals_single_pass(T, chunk):
    q = RNG.standard_normal(64) * 3
    K = RNG.standard_normal((T, 64))
    V = RNG.standard_normal((T, 64))
    two = attention_heads(q[None], K[:, None, :], V[:, None, :], 1)[0]
    assert np.allclose(attention_split_merge(q, K, V, chunk), two, rtol=1e-11, atol=1e-14)


def test_argmax_lowest_index_on_ties():
    x = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0], [-1.0, -2.0, -1.0, -3.0]])
    assert list(argmax_first(x)) == [1, 0, 0]
