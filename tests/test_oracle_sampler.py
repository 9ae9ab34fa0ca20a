"""Pins of the oracle's sampler (nanoinfer page, phase 5). Each is a value the page
prints or a property its definition fixes, chosen so that a plausible slip fails:
the descending top-p rule, an unstable sort, top-k dropping boundary ties, top-p
before temperature, a draw that is not the inverse CDF in token order, or a
running sum taken in another order or precision."""
import numpy as np
import pytest

from oracle.qwen2 import argmax_first
from oracle.sampler import _running, sample_row


def test_running_sum_of_the_page_example():
    # the page prints the float32 sum of fifty 1/100 probabilities
    p = np.full(100, np.float32(1.0) / np.float32(100.0), np.float32)
    assert float(_running(p)[49]) == 0.4999997913837433


def test_hundred_equiprobable_tokens_keep_fifty():
    lg = np.zeros(100, np.float32)
    d = sample_row(lg, 1.0, 100, 0.5, 0.0)
    assert d.kept.tolist() == list(range(50, 100))     # the ascending rule; ">= p" descending keeps 51
    assert sample_row(lg, 1.0, 100, 0.5, 0.0).token == 50
    assert sample_row(lg, 1.0, 100, 0.5, 0.999).token == 99


def test_stable_sort_decides_the_most_likely_of_a_tie():
    lg = np.array([1.0, 1.0, 0.0, 0.0], np.float32)
    for u in (0.0, 0.5, 0.99):
        d = sample_row(lg, 1.0, 4, 0.05, u)
        assert d.kept.tolist() == [1] and d.token == 1   # [2, 3, 0, 1]: index 1 sorts last


def test_temperature_zero_and_k_one_are_the_argmax():
    rng = np.random.default_rng(0)
    lg = rng.standard_normal(500).astype(np.float32)
    lg[[17, 300]] = lg.max() + 1.0                          # a tie at the top: lowest index
    assert sample_row(lg, 0.0, 20, 0.8, 0.7).token == int(argmax_first(lg[None])[0]) == 17
    lg2 = rng.standard_normal(500).astype(np.float32)
    for u in (0.0, 0.3, 0.99):
        assert sample_row(lg2, 0.7, 1, 0.9, u).token == int(np.argmax(lg2))
        assert sample_row(lg2, 0.7, 50, 1e-6, u).token == int(np.argmax(lg2))


def test_top_k_keeps_ties_at_the_boundary():
    lg = np.array([5.0, 4.0, 4.0, 4.0, 1.0], np.float32)
    d = sample_row(lg, 1.0, 2, 1.0, 0.5)
    assert d.kept.tolist() == [0, 1, 2, 3]


def test_draw_is_the_inverse_cdf_in_token_order():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal(64).astype(np.float32)
    p = np.exp(lg.astype(np.float64) - lg.max())
    p /= p.sum()
    cdf = np.cumsum(p)
    for i in range(64):
        u = (cdf[i] - p[i] / 2)                    # the middle of token i's interval
        assert sample_row(lg, 1.0, 64, 1.0, u).token == i


def test_temperature_acts_before_top_p():
    rng = np.random.default_rng(2)
    lg = (rng.standard_normal(1000) * 2).astype(np.float32)
    sizes = [len(sample_row(lg, t, 1000, 0.8, 0.5).kept) for t in (0.3, 0.7, 1.5, 3.0)]
    assert sizes == sorted(sizes) and sizes[0] < sizes[-1]   # hotter -> flatter -> wider nucleus
    # a nucleus cut on the raw logits and then rescaled would not change with T
    raw = len(sample_row(lg, 1.0, 1000, 0.8, 0.5).kept)
    assert sizes[0] != raw or sizes[-1] != raw


def test_top_p_alone_is_the_whole_vocabulary():
    # "top-p alone": no top-k step, so every token is a candidate; the page's
    # 100-equiprobable example keeps the same 50 without a top-k
    lg = np.zeros(100, np.float32)
    for k in (0, -1, 100, 1000):
        assert sample_row(lg, 1.0, k, 0.5, 0.0).kept.tolist() == list(range(50, 100))
    # top-p alone at p = 1 keeps every token, and the draw is the inverse CDF of the
    # full softmax: u just below the first token's probability picks token 0
    lg = np.array([0.0, np.log(3.0), np.log(6.0)], np.float32)    # probabilities 0.1, 0.3, 0.6
    assert sample_row(lg, 1.0, 0, 1.0, 0.0).kept.tolist() == [0, 1, 2]
    assert sample_row(lg, 1.0, 0, 1.0, 0.09).token == 0
    assert sample_row(lg, 1.0, 0, 1.0, 0.11).token == 1
    assert sample_row(lg, 1.0, 0, 1.0, 0.41).token == 2
    # p = 0.65, 1 - p = 0.35: of the ascending sums 0.1, 0.4, 1.0 only 0.1 is <= 0.35,
    # so token 0 alone goes
    d = sample_row(lg, 1.0, 0, 0.65, 0.0)
    assert d.kept.tolist() == [1, 2]
