"""GPU parity of qd_sample (nanoinfer page, phase 5 sampler) against oracle.sampler.

Tokens must be identical. A row whose decision sits within 1e-5 of a rounding
boundary (the float32 running sum next to the top-p cut against 1 - p, or the
chosen token's running value against u * total) may land on either side: the
GPU's exp and its tree-summed normaliser differ from numpy's in the last bits.
Such a row must still return one of the top-k candidates; every test reports how
many rows were exact.
"""
import numpy as np
import pytest
import torch

from oracle.qwen2 import argmax_first
from oracle.sampler import sample_row

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _gpu(logits: np.ndarray, T, k, p, u):
    from decode_step_amd.runner import sample
    lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
    uu = torch.from_numpy(np.ascontiguousarray(u, np.float32)).cuda() if u is not None else None
    t = sample(lg, T, k, p, uu)
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("T,k,p", [(0.7, 20, 0.8), (1.0, 1024, 0.95), (0.5, 5, 1.0), (1.3, 256, 0.5),
                                   (2.0, 1000, 0.999)])
def test_sample_matches_oracle(T, k, p):
    rng = np.random.default_rng(int(T * 100) + k)
    B, V = 16, 151936
    logits = (rng.standard_normal((B, V)) * 3.0).astype(np.float32)
    u = rng.random(B).astype(np.float32)
    got = _gpu(logits, T, k, p, u)
    exact = 0
    for b in range(B):
        d = sample_row(logits[b], T, k, p, float(u[b]))
        if got[b] == d.token:
            exact += 1
            continue
        assert min(d.cut_margin, d.draw_margin) < 1e-5, (b, got[b], d.token)
        kth = np.sort(logits[b])[::-1][min(k, V) - 1]
        assert logits[b][got[b]] >= kth
    print(f"T={T} k={k} p={p}: {exact}/{B} rows identical")
    assert exact >= B - 1


def test_greedy_is_the_argmax():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((16, 151936)).astype(np.float32)
    logits[3, [10, 20000]] = 99.0                  # a tie: the lower index
    got = _gpu(logits, 0.0, 20, 0.8, None)
    assert got.tolist() == argmax_first(logits).tolist()


def test_page_examples():
    eq = np.zeros((3, 100), np.float32)            # 100 equiprobable tokens, p = 0.5: 50 kept
    got = _gpu(eq, 1.0, 100, 0.5, np.array([0.0, 0.999, 0.5], np.float32))
    assert got.tolist() == [sample_row(eq[0], 1.0, 100, 0.5, u).token for u in (0.0, 0.999, 0.5)]
    assert got[0] == 50 and got[1] == 99
    ties = np.array([[1.0, 1.0, 0.0, 0.0]] * 3, np.float32)   # the stable sort keeps index 1
    assert _gpu(ties, 1.0, 4, 0.05, np.array([0.0, 0.5, 0.99], np.float32)).tolist() == [1, 1, 1]


def test_top_k_boundary_ties():
    lg = np.array([[5.0, 4.0, 4.0, 4.0, 1.0]] * 4, np.float32)
    u = np.array([0.0, 0.4, 0.8, 0.999], np.float32)
    got = _gpu(lg, 1.0, 2, 1.0, u)
    assert got.tolist() == [sample_row(lg[0], 1.0, 2, 1.0, float(x)).token for x in u]
    assert set(got.tolist()) <= {0, 1, 2, 3}
    flat = np.zeros((3, 4096), np.float32)         # 4096 logits tie at the boundary: every one a candidate
    u = np.array([0.5, 0.0, 0.999], np.float32)
    got = _gpu(flat, 1.0, 10, 0.9, u)
    assert got.tolist() == [sample_row(flat[0], 1.0, 10, 0.9, float(x)).token for x in u]


@pytest.mark.parametrize("T,k,p", [(1.0, 10, 0.9), (0.7, 5, 0.5), (1.0, 64, 1.0), (1.5, 3, 0.3)])
def test_more_boundary_ties_than_candidate_slots(T, k, p):
    """Thousands of logits tie at the k-th largest value (more than the 2048
    candidate slots in LDS), a few lie above it: the top-p cut may fall inside the
    tied group (then the draw reads the row in token order) or among the ones above
    (then the usual path runs over those); tokens as the oracle's."""
    rng = np.random.default_rng(int(T * 10) + k)
    B, V = 8, 151936
    logits = np.full((B, V), -4.0, np.float32)
    exact = 0
    for b in range(B):
        tied = rng.choice(V, size=3000 + 500 * b, replace=False)
        logits[b, tied] = 1.0
        above = rng.choice(np.setdiff1d(np.arange(V), tied), size=k - 1, replace=False)
        logits[b, above] = (1.5 + 2.0 * rng.random(k - 1) * (b % 3)).astype(np.float32)
    u = rng.random(B).astype(np.float32)
    got = _gpu(logits, T, k, p, u)
    for b in range(B):
        d = sample_row(logits[b], T, k, p, float(u[b]))
        if got[b] == d.token:
            exact += 1
            continue
        assert min(d.cut_margin, d.draw_margin) < 1e-5, (b, got[b], d.token)
        assert logits[b][got[b]] >= 1.0
    print(f"T={T} k={k} p={p}: {exact}/{B} rows identical")
    assert exact >= B - 1
