"""GPU parity of qd_sample (nanoinfer page, phase 5 sampler) against oracle.sampler.

Tokens must be identical. A row whose decision sits within 1e-5 of a rounding
boundary (the float32 running sum next to the top-p cut against 1 - p, or the
chosen token's running value against u * total) may land on either side: the
GPU's exp and its tree-summed normaliser differ from numpy's in the last bits.
Such a row must still return one of the top-k candidates; every test reports how
many rows were exact.

Without top-k (top-p over the whole vocabulary) the oracle's cut is a float32
sum of up to 151,936 terms taken one at a time, and so is its draw over the kept
tokens; the GPU sums the same terms in bins and in chunked prefix sums. A float32
sum of n nonnegative terms taken one at a time is within (n - 1) 2^-24 of its
total of the exact sum, and the GPU's sums are within that too, so a row may
differ only when its cut (or draw) lies within 2 n 2^-24 of the boundary, n the
candidates (or the kept tokens); it must then return a token the oracle keeps or
one within the boundary's reach. On logits ~ N(0, 3) the sums' errors are far
below that bound and nearly every row is identical; a cut inside a large group of
equal logits adds equal terms, whose rounding errors do not cancel.
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


@pytest.mark.parametrize("whole", [False, True])
def test_page_examples(whole):
    """The page's two examples, through the top-k path (k one below the vocabulary,
    every token still a candidate) and without top-k (top-p over the whole
    vocabulary)."""
    eq = np.zeros((4, 100), np.float32)            # 100 equiprobable tokens, p = 0.5: 50 kept
    k = 0 if whole else 99
    us = (0.0, 0.999, 0.51, 0.5)
    got = _gpu(eq, 1.0, k, 0.5, np.array(us, np.float32))
    ref = [sample_row(eq[0], 1.0, k, 0.5, u) for u in us]
    assert got[:3].tolist() == [d.token for d in ref[:3]] == [50, 99, 75]
    # u = 0.5 puts the draw exactly on the boundary between tokens 74 and 75 (25 of 50
    # equal probabilities): the oracle's one-at-a-time sum decides it by its rounding,
    # the whole-vocabulary path sums a chunk's terms as a tree
    assert got[3] == ref[3].token or (ref[3].draw_margin < 1e-5 and got[3] in (74, 75))
    ties = np.array([[1.0, 1.0, 0.0, 0.0]] * 3, np.float32)   # the stable sort keeps index 1
    k = 0 if whole else 3
    assert _gpu(ties, 1.0, k, 0.05, np.array([0.0, 0.5, 0.99], np.float32)).tolist() == [1, 1, 1]


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


def _check_whole(logits, T, p, u, got, label):
    """Top-p alone: exact tokens except rows whose cut or draw lies within the
    bound of its boundary; those must return a token the oracle keeps, or one at
    most a few places below its cut in the ascending order (the kept set is the
    top of that order)."""
    B, V = logits.shape
    exact = 0
    for b in range(B):
        d = sample_row(logits[b], T, 0, p, float(u[b]))
        if got[b] == d.token:
            exact += 1
            continue
        cut_bound, draw_bound = 2.0 * V * 2.0 ** -24, 2.0 * len(d.kept) * 2.0 ** -24
        print(f"  row {b}: gpu {got[b]} oracle {d.token}, cut margin {d.cut_margin:.2e} (bound {cut_bound:.1e}), "
              f"draw margin {d.draw_margin:.2e} (bound {draw_bound:.1e})")
        assert d.cut_margin < cut_bound or d.draw_margin < draw_bound, (label, b)
        order = np.argsort(logits[b], kind="stable")
        near = set(order[max(0, V - len(d.kept) - 8):].tolist())
        assert got[b] in near, (label, b, got[b])
    print(f"{label}: {exact}/{B} rows identical")
    return exact


@pytest.mark.timeout(300)
@pytest.mark.parametrize("T,p", [(0.7, 0.8), (1.0, 0.5), (1.0, 0.95), (0.5, 1.0), (1.3, 0.9), (0.7, 1e-6)])
def test_top_p_alone_matches_oracle(T, p):
    """top_k = 0 over 151,936 logits ~ N(0, 3): the cut by mass over the whole
    vocabulary and the draw in token order."""
    rng = np.random.default_rng(int(T * 1000 + p * 100))
    B, V = 16, 151936
    logits = (rng.standard_normal((B, V)) * 3.0).astype(np.float32)
    u = rng.random(B).astype(np.float32)
    got = _gpu(logits, T, 0, p, u)
    exact = _check_whole(logits, T, p, u, got, f"top-p alone T={T} p={p}")
    assert exact >= B - 2
    if p < 1e-3:   # keeps the largest only
        assert got.tolist() == np.argmax(logits, axis=1).tolist()


@pytest.mark.timeout(300)
@pytest.mark.parametrize("n_tied", [5, 1500, 3000])
def test_top_p_alone_ties_at_the_cut(n_tied):
    """The cut falls inside a group of equal logits (p = 0.8; p = 0.3 puts it among
    the four above for the smallest group): the tied tokens are removed in id order
    (the stable ascending order) while the running sum stays <= 1 - p; a group
    beyond the 2048 LDS slots is ranked by reading the row in id order. The rest of
    the vocabulary sits at -12 (under 1% of the mass)."""
    rng = np.random.default_rng(n_tied)
    B, V = 8, 151936
    logits = np.full((B, V), -12.0, np.float32)
    for b in range(B):
        tied = rng.choice(V, size=n_tied, replace=False)
        logits[b, tied] = 2.0
        above = rng.choice(np.setdiff1d(np.arange(V), tied), size=4, replace=False)
        logits[b, above] = np.float32(2.5 + b * 0.25)
    u = rng.random(B).astype(np.float32)
    for p in (0.8, 0.3):
        got = _gpu(logits, 1.0, 0, p, u)
        exact = _check_whole(logits, 1.0, p, u, got, f"ties {n_tied} p={p}")
        assert exact >= B // 2


def test_top_p_alone_ties_at_the_top():
    """p so small that only the largest stays: of tied maxima the one with the
    highest id (it sorts last in the stable ascending order)."""
    lg = np.zeros((4, 5000), np.float32)
    lg[:, [7, 1234, 4000]] = 3.0
    got = _gpu(lg, 1.0, 0, 1e-6, np.array([0.0, 0.3, 0.6, 0.99], np.float32))
    assert got.tolist() == [4000] * 4 == [sample_row(lg[0], 1.0, 0, 1e-6, x).token for x in (0.0, 0.3, 0.6, 0.99)]
