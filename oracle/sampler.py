"""Next-token sampling from logits (test infrastructure only).

nanoinfer page, phase 5 (sampling.py: temperature, top-k, top-p, seeded draw):
  * the order is temperature -> top-k -> top-p -> softmax -> draw, and it is not
    interchangeable; temperature 0 is the argmax (the limit of the distribution);
  * top-p follows the reference warper, not "sort descending, accumulate until
    the sum reaches p": sort ascending, accumulate the softmax probabilities,
    remove every token whose running sum is <= 1 - p; for 100 equiprobable
    tokens at p = 0.5 the float32 running sum after 50 terms is
    0.4999997913837433, so this rule keeps 50 where the descending rule keeps 51;
  * the sort is stable: [1, 1, 0, 0] sorts ascending to [2, 3, 0, 1], so of a
    tied pair the higher index counts as the more likely;
  * the draw is an inverse-CDF search, which does not need the probabilities to
    sum to exactly 1.0.
  * "top-p alone" (the page's per-token cost table) is the same pipeline without
    the top-k step: top_k <= 0 (or >= the vocabulary) keeps every token.
Readings where the page is silent: the arithmetic is float32, as the page's
tensors are, with every running sum taken one term at a time (the printed
0.4999997913837433 is exactly that sum); top-k keeps every token whose logit is
>= the k-th largest (the reference warper removes the scores below it), taken on
the logits since dividing by a positive temperature keeps their order; the kept
probabilities are searched in token-id order for the first running value that
exceeds u * total, u in [0, 1) given.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .qwen2 import argmax_first


@dataclass
class Draw:
    token: int
    kept: np.ndarray          # kept token ids, ascending
    cut_margin: float         # distance of the running sums next to the top-p cut from 1 - p
    draw_margin: float        # distance of the chosen token's running value from u * total


def _running(values: np.ndarray) -> np.ndarray:
    """Float32 running sums, one term at a time."""
    out = np.empty(len(values), np.float32)
    acc = np.float32(0.0)
    for i, v in enumerate(values):
        acc = np.float32(acc + v)
        out[i] = acc
    return out


def sample_row(logits: np.ndarray, temperature: float, top_k: int, top_p: float, u: float) -> Draw:
    lg = np.asarray(logits, dtype=np.float32)
    if temperature == 0.0:
        t = int(argmax_first(lg[None, :])[0])
        return Draw(t, np.array([t]), np.inf, np.inf)
    V = lg.size
    k = V if int(top_k) <= 0 else min(int(top_k), V)             # top_k <= 0: no top-k ("top-p alone")
    kth = np.sort(lg)[::-1][k - 1]
    cand = np.nonzero(lg >= kth)[0]                              # top-k, ties kept; ids ascending
    z = (lg[cand] / np.float32(temperature)).astype(np.float32)  # temperature
    order = np.argsort(z, kind="stable")                         # ascending; ties keep id order
    zs, ids = z[order], cand[order]
    e = np.exp((zs - zs[-1]).astype(np.float32)).astype(np.float32)
    S = np.float32(np.sum(e, dtype=np.float32))
    j0, cut_margin = 0, np.inf
    if top_p < 1.0:                                              # top-p
        thr = np.float32(1.0 - float(np.float32(top_p)))
        cum = _running((e / S).astype(np.float32))
        removed = cum[:-1] <= thr
        j0 = int(np.argmin(removed)) if not removed.all() else len(e) - 1
        near = cum[max(j0 - 1, 0):j0 + 1]
        cut_margin = float(np.min(np.abs(near.astype(np.float64) - float(thr))))
    kept_ids, kept_e = ids[j0:], e[j0:]
    o = np.argsort(kept_ids)
    kept_ids, kept_e = kept_ids[o], kept_e[o]
    Sk = np.float32(np.sum(kept_e, dtype=np.float32))
    run = _running((kept_e / Sk).astype(np.float32))             # softmax over the kept, id order
    target = np.float32(np.float32(u) * run[-1])
    hit = np.nonzero(run > target)[0]
    j = int(hit[0]) if hit.size else len(run) - 1
    lo = run[j - 1] if j > 0 else np.float32(0.0)
    draw_margin = float(min(abs(float(run[j]) - float(target)), abs(float(target) - float(lo))))
    return Draw(int(kept_ids[j]), kept_ids, cut_margin, draw_margin)


def sample(logits: np.ndarray, temperature: float, top_k: int, top_p: float, uniforms: np.ndarray):
    """One Draw per row of logits [B][V]."""
    return [sample_row(logits[b], temperature, top_k, top_p, float(uniforms[b])) for b in range(len(logits))]
