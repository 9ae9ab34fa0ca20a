"""Plain float64 definition of the Qwen2-style GQA decode step (test infrastructure only).

Sources, by page and section:
  * nanoinfer page, phase 3 (float32 forward pass, no cache): the pre-norm block
    x = x + attention(rms_norm(x)); x = x + feed_forward(rms_norm(x)); RMSNorm;
    SwiGLU; RoPE half-split pairing i with i + d/2; GQA repeats each KV head
    for `group` consecutive query heads; a token attends to itself (j <= i);
    the final hidden state is taken after the final norm.
  * nanoinfer page, model notes: biases on q/k/v only, none on o_proj; tied
    embeddings, logits = hidden @ embed_tokens.T; greedy = argmax.
  * nanoinfer page, phase 4 (KV cache): keys are rotated once, on insert;
    decode positions continue at the cached length.
  * nanoinfer page, phase 7: sigmoid from e = exp(-|x|) as 1/(1+e) for x >= 0
    and e/(1+e) otherwise.
  * nanocompile page, phase 1: RMSNorm's mean square is a sum then a divide;
    epsilon is added before the square root.
  * nanoserve day 49: the paged read writes this step's K/V into its slot
    before attending; slot of position p = (block_table[p // page], p % page).
  * Tang page, section 2.2 (comprehensions and monoids): online softmax is a
    monoid on (running max, rescaled sum) carrying the weighted values; that
    form and the split/merge form are alternate forms here, proved equal to
    the two-pass definition by the tests, never used for expected values.
Readings where the pages are silent (each listed in the design notes): scores
are scaled by 1/sqrt(head_dim); RoPE angle for pair i at position p is
p * theta^(-2i/hd), evaluated in float64; the q/k bias is added before the
rotation; per-head q/k RMSNorm (8B-class shape) uses one gain vector of length
head_dim shared by all heads, applied after the projection and before RoPE.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .numerics import widen, round_f32, round_bf16, store_kv


# ----------------------------------------------------------------------------- primitives

def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x * (1 / sqrt(sum(x^2)/n + eps)) * g over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    mean_sq = np.sum(x * x, axis=-1, keepdims=True) / n
    r = 1.0 / np.sqrt(mean_sq + eps)
    return x * r * g


def linear(w: np.ndarray, x: np.ndarray, b: Optional[np.ndarray] = None) -> np.ndarray:
    """y = W x (+ b) for W stored row-major [out][in]; x is [in] or [rows, in]."""
    y = np.asarray(x, dtype=np.float64) @ w.T
    if b is not None:
        y = y + b
    return y


def sigmoid(z: np.ndarray) -> np.ndarray:
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


def rope_angles(pos: int, hd: int, theta: float) -> np.ndarray:
    i = np.arange(hd // 2, dtype=np.float64)
    inv_freq = theta ** (-(2.0 * i) / hd)
    return float(pos) * inv_freq


def rope(u: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Half-split rotation of each row of u [..., hd] by the angles of position pos."""
    u = np.asarray(u, dtype=np.float64)
    hd = u.shape[-1]
    h = hd // 2
    a = rope_angles(pos, hd, theta)
    c, s = np.cos(a), np.sin(a)
    lo, hi = u[..., :h], u[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def rope_interleaved(u: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """The other convention (pairs 2i, 2i+1); kept only so a test can show it differs."""
    u = np.asarray(u, dtype=np.float64)
    hd = u.shape[-1]
    a = rope_angles(pos, hd, theta)
    c, s = np.cos(a), np.sin(a)
    ev, od = u[..., 0::2], u[..., 1::2]
    out = np.empty_like(u)
    out[..., 0::2] = ev * c - od * s
    out[..., 1::2] = od * c + ev * s
    return out


def softmax(s: np.ndarray) -> np.ndarray:
    """Two-pass softmax over the last axis: subtract the max, exponentiate, divide by the sum."""
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_heads(q: np.ndarray, K: np.ndarray, V: np.ndarray, group: int) -> np.ndarray:
    """One query row: q [Hq, hd] against keys/values K, V [T, Hkv, hd].
    Query head h reads KV head h // group (repeat, not tile)."""
    Hq, hd = q.shape
    out = np.empty((Hq, V.shape[-1]), dtype=np.float64)
    for h in range(Hq):
        g = h // group
        s = (K[:, g, :] @ q[h]) / np.sqrt(hd)
        p = softmax(s)
        out[h] = p @ V[:, g, :]
    return out


def attention_online(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Alternate form for one head: q [hd], K, V [T, hd], streamed one key at a time
    with state (m, l, o): m' = max(m, s); l' = l e^(m-m') + e^(s-m'); o' = o e^(m-m') + e^(s-m') v."""
    hd = q.shape[0]
    m, l, o = -np.inf, 0.0, np.zeros(V.shape[-1])
    for t in range(K.shape[0]):
        s = float(K[t] @ q) / np.sqrt(hd)
        m_new = max(m, s)
        a = np.exp(m - m_new) if np.isfinite(m) else 0.0
        b = np.exp(s - m_new)
        l = l * a + b
        o = o * a + b * V[t]
        m = m_new
    return o / l


def attention_split_merge(q: np.ndarray, K: np.ndarray, V: np.ndarray, chunk: int) -> np.ndarray:
    """Alternate form for one head: per-chunk partials (m, l, o) merged pairwise with
    M = max(m1, m2): (M, l1 e^(m1-M) + l2 e^(m2-M), o1 e^(m1-M) + o2 e^(m2-M))."""
    hd = q.shape[0]
    parts = []
    for t0 in range(0, K.shape[0], chunk):
        s = (K[t0:t0 + chunk] @ q) / np.sqrt(hd)
        m = float(np.max(s))
        e = np.exp(s - m)
        parts.append((m, float(np.sum(e)), e @ V[t0:t0 + chunk]))
    m, l, o = parts[0]
    for m2, l2, o2 in parts[1:]:
        M = max(m, m2)
        l = l * np.exp(m - M) + l2 * np.exp(m2 - M)
        o = o * np.exp(m - M) + o2 * np.exp(m2 - M)
        m = M
    return o / l


def argmax_first(logits: np.ndarray) -> np.ndarray:
    """Index of the largest value per row, the lowest index on a tie."""
    return np.argmax(logits, axis=-1).astype(np.int32)


# ----------------------------------------------------------------------------- weights

class OracleWeights:
    """Host weights (bf16 bits or float32) widened to float64 on demand.

    `cache_layers` keeps widened layers for reuse across steps (about 8 bytes
    per parameter); the 8B-class shape widens one layer at a time instead."""

    def __init__(self, shape, host: dict, cache_layers: bool = True):
        self.shape = shape
        self.host = host
        self.cache_layers = cache_layers
        self._layers = {}
        self._final_norm = None

    def layer(self, l: int) -> dict:
        if l in self._layers:
            return self._layers[l]
        L = {k: (widen(v) if v is not None else None) for k, v in self.host["layers"][l].items()}
        if self.cache_layers:
            self._layers[l] = L
        return L

    def embed_rows(self, tokens: np.ndarray) -> np.ndarray:
        return widen(self.host["embed"][np.asarray(tokens, dtype=np.int64)])

    def final_norm(self) -> np.ndarray:
        if self._final_norm is None:
            self._final_norm = widen(self.host["final_norm"])
        return self._final_norm

    def lm_head(self, n: np.ndarray, rows_per_chunk: int = 16384) -> np.ndarray:
        """logits = W_lm n with W_lm = the embedding when tied; n is [B, D]."""
        W = self.host["embed"] if self.host.get("lm_head") is None else self.host["lm_head"]
        V = W.shape[0]
        out = np.empty((n.shape[0], V), dtype=np.float64)
        for r0 in range(0, V, rows_per_chunk):
            out[:, r0:r0 + rows_per_chunk] = n @ widen(W[r0:r0 + rows_per_chunk]).T
        return out


# ----------------------------------------------------------------------------- KV cache

def cache_rows(pool: np.ndarray, table_row: np.ndarray, n: int, page: int) -> np.ndarray:
    """Stored rows 0..n-1 of one sequence as float64 [n, Hkv, hd]; pool is [pages][Hkv][page][hd]."""
    t = np.arange(n)
    return widen(pool[table_row[t // page], :, t % page, :])


def cache_write(pool: np.ndarray, table_row: np.ndarray, p: int, page: int, x: np.ndarray,
                kv_dtype: str) -> None:
    """Store x [Hkv, hd] as position p of one sequence, in the cache's storage type."""
    pool[table_row[p // page], :, p % page, :] = store_kv(x, kv_dtype)


# ----------------------------------------------------------------------------- the step

@dataclass
class StepResult:
    x_out: np.ndarray          # [B, D] last layer's output (before the final norm)
    layer_out: np.ndarray      # [L, B, D] residual stream after each layer
    logits: Optional[np.ndarray] = None   # [B, V], float32 values as float64
    next_tokens: Optional[np.ndarray] = None  # [B] int32


def _layer_decode(shape, W: dict, x: np.ndarray, pos: np.ndarray, k_pool, v_pool,
                  table: np.ndarray) -> np.ndarray:
    """One decoder layer for a batch of single-token rows x [B, D] at positions pos [B]."""
    Hq, Hkv, hd, eps = shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.rms_eps
    B = x.shape[0]
    n = rms_norm(x, W["attn_norm"], eps)
    q = linear(W["wq"], n, W.get("bq")).reshape(B, Hq, hd)
    k = linear(W["wk"], n, W.get("bk")).reshape(B, Hkv, hd)
    v = linear(W["wv"], n, W.get("bv")).reshape(B, Hkv, hd)
    if shape.qk_norm:
        q = rms_norm(q, W["q_norm"], eps)
        k = rms_norm(k, W["k_norm"], eps)
    ctx = np.empty((B, Hq * hd), dtype=np.float64)
    for b in range(B):
        p = int(pos[b])
        qb = rope(q[b], p, shape.rope_theta)
        kb = rope(k[b], p, shape.rope_theta)
        cache_write(k_pool, table[b], p, shape.page_size, kb, shape.kv_dtype)
        cache_write(v_pool, table[b], p, shape.page_size, v[b], shape.kv_dtype)
        K = cache_rows(k_pool, table[b], p + 1, shape.page_size)
        V = cache_rows(v_pool, table[b], p + 1, shape.page_size)
        ctx[b] = attention_heads(qb, K, V, shape.group).reshape(-1)
    x = x + linear(W["wo"], ctx)
    n2 = rms_norm(x, W["mlp_norm"], eps)
    h = silu(linear(W["w_gate"], n2)) * linear(W["w_up"], n2)
    return x + linear(W["w_down"], h)


def decode_step(shape, weights: OracleWeights, k_pools: list, v_pools: list,
                block_table: np.ndarray, pos: np.ndarray, tokens: Optional[np.ndarray] = None,
                x_in: Optional[np.ndarray] = None, with_logits: bool = True) -> StepResult:
    """One decode forward step for B sequences, one new token each.

    pos[b] is the number of tokens already cached for sequence b; the new token
    sits at position pos[b]. Its K/V are written into the pools (mutated in
    place) before it attends over positions 0..pos[b] as stored. The input is
    the embedding row of tokens[b], or x_in[b] for a block-only step."""
    pos = np.asarray(pos)
    if tokens is not None:
        x = weights.embed_rows(tokens)
    else:
        x = np.asarray(x_in, dtype=np.float64)
        if x.ndim == 1:
            x = x[None, :]
    L = shape.n_layers
    layer_out = np.empty((L,) + x.shape, dtype=np.float64)
    for l in range(L):
        x = _layer_decode(shape, weights.layer(l), x, pos, k_pools[l], v_pools[l], block_table)
        layer_out[l] = x
    res = StepResult(x_out=x, layer_out=layer_out)
    if with_logits:
        n = rms_norm(x, weights.final_norm(), shape.rms_eps)
        logits = round_f32(weights.lm_head(n))
        res.logits = logits
        res.next_tokens = argmax_first(logits)
    return res


def prefill_block(shape, W: dict, k_pool: np.ndarray, v_pool: np.ndarray, table_row: np.ndarray,
                  start: int, x_in: np.ndarray, return_operands: bool = False):
    """One decoder block over N consecutive tokens of one sequence at positions
    start..start+N-1, causal (row i attends to positions 0..start+i).

    The projections are bf16 matrix products with float32 accumulation, so their
    activation operands are rounded to bf16: the normed input, the attention
    context, the second normed input and the SwiGLU output. K/V are stored in the
    cache type and read back as stored; q and the attention probabilities are not
    rounded. The residual stream is float64 here (float32 on the device).
    Returns x_out [N, D]; with return_operands, also a dict of the intermediate
    values (n, q, ctx, x_mid, n2, h) for the tests that pin where the rounding
    falls."""
    Hq, Hkv, hd, eps = shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.rms_eps
    # operand rounding of the matrix products: bf16 for bf16 weights, float32 otherwise
    op = round_bf16 if shape.w_dtype == "bf16" else round_f32
    X = widen(x_in)
    N = X.shape[0]
    n = op(rms_norm(X, W["attn_norm"], eps))
    Q = linear(W["wq"], n, W.get("bq")).reshape(N, Hq, hd)
    K = linear(W["wk"], n, W.get("bk")).reshape(N, Hkv, hd)
    Vv = linear(W["wv"], n, W.get("bv")).reshape(N, Hkv, hd)
    if shape.qk_norm:
        Q = rms_norm(Q, W["q_norm"], eps)
        K = rms_norm(K, W["k_norm"], eps)
    for i in range(N):
        p = start + i
        Q[i] = rope(Q[i], p, shape.rope_theta)
        cache_write(k_pool, table_row, p, shape.page_size, rope(K[i], p, shape.rope_theta),
                    shape.kv_dtype)
        cache_write(v_pool, table_row, p, shape.page_size, Vv[i], shape.kv_dtype)
    Kc = cache_rows(k_pool, table_row, start + N, shape.page_size)
    Vc = cache_rows(v_pool, table_row, start + N, shape.page_size)
    ctx = np.empty((N, Hq * hd), dtype=np.float64)
    for i in range(N):
        p = start + i
        ctx[i] = attention_heads(Q[i], Kc[:p + 1], Vc[:p + 1], shape.group).reshape(-1)
    ctx_op = op(ctx)
    X = X + linear(W["wo"], ctx_op)
    n2 = op(rms_norm(X, W["mlp_norm"], eps))
    H = op(silu(linear(W["w_gate"], n2)) * linear(W["w_up"], n2))
    out = X + linear(W["w_down"], H)
    if return_operands:
        return out, {"n": n, "q": Q.reshape(N, -1), "ctx": ctx_op, "x_mid": X, "n2": n2, "h": H}
    return out
