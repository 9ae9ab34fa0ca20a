"""Seeded synthetic inputs for the decode step and the prefill block.

This module only draws numbers; it holds none of the forward pass's arithmetic.
Every tensor gets its own generator, seeded from (seed, tensor name), so a
tensor's values do not depend on which other tensors were drawn. The same call
on the same device type always gives the same values; the GPU tests draw once
and hand the oracle host copies of exactly what the GPU received.

Recipe (no dataset or trained weight is needed; seeded tensors of the real
shapes stand in for them, as nanoinfer's synthetic mode does):
  * matrices and biases ~ N(0, 0.02); norm gains ~ 1 + N(0, 0.02)
    (gain_mode="literal" draws gains ~ N(0, 0.02) instead);
  * cached K/V ~ N(0, 1), taken as already rotated (keys are rotated once on
    insert);
  * decode block input ~ N(0, 1) fp32; prefill input ~ N(0, 1) bf16;
  * token ids ~ U{0..V-1}; context lengths ~ U{lo..hi};
  * page pool of sum_b ceil((ctx_b + extra)/page) pages, randomly permuted when
    the workload asks for a random block table, handed out in order.
bf16 tensors come from torch's float32 -> bfloat16 conversion.
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from .shapes import ModelShape

W_STD = 0.02


def _seed_for(seed: int, name: str) -> int:
    return (seed * 0x9E3779B1 + zlib.crc32(name.encode())) & 0x7FFF_FFFF_FFFF


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed_for(seed, name))
    return g


def _torch_dtype(d: str):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[d]


def normal(shape, std: float, mean: float, dtype: str, seed: int, name: str, device="cpu"):
    g = _gen(seed, name, device)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(_torch_dtype(dtype))


def uniform_int(n: int, lo: int, hi: int, seed: int, name: str) -> np.ndarray:
    """n integers uniform on [lo, hi] inclusive, drawn on the host."""
    g = _gen(seed, name, "cpu")
    return torch.randint(lo, hi + 1, (n,), generator=g).numpy().astype(np.int32)


def make_weights(shape: ModelShape, seed: int = 0, device="cpu", gain_mode: str = "one_plus",
                 with_embed: bool = True, w_std: float = W_STD) -> dict:
    """All weights of the model as torch tensors on `device`, row-major [out][in].
    An int8 shape ("i8") is drawn in bf16, the form its codes are quantized from."""
    wd = "bf16" if shape.w_dtype == "i8" else shape.w_dtype
    gmean = 1.0 if gain_mode == "one_plus" else 0.0
    D, F = shape.hidden, shape.ffn
    out = {"layers": []}
    if with_embed:
        out["embed"] = normal((shape.vocab, D), w_std, 0.0, wd, seed, "embed", device)
        out["final_norm"] = normal((D,), w_std, gmean, wd, seed, "final_norm", device)
        out["lm_head"] = (None if shape.tied else
                          normal((shape.vocab, D), w_std, 0.0, wd, seed, "lm_head", device))
    for l in range(shape.n_layers):
        p = f"layers.{l}."
        L = {
            "attn_norm": normal((D,), w_std, gmean, wd, seed, p + "attn_norm", device),
            "wq": normal((shape.q_dim, D), w_std, 0.0, wd, seed, p + "wq", device),
            "wk": normal((shape.kv_dim, D), w_std, 0.0, wd, seed, p + "wk", device),
            "wv": normal((shape.kv_dim, D), w_std, 0.0, wd, seed, p + "wv", device),
            "wo": normal((D, shape.q_dim), w_std, 0.0, wd, seed, p + "wo", device),
            "mlp_norm": normal((D,), w_std, gmean, wd, seed, p + "mlp_norm", device),
            "w_gate": normal((F, D), w_std, 0.0, wd, seed, p + "w_gate", device),
            "w_up": normal((F, D), w_std, 0.0, wd, seed, p + "w_up", device),
            "w_down": normal((D, F), w_std, 0.0, wd, seed, p + "w_down", device),
        }
        if shape.qkv_bias:
            L["bq"] = normal((shape.q_dim,), w_std, 0.0, wd, seed, p + "bq", device)
            L["bk"] = normal((shape.kv_dim,), w_std, 0.0, wd, seed, p + "bk", device)
            L["bv"] = normal((shape.kv_dim,), w_std, 0.0, wd, seed, p + "bv", device)
        if shape.qk_norm:
            L["q_norm"] = normal((shape.head_dim,), w_std, gmean, wd, seed, p + "q_norm", device)
            L["k_norm"] = normal((shape.head_dim,), w_std, gmean, wd, seed, p + "k_norm", device)
        out["layers"].append(L)
    return out


@dataclass
class PagedKV:
    """Per-layer K/V page pools [pages][Hkv][page][hd] and one block table [B][max_blocks]."""
    k: List[torch.Tensor]
    v: List[torch.Tensor]
    block_table: np.ndarray          # int32 [B][max_blocks], -1 where unused
    num_pages: int
    page_size: int

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])


def make_block_table(ctx: np.ndarray, extra: int, page: int, seed: int, random_order: bool):
    need = [int(math.ceil((int(c) + extra) / page)) for c in ctx]
    total = int(sum(need))
    if random_order:
        g = _gen(seed, "block_table", "cpu")
        order = torch.randperm(total, generator=g).numpy().astype(np.int32)
    else:
        order = np.arange(total, dtype=np.int32)
    table = np.full((len(ctx), max(need)), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(need):
        table[b, :n] = order[k:k + n]
        k += n
    return table, total


def make_kv(shape: ModelShape, ctx: np.ndarray, extra: int, seed: int = 0, device="cpu",
            random_order: bool = False, fill: str = "normal") -> PagedKV:
    table, total = make_block_table(ctx, extra, shape.page_size, seed, random_order)
    dims = (total, shape.n_kv_heads, shape.page_size, shape.head_dim)
    ks, vs = [], []
    for l in range(shape.n_layers):
        if fill == "normal":
            ks.append(normal(dims, 1.0, 0.0, shape.kv_dtype, seed, f"kcache.{l}", device))
            vs.append(normal(dims, 1.0, 0.0, shape.kv_dtype, seed, f"vcache.{l}", device))
        else:
            ks.append(torch.zeros(dims, dtype=_torch_dtype(shape.kv_dtype), device=device))
            vs.append(torch.zeros(dims, dtype=_torch_dtype(shape.kv_dtype), device=device))
    return PagedKV(ks, vs, table, total, shape.page_size)


def make_ctx(batch: int, past: Optional[int], ctx_range: Optional[tuple], seed: int) -> np.ndarray:
    if ctx_range is not None:
        return uniform_int(batch, ctx_range[0], ctx_range[1], seed, "ctx_lens")
    return np.full(batch, int(past), dtype=np.int32)


def make_tokens(batch: int, vocab: int, seed: int, name: str = "tokens") -> np.ndarray:
    return uniform_int(batch, 0, vocab - 1, seed, name)


def make_x(batch: int, hidden: int, seed: int, dtype: str = "f32", device="cpu",
           name: str = "x_in") -> torch.Tensor:
    return normal((batch, hidden), 1.0, 0.0, dtype, seed, name, device)


def to_host_bits(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Host numpy copy: bf16 as raw uint16 bit patterns, fp32 as float32."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def weights_to_host(w: dict) -> dict:
    out = {k: to_host_bits(v) for k, v in w.items() if k != "layers"}
    out["layers"] = [{k: to_host_bits(v) for k, v in L.items()} for L in w["layers"]]
    return out
