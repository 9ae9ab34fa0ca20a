"""Shared set-up for the GPU parity tests: seeded inputs drawn once on the
device, the libqd runner over them, and host copies for the oracle."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from oracle.qwen2 import OracleWeights, decode_step
from workloads import synth


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))


@dataclass
class Case:
    shape: object
    w: dict
    kv: object
    runner: object
    host_w: dict
    k_host: list
    v_host: list
    ctx: np.ndarray


def make_case(shape, ctx, seed=0, extra=4, random_order=False, max_batch=None, device="cuda",
              gain_mode="one_plus", prefill_tokens=0) -> Case:
    from decode_step_amd.runner import DecodeRunner
    ctx = np.asarray(ctx, dtype=np.int32)
    w = synth.make_weights(shape, seed=seed, device=device, gain_mode=gain_mode)
    kv = synth.make_kv(shape, ctx, extra=extra, seed=seed, device=device, random_order=random_order)
    B = len(ctx) if max_batch is None else max_batch
    runner = DecodeRunner(shape, w, kv.k, kv.v, kv.block_table, max_batch=B,
                          max_ctx=int(ctx.max()) + extra + 1, device=device,
                          prefill_tokens=prefill_tokens)
    host_w = synth.weights_to_host(w)
    kh = [synth.to_host_bits(t).copy() for t in kv.k]
    vh = [synth.to_host_bits(t).copy() for t in kv.v]
    return Case(shape, w, kv, runner, host_w, kh, vh, ctx)


def dev_i32(a, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def guarded(n: int, device="cuda", pad: int = 1024, fill=float("nan")):
    """A float buffer of n elements between two canary regions; returns (full, view)."""
    full = torch.full((n + 2 * pad,), fill, dtype=torch.float32, device=device)
    full[:pad] = 12345.0
    full[pad + n:] = 12345.0
    return full, full[pad:pad + n]


def canaries_intact(full: torch.Tensor, n: int, pad: int = 1024) -> bool:
    f = full.cpu()
    return bool(torch.all(f[:pad] == 12345.0)) and bool(torch.all(f[pad + n:] == 12345.0))


def kv_mismatch(dev_pool, host_pool, abs_frac=1e-4) -> str:
    """Stored K/V agree when every element is within one bf16 step of its own
    value (the float32 value the GPU rounds may sit across a rounding boundary
    from the oracle's) plus abs_frac of the pool's largest magnitude (a value
    that cancels to near zero carries the projection's absolute rounding
    error, which can be many of its own tiny bf16 steps). Float32 pools use a
    1e-5 relative bound instead of the bf16 step. Returns "" when they agree,
    else a description of the worst element and the count over tolerance."""
    g = synth.to_host_bits(dev_pool)
    if g.dtype == np.uint16:
        gw = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        hw = (np.asarray(host_pool).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        step = np.ldexp(1.0, np.frexp(np.abs(hw))[1] - 8)
    else:
        gw = g.astype(np.float64)
        hw = np.asarray(host_pool, dtype=np.float64)
        step = 1e-5 * np.abs(hw)
    tol = step + abs_frac * np.max(np.abs(hw))
    over = np.abs(gw - hw) / tol
    if np.all(over <= 1.0):
        return ""
    i = int(np.argmax(over))
    idx = np.unravel_index(i, gw.shape)
    return (f"{int(np.sum(over > 1.0))} of {over.size} elements over tolerance; worst at {idx}: "
            f"gpu {gw.flat[i]:.6g} oracle {hw.flat[i]:.6g} tol {tol.flat[i]:.3g}")


def kv_matches(dev_pool, host_pool, abs_frac=1e-4) -> bool:
    return kv_mismatch(dev_pool, host_pool, abs_frac) == ""


def check_argmax_tie(case, pos, tok):
    """Planted exact tie: the winning lm_head row copied to a higher and then to a
    lower vocabulary index gives two bitwise-equal largest logits; the step (and
    the oracle) must return the lower index both times."""
    sh = case.shape
    lm = case.w["lm_head"] if case.w.get("lm_head") is not None else case.w["embed"]
    key = "lm_head" if case.w.get("lm_head") is not None else "embed"
    logits = torch.empty(1, sh.vocab, device="cuda")
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    case.runner.step(pos, dev_i32(pos), tokens=dev_i32(tok), logits=logits, next_tokens=nxt)
    torch.cuda.synchronize()
    i = int(nxt.cpu()[0])
    for j in ((i + 1 + 37) % sh.vocab, (i + sh.vocab - 23) % sh.vocab):
        assert j not in (i, int(tok[0]))
        lm[j].copy_(lm[i])
        case.host_w[key][j] = case.host_w[key][i]
        case.runner.step(pos, dev_i32(pos), tokens=dev_i32(tok), logits=logits, next_tokens=nxt)
        torch.cuda.synchronize()
        lg = logits.cpu().numpy()[0]
        assert lg[i] == lg[j] and lg[i] == lg.max()
        assert int(nxt.cpu()[0]) == min(i, j)
        ow = OracleWeights(sh, case.host_w, cache_layers=False)
        ref = decode_step(sh, ow, case.k_host, case.v_host, case.kv.block_table, pos, tokens=tok)
        assert int(ref.next_tokens[0]) == min(i, j)
        i = min(i, j)
