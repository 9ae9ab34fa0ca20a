"""Model shapes and workload presets for the Qwen2-style decode step.

Plain data only: no arithmetic of the forward pass lives here. Both the GPU
path's tests/bench and the CPU oracle read these presets.

Shapes follow the nanoinfer page (Qwen2.5-0.5B: 24 layers, hidden 896, 14 query
heads sharing 2 key/value heads, SwiGLU width 4864, vocabulary 151936, tied
embeddings, biases on q/k/v only) and an 8B-class GQA shape with per-head q/k
RMSNorm (36 layers, hidden 4096, 32/8 heads of 128, SwiGLU width 12288).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    qkv_bias: bool = True
    qk_norm: bool = False
    tied: bool = True
    w_dtype: str = "bf16"      # "bf16" | "f32": matrices, embedding, norms, biases;
                               # "i8": int8 matrices and embedding with row scales, bf16 norms/biases
    kv_dtype: str = "bf16"     # "bf16" | "f32": the KV cache storage type
    page_size: int = 16

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def qkv_rows(self) -> int:
        return self.q_dim + 2 * self.kv_dim

    def param_counts(self) -> dict:
        """Parameter census in the nanoinfer page's four groups."""
        D, F = self.hidden, self.ffn
        emb = self.vocab * D * (1 if self.tied else 2)
        attn = self.n_layers * (self.q_dim * D + 2 * self.kv_dim * D + D * self.q_dim
                                + ((self.q_dim + 2 * self.kv_dim) if self.qkv_bias else 0))
        mlp = self.n_layers * 3 * D * F
        norms = self.n_layers * 2 * D + D + (self.n_layers * 2 * self.head_dim if self.qk_norm else 0)
        return {"embeddings": emb, "attention": attn, "mlp": mlp, "norms": norms,
                "total": emb + attn + mlp + norms}


QWEN2_0P5B = ModelShape(n_layers=24, hidden=896, n_q_heads=14, n_kv_heads=2, head_dim=64,
                        ffn=4864, vocab=151936)

QWEN_8B_QKNORM = ModelShape(n_layers=36, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
                            ffn=12288, vocab=151936, qkv_bias=False, qk_norm=True, tied=False)


@dataclass(frozen=True)
class Workload:
    """One decode or prefill workload: a shape plus batch/context/seed recipe."""
    name: str
    shape: ModelShape
    kind: str                      # "decode" | "prefill"
    batch: int = 1
    past: Optional[int] = None     # fixed cached length for every sequence
    ctx_range: Optional[tuple] = None  # (lo, hi) inclusive, drawn per sequence
    paged_random: bool = False     # seeded random block table (else identity order)
    greedy_steps: int = 0          # decode steps for the greedy-identity check
    prefill_tokens: int = 0
    block_only: bool = False       # one decoder block, fp32 input vector, no embed / lm_head
    seed: int = 0
    extra: dict = field(default_factory=dict)


# One Qwen2 decoder block in fp32, batch 1, one new token after 16 cached ones.
QWEN2_BLOCK_F32_PAST16 = Workload(
    name="qwen2-0.5b-block-f32-b1-past16",
    shape=replace(QWEN2_0P5B, n_layers=1, w_dtype="f32", kv_dtype="f32"),
    kind="decode", batch=1, past=16, block_only=True)

# Full 24-layer 0.5B decode, bf16 weights/KV, batch 1, 512 cached tokens, 32 greedy steps.
QWEN2_0P5B_B1_PAST512 = Workload(
    name="qwen2-0.5b-bf16-b1-past512",
    shape=QWEN2_0P5B, kind="decode", batch=1, past=512, greedy_steps=32)

# 0.5B, batch 16, per-sequence context uniform in [128, 4096], random paged block table.
QWEN2_0P5B_B16_PAGED = Workload(
    name="qwen2-0.5b-bf16-b16-ctx128to4096-paged",
    shape=QWEN2_0P5B, kind="decode", batch=16, ctx_range=(128, 4096), paged_random=True,
    greedy_steps=4)

# The 0.5B step with per-row int8 weights (quantized from the bf16 draw), batch 1, past 512.
QWEN2_0P5B_INT8_B1_PAST512 = Workload(
    name="qwen2-0.5b-int8-b1-past512",
    shape=replace(QWEN2_0P5B, w_dtype="i8"), kind="decode", batch=1, past=512, greedy_steps=8)

# The batch-16 paged step with per-row int8 weights.
QWEN2_0P5B_INT8_B16_PAGED = Workload(
    name="qwen2-0.5b-int8-b16-ctx128to4096-paged",
    shape=replace(QWEN2_0P5B, w_dtype="i8"), kind="decode", batch=16, ctx_range=(128, 4096),
    paged_random=True, greedy_steps=4)

# 8B-class shape with per-head q/k RMSNorm, batch 1, 4096 cached tokens.
QWEN_8B_B1_PAST4096 = Workload(
    name="qwen-8b-qknorm-bf16-b1-past4096",
    shape=QWEN_8B_QKNORM, kind="decode", batch=1, past=4096, greedy_steps=2)

# One 8B-class decoder block, 512-token causal prefill from an empty cache.
QWEN_8B_BLOCK_PREFILL512 = Workload(
    name="qwen-8b-qknorm-block-prefill512",
    shape=replace(QWEN_8B_QKNORM, n_layers=1), kind="prefill", batch=1, past=0,
    prefill_tokens=512, block_only=True)

# Sampling the next token of 16 sequences from 0.5B-vocabulary logits ~ N(0, 3) with the
# settings the nanoinfer page reads from the model (temperature 0.7, top-k 20, top-p 0.8).
QWEN2_SAMPLER_B16 = Workload(
    name="qwen2-sampler-b16-t0.7-k20-p0.8", shape=QWEN2_0P5B, kind="sample", batch=16,
    extra={"temperature": 0.7, "top_k": 20, "top_p": 0.8, "logit_std": 3.0})

# The same rows with top-p alone (no top-k: the cut over the whole vocabulary), the
# page's most expensive sampler configuration.
QWEN2_SAMPLER_TOPP_B16 = Workload(
    name="qwen2-sampler-b16-t0.7-topp0.8", shape=QWEN2_0P5B, kind="sample", batch=16,
    extra={"temperature": 0.7, "top_k": 0, "top_p": 0.8, "logit_std": 3.0})

WORKLOADS = {w.name: w for w in (QWEN2_BLOCK_F32_PAST16, QWEN2_0P5B_B1_PAST512,
                                 QWEN2_0P5B_B16_PAGED, QWEN_8B_B1_PAST4096,
                                 QWEN_8B_BLOCK_PREFILL512, QWEN2_0P5B_INT8_B1_PAST512,
                                 QWEN2_0P5B_INT8_B16_PAGED, QWEN2_SAMPLER_B16, QWEN2_SAMPLER_TOPP_B16)}


def tiny_shape(**over) -> ModelShape:
    """A tiny GQA shape for brute-force checks (2 layers, hidden 64)."""
    base = ModelShape(n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16, ffn=96,
                      vocab=200, page_size=16)
    return replace(base, **over)
