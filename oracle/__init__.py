"""CPU oracle for the Qwen2-style decode step and prefill block.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the package's
smoke check and the benchmark's CPU-baseline leg may import or call anything in
this package. The GPU path never routes through it, and it shares no code,
table or helper with the GPU path: it reads only host numpy arrays.

It is the plain definition of what one decode forward step computes, written
out in float64 with numpy (a matrix-vector product is the one library
primitive it leans on), rounding only where the method itself stores a value
at lower precision:
  * K/V are stored in the cache dtype (bf16 by round-half-to-even from the
    float32 value, or float32) and read back as stored;
  * logits are float32 and the greedy argmax is taken over those float32 values
    (lowest index wins a tie);
  * in the prefill block, the activation operands of the bf16 matrix products
    (the two normed inputs, the attention context, the SwiGLU output) are
    rounded to bf16; the rotated q, the attention probabilities and the
    residual stream are not.
Attention is the two-pass softmax over every key, not an online or split form;
those appear only as alternate forms that the tests prove equal to it.

Pins (tests/test_oracle_*.py): RMSNorm closed forms, softmax rows summing to
one and shift invariance, one-token attention returning V exactly, identical
keys giving mean(V), GQA repeat-not-tile, RoPE norm preservation / identity at
position 0 / relative-position property / a hand-worked hd=4 rotation, SiLU
symmetry, bf16 round trip and tie cases, GEMV against exact integer brute
force, online == two-pass and split-merge == single pass, fused == unfused
forms, paged == contiguous, batched == single, cached decode == uncached
prefill, and the whole forward against the transformers library's Qwen2 and
Qwen3 models run in float64.
"""
from .numerics import bf16_bits_to_f32, f32_to_bf16_bits, widen, round_f32, store_kv
from .qwen2 import (rms_norm, linear, silu, rope, rope_interleaved, softmax, attention_heads,
                    attention_online, attention_split_merge, decode_step, prefill_block,
                    argmax_first, OracleWeights)

__all__ = ["bf16_bits_to_f32", "f32_to_bf16_bits", "widen", "round_f32", "store_kv", "rms_norm",
           "linear", "silu", "rope", "rope_interleaved", "softmax", "attention_heads",
           "attention_online", "attention_split_merge", "decode_step", "prefill_block",
           "argmax_first", "OracleWeights"]
