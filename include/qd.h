/*
 * qd.h -- C ABI of the MI355X (gfx950) decode-step library libqd.so.
 *
 * One decode forward step of a Qwen2-style grouped-query-attention transformer,
 * plus the one-block causal prefill and the KV append, as hand-written HIP
 * kernels enqueued on the caller's stream.
 *
 * What is computed (per the pages; each entry point names its passages):
 *   x = embed[token]                                   (nanoinfer, model notes: tied embeddings)
 *   per layer (nanoinfer, phase 3: the pre-norm block):
 *     n = x * (1/sqrt(sum(x^2)/D + eps)) * g_attn       (nanocompile, phase 1: sum then divide)
 *     q, k, v = W n + b                                 (nanoinfer, model notes: q/k/v biases only)
 *     [per-head RMSNorm of q and k]                     (8B-class shape only)
 *     RoPE half-split at position pos[b]                (nanoinfer, phase 3; phase 4: rotate on insert)
 *     K/V of the new token -> cache slot, then attend   (nanoserve day 49: write before the read)
 *     o_h = softmax(q_h K_g^T / sqrt(hd)) V_g, g = h / group   (nanoinfer, phase 3: repeat, j <= i)
 *     x += W_o o ;  n2 = rmsnorm(x) ;  x += W_d (silu(W_g n2) * (W_u n2))
 *   logits = W_lm rmsnorm(x; g_final) ; next = argmax (lowest index on a tie)
 * Attention runs as split-K online softmax with a merge (Tang, section 2.2 and
 * Table 1: online softmax and split reductions are monoids), which changes only
 * the rounding, not the result.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless the name ends in _host.
 *   - Matrices are row-major [out][in]; weight dtype from qd_config.w_dtype
 *     (QD_BF16: raw bf16, QD_F32: float; biases and gains use the same dtype;
 *     QD_I8: int8 matrices with one float scale per row, see below).
 *   - The caller owns and allocates everything (weights, KV pages, block table,
 *     workspace, outputs). The library never allocates device memory, never
 *     synchronises the stream and never reads device memory back to the host.
 *   - All work is enqueued in order on `stream` (a hipStream_t passed as void*;
 *     NULL is the default stream). The call returns once it is enqueued.
 *   - Arguments are checked on the host BEFORE anything is enqueued; a non-OK
 *     status means nothing was enqueued (except QD_EHIP, which reports a failed
 *     launch part-way). qd_last_error() gives a message (thread-local).
 *   - Faults inside a kernel surface as HIP errors at the caller's next sync.
 *   - Calls on different streams are independent iff they use different
 *     workspaces and touch different KV slots.
 */
#ifndef QD_H
#define QD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QD_ABI_VERSION 5

typedef enum {
    QD_OK = 0,
    QD_EINVAL = -1,        /* a required pointer is NULL, or an enum is out of range      */
    QD_ESHAPE = -2,        /* sizes inconsistent or outside the supported set             */
    QD_EALIGN = -3,        /* a pointer lacks its required alignment: 16 bytes for        *
                            * matrices, pools, x_in of a prefill and the workspace (128-  *
                            * bit loads), 4 bytes for float / int32 vectors               */
    QD_ECAPACITY = -4,     /* a position lies beyond the block table or the page pool     */
    QD_EPOSITION = -5,     /* a position is negative                                       */
    QD_EWORKSPACE = -6,    /* workspace NULL or smaller than qd_workspace_bytes()         */
    QD_EUNSUPPORTED = -7,  /* a dtype / option combination that is not implemented        */
    QD_EHIP = -8           /* a HIP launch failed (message names the kernel)              */
} qd_status;

typedef enum { QD_F32 = 0, QD_BF16 = 1, QD_I8 = 2 } qd_dtype;

/* Model configuration. hidden, ffn and head_dim must be multiples of 8;
 * n_q_heads must be a multiple of n_kv_heads; head_dim in {64, 128};
 * page_size in {16}; n_q_heads / n_kv_heads <= 8. */
typedef struct {
    int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, page_size;
    float rms_eps, rope_theta;
    int32_t qk_norm;   /* 1: per-head RMSNorm of q and k (gain [head_dim]) before RoPE */
    int32_t w_dtype;   /* qd_dtype of matrices, biases, gains and the embedding; QD_I8:
                        * int8 matrices and embedding (per-row scales), bf16 biases
                        * and gains (nanoinfer, phase 6: norms and biases are never
                        * quantized); decode steps only (batch 1..16; prefill blocks
                        * need QD_BF16)                                             */
    int32_t kv_dtype;  /* qd_dtype of the KV cache                                      */
} qd_config;

/* One decoder layer. Shapes: wq [Hq*hd][D], wk/wv [Hkv*hd][D], wo [D][Hq*hd],
 * w_gate/w_up [F][D], w_down [D][F]; attn_norm/mlp_norm [D]; bq [Hq*hd],
 * bk/bv [Hkv*hd] (NULL: no bias); q_norm/k_norm [hd] (used iff qk_norm).
 * s_* (QD_I8 only, else ignored): float [rows] scale of each matrix row, so that
 * row r of the matrix is q[r][:] * s[r] (qd_quantize_rows_int8 makes them). */
typedef struct {
    const void *attn_norm, *wq, *wk, *wv, *bq, *bk, *bv, *q_norm, *k_norm;
    const void *wo, *mlp_norm, *w_gate, *w_up, *w_down;
    const float *s_q, *s_k, *s_v, *s_o, *s_gate, *s_up, *s_down;
} qd_layer;

/* Whole-model weights. embed [V][D]; final_norm [D]; lm_head [V][D] or equal to
 * embed (tied). `layers_host` is a HOST array of n_layers qd_layer structs.
 * s_embed / s_lm_head: float [V] row scales (QD_I8 only; equal when tied). */
typedef struct {
    const void *embed, *final_norm, *lm_head;
    const qd_layer *layers_host;
    const float *s_embed, *s_lm_head;
} qd_weights;

/* Paged KV cache. For each layer l, k_pages_host[l] / v_pages_host[l] are device
 * pointers to a page pool [num_pages][n_kv_heads][page_size][head_dim] in
 * kv_dtype. block_table is device int32 [batch][max_blocks]: position p of
 * sequence b lives in page block_table[b][p / page_size], slot p % page_size
 * (nanoserve day 49, BlockTable.slot). block_table_host is the same table on the
 * host; every entry a call touches is checked against [0, num_pages). All layers
 * share the one table. */
typedef struct {
    void *const *k_pages_host;
    void *const *v_pages_host;
    const int32_t *block_table;
    const int32_t *block_table_host;
    int32_t max_blocks, num_pages;
} qd_kv;

/* Workspace bytes a call needs: for a decode step over at most `batch` sequences
 * whose positions are all < max_ctx (prefill_tokens = 0), or a prefill of
 * prefill_tokens tokens (batch = 1). Returns 0 if the config is invalid.
 * The caller sizes and owns this scratch once, so a step itself allocates
 * nothing (Tang page, section 5 Lowering: the generated run function performs
 * no allocation). */
size_t qd_workspace_bytes(const qd_config *cfg, int32_t batch, int32_t max_ctx,
                          int32_t prefill_tokens);

/* One decode step for `batch` sequences, one new token each: embedding,
 * every layer, final norm, lm_head and greedy argmax.
 *   tokens      [B] int32 token ids, or NULL when x_in is given
 *   x_in        [B][D] float input of layer 0 (block-only use), or NULL
 *   pos         [B] int32 device: tokens already cached = position of the new token
 *   pos_host    [B] int32 host copy of pos, used for checks and work partitioning
 *   logits      [B][V] float out, or NULL
 *   next_tokens [B] int32 out (greedy argmax of the logits), or NULL
 *   x_out       [B][D] float out: the last layer's output (before the final norm), or NULL
 *   layer_out   [n_layers][B][D] float out: residual stream after each layer, or NULL
 * tokens, pos, x_in and every output must be 4-byte aligned (QD_EALIGN).
 * The new token's K/V are written into every layer's cache at pos[b] before it
 * attends over positions 0..pos[b]; re-running at the same pos is idempotent.
 * lm_head / final_norm may be NULL only when logits and next_tokens are NULL.
 * HIP graphs: the launch configuration (attention splits, and at batch 2..16 the
 * grid of splits that hold keys) is planned from pos_host. A captured step
 * replays that plan, so a replay is valid only while every sequence's position
 * stays inside the captured plan: the same qd_decode_plan for the new positions
 * and no sequence reaching a split (chunk) it did not have at capture. Capture
 * again when a sequence crosses a chunk boundary. */
qd_status qd_decode_step(const qd_config *cfg, const qd_weights *w, const qd_kv *kv,
                         int32_t batch, const int32_t *tokens, const float *x_in,
                         const int32_t *pos, const int32_t *pos_host,
                         float *logits, int32_t *next_tokens, float *x_out, float *layer_out,
                         void *workspace, size_t workspace_bytes, void *stream);

/* qd_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * same step with the same arguments, minus the workspace: its scratch memory is
 * a static device array of QD_NOALLOC_SCRATCH_BYTES inside the library, one per
 * GPU (taken by the first call on that GPU, held until the process ends). The
 * call allocates nothing. A step whose workspace (qd_workspace_bytes) exceeds
 * that size returns QD_EWORKSPACE before anything is enqueued. Every call on a
 * GPU shares that GPU's scratch: calls that overlap on one GPU (different
 * streams, or different threads) race and must be serialised by the caller;
 * nothing of a call's scratch is read by the next (each step writes what it
 * reads). The stream's device is the GPU used. */
#define QD_NOALLOC_SCRATCH_BYTES (16u << 20)
qd_status qd_decode_step_noalloc(const qd_config *cfg, const qd_weights *w, const qd_kv *kv,
                                 int32_t batch, const int32_t *tokens, const float *x_in,
                                 const int32_t *pos, const int32_t *pos_host,
                                 float *logits, int32_t *next_tokens, float *x_out, float *layer_out,
                                 void *stream);

/* One decoder block over n_tokens consecutive tokens of sequence 0 of the block
 * table, at positions start_pos .. start_pos + n_tokens - 1, causal (row i
 * attends to positions 0..start_pos+i). bf16 weights only: the projections are
 * MFMA bf16 matrix products with float accumulation, their activation operands
 * rounded to bf16. x_in [N][D] in x_dtype (QD_BF16 or QD_F32); x_out [N][D] float;
 * both 16-byte aligned.
 * K/V of all N tokens are rotated once and written into layer `layer`'s cache
 * before any row attends (nanoinfer page, attention pitfalls: keys rotated once,
 * on insert, and the causal boundary is j <= i, a token attending to itself;
 * nanoserve day 49, lesson 1: this step's K/V are written before it attends).
 * Rows attend through the cache, so a chunk at start_pos > 0 sees every earlier
 * token already stored there. */
qd_status qd_prefill_block(const qd_config *cfg, const qd_layer *layer, int32_t layer_index,
                           const qd_kv *kv, int32_t n_tokens, int32_t start_pos,
                           const void *x_in, int32_t x_dtype, float *x_out,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Store already-rotated k and v ([B][Hkv][hd] float) of `batch` sequences at
 * positions pos[b] of layer `layer_index`, in the cache dtype (bf16: round half
 * to even; nanoinfer, phase 1). nanoinfer, phase 4: keys are rotated once, on
 * insert; this call only stores. */
qd_status qd_kv_append(const qd_config *cfg, const qd_kv *kv, int32_t layer_index,
                       int32_t batch, const int32_t *pos, const int32_t *pos_host,
                       const float *k, const float *v, void *stream);

/* Per-output-channel symmetric int8 weight quantization (nanoinfer, phase 6):
 * for each row r of the row-major [rows][cols] matrix w (w_dtype QD_F32 or
 * QD_BF16, widened exactly to float), scale[r] = max_k |w[r][k]| / 127 and
 * q[r][k] = round(w[r][k] / scale[r]), both quotients in float32 with IEEE
 * rounding, the integer rounding half away from zero (the range is [-127, 127],
 * so a weight and its negation give opposite codes); a row of zeros gets scale 0
 * and codes 0. q: int8 [rows][cols] out; scale: float [rows] out. cols must be a
 * multiple of 16 and every pointer 16-byte aligned. An offline weight
 * conversion: one workgroup per row, enqueued on `stream`. */
qd_status qd_quantize_rows_int8(const void *w, int32_t w_dtype, int64_t rows, int32_t cols,
                                int8_t *q, float *scale, void *stream);

/* One next token per row of logits [batch][vocab] (nanoinfer, phase 5), in the
 * page's order: temperature -> top-k -> top-p -> softmax -> inverse-CDF draw.
 *   temperature == 0: the argmax (lowest index on a tie); uniforms may be NULL.
 *   temperature  > 0: z = logits / temperature (float32); top-k keeps every token
 *     whose logit is >= the k-th largest (ties at the boundary stay), with
 *     1 <= top_k <= 1024; top_k <= 0 or >= vocab applies no top-k (top-p over
 *     the whole vocabulary, the page's "top-p alone"; other values:
 *     QD_EUNSUPPORTED); top-p in (0, 1] sorts
 *     the survivors ascending by (z, token id), takes the float32 cumulative sum
 *     of their softmax probabilities in that order, one term at a time, and
 *     removes every token whose sum is <= float32(1 - top_p), keeping at least
 *     the largest (top_p = 1 removes none); the kept tokens, in token-id order,
 *     are drawn by the first whose running probability exceeds u * total, with
 *     u = uniforms[b] in [0, 1) supplied by the caller.
 *   tokens [batch] int32 out (-1 only for a row of NaN logits, which yields no
 *     candidate). Any number of logits may tie at the top-k boundary; past 2048
 *     candidates the row's draw reads it in token order (slower, same rule).
 *     Without top-k the cut and the draw sum the probabilities in another order
 *     than one at a time (the rule is the same; a row whose decision lies within
 *     that rounding of a boundary may land on its other side).
 * One workgroup per row, enqueued on `stream`; no device memory is used beyond
 * the arguments. */
qd_status qd_sample(const float *logits, int32_t batch, int32_t vocab, float temperature,
                    int32_t top_k, float top_p, const float *uniforms, int32_t *tokens,
                    void *stream);

/* Kernel kinds for the optional event timing below. */
typedef enum {
    QD_K_EMBED = 0, QD_K_QKV = 1, QD_K_QKV_POST = 2, QD_K_ATTN = 3, QD_K_MERGE = 4,
    QD_K_O = 5, QD_K_GATEUP = 6, QD_K_DOWN = 7, QD_K_LMHEAD = 8, QD_K_ARGMAX = 9,
    QD_K_PREFILL_GEMM = 10, QD_K_PREFILL_ATTN = 11, QD_K_OTHER = 12,
    QD_K_STEP = 13   /* the batch-1 one-launch step kernel */
} qd_kernel_kind;

/* Measurement hook, off by default: while bit k of kind_mask is set, every launch
 * of kernel kind k records a HIP event on the call's stream just before and just
 * after it (process-wide, up to 8192 launches until the next enable or reset).
 * qd_profile_read waits for those events and returns the number of timed launches
 * of `kind` and their summed durations in milliseconds. Not thread-safe; meant
 * for benchmarks. The first enable creates the events (no device allocation). */
int32_t qd_profile_enable(uint32_t kind_mask);
int32_t qd_profile_read(int32_t kind, int32_t *launches, double *total_ms);
void qd_profile_reset(void);

/* Message for the last non-OK status returned on this thread ("" if none).
 * Every unsupported or invalid request returns its own status with a message and
 * enqueues nothing; nothing falls back to another implementation (ForgeML page,
 * ONNX subset: what lies outside the supported set fails explicitly instead of
 * falling back). */
const char *qd_last_error(void);

/* QD_ABI_VERSION of the loaded library, for a binding to check that it was
 * built against this header (no passage defines it: a build convention). */
int32_t qd_abi_version(void);

/* How qd_decode_step would run `batch` sequences whose longest context is
 * max_tokens (largest position + 1): a host-only query, no device work. Lets a
 * caller (or a test) see which kernels a step takes, and whether a captured
 * graph stays valid for new positions (same plan). QD_ECAPACITY when the
 * context needs more attention splits than one merge combines. */
typedef struct {
    int32_t chunk;                  /* keys per attention split                               */
    int32_t splits;                 /* attention splits of the longest sequence               */
    int32_t heads_per_wg;           /* query heads per attention workgroup                    */
    int32_t matrix_core_attention;  /* 1: the MFMA grouped attention kernel                    */
    int32_t qkv_partials;           /* > 0: q|k|v as that many K-range partial products,      *
                                     * finished inside the attention kernel                   */
    int32_t merge_in_o_proj;        /* 1: batch 1, o_proj merges the splits (no merge launch); *
                                     * 2: batch 1, o_proj by head slices, each merging its    *
                                     * head's splits, the slices added into the residual with *
                                     * float atomics (no merge launch; off when               *
                                     * QD_DETERMINISTIC=1 or QD_O_HEADS=0 is set)             */
    int32_t step_kernel;            /* 1: batch 1 eligible for the one-launch step, taken      *
                                     * when QD_STEP_KERNEL=1 is set in the environment        */
    int32_t fused_qkv;              /* 1: batch 1, the q|k|v projection runs inside the        *
                                     * attention launch (no projection launch); off when      *
                                     * QD_FUSED_QKV=0 is set in the environment               */
} qd_decode_plan_info;
qd_status qd_decode_plan(const qd_config *cfg, int32_t batch, int32_t max_tokens,
                         qd_decode_plan_info *out);

#ifdef __cplusplus
}
#endif
#endif /* QD_H */
