// Host-side launchers of the libqd kernels. Each returns hipSuccess or the
// launch error; shapes are checked by the C-ABI layer before these run.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qd {

enum Epi { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };

// y[b][row] (op)= sum_k W[row][k] * xn[b][k], where xn = x, or the RMSNorm of x
// with `gain` when gain != nullptr. Rows come from up to three row-major
// segments stacked in order (q/k/v; unused seg_end entries = N); SWIGLU reads row r of w[0] (gate) and of
// w[1] (up) and stores silu(gate) * up.
struct GemvArgs {
    const void* w[3];
    const void* bias[3];
    int seg_end[3];
    int nseg;
    int N, K, B;
    const float* x;
    const void* gain;
    float eps;
    float* y;
    float* part_val;   // EPI_LOGITS: per-(b, workgroup) best value
    int* part_idx;     //             and its row
    int kt;            // K elements staged in LDS per pass
    unsigned* zero_ptr;  // optional: workgroup 0 stores zeros here (counters of a later kernel)
    int zero_n;
    // optional, batch-1 residual product only: x is the decode attention's context,
    // merged here from its split partials (AttnArgs::part / part_ml, [Hq][S]) with
    // ns = ceil((pos[0] + 1) / part_chunk) valid splits; then K = Hq * part_hd
    const float* part;
    const float2* part_ml;
    const int* part_pos;
    int part_S, part_chunk, part_hd;
    // optional, with part: the new token comes as one more split, from the
    // attention's projection output (AttnArgs::fq_out: rotated q [Hq][hd], then the
    // stored k and v of the Hkv = part_kv_heads KV heads): its score is q . k_new
    // times part_scale2 (1/sqrt(hd) * log2 e), its weight sum 1 and its output
    // v_new; the other splits cover positions 0 .. pos[0] - 1
    const float* part_new;
    int part_kv_heads;
    float part_scale2;
    // int8 weights: float scale of each row, per segment (SWIGLU: [0] gate, [1] up);
    // the product of row r is scaled by it
    const float* wscale[3];
    // batch 2..16 residual products (launch_gemm16, EPI_RESID): nonzero takes one K
    // range per output block (no float atomics, bitwise repeatable)
    int deterministic;
    // optional, batch 2..16 normed store product (launch_gemm16, EPI_STORE) cut into
    // gemm16_store_splits(K, N) K ranges: y receives [splits][B][N] partial products
    // (neither the RMSNorm scale nor the bias applied) and ss_out [splits][B] the
    // partial sums of squares of x over each range; the consumer finishes
    float* ss_out;
};
// batch 1..16 on the vector ALUs (qd_decode.hip); w_type 0 float, 1 bf16, 2 int8 rows
// with a.wscale (K and a.kt multiples of 16)
hipError_t launch_gemv(const GemvArgs& a, int w_type, int epi, int grid_cap, int* grid_out,
                       hipStream_t s);
// batch-1 fast path (qd_gemv.hip); part_val/part_idx hold one entry per workgroup;
// w_type 0 float, 1 bf16, 2 int8 rows with a.wscale (K a multiple of 16)
hipError_t launch_gemv1(const GemvArgs& a, int w_type, int epi, int grid_cap, int* grid_out,
                        hipStream_t s);
int gemv_rows_per_tile(int K);
// most attention splits launch_gemv1 merges itself (GemvArgs::part)
int gemv1_merge_max_splits();
// batch 1, bf16 rows: the residual product by head slices over the attention's
// split partials (GemvArgs::part, part_ml, part_pos, part_S <= 64, part_chunk,
// part_hd 64 or 128), adding into y with float atomics
hipError_t launch_oproj_heads(const GemvArgs& a, hipStream_t s);
// batch 2..16 on the matrix cores (qd_gemm16.hip): w_type 1 bf16 rows, 2 int8 rows
// with a.wscale (K a multiple of 16, widened to bf16 exactly); a.kt must be
// gemm16_chunk(a.K); part_val/part_idx hold [B][grid] entries
hipError_t launch_gemm16(const GemvArgs& a, int w_type, int epi, int grid_cap, int* grid_out, hipStream_t s);
int gemm16_chunk(int K);
// K ranges of a normed store product given GemvArgs::ss_out (1: no partial form)
int gemm16_store_splits(int K, int N);
constexpr int kGemm16MaxStoreSplits = 3;

// Decode attention with the q/k norm, RoPE, the new token's KV append and the
// split merge fused in (one launch per layer); see qd_attention.hip.
constexpr int kAttnMaxBatch = 16;   // sequences of one decode step at most
struct AttnArgs {
    const float* qkv;       // [B][Hq*hd + 2*Hkv*hd] projections (bias added)
    void* k_cache;
    void* v_cache;          // page pools [pages][Hkv][page][hd]
    const int* block_table;
    int max_blocks, num_pages;
    const int* pos;
    int capacity;           // max_blocks * page
    const void* q_norm;
    const void* k_norm;
    int qk_norm;
    float eps, theta;
    float* part;            // [B][Hq][S][hd]: o of each split (sum of e^(s - m) v)
    float2* part_ml;        // [B][Hq][S]: (m, l) of each split, m in base-2 units
    int part_always;        // publish (o, m, l) even when the context fits one split
                            // (batch 1: the o_proj GEMV merges the splits itself)
    const float2* rope;     // [B][hd/2] (cos, sin) of the step's positions
    float* ctx;             // [B][Hq*hd]
    int Hq, Hkv, hd, page, chunk, S, B;
    int hpw;                // query heads per workgroup
    float scale;
    // prefill mode (prefill_start >= 0): work item z is row z of one sequence at
    // position prefill_start + z, its q already normed and rotated in q_rot
    // [rows][Hq][hd], its K/V already in the cache (block table row 0)
    int prefill_start;
    const float* q_rot;
    // qkv_slabs > 0 (matrix-core kernel, bf16 weights only): qkv holds that many K-range partial
    // products of the q|k|v projection (slab stride qkv_slab_stride floats), without
    // the RMSNorm scale or the bias; qkv_ss [slabs][B] holds the partial sums of
    // squares of the normed input (x_dim elements) and qkv_bias the q, k and v biases
    // (the weights' type, NULL: none). The kernel forms r * sum + bias itself.
    int qkv_slabs;
    long qkv_slab_stride;
    const float* qkv_ss;
    const void* qkv_bias[3];
    const float* qkv_scale[3];   // int8 rows: the q, k and v row scales (NULL: bf16 rows)
    int x_dim;
    // optional (matrix-core kernel): a one-dimensional grid of only the splits that
    // hold keys, sequence b's at wg_base[b] .. wg_base[b + 1] - 1 (split-major, then
    // KV head), from the host copy of the positions; wg_base[0] = 0, B + 1 entries
    int compact;
    int wg_base[kAttnMaxBatch + 1];
    // optional, batch 1 (fq = 1): the q|k|v projection is formed inside the
    // attention launch instead of read from qkv. One query head per workgroup, bf16
    // or int8 rows (fq_scale), hd 64, no per-head norm, x_dim <= kFqMaxD and a
    // multiple of 8 (bf16) or 16 (int8). The
    // grid is one-dimensional: the attention workgroups (one per split and query
    // head, the splits of a head on one XCD), each projecting its query head from
    // x (RMSNorm with fq_gain and eps, rows of fq_w[0], bias qkv_bias[0]) and
    // rotating it, then 2 * Hkv workgroups that
    // project the new token's k (rotated) and v of one KV head (fq_w[1], fq_w[2],
    // biases qkv_bias[1], qkv_bias[2]) and store them in the cache at the position.
    // The attention then covers the cached positions 0 .. p - 1 only, and fq_out
    // ([Hq + 2 Hkv][hd]) receives the rotated query heads followed by the new k and
    // v rows as stored (widened to float), from which the residual product adds
    // the new token as one more split (needs part_always).
    int fq;
    const float* fq_x;
    const void* fq_gain;
    const void* fq_w[3];
    const float* fq_scale[3];   // int8 rows: the q, k and v row scales (NULL: bf16 rows)
    float* fq_out;
    // batch 1 with the projection in the launch, first layer (fq_tok != NULL): x is
    // the embedding row of token fq_tok[0] (int8 rows: times fq_embed_scale of the
    // token; an id outside [0, fq_vocab) gives a zero row) and the RoPE table is
    // formed in the launch; workgroup 0 stores both (x to fq_x, the table to rope)
    // for the launches that follow, in place of the step-input launch
    const int* fq_tok;
    const void* fq_embed;
    const float* fq_embed_scale;
    int fq_vocab;
};
constexpr int kFqMaxD = 1024;
// attention kernel, plus the split merge kernel when S > 1
hipError_t launch_attention(const AttnArgs& a, int w_is_bf16, int kv_is_bf16, hipStream_t s);
// whether launch_attention takes the matrix-core grouped kernel for these arguments
bool attn_uses_mfma(const AttnArgs& a, int kv_is_bf16);
// whether these arguments allow the projection in the attention launch (fq);
// w_type 1 bf16 rows, 2 int8 rows
bool attn_fq_ok(const AttnArgs& a, int w_type, int kv_is_bf16);
int attn_max_chunk(int hd, int kv_is_bf16, int grouped);
int attn_max_splits();

// Causal prefill attention on the matrix cores (qd_prefill_attn.hip): bf16 K/V
// cache, q rotated in float32 [rows][Hq][hd], context out in bf16 [rows][Hq*hd].
struct PrefillAttnArgs {
    const float* q;
    const void* k_cache;
    const void* v_cache;      // page pools [pages][Hkv][page][hd], bf16
    const int* block_table;   // the sequence's row
    int num_pages;
    int rows, start;          // query row i sits at position start + i
    int Hq, Hkv, hd, page;
    float scale;
    uint16_t* out;
};
hipError_t launch_prefill_attn_mfma(const PrefillAttnArgs& a, hipStream_t s);

// Batch-1 decode step as one persistent cooperative launch (qd_step.hip): bf16
// weights and KV, one workgroup per CU, activations exchanged as tagged 64-bit
// words. Pointers of every layer travel in the arguments.
constexpr int kStepWgs = 256;
constexpr int kStepMaxLayers = 64;
struct StepLayer {
    const void *attn_norm, *wq, *wk, *wv, *bq, *bk, *bv, *q_norm, *k_norm;
    const void *wo, *mlp_norm, *w_gate, *w_up, *w_down;
    void *kc, *vc;           // the layer's K and V page pools
};
struct StepArgs {
    int L, D, Hq, Hkv, hd, G, F, V, qkvr;
    float eps, scale;
    int qk_norm, has_bias;
    int S, C;                // attention splits of C keys (C a multiple of 64)
    int up_wa, up_wb, down_wa, down_wb;   // gate|up and down row weights: XCDs < Hkv, the others
    const int* pos;
    const int* block_table;  // row 0
    int max_blocks, num_pages;
    const void* final_norm;
    const void* lm_head;     // NULL: no head
    float* logits;           // [V]
    float* x_out;            // [D] or NULL
    float* layer_out;        // [L][D] or NULL
    float* argmax_val;       // [kStepWgs] per-workgroup partials
    int* argmax_idx;
    float *xb, *y, *h;       // vectors read across XCDs, two layer parities each: x [2][D],
                             // y [2][Hkv][D], h [2][F]
    unsigned long long *qkv, *part;   // tagged words read within an XCD, two parities each
    long part_stride;        // words per parity of part
    uint32_t* cnt;           // completion counters [3][kStepMaxLayers][8 XCDs][32]
    float2* rope;            // [hd/2] (cos, sin) of the step's position
    uint32_t* err;           // [4]: abort flag, code of the wait that gave up
    unsigned long long* clear_from;   // words the prologue clears: tagged words and counters
    long clear_n;
    StepLayer layer[kStepMaxLayers];
};
// the prologue (embedding or x_in, RoPE table, cleared tags), then the step kernel
hipError_t launch_step_prologue(const StepArgs& a, const int* tokens, const void* embed, const float* x_in,
                                float theta, hipStream_t s);
hipError_t launch_step_kernel(const StepArgs& a, hipStream_t s);

// x = embedding rows of `tokens` (or a copy of x_in), plus the RoPE table of the
// step's positions (qd_attention.hip).
struct StepInputArgs {
    const int* tokens;
    const void* embed;
    const float* embed_scale;   // int8 embedding: row scales
    const float* x_in;
    float* x;
    const int* pos;
    float2* rope;           // [B][hd/2]
    int B, D, V, hd;
    float theta;
};
hipError_t launch_step_input(const StepInputArgs& a, int w_type, hipStream_t s);   // 0 f32, 1 bf16, 2 int8

hipError_t launch_copy(const float* src, float* dst, long n, hipStream_t s);
hipError_t launch_argmax(const float* part_val, const int* part_idx, int nparts, int* out, int B,
                         hipStream_t s);
hipError_t launch_kv_append(const float* k, const float* v, void* k_cache, void* v_cache,
                            const int* block_table, int max_blocks, int num_pages, const int* pos,
                            int capacity, int Hkv, int hd, int page, int B, int kv_is_bf16,
                            hipStream_t s);

// Prefill block (qd_prefill.hip).
enum GemmEpi { GEMM_STORE = 0, GEMM_RESID = 1, GEMM_SWIGLU = 2 };
struct GemmArgs {
    const void* A;          // bf16 [M][K]
    const void* w[3];       // bf16 row-major [rows][K] segments (SWIGLU: w[0] gate, w[1] up)
    const void* bias[3];    // GEMM_STORE: optional per-segment bias (bf16)
    int seg_end[3];         // cumulative rows of the segments (unused entries = N)
    int M, N, K;            // N = output columns (SWIGLU: h columns)
    void* C;                // float [M][ldc] (STORE, RESID) or bf16 [M][ldc] (SWIGLU)
    int ldc;
};
// splits > 1 (not for SwiGLU): K is cut into that many ranges whose partial products
// are added into C with float atomics (RESID: onto the residual; STORE: C zeroed
// beforehand, bias added by the first range); splits = 0 picks a value
hipError_t launch_mfma_gemm(const GemmArgs& a, int epi, int splits, hipStream_t s);
int mfma_gemm_splits(const GemmArgs& a, int epi);
// Wide-tile products with float32 partial slabs: mfma_gemm_slabs gives the number
// of K ranges (slabs) the plan takes for an M x N x K product (0: not this path);
// launch_mfma_gemm_slabs writes slab s of C = A W^T over K range s to
// a.C + s * M * ldc (no bias; the consumer adds the slabs and the bias).
int mfma_gemm_slabs(int M, int N, int K, int epi);
hipError_t launch_mfma_gemm_slabs(const GemmArgs& a, int slabs, hipStream_t s);
// x[i] += sum of the nslab slabs part[s * stride + i], i < n
hipError_t launch_add_slabs(float* x, const float* part, int nslab, long stride, long n, hipStream_t s);

struct PrefillNormArgs {
    const void* x_bf16;     // input rows, bf16 ... or
    const float* x_f32;     // ... float (exactly one is set)
    float* x_res;           // optional: input widened into the float32 residual
    const void* gain;
    uint16_t* out;          // bf16 [rows][D]
    int rows, D;
    float eps;
    float* zero;            // optional: zero_n floats cleared (the next split-K GEMM's output)
    long zero_n;
    const float* part;      // optional (with x_f32): nslab float32 slabs [rows][D], slab_stride
    int nslab;              // floats apart, added to the input row (x_res gets the sum)
    long slab_stride;
};
hipError_t launch_prefill_norm(const PrefillNormArgs& a, int w_is_bf16, hipStream_t s);

struct PrefillRopeArgs {
    const float* qkv;       // [rows][Hq*hd + 2*Hkv*hd]
    float* q_out;           // [rows][Hq][hd]
    void* k_cache;
    void* v_cache;
    const int* block_table; // the sequence's row of the block table
    int num_pages, capacity, start, rows;
    const void* q_norm;
    const void* k_norm;
    int qk_norm;
    float eps, theta;
    int Hq, Hkv, hd, page;
    int nslab;              // qkv holds nslab partial slabs slab_stride floats apart (0 or 1: one)
    long slab_stride;
    const void* bias[3];    // with slabs: optional bf16 q/k/v biases, segments ending at seg_end
    int seg_end[3];
};
hipError_t launch_prefill_rope_append(const PrefillRopeArgs& a, int w_is_bf16, int kv_is_bf16, hipStream_t s);
hipError_t launch_to_bf16(const float* x, void* y, long n, hipStream_t s);

// Temperature / top-k / top-p sampling of one token per row of logits (qd_sample.hip).
constexpr int kSampleMaxK = 1024;
struct SampleArgs {
    const float* logits;    // [B][V]
    int B, V;
    float temperature;      // 0: argmax
    int top_k;              // 1 .. kSampleMaxK when temperature > 0, or <= 0 / >= V: no top-k
    float top_p;            // (0, 1]; 1 keeps every top-k candidate
    float one_minus_p;      // the top-p threshold, float32(1 - p) formed in double
    const float* uniforms;  // [B] in [0, 1)
    int* tokens;            // [B] out
};
hipError_t launch_sample(const SampleArgs& a, hipStream_t s);

// Per-row symmetric int8 quantization of a [rows][cols] matrix (qd_quant.hip).
hipError_t launch_quantize_rows(const void* w, int w_is_bf16, long rows, int cols, int8_t* q, float* scale,
                                hipStream_t s);

}  // namespace qd
