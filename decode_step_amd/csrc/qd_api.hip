// C ABI of libqd (declared in include/qd.h): argument checks on the host, the
// workspace plan, and the in-order launch sequence of one decode step on the
// caller's stream. Nothing here allocates, synchronises or reads device memory.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/qd.h"
#include "qd_launch.h"
#include "qd_step_sched.h"
#include <cmath>
#include <cstdlib>

namespace {

thread_local std::string g_err;

qd_status fail(qd_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr int kMaxBatch = 16;
constexpr int kLogitsGridCap = 2048;  // workgroups of the lm_head GEMV = argmax partials per row
constexpr int kGemvGridCap = 4096;
#ifndef QD_GEMV1_GRID_CAP
#define QD_GEMV1_GRID_CAP 512
#endif
constexpr int kGemv1GridCap = QD_GEMV1_GRID_CAP;   // batch-1 projections grid-stride beyond this
constexpr size_t kGemvLds = 60 * 1024;   // dynamic LDS of the GEMV, below the 64 KB launch limit

qd_status check_config(const qd_config* c) {
    if (!c) return fail(QD_EINVAL, "cfg is NULL");
    if (c->n_layers < 1 || c->hidden < 8 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->ffn < 8 ||
        c->vocab < 1)
        return fail(QD_ESHAPE, "config sizes must be positive (layers %d hidden %d heads %d/%d ffn %d vocab %d)",
                    c->n_layers, c->hidden, c->n_q_heads, c->n_kv_heads, c->ffn, c->vocab);
    if (c->hidden % 8 || c->ffn % 8)
        return fail(QD_ESHAPE, "hidden (%d) and ffn (%d) must be multiples of 8", c->hidden, c->ffn);
    if (c->hidden > 16384) return fail(QD_ESHAPE, "hidden %d > 16384", c->hidden);
    if (c->head_dim != 64 && c->head_dim != 128)
        return fail(QD_ESHAPE, "head_dim %d not in {64, 128}", c->head_dim);
    if (c->n_q_heads % c->n_kv_heads)
        return fail(QD_ESHAPE, "n_q_heads %d not a multiple of n_kv_heads %d", c->n_q_heads, c->n_kv_heads);
    if (c->n_q_heads / c->n_kv_heads > 8)
        return fail(QD_ESHAPE, "group %d > 8", c->n_q_heads / c->n_kv_heads);
    if (c->page_size != 16) return fail(QD_ESHAPE, "page_size %d != 16", c->page_size);
    if ((c->w_dtype != QD_F32 && c->w_dtype != QD_BF16 && c->w_dtype != QD_I8) ||
        (c->kv_dtype != QD_F32 && c->kv_dtype != QD_BF16))
        return fail(QD_EINVAL, "dtype out of range (w %d kv %d)", c->w_dtype, c->kv_dtype);
    if (c->w_dtype == QD_I8 && (c->hidden % 16 || c->ffn % 16))
        return fail(QD_ESHAPE, "int8 weights need hidden (%d) and ffn (%d) multiples of 16", c->hidden, c->ffn);
    if (!(c->rms_eps > 0.f) || !(c->rope_theta > 0.f))
        return fail(QD_ESHAPE, "rms_eps and rope_theta must be > 0");
    return QD_OK;
}

struct DecodePlan {
    int B, D, Hq, Hkv, hd, G, F, V, qkvr;
    int chunk, S;
    size_t off_x, off_qkv, off_qss, off_part, off_rope, off_ctx, off_h, off_logits, off_pv, off_pi, total;
    // batch-1 one-launch step: tagged words (two layer parities each), argmax partials,
    // RoPE table, error words
    int step_S;   // attention splits the part region holds
    size_t off_sxb, off_scnt, off_sqkv, off_spart, off_sy, off_sh, off_send, off_sam_v, off_sam_i, off_srope, off_serr;
};



// Attention work split. Grouped: one workgroup holds all query heads of a KV
// head (each K/V row is read once) and a split of `chunk` tokens, the chunk
// sized so the (sequence, KV head, split) items come to about kAttnTargetWgs
// workgroups, at least kAttnMinChunk tokens and at most what one workgroup
// holds in registers. When that leaves fewer than kAttnMinWgs workgroups (one
// short sequence), the query heads go to separate workgroups instead (hpw = 1)
// with the largest chunk, which spreads the score and value arithmetic over
// more CUs. Returns false when the context needs more splits than one merge
// combines.
#ifndef QD_ATTN_TARGET
#define QD_ATTN_TARGET 1024
#endif
constexpr int kAttnTargetWgs = QD_ATTN_TARGET;
constexpr int kAttnMinWgs = 128;
constexpr int kAttnMinChunk = 64;
#ifndef QD_B1_CHUNK
#define QD_B1_CHUNK 144     // tokens per split at batch 1 (o_proj merges the splits)
#endif
#ifndef QD_B1_WIDE_SPLITS
#define QD_B1_WIDE_SPLITS 32   // most splits of a batch-1 step whose o_proj cannot merge them itself
#endif
#ifndef QD_B1_HPW
#define QD_B1_HPW 1         // query heads per workgroup at batch 1 (0: the whole group)
#endif

// Batch-1 decode whose o_proj GEMV merges the attention splits itself (no merge
// launch): splits of at least QD_B1_CHUNK tokens, at most gemv1_merge_max_splits()
// of them, each small enough for the grouped attention kernel. Needs the context
// vector (Hq * hd) within 1024 and Hq within 32.
static bool plan_b1_merge(const qd_config* c, int max_tokens, int* chunk, int* S, int* hpw) {
    const int pg = c->page_size, G = c->n_q_heads / c->n_kv_heads;
    const int qdim = c->n_q_heads * c->head_dim;
    if (qdim > 1024 || c->n_q_heads > 32 || c->head_dim % 4) return false;
    const int ch_max = qd::attn_max_chunk(c->head_dim, c->kv_dtype == QD_BF16, 1) / pg * pg;
    const int T = max_tokens < 1 ? 1 : max_tokens;
    const int smax = qd::gemv1_merge_max_splits();
    int ch = (T + smax - 1) / smax;
    if (ch < QD_B1_CHUNK) ch = QD_B1_CHUNK;
    ch = (ch + pg - 1) / pg * pg;
    if (ch > ch_max) return false;
    *chunk = ch;
    *S = (T + ch - 1) / ch;
    *hpw = (QD_B1_HPW > 0 && QD_B1_HPW < G) ? QD_B1_HPW : G;
    return true;
}

bool plan_split(const qd_config* c, int B, int max_tokens, int* chunk, int* S, int* hpw, bool* merge_in_o = nullptr) {
    // B = sequences (decode) or query rows (prefill); max_tokens = longest context.
    // merge_in_o != nullptr: a decode step, whose batch-1 form may merge in o_proj
    if (merge_in_o) *merge_in_o = false;
    if (merge_in_o && B == 1 && plan_b1_merge(c, max_tokens, chunk, S, hpw)) {
        *merge_in_o = true;
        return true;
    }
    const int pg = c->page_size;
    const int ch_max = qd::attn_max_chunk(c->head_dim, c->kv_dtype == QD_BF16, 1) / pg * pg;
    const int ch_wide = qd::attn_max_chunk(c->head_dim, c->kv_dtype == QD_BF16, 0) / pg * pg;
    const long work = (long)B * c->n_kv_heads;
    const int tokens = max_tokens < 1 ? 1 : max_tokens;
    long ch = (tokens * work + kAttnTargetWgs - 1) / kAttnTargetWgs;
    ch = (ch + pg - 1) / pg * pg;
    if (ch < kAttnMinChunk) ch = kAttnMinChunk;
    const long need = (tokens + qd::attn_max_splits() - 1) / qd::attn_max_splits();   // merge capacity
    if (ch < need) ch = (need + pg - 1) / pg * pg;
    // a batch-1 decode step: at most QD_B1_WIDE_SPLITS splits where the chunk allows
    // (fewer partials for the residual product to merge)
    const long need1 = (tokens + QD_B1_WIDE_SPLITS - 1) / QD_B1_WIDE_SPLITS;
    if (merge_in_o && B == 1 && ch < need1) ch = (need1 + pg - 1) / pg * pg;
    if (ch > ch_max) ch = ch_max;
    *chunk = (int)ch;
    *S = (tokens + *chunk - 1) / *chunk;
    *hpw = c->n_q_heads / c->n_kv_heads;
    if ((long)(*S) * work < kAttnMinWgs && *hpw > 1) {
        *chunk = ch_wide;
        *S = (tokens + ch_wide - 1) / ch_wide;
        *hpw = 1;
    } else if (*S > qd::attn_max_splits()) {   // beyond the grouped chunk: the wide one
        *chunk = ch_wide;
        *S = (tokens + ch_wide - 1) / ch_wide;
    }
    return *S <= qd::attn_max_splits();
}

DecodePlan plan_decode(const qd_config* c, int B, int S, int chunk) {
    DecodePlan p{};
    p.B = B; p.D = c->hidden; p.Hq = c->n_q_heads; p.Hkv = c->n_kv_heads; p.hd = c->head_dim;
    p.G = p.Hq / p.Hkv; p.F = c->ffn; p.V = c->vocab;
    p.qkvr = (p.Hq + 2 * p.Hkv) * p.hd;
    p.chunk = chunk; p.S = S;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = round_up(o + bytes, 256); return at; };
    p.off_x = take(sizeof(float) * B * p.D);
    // q|k|v, or (batch 2..16) its K-range partial products and their sums of squares
    p.off_qkv = take(sizeof(float) * qd::kGemm16MaxStoreSplits * B * p.qkvr);
    p.off_qss = take(sizeof(float) * qd::kGemm16MaxStoreSplits * B);
    p.off_part = take(sizeof(float) * (size_t)B * p.Hq * S * (p.hd + 2));
    p.off_rope = take(sizeof(float) * 2 * B * (p.hd / 2));
    p.off_ctx = take(sizeof(float) * B * p.Hq * p.hd);
    p.off_h = take(sizeof(float) * (size_t)B * p.F);
    p.off_logits = take(sizeof(float) * (size_t)B * p.V);
    p.off_pv = take(sizeof(float) * B * kLogitsGridCap);
    p.off_pi = take(sizeof(int) * B * kLogitsGridCap);
    p.step_S = 0;
    if (B == 1 && qd::step::step_config_ok(c)) {
        const int S1 = qd::step::step_split_cap(c);
        p.step_S = S1;
        const size_t w = sizeof(unsigned long long);
        p.off_sxb = take(sizeof(float) * 2 * p.D);
        p.off_sy = take(sizeof(float) * 2 * (size_t)p.Hkv * p.D);
        p.off_sh = take(sizeof(float) * 2 * (size_t)p.F);
        p.off_sqkv = o;   // the prologue clears from here to off_send: tagged words, then counters
        o += w * 2 * p.qkvr;
        p.off_spart = o; o += w * 2 * (size_t)p.Hkv * S1 * p.G * (p.hd + 2);
        p.off_scnt = o; o += sizeof(uint32_t) * 3 * qd::kStepMaxLayers * 8 * 32;
        p.off_send = o;
        o = round_up(o, 256);
        p.off_sam_v = take(sizeof(float) * qd::kStepWgs);
        p.off_sam_i = take(sizeof(int) * qd::kStepWgs);
        p.off_srope = take(sizeof(float) * 2 * (p.hd / 2));
        p.off_serr = take(sizeof(uint32_t) * 4);
    }
    p.total = o;
    return p;
}

struct PrefillPlan {
    size_t off_nrm, off_qkv, off_q, off_part, off_ctx, off_ctxb, off_h, off_slab, total;
    int slabs_qkv, slabs_o, slabs_down;   // K-range slabs of the wide-tile products (0: other kernels)
};

PrefillPlan plan_prefill(const qd_config* c, int N, int S) {
    PrefillPlan p{};
    const int qkvr = (c->n_q_heads + 2 * c->n_kv_heads) * c->head_dim;
    const size_t qdim = (size_t)c->n_q_heads * c->head_dim;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = round_up(o + bytes, 256); return at; };
    p.off_nrm = take(2 * (size_t)N * c->hidden);            // bf16 normed rows (reused by the MLP norm)
    p.off_qkv = take(4 * (size_t)N * qkvr);
    p.off_q = take(4 * (size_t)N * qdim);
    p.off_part = take(4 * (size_t)N * qdim / c->head_dim * S * (c->head_dim + 2));
    p.off_ctx = take(4 * (size_t)N * qdim);
    p.off_ctxb = take(2 * (size_t)N * qdim);
    p.off_h = take(2 * (size_t)N * c->ffn);
    p.slabs_qkv = qd::mfma_gemm_slabs(N, qkvr, c->hidden, qd::GEMM_STORE);
    p.slabs_o = qd::mfma_gemm_slabs(N, c->hidden, (int)qdim, qd::GEMM_RESID);
    p.slabs_down = qd::mfma_gemm_slabs(N, c->hidden, c->ffn, qd::GEMM_RESID);
    const size_t slab_floats = std::max((size_t)p.slabs_qkv * qkvr,
                                        (size_t)std::max(p.slabs_o, p.slabs_down) * c->hidden) * (size_t)N;
    p.off_slab = take(4 * slab_floats);   // one region: each product's slabs are consumed before the next
    p.total = o;
    return p;
}

int gemv_kt(int B, int K) {
    int kt = (int)(kGemvLds / (sizeof(float) * (size_t)B));
    kt = kt / 64 * 64;
    return kt >= K ? K : kt;
}

// Optional event timing of selected kernel kinds (qd_profile_*): when a kind is
// enabled, a HIP event is recorded on the caller's stream just before and just
// after each of its launches; the pairs are read back only by qd_profile_read.
constexpr int kProfSlots = 8192;
struct ProfState {
    bool ready = false;
    uint32_t mask = 0;
    int next = 0;
    hipEvent_t ev[2 * kProfSlots];
    int kind[kProfSlots];
};
ProfState g_prof;

inline int prof_begin(int kind, hipStream_t s) {
    if (!(g_prof.mask & (1u << kind)) || g_prof.next >= kProfSlots) return -1;
    const int slot = g_prof.next++;
    g_prof.kind[slot] = kind;
    (void)hipEventRecord(g_prof.ev[2 * slot], s);
    return slot;
}
inline void prof_end(int slot, hipStream_t s) {
    if (slot >= 0) (void)hipEventRecord(g_prof.ev[2 * slot + 1], s);
}

#define QD_LAUNCH_K(kind, expr, name)                                                   \
    do {                                                                               \
        const int slot_ = prof_begin((kind), s);                                       \
        hipError_t e_ = (expr);                                                        \
        prof_end(slot_, s);                                                            \
        if (e_ != hipSuccess) return fail(QD_EHIP, "%s launch failed: %s", name, hipGetErrorString(e_)); \
    } while (0)
#define QD_LAUNCH(expr, name) QD_LAUNCH_K(QD_K_OTHER, expr, name)

qd_status check_layer(const qd_config* c, const qd_layer* L, int l) {
    const void* need[] = {L->attn_norm, L->wq, L->wk, L->wv, L->wo, L->mlp_norm, L->w_gate, L->w_up, L->w_down};
    const char* names[] = {"attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"};
    for (int i = 0; i < 9; ++i) {
        if (!need[i]) return fail(QD_EINVAL, "layer %d: %s is NULL", l, names[i]);
        if (!aligned16(need[i])) return fail(QD_EALIGN, "layer %d: %s not 16-byte aligned", l, names[i]);
    }
    if (c->qk_norm && (!L->q_norm || !L->k_norm))
        return fail(QD_EINVAL, "layer %d: qk_norm set but q_norm/k_norm NULL", l);
    if (c->w_dtype == QD_I8) {
        const float* sc[] = {L->s_q, L->s_k, L->s_v, L->s_o, L->s_gate, L->s_up, L->s_down};
        for (const float* p : sc)
            if (!p || ((uintptr_t)p & 3u)) return fail(QD_EINVAL, "layer %d: int8 row scales NULL or misaligned", l);
    }
    const void* opt[] = {L->bq, L->bk, L->bv, L->q_norm, L->k_norm};
    for (const void* p : opt)
        if (p && !aligned4(p)) return fail(QD_EALIGN, "layer %d: bias/gain not 4-byte aligned", l);
    return QD_OK;
}

// Batch-1 steps form the q|k|v projection inside the attention launch when the
// shape allows it (qd::attn_fq_ok); QD_FUSED_QKV=0 in the environment keeps the
// separate projection launch (read at every call, so a process can compare the two).
bool fused_qkv_enabled() {
    const char* e = getenv("QD_FUSED_QKV");
    return !(e && e[0] == '0');
}

// QD_DETERMINISTIC=1 in the environment: batch 2..16 residual products take one K
// range per output block instead of adding K ranges with float atomics (read at
// every call).
bool deterministic_enabled() {
    const char* e = getenv("QD_DETERMINISTIC");
    return e && e[0] == '1';
}

// QD_INT8_VALU=1 in the environment: batch 2..16 int8 projections on the vector
// ALUs instead of the matrix cores (read at every call, so a process can compare).
bool int8_valu_enabled() {
    const char* e = getenv("QD_INT8_VALU");
    return e && e[0] == '1';
}

// The attention arguments that decide the batch-1 fused projection.
bool b1_fused_qkv(const qd_config* c, int B, bool merge_in_o, int chunk, int S, int hpw) {
    if (B != 1 || !merge_in_o || !fused_qkv_enabled()) return false;
    qd::AttnArgs at{};
    at.Hq = c->n_q_heads; at.Hkv = c->n_kv_heads; at.hd = c->head_dim; at.page = c->page_size;
    at.chunk = chunk; at.S = S; at.B = B; at.hpw = hpw; at.prefill_start = -1; at.qk_norm = c->qk_norm;
    at.part_always = 1; at.x_dim = c->hidden;
    return qd::attn_fq_ok(at, c->w_dtype == QD_BF16 ? 1 : (c->w_dtype == QD_I8 ? 2 : 0), c->kv_dtype == QD_BF16);
}

// Batch-1 steps whose context is too wide for the o_proj GEMV to merge the
// attention splits itself (more than 1024 values, or more splits than it takes)
// run o_proj by head slices over the split partials instead of a merge launch
// and a GEMV; the head slices meet through float atomics, so this form is off
// with QD_DETERMINISTIC=1, and QD_O_HEADS=0 in the environment keeps the merge
// launch (both read at every call).
bool o_heads_enabled() {
    const char* e = getenv("QD_O_HEADS");
    return !(e && e[0] == '0');
}
bool b1_o_heads(const qd_config* c, int B, bool merge_in_o, int S) {
    return B == 1 && !merge_in_o && S > 1 && S <= 64 && c->w_dtype == QD_BF16 &&
           (c->head_dim == 64 || c->head_dim == 128) && o_heads_enabled() && !deterministic_enabled();
}

// QD_STEP_KERNEL=1 in the environment sends eligible batch-1 steps to the one-launch
// step kernel; otherwise they take the per-op launch path (read at every call, so a
// process can compare the two).
bool step_kernel_enabled() {
    const char* e = getenv("QD_STEP_KERNEL");
    return e && e[0] == '1';
}

// The one-launch step needs the 256 CUs in 8 XCDs of an MI355X (checked once per
// device).
bool device_runs_step_grid(hipStream_t s) {
    static std::mutex mu;
    static signed char known[64] = {};
    int dev = 0;
    if (hipStreamGetDevice(s, &dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    std::lock_guard<std::mutex> lock(mu);
    if (!known[dev]) {
        int n = 0;
        known[dev] = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                      n == qd::kStepWgs) ? 1 : -1;
    }
    return known[dev] > 0;
}

// Pointers the step's loader copies by LDS DMA must be 16-byte aligned, and every
// layer must have all of the q/k/v biases or none.
bool step_pointers_ok(const qd_config* c, const qd_weights* w, bool head) {
    if (head && !aligned16(w->final_norm)) return false;
    const bool b0 = w->layers_host[0].bq != nullptr;
    for (int l = 0; l < c->n_layers; ++l) {
        const qd_layer& L = w->layers_host[l];
        const bool b = L.bq != nullptr;
        if (b != b0 || (L.bk != nullptr) != b || (L.bv != nullptr) != b) return false;
        if (b && (!aligned16(L.bq) || !aligned16(L.bk) || !aligned16(L.bv))) return false;
        if (c->qk_norm && (!aligned16(L.q_norm) || !aligned16(L.k_norm))) return false;
    }
    return true;
}

qd_status check_kv_positions(const qd_config* c, const qd_kv* kv, int B, const int32_t* pos_host,
                             int* max_tokens) {
    if (!kv || !kv->k_pages_host || !kv->v_pages_host || !kv->block_table || !kv->block_table_host)
        return fail(QD_EINVAL, "kv pointers NULL");
    if (kv->max_blocks < 1 || kv->num_pages < 1)
        return fail(QD_ESHAPE, "kv max_blocks %d / num_pages %d", kv->max_blocks, kv->num_pages);
    if (!pos_host) return fail(QD_EINVAL, "pos_host is NULL");
    const long cap = (long)kv->max_blocks * c->page_size;
    int mt = 0;
    for (int b = 0; b < B; ++b) {
        const int p = pos_host[b];
        if (p < 0) return fail(QD_EPOSITION, "pos[%d] = %d < 0", b, p);
        if (p >= cap) return fail(QD_ECAPACITY, "pos[%d] = %d >= block table capacity %ld", b, p, cap);
        for (int j = 0; j <= p / c->page_size; ++j) {
            const int pg = kv->block_table_host[(long)b * kv->max_blocks + j];
            if (pg < 0 || pg >= kv->num_pages)
                return fail(QD_ECAPACITY, "block_table[%d][%d] = %d outside [0, %d)", b, j, pg, kv->num_pages);
        }
        if (p + 1 > mt) mt = p + 1;
    }
    *max_tokens = mt;
    return QD_OK;
}

}  // namespace

extern "C" {

const char* qd_last_error(void) { return g_err.c_str(); }

int32_t qd_abi_version(void) { return QD_ABI_VERSION; }

qd_status qd_decode_plan(const qd_config* cfg, int32_t batch, int32_t max_tokens, qd_decode_plan_info* out) {
    g_err.clear();
    if (!out) return fail(QD_EINVAL, "out is NULL");
    qd_status st = check_config(cfg);
    if (st != QD_OK) return st;
    if (batch < 1 || batch > kMaxBatch) return fail(QD_ESHAPE, "batch %d not in [1, %d]", batch, kMaxBatch);
    if (max_tokens < 1) return fail(QD_ESHAPE, "max_tokens %d < 1", max_tokens);
    int chunk, S, hpw;
    bool merge_in_o = false;
    if (!plan_split(cfg, batch, max_tokens, &chunk, &S, &hpw, &merge_in_o))
        return fail(QD_ECAPACITY, "context of %d tokens needs more than %d attention splits", max_tokens,
                    qd::attn_max_splits());
    qd::AttnArgs at{};
    at.Hq = cfg->n_q_heads; at.Hkv = cfg->n_kv_heads; at.hd = cfg->head_dim; at.page = cfg->page_size;
    at.chunk = chunk; at.S = S; at.B = batch; at.hpw = hpw; at.prefill_start = -1;
    const bool kvbf = cfg->kv_dtype == QD_BF16, wbf = cfg->w_dtype == QD_BF16;
    const bool mfma = qd::attn_uses_mfma(at, kvbf);
    const int qkvr = (cfg->n_q_heads + 2 * cfg->n_kv_heads) * cfg->head_dim;
    const int qkv_splits = qd::gemm16_store_splits(cfg->hidden, qkvr);
    *out = qd_decode_plan_info{};
    out->chunk = chunk;
    out->splits = S;
    out->heads_per_wg = hpw;
    out->matrix_core_attention = mfma ? 1 : 0;
    out->qkv_partials = (batch > 1 && (wbf || (cfg->w_dtype == QD_I8 && !int8_valu_enabled())) && qkv_splits > 1 &&
                         mfma) ? qkv_splits : 0;
    out->merge_in_o_proj = merge_in_o ? 1 : (b1_o_heads(cfg, batch, merge_in_o, S) ? 2 : 0);
    out->fused_qkv = b1_fused_qkv(cfg, batch, merge_in_o, chunk, S, hpw) ? 1 : 0;
    out->step_kernel = (batch == 1 && qd::step::step_config_ok(cfg) && qd::step::plan_step(cfg, max_tokens).ok) ? 1 : 0;
    return QD_OK;
}

size_t qd_workspace_bytes(const qd_config* cfg, int32_t batch, int32_t max_ctx, int32_t prefill_tokens) {
    if (check_config(cfg) != QD_OK) return 0;
    if (prefill_tokens > 0) {
        if (max_ctx < prefill_tokens) return 0;
        int chunk, S, hpw;
        if (!plan_split(cfg, prefill_tokens, max_ctx, &chunk, &S, &hpw)) return 0;
        return plan_prefill(cfg, prefill_tokens, S).total;
    }
    if (batch < 1 || batch > kMaxBatch || max_ctx < 1) return 0;
    int chunk, S, hpw;
    bool merge_in_o = false;
    if (!plan_split(cfg, batch, max_ctx, &chunk, &S, &hpw, &merge_in_o)) return 0;
    // any batch up to `batch` (batch 1 adds the one-launch step's buffers), and a
    // shorter context can take finer splits, so more of them: size for the most
    // splits any context up to max_ctx takes at each batch (only the split count
    // sizes the partials region)
    size_t need = 0;
    for (int b = 1; b <= batch; ++b) {
        int s_max = 0, ch_b = chunk;
        for (int t = 1; t <= max_ctx; ++t) {
            int ch_t, s_t, h_t;
            bool m_t = false;
            if (plan_split(cfg, b, t, &ch_t, &s_t, &h_t, &m_t) && s_t > s_max) { s_max = s_t; ch_b = ch_t; }
        }
        if (s_max > 0) need = std::max(need, plan_decode(cfg, b, s_max, ch_b).total);
    }
    return need;
}

}  // extern "C"

namespace {

// The decode step behind qd_decode_step and qd_decode_step_noalloc. `workspace`
// NULL with scratch_bytes > 0 means: checks only up to the workspace size (the
// caller resolves its scratch memory afterwards and calls again with it).
qd_status decode_step_impl(const qd_config* cfg, const qd_weights* w, const qd_kv* kv, int32_t batch,
                           const int32_t* tokens, const float* x_in, const int32_t* pos,
                           const int32_t* pos_host, float* logits, int32_t* next_tokens, float* x_out,
                           float* layer_out, void* workspace, size_t workspace_bytes, void* stream,
                           bool checks_only = false) {
    g_err.clear();
    qd_status st = check_config(cfg);
    if (st != QD_OK) return st;
    const qd_config& c = *cfg;
    if (batch < 1 || batch > kMaxBatch) return fail(QD_ESHAPE, "batch %d not in [1, %d]", batch, kMaxBatch);
    if (!w || !w->layers_host) return fail(QD_EINVAL, "weights or layers_host is NULL");
    if (!tokens && !x_in) return fail(QD_EINVAL, "tokens and x_in are both NULL");
    if (tokens && !w->embed) return fail(QD_EINVAL, "tokens given but embed is NULL");
    if (tokens && !aligned4(tokens)) return fail(QD_EALIGN, "tokens not 4-byte aligned");
    if (x_in && !aligned4(x_in)) return fail(QD_EALIGN, "x_in not 4-byte aligned");
    if (!pos) return fail(QD_EINVAL, "pos is NULL");
    if (!aligned4(pos)) return fail(QD_EALIGN, "pos not 4-byte aligned");
    {
        const void* outs[] = {logits, next_tokens, x_out, layer_out};
        const char* names[] = {"logits", "next_tokens", "x_out", "layer_out"};
        for (int i = 0; i < 4; ++i)
            if (outs[i] && !aligned4(outs[i])) return fail(QD_EALIGN, "%s not 4-byte aligned", names[i]);
    }
    const bool want_head = logits || next_tokens;
    if (want_head && (!w->final_norm || !w->lm_head))
        return fail(QD_EINVAL, "logits/next_tokens requested but final_norm or lm_head is NULL");
    if (want_head && !aligned16(w->lm_head)) return fail(QD_EALIGN, "lm_head not 16-byte aligned");
    for (int l = 0; l < c.n_layers; ++l)
        if ((st = check_layer(cfg, &w->layers_host[l], l)) != QD_OK) return st;
    if (c.w_dtype == QD_I8) {
        if (tokens && !w->s_embed) return fail(QD_EINVAL, "int8 weights: s_embed is NULL");
        if (want_head && !w->s_lm_head) return fail(QD_EINVAL, "int8 weights: s_lm_head is NULL");
    }
    int max_tokens = 0;
    if ((st = check_kv_positions(cfg, kv, batch, pos_host, &max_tokens)) != QD_OK) return st;
    for (int l = 0; l < c.n_layers; ++l) {
        if (!kv->k_pages_host[l] || !kv->v_pages_host[l])
            return fail(QD_EINVAL, "kv pages of layer %d NULL", l);
        if (!aligned16(kv->k_pages_host[l]) || !aligned16(kv->v_pages_host[l]))
            return fail(QD_EALIGN, "kv pages of layer %d not 16-byte aligned", l);
    }
    int chunk, S, hpw;
    bool merge_in_o = false;
    if (!plan_split(cfg, batch, max_tokens, &chunk, &S, &hpw, &merge_in_o))
        return fail(QD_ECAPACITY, "context of %d tokens needs %d attention splits > %d", max_tokens, S,
                    qd::attn_max_splits());
    const DecodePlan P = plan_decode(cfg, batch, S, chunk);
    if (workspace_bytes < P.total)
        return fail(QD_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, P.total);
    if (checks_only) return QD_OK;
    if (!workspace) return fail(QD_EWORKSPACE, "workspace is NULL");
    if (((uintptr_t)workspace & 255u) != 0) return fail(QD_EALIGN, "workspace not 256-byte aligned");

    hipStream_t s = (hipStream_t)stream;
    char* ws = (char*)workspace;
    float* x = (float*)(ws + P.off_x);
    float* qkv = (float*)(ws + P.off_qkv);
    float* qss = (float*)(ws + P.off_qss);
    const int qkv_splits = qd::gemm16_store_splits(P.D, P.qkvr);
    float* part = (float*)(ws + P.off_part);
    float2* part_ml = (float2*)(part + (size_t)batch * P.Hq * S * P.hd);
    float2* rope = (float2*)(ws + P.off_rope);
    float* ctx = (float*)(ws + P.off_ctx);
    float* h = (float*)(ws + P.off_h);
    float* lg = logits ? logits : (float*)(ws + P.off_logits);
    float* pv = (float*)(ws + P.off_pv);
    int* pi = (int*)(ws + P.off_pi);
    // wbf: bf16 gains and biases (bf16 or int8 matrices); wty: the GEMV's weight type
    const int wbf = c.w_dtype != QD_F32, kvbf = c.kv_dtype == QD_BF16, wty = c.w_dtype;
    const int B = batch, D = P.D;
    const int cap = kv->max_blocks * c.page_size;
    auto gemv = [&](const qd::GemvArgs& g, int epi, int grid_cap, int* grid_out) {
        if (B == 1) return qd::launch_gemv1(g, wty, epi, epi == qd::EPI_LOGITS ? grid_cap : kGemv1GridCap,
                                            grid_out, s);
        if (wty == QD_BF16 || (wty == QD_I8 && !int8_valu_enabled())) {   // the matrix cores
            qd::GemvArgs m = g;
            m.kt = qd::gemm16_chunk(g.K);
            return qd::launch_gemm16(m, wty, epi, grid_cap, grid_out, s);
        }
        return qd::launch_gemv(g, wty, epi, grid_cap, grid_out, s);   // float rows (or int8, see above)
    };

    // batch 1: the one-launch step, when the config, the device and the position allow
    if (B == 1 && P.step_S > 0 && step_kernel_enabled() && device_runs_step_grid(s) &&
        step_pointers_ok(cfg, w, want_head)) {
        const qd::step::StepPlan sp = qd::step::plan_step(cfg, max_tokens);
        if (sp.ok && sp.S <= P.step_S) {
            qd::StepArgs sa{};
            sa.L = c.n_layers; sa.D = D; sa.Hq = P.Hq; sa.Hkv = P.Hkv; sa.hd = P.hd; sa.G = P.G; sa.F = P.F;
            sa.V = c.vocab; sa.qkvr = P.qkvr; sa.eps = c.rms_eps; sa.scale = 1.0f / sqrtf((float)P.hd);
            sa.qk_norm = c.qk_norm; sa.has_bias = w->layers_host[0].bq != nullptr;
            sa.S = sp.S; sa.C = sp.C;
            sa.up_wa = sp.up_wa; sa.up_wb = sp.up_wb; sa.down_wa = sp.down_wa; sa.down_wb = sp.down_wb;
            sa.pos = pos; sa.block_table = kv->block_table; sa.max_blocks = kv->max_blocks; sa.num_pages = kv->num_pages;
            sa.final_norm = want_head ? w->final_norm : nullptr;
            sa.lm_head = want_head ? w->lm_head : nullptr;
            sa.logits = lg; sa.x_out = x_out; sa.layer_out = layer_out;
            sa.argmax_val = (float*)(ws + P.off_sam_v); sa.argmax_idx = (int*)(ws + P.off_sam_i);
            typedef unsigned long long u64;
            sa.xb = (float*)(ws + P.off_sxb); sa.y = (float*)(ws + P.off_sy); sa.h = (float*)(ws + P.off_sh);
            sa.qkv = (u64*)(ws + P.off_sqkv); sa.part = (u64*)(ws + P.off_spart);
            sa.part_stride = (long)P.Hkv * sp.S * P.G * (P.hd + 2);
            sa.cnt = (uint32_t*)(ws + P.off_scnt);
            sa.rope = (float2*)(ws + P.off_srope); sa.err = (uint32_t*)(ws + P.off_serr);
            sa.clear_from = sa.qkv; sa.clear_n = (long)((P.off_send - P.off_sqkv) / sizeof(u64));
            for (int l = 0; l < c.n_layers; ++l) {
                const qd_layer& L = w->layers_host[l];
                qd::StepLayer& t = sa.layer[l];
                t.attn_norm = L.attn_norm; t.wq = L.wq; t.wk = L.wk; t.wv = L.wv; t.bq = L.bq; t.bk = L.bk; t.bv = L.bv;
                t.q_norm = L.q_norm; t.k_norm = L.k_norm; t.wo = L.wo; t.mlp_norm = L.mlp_norm; t.w_gate = L.w_gate;
                t.w_up = L.w_up; t.w_down = L.w_down; t.kc = kv->k_pages_host[l]; t.vc = kv->v_pages_host[l];
            }
            QD_LAUNCH_K(QD_K_EMBED, qd::launch_step_prologue(sa, tokens, w->embed, x_in, c.rope_theta, s),
                        "step prologue");
            QD_LAUNCH_K(QD_K_STEP, qd::launch_step_kernel(sa, s), "step kernel");
            if (next_tokens)
                QD_LAUNCH_K(QD_K_ARGMAX, qd::launch_argmax(sa.argmax_val, sa.argmax_idx, qd::kStepWgs, next_tokens, 1, s),
                            "argmax");
            return QD_OK;
        }
    }

    const bool fq = b1_fused_qkv(cfg, B, merge_in_o, chunk, S, hpw);
    // with the projection in the attention launch and a token to embed, the first
    // layer's launch gathers the embedding row and forms the RoPE table itself
    const bool emb_in_fq = fq && tokens;
    if (!emb_in_fq) {
        qd::StepInputArgs si{};
        si.tokens = tokens; si.embed = w->embed; si.embed_scale = w->s_embed; si.x_in = x_in; si.x = x;
        si.pos = pos; si.rope = rope;
        si.B = B; si.D = D; si.V = c.vocab; si.hd = P.hd; si.theta = c.rope_theta;
        QD_LAUNCH_K(QD_K_EMBED, qd::launch_step_input(si, wty, s), "step input");
    }

    const int det = deterministic_enabled() ? 1 : 0;
    const bool o_heads = b1_o_heads(cfg, B, merge_in_o, S);
    for (int l = 0; l < c.n_layers; ++l) {
        const qd_layer& L = w->layers_host[l];
        // RMSNorm -> q|k|v GEMV + bias
        qd::GemvArgs g{};
        g.w[0] = L.wq; g.w[1] = L.wk; g.w[2] = L.wv;
        g.bias[0] = L.bq; g.bias[1] = L.bk; g.bias[2] = L.bv;
        g.seg_end[0] = P.Hq * P.hd; g.seg_end[1] = (P.Hq + P.Hkv) * P.hd; g.seg_end[2] = P.qkvr;
        g.wscale[0] = L.s_q; g.wscale[1] = L.s_k; g.wscale[2] = L.s_v;
        g.nseg = 3; g.N = P.qkvr; g.K = D; g.B = B; g.x = x; g.gain = L.attn_norm; g.eps = c.rms_eps;
        g.y = qkv; g.kt = gemv_kt(B, D);
        // [q/k norm] + RoPE + KV append + split-K attention + merge
        qd::AttnArgs at{};
        at.qkv = qkv; at.k_cache = kv->k_pages_host[l]; at.v_cache = kv->v_pages_host[l];
        at.block_table = kv->block_table; at.max_blocks = kv->max_blocks; at.num_pages = kv->num_pages;
        at.pos = pos; at.capacity = cap; at.q_norm = L.q_norm; at.k_norm = L.k_norm; at.qk_norm = c.qk_norm;
        at.eps = c.rms_eps; at.theta = c.rope_theta; at.part = part; at.part_ml = part_ml;
        at.part_always = (merge_in_o || o_heads) ? 1 : 0; at.rope = rope; at.ctx = ctx;
        at.Hq = P.Hq; at.Hkv = P.Hkv; at.hd = P.hd; at.page = c.page_size; at.chunk = P.chunk; at.S = P.S;
        at.B = B; at.hpw = hpw; at.scale = 1.0f / sqrtf((float)P.hd);
        at.prefill_start = -1; at.q_rot = nullptr;
        // the matrix-core kernel's grid at batch 2..16: only the splits that hold keys
        // (positions from the host copy). The grid is sized by the longest sequence, and
        // at batch 16 over 128..4096 tokens more than half of its workgroups would exit
        // at once, yet take their turn in the dispatch: 10.2 -> 8.9 us per launch.
        if (B > 1 && qd::attn_uses_mfma(at, kvbf)) {
            at.compact = 1;
            int acc = 0;
            at.wg_base[0] = 0;
            for (int b = 0; b < B; ++b) {
                const int p = pos_host[b];
                const int ns = (p >= 0 && p < cap) ? std::min(P.S, (p + P.chunk) / P.chunk) : 0;
                acc += ns * P.Hkv;
                at.wg_base[b + 1] = acc;
            }
        }
        // batch 2..16 on the matrix cores: q|k|v as K-range partial products, which
        // the attention kernel finishes (RMSNorm scale, bias) as it loads them
        if (B > 1 && (wty == QD_BF16 || (wty == QD_I8 && !int8_valu_enabled())) && qkv_splits > 1 &&
            qd::attn_uses_mfma(at, kvbf)) {
            g.ss_out = qss;
            at.qkv_slabs = qkv_splits; at.qkv_slab_stride = (long)B * P.qkvr; at.qkv_ss = qss;
            at.qkv_bias[0] = L.bq; at.qkv_bias[1] = L.bk; at.qkv_bias[2] = L.bv; at.x_dim = D;
            if (wty == QD_I8) { at.qkv_scale[0] = L.s_q; at.qkv_scale[1] = L.s_k; at.qkv_scale[2] = L.s_v; }
        }
        if (fq) {   // batch 1: the projection inside the attention launch
            at.fq = 1; at.fq_x = x; at.fq_gain = L.attn_norm; at.fq_out = qkv; at.x_dim = D;
            if (emb_in_fq && l == 0) {
                at.fq_tok = tokens; at.fq_embed = w->embed; at.fq_embed_scale = w->s_embed; at.fq_vocab = c.vocab;
            }
            at.fq_w[0] = L.wq; at.fq_w[1] = L.wk; at.fq_w[2] = L.wv;
            if (wty == QD_I8) { at.fq_scale[0] = L.s_q; at.fq_scale[1] = L.s_k; at.fq_scale[2] = L.s_v; }
            at.qkv_bias[0] = L.bq; at.qkv_bias[1] = L.bk; at.qkv_bias[2] = L.bv;
        } else {
            QD_LAUNCH_K(QD_K_QKV, gemv(g, qd::EPI_STORE, kGemvGridCap, nullptr), "qkv gemv");
        }
        QD_LAUNCH_K(QD_K_ATTN, qd::launch_attention(at, wbf, kvbf, s), "attention");
        // o_proj + residual
        qd::GemvArgs go{};
        go.w[0] = L.wo; go.wscale[0] = L.s_o; go.seg_end[0] = go.seg_end[1] = go.seg_end[2] = D; go.nseg = 1;
        go.N = D; go.K = P.Hq * P.hd; go.B = B; go.x = ctx; go.gain = nullptr; go.y = x; go.deterministic = det;
        go.kt = gemv_kt(B, go.K);
        if (merge_in_o) {   // the context is merged from the attention's splits here
            go.part = part; go.part_ml = part_ml; go.part_pos = pos;
            go.part_S = S; go.part_chunk = chunk; go.part_hd = P.hd;
            if (fq) {   // ... and the new token's split from the projections
                go.part_new = qkv; go.part_kv_heads = P.Hkv; go.part_scale2 = at.scale * 1.4426950408889634f;
            }
        }
        if (o_heads) {   // ... or by head slices, each merging its head's splits
            go.part = part; go.part_ml = part_ml; go.part_pos = pos;
            go.part_S = S; go.part_chunk = chunk; go.part_hd = P.hd;
            QD_LAUNCH_K(QD_K_O, qd::launch_oproj_heads(go, s), "o_proj by head slices");
        } else {
            QD_LAUNCH_K(QD_K_O, gemv(go, qd::EPI_RESID, kGemvGridCap, nullptr), "o_proj gemv");
        }
        // RMSNorm -> gate|up GEMV -> SwiGLU
        qd::GemvArgs gu{};
        gu.w[0] = L.w_gate; gu.w[1] = L.w_up; gu.wscale[0] = L.s_gate; gu.wscale[1] = L.s_up;
        gu.seg_end[0] = gu.seg_end[1] = gu.seg_end[2] = P.F;
        gu.nseg = 1; gu.N = P.F; gu.K = D; gu.B = B; gu.x = x; gu.gain = L.mlp_norm; gu.eps = c.rms_eps;
        gu.y = h; gu.kt = gemv_kt(B, D);
        QD_LAUNCH_K(QD_K_GATEUP, gemv(gu, qd::EPI_SWIGLU, kGemvGridCap, nullptr), "gate/up gemv");
        // down + residual
        qd::GemvArgs gd{};
        gd.w[0] = L.w_down; gd.wscale[0] = L.s_down; gd.seg_end[0] = gd.seg_end[1] = gd.seg_end[2] = D; gd.nseg = 1;
        gd.N = D; gd.K = P.F; gd.B = B; gd.x = h; gd.gain = nullptr; gd.y = x; gd.kt = gemv_kt(B, P.F);
        gd.deterministic = det;
        QD_LAUNCH_K(QD_K_DOWN, gemv(gd, qd::EPI_RESID, kGemvGridCap, nullptr), "down gemv");
        if (layer_out) QD_LAUNCH(qd::launch_copy(x, layer_out + (size_t)l * B * D, (long)B * D, s), "layer_out copy");
    }
    if (x_out) QD_LAUNCH(qd::launch_copy(x, x_out, (long)B * D, s), "x_out copy");
    if (want_head) {
        qd::GemvArgs gl{};
        gl.w[0] = w->lm_head; gl.wscale[0] = w->s_lm_head; gl.seg_end[0] = gl.seg_end[1] = gl.seg_end[2] = c.vocab;
        gl.nseg = 1;
        gl.N = c.vocab; gl.K = D; gl.B = B; gl.x = x; gl.gain = w->final_norm; gl.eps = c.rms_eps;
        gl.y = lg; gl.part_val = pv; gl.part_idx = pi; gl.kt = gemv_kt(B, D);
        int grid = 0;
        QD_LAUNCH_K(QD_K_LMHEAD, gemv(gl, qd::EPI_LOGITS, kLogitsGridCap, &grid), "lm_head gemv");
        if (next_tokens) QD_LAUNCH_K(QD_K_ARGMAX, qd::launch_argmax(pv, pi, grid, next_tokens, B, s), "argmax");
    }
    return QD_OK;
}

// Device scratch of qd_decode_step_noalloc: one copy per GPU, held until the
// process ends. In host code `scratch` names a host-side stand-in, so its device
// address on each GPU is taken once with hipGetSymbolAddress (that GPU current)
// and only that address is ever handed to kernels.
constexpr size_t kScratchBytes = QD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

qd_status scratch_of_stream(hipStream_t s, void** out) {
    int dev = -1, cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail(QD_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    e = hipStreamGetDevice(s, &dev);
    if (e != hipSuccess) return fail(QD_EHIP, "hipStreamGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(QD_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(QD_EHIP, "hipSetDevice(%d) failed: %s", dev, hipGetErrorString(e));
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p)
            return fail(QD_EHIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QD_OK;
}

}  // namespace

extern "C" {

qd_status qd_decode_step(const qd_config* cfg, const qd_weights* w, const qd_kv* kv, int32_t batch,
                         const int32_t* tokens, const float* x_in, const int32_t* pos,
                         const int32_t* pos_host, float* logits, int32_t* next_tokens, float* x_out,
                         float* layer_out, void* workspace, size_t workspace_bytes, void* stream) {
    return decode_step_impl(cfg, w, kv, batch, tokens, x_in, pos, pos_host, logits, next_tokens, x_out,
                            layer_out, workspace, workspace_bytes, stream);
}

qd_status qd_decode_step_noalloc(const qd_config* cfg, const qd_weights* w, const qd_kv* kv, int32_t batch,
                                 const int32_t* tokens, const float* x_in, const int32_t* pos,
                                 const int32_t* pos_host, float* logits, int32_t* next_tokens, float* x_out,
                                 float* layer_out, void* stream) {
    // every host check first, the size against the scratch maximum included
    qd_status st = decode_step_impl(cfg, w, kv, batch, tokens, x_in, pos, pos_host, logits, next_tokens,
                                    x_out, layer_out, nullptr, kScratchBytes, stream, /*checks_only=*/true);
    if (st != QD_OK) {
        if (st == QD_EWORKSPACE)
            return fail(QD_EWORKSPACE, "qd_decode_step_noalloc: this step needs more than the %zu-byte static "
                        "scratch (%s)", kScratchBytes, g_err.c_str());
        return st;
    }
    void* ws = nullptr;
    if ((st = scratch_of_stream((hipStream_t)stream, &ws)) != QD_OK) return st;
    return decode_step_impl(cfg, w, kv, batch, tokens, x_in, pos, pos_host, logits, next_tokens, x_out,
                            layer_out, ws, kScratchBytes, stream);
}

qd_status qd_quantize_rows_int8(const void* w, int32_t w_dtype, int64_t rows, int32_t cols, int8_t* q,
                                float* scale, void* stream) {
    if (!w || !q || !scale) return fail(QD_EINVAL, "w, q or scale is NULL");
    if (w_dtype != QD_F32 && w_dtype != QD_BF16) return fail(QD_EINVAL, "w_dtype %d not F32 or BF16", w_dtype);
    if (rows < 1 || rows > 0x7fffffffLL || cols < 16 || cols % 16)
        return fail(QD_ESHAPE, "rows %lld / cols %d (cols a positive multiple of 16)", (long long)rows, cols);
    if (!aligned16(w) || !aligned16(q) || !aligned16(scale)) return fail(QD_EALIGN, "w, q or scale not 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    QD_LAUNCH(qd::launch_quantize_rows(w, w_dtype == QD_BF16, (long)rows, cols, q, scale, s), "quantize");
    return QD_OK;
}

qd_status qd_sample(const float* logits, int32_t batch, int32_t vocab, float temperature, int32_t top_k,
                    float top_p, const float* uniforms, int32_t* tokens, void* stream) {
    if (!logits || !tokens) return fail(QD_EINVAL, "logits or tokens is NULL");
    if (batch < 1 || vocab < 1) return fail(QD_ESHAPE, "batch %d / vocab %d must be positive", batch, vocab);
    if (!(temperature >= 0.f) || !std::isfinite(temperature))
        return fail(QD_EINVAL, "temperature %g must be finite and >= 0", (double)temperature);
    if (!(top_p > 0.f && top_p <= 1.f)) return fail(QD_EINVAL, "top_p %g not in (0, 1]", (double)top_p);
    if (temperature > 0.f) {
        if (!uniforms) return fail(QD_EINVAL, "uniforms is NULL");
        if (top_k > qd::kSampleMaxK && top_k < vocab)
            return fail(QD_EUNSUPPORTED, "top_k %d: sampling takes 1 <= top_k <= %d, or top_k <= 0 / >= vocab %d "
                        "(no top-k)", top_k, qd::kSampleMaxK, vocab);
    }
    if (!aligned4(logits) || !aligned4(tokens) || (uniforms && !aligned4(uniforms)))
        return fail(QD_EALIGN, "logits, uniforms or tokens not 4-byte aligned");
    qd::SampleArgs a{};
    a.logits = logits; a.B = batch; a.V = vocab; a.temperature = temperature; a.top_k = top_k;
    a.top_p = top_p; a.one_minus_p = (float)(1.0 - (double)top_p); a.uniforms = uniforms; a.tokens = tokens;
    hipStream_t s = (hipStream_t)stream;
    QD_LAUNCH_K(QD_K_ARGMAX, qd::launch_sample(a, s), "sample");
    return QD_OK;
}

int32_t qd_profile_enable(uint32_t kind_mask) {
    if (!g_prof.ready) {
        for (int i = 0; i < 2 * kProfSlots; ++i)
            if (hipEventCreate(&g_prof.ev[i]) != hipSuccess) return fail(QD_EHIP, "hipEventCreate failed");
        g_prof.ready = true;
    }
    g_prof.mask = kind_mask;
    g_prof.next = 0;
    return QD_OK;
}

int32_t qd_profile_read(int32_t kind, int32_t* launches, double* total_ms) {
    if (!launches || !total_ms) return fail(QD_EINVAL, "launches/total_ms NULL");
    *launches = 0;
    *total_ms = 0.0;
    for (int slot = 0; slot < g_prof.next; ++slot) {
        if (g_prof.kind[slot] != kind) continue;
        if (hipEventSynchronize(g_prof.ev[2 * slot + 1]) != hipSuccess)
            return fail(QD_EHIP, "hipEventSynchronize failed");
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, g_prof.ev[2 * slot], g_prof.ev[2 * slot + 1]) != hipSuccess)
            return fail(QD_EHIP, "hipEventElapsedTime failed");
        *launches += 1;
        *total_ms += ms;
    }
    return QD_OK;
}

void qd_profile_reset(void) { g_prof.next = 0; }

qd_status qd_kv_append(const qd_config* cfg, const qd_kv* kv, int32_t layer_index, int32_t batch,
                       const int32_t* pos, const int32_t* pos_host, const float* k, const float* v,
                       void* stream) {
    g_err.clear();
    qd_status st = check_config(cfg);
    if (st != QD_OK) return st;
    if (batch < 1) return fail(QD_ESHAPE, "batch %d < 1", batch);
    if (layer_index < 0 || layer_index >= cfg->n_layers)
        return fail(QD_ESHAPE, "layer_index %d outside [0, %d)", layer_index, cfg->n_layers);
    if (!k || !v || !pos) return fail(QD_EINVAL, "k, v or pos is NULL");
    int mt = 0;
    if ((st = check_kv_positions(cfg, kv, batch, pos_host, &mt)) != QD_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    void* kc = kv->k_pages_host[layer_index];
    void* vc = kv->v_pages_host[layer_index];
    if (!kc || !vc) return fail(QD_EINVAL, "kv pages of layer %d NULL", layer_index);
    QD_LAUNCH(qd::launch_kv_append(k, v, kc, vc, kv->block_table, kv->max_blocks, kv->num_pages, pos,
                                   kv->max_blocks * cfg->page_size, cfg->n_kv_heads, cfg->head_dim,
                                   cfg->page_size, batch, cfg->kv_dtype == QD_BF16, s),
              "kv append");
    return QD_OK;
}

qd_status qd_prefill_block(const qd_config* cfg, const qd_layer* layer, int32_t layer_index, const qd_kv* kv,
                           int32_t n_tokens, int32_t start_pos, const void* x_in, int32_t x_dtype,
                           float* x_out, void* workspace, size_t workspace_bytes, void* stream) {
    g_err.clear();
    qd_status st = check_config(cfg);
    if (st != QD_OK) return st;
    const qd_config& c = *cfg;
    if (c.w_dtype != QD_BF16) return fail(QD_EUNSUPPORTED, "prefill needs bf16 weights (MFMA bf16 GEMMs)");
    if (!layer) return fail(QD_EINVAL, "layer is NULL");
    if ((st = check_layer(cfg, layer, layer_index)) != QD_OK) return st;
    if (layer_index < 0 || layer_index >= c.n_layers)
        return fail(QD_ESHAPE, "layer_index %d outside [0, %d)", layer_index, c.n_layers);
    if (n_tokens < 1) return fail(QD_ESHAPE, "n_tokens %d < 1", n_tokens);
    if (start_pos < 0) return fail(QD_EPOSITION, "start_pos %d < 0", start_pos);
    if (!x_in || !x_out) return fail(QD_EINVAL, "x_in or x_out is NULL");
    if (x_dtype != QD_BF16 && x_dtype != QD_F32) return fail(QD_EINVAL, "x_dtype %d", x_dtype);
    if (!aligned16(x_in) || !aligned16(x_out)) return fail(QD_EALIGN, "x_in / x_out not 16-byte aligned");
    // every position start .. start + n - 1 must have a page in row 0 of the block table
    const int32_t last = start_pos + n_tokens - 1;
    int max_tokens = 0;
    if ((st = check_kv_positions(cfg, kv, 1, &last, &max_tokens)) != QD_OK) return st;
    void* kc = kv->k_pages_host[layer_index];
    void* vc = kv->v_pages_host[layer_index];
    if (!kc || !vc) return fail(QD_EINVAL, "kv pages of layer %d NULL", layer_index);
    if (!aligned16(kc) || !aligned16(vc)) return fail(QD_EALIGN, "kv pages of layer %d not 16-byte aligned", layer_index);
    int chunk, S, hpw;
    if (!plan_split(cfg, n_tokens, max_tokens, &chunk, &S, &hpw))
        return fail(QD_ECAPACITY, "context of %d tokens needs %d attention splits > %d", max_tokens, S,
                    qd::attn_max_splits());
    const PrefillPlan P = plan_prefill(cfg, n_tokens, S);
    if (!workspace) return fail(QD_EWORKSPACE, "workspace is NULL");
    if (((uintptr_t)workspace & 255u) != 0) return fail(QD_EALIGN, "workspace not 256-byte aligned");
    if (workspace_bytes < P.total)
        return fail(QD_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, P.total);

    hipStream_t s = (hipStream_t)stream;
    char* ws = (char*)workspace;
    uint16_t* nrm = (uint16_t*)(ws + P.off_nrm);
    float* qkv = (float*)(ws + P.off_qkv);
    float* qrot = (float*)(ws + P.off_q);
    float* part = (float*)(ws + P.off_part);
    float* ctx = (float*)(ws + P.off_ctx);
    uint16_t* ctxb = (uint16_t*)(ws + P.off_ctxb);
    uint16_t* h = (uint16_t*)(ws + P.off_h);
    float* slab = (float*)(ws + P.off_slab);
    const qd_layer& L = *layer;
    const int N = n_tokens, D = c.hidden, Hq = c.n_q_heads, Hkv = c.n_kv_heads, hd = c.head_dim;
    const int qkvr = (Hq + 2 * Hkv) * hd;
    const int kvbf = c.kv_dtype == QD_BF16;

    // RMSNorm -> bf16 operand; the input rows become the float32 residual in x_out
    qd::PrefillNormArgs nr{};
    if (x_dtype == QD_BF16) nr.x_bf16 = x_in; else nr.x_f32 = (const float*)x_in;
    nr.x_res = x_out; nr.gain = L.attn_norm; nr.out = nrm; nr.rows = N; nr.D = D; nr.eps = c.rms_eps;
    // q|k|v = norm(x) W^T (+ bias); a K-split product accumulates into a cleared buffer
    qd::GemmArgs g{};
    g.A = nrm; g.w[0] = L.wq; g.w[1] = L.wk; g.w[2] = L.wv; g.bias[0] = L.bq; g.bias[1] = L.bk; g.bias[2] = L.bv;
    g.seg_end[0] = Hq * hd; g.seg_end[1] = (Hq + Hkv) * hd; g.seg_end[2] = qkvr;
    g.M = N; g.N = qkvr; g.K = D; g.C = qkv; g.ldc = qkvr;
    qd::PrefillRopeArgs rp{};
    rp.qkv = qkv;
    if (P.slabs_qkv > 0) {   // K-range slabs; the RoPE kernel adds them and the bias
        g.C = slab;
        QD_LAUNCH(qd::launch_prefill_norm(nr, 1, s), "prefill norm");
        QD_LAUNCH_K(QD_K_PREFILL_GEMM, qd::launch_mfma_gemm_slabs(g, P.slabs_qkv, s), "qkv gemm");
        rp.qkv = slab; rp.nslab = P.slabs_qkv; rp.slab_stride = (long)N * qkvr;
        for (int i = 0; i < 3; ++i) { rp.bias[i] = g.bias[i]; rp.seg_end[i] = g.seg_end[i]; }
    } else {
        const int qkv_splits = qd::mfma_gemm_splits(g, qd::GEMM_STORE);
        if (qkv_splits > 1) { nr.zero = qkv; nr.zero_n = (long)N * qkvr; }
        QD_LAUNCH(qd::launch_prefill_norm(nr, 1, s), "prefill norm");
        QD_LAUNCH_K(QD_K_PREFILL_GEMM, qd::launch_mfma_gemm(g, qd::GEMM_STORE, qkv_splits, s), "qkv gemm");
    }
    // [q/k norm] + RoPE; K/V of every row into the cache
    rp.q_out = qrot; rp.k_cache = kc; rp.v_cache = vc; rp.block_table = kv->block_table;
    rp.num_pages = kv->num_pages; rp.capacity = kv->max_blocks * c.page_size; rp.start = start_pos; rp.rows = N;
    rp.q_norm = L.q_norm; rp.k_norm = L.k_norm; rp.qk_norm = c.qk_norm; rp.eps = c.rms_eps; rp.theta = c.rope_theta;
    rp.Hq = Hq; rp.Hkv = Hkv; rp.hd = hd; rp.page = c.page_size;
    QD_LAUNCH(qd::launch_prefill_rope_append(rp, 1, kvbf, s), "prefill rope/append");
    // causal attention: row i attends over positions 0 .. start + i
    if (kvbf) {   // matrix cores; the context comes out in bf16, the o_proj operand
        qd::PrefillAttnArgs pa{};
        pa.q = qrot; pa.k_cache = kc; pa.v_cache = vc; pa.block_table = kv->block_table;
        pa.num_pages = kv->num_pages; pa.rows = N; pa.start = start_pos; pa.Hq = Hq; pa.Hkv = Hkv; pa.hd = hd;
        pa.page = c.page_size; pa.scale = 1.0f / sqrtf((float)hd); pa.out = ctxb;
        QD_LAUNCH_K(QD_K_PREFILL_ATTN, qd::launch_prefill_attn_mfma(pa, s), "prefill attention");
    } else {
    qd::AttnArgs at{};
    at.k_cache = kc; at.v_cache = vc; at.block_table = kv->block_table; at.max_blocks = kv->max_blocks;
    at.num_pages = kv->num_pages; at.pos = nullptr; at.capacity = kv->max_blocks * c.page_size;
    at.part = part; at.part_ml = (float2*)(part + (size_t)N * Hq * S * hd);
    at.ctx = ctx; at.Hq = Hq; at.Hkv = Hkv; at.hd = hd; at.page = c.page_size;
    at.chunk = chunk; at.S = S; at.B = N; at.hpw = hpw; at.scale = 1.0f / sqrtf((float)hd);
    at.prefill_start = start_pos; at.q_rot = qrot;
    QD_LAUNCH_K(QD_K_PREFILL_ATTN, qd::launch_attention(at, 1, kvbf, s), "prefill attention");
    QD_LAUNCH(qd::launch_to_bf16(ctx, ctxb, (long)N * Hq * hd, s), "context to bf16");
    }
    // x += ctx W_o^T
    qd::GemmArgs go{};
    go.A = ctxb; go.w[0] = L.wo; go.seg_end[0] = go.seg_end[1] = go.seg_end[2] = D;
    go.M = N; go.N = D; go.K = Hq * hd; go.C = x_out; go.ldc = D;
    // RMSNorm -> bf16; h = silu(n W_g^T) * (n W_u^T) in bf16
    qd::PrefillNormArgs n2{};
    n2.x_f32 = x_out; n2.gain = L.mlp_norm; n2.out = nrm; n2.rows = N; n2.D = D; n2.eps = c.rms_eps;
    if (P.slabs_o > 0) {   // the MLP norm adds the slabs into the residual as it reads it
        go.C = slab;
        QD_LAUNCH_K(QD_K_PREFILL_GEMM, qd::launch_mfma_gemm_slabs(go, P.slabs_o, s), "o_proj gemm");
        n2.part = slab; n2.nslab = P.slabs_o; n2.slab_stride = (long)N * D; n2.x_res = x_out;
    } else {
        QD_LAUNCH_K(QD_K_PREFILL_GEMM, qd::launch_mfma_gemm(go, qd::GEMM_RESID, 0, s), "o_proj gemm");
    }
    QD_LAUNCH(qd::launch_prefill_norm(n2, 1, s), "prefill mlp norm");
    qd::GemmArgs gu{};
    gu.A = nrm; gu.w[0] = L.w_gate; gu.w[1] = L.w_up; gu.seg_end[0] = gu.seg_end[1] = gu.seg_end[2] = c.ffn;
    gu.M = N; gu.N = c.ffn; gu.K = D; gu.C = h; gu.ldc = c.ffn;
    QD_LAUNCH_K(QD_K_PREFILL_GEMM, qd::launch_mfma_gemm(gu, qd::GEMM_SWIGLU, 1, s), "gate/up gemm");
    // x += h W_d^T
    qd::GemmArgs gd{};
    gd.A = h; gd.w[0] = L.w_down; gd.seg_end[0] = gd.seg_end[1] = gd.seg_end[2] = D;
    gd.M = N; gd.N = D; gd.K = c.ffn; gd.C = x_out; gd.ldc = D;
    if (P.slabs_down > 0) {
        gd.C = slab;
        QD_LAUNCH_K(QD_K_PREFILL_GEMM, qd::launch_mfma_gemm_slabs(gd, P.slabs_down, s), "down gemm");
        QD_LAUNCH_K(QD_K_PREFILL_GEMM, qd::launch_add_slabs(x_out, slab, P.slabs_down, (long)N * D, (long)N * D, s),
                    "down slabs");
    } else {
        QD_LAUNCH_K(QD_K_PREFILL_GEMM, qd::launch_mfma_gemm(gd, qd::GEMM_RESID, 0, s), "down gemm");
    }
    return QD_OK;
}

}  // extern "C"
