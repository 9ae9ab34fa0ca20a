// Schedule of the one-launch batch-1 step (qd_step.hip): which bytes of which
// tensors each workgroup's loader streams into its LDS ring, in what order, and
// the ring slot each lands in; shared by the kernel and the host-side checker
// (tests/step_schedule_check.cpp), so both walk the same arithmetic.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qd.h"
#include "qd_launch.h"

#define QD_HD __host__ __device__

namespace qd {
namespace step {

QD_HD inline int qd_min(int a, int b) { return a < b ? a : b; }
QD_HD inline int qd_max(int a, int b) { return a > b ? a : b; }
QD_HD inline uint32_t qd_min(uint32_t a, uint32_t b) { return a < b ? a : b; }
QD_HD inline long qd_min(long a, long b) { return a < b ? a : b; }

constexpr int kXcd = 8;
constexpr int kWgs = kStepWgs;           // one per CU
constexpr int kSlotsPerXcd = kWgs / kXcd;
constexpr int kNcw = 4;                  // compute waves
constexpr int kThreads = 64 * (1 + kNcw);
constexpr int kRingSlots = 112;          // 1 KB LDS slots
constexpr int kWork = 5120;              // floats of the workgroup's work buffer
constexpr int kXs = 2560;                // words of each half of the split product input (2 elements each)
constexpr int kMaxOut = 56;              // DMA instructions the loader keeps in flight
constexpr int kBatch = 8;                // DMAs the loader issues between two progress updates
constexpr uint32_t kSpinMax = 1u << 21;  // polls before a wait gives up
constexpr int kP3Rows = 8;               // gate (and up) rows per P3 block
constexpr int kLmRows = 16;              // lm_head rows per block
constexpr int kMaxPages = 16;            // pages of one attention split (C <= 256)

// One piece of the loader's schedule: `rows` runs of `seg` bytes (a multiple of
// 16) at src + r * stride, packed back to back into the ring from a slot
// boundary; a block may wrap at the ring's end (readers wrap each 16-byte chunk,
// which never straddles it).
struct Blk {
    const char* src;
    int rows, seg;
    long stride;
};
QD_HD inline int blk_bytes(const Blk& b) { return b.rows * b.seg; }
QD_HD inline uint32_t blk_slots(const Blk& b) { return (uint32_t)((blk_bytes(b) + 1023) >> 10); }

// Rows [r0, r1) of workgroup w when n rows are dealt over the grid in proportion
// to weight wa (workgroups on XCDs < nx) or wb (the others).
QD_HD inline void weighted_range(int w, int n, int nx, int wa, int wb, int* r0, int* r1) {
    auto cum = [&](int k) {
        const int full = k / kXcd, rem = k % kXcd;
        const long na = (long)full * nx + qd_min(rem, nx);
        return na * wa + (long)(k - na) * wb;
    };
    const long tot = cum(kWgs);
    *r0 = (int)((long)n * cum(w) / tot);
    *r1 = (int)((long)n * cum(w + 1) / tot);
}

enum { PH_QKV = 0, PH_ATTN = 1, PH_O = 2, PH_UP = 3, PH_DOWN = 4, PH_HEAD = 5 };

struct Sched {
    int wg, xcd, slot;      // slot: rank among the XCD's workgroups
    int p;                  // position of the new token
    int pg0, npg;           // attention: first page index of the split and page count
    int f0, f1;             // gate|up rows of the workgroup
    int d0, d1;             // down rows
    int v0, v1;             // lm_head rows
    int pid_p;              // page of the new token (its attention split only; -1 elsewhere)
};

// The workgroup's row ranges, fixed for the whole step (computed once: the
// 64-bit divisions of weighted_range are long instruction sequences).
QD_HD inline void init_rows(const StepArgs& a, Sched& S) {
    weighted_range(S.wg, a.F, a.Hkv, a.up_wa, a.up_wb, &S.f0, &S.f1);
    weighted_range(S.wg, a.D, a.Hkv, a.down_wa, a.down_wb, &S.d0, &S.d1);
    S.v0 = (int)((long)a.V * S.wg / kWgs);
    S.v1 = (int)((long)a.V * (S.wg + 1) / kWgs);
}

// P0: group rows [gr0, gr1) of slot j out of group g's (G + 2) hd rows (q heads,
// then k, then v), as up to three sub-ranges of wq, wk, wv
struct QkvPart { int mat, r0, n, out0; };   // matrix, first row in it, rows, first output row
// part k of slot j's rows (k < qkv_nparts); computed in registers, no arrays
QD_HD inline void qkv_span(const StepArgs& a, int m, int* lo, int* hi) {
    const int qn = a.G * a.hd;
    *lo = m == 0 ? 0 : m == 1 ? qn : qn + a.hd;
    *hi = m == 0 ? qn : m == 1 ? qn + a.hd : qn + 2 * a.hd;
}
QD_HD inline int qkv_nparts(const StepArgs& a, int j) {
    const int RG = (a.G + 2) * a.hd;
    const int gr0 = j * RG / kSlotsPerXcd, gr1 = (j + 1) * RG / kSlotsPerXcd;
    int np = 0;
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        int lo, hi;
        qkv_span(a, m, &lo, &hi);
        np += qd_max(gr0, lo) < qd_min(gr1, hi) ? 1 : 0;
    }
    return np;
}
QD_HD inline QkvPart qkv_part(const StepArgs& a, int g, int j, int k) {
    const int RG = (a.G + 2) * a.hd, hd = a.hd, qn = a.G * a.hd;
    const int gr0 = j * RG / kSlotsPerXcd, gr1 = (j + 1) * RG / kSlotsPerXcd;
    QkvPart out{0, 0, 0, 0};
    int seen = 0;
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        int lo, hi;
        qkv_span(a, m, &lo, &hi);
        const int s = qd_max(gr0, lo), e = qd_min(gr1, hi);
        if (s < e) {
            if (seen == k) {
                const int base = m == 0 ? g * qn : g * hd;
                const int outb = m == 0 ? 0 : m == 1 ? a.Hq * hd : a.Hq * hd + a.Hkv * hd;
                out = QkvPart{m, base + s - lo, e - s, outb + base + s - lo};
            }
            ++seen;
        }
    }
    return out;
}
QD_HD inline const void* qkv_mat(const StepLayer& L, int m) { return m == 0 ? L.wq : m == 1 ? L.wk : L.wv; }
QD_HD inline const void* qkv_bias(const StepLayer& L, int m) { return m == 0 ? L.bq : m == 1 ? L.bk : L.bv; }

// bias of matrix rows [r0, r0 + n): the covering 16-byte-aligned range
QD_HD inline Blk bias_blk(const void* b, int r0, int n) {
    const long s = ((long)r0 * 2) & ~15L, e = (((long)(r0 + n) * 2) + 15) & ~15L;
    return Blk{(const char*)b + s, 1, (int)(e - s), 0};
}

// Blocks of one phase. P1's K/V pages are handled apart (their ids come from the
// block table, read once by the loader).
QD_HD inline int n_blocks(const StepArgs& a, const Sched& S, int ph) {
    const bool grp = S.xcd < a.Hkv;
    switch (ph) {
    case PH_QKV: {
        if (!grp) return 0;
        return 1 + qkv_nparts(a, S.slot) * (a.has_bias ? 2 : 1);
    }
    case PH_ATTN: return (grp && S.slot < a.S) ? (a.qk_norm ? 2 : 0) + 2 * S.npg : 0;
    case PH_O: return grp ? 1 : 0;
    case PH_UP: return 1 + 2 * ((S.f1 - S.f0 + kP3Rows - 1) / kP3Rows);
    case PH_DOWN: return 1;
    default: return a.lm_head ? 1 + (S.v1 - S.v0 + kLmRows - 1) / kLmRows : 0;
    }
}

// block k of phase ph of layer l (for PH_ATTN: the two norm gains only)
QD_HD inline Blk get_block(const StepArgs& a, const Sched& S, int l, int ph, int k) {
    const StepLayer& L = a.layer[l];
    const int D = a.D;
    switch (ph) {
    case PH_QKV: {
        if (k == 0) return Blk{(const char*)L.attn_norm, 1, D * 2, 0};
        const int per = a.has_bias ? 2 : 1;
        const QkvPart q = qkv_part(a, S.xcd, S.slot, (k - 1) / per);
        if (a.has_bias && ((k - 1) % per) == 0) return bias_blk(qkv_bias(L, q.mat), q.r0, q.n);
        return Blk{(const char*)qkv_mat(L, q.mat) + (long)q.r0 * D * 2, 1, q.n * D * 2, 0};
    }
    case PH_ATTN: return Blk{(const char*)(k == 0 ? L.q_norm : L.k_norm), 1, a.hd * 2, 0};
    case PH_O: {
        const int r0 = S.slot * D / kSlotsPerXcd, r1 = (S.slot + 1) * D / kSlotsPerXcd;
        const int cw = a.G * a.hd;   // the columns of group g
        return Blk{(const char*)L.wo + ((long)r0 * a.Hq * a.hd + (long)S.xcd * cw) * 2, r1 - r0, cw * 2,
                   (long)a.Hq * a.hd * 2};
    }
    case PH_UP: {
        if (k == 0) return Blk{(const char*)L.mlp_norm, 1, D * 2, 0};
        const int blk = (k - 1) >> 1, up = (k - 1) & 1;
        const int r0 = S.f0 + blk * kP3Rows, n = qd_min(kP3Rows, S.f1 - r0);
        return Blk{(const char*)(up ? L.w_up : L.w_gate) + (long)r0 * D * 2, 1, n * D * 2, 0};
    }
    case PH_DOWN: return Blk{(const char*)L.w_down + (long)S.d0 * a.F * 2, 1, (S.d1 - S.d0) * a.F * 2, 0};
    default: {
        if (k == 0) return Blk{(const char*)a.final_norm, 1, D * 2, 0};
        const int r0 = S.v0 + (k - 1) * kLmRows, n = qd_min(kLmRows, S.v1 - r0);
        return Blk{(const char*)a.lm_head + (long)r0 * D * 2, 1, n * D * 2, 0};
    }
    }
}

// the K (v = 0) or V (v = 1) page-head block of one page of group g
QD_HD inline Blk page_block(const StepArgs& a, int l, int g, int page_id, int v) {
    const StepLayer& L = a.layer[l];
    const long off = ((long)page_id * a.Hkv + g) * 16 * a.hd * 2;
    return Blk{(const char*)(v ? L.vc : L.kc) + off, 1, 16 * a.hd * 2, 0};
}

// Source of lane `lane`'s 16 bytes of slot i of block b, and whether the lane
// has bytes there (only a block's last slot can be partial).
QD_HD inline const char* dma_src(const Blk& b, uint32_t i, uint32_t lane, bool* active) {
    const uint32_t o = i * 1024u + lane * 16u;
    *active = (int)o < blk_bytes(b);
    if (b.rows == 1) return b.src + o;
    return b.src + (long)(o / (uint32_t)b.seg) * b.stride + (o % (uint32_t)b.seg);
}

// First page index and page count of split `slot` of C keys when the new token
// sits at position p (keys 0..p); no pages for a split past p.
QD_HD inline void split_pages(int slot, int C, int p, int* pg0, int* npg) {
    const int t0 = slot * C, t1 = qd_min(t0 + C, p + 1);
    *pg0 = t0 / 16;
    *npg = t1 > t0 ? (t1 - 1) / 16 - t0 / 16 + 1 : 0;
}

// Whether the one-launch batch-1 step takes a config (bf16 weights and KV cache,
// head_dim 64, every q/k/v bias or none, sizes its LDS buffers hold), and its
// attention plan for `tokens` keys: S splits of C keys (C a multiple of 64, at most
// 256; S at most 32, the workgroups of one XCD, and within what one input buffer
// holds of the split partials).
struct StepPlan {
    bool ok;
    int S, C;
    int up_wa, up_wb, down_wa, down_wb;   // row weights of gate|up and down: XCDs < Hkv, the others
};
inline int step_split_cap(const qd_config* c) {
    const int G = c->n_q_heads / c->n_kv_heads;
    return qd_min(32, kWork / (G * (c->head_dim + 2)));
}
inline bool step_config_ok(const qd_config* c) {
    const int G = c->n_q_heads / c->n_kv_heads, D = c->hidden, F = c->ffn;
    return c->w_dtype == QD_BF16 && c->kv_dtype == QD_BF16 && c->head_dim == 64 && c->n_kv_heads <= 8 &&
           G <= 8 && c->n_kv_heads * D <= 2048 && c->n_layers <= kStepMaxLayers && D <= 1024 && D % 8 == 0 &&
           F <= 2 * kXs && F % 8 == 0 && G * c->head_dim <= 512 && step_split_cap(c) >= 1 &&
           (long)((D + 255) / 256) * F * 2 <= 96 * 1024;   // a workgroup's down rows fit the ring
}
inline StepPlan plan_step(const qd_config* c, int tokens) {
    StepPlan sp{false, 0, 0, 1, 2, 1, 2};   // XCDs < Hkv also run q|k|v, attention and o_proj
    if (!step_config_ok(c)) return sp;
    const int cap = step_split_cap(c);
    int C = (tokens + cap - 1) / cap;
    C = qd_max(64, (C + 63) / 64 * 64);
    if (C > 256) return sp;
    sp.C = C;
    sp.S = (tokens + C - 1) / C;
    sp.ok = sp.S <= cap;
    return sp;
}

}  // namespace step
}  // namespace qd
