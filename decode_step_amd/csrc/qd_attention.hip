// Decode attention for gfx950: per-head q/k RMSNorm, RoPE, the KV append of the
// new token and split-K softmax attention over the paged cache.
//
// Work item = (split s of the context, group of `hpw` query heads of KV head g,
// sequence b), one workgroup of NWV waves each. LPT lanes hold one token's
// 16-byte row chunks, so a wave covers 64/LPT tokens per pass and every lane
// issues the loads of all its passes up front (page ids come from LDS, so no
// load waits on another). Query head h reads KV head h / group (repeat, not
// tile -- nanoinfer page, phase 3); splitting the query heads of one KV head
// over several workgroups spreads the score and value arithmetic over more
// CUs (each re-reads the same K/V rows, mostly from cache).
//
// Within a split the softmax is the plain two-pass one (scores to LDS, max,
// exp, sum). A context that fits one split writes the attention output
// directly; otherwise each split publishes (o, m, l) = (sum exp(s - m) v, max s,
// sum exp(s - m)) and a merge kernel combines them with weights exp(m_s - M),
// M = max m_s (Tang page, section 2.2: online softmax is a monoid; Table 1:
// split-K).
//
// The new token (position p) is not read from the cache: its k is projected,
// normed (8B-class shape), rotated, rounded to the cache type, written to its
// slot by one workgroup, and that stored value is what the scores use
// (nanoserve day 49: the step writes this token's K/V into its row before it
// attends; nanoinfer page, phase 4: keys are rotated once, on insert). Wave 0
// norms and rotates the query heads and the new k with the step's cos/sin table
// (built once per step by the input kernel; RoPE pairs i and i + hd/2, nanoinfer
// page, phase 3): a lane holds CE consecutive elements of a head and loads their
// rotation partners.
#include "qd_device.h"
#include "qd_launch.h"

namespace qd {

constexpr int kMaxGroup = 8;
constexpr int kAttnWaves = 8;    // waves per workgroup
// Token passes whose K/V rows a lane holds in registers: many for one query
// head per workgroup (a short context in one split), few for grouped heads,
// where fewer registers let two workgroups share a CU.
constexpr int kAttnPassesWide = 9;
constexpr int kAttnPassesGrouped = 4;
constexpr int kMaxSplits = 64;
constexpr int kAttnPage = 16;     // tokens per KV page (the only page size the library takes)
constexpr float kLog2e = 1.4426950408889634f;
// the matrix-core grouped kernel (attn_mfma_kernel)
constexpr int kAmKeys = 32;      // keys per block
constexpr int kAmWaves = 4;
constexpr int kAmBlocksPerWave = 2;
constexpr int kAmChunk = kAmWaves * kAmBlocksPerWave * kAmKeys;   // keys per split at most
constexpr int kAmHeads = 16;     // query heads per workgroup at most (the MFMA's columns)


// What a masked K/V row load (a key past the split, or without a page in the
// pool) reads instead of the cache: the load's address is chosen, not its
// result, so no load waits on a select before the next one is issued. Static
// device memory, zero from load time and never written (one row, any type).
__device__ __align__(16) uint32_t kAttnZeros[128];

// 2^x from the hardware exp2 (v_exp_f32); e^x = 2^(x log2 e)
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

template <int HD, typename KVT, int NP>
constexpr int attn_chunk() { return NP * kAttnWaves * (kWave / (HD / VecN<KVT>::n)); }

int attn_max_chunk(int hd, int kv_is_bf16, int grouped) {
    if (grouped && kv_is_bf16) return kAmChunk;   // the matrix-core kernel (decode steps)
    if (grouped) {
        if (hd == 64) return kv_is_bf16 ? attn_chunk<64, uint16_t, kAttnPassesGrouped>() : attn_chunk<64, float, kAttnPassesGrouped>();
        return kv_is_bf16 ? attn_chunk<128, uint16_t, kAttnPassesGrouped>() : attn_chunk<128, float, kAttnPassesGrouped>();
    }
    if (hd == 64) return kv_is_bf16 ? attn_chunk<64, uint16_t, kAttnPassesWide>() : attn_chunk<64, float, kAttnPassesWide>();
    return kv_is_bf16 ? attn_chunk<128, uint16_t, kAttnPassesWide>() : attn_chunk<128, float, kAttnPassesWide>();
}
int attn_max_splits() { return kMaxSplits; }

__device__ __forceinline__ void load_f32xN(const float* p, float* f, int n) {
#pragma unroll
    for (int q = 0; q < n / 4; ++q) {
        const float4 t = ((const float4*)p)[q];
        f[4 * q] = t.x; f[4 * q + 1] = t.y; f[4 * q + 2] = t.z; f[4 * q + 3] = t.w;
    }
}

// Half-split rotation of the CE elements a lane holds (`lower`: its elements are
// in the first half of the head); `pr` holds the partner elements i +- hd/2.
template <int CE>
__device__ __forceinline__ void rope_lane(float (&u)[CE], const float (&pr)[CE], const float (&c)[CE],
                                          const float (&sn)[CE], bool lower) {
#pragma unroll
    for (int e = 0; e < CE; ++e) u[e] = lower ? u[e] * c[e] - pr[e] * sn[e] : u[e] * c[e] + pr[e] * sn[e];
}

// Batch 1 with the projection in the attention launch (AttnArgs::fq): each
// workgroup forms 64 projection rows (one head) from x itself. 512 threads in 16
// groups of 32 lanes; group q takes rows 4q .. 4q + 3, and lane li of a group the
// 16-byte chunks li, li + 32, ... of those rows (8 bf16 or 16 int8 columns each),
// at most FqT<RT>::NC of them (x_dim <= kFqMaxD), so each chunk of x read from LDS
// serves four rows and a group's load of one row covers 512 contiguous bytes. All
// of a lane's row loads are issued before x is used; a chunk index past the row
// reads chunk 0 and meets a block of zeros in LDS (no load under a per-lane
// condition). int8 rows (nanoinfer page, phase 6) carry a float scale per row,
// applied to the finished dot product.
constexpr int kFqLanes = 32;
constexpr int kFqRows = 4;
template <typename RT> struct FqT {
    static constexpr int CE = VecN<RT>::n;                      // columns per 16-byte chunk
    static constexpr int NC = kFqMaxD / (CE * kFqLanes);        // chunks per lane per row
};

template <typename RT>
struct FqLoads {
    uint4 w[kFqRows][FqT<RT>::NC];
    float4 x;
    uint2 gain;
    float bias;    // of row 4q + (li & 3)
    float scale;   // int8: that row's scale (1 for bf16 rows)
    uint2 xe;      // x from the embedding: 4 bf16 values, or 4 int8 codes in xe.x
    float xs;      // ... their factor (int8: the row scale; 0 for an id outside the table)
};

// (cos, sin) of pair i of the RoPE table at position p: the angle p * theta^(-2i/hd)
// is formed and reduced modulo 2*pi in double, then its cosine and sine are taken in
// float (the step-input kernel and the first layer's fused launch share it).
__device__ __forceinline__ float2 rope_cs(float theta, int hd, int i, int p) {
    const double inv = pow((double)theta, -2.0 * (double)i / (double)hd);
    double ang = (double)p * inv;
    const double two_pi = 6.283185307179586476925286766559;
    ang -= two_pi * rint(ang / two_pi);
    float sv, cv;
    sincosf((float)ang, &sv, &cv);
    return make_float2(cv, sv);
}

// x as 4 floats: loaded, or widened from the embedding row
template <typename RT, bool EMB>
__device__ __forceinline__ float4 fq_xval(const FqLoads<RT>& f) {
    if constexpr (!EMB) {
        return f.x;
    } else if constexpr (sizeof(RT) == 1) {
        const uint32_t c = f.xe.x;
        return make_float4((float)(int8_t)(c & 0xffu) * f.xs, (float)(int8_t)((c >> 8) & 0xffu) * f.xs,
                           (float)(int8_t)((c >> 16) & 0xffu) * f.xs, (float)(int8_t)(c >> 24) * f.xs);
    } else {
        return make_float4(bf16_to_f32(f.xe.x & 0xffffu) * f.xs, bf16_to_f32(f.xe.x >> 16) * f.xs,
                           bf16_to_f32(f.xe.y & 0xffffu) * f.xs, bf16_to_f32(f.xe.y >> 16) * f.xs);
    }
}

// Issue the loads of rows row0 .. row0 + 63 of the matrix w ([rows][x_dim]), their
// bias (bf16, may be NULL), int8 row scale, x and its RMSNorm gain. The small loads
// go first and none sits under a condition (without a bias a weight is loaded and
// scaled by 0), so that waiting for them, or for anything issued before, leaves the
// rows in flight (loads complete in issue order). Compiler-only memory fences keep
// that order and keep the row loads ahead of any branch that follows (left alone,
// the compiler moves them below an early exit, behind a wait for the position).
template <typename RT, bool EMB>
__device__ __forceinline__ void fq_issue(const AttnArgs& a, const void* w, const void* bias, const float* scale,
                                         int row0, FqLoads<RT>& f) {
    constexpr int CE = FqT<RT>::CE, NC = FqT<RT>::NC;
    const int tid = threadIdx.x, D = a.x_dim, KC = D / CE;
    const int e4 = tid < D / 4 ? tid : 0;
    const int r0 = row0 + (tid / kFqLanes) * kFqRows, li = tid % kFqLanes;
    const long rbytes = (long)D * sizeof(RT);
    gbyte* wr = sgpr_gptr(w) + r0 * rbytes;
    if constexpr (!EMB) f.x = ((const float4*)a.fq_x)[e4];
    f.gain = ((const uint2*)a.fq_gain)[e4];
    gbyte* bp = sgpr_gptr(bias ? bias : w);
    f.bias = gld_scalar<uint16_t>(bp, bias ? r0 + (li & 3) : 0) * (bias ? 1.f : 0.f);
    if constexpr (sizeof(RT) == 1) f.scale = gld_scalar<float>(sgpr_gptr(scale), r0 + (li & 3));
    else f.scale = 1.f;
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < kFqRows; ++u)
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const int c = li + j * kFqLanes;
            f.w[u][j] = gld16(wr + (u * rbytes + (c < KC ? c : 0) * 16));
        }
    asm volatile("" ::: "memory");
    if constexpr (EMB) {   // behind the rows: its address waits for the token id
        const int tok = *(const __attribute__((address_space(4))) int*)a.fq_tok;
        const bool ok = tok >= 0 && tok < a.fq_vocab;
        const long e0 = (ok ? (long)tok * D : 0L) + 4L * e4;
        if constexpr (sizeof(RT) == 1) {
            f.xe = make_uint2(*(const uint32_t*)((const int8_t*)a.fq_embed + e0), 0u);
            f.xs = ok ? a.fq_embed_scale[tok] : 0.f;
        } else {
            f.xe = *(const uint2*)((const uint16_t*)a.fq_embed + e0);
            f.xs = ok ? 1.f : 0.f;
        }
    }
}

// The 64 rows' values r * (W (x * g)) + bias into out[64] (LDS), r = 1/sqrt(mean(x^2) + eps)
// (the RMSNorm folded into the product, as in the GEMV kernels). Barriers inside
// (every thread of the workgroup calls it); they are LDS-only, so loads issued
// after the rows (the K/V rows of the attention) stay in flight across them.
template <typename RT, bool EMB>
__device__ __forceinline__ void fq_finish(const AttnArgs& a, const FqLoads<RT>& f, float* out) {
    constexpr int NWV = kAttnWaves, CE = FqT<RT>::CE, NC = FqT<RT>::NC;
    static_assert(kFqRows == 4, "a row's bias and scale sit in lane li & 3");
    __shared__ __align__(16) float xg[kFqMaxD + 16];   // x * g, then one zero chunk
    __shared__ float wsq[NWV];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int D = a.x_dim, KC = D / CE;
    float ss = 0.f;
    if (tid < D / 4) {   // (waits for x only: the row loads stay in flight)
        const float4 v = fq_xval<RT, EMB>(f);
        ss = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        if (EMB && blockIdx.x == 0) ((float4*)const_cast<float*>(a.fq_x))[tid] = v;   // x for the launches that follow
        ((float4*)xg)[tid] = make_float4(v.x * bf16_to_f32(f.gain.x & 0xffffu), v.y * bf16_to_f32(f.gain.x >> 16),
                                         v.z * bf16_to_f32(f.gain.y & 0xffffu), v.w * bf16_to_f32(f.gain.y >> 16));
    }
    if (tid < CE) xg[KC * CE + tid] = 0.f;
    ss = group_sum<kWave>(ss);
    if (lane == 0) wsq[wave] = ss;
    lds_barrier();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) tot += wsq[w];
    const float r = 1.0f / sqrtf(tot / (float)D + a.eps);
    const int li = tid % kFqLanes;
    float acc[kFqRows] = {};
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c = li + j * kFqLanes;
        const float4* xp = (const float4*)(xg + (c < KC ? c : KC) * CE);
        float xv[CE];
#pragma unroll
        for (int q = 0; q < CE / 4; ++q) {
            const float4 t = xp[q];
            xv[4 * q] = t.x; xv[4 * q + 1] = t.y; xv[4 * q + 2] = t.z; xv[4 * q + 3] = t.w;
        }
#pragma unroll
        for (int u = 0; u < kFqRows; ++u) {
            float wf[CE];
            widen16(f.w[u][j], wf);
            float t = acc[u];
#pragma unroll
            for (int e = 0; e < CE; ++e) t = fmaf(wf[e], xv[e], t);
            acc[u] = t;
        }
    }
#pragma unroll
    for (int u = 0; u < kFqRows; ++u) acc[u] = group_sum<kFqLanes>(acc[u]);
    const int u = li & 3;
    const float mine = u == 0 ? acc[0] : u == 1 ? acc[1] : u == 2 ? acc[2] : acc[3];
    if (li < kFqRows) out[(tid / kFqLanes) * kFqRows + li] = fmaf(mine * f.scale, r, f.bias);
    lds_barrier();
}

// The step's position of sequence 0 as a scalar load (the constant address space):
// waiting for it leaves the vector loads in flight.
__device__ __forceinline__ int fq_pos(const AttnArgs& a) {
    return *(const __attribute__((address_space(4))) int*)a.pos;
}

// Element d of a 64-element head rotated by the step's table (pairs d and d ^ 32).
__device__ __forceinline__ float fq_rope(const float* v, const float2* tab, int d) {
    const float2 cs = tab[d & 31];
    const float u = v[d], pr = v[d ^ 32];
    return d < 32 ? u * cs.x - pr * cs.y : u * cs.x + pr * cs.y;
}

template <typename WT, typename KVT, int HD, int NP, bool FQ = false, typename RT = uint16_t, bool EMB = false>
__device__ __forceinline__ void attn_body(const AttnArgs& a, const int s, const int by, const int bz) {
    static_assert(!FQ || (HD == 64 && NP <= kAttnPassesGrouped), "projection in the launch: hd 64, grouped");
    constexpr int CE = VecN<KVT>::n;
    constexpr int LPT = HD / CE;
    constexpr int TPW = kWave / LPT;
    constexpr int NWV = kAttnWaves;
    constexpr int TPB = NWV * TPW;
    constexpr int MAXT = NP * TPB;
    constexpr int NT = NWV * kWave;
    constexpr int PG = kAttnPage;
    __shared__ float red[NWV][kMaxGroup][HD];   // each wave's o per head
    __shared__ float2 wml[NWV][kMaxGroup];      // each wave's (m, l) per head
    __shared__ float qs[kMaxGroup][HD];
    __shared__ uint4 knew[LPT];   // the new token's K and V rows in stored (cache-type) form
    __shared__ uint4 vnew[LPT];
    __shared__ int spage[MAXT / PG + 2];

    const int G = a.Hq / a.Hkv;
    const int hgroups = (G + a.hpw - 1) / a.hpw;
    const int g = by / hgroups, hg = by % hgroups, b = bz;
    const int h0 = hg * a.hpw, nh = min(a.hpw, G - h0);   // query heads g*G + h0 .. + nh - 1
    const bool prefill = a.prefill_start >= 0;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int li = lane % LPT, slot = lane / LPT;
    const int* bt = a.block_table + (prefill ? 0L : (long)b * a.max_blocks);
    const int t_begin = s * a.chunk;
    const int pg0 = t_begin / PG;

    // 1. the loads that do not need the position go out together with it: the page
    //    ids of the split's whole range and the q/k/v rows of the rotation (one
    //    head-chunk of CE elements per thread, LPT threads per head; item nh is the
    //    new k, loaded by every split and used by the one that holds p)
    int pgv = -1;
    if (tid < (a.chunk + PG - 1) / PG + 1 && pg0 + tid < a.max_blocks) pgv = bt[pg0 + tid];
    // (projection in this launch: the position, then the query head's rows and x
    // behind the page ids)
    FqLoads<RT> fql;
    int p_fq = 0;
    if constexpr (FQ) {
        p_fq = fq_pos(a);
        fq_issue<RT, EMB>(a, a.fq_w[0], a.qkv_bias[0], a.fq_scale[0], (g * G + h0) * HD, fql);
    }
    // first layer: the table row of this position, formed while the loads are out
    // (workgroup 0 stores it for the launches that follow)
    __shared__ float2 rtab[FQ && EMB ? 32 : 1];
    if constexpr (FQ && EMB) {
        if (tid < 32) {
            const float2 cs = rope_cs(a.theta, HD, tid, p_fq);
            rtab[tid] = cs;
            if (blockIdx.x == 0) const_cast<float2*>(a.rope)[tid] = cs;
        }
    }
    const int qkvr = (a.Hq + 2 * a.Hkv) * HD;
    const bool pro_ld = !FQ && !prefill && nh > 0 && tid < (nh + 1) * LPT;
    const int phl = tid / LPT, pl2 = tid % LPT, plp2 = pl2 ^ (LPT / 2);
    float u[CE], up[CE], cs[CE], sn[CE], vn[CE], gn[CE], gnp[CE];
    if (pro_ld) {
        const float* src = a.qkv + (long)b * qkvr;
        const float* hsrc = phl < nh ? src + (g * G + h0 + phl) * HD : src + a.Hq * HD + g * HD;
        load_f32xN(hsrc + pl2 * CE, u, CE);
        load_f32xN(hsrc + plp2 * CE, up, CE);
        const float2* tab = a.rope + (long)b * (HD / 2) + (pl2 % (LPT / 2)) * CE;
#pragma unroll
        for (int e = 0; e < CE; ++e) { const float2 t = tab[e]; cs[e] = t.x; sn[e] = t.y; }
        if (phl == nh) load_f32xN(src + (a.Hq + a.Hkv) * HD + g * HD + pl2 * CE, vn, CE);
        if (a.qk_norm) {   // the per-head norm gains of the lane's elements and partners
            const void* gain = phl < nh ? a.q_norm : a.k_norm;
#pragma unroll
            for (int e = 0; e < CE; ++e) { gn[e] = load_scalar<WT>(gain, pl2 * CE + e); gnp[e] = load_scalar<WT>(gain, plp2 * CE + e); }
        }
    }
    const int p = FQ ? p_fq : (prefill ? a.prefill_start + b : a.pos[b]);
    if (p < 0 || p >= a.capacity || a.chunk > MAXT || a.hpw > kMaxGroup || nh <= 0) return;
    // keys 0 .. p (0 .. p - 1 when the new token is the residual product's split);
    // split 0 always forms and publishes the rotated query head
    const int T = FQ ? p : p + 1;
    const int ns = min(a.S, (T + a.chunk - 1) / a.chunk);
    if (t_begin >= T && !(FQ && s == 0)) return;
    const int t_end = min(T, t_begin + a.chunk);
    const int n = t_end - t_begin;
    const bool has_new = !FQ && !prefill && p >= t_begin && p < t_end;
    const bool pro = pro_ld && tid < (nh + (has_new ? 1 : 0)) * LPT;   // whole LPT-lane groups
    if (prefill) {   // q already normed and rotated
        for (int idx = tid; idx < nh * HD; idx += NT) {
            const int hl = idx / HD, d = idx - hl * HD;
            qs[hl][d] = a.q_rot[((long)b * a.Hq + g * G + h0 + hl) * HD + d];
        }
    }

    // 2. page ids of this split's pages to LDS (an entry outside the pool reads as
    //    page 0 and is masked), then every K/V row load issued back to back
    const int npg = (t_end - 1) / PG - pg0 + 1;
    if (tid < npg) spage[tid] = (pgv >= 0 && pgv < a.num_pages) ? pgv : -1;
    if constexpr (FQ) lds_barrier();   // the projection rows stay in flight
    else __syncthreads();
    // (straight-line: a pass past the split reads the zero row, so no load result
    // is moved or selected before the last load is issued)
    uint4 kraw[NP], vraw[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int t = t_begin + i * TPB + wave * TPW + slot;
        const int tt = t < t_end ? t : t_begin;
        const int pg = spage[tt / PG - pg0];
        const bool ok = t < t_end && pg >= 0;   // the row at p is replaced below
        const long off = (((long)max(pg, 0) * a.Hkv + g) * PG + (tt % PG)) * HD + li * CE;
        const KVT* zr = (const KVT*)kAttnZeros + li * CE;
        kraw[i] = *(const uint4*)(ok ? (const KVT*)a.k_cache + off : zr);
        vraw[i] = *(const uint4*)(ok ? (const KVT*)a.v_cache + off : zr);
    }
    if constexpr (FQ) {   // the query head: project, rotate, publish (split 0)
        __shared__ float qraw[HD];
        fq_finish<RT, EMB>(a, fql, qraw);
        if (tid < HD) {
            const float q = fq_rope(qraw, EMB ? rtab : a.rope, tid);
            qs[0][tid] = q;
            if (s == 0) a.fq_out[(g * G + h0) * HD + tid] = q;
        }
        if (n <= 0) return;
    }

    // 3. [per-head q/k RMSNorm] and RoPE of the loaded rows; the new k and v go to
    //    LDS in stored form and (one workgroup per sequence and KV head) to the cache
    if (pro) {
        if (a.qk_norm) {   // per-head RMSNorm: the sum of squares over the head's LPT lanes
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < CE; ++e) ss += u[e] * u[e];
            ss = group_sum<LPT>(ss);
            const float r = 1.0f / sqrtf(ss / (float)HD + a.eps);
#pragma unroll
            for (int e = 0; e < CE; ++e) {
                u[e] = u[e] * r * gn[e];
                up[e] = up[e] * r * gnp[e];
            }
        }
        rope_lane<CE>(u, up, cs, sn, pl2 < LPT / 2);
        if (phl < nh) {
#pragma unroll
            for (int e = 0; e < CE; ++e) qs[phl][pl2 * CE + e] = u[e];
        } else {
            const uint4 kst = pack16<KVT>(u), vst = pack16<KVT>(vn);
            knew[pl2] = kst;
            vnew[pl2] = vst;
            if (hg == 0) {
                const int page_id = bt[p / PG];
                if (page_id >= 0 && page_id < a.num_pages) {
                    const long off = (((long)page_id * a.Hkv + g) * PG + (p % PG)) * HD + pl2 * CE;
                    *(uint4*)((KVT*)a.k_cache + off) = kst;
                    *(uint4*)((KVT*)a.v_cache + off) = vst;
                }
            }
        }
    }
    __syncthreads();
    // the new token's row, in stored form, replaces the (unread) cache row
    if (has_new) {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int t = t_begin + i * TPB + wave * TPW + slot;
            if (t == p) { kraw[i] = knew[li]; vraw[i] = vnew[li]; }
        }
    }

    // scores in base-2 units, s * log2(e), so that e^(s - m) = 2^(s' - m') comes from
    // the hardware exp2 (v_exp_f32, about 1 ulp); the partials for the merge keep
    // m in the same units
    const float scale2 = a.scale * kLog2e;
    const int hq0 = g * G + h0;   // first query head of this workgroup

    if (NP <= kAttnPassesGrouped && nh > 1) {
        // Grouped heads: scores to LDS, one wave per head takes the split's max, exp
        // and sum (each exponential once), then o = sum p v per head. (One head per
        // workgroup takes the per-wave form below: no score round trip through LDS
        // and no single-wave softmax.)
        __shared__ float sc[kMaxGroup][MAXT];
        __shared__ float mls[kMaxGroup][2];
        for (int hl = 0; hl < nh; ++hl) {
            float qv[CE];
#pragma unroll
            for (int e = 0; e < CE; ++e) qv[e] = qs[hl][li * CE + e];
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                if (i * TPB >= n) continue;
                const int j = i * TPB + wave * TPW + slot;
                float kf[CE];
                widen16(kraw[i], kf);
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < CE; ++e) d = fmaf(qv[e], kf[e], d);
                d = group_sum<LPT>(d);
                if (li == 0 && j < n) sc[hl][j] = d * scale2;
            }
        }
        __syncthreads();
        for (int hl = wave; hl < nh; hl += NWV) {
            float m = -INFINITY;
            for (int j = lane; j < n; j += kWave) m = fmaxf(m, sc[hl][j]);
            m = group_max<kWave>(m);
            float l = 0.f;
            for (int j = lane; j < n; j += kWave) {
                const float e = exp2_hw(sc[hl][j] - m);
                sc[hl][j] = e;
                l += e;
            }
            l = group_sum<kWave>(l);
            if (lane == 0) { mls[hl][0] = m; mls[hl][1] = l; }
        }
        __syncthreads();
        for (int hl = 0; hl < nh; ++hl) {
            float pr[NP], o[CE];
#pragma unroll
            for (int i = 0; i < NP; ++i) {   // the lane's probabilities up front (masked)
                const int j = i * TPB + wave * TPW + slot;
                const float v = sc[hl][j < n ? j : 0];
                pr[i] = j < n ? v : 0.f;
            }
#pragma unroll
            for (int e = 0; e < CE; ++e) o[e] = 0.f;
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                if (i * TPB >= n) continue;
                float vf[CE];
                widen16(vraw[i], vf);
#pragma unroll
                for (int e = 0; e < CE; ++e) o[e] = fmaf(pr[i], vf[e], o[e]);
            }
#pragma unroll
            for (int e = 0; e < CE; ++e) {
                const float v = strided_sum<LPT>(o[e]);
                if (slot == 0) red[wave][hl][li * CE + e] = v;
            }
        }
        __syncthreads();
        for (int idx = tid; idx < nh * HD; idx += NT) {
            const int hl = idx / HD, d = idx - hl * HD;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < NWV; ++w) v += red[w][hl][d];
            if (ns == 1 && !a.part_always) {
                a.ctx[((long)b * a.Hq + hq0) * HD + idx] = v / mls[hl][1];
            } else {   // publish (o, m, l) for the merge
                const long pi = ((long)b * a.Hq + hq0 + hl) * a.S + s;
                a.part[pi * HD + d] = v;
                if (d == 0) a.part_ml[pi] = make_float2(mls[hl][0], mls[hl][1]);
            }
        }
        return;
    }

    // 4. (one head per workgroup: many passes, or a split that fits the grouped
    //    form) per head, each wave over its own
    //    tokens: scores s = q.k/sqrt(hd) kept in
    //    registers, m = max s, p = exp(s - m), l = sum p, o = sum p v (the online
    //    softmax of Tang page, section 2.2, with the waves as its blocks)
    for (int hl = 0; hl < nh; ++hl) {
        float qv[CE];
#pragma unroll
        for (int e = 0; e < CE; ++e) qv[e] = qs[hl][li * CE + e];
        float sv[NP];
        float mw = -INFINITY;
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            sv[i] = -INFINITY;
            if (i * TPB >= n) continue;   // uniform; the loop itself is fully unrolled
            float kf[CE];
            widen16(kraw[i], kf);
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < CE; ++e) d = fmaf(qv[e], kf[e], d);
            d = group_sum<LPT>(d);
            const int j = i * TPB + wave * TPW + slot;
            sv[i] = j < n ? d * scale2 : -INFINITY;
            mw = fmaxf(mw, sv[i]);
        }
        mw = wave_max(mw);
        float lw = 0.f, o[CE];
#pragma unroll
        for (int e = 0; e < CE; ++e) o[e] = 0.f;
#pragma unroll
        for (int i = 0; i < NP; ++i) {   // fixed trip count (no early exit): the K/V
            if (i * TPB < n) {           // rows stay in registers, fully unrolled
                const float pr = sv[i] == -INFINITY ? 0.f : exp2_hw(sv[i] - mw);
                lw += pr;
                float vf[CE];
                widen16(vraw[i], vf);
#pragma unroll
                for (int e = 0; e < CE; ++e) o[e] = fmaf(pr, vf[e], o[e]);
            }
        }
        lw = strided_sum<LPT>(lw);
#pragma unroll
        for (int e = 0; e < CE; ++e) {
            const float v = strided_sum<LPT>(o[e]);
            if (slot == 0) red[wave][hl][li * CE + e] = v;
        }
        if (lane == 0) wml[wave][hl] = make_float2(mw, lw);
    }
    __syncthreads();

    // 5. the waves' (m, l, o) combined: M = max m_w, weights e^(m_w - M) (a wave
    //    without a valid token has m_w = -inf and weight 0)
    for (int idx = tid; idx < nh * HD; idx += NT) {
        const int hl = idx / HD, d = idx - hl * HD;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWV; ++w) M = fmaxf(M, wml[w][hl].x);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) {
            const float e = wml[w][hl].x == -INFINITY ? 0.f : exp2_hw(wml[w][hl].x - M);
            L = fmaf(wml[w][hl].y, e, L);
            O = fmaf(red[w][hl][d], e, O);
        }
        if (ns == 1 && !a.part_always) {
            a.ctx[((long)b * a.Hq + hq0) * HD + idx] = O / L;
        } else {   // publish (o, m, l) for the merge
            const long pi = ((long)b * a.Hq + hq0 + hl) * a.S + s;
            a.part[pi * HD + d] = O;
            if (d == 0) a.part_ml[pi] = make_float2(M, L);
        }
    }
}

// Two launch shapes of the same body: the grouped one (few passes) keeps its
// registers low enough for two workgroups per CU; the wide one (9 passes of K/V
// rows in registers) may use up to 256 VGPRs, one workgroup per CU, rather than
// spill.
template <typename WT, typename KVT, int HD, int NP>
__global__ __launch_bounds__(kAttnWaves * kWave) void attn_kernel(AttnArgs a) {
    attn_body<WT, KVT, HD, NP>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}
template <typename WT, typename KVT, int HD, int NP>
__global__ __launch_bounds__(kAttnWaves * kWave) __attribute__((amdgpu_waves_per_eu(1, 2)))
void attn_wide_kernel(AttnArgs a) {
    attn_body<WT, KVT, HD, NP>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

// The new token's k or v row of one KV head (workgroup j: KV head j / 2, k when j
// is even), projected like the query heads, k rotated, rounded to the cache type
// and stored at the position (nanoinfer page, phase 4: keys are rotated once, on
// insert); the stored values, widened, go to fq_out for the residual product.
template <typename RT, typename KVT, bool EMB>
__device__ __forceinline__ void fq_kv_body(const AttnArgs& a, int j) {
    constexpr int HD = 64, CE = VecN<KVT>::n, PG = kAttnPage;
    __shared__ float row[HD], st[HD];
    __shared__ float2 rtab[EMB ? 32 : 1];
    const int g = j >> 1, is_v = j & 1, tid = threadIdx.x;
    const int p = fq_pos(a);
    FqLoads<RT> f;
    fq_issue<RT, EMB>(a, is_v ? a.fq_w[2] : a.fq_w[1], is_v ? a.qkv_bias[2] : a.qkv_bias[1],
                      is_v ? a.fq_scale[2] : a.fq_scale[1], g * HD, f);
    if (p < 0 || p >= a.capacity) return;
    if constexpr (EMB) {   // first layer: the table row of this position
        if (tid < 32) rtab[tid] = rope_cs(a.theta, HD, tid, p);
    }
    fq_finish<RT, EMB>(a, f, row);   // (its barriers order the table's writes too)
    if (tid < HD) st[tid] = is_v ? row[tid] : fq_rope(row, EMB ? rtab : a.rope, tid);
    lds_barrier();
    if (tid < HD / CE) {
        float v[CE];
#pragma unroll
        for (int e = 0; e < CE; ++e) v[e] = st[tid * CE + e];
        const uint4 packed = pack16<KVT>(v);
        float w[CE];
        widen16(packed, w);
        float* out = a.fq_out + (long)(a.Hq + is_v * a.Hkv + g) * HD + tid * CE;
#pragma unroll
        for (int e = 0; e < CE; ++e) out[e] = w[e];
        const int page_id = a.block_table[p / PG];
        if (page_id >= 0 && page_id < a.num_pages) {
            const long off = (((long)page_id * a.Hkv + g) * PG + (p % PG)) * HD + tid * CE;
            *(uint4*)((KVT*)(is_v ? a.v_cache : a.k_cache) + off) = packed;
        }
    }
}

// Batch 1, projection in the launch: fq_attn_wgs(S, Hq) attention workgroups, then
// 2 * Hkv new-k/v workgroups. Workgroups whose ids agree mod 8 run on one XCD (one
// L2), so the S splits of a query head, which all read its projection rows, take
// ids 8 apart: id = 8 (S (h / 8) + s) + h % 8 (ids of heads past Hq exit at once).
__host__ __device__ constexpr int fq_attn_wgs(int S, int Hq) { return 8 * S * ((Hq + 7) / 8); }

template <typename RT, typename KVT, bool EMB>
__global__ __launch_bounds__(kAttnWaves * kWave) void attn_fq_kernel(AttnArgs a) {
    static_assert(kAttnWaves * kWave == 64 / kFqRows * kFqLanes, "one 64-row block per workgroup");
    const int n_att = fq_attn_wgs(a.S, a.Hq);
    const int id = blockIdx.x;
    if (id >= n_att) {
        fq_kv_body<RT, KVT, EMB>(a, id - n_att);
        return;
    }
    const int slot = id >> 3, h = (slot / a.S) * 8 + (id & 7), s = slot % a.S;
    if (h >= a.Hq) return;
    attn_body<uint16_t, KVT, 64, kAttnPassesGrouped, true, RT, EMB>(a, s, h, 0);
}

// ---------------------------------------------------------------------------
// Grouped decode attention on the matrix cores (bf16 KV cache, decode steps):
// one workgroup takes every query head of one KV head (G <= 16) over one split
// of the context, so each K/V row is read once, and the dot products run on
// v_mfma_f32_16x16x32_bf16 instead of lane reductions.
//
// Scores, transposed: S^T[key][head] = K Q^T with K straight from the paged
// cache as the A operand (a lane's 16-byte fragment is 8 consecutive dims of
// one key row) and q as the B operand (head = column; columns past G are
// zero). A lane then holds one head's scores for 4 keys of each 16-key half of
// a 32-key block, and those 8 scores are directly its B fragment of P^T for the
// product O^T[dim][head] = V^T P^T: the contraction runs over keys in the order
// (4 keys of half 0, 4 of half 1) per lane, and the V^T fragment (A operand)
// is read from LDS in that same key order. V is written into LDS transposed,
// [dim][key], per wave. q and P are float32, each split into bf16 hi + lo and
// multiplied twice (K and V are exact in bf16), keeping float32 accuracy.
//
// Each wave keeps an online softmax (m, l) per head over its blocks (Tang page,
// section 2.2); the waves' states meet in LDS and the split publishes
// (o, m, l) for the merge, or writes the context when it is the only split.
// The new token's q/k norm, RoPE and KV append are as in attn_body.
typedef __attribute__((ext_vector_type(8))) __bf16 am_bf16x8;
typedef __attribute__((ext_vector_type(4))) float am_f32x4;
__device__ __forceinline__ am_bf16x8 am_frag(uint4 v) { return __builtin_bit_cast(am_bf16x8, v); }


template <typename WT, int HD, int NSL>
__global__ __launch_bounds__(kAmWaves * kWave) void attn_mfma_kernel(AttnArgs a) {
    constexpr int NWV = kAmWaves, NBW = kAmBlocksPerWave;
    constexpr int NT = NWV * kWave;
    constexpr int KS = HD / 32;          // 32-dim slices of the score contraction
    constexpr int DT = HD / 16;          // 16-dim tiles of the output
    constexpr int VL = HD / 16;          // 16-byte V loads per lane per block (half a key row)
    constexpr int VTS = kAmKeys + 8;     // u16 per transposed V row (padded)
    constexpr int RS = HD + 4;           // floats per row of the wave-combine tile (padded)
    constexpr int LPT = HD / 8;          // lanes per head row in the rotation (8 elements each)
    constexpr int PG = kAttnPage;
    constexpr int VT_BYTES = NWV * HD * VTS * 2;
    static_assert(NWV * kAmHeads * RS * 4 <= VT_BYTES, "combine tile must fit the V tiles");
    __shared__ __align__(16) char smem[VT_BYTES];       // V^T tiles, then the combine tile
    __shared__ __align__(16) float qs[kAmHeads][HD];
    __shared__ uint4 knew[LPT];
    __shared__ uint4 vnew[LPT];
    __shared__ int spage[kAmChunk / PG + 2];
    __shared__ float2 wml[NWV][kAmHeads];

    const int G = a.Hq / a.Hkv;
    int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    if (a.compact) {   // the grid holds only splits with keys: find the sequence (uniform scan)
        const int id = blockIdx.x;
        b = 0;
        while (b + 1 < a.B && a.wg_base[b + 1] <= id) ++b;
        const int local = id - a.wg_base[b];
        s = local / a.Hkv;
        g = local - s * a.Hkv;
    }
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int c16 = lane & 15, q4 = lane >> 4;
    const int* bt = a.block_table + (long)b * a.max_blocks;
    const int t_begin = s * a.chunk;
    const int pg0 = t_begin / PG;

    // 1. loads that do not need the position, issued with it: the page ids of the
    //    split's whole range and the q/k rotation rows (the G query heads of KV
    //    head g and the new k (row G) and v, used by the split that holds p)
    int pgv = -1;
    if (tid < (a.chunk + PG - 1) / PG + 1 && pg0 + tid < a.max_blocks) pgv = bt[pg0 + tid];
    const int p = a.pos[b];
    const int qkvr = (a.Hq + 2 * a.Hkv) * HD;
    const bool pro_ld = G <= kAmHeads && tid < (G + 1) * LPT;
    const int phl = tid / LPT, pl2 = tid % LPT, plp2 = pl2 ^ (LPT / 2);
    float u[8], up[8], cs[8], sn[8], vn[8], gn[8], gnp[8];
    // q|k|v rows: the finished projection (NSL = 1), or its K-range partial products
    // (NSL slabs, the count given by the arguments, slabs past it read zeros), summed
    // after the barrier below as r * sum + bias with r the RMSNorm scale of the step's
    // input. Either way the loads go out here, with the position and the page ids,
    // and nothing waits for them before that barrier.
    constexpr bool PART = NSL > 1;
    float t[NSL][3][8], ssv[NSL];
    uint32_t bq[3][4];              // biases (PART), bf16 pairs (4-byte aligned: biases need no more)
    float sc[3][8];                 // int8 rows (PART): the rows' scales
    if (pro_ld) {
        const float* src = a.qkv + (long)b * qkvr;
        const int hoff = phl < G ? (g * G + phl) * HD : a.Hq * HD + g * HD;
        const int voff = (a.Hq + a.Hkv) * HD + g * HD;
        const float* z = (const float*)kAttnZeros;
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) {
            const bool on = !PART || sl < a.qkv_slabs;
            const float* ss = src + (long)sl * a.qkv_slab_stride;
            load_f32xN(on ? ss + hoff + pl2 * 8 : z, t[sl][0], 8);
            load_f32xN(on ? ss + hoff + plp2 * 8 : z, t[sl][1], 8);
            load_f32xN(on && phl == G ? ss + voff + pl2 * 8 : z, t[sl][2], 8);
            if (PART) ssv[sl] = *(on ? a.qkv_ss + sl * a.B + b : z);
        }
        if (PART) {
            // bias rows of the lane's head (pointers chosen among scalar registers)
            gbyte* const zb = (gbyte*)kAttnZeros;
            gbyte* const pq = sgpr_gptr(a.qkv_bias[0]);
            gbyte* const pk = sgpr_gptr(a.qkv_bias[1]);
            gbyte* const pv = sgpr_gptr(a.qkv_bias[2]);
            const bool hq = a.qkv_bias[0] != nullptr, hk = a.qkv_bias[1] != nullptr, hv = a.qkv_bias[2] != nullptr;
            const bool oh = phl < G ? hq : hk, ov = hv && phl == G;
            gbyte* const bh = phl < G ? pq + 2 * (g * G + phl) * HD : pk + 2 * g * HD;
            gbyte* const b0 = oh ? bh + 2 * pl2 * 8 : zb;
            gbyte* const b1 = oh ? bh + 2 * plp2 * 8 : zb;
            gbyte* const b2 = ov ? pv + 2 * (g * HD + pl2 * 8) : zb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bq[0][e] = *(const __attribute__((address_space(1))) uint32_t*)(b0 + 4 * e);
                bq[1][e] = *(const __attribute__((address_space(1))) uint32_t*)(b1 + 4 * e);
                bq[2][e] = *(const __attribute__((address_space(1))) uint32_t*)(b2 + 4 * e);
            }
            // int8 rows: the scales of the same rows (bf16 rows read zeros, unused)
            const bool i8 = a.qkv_scale[0] != nullptr;
            const float* const sh = phl < G ? a.qkv_scale[0] + (g * G + phl) * HD : a.qkv_scale[1] + g * HD;
            load_f32xN(i8 ? sh + pl2 * 8 : z, sc[0], 8);
            load_f32xN(i8 ? sh + plp2 * 8 : z, sc[1], 8);
            load_f32xN(i8 && phl == G ? a.qkv_scale[2] + g * HD + pl2 * 8 : z, sc[2], 8);
        }
        const float2* tab = a.rope + (long)b * (HD / 2) + (pl2 % (LPT / 2)) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) { const float2 t = tab[e]; cs[e] = t.x; sn[e] = t.y; }
        if (a.qk_norm) {   // the per-head norm gains of the lane's elements and partners
            const void* gain = phl < G ? a.q_norm : a.k_norm;
#pragma unroll
            for (int e = 0; e < 8; ++e) { gn[e] = load_scalar<WT>(gain, pl2 * 8 + e); gnp[e] = load_scalar<WT>(gain, plp2 * 8 + e); }
        }
    }
    if (p < 0 || p >= a.capacity || a.chunk > kAmChunk || G > kAmHeads) return;
    const int T = p + 1;
    const int ns = min(a.S, (T + a.chunk - 1) / a.chunk);
    if (t_begin >= T) return;
    const int t_end = min(T, t_begin + a.chunk);
    const int n = t_end - t_begin;
    const bool has_new = p >= t_begin && p < t_end;
    const bool pro = pro_ld && tid < (G + (has_new ? 1 : 0)) * LPT;

    // 2. page ids of the split to LDS (an entry outside the pool reads as page 0, masked)
    const int npg = (t_end - 1) / PG - pg0 + 1;
    if (tid < npg) spage[tid] = (pgv >= 0 && pgv < a.num_pages) ? pgv : -1;
    __syncthreads();
    if (pro_ld) {
        float ssl = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) { u[e] = t[0][0][e]; up[e] = t[0][1][e]; vn[e] = t[0][2][e]; }
        if (PART) ssl = ssv[0];
#pragma unroll
        for (int sl = 1; sl < NSL; ++sl) {
            ssl += ssv[sl];
#pragma unroll
            for (int e = 0; e < 8; ++e) { u[e] += t[sl][0][e]; up[e] += t[sl][1][e]; vn[e] += t[sl][2][e]; }
        }
        if (PART) {
            const float r = 1.0f / sqrtf(ssl / (float)a.x_dim + a.eps);
            const bool i8 = a.qkv_scale[0] != nullptr;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int sh = (e & 1) ? 16 : 0;
                u[e] = u[e] * (i8 ? r * sc[0][e] : r) + bf16_to_f32((bq[0][e >> 1] >> sh) & 0xffffu);
                up[e] = up[e] * (i8 ? r * sc[1][e] : r) + bf16_to_f32((bq[1][e >> 1] >> sh) & 0xffffu);
                vn[e] = vn[e] * (i8 ? r * sc[2][e] : r) + bf16_to_f32((bq[2][e >> 1] >> sh) & 0xffffu);
            }
        }
    }

    // 3. every K/V load of this wave's blocks (block wave + NWV j of the split): K as
    //    A fragments (key half*16 + c16, dims 32 kk + 8 q4), V rows (key lane % 32,
    //    dims (lane / 32) * HD/2 + 8 jj); a key past the split, at p or without a page
    //    reads a valid row and is zeroed
    uint4 kf[NBW][2][KS], vf[NBW][VL];
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
        const int kb = wave + NWV * j;
        const int kbase = t_begin + kb * kAmKeys;
        if (kb * kAmKeys >= n) {   // past the split (uniform over the wave): no loads
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) kf[j][half][kk] = make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int jj = 0; jj < VL; ++jj) vf[j][jj] = make_uint4(0, 0, 0, 0);
            continue;
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int t = kbase + half * 16 + c16;
            const int tt = t < t_end ? t : t_begin;
            const int pg = spage[tt / PG - pg0];
            const bool ok = t < t_end && pg >= 0;   // the row at p is replaced below
            const long off = (((long)max(pg, 0) * a.Hkv + g) * PG + (tt % PG)) * HD + 8 * q4;
            const uint16_t* src = ok ? (const uint16_t*)a.k_cache + off : (const uint16_t*)kAttnZeros + 8 * q4;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) kf[j][half][kk] = *(const uint4*)(src + 32 * kk);
        }
        {
            const int t = kbase + (lane & 31);
            const int tt = t < t_end ? t : t_begin;
            const int pg = spage[tt / PG - pg0];
            const bool ok = t < t_end && pg >= 0;
            const long off = (((long)max(pg, 0) * a.Hkv + g) * PG + (tt % PG)) * HD + (lane >> 5) * (HD / 2);
            const uint16_t* src = ok ? (const uint16_t*)a.v_cache + off : (const uint16_t*)kAttnZeros + (lane >> 5) * (HD / 2);
#pragma unroll
            for (int jj = 0; jj < VL; ++jj) vf[j][jj] = *(const uint4*)(src + 8 * jj);
        }
    }

    // 4. [per-head q/k RMSNorm] and RoPE; the new k and v rounded to bf16 go to LDS
    //    and to the cache (this is the only workgroup of (sequence, KV head) whose
    //    split holds p)
    if (pro) {
        if (a.qk_norm) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += u[e] * u[e];
            ss = group_sum<LPT>(ss);
            const float r = 1.0f / sqrtf(ss / (float)HD + a.eps);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                u[e] = u[e] * r * gn[e];
                up[e] = up[e] * r * gnp[e];
            }
        }
        rope_lane<8>(u, up, cs, sn, pl2 < LPT / 2);
        if (phl < G) {
#pragma unroll
            for (int e = 0; e < 8; ++e) qs[phl][pl2 * 8 + e] = u[e];
        } else {
            const uint4 kst = pack16<uint16_t>(u), vst = pack16<uint16_t>(vn);
            knew[pl2] = kst;
            vnew[pl2] = vst;
            const int page_id = bt[p / PG];
            if (page_id >= 0 && page_id < a.num_pages) {
                const long off = (((long)page_id * a.Hkv + g) * PG + (p % PG)) * HD + pl2 * 8;
                *(uint4*)((uint16_t*)a.k_cache + off) = kst;
                *(uint4*)((uint16_t*)a.v_cache + off) = vst;
            }
        }
    }
    __syncthreads();
    if (has_new) {   // the new token's rows, in stored form, replace the (unread) cache rows
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            const int kbase = t_begin + (wave + NWV * j) * kAmKeys;
#pragma unroll
            for (int half = 0; half < 2; ++half)
                if (kbase + half * 16 + c16 == p)
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk) kf[j][half][kk] = knew[4 * kk + q4];
            if (kbase + (lane & 31) == p)
#pragma unroll
                for (int jj = 0; jj < VL; ++jj) vf[j][jj] = vnew[(lane >> 5) * (HD / 16) + jj];
        }
    }

    // 5. q^T as B fragments: head c16 (zero past G), dims 32 kk + 8 q4, bf16 hi + lo
    uint4 qh[KS], ql[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = c16 < G ? qs[c16][32 * kk + 8 * q4 + e] : 0.f;
        split_hi_lo(v, qh[kk], ql[kk]);
    }

    // 6. the wave's blocks: scores in base-2 units (s * log2 e, so that e^(s - m) is the
    //    hardware exp2 of s' - m'), online softmax for head c16, O^T += V^T P^T
    const float scale2 = a.scale * kLog2e;
    float m = -INFINITY, l = 0.f;        // l: this lane's share (its keys of each block)
    am_f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = am_f32x4{0.f, 0.f, 0.f, 0.f};
    uint16_t* vtw = (uint16_t*)smem + wave * HD * VTS;
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
        const int kb = wave + NWV * j;
        if (kb * kAmKeys >= n) break;    // uniform over the wave
        const int kbase = t_begin + kb * kAmKeys;
        // V^T of the block into the wave's tile: vtw[dim][key]
#pragma unroll
        for (int jj = 0; jj < VL; ++jj) {
            const uint32_t w4[4] = {vf[j][jj].x, vf[j][jj].y, vf[j][jj].z, vf[j][jj].w};
            const int d0 = (lane >> 5) * (HD / 2) + 8 * jj;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vtw[(d0 + 2 * e) * VTS + (lane & 31)] = (uint16_t)(w4[e] & 0xffffu);
                vtw[(d0 + 2 * e + 1) * VTS + (lane & 31)] = (uint16_t)(w4[e] >> 16);
            }
        }
        float sv[8];
        float mx = -INFINITY;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            am_f32x4 sacc = am_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am_frag(kf[j][half][kk]), am_frag(qh[kk]), sacc, 0, 0, 0);
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am_frag(kf[j][half][kk]), am_frag(ql[kk]), sacc, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool valid = kbase + half * 16 + 4 * q4 + e < t_end;
                sv[half * 4 + e] = valid ? sacc[e] * scale2 : -INFINITY;
                mx = fmaxf(mx, sv[half * 4 + e]);
            }
        }
        mx = swap32_max(swap16_max(mx));       // over the block's 32 keys
        const float mn = fmaxf(m, mx);         // finite: key kbase is valid
        const float alpha = exp2_hw(m - mn);   // 0 while m = -inf
        float pv[8];
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            pv[i] = sv[i] == -INFINITY ? 0.f : exp2_hw(sv[i] - mn);
            ps += pv[i];
        }
        l = fmaf(l, alpha, ps);
        m = mn;
        uint4 ph, pl;
        split_hi_lo(pv, ph, pl);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            o[dt] *= alpha;
            const uint16_t* row = vtw + (dt * 16 + c16) * VTS;
            const uint2 v0 = *(const uint2*)(row + 4 * q4);
            const uint2 v1 = *(const uint2*)(row + 16 + 4 * q4);
            const uint4 vfr = make_uint4(v0.x, v0.y, v1.x, v1.y);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am_frag(vfr), am_frag(ph), o[dt], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am_frag(vfr), am_frag(pl), o[dt], 0, 0, 0);
        }
    }

    // 7. l over the lanes of head c16; the waves' (m, l, o) meet in LDS: M = max m_w,
    //    weights 2^(m_w - M) (a wave without a block has m_w = -inf and weight 0)
    l = strided_sum<16>(l);
    __syncthreads();                       // every wave is done with its V tile
    float* red = (float*)smem;             // [NWV][16][RS]: o^T of each wave, as [head][dim]
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        *(float4*)(red + (wave * kAmHeads + c16) * RS + dt * 16 + 4 * q4) =
            make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (lane < kAmHeads) wml[wave][lane] = make_float2(m, l);
    __syncthreads();
    const int hq0 = g * G;
    for (int idx = tid; idx < G * HD; idx += NT) {
        const int hl = idx / HD, d = idx - hl * HD;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWV; ++w) M = fmaxf(M, wml[w][hl].x);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) {
            const float e = wml[w][hl].x == -INFINITY ? 0.f : exp2_hw(wml[w][hl].x - M);
            L = fmaf(wml[w][hl].y, e, L);
            O = fmaf(red[(w * kAmHeads + hl) * RS + d], e, O);
        }
        if (ns == 1 && !a.part_always) {
            a.ctx[((long)b * a.Hq + hq0) * HD + idx] = O / L;
        } else {   // publish (o, m, l) for the merge
            const long pi = ((long)b * a.Hq + hq0 + hl) * a.S + s;
            a.part[pi * HD + d] = O;
            if (d == 0) a.part_ml[pi] = make_float2(M, L);
        }
    }
}

// Merge of the split partials of one (query head, sequence): M = max_s m_s,
// ctx = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M) (the attention kernel keeps
// m in base-2 units, so this is the e^(m_s - M) weighting). The 256 threads form
// 256/hd groups that take every (256/hd)-th split: the first 32 of each group
// are loaded together with the (m, l) pairs, any further ones 16 at a time; the
// groups' sums meet in LDS in a fixed order.
constexpr int kMergeThreads = 256;
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(AttnArgs a) {
    __shared__ float wgt[kMaxSplits];
    __shared__ float lsum;
    __shared__ float osum[kMergeThreads];
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int p = a.prefill_start >= 0 ? a.prefill_start + b : a.pos[b];
    if (p < 0 || p >= a.capacity) return;
    const int ns = min(min(a.S, kMaxSplits), (p + 1 + a.chunk - 1) / a.chunk);
    if (ns <= 1) return;   // one split: the attention kernel wrote the output itself
    const int hd = a.hd;
    const float* base = a.part + ((long)b * a.Hq + h) * a.S * hd;
    const float2* mlb = a.part_ml + ((long)b * a.Hq + h) * a.S;
    const int ng = kMergeThreads / hd, grp = tid / hd, d = tid - grp * hd;
    // the first 32 partials of this thread's group are loaded before anything waits,
    // so they share one memory round trip with the (m, l) loads below
    constexpr int kFirst = 32;
    float v0[kFirst];
#pragma unroll
    for (int u = 0; u < kFirst; ++u) {
        const int j = grp + u * ng;
        v0[u] = base[(j < ns ? j : 0) * hd + d];
    }
    if (tid < kWave) {   // wave 0: weights of the splits
        const float2 ml = mlb[tid < ns ? tid : 0];
        const float mj = tid < ns ? ml.x : -INFINITY;
        const float lj = tid < ns ? ml.y : 0.f;
        const float m = group_max<kWave>(mj);
        const float w = tid < ns ? exp2_hw(mj - m) : 0.f;   // m in base-2 units
        if (tid < ns) wgt[tid] = w;
        const float l = group_sum<kWave>(lj * w);
        if (tid == 0) lsum = l;
    }
    __syncthreads();
    float o = 0.f;
#pragma unroll
    for (int u = 0; u < kFirst; ++u) {
        const int j = grp + u * ng;
        if (j < ns) o = fmaf(v0[u], wgt[j], o);
    }
    for (int j0 = grp + kFirst * ng; j0 < ns; j0 += 16 * ng) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int j = j0 + u * ng;
            v[u] = base[(j < ns ? j : 0) * hd + d];
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int j = j0 + u * ng;
            if (j < ns) o = fmaf(v[u], wgt[j], o);
        }
    }
    osum[tid] = o;
    __syncthreads();
    if (tid < hd) {
        float t = osum[tid];
        for (int q = 1; q < ng; ++q) t += osum[q * hd + tid];
        a.ctx[((long)b * a.Hq + h) * hd + tid] = t / lsum;
    }
}

bool attn_uses_mfma(const AttnArgs& a, int kv_is_bf16) {
    const int G = a.Hq / a.Hkv;
    return kv_is_bf16 && a.prefill_start < 0 && a.hpw == G && G <= kAmHeads &&
           (G + 1) * (a.hd / 8) <= kAmWaves * kWave && a.chunk <= kAmChunk && (a.hd == 64 || a.hd == 128);
}

bool attn_fq_ok(const AttnArgs& a, int w_type, int kv_is_bf16) {
    const int chunk_max = kv_is_bf16 ? attn_chunk<64, uint16_t, kAttnPassesGrouped>()
                                     : attn_chunk<64, float, kAttnPassesGrouped>();
    const int ce = w_type == 2 ? 16 : 8;   // columns per 16-byte chunk (int8 or bf16 rows)
    return (w_type == 1 || w_type == 2) && a.B == 1 && a.hd == 64 && a.hpw == 1 && !a.qk_norm &&
           a.prefill_start < 0 && a.part_always && !a.compact && a.qkv_slabs == 0 && a.x_dim >= ce &&
           a.x_dim <= kFqMaxD && a.x_dim % ce == 0 && a.chunk <= chunk_max && a.Hq % a.Hkv == 0;
}

hipError_t launch_attention(const AttnArgs& a, int w_is_bf16, int kv_is_bf16, hipStream_t s) {
    if (a.page != kAttnPage) return hipErrorInvalidValue;
    if (a.fq) {   // int8 rows when the row scales are given
        const bool i8 = a.fq_scale[0] != nullptr;
        if (!w_is_bf16 || !attn_fq_ok(a, i8 ? 2 : 1, kv_is_bf16) || !a.fq_x || !a.fq_gain || !a.fq_w[0] ||
            !a.fq_w[1] || !a.fq_w[2] || !a.fq_out || (i8 && (!a.fq_scale[1] || !a.fq_scale[2])))
            return hipErrorInvalidValue;
        if (a.fq_tok && (!a.fq_embed || a.fq_vocab < 1 || !a.rope || (i8 && !a.fq_embed_scale)))
            return hipErrorInvalidValue;
        const dim3 grid(fq_attn_wgs(a.S, a.Hq) + 2 * a.Hkv), block(kAttnWaves * kWave);
#define QD_FQ(RT, KVT)                                                                            \
        if (a.fq_tok) hipLaunchKernelGGL((attn_fq_kernel<RT, KVT, true>), grid, block, 0, s, a); \
        else hipLaunchKernelGGL((attn_fq_kernel<RT, KVT, false>), grid, block, 0, s, a);
        if (i8) {
            if (kv_is_bf16) { QD_FQ(int8_t, uint16_t) } else { QD_FQ(int8_t, float) }
        } else {
            if (kv_is_bf16) { QD_FQ(uint16_t, uint16_t) } else { QD_FQ(uint16_t, float) }
        }
#undef QD_FQ
        return hipGetLastError();
    }
    const int G = a.Hq / a.Hkv;
    const int hgroups = (G + a.hpw - 1) / a.hpw;
    const bool mfma = attn_uses_mfma(a, kv_is_bf16);
    if (a.qkv_slabs > 0 && (!mfma || !w_is_bf16 || a.qkv_slabs > kGemm16MaxStoreSplits || !a.qkv_ss || a.x_dim < 1))
        return hipErrorInvalidValue;
    if (a.compact && (!mfma || a.B > kAttnMaxBatch || a.wg_base[0] != 0)) return hipErrorInvalidValue;
    if (mfma) {
        const dim3 grid = a.compact ? dim3(a.wg_base[a.B]) : dim3(a.S, a.Hkv, a.B), block(kAmWaves * kWave);
        if (a.compact && a.wg_base[a.B] < 1) return hipSuccess;   // no keys anywhere (positions out of range)
#define QD_AM(WT, NSL)                                                                             \
        if (a.hd == 64) hipLaunchKernelGGL((attn_mfma_kernel<WT, 64, NSL>), grid, block, 0, s, a); \
        else hipLaunchKernelGGL((attn_mfma_kernel<WT, 128, NSL>), grid, block, 0, s, a);
        if (a.qkv_slabs > 0) { QD_AM(uint16_t, kGemm16MaxStoreSplits) }
        else if (w_is_bf16) { QD_AM(uint16_t, 1) } else { QD_AM(float, 1) }
#undef QD_AM
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || a.S == 1 || a.part_always) return e;
        hipLaunchKernelGGL(attn_merge_kernel, dim3(a.Hq, a.B), dim3(kMergeThreads), 0, s, a);
        return hipGetLastError();
    }
    dim3 grid(a.S, a.Hkv * hgroups, a.B);
    dim3 block(kAttnWaves * kWave);
#define QD_ATTN(WT, KVT, HD)                                                                          \
    do {                                                                                              \
        if (a.chunk <= attn_chunk<HD, KVT, kAttnPassesGrouped>())                                     \
            hipLaunchKernelGGL((attn_kernel<WT, KVT, HD, kAttnPassesGrouped>), grid, block, 0, s, a); \
        else                                                                                          \
            hipLaunchKernelGGL((attn_wide_kernel<WT, KVT, HD, kAttnPassesWide>), grid, block, 0, s, a); \
    } while (0)
    if (a.hd == 64) {
        if (w_is_bf16) { if (kv_is_bf16) QD_ATTN(uint16_t, uint16_t, 64); else QD_ATTN(uint16_t, float, 64); }
        else { if (kv_is_bf16) QD_ATTN(float, uint16_t, 64); else QD_ATTN(float, float, 64); }
    } else {
        if (w_is_bf16) { if (kv_is_bf16) QD_ATTN(uint16_t, uint16_t, 128); else QD_ATTN(uint16_t, float, 128); }
        else { if (kv_is_bf16) QD_ATTN(float, uint16_t, 128); else QD_ATTN(float, float, 128); }
    }
#undef QD_ATTN
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.S == 1 || a.part_always) return e;   // part_always: the consumer merges
    hipLaunchKernelGGL(attn_merge_kernel, dim3(a.Hq, a.B), dim3(kMergeThreads), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Step input: x = embedding row (exact widen; tied table, nanoinfer page, model
// notes) or the given x_in row, and the step's RoPE table: for position p and
// pair i, the angle p * theta^(-2i/hd) is formed and reduced modulo 2*pi in
// double, then its cosine and sine are taken in float. An id outside [0, V)
// yields a zero row instead of a fault.
template <typename WT>
__global__ __launch_bounds__(256) void step_input_kernel(StepInputArgs a) {
    const int b = blockIdx.x, tid = threadIdx.x;
    float* x = a.x + (long)b * a.D;
    if (a.tokens) {
        const int tok = a.tokens[b];
        const bool ok = tok >= 0 && tok < a.V;
        const void* row = (const char*)a.embed + (ok ? (long)tok * a.D * (long)sizeof(WT) : 0L);
        if constexpr (sizeof(WT) == 1) {   // int8 row times its scale (nanoinfer, phase 6)
            const float sc = ok ? a.embed_scale[tok] : 0.f;
            for (int d = tid; d < a.D; d += blockDim.x) x[d] = (float)((const int8_t*)row)[d] * sc;
        } else {
            for (int d = tid; d < a.D; d += blockDim.x) x[d] = ok ? load_scalar<WT>(row, d) : 0.f;
        }
    } else {
        for (int d = tid; d < a.D; d += blockDim.x) x[d] = a.x_in[(long)b * a.D + d];
    }
    const int half = a.hd / 2;
    if (tid < half) a.rope[(long)b * half + tid] = rope_cs(a.theta, a.hd, tid, a.pos[b]);
}

hipError_t launch_step_input(const StepInputArgs& a, int w_type, hipStream_t s) {
    if (w_type == 2) hipLaunchKernelGGL((step_input_kernel<int8_t>), dim3(a.B), dim3(256), 0, s, a);
    else if (w_type == 1) hipLaunchKernelGGL((step_input_kernel<uint16_t>), dim3(a.B), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((step_input_kernel<float>), dim3(a.B), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace qd
