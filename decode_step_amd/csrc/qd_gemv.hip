// Single-row (batch 1) GEMV for gfx950, tuned for latency.
//
// A decode-step projection is an HBM stream of a row-major [N][K] weight
// matrix against one activation vector. Each lane issues every weight load of
// its tile before anything else; the activation (and the RMSNorm gain) go to
// LDS by DMA behind them, so a workgroup waits for memory once per tile.
//
// RMSNorm is folded into the product (Tang page, section 2.3, epilogues on the
// reducing thread): W (x * r * g) = r * (W (x * g)) with r = 1/sqrt(sum(x^2)/K + eps)
// (nanocompile page, phase 1: the mean square is a sum then a divide; eps
// inside the root); one pass over the staged x forms x * g and sum(x^2), and r
// scales the finished dot product.
//
// Layout of one workgroup (256 threads = 4 waves): LPR lanes share a row and
// read 16-byte chunks lane-interleaved (each wave load covers 64/LPR rows of
// LPR*16 contiguous bytes); WK waves split K and meet in LDS; UR row groups
// per lane; CPL chunks per lane per row per pass.
//
// No load sits under a per-lane condition: a lane whose chunk lies past its K
// range (or whose row lies past N) loads a valid chunk of a valid row and
// multiplies it by a block of zeros kept in LDS behind x. (A masked load would
// be turned into a branch, and the compiler then waits for every outstanding
// load where the branches join.)
#include "qd_device.h"
#include "qd_launch.h"

namespace qd {

constexpr int kCus = 256;
#ifndef QD_B1_OCFG
#define QD_B1_OCFG 0        // GEMV shape of the residual product that merges attention splits
#endif

// floats of x staged in LDS: K rounded up to whole 1 KB DMA blocks
__host__ __device__ constexpr int gemv1_xpad(int K) { return (K + 255) & ~255; }
// bytes of gain staged in LDS (whole 1 KB blocks)
__host__ __device__ constexpr int gemv1_gpad(int K, int wbytes) { return (K * wbytes + 1023) & ~1023; }
// floats of zeros staged behind x (one chunk of the widest weight type, int8's 16)
constexpr int kG1Zeros = 16;

// Splits of the decode attention that the residual product can merge itself
// (MS > 0: x is formed from the attention's partials, at most MS of them).
constexpr int kG1MergeHeads = 32;

template <typename WT, int LPR, int WK, int UR, int CPL, int EPI, int MS = 0>
__global__ __launch_bounds__(256) void gemv1_kernel(GemvArgs a) {
    constexpr int CE = VecN<WT>::n;
    using GT = typename GainT<WT>::type;      // gains and biases
    constexpr bool I8 = sizeof(WT) == 1;      // int8 rows carry a float scale each
    constexpr int RPW = kWave / LPR;
    constexpr int WR = 4 / WK;
    constexpr int RPT = WR * RPW * UR;
    constexpr int NW = (EPI == EPI_SWIGLU) ? 2 : 1;
    extern __shared__ __align__(16) float xs[];   // x (then x * g) [xpad] | zeros [16] | gain [gpad bytes]
    __shared__ float wsum[4];
    __shared__ float red[WK][RPT][NW];
    __shared__ float red_v[4];
    __shared__ int red_i[4];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int wr = wave % WR, wk = wave / WR;
    const int li = lane % LPR, slot = lane / LPR;
    const int K = a.K, N = a.N, KC = K / CE;
    const int kcw = (KC + WK - 1) / WK;
    const int kc0 = min(KC, wk * kcw), kc1 = min(KC, kc0 + kcw);
    const int ntiles = (N + RPT - 1) / RPT;
    const int xpad = gemv1_xpad(K);
    const int cz = xpad / CE;                 // chunk index of the zero block
    float* gs = xs + xpad + kG1Zeros;

    gbyte* wseg[3] = {sgpr_gptr(a.w[0]), sgpr_gptr(a.w[1]), sgpr_gptr(a.w[2])};
    gbyte* bseg[3] = {sgpr_gptr(a.bias[0]), sgpr_gptr(a.bias[1]), sgpr_gptr(a.bias[2])};
    gbyte* sseg[3] = {sgpr_gptr(a.wscale[0]), sgpr_gptr(a.wscale[1]), sgpr_gptr(a.wscale[2])};
    auto wptr = [&](int r, int n) -> gbyte* {   // r < N
        if (EPI == EPI_SWIGLU) return wseg[n] + (long)r * K * (long)sizeof(WT);
        const bool s0 = r < a.seg_end[0], s1 = r < a.seg_end[1];
        gbyte* w = s0 ? wseg[0] : (s1 ? wseg[1] : wseg[2]);
        const int base = s0 ? 0 : (s1 ? a.seg_end[0] : a.seg_end[1]);
        return w + (long)(r - base) * K * (long)sizeof(WT);
    };
    uint4 wv[UR][NW][CPL];
    float pre[UR] = {};   // RESID: the residual row; STORE: the bias, times psc (0 without one)
    float psc[UR] = {};
    float srow[UR][NW];   // int8: the rows' scales (1 otherwise)
#pragma unroll
    for (int u = 0; u < UR; ++u)
#pragma unroll
        for (int n = 0; n < NW; ++n) srow[u][n] = 1.f;
    auto issue = [&](int tile, int cbase, bool first) {
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int r = tile * RPT + (wr * UR + u) * RPW + slot;
            const int rr = r < N ? r : N - 1;
#pragma unroll
            for (int n = 0; n < NW; ++n) {
                gbyte* wp = wptr(rr, n);
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    const int c = cbase + li + j * LPR;
                    wv[u][n][j] = gld16(wp + (long)(c < kc1 ? c : 0) * 16);
                }
            }
            if (first && EPI == EPI_RESID) { pre[u] = a.y[rr]; psc[u] = 1.f; }
            if (first && EPI == EPI_STORE) {
                const bool s0 = rr < a.seg_end[0], s1 = rr < a.seg_end[1];
                gbyte* bsel = s0 ? bseg[0] : (s1 ? bseg[1] : bseg[2]);
                const int base = s0 ? 0 : (s1 ? a.seg_end[0] : a.seg_end[1]);
                // without a bias: load a valid weight and scale it by 0 (the scale is
                // applied in the epilogue, so nothing waits for this load before then)
                pre[u] = gld_scalar<GT>(bsel ? bsel : wseg[0], bsel ? rr - base : 0);
                psc[u] = bsel ? 1.f : 0.f;
            }
            if (first && I8) {
#pragma unroll
                for (int n = 0; n < NW; ++n) {
                    if (EPI == EPI_SWIGLU) {
                        srow[u][n] = gld_scalar<float>(sseg[n], rr);
                    } else {
                        const bool s0 = rr < a.seg_end[0], s1 = rr < a.seg_end[1];
                        gbyte* ssel = s0 ? sseg[0] : (s1 ? sseg[1] : sseg[2]);
                        srow[u][n] = gld_scalar<float>(ssel, rr - (s0 ? 0 : (s1 ? a.seg_end[0] : a.seg_end[1])));
                    }
                }
            }
        }
    };
    int tile = blockIdx.x;

    // The vector (or the attention partials) goes out first and the weights right
    // behind it, so that waiting for it leaves the weights in flight and the RMSNorm
    // pass (or the merge of the attention splits) runs under their latency; the
    // wide-row shapes (LPR = 64, the K = 4096+ rows of the 8B-class shape) keep the
    // weights first (measured: x first costs them about 1%). MS > 0: this thread's
    // four context elements from every
    // split, and (threads below Hq) head tid's split maxima and sums, from clamped
    // (always valid) indices; splits past the valid count are masked below.
    float4 ov[MS > 0 ? MS : 1];
    float2 mlv[MS > 0 ? MS : 1];
    float4 qn, kn, vn;   // with part_new: this thread's elements of q, k_new and v_new
    int ns = 0;
    if constexpr (MS > 0) {
        const int hd = a.part_hd, S = a.part_S;
        const int e0 = 4 * tid < K ? 4 * tid : 0;
        const int hh = e0 / hd, d = e0 - hh * hd;
        const int hm = tid < K / hd ? tid : 0;
#pragma unroll
        for (int sp = 0; sp < MS; ++sp) {
            const int sc = sp < S ? sp : S - 1;
            ov[sp] = *(const float4*)(a.part + ((long)hh * S + sc) * hd + d);
        }
        const int p = a.part_pos[0];
        if (a.part_new) {   // every thread: its head's (m, l) pairs and its new-token elements
#pragma unroll
            for (int sp = 0; sp < MS; ++sp) mlv[sp] = a.part_ml[(long)hh * S + (sp < S ? sp : S - 1)];
            const int Hq = K / hd, gk = hh / (Hq / a.part_kv_heads);
            qn = *(const float4*)(a.part_new + e0);
            kn = *(const float4*)(a.part_new + (long)(Hq + gk) * hd + d);
            vn = *(const float4*)(a.part_new + (long)(Hq + a.part_kv_heads + gk) * hd + d);
            ns = p >= 0 ? min(S, (p + a.part_chunk - 1) / a.part_chunk) : 0;
        } else {
            if (wave == 0) {   // wave-uniform: the (m, l) pairs are wave 0's (Hq <= 32)
#pragma unroll
                for (int sp = 0; sp < MS; ++sp) mlv[sp] = a.part_ml[(long)hm * S + (sp < S ? sp : S - 1)];
            }
            ns = p >= 0 ? min(S, (p + 1 + a.part_chunk - 1) / a.part_chunk) : 0;
        }
    }
    // x and the gain into LDS by DMA (source indices clamped to the vectors; what
    // lands past K is never read)
    auto stage_x = [&]() {
        const uint32_t xl = lds_addr(xs);
        for (int j = wave; j < xpad / 256; j += 4) {
            const int f = min(j * 256 + lane * 4, K - 4);
            lds_dma16(a.x + f, __builtin_amdgcn_readfirstlane(xl + j * 1024));
        }
        if (a.gain) {
            constexpr int GE = 16 / (int)sizeof(GT);      // gain elements per lane
            const uint32_t gl = lds_addr(gs);
            for (int j = wave; j < gemv1_gpad(K, sizeof(GT)) / 1024; j += 4) {
                const int e = min(j * 64 * GE + lane * GE, K - GE);
                lds_dma16((const GT*)a.gain + e, __builtin_amdgcn_readfirstlane(gl + j * 1024));
            }
        }
    };
    // the weight loads each lane issues in the first issue() (its bias/residual/scale
    // loads, which the compiler may turn into scalar loads, are not counted): with
    // the vector first, waiting until no more than that many vector-memory operations
    // are outstanding means the vector's loads landed (they retire in issue order)
    constexpr int kLoadsAfterX = UR * NW * CPL;
    static_assert(kLoadsAfterX <= 63, "vmcnt range");
    const int tile0 = tile < ntiles ? tile : ntiles - 1;
    if constexpr (MS > 0 || LPR < 64) {
        if constexpr (MS == 0) stage_x();
        issue(tile0, kc0, true);   // unconditional: no join for the loads to wait at
        __builtin_amdgcn_s_waitcnt(wait_vm(kLoadsAfterX));   // this wave's vector loads / DMA landed
    } else {
        issue(tile0, kc0, true);
        stage_x();
        __builtin_amdgcn_s_waitcnt(wait_vm(0));              // this wave's weights and DMA landed
    }
    lds_barrier();                                           // ... and every wave's DMA
    // counters a later kernel of the step starts from zero
    if (a.zero_ptr && blockIdx.x == 0)
        for (int i = tid; i < a.zero_n; i += 256) a.zero_ptr[i] = 0u;

    if (MS > 0 && a.part_new) {
        // the same merge with the new token as one more split: score q . k_new
        // (summed over the hd/4 threads of the head, aligned groups within a wave),
        // weight sum 1, output v_new; every thread forms its own head's weights
        float dq = qn.x * kn.x + qn.y * kn.y + qn.z * kn.z + qn.w * kn.w;
        dq = a.part_hd == 64 ? group_sum<16>(dq) : group_sum<32>(dq);
        const float sn = dq * a.part_scale2;
        float M = sn;
#pragma unroll
        for (int sp = 0; sp < MS; ++sp) M = sp < ns ? fmaxf(M, mlv[sp].x) : M;
        const float wn = __builtin_amdgcn_exp2f(sn - M);
        float L = wn;
        float4 o = make_float4(vn.x * wn, vn.y * wn, vn.z * wn, vn.w * wn);
#pragma unroll
        for (int sp = 0; sp < MS; ++sp) {
            const float w = sp < ns ? __builtin_amdgcn_exp2f(mlv[sp].x - M) : 0.f;
            L = fmaf(mlv[sp].y, w, L);
            o.x = fmaf(ov[sp].x, w, o.x); o.y = fmaf(ov[sp].y, w, o.y);
            o.z = fmaf(ov[sp].z, w, o.z); o.w = fmaf(ov[sp].w, w, o.w);
        }
        const float rl = 1.0f / L;
        if (4 * tid < K) ((float4*)xs)[tid] = make_float4(o.x * rl, o.y * rl, o.z * rl, o.w * rl);
    } else if constexpr (MS > 0) {
        // merge of the splits (Tang page, section 2.2: the online-softmax monoid):
        // with M = max m_s over the valid splits (base-2 units), head h's context is
        // sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M)
        __shared__ float wgt[kG1MergeHeads][MS];
        const int hd = a.part_hd;
        if (tid < K / hd) {
            float M = -INFINITY;
#pragma unroll
            for (int sp = 0; sp < MS; ++sp) M = sp < ns ? fmaxf(M, mlv[sp].x) : M;
            float w[MS], L = 0.f;
#pragma unroll
            for (int sp = 0; sp < MS; ++sp) {
                w[sp] = sp < ns ? __builtin_amdgcn_exp2f(mlv[sp].x - M) : 0.f;
                L = fmaf(mlv[sp].y, w[sp], L);
            }
            const float rl = ns > 0 ? 1.0f / L : 0.f;
#pragma unroll
            for (int sp = 0; sp < MS; ++sp) wgt[tid][sp] = w[sp] * rl;
        }
        lds_barrier();
        if (4 * tid < K) {
            const int hh = 4 * tid / hd;
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int sp = 0; sp < MS; ++sp) {
                const float wv_ = wgt[hh][sp];
                o.x = fmaf(ov[sp].x, wv_, o.x); o.y = fmaf(ov[sp].y, wv_, o.y);
                o.z = fmaf(ov[sp].z, wv_, o.z); o.w = fmaf(ov[sp].w, wv_, o.w);
            }
            ((float4*)xs)[tid] = o;
        }
    }

    // x * g and sum(x^2) in place; the zero block behind x
    float ss = 0.f;
    if (a.gain) {
        for (int k4 = tid; k4 < K / 4; k4 += 256) {
            float4 v = ((const float4*)xs)[k4];
            float g[4];
            if (sizeof(GT) == 2) {
                const uint2 gb = ((const uint2*)gs)[k4];
                g[0] = __uint_as_float(gb.x << 16); g[1] = __uint_as_float(gb.x & 0xffff0000u);
                g[2] = __uint_as_float(gb.y << 16); g[3] = __uint_as_float(gb.y & 0xffff0000u);
            } else {
                const float4 gf = ((const float4*)gs)[k4];
                g[0] = gf.x; g[1] = gf.y; g[2] = gf.z; g[3] = gf.w;
            }
            ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
            v.x *= g[0]; v.y *= g[1]; v.z *= g[2]; v.w *= g[3];
            ((float4*)xs)[k4] = v;
        }
        ss = group_sum<kWave>(ss);
        if (lane == 0) wsum[wave] = ss;
    }
    if (tid < kG1Zeros) xs[xpad + tid] = 0.f;
    lds_barrier();
    const float rscale = a.gain ? 1.0f / sqrtf((wsum[0] + wsum[1] + wsum[2] + wsum[3]) / (float)K + a.eps) : 1.0f;

    float best_v = -INFINITY;
    int best_i = 0x7fffffff;
    for (; tile < ntiles; tile += gridDim.x) {
        float acc[UR][NW];
#pragma unroll
        for (int u = 0; u < UR; ++u)
#pragma unroll
            for (int n = 0; n < NW; ++n) acc[u][n] = 0.f;
        for (int cbase = kc0; cbase < kc1; cbase += CPL * LPR) {
            if (cbase != kc0) issue(tile, cbase, false);
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = cbase + li + j * LPR;
                const float* xp = xs + (c < kc1 ? c : cz) * CE;
                float xv[CE];
#pragma unroll
                for (int q = 0; q < CE / 4; ++q) {
                    const float4 t = ((const float4*)xp)[q];
                    xv[4 * q] = t.x; xv[4 * q + 1] = t.y; xv[4 * q + 2] = t.z; xv[4 * q + 3] = t.w;
                }
#pragma unroll
                for (int u = 0; u < UR; ++u)
#pragma unroll
                    for (int n = 0; n < NW; ++n) {
                        float wf[CE];
                        widen16(wv[u][n][j], wf);
#pragma unroll
                        for (int e = 0; e < CE; ++e) acc[u][n] = fmaf(wf[e], xv[e], acc[u][n]);
                    }
            }
        }
        float cur[UR], csc[UR], cs_[UR][NW];
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            cur[u] = pre[u]; csc[u] = psc[u];
#pragma unroll
            for (int n = 0; n < NW; ++n) cs_[u][n] = srow[u][n];
        }
        const int this_tile = tile;
        const int next = tile + gridDim.x;
        if (next < ntiles) issue(next, kc0, true);
#pragma unroll
        for (int u = 0; u < UR; ++u)
#pragma unroll
            for (int n = 0; n < NW; ++n) acc[u][n] = group_sum<LPR>(acc[u][n]);
        if (WK > 1) {
            if (li == 0) {
#pragma unroll
                for (int u = 0; u < UR; ++u)
#pragma unroll
                    for (int n = 0; n < NW; ++n) red[wk][(wr * UR + u) * RPW + slot][n] = acc[u][n];
            }
            lds_barrier();
#pragma unroll
            for (int u = 0; u < UR; ++u)
#pragma unroll
                for (int n = 0; n < NW; ++n) {
                    float v = 0.f;
#pragma unroll
                    for (int q = 0; q < WK; ++q) v += red[q][(wr * UR + u) * RPW + slot][n];
                    acc[u][n] = v;
                }
            lds_barrier();   // red is rewritten by the next tile
        }
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int r = this_tile * RPT + (wr * UR + u) * RPW + slot;
            const float v0 = I8 ? acc[u][0] * cs_[u][0] * rscale : acc[u][0] * rscale;
            float out;
            if (EPI == EPI_STORE || EPI == EPI_RESID) out = fmaf(cur[u], csc[u], v0);
            else if (EPI == EPI_SWIGLU)
                out = silu(v0) * (I8 ? acc[u][NW - 1] * cs_[u][NW - 1] * rscale : acc[u][NW - 1] * rscale);
            else out = v0;
            if (wk == 0 && li == 0 && r < N) {
                a.y[r] = out;
                if (EPI == EPI_LOGITS && better(v0, r, best_v, best_i)) { best_v = v0; best_i = r; }
            }
        }
    }
    if (EPI == EPI_LOGITS) {
        wave_argmax(best_v, best_i);
        if (lane == 0) { red_v[wave] = best_v; red_i[wave] = best_i; }
        __syncthreads();
        if (tid == 0) {
            for (int w = 1; w < 4; ++w)
                if (better(red_v[w], red_i[w], red_v[0], red_i[0])) { red_v[0] = red_v[w]; red_i[0] = red_i[w]; }
            a.part_val[blockIdx.x] = red_v[0];
            a.part_idx[blockIdx.x] = red_i[0];
        }
    }
}

// (LPR, WK, UR, CPL) shapes compiled; every one handles any K and N. RPT rows per
// workgroup tile = (4 / WK) * (64 / LPR) * UR; one pass over K covers
// CPL * LPR * WK 16-byte chunks (8 bf16 or 16 int8 columns each; more take
// further passes, each a memory round trip). The first G_NCFG serve float and
// bf16 rows; int8 rows, whose chunks hold twice the columns, take their own
// shapes sized to the 0.5B rows (56 chunks at K = 896, 304 at K = 4864) so that
// few lanes idle.
struct Gemv1Shape { int lpr, wk, ur, cpl; };
enum Gemv1Cfg { G_SMALLK_FEWROWS = 0, G_SMALLK = 1, G_SMALLK_UR2 = 2, G_BIGK_FEWROWS = 3, G_BIGK = 4,
                G_BIGK_UR2 = 5, G_SMALLK_8 = 6, G_LONGK_4 = 7, G_NCFG = 8,
                G_I8_WIDE = 8, G_I8_NARROW = 9, G_I8_LONGK = 10, G_I8_MID = 11, G_I8_MID2 = 12, G_NALL = 13 };
constexpr Gemv1Shape kGemv1Shapes[G_NALL] = {
    {16, 4, 1, 2}, {16, 1, 1, 8}, {16, 1, 2, 8}, {32, 4, 1, 6}, {64, 1, 1, 8}, {64, 1, 2, 8}, {16, 2, 1, 4},
    {16, 4, 1, 10},
    {8, 1, 2, 7}, {8, 4, 1, 2}, {16, 4, 1, 5}, {8, 1, 1, 7}, {16, 1, 2, 4}};
constexpr int gemv1_rpt(int c) { return (4 / kGemv1Shapes[c].wk) * (64 / kGemv1Shapes[c].lpr) * kGemv1Shapes[c].ur; }
// columns one pass covers, for CE weight elements per 16-byte chunk
constexpr int gemv1_kpass(int c, int ce = 8) { return kGemv1Shapes[c].cpl * kGemv1Shapes[c].lpr * kGemv1Shapes[c].wk * ce; }

template <typename WT, int EPI, int MS = 0>
static hipError_t gemv1_dispatch(const GemvArgs& a, int cfg, int* grid_out, int grid_cap, hipStream_t s) {
    using GT = typename GainT<WT>::type;
    const size_t shm = (size_t)(gemv1_xpad(a.K) + kG1Zeros) * sizeof(float) + (a.gain ? gemv1_gpad(a.K, sizeof(GT)) : 0);
    auto go = [&](auto kern, int rpt) {
        if (shm > 65536 && hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm) != hipSuccess)
            return hipErrorInvalidValue;
        const int tiles = (a.N + rpt - 1) / rpt;
        const int grid = tiles < grid_cap ? tiles : grid_cap;
        if (grid_out) *grid_out = grid;
        hipLaunchKernelGGL(kern, dim3(grid), dim3(256), shm, s, a);
        return hipGetLastError();
    };
#define QD_G1C(C) \
    case C: return go(gemv1_kernel<WT, kGemv1Shapes[C].lpr, kGemv1Shapes[C].wk, kGemv1Shapes[C].ur, kGemv1Shapes[C].cpl, EPI, MS>, gemv1_rpt(C));
    if constexpr (sizeof(WT) == 1) {
        if constexpr (MS > 0) {
            switch (cfg) {
                QD_G1C(G_I8_NARROW)
                default: return hipErrorInvalidValue;
            }
        } else {
            switch (cfg) {
                QD_G1C(G_I8_WIDE) QD_G1C(G_I8_NARROW) QD_G1C(G_I8_LONGK) QD_G1C(G_I8_MID) QD_G1C(G_I8_MID2)
                default: return hipErrorInvalidValue;
            }
        }
    } else if constexpr (MS > 0) {
        switch (cfg) {
            QD_G1C(G_SMALLK_FEWROWS) QD_G1C(G_SMALLK)
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (cfg) {
            QD_G1C(G_SMALLK_FEWROWS) QD_G1C(G_SMALLK) QD_G1C(G_SMALLK_UR2) QD_G1C(G_BIGK_FEWROWS) QD_G1C(G_BIGK)
            QD_G1C(G_SMALLK_8) QD_G1C(G_LONGK_4)
            default: return go(gemv1_kernel<WT, 64, 1, 2, 8, EPI>, gemv1_rpt(G_BIGK_UR2));
        }
    }
#undef QD_G1C
}

// Shape choice. A batch-1 projection is about one memory round trip plus the
// transfer, so a second partial round of workgroups on the 256 CUs nearly
// doubles it: among the shapes that cover K in one pass, take the smallest
// row tile whose tiles fit one round (spreading the matrix over as many CUs as
// possible); a matrix too tall for that takes the largest such tile and a
// capped, grid-strided grid; a K no shape covers in one pass keeps the old
// rule (largest tile with at least 256 workgroups). The lm_head keeps its
// grid-strided wide tile. A bf16/float gate|up product counts a round as 1024
// workgroups (four per CU fit): at the 0.5B shape its 608 eight-row tiles beat
// 152 32-row ones by about 0.8 us (measured; other products and int8 gain nothing).
static int gemv1_pick(int N, int K, int epi, int ce) {
    const bool small_k = K <= 2048, i8 = ce == 16;
    const int round = (epi == EPI_SWIGLU && !i8) ? 4 * kCus : kCus;
    if (epi == EPI_LOGITS) return i8 ? (K <= gemv1_kpass(G_I8_WIDE, ce) ? G_I8_WIDE : G_I8_LONGK)
                                     : (small_k ? G_SMALLK_UR2 : G_BIGK_UR2);
    int best = -1, widest = -1;
    for (int c = i8 ? G_NCFG : 0; c < (i8 ? G_NALL : G_NCFG); ++c) {
        if (gemv1_kpass(c, ce) < K) continue;
        const int tiles = (N + gemv1_rpt(c) - 1) / gemv1_rpt(c);
        // ties on the row tile go to the shape with the least idle lanes (smallest pass)
        if (tiles <= round && (best < 0 || gemv1_rpt(c) < gemv1_rpt(best) ||
                              (gemv1_rpt(c) == gemv1_rpt(best) && gemv1_kpass(c, ce) < gemv1_kpass(best, ce))))
            best = c;
        if (widest < 0 || gemv1_rpt(c) > gemv1_rpt(widest) ||
            (gemv1_rpt(c) == gemv1_rpt(widest) && gemv1_kpass(c, ce) < gemv1_kpass(widest, ce)))
            widest = c;
    }
    if (best >= 0) return best;
    if (widest >= 0 || i8) return i8 && widest < 0 ? G_I8_LONGK : widest;
    const int cfgs_big[3] = {G_BIGK_UR2, G_BIGK, G_BIGK_FEWROWS};
    for (int i = 0; i < 3; ++i)
        if ((N + gemv1_rpt(cfgs_big[i]) - 1) / gemv1_rpt(cfgs_big[i]) >= kCus) return cfgs_big[i];
    return G_BIGK_FEWROWS;
}

int gemv1_merge_max_splits() { return 16; }

hipError_t launch_gemv1(const GemvArgs& a, int w_type, int epi, int grid_cap, int* grid_out, hipStream_t s) {
    // w_type: 0 float, 1 bf16, 2 int8 (with a.wscale); the picker counts bf16-sized
    // chunks for float and bf16, 16-element ones for int8
    if (w_type == 2 && (a.K % 16 || !a.wscale[0])) return hipErrorInvalidValue;
    const int cfg = gemv1_pick(a.N, a.K, epi, w_type == 2 ? 16 : 8);
    if (a.part) {   // residual product over the merged attention context
        if (epi != EPI_RESID || a.gain || a.part_hd % 4 || a.K % a.part_hd || a.K > 1024 ||
            a.K / a.part_hd > kG1MergeHeads || a.part_S < 1 || a.part_S > 16 || a.part_chunk < 1)
            return hipErrorInvalidValue;
        if (a.part_new && ((a.part_hd != 64 && a.part_hd != 128) || a.part_kv_heads < 1 ||
                           (a.K / a.part_hd) % a.part_kv_heads))
            return hipErrorInvalidValue;
        // one shape (it covers K <= 1024 in one pass); MS = the smallest of 2, 4, 8, 16 >= S
        const int mc = w_type == 2 ? (int)G_I8_NARROW : QD_B1_OCFG;
#define QD_G1M(WT)                                                                                      \
        if (a.part_S <= 2) return gemv1_dispatch<WT, EPI_RESID, 2>(a, mc, grid_out, grid_cap, s);      \
        if (a.part_S <= 4) return gemv1_dispatch<WT, EPI_RESID, 4>(a, mc, grid_out, grid_cap, s);      \
        if (a.part_S <= 8) return gemv1_dispatch<WT, EPI_RESID, 8>(a, mc, grid_out, grid_cap, s);      \
        return gemv1_dispatch<WT, EPI_RESID, 16>(a, mc, grid_out, grid_cap, s);
        if (w_type == 2) { QD_G1M(int8_t) } else if (w_type == 1) { QD_G1M(uint16_t) } else { QD_G1M(float) }
#undef QD_G1M
    }
#define QD_G1(WT)                                                                                 \
    switch (epi) {                                                                                \
        case EPI_STORE: return gemv1_dispatch<WT, EPI_STORE>(a, cfg, grid_out, grid_cap, s);      \
        case EPI_RESID: return gemv1_dispatch<WT, EPI_RESID>(a, cfg, grid_out, grid_cap, s);      \
        case EPI_SWIGLU: return gemv1_dispatch<WT, EPI_SWIGLU>(a, cfg, grid_out, grid_cap, s);    \
        default: return gemv1_dispatch<WT, EPI_LOGITS>(a, cfg, grid_out, grid_cap, s);            \
    }
    if (w_type == 2) { QD_G1(int8_t) } else if (w_type == 1) { QD_G1(uint16_t) } else { QD_G1(float) }
#undef QD_G1
}


// ---------------------------------------------------------------------------
// Batch-1 residual product by head slices, for contexts too wide for one
// workgroup to merge (Hq * hd > 1024) and split over several attention
// workgroups. Workgroup (query head h, block of R output rows):
//   1. loads head h's split partials (o_s, and the (m_s, l_s) pairs in base-2
//      units), then its R rows' slice of W (columns h*hd .. h*hd+hd-1), so the
//      merge below runs under the weights' latency;
//   2. merges the valid splits (Tang page, section 2.2: the online-softmax
//      monoid): ctx_h = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M), with M the
//      largest m_s, in a fixed order;
//   3. adds W[r, h-slice] . ctx_h into y[r] with a float atomic: y holds the
//      residual, and the Hq head slices of each row meet there (their order of
//      addition varies from run to run).
// One 16-byte chunk per lane per row (hd/8 lanes per row slice), kOhLoads rows
// per lane: R = 4 * (64 / (hd/8)) * kOhLoads rows per workgroup. Workgroups of
// one head are 8 ids apart when Hq is a multiple of 8, so they share an XCD and
// read the head's partials through one L2.
#ifndef QD_OH_LOADS
#define QD_OH_LOADS 8
#endif
constexpr int kOhLoads = QD_OH_LOADS;
constexpr int kOhMaxSplits = 64;
__host__ __device__ constexpr int oproj_heads_rows(int hd) { return 4 * (64 / (hd / 8)) * kOhLoads; }

template <int HD, int MS>
__global__ __launch_bounds__(256) void oproj_heads_kernel(GemvArgs a) {
    constexpr int LPR = HD / 8;                    // lanes per row slice
    constexpr int RPI = 4 * (kWave / LPR);         // rows per workgroup load
    constexpr int R = RPI * kOhLoads;
    constexpr int Q4 = HD / 4;                     // float4s per split's context row
    constexpr int NG = 256 / Q4;                   // split groups of threads
    constexpr int MSL = (MS + NG - 1) / NG;        // partial loads per thread (MS >= part_S)
    __shared__ float wgt[kOhMaxSplits];
    __shared__ float4 red[NG][Q4];
    __shared__ float4 ctx4[Q4];

    const int N = a.N, K = a.K, Hq = K / HD, NB = (N + R - 1) / R, S = a.part_S;
    const int id = blockIdx.x;
    int h, rb;
    if ((Hq & 7) == 0) { const int k = id >> 3; h = (k / NB) * 8 + (id & 7); rb = k - (k / NB) * NB; }
    else { h = id / NB; rb = id - h * NB; }
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    // the position as a scalar load (a vector load issued here would return after
    // the weights, and the merge would wait for them)
    const int p = *(const __attribute__((address_space(4))) int*)a.part_pos;

    // partials first (indices clamped to valid splits; the invalid are weighted 0)
    const int q4 = tid % Q4, grp = tid / Q4;
    const float* pb = a.part + (long)h * S * HD + 4 * q4;
    float4 ov[MSL];
#pragma unroll
    for (int u = 0; u < MSL; ++u) {
        const int j = grp + u * NG;
        ov[u] = *(const float4*)(pb + (long)(j < S ? j : S - 1) * HD);
    }
    const float2 ml = a.part_ml[(long)h * S + (lane < S ? lane : S - 1)];
    asm volatile("" ::: "memory");
    gbyte* wb = sgpr_gptr(a.w[0]) + (long)h * HD * 2 + (lane % LPR) * 16;
    const int row0 = rb * R + wave * (kWave / LPR) + lane / LPR;
    uint4 wv[kOhLoads];
#pragma unroll
    for (int i = 0; i < kOhLoads; ++i) {
        const int r = row0 + i * RPI;
        wv[i] = gld16(wb + (long)(r < N ? r : N - 1) * K * 2);
    }
    asm volatile("" ::: "memory");

    const int ns = p >= 0 ? min(S, (p + a.part_chunk) / a.part_chunk) : 0;
    if (wave == 0) {   // the splits' weights, 1/L folded in
        const float mj = lane < ns ? ml.x : -INFINITY;
        const float m = group_max<kWave>(mj);
        const float w = lane < ns ? __builtin_amdgcn_exp2f(mj - m) : 0.f;
        const float l = group_sum<kWave>((lane < ns ? ml.y : 0.f) * w);
        wgt[lane] = ns > 0 ? w / l : 0.f;
    }
    lds_barrier();
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < MSL; ++u) {
        const int j = grp + u * NG;
        const float wj = j < ns ? wgt[j < kOhMaxSplits ? j : 0] : 0.f;
        o.x = fmaf(ov[u].x, wj, o.x); o.y = fmaf(ov[u].y, wj, o.y);
        o.z = fmaf(ov[u].z, wj, o.z); o.w = fmaf(ov[u].w, wj, o.w);
    }
    red[grp][q4] = o;
    lds_barrier();
    if (tid < Q4) {
        float4 t = red[0][tid];
#pragma unroll
        for (int g = 1; g < NG; ++g) {
            const float4 v = red[g][tid];
            t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w;
        }
        ctx4[tid] = t;
    }
    lds_barrier();
    const int li = lane % LPR;
    const float4 c0 = ctx4[2 * li], c1 = ctx4[2 * li + 1];
    const float cx[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
    for (int i = 0; i < kOhLoads; ++i) {
        float wf[8];
        widen16(wv[i], wf);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(wf[e], cx[e], acc);
        acc = group_sum<LPR>(acc);
        const int r = row0 + i * RPI;
        if (li == 0 && r < N && ns > 0) unsafeAtomicAdd(a.y + r, acc);
    }
}

hipError_t launch_oproj_heads(const GemvArgs& a, hipStream_t s) {
    const int hd = a.part_hd;
    if ((hd != 64 && hd != 128) || !a.part || !a.part_ml || !a.part_pos || !a.w[0] || !a.y || a.gain ||
        a.part_S < 1 || a.part_S > kOhMaxSplits || a.part_chunk < 1 || a.N < 1 || a.K < hd || a.K % hd ||
        a.B != 1)
        return hipErrorInvalidValue;
    const int R = oproj_heads_rows(hd), nb = (a.N + R - 1) / R;
    const dim3 grid((a.K / hd) * nb), block(256);
#define QD_OH(HD)                                                                                              \
    if (a.part_S <= 16) hipLaunchKernelGGL((oproj_heads_kernel<HD, 16>), grid, block, 0, s, a);                \
    else if (a.part_S <= 32) hipLaunchKernelGGL((oproj_heads_kernel<HD, 32>), grid, block, 0, s, a);           \
    else hipLaunchKernelGGL((oproj_heads_kernel<HD, 64>), grid, block, 0, s, a);
    if (hd == 64) { QD_OH(64) } else { QD_OH(128) }
#undef QD_OH
    return hipGetLastError();
}

}  // namespace qd
