// Single-row (batch 1) GEMV for gfx950, tuned for latency.
//
// A decode-step projection is an HBM stream of a row-major [N][K] weight
// matrix against one activation vector; at 0.5B shapes a whole matrix is only
// one or two memory latencies' worth of data, so each lane issues every weight
// load it will need before it touches the activation, and the activation is
// staged into LDS in a single pass.
//
// RMSNorm is folded into the product (Tang page, section 2.3, epilogues on the
// reducing thread): W (x * r * g) = r * (W (x * g)) with r = 1/sqrt(sum(x^2)/K + eps)
// (nanocompile page, phase 1: the mean square is a sum then a divide; eps
// inside the root), so the staging pass stores x * g and accumulates sum(x^2)
// at the same time, and r scales the finished dot product.
//
// Layout of one workgroup (256 threads = 4 waves): LPR lanes share a row and
// read 16-byte chunks lane-interleaved (each wave load covers 64/LPR rows of
// LPR*16 contiguous bytes); WK waves split K and meet in LDS; UR row groups
// per lane; CPL chunks per lane per row per pass.
#include "qd_device.h"
#include "qd_launch.h"

namespace qd {

constexpr int kCus = 256;

template <typename WT, int LPR, int WK, int UR, int CPL, int EPI>
__global__ __launch_bounds__(256) void gemv1_kernel(GemvArgs a) {
    constexpr int CE = VecN<WT>::n;
    constexpr int RPW = kWave / LPR;
    constexpr int WR = 4 / WK;
    constexpr int RPT = WR * RPW * UR;
    constexpr int NW = (EPI == EPI_SWIGLU) ? 2 : 1;
    extern __shared__ float xs[];
    __shared__ float wsum[4];
    __shared__ float red[WK][RPT][NW];
    __shared__ float red_v[4];
    __shared__ int red_i[4];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int wr = wave % WR, wk = wave / WR;
    const int li = lane % LPR, slot = lane / LPR;
    const int K = a.K, N = a.N, KC = K / CE;
    const int kcw = (KC + WK - 1) / WK;
    const int kc0 = wk * kcw, kc1 = min(KC, kc0 + kcw);
    const int ntiles = (N + RPT - 1) / RPT;

    auto wptr = [&](int r, int n) -> const WT* {
        if (EPI == EPI_SWIGLU) return (const WT*)a.w[n] + (long)r * K;
        const bool s0 = r < a.seg_end[0], s1 = r < a.seg_end[1];
        const void* w = s0 ? a.w[0] : (s1 ? a.w[1] : a.w[2]);
        const int base = s0 ? 0 : (s1 ? a.seg_end[0] : a.seg_end[1]);
        return (const WT*)w + (long)(r - base) * K;
    };
    uint4 wv[UR][NW][CPL];
    auto issue = [&](int tile, int cbase) {
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int r = tile * RPT + (wr * UR + u) * RPW + slot;
#pragma unroll
            for (int n = 0; n < NW; ++n) {
                const WT* wp = r < N ? wptr(r, n) : nullptr;
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    const int c = cbase + li + j * LPR;
                    wv[u][n][j] = (wp && c < kc1) ? *(const uint4*)(wp + c * CE) : make_uint4(0, 0, 0, 0);
                }
            }
        }
    };
    int tile = blockIdx.x;
    if (tile < ntiles) issue(tile, kc0);

    // counters a later kernel of the step starts from zero
    if (a.zero_ptr && blockIdx.x == 0)
        for (int i = tid; i < a.zero_n; i += 256) a.zero_ptr[i] = 0u;

    // stage x * g (or x) and sum(x^2)
    float ss = 0.f;
    for (int k4 = tid; k4 < K / 4; k4 += 256) {
        float4 v = ((const float4*)a.x)[k4];
        if (a.gain) {
            ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
            const int k = 4 * k4;
            v.x *= load_scalar<WT>(a.gain, k);
            v.y *= load_scalar<WT>(a.gain, k + 1);
            v.z *= load_scalar<WT>(a.gain, k + 2);
            v.w *= load_scalar<WT>(a.gain, k + 3);
        }
        ((float4*)xs)[k4] = v;
    }
    if (a.gain) {
        ss = group_sum<kWave>(ss);
        if (lane == 0) wsum[wave] = ss;
    }
    __syncthreads();
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
            if (cbase != kc0) issue(tile, cbase);
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = cbase + li + j * LPR;
                if (c >= kc1) break;
                float xv[CE];
#pragma unroll
                for (int q = 0; q < CE / 4; ++q) {
                    const float4 t = ((const float4*)(xs + c * CE))[q];
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
        const int next = tile + gridDim.x;
        if (next < ntiles) issue(next, kc0);
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
            __syncthreads();
            if (wk == 0 && li == 0) {
#pragma unroll
                for (int u = 0; u < UR; ++u)
#pragma unroll
                    for (int n = 0; n < NW; ++n) {
                        float v = 0.f;
#pragma unroll
                        for (int q = 0; q < WK; ++q) v += red[q][(wr * UR + u) * RPW + slot][n];
                        acc[u][n] = v;
                    }
            }
            __syncthreads();
        }
        if (wk == 0 && li == 0) {
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int r = tile * RPT + (wr * UR + u) * RPW + slot;
                if (r >= N) continue;
                float* yp = a.y + r;
                const float v0 = acc[u][0] * rscale;
                if (EPI == EPI_STORE) {
                    const bool s0 = r < a.seg_end[0], s1 = r < a.seg_end[1];
                    const void* bsel = s0 ? a.bias[0] : (s1 ? a.bias[1] : a.bias[2]);
                    const int base = s0 ? 0 : (s1 ? a.seg_end[0] : a.seg_end[1]);
                    *yp = bsel ? v0 + load_scalar<WT>(bsel, r - base) : v0;
                } else if (EPI == EPI_RESID) {
                    *yp = *yp + v0;
                } else if (EPI == EPI_SWIGLU) {
                    *yp = silu(v0) * (acc[u][NW - 1] * rscale);
                } else {
                    *yp = v0;
                    if (better(v0, r, best_v, best_i)) { best_v = v0; best_i = r; }
                }
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
// CPL * LPR * WK * 8 columns (more take further passes, each a memory round trip).
struct Gemv1Shape { int lpr, wk, ur, cpl; };
enum Gemv1Cfg { G_SMALLK_FEWROWS = 0, G_SMALLK = 1, G_SMALLK_UR2 = 2, G_BIGK_FEWROWS = 3, G_BIGK = 4,
                G_BIGK_UR2 = 5, G_SMALLK_8 = 6, G_LONGK_4 = 7, G_NCFG = 8 };
constexpr Gemv1Shape kGemv1Shapes[G_NCFG] = {
    {16, 4, 1, 2}, {16, 1, 1, 8}, {16, 1, 2, 8}, {32, 4, 1, 6}, {64, 1, 1, 8}, {64, 1, 2, 8}, {16, 2, 1, 4},
    {16, 4, 1, 10}};
constexpr int gemv1_rpt(int c) { return (4 / kGemv1Shapes[c].wk) * (64 / kGemv1Shapes[c].lpr) * kGemv1Shapes[c].ur; }
constexpr int gemv1_kpass(int c) { return kGemv1Shapes[c].cpl * kGemv1Shapes[c].lpr * kGemv1Shapes[c].wk * 8; }

template <typename WT, int EPI>
static hipError_t gemv1_dispatch(const GemvArgs& a, int cfg, int* grid_out, int grid_cap, hipStream_t s) {
    const size_t shm = (size_t)a.K * sizeof(float);
    auto go = [&](auto kern, int rpt) {
        const int tiles = (a.N + rpt - 1) / rpt;
        const int grid = tiles < grid_cap ? tiles : grid_cap;
        if (grid_out) *grid_out = grid;
        hipLaunchKernelGGL(kern, dim3(grid), dim3(256), shm, s, a);
        return hipGetLastError();
    };
#define QD_G1C(C) \
    case C: return go(gemv1_kernel<WT, kGemv1Shapes[C].lpr, kGemv1Shapes[C].wk, kGemv1Shapes[C].ur, kGemv1Shapes[C].cpl, EPI>, gemv1_rpt(C));
    switch (cfg) {
        QD_G1C(G_SMALLK_FEWROWS) QD_G1C(G_SMALLK) QD_G1C(G_SMALLK_UR2) QD_G1C(G_BIGK_FEWROWS) QD_G1C(G_BIGK)
        QD_G1C(G_SMALLK_8) QD_G1C(G_LONGK_4)
        default: return go(gemv1_kernel<WT, 64, 1, 2, 8, EPI>, gemv1_rpt(G_BIGK_UR2));
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
// grid-strided wide tile.
static int gemv1_pick(int N, int K, int epi) {
    const bool small_k = K <= 2048;
    if (epi == EPI_LOGITS) return small_k ? G_SMALLK_UR2 : G_BIGK_UR2;
    int best = -1, widest = -1;
    for (int c = 0; c < G_NCFG; ++c) {
        if (gemv1_kpass(c) < K) continue;
        const int tiles = (N + gemv1_rpt(c) - 1) / gemv1_rpt(c);
        // ties on the row tile go to the shape with the least idle lanes (smallest pass)
        if (tiles <= kCus && (best < 0 || gemv1_rpt(c) < gemv1_rpt(best) ||
                              (gemv1_rpt(c) == gemv1_rpt(best) && gemv1_kpass(c) < gemv1_kpass(best))))
            best = c;
        if (widest < 0 || gemv1_rpt(c) > gemv1_rpt(widest) ||
            (gemv1_rpt(c) == gemv1_rpt(widest) && gemv1_kpass(c) < gemv1_kpass(widest)))
            widest = c;
    }
    if (best >= 0) return best;
    if (widest >= 0) return widest;
    const int cfgs_big[3] = {G_BIGK_UR2, G_BIGK, G_BIGK_FEWROWS};
    for (int i = 0; i < 3; ++i)
        if ((N + gemv1_rpt(cfgs_big[i]) - 1) / gemv1_rpt(cfgs_big[i]) >= kCus) return cfgs_big[i];
    return G_BIGK_FEWROWS;
}

hipError_t launch_gemv1(const GemvArgs& a, int w_is_bf16, int epi, int grid_cap, int* grid_out, hipStream_t s) {
    const int cfg = gemv1_pick(a.N, a.K, epi);
#define QD_G1(WT)                                                                                 \
    switch (epi) {                                                                                \
        case EPI_STORE: return gemv1_dispatch<WT, EPI_STORE>(a, cfg, grid_out, grid_cap, s);      \
        case EPI_RESID: return gemv1_dispatch<WT, EPI_RESID>(a, cfg, grid_out, grid_cap, s);      \
        case EPI_SWIGLU: return gemv1_dispatch<WT, EPI_SWIGLU>(a, cfg, grid_out, grid_cap, s);    \
        default: return gemv1_dispatch<WT, EPI_LOGITS>(a, cfg, grid_out, grid_cap, s);            \
    }
    if (w_is_bf16) { QD_G1(uint16_t) } else { QD_G1(float) }
#undef QD_G1
}

}  // namespace qd
