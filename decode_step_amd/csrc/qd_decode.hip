// Decode-step kernels for gfx950 (CDNA4, 64-lane wavefronts).
//
// Decode at batch 1..16 is HBM-bound: every weight is read once per step and
// used for B fused multiply-adds. The GEMV streams row-major [out][in] weights
// with 16-byte loads, LPR lanes sharing one row so each wave load covers
// 64/LPR rows x LPR*16 contiguous bytes. The activation (with its RMSNorm
// applied) sits in LDS; each lane's partial dot products are combined with
// cross-lane shuffles, and the bias / residual / SwiGLU / argmax epilogue runs
// on the lane holding the total (Tang page, section 2.3: epilogues on the
// reducing thread; gate|up as one sibling reduction reading the normed input
// once). Rows are float, bf16 or int8 codes with one float scale per row
// (nanoinfer page, phase 6: per-row symmetric weight-only int8), the scale
// applied to the finished dot product; gains and biases of int8 models are bf16.
#include "qd_device.h"
#include "qd_launch.h"

namespace qd {

constexpr int kGemvThreads = 256;
constexpr int kGemvUR = 2;     // row groups in flight per lane
constexpr int kGemvJB = 4;     // 16-byte chunks loaded per lane before use

template <int LPR>
constexpr int rows_per_tile() { return 4 * (kWave / LPR) * kGemvUR; }

int gemv_rows_per_tile(int K) { return K <= 2048 ? rows_per_tile<16>() : rows_per_tile<64>(); }

template <typename WT, int LPR, int BM, int EPI>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(GemvArgs a) {
    constexpr int CE = VecN<WT>::n;
    using GT = typename GainT<WT>::type;      // gains and biases
    constexpr bool I8 = sizeof(WT) == 1;
    constexpr int RPW = kWave / LPR;
    constexpr int UR = kGemvUR;
    constexpr int RPT = 4 * RPW * UR;
    constexpr int NW = (EPI == EPI_SWIGLU) ? 2 : 1;
    extern __shared__ float xs[];          // [B][kt] staged activation
    __shared__ float rscale[16];
    __shared__ float red_v[4][16];
    __shared__ int red_i[4][16];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int li = lane % LPR, slot = lane / LPR;
    const int B = a.B, K = a.K, N = a.N, kt_max = a.kt;
    if (a.zero_ptr && blockIdx.x == 0)
        for (int i = tid; i < a.zero_n; i += kGemvThreads) a.zero_ptr[i] = 0u;

    if (a.gain) {   // RMSNorm scale of each batch row over the whole K
        for (int b = wave; b < B; b += 4) {
            float s = 0.f;
            for (int k = lane; k < K; k += kWave) { float v = a.x[(long)b * K + k]; s += v * v; }
            s = group_sum<kWave>(s);
            if (lane == 0) rscale[b] = 1.0f / sqrtf(s / (float)K + a.eps);
        }
        __syncthreads();
    }
    auto stage = [&](int k0, int kt) {
        for (int idx = tid; idx < B * kt; idx += kGemvThreads) {
            int b = idx / kt, k = idx - b * kt;
            float v = a.x[(long)b * K + k0 + k];
            if (a.gain) v = v * rscale[b] * load_scalar<GT>(a.gain, k0 + k);
            xs[b * kt + k] = v;
        }
    };
    const bool one_pass = kt_max >= K;
    if (one_pass) { stage(0, K); __syncthreads(); }

    float best_v[BM];
    int best_i[BM];
#pragma unroll
    for (int b = 0; b < BM; ++b) { best_v[b] = -INFINITY; best_i[b] = 0x7fffffff; }

    const int ntiles = (N + RPT - 1) / RPT;
    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        float acc[UR][NW][BM];
        const WT* wp[UR][NW];
        int rows[UR];
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            rows[u] = tile * RPT + (wave * UR + u) * RPW + slot;
            const int r = rows[u];
#pragma unroll
            for (int n = 0; n < NW; ++n) {
                wp[u][n] = nullptr;
#pragma unroll
                for (int b = 0; b < BM; ++b) acc[u][n][b] = 0.f;
            }
            if (r < N) {
                if (EPI == EPI_SWIGLU) {
                    wp[u][0] = (const WT*)a.w[0] + (long)r * K;
                    wp[u][NW - 1] = (const WT*)a.w[1] + (long)r * K;
                } else {
                    const bool s0 = r < a.seg_end[0], s1 = r < a.seg_end[1];
                    const void* wsel = s0 ? a.w[0] : (s1 ? a.w[1] : a.w[2]);
                    const int base = s0 ? 0 : (s1 ? a.seg_end[0] : a.seg_end[1]);
                    wp[u][0] = (const WT*)wsel + (long)(r - base) * K;
                }
            }
        }
        for (int k0 = 0; k0 < K; k0 += kt_max) {
            const int kt = min(kt_max, K - k0);
            if (!one_pass) { __syncthreads(); stage(k0, kt); __syncthreads(); }
            const int nck = kt / CE;
            for (int c0 = 0; c0 < nck; c0 += LPR * kGemvJB) {
                uint4 wv[UR][NW][kGemvJB];
#pragma unroll
                for (int u = 0; u < UR; ++u)
#pragma unroll
                    for (int n = 0; n < NW; ++n)
#pragma unroll
                        for (int j = 0; j < kGemvJB; ++j) {
                            const int c = c0 + li + j * LPR;
                            if (wp[u][n] && c < nck)
                                wv[u][n][j] = *(const uint4*)(wp[u][n] + k0 + c * CE);
                            else
                                wv[u][n][j] = make_uint4(0, 0, 0, 0);
                        }
#pragma unroll
                for (int j = 0; j < kGemvJB; ++j) {
                    const int c = c0 + li + j * LPR;
                    if (c >= nck) break;
                    float wf[UR][NW][CE];
#pragma unroll
                    for (int u = 0; u < UR; ++u)
#pragma unroll
                        for (int n = 0; n < NW; ++n) widen16(wv[u][n][j], wf[u][n]);
#pragma unroll
                    for (int b = 0; b < BM; ++b) {
                        if (b >= B) break;
                        float xv[CE];
                        const float4* xp = (const float4*)(xs + b * kt + c * CE);
#pragma unroll
                        for (int q = 0; q < CE / 4; ++q) {
                            float4 t = xp[q];
                            xv[4 * q] = t.x; xv[4 * q + 1] = t.y; xv[4 * q + 2] = t.z; xv[4 * q + 3] = t.w;
                        }
#pragma unroll
                        for (int u = 0; u < UR; ++u)
#pragma unroll
                            for (int n = 0; n < NW; ++n)
#pragma unroll
                                for (int e = 0; e < CE; ++e)
                                    acc[u][n][b] = fmaf(wf[u][n][e], xv[e], acc[u][n][b]);
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < UR; ++u)
#pragma unroll
            for (int n = 0; n < NW; ++n)
#pragma unroll
                for (int b = 0; b < BM; ++b) acc[u][n][b] = group_sum<LPR>(acc[u][n][b]);

        if (li == 0) {
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int r = rows[u];
                if (r >= N) continue;
                float bias = 0.f, sc0 = 1.f, sc1 = 1.f;   // int8: the rows' scales
                {
                    const bool s0 = r < a.seg_end[0], s1 = r < a.seg_end[1];
                    const int base = s0 ? 0 : (s1 ? a.seg_end[0] : a.seg_end[1]);
                    if (EPI == EPI_STORE) {
                        const void* bsel = s0 ? a.bias[0] : (s1 ? a.bias[1] : a.bias[2]);
                        if (bsel) bias = load_scalar<GT>(bsel, r - base);
                    }
                    if (I8) {
                        if (EPI == EPI_SWIGLU) { sc0 = a.wscale[0][r]; sc1 = a.wscale[1][r]; }
                        else sc0 = (s0 ? a.wscale[0] : (s1 ? a.wscale[1] : a.wscale[2]))[r - base];
                    }
                }
#pragma unroll
                for (int b = 0; b < BM; ++b) {
                    if (b >= B) break;
                    float* yp = a.y + (long)b * N + r;
                    const float v0 = I8 ? acc[u][0][b] * sc0 : acc[u][0][b];
                    if (EPI == EPI_STORE) *yp = v0 + bias;
                    else if (EPI == EPI_RESID) *yp = *yp + v0;
                    else if (EPI == EPI_SWIGLU) *yp = silu(v0) * (I8 ? acc[u][NW - 1][b] * sc1 : acc[u][NW - 1][b]);
                    else {
                        *yp = v0;
                        if (better(v0, r, best_v[b], best_i[b])) {
                            best_v[b] = v0;
                            best_i[b] = r;
                        }
                    }
                }
            }
        }
    }
    if (EPI == EPI_LOGITS) {
#pragma unroll
        for (int b = 0; b < BM; ++b) {
            if (b >= B) break;
            float v = best_v[b];
            int i = best_i[b];
            wave_argmax(v, i);
            if (lane == 0) { red_v[wave][b] = v; red_i[wave][b] = i; }
        }
        __syncthreads();
        if (tid < B) {
            float v = red_v[0][tid];
            int i = red_i[0][tid];
            for (int w = 1; w < 4; ++w)
                if (better(red_v[w][tid], red_i[w][tid], v, i)) { v = red_v[w][tid]; i = red_i[w][tid]; }
            a.part_val[tid * gridDim.x + blockIdx.x] = v;
            a.part_idx[tid * gridDim.x + blockIdx.x] = i;
        }
    }
}

template <typename WT, int LPR, int BM>
static hipError_t gemv_dispatch_epi(const GemvArgs& a, int epi, int grid, size_t shm, hipStream_t s) {
    switch (epi) {
        case EPI_STORE: hipLaunchKernelGGL((gemv_kernel<WT, LPR, BM, EPI_STORE>), dim3(grid), dim3(kGemvThreads), shm, s, a); break;
        case EPI_RESID: hipLaunchKernelGGL((gemv_kernel<WT, LPR, BM, EPI_RESID>), dim3(grid), dim3(kGemvThreads), shm, s, a); break;
        case EPI_SWIGLU: hipLaunchKernelGGL((gemv_kernel<WT, LPR, BM, EPI_SWIGLU>), dim3(grid), dim3(kGemvThreads), shm, s, a); break;
        default: hipLaunchKernelGGL((gemv_kernel<WT, LPR, BM, EPI_LOGITS>), dim3(grid), dim3(kGemvThreads), shm, s, a); break;
    }
    return hipGetLastError();
}

template <typename WT, int LPR>
static hipError_t gemv_dispatch_bm(const GemvArgs& a, int epi, int grid, size_t shm, hipStream_t s) {
    if (a.B <= 1) return gemv_dispatch_epi<WT, LPR, 1>(a, epi, grid, shm, s);
    if (a.B <= 4) return gemv_dispatch_epi<WT, LPR, 4>(a, epi, grid, shm, s);
    return gemv_dispatch_epi<WT, LPR, 16>(a, epi, grid, shm, s);
}

hipError_t launch_gemv(const GemvArgs& a, int w_type, int epi, int grid_cap, int* grid_out,
                       hipStream_t s) {
    if (w_type == 2 && (a.K % 16 || (a.kt < a.K && a.kt % 16) || !a.wscale[0] ||
                        (epi == EPI_SWIGLU && !a.wscale[1])))
        return hipErrorInvalidValue;
    const int rpt = gemv_rows_per_tile(a.K);
    const int tiles = (a.N + rpt - 1) / rpt;
    const int grid = tiles < grid_cap ? tiles : grid_cap;
    if (grid_out) *grid_out = grid;
    const size_t shm = (size_t)a.B * (size_t)(a.kt < a.K ? a.kt : a.K) * sizeof(float);
    if (a.K <= 2048) {
        if (w_type == 2) return gemv_dispatch_bm<int8_t, 16>(a, epi, grid, shm, s);
        return w_type == 1 ? gemv_dispatch_bm<uint16_t, 16>(a, epi, grid, shm, s)
                           : gemv_dispatch_bm<float, 16>(a, epi, grid, shm, s);
    }
    if (w_type == 2) return gemv_dispatch_bm<int8_t, 64>(a, epi, grid, shm, s);
    return w_type == 1 ? gemv_dispatch_bm<uint16_t, 64>(a, epi, grid, shm, s)
                       : gemv_dispatch_bm<float, 64>(a, epi, grid, shm, s);
}

__global__ __launch_bounds__(256) void copy_kernel(const float* src, float* dst, long n) {
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

hipError_t launch_copy(const float* src, float* dst, long n, hipStream_t s) {
    long blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

// Final greedy argmax over the per-workgroup (value, row) partials of the
// lm_head; the argmax pair is a monoid (Tang page, section 2.2), lowest row wins ties.
__global__ __launch_bounds__(256) void argmax_kernel(const float* pv, const int* pi, int nparts, int* out) {
    __shared__ float sv[4];
    __shared__ int si[4];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float v = -INFINITY;
    int i = 0x7fffffff;
    for (int j = tid; j < nparts; j += 256) {
        const float ov = pv[(long)b * nparts + j];
        const int oi = pi[(long)b * nparts + j];
        if (better(ov, oi, v, i)) { v = ov; i = oi; }
    }
    wave_argmax(v, i);
    if (lane == 0) { sv[wave] = v; si[wave] = i; }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < 4; ++w)
            if (better(sv[w], si[w], sv[0], si[0])) { sv[0] = sv[w]; si[0] = si[w]; }
        out[b] = si[0];
    }
}

hipError_t launch_argmax(const float* part_val, const int* part_idx, int nparts, int* out, int B,
                         hipStream_t s) {
    hipLaunchKernelGGL(argmax_kernel, dim3(B), dim3(256), 0, s, part_val, part_idx, nparts, out);
    return hipGetLastError();
}

// Store already-rotated k, v ([B][Hkv][hd] float) at positions pos[b].
template <typename KVT>
__global__ __launch_bounds__(128) void kv_append_kernel(const float* k, const float* v, void* kc, void* vc,
                                                        const int* bt, int max_blocks, int num_pages,
                                                        const int* pos, int capacity, int Hkv, int hd,
                                                        int page) {
    const int g = blockIdx.x, b = blockIdx.y;
    const int p = pos[b];
    if (p < 0 || p >= capacity) return;
    const int page_id = bt[(long)b * max_blocks + p / page];
    if (page_id < 0 || page_id >= num_pages) return;
    const long off = (((long)page_id * Hkv + g) * page + (p % page)) * hd;
    for (int d = threadIdx.x; d < hd; d += blockDim.x) {
        ((KVT*)kc)[off + d] = from_f32<KVT>(k[((long)b * Hkv + g) * hd + d]);
        ((KVT*)vc)[off + d] = from_f32<KVT>(v[((long)b * Hkv + g) * hd + d]);
    }
}

hipError_t launch_kv_append(const float* k, const float* v, void* k_cache, void* v_cache,
                            const int* block_table, int max_blocks, int num_pages, const int* pos,
                            int capacity, int Hkv, int hd, int page, int B, int kv_is_bf16,
                            hipStream_t s) {
    dim3 grid(Hkv, B);
    if (kv_is_bf16)
        hipLaunchKernelGGL((kv_append_kernel<uint16_t>), grid, dim3(128), 0, s, k, v, k_cache, v_cache,
                           block_table, max_blocks, num_pages, pos, capacity, Hkv, hd, page);
    else
        hipLaunchKernelGGL((kv_append_kernel<float>), grid, dim3(128), 0, s, k, v, k_cache, v_cache,
                           block_table, max_blocks, num_pages, pos, capacity, Hkv, hd, page);
    return hipGetLastError();
}

}  // namespace qd
