// Prefill block kernels for gfx950: the multi-token projections are dense
// contractions, so they run as bf16 MFMA GEMMs with float32 accumulation
// (v_mfma_f32_32x32x16_bf16); their activation operands are rounded to bf16
// at the points the block stores them (normed input, attention context,
// SwiGLU output). The residual stream stays float32.
//
// GEMM: C[M][N] (op)= A[M][K] . W[N][K]^T with both operands K-contiguous, as
// the weights are stored row-major [out][in]. One workgroup of 4 waves owns a
// 128 x 128 tile (2 x 2 waves of 64 x 64, each 2 x 2 MFMA tiles of 32 x 32),
// walks K in steps of 32 with the A and W tiles staged in LDS (double
// buffered, padded rows against bank conflicts), and the next K step's global
// loads are issued before the current step's MFMAs. Epilogues (Tang page,
// section 2.3): store float32 (q|k|v), add into the float32 residual (o_proj,
// down), or silu(gate) * up rounded to bf16 with gate and up tiles of the same
// columns held by the same lane (sibling reductions merged).
#include "qd_device.h"
#include "qd_launch.h"

namespace qd {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int kGemmBM = 128, kGemmBN = 128, kGemmBK = 32;
constexpr int kGemmLdsRow = kGemmBK + 8;   // bf16 elements per padded LDS row (80 bytes)

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// W row pointer of output column n (stacked segments, as in the decode GEMV)
__device__ __forceinline__ const uint16_t* gemm_wrow(const GemmArgs& a, int n) {
    const bool s0 = n < a.seg_end[0], s1 = n < a.seg_end[1];
    const void* w = s0 ? a.w[0] : (s1 ? a.w[1] : a.w[2]);
    const int base = s0 ? 0 : (s1 ? a.seg_end[0] : a.seg_end[1]);
    return (const uint16_t*)w + (long)(n - base) * a.K;
}

template <int EPI>
__global__ __launch_bounds__(256) void mfma_gemm_kernel(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kGemmBM * kGemmLdsRow];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[2][kGemmBN * kGemmLdsRow];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int M = a.M, K = a.K;
    // output tile: rows m0.., columns: for SwiGLU the tile holds 64 h-columns as
    // 64 gate rows followed by 64 up rows of W; otherwise 128 columns of C
    const int m0 = blockIdx.y * kGemmBM;
    const int tileN = blockIdx.x;

    // each thread loads 2 chunks (16 bytes = 8 bf16) of the A tile and 2 of the W tile per K step
    int a_row[2], a_kc[2], w_row[2], w_kc[2];
    const uint16_t* a_ptr[2];
    const uint16_t* w_ptr[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int idx = tid + r * 256;           // 0..511: row = idx / 4, chunk = idx % 4
        a_row[r] = idx >> 2; a_kc[r] = idx & 3;
        w_row[r] = idx >> 2; w_kc[r] = idx & 3;
        const int m = m0 + a_row[r];
        a_ptr[r] = (m < M) ? (const uint16_t*)a.A + (long)m * K : nullptr;
        int n;
        bool valid;
        if (EPI == GEMM_SWIGLU) {
            const int hcol = tileN * 64 + (w_row[r] & 63);
            valid = hcol < a.N;
            w_ptr[r] = valid ? (const uint16_t*)a.w[w_row[r] >> 6] + (long)hcol * K : nullptr;
        } else {
            n = tileN * kGemmBN + w_row[r];
            valid = n < a.N;
            w_ptr[r] = valid ? gemm_wrow(a, n) : nullptr;
        }
    }
    auto load_tile = [&](int k0, uint4 (&ra)[2], uint4 (&rw)[2]) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int ka = k0 + a_kc[r] * 8, kw = k0 + w_kc[r] * 8;
            ra[r] = (a_ptr[r] && ka < K) ? *(const uint4*)(a_ptr[r] + ka) : make_uint4(0, 0, 0, 0);
            rw[r] = (w_ptr[r] && kw < K) ? *(const uint4*)(w_ptr[r] + kw) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_tile = [&](int buf, const uint4 (&ra)[2], const uint4 (&rw)[2]) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            *(uint4*)&As[buf][a_row[r] * kGemmLdsRow + a_kc[r] * 8] = ra[r];
            *(uint4*)&Ws[buf][w_row[r] * kGemmLdsRow + w_kc[r] * 8] = rw[r];
        }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    uint4 ra[2], rw[2];
    load_tile(0, ra, rw);
    store_tile(0, ra, rw);
    __syncthreads();
    const int nk = (K + kGemmBK - 1) / kGemmBK;
    // lane's operand rows within the wave tile and k offset within a 16-wide step
    const int lrow = lane & 31, lk = (lane >> 5) * 8;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_tile((kt + 1) * kGemmBK, ra, rw);
#pragma unroll
        for (int ks = 0; ks < kGemmBK; ks += 16) {
            bf16x8_t av[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                av[i] = as_bf16x8(*(const uint4*)&As[buf][(wm * 64 + i * 32 + lrow) * kGemmLdsRow + ks + lk]);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                // SwiGLU: wave column-half wn holds h-columns wn*32..; j = 0 gate rows, j = 1 up rows
                const int wrow = (EPI == GEMM_SWIGLU) ? (j * 64 + wn * 32 + lrow) : (wn * 64 + j * 32 + lrow);
                bv[j] = as_bf16x8(*(const uint4*)&Ws[buf][wrow * kGemmLdsRow + ks + lk]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            store_tile(buf ^ 1, ra, rw);
            __syncthreads();
        }
    }
    // epilogue: lane holds column (lane % 32) of each 32 x 32 tile and rows
    // (e / 4) * 8 + (lane / 32) * 4 + (e % 4)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int m = m0 + wm * 64 + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
            if (m >= M) continue;
            if (EPI == GEMM_SWIGLU) {
                const int hcol = tileN * 64 + wn * 32 + lrow;
                if (hcol < a.N) {
                    const float g = acc[i][0][e], u = acc[i][1][e];
                    ((uint16_t*)a.C)[(long)m * a.ldc + hcol] = f32_to_bf16(silu(g) * u);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int n = tileN * kGemmBN + wn * 64 + j * 32 + lrow;
                    if (n >= a.N) continue;
                    float* cp = (float*)a.C + (long)m * a.ldc + n;
                    if (EPI == GEMM_STORE) {
                        const bool s0 = n < a.seg_end[0], s1 = n < a.seg_end[1];
                        const void* bsel = s0 ? a.bias[0] : (s1 ? a.bias[1] : a.bias[2]);
                        const int base = s0 ? 0 : (s1 ? a.seg_end[0] : a.seg_end[1]);
                        *cp = bsel ? acc[i][j][e] + bf16_to_f32(((const uint16_t*)bsel)[n - base]) : acc[i][j][e];
                    } else {
                        *cp = *cp + acc[i][j][e];
                    }
                }
            }
        }
    }
}

hipError_t launch_mfma_gemm(const GemmArgs& a, int epi, hipStream_t s) {
    const int cols = epi == GEMM_SWIGLU ? 64 : kGemmBN;
    dim3 grid((a.N + cols - 1) / cols, (a.M + kGemmBM - 1) / kGemmBM);
    switch (epi) {
        case GEMM_STORE: hipLaunchKernelGGL((mfma_gemm_kernel<GEMM_STORE>), grid, dim3(256), 0, s, a); break;
        case GEMM_RESID: hipLaunchKernelGGL((mfma_gemm_kernel<GEMM_RESID>), grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((mfma_gemm_kernel<GEMM_SWIGLU>), grid, dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row RMSNorm to a bf16 GEMM operand: n = bf16(x * (1/sqrt(sum(x^2)/D + eps)) * g)
// (nanocompile page, phase 1: sum then divide, eps inside the root). With
// x_res set, the input row (bf16 or float) is also widened into the float32
// residual stream.
template <typename WT>
__global__ __launch_bounds__(256) void prefill_norm_kernel(PrefillNormArgs a) {
    __shared__ float wsum[4];
    const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int D = a.D;
    float ss = 0.f;
    for (int d = tid; d < D; d += 256) {
        const float v = a.x_bf16 ? bf16_to_f32(((const uint16_t*)a.x_bf16)[(long)row * D + d])
                                 : a.x_f32[(long)row * D + d];
        ss += v * v;
        if (a.x_res) a.x_res[(long)row * D + d] = v;
    }
    ss = group_sum<kWave>(ss);
    if (lane == 0) wsum[wave] = ss;
    __syncthreads();
    const float r = 1.0f / sqrtf((wsum[0] + wsum[1] + wsum[2] + wsum[3]) / (float)D + a.eps);
    for (int d = tid; d < D; d += 256) {
        const float v = a.x_bf16 ? bf16_to_f32(((const uint16_t*)a.x_bf16)[(long)row * D + d])
                                 : a.x_f32[(long)row * D + d];
        a.out[(long)row * D + d] = f32_to_bf16(v * r * load_scalar<WT>(a.gain, d));
    }
}

hipError_t launch_prefill_norm(const PrefillNormArgs& a, int w_is_bf16, hipStream_t s) {
    if (w_is_bf16) hipLaunchKernelGGL((prefill_norm_kernel<uint16_t>), dim3(a.rows), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((prefill_norm_kernel<float>), dim3(a.rows), dim3(256), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per (row i, head): optional per-head q/k RMSNorm, RoPE at position start + i
// (half-split, angle in double reduced mod 2*pi, sine/cosine in float), q to a
// float32 buffer, k and v stored into the cache slot of that position in the
// cache type (keys rotated once, on insert -- nanoinfer page, phase 4). One
// wavefront per (row, head); lane i rotates the pair (i, i + hd/2).
template <typename WT, typename KVT>
__global__ __launch_bounds__(64) void prefill_rope_append_kernel(PrefillRopeArgs a) {
    const int row = blockIdx.x, h = blockIdx.y, i = threadIdx.x;
    const int hd = a.hd, half = hd >> 1;
    const int p = a.start + row;
    if (p < 0 || p >= a.capacity) return;
    const int qkvr = (a.Hq + 2 * a.Hkv) * hd;
    const bool is_q = h < a.Hq;
    const float* src = a.qkv + (long)row * qkvr + (is_q ? h * hd : a.Hq * hd + (h - a.Hq) * hd);
    const bool act = i < half;
    float lo = act ? src[i] : 0.f, hi = act ? src[i + half] : 0.f;
    if (a.qk_norm) {
        const float ss = group_sum<kWave>(lo * lo + hi * hi);
        const float r = 1.0f / sqrtf(ss / (float)hd + a.eps);
        const void* g = is_q ? a.q_norm : a.k_norm;
        if (act) {
            lo = lo * r * load_scalar<WT>(g, i);
            hi = hi * r * load_scalar<WT>(g, i + half);
        }
    }
    if (!act) return;
    const double inv = pow((double)a.theta, -2.0 * (double)i / (double)hd);
    double ang = (double)p * inv;
    const double two_pi = 6.283185307179586476925286766559;
    ang -= two_pi * rint(ang / two_pi);
    float sn, cs;
    sincosf((float)ang, &sn, &cs);
    const float lo2 = lo * cs - hi * sn, hi2 = hi * cs + lo * sn;
    if (is_q) {
        float* q = a.q_out + ((long)row * a.Hq + h) * hd;
        q[i] = lo2;
        q[i + half] = hi2;
    } else {
        const int g = h - a.Hq;
        const int page_id = a.block_table[p / a.page];
        if (page_id < 0 || page_id >= a.num_pages) return;
        const long off = (((long)page_id * a.Hkv + g) * a.page + (p % a.page)) * hd;
        const float* vs = a.qkv + (long)row * qkvr + (a.Hq + a.Hkv) * hd + g * hd;
        KVT* kc = (KVT*)a.k_cache + off;
        KVT* vc = (KVT*)a.v_cache + off;
        kc[i] = from_f32<KVT>(lo2);
        kc[i + half] = from_f32<KVT>(hi2);
        vc[i] = from_f32<KVT>(vs[i]);
        vc[i + half] = from_f32<KVT>(vs[i + half]);
    }
}

hipError_t launch_prefill_rope_append(const PrefillRopeArgs& a, int w_is_bf16, int kv_is_bf16, hipStream_t s) {
    dim3 grid(a.rows, a.Hq + a.Hkv);
    if (w_is_bf16) {
        if (kv_is_bf16) hipLaunchKernelGGL((prefill_rope_append_kernel<uint16_t, uint16_t>), grid, dim3(64), 0, s, a);
        else hipLaunchKernelGGL((prefill_rope_append_kernel<uint16_t, float>), grid, dim3(64), 0, s, a);
    } else {
        if (kv_is_bf16) hipLaunchKernelGGL((prefill_rope_append_kernel<float, uint16_t>), grid, dim3(64), 0, s, a);
        else hipLaunchKernelGGL((prefill_rope_append_kernel<float, float>), grid, dim3(64), 0, s, a);
    }
    return hipGetLastError();
}

// Float32 -> bf16 (round half to even), n elements: the attention context as
// the o_proj GEMM operand.
__global__ __launch_bounds__(256) void to_bf16_kernel(const float* x, uint16_t* y, long n) {
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) y[i] = f32_to_bf16(x[i]);
}

hipError_t launch_to_bf16(const float* x, void* y, long n, hipStream_t s) {
    long blocks = (n + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, (uint16_t*)y, n);
    return hipGetLastError();
}

}  // namespace qd
