// Batched decode projections (2..16 sequences) on the gfx950 matrix cores.
//
// A decode projection at batch B streams a row-major [N][K] bf16 weight matrix
// once and does B multiply-adds per weight. At B = 16 that is 16 FMAs per two
// bytes: at 8 TB/s the vector ALUs would have to run near their fp32 peak, so
// the product goes to v_mfma_f32_16x16x32_bf16 instead, with the weights as
// the A operand (16 output rows) and the B token vectors as the 16 columns of
// the B operand (columns past B are zeros).
//
// The matrix cores take bf16 operands, but a decode step keeps its activations
// in float32. Each activation (RMSNorm gain applied) is split into two bf16
// values, hi = bf16(v) and lo = bf16(v - hi); W v = W hi + W lo up to
// 2^-17 |v| per term, so the product keeps float32-level accuracy at the cost
// of a second MFMA, and the matrix cores stay far from busy (the kernel is HBM
// bound). RMSNorm is folded in as in the batch-1 GEMV (Tang page, section 2.3):
// the staged operand is x * g, and r = 1/sqrt(sum(x^2)/K + eps) (nanocompile
// page, phase 1) scales each finished output.
//
// Workgroup: 4 waves; WR = 4/WK waves along rows, WK waves split each K chunk
// and meet in LDS in a fixed order (deterministic). A wave owns R blocks of 16
// rows (two per block for gate|up). The activation chunk sits in LDS in the
// MFMA B-fragment layout, [k/8][token] of 16-byte groups, hi and lo apart, so
// a fragment read is one conflict-free 16-byte LDS read per lane. Weight
// fragments are loaded U k-steps ahead of their use.
#include <algorithm>

#include "qd_device.h"
#include "qd_launch.h"

namespace qd {

typedef __attribute__((ext_vector_type(8))) __bf16 g16_bf16x8;
typedef __attribute__((ext_vector_type(4))) float g16_f32x4;

constexpr int kG16Chunk = 1024;   // K elements staged per chunk: 64 KB of LDS for 16 tokens
constexpr int kG16U = 2;          // k-steps (of 32) per pipeline stage (lm_head at batch 16: 59.5 us at 2, 62.4 at 4, 63.8 at 8)
constexpr int kG16Cus = 256;      // compute units of the chip (MI355X)
// Waves of a gemm16_rows_kernel workgroup and its grid (8 waves per CU): at batch 16
// the 0.5B gate|up takes 8.55 us with two 4-wave workgroups per CU against 8.67
// with one of 8 (one staged activation per CU) for bf16 rows, and 9.94 against
// 9.52 us for int8 rows, so int8 rows take the 8-wave form.
template <typename WT> constexpr int g16_rows_waves() { return sizeof(WT) == 1 ? 8 : 4; }
template <typename WT> constexpr int g16_rows_wgs() { return 8 * kG16Cus / g16_rows_waves<WT>(); }

__device__ __forceinline__ g16_bf16x8 g16_frag(uint4 v) { return __builtin_bit_cast(g16_bf16x8, v); }

// Loads are issued unconditionally and masked by their address: a masked lane
// reads a static zero block instead. (A load under a per-lane branch makes the
// compiler wait for every outstanding load before the branch joins, and a select
// on a load's result makes it wait for that load before issuing the next one;
// either would empty the prefetch pipeline.)
__device__ __align__(16) uint32_t kG16Zeros[8];   // zero from load time, never written
template <typename T>
__device__ __forceinline__ T load_or_zero(const void* p, bool ok) {
    return *(const T*)(ok ? p : (const void*)kG16Zeros);
}

// Weight rows: bf16 (a lane's 8 weights of a k-step in one 16-byte load), or int8
// codes with one float scale per row (nanoinfer page, phase 6), whose 8 codes come
// in one 8-byte load and are widened to bf16 exactly (|code| <= 127 fits the 8-bit
// significand), so the same MFMAs run; the row's scale multiplies the finished
// product. Gains and biases stay bf16.
template <typename WT> struct G16W;
template <> struct G16W<uint16_t> {
    using L = uint4;
    static __device__ __forceinline__ uint4 frag(uint4 v) { return v; }
};
template <> struct G16W<int8_t> {
    using L = uint2;
    static __device__ __forceinline__ uint4 frag(uint2 v) {
        typedef __attribute__((ext_vector_type(2))) float f2;
        typedef __attribute__((ext_vector_type(2))) __bf16 b2;
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {   // codes 2i, 2i + 1 (memory order) -> one bf16 pair
            const uint32_t w = i < 2 ? v.x : v.y;
            const int sh = (i & 1) * 16;
            const float lo = (float)(int8_t)(w >> sh), hi = (float)(int8_t)(w >> (sh + 8));
            o[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{lo, hi}, b2));
        }
        return make_uint4(o[0], o[1], o[2], o[3]);
    }
};
// the scale of output row r (1 for bf16 rows): matrix n of a SwiGLU pair, else the
// segment that holds r
template <typename WT, int EPI>
__device__ __forceinline__ float g16_scale(const GemvArgs& a, int r, int n) {
    if constexpr (sizeof(WT) == 2) {
        return 1.f;
    } else {
        if (EPI == EPI_SWIGLU) return a.wscale[n][r];
        const bool q0 = r < a.seg_end[0], q1 = r < a.seg_end[1];
        const int base = q0 ? 0 : (q1 ? a.seg_end[0] : a.seg_end[1]);
        return (q0 ? a.wscale[0] : (q1 ? a.wscale[1] : a.wscale[2]))[r - base];
    }
}

template <typename WT, int EPI, int R, int WK>
__global__ __launch_bounds__(256) void gemm16_kernel(GemvArgs a) {
    using WL = typename G16W<WT>::L;
    // int8 rows: one 16-byte load per lane covers a pair of k-steps (s, s + 1): lane
    // kq holds the 16 codes at 32 s + 16 kq, codes 8u .. 8u + 7 feeding the pair's
    // MFMA u with the activation group (32 s + 16 kq + 8 u) / 8, the same products
    // in another k order, and half the load instructions of 8-byte loads
    constexpr bool PAIR = sizeof(WT) == 1;
    constexpr int NW = (EPI == EPI_SWIGLU) ? 2 : 1;
    constexpr int WR = 4 / WK;
    constexpr int TR = WR * R * 16;          // output rows per tile
    constexpr int U = sizeof(WT) == 1 ? 2 * kG16U : kG16U;   // int8: as many load instructions per stage as bf16
    extern __shared__ uint4 xs[];            // hi: [chunk/8][16], then lo: [chunk/8][16]
    __shared__ float ssum[4][16];
    __shared__ g16_f32x4 red[WK > 1 ? WK - 1 : 1][WR][R][NW][kWave];
    __shared__ float bv_s[4][16];
    __shared__ int bi_s[4][16];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int wr = wave % WR, wk = wave / WR;
    const int col = lane & 15, kq = lane >> 4;
    const int B = a.B, K = a.K, N = a.N;
    const int kc_max = a.kt;                 // multiple of 32
    const int nchunk = (K + kc_max - 1) / kc_max;
    const int ntiles = (N + TR - 1) / TR;
    uint4* xhi = xs;
    uint4* xlo = xs + (kc_max / 8) * 16;

    if (a.zero_ptr && blockIdx.x == 0)
        for (int i = tid; i < a.zero_n; i += 256) a.zero_ptr[i] = 0u;

    // Stage x[:, k0 .. k0 + kcp) (times the gain) as hi/lo bf16 fragments; items past
    // K or B are zeros. Thread tid always handles token tid % 16, so its running
    // sum of squares belongs to one token.
    float ss = 0.f;
    auto stage = [&](int k0, int kcp, bool acc_ss) {
        for (int i = tid; i < (kcp / 8) * 16; i += 256) {
            const int t = i & 15, j = i >> 4, k = k0 + j * 8;
            float v[8];
            if (t < B && k < K) {
                const float4 p0 = *(const float4*)(a.x + (long)t * K + k);
                const float4 p1 = *(const float4*)(a.x + (long)t * K + k + 4);
                v[0] = p0.x; v[1] = p0.y; v[2] = p0.z; v[3] = p0.w;
                v[4] = p1.x; v[5] = p1.y; v[6] = p1.z; v[7] = p1.w;
                if (a.gain) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if (acc_ss) ss += v[e] * v[e];
                        v[e] *= load_scalar<uint16_t>(a.gain, k + e);
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = 0.f;
            }
            split_hi_lo(v, xhi[j * 16 + t], xlo[j * 16 + t]);
        }
    };

    const bool one_chunk = nchunk == 1;
    if (one_chunk) {
        stage(0, (K + 31) & ~31, true);
        __syncthreads();
    }
    float rs = 1.0f;          // RMSNorm scale of token `col`
    bool have_rs = false;
    float best_v = -INFINITY;
    int best_i = 0x7fffffff;

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        // weight row pointers of this lane's A fragments (row = block base + col)
        const WT* wrow[R][NW];      // rows past N read row 0 (masked)
        bool rok[R];
#pragma unroll
        for (int rb = 0; rb < R; ++rb) {
            const int r = tile * TR + (wr * R + rb) * 16 + col;
            rok[rb] = r < N;
#pragma unroll
            for (int n = 0; n < NW; ++n) {
                const WT* p = (const WT*)a.w[n];
                if (r < N) {
                    if (EPI == EPI_SWIGLU) {
                        p = (const WT*)a.w[n] + (long)r * K;
                    } else {
                        const bool s0 = r < a.seg_end[0], s1 = r < a.seg_end[1];
                        const void* w = s0 ? a.w[0] : (s1 ? a.w[1] : a.w[2]);
                        const int base = s0 ? 0 : (s1 ? a.seg_end[0] : a.seg_end[1]);
                        p = (const WT*)w + (long)(r - base) * K;
                    }
                }
                wrow[rb][n] = p;
            }
        }
        g16_f32x4 acc[R][NW];
#pragma unroll
        for (int rb = 0; rb < R; ++rb)
#pragma unroll
            for (int n = 0; n < NW; ++n) acc[rb][n] = g16_f32x4{0.f, 0.f, 0.f, 0.f};

        for (int ch = 0; ch < nchunk; ++ch) {
            const int k0 = ch * kc_max;
            const int kc = min(kc_max, K - k0);
            const int kcp = (kc + 31) & ~31;
            if (!one_chunk) {
                __syncthreads();                       // previous chunk's readers are done
                stage(k0, kcp, !have_rs);
                __syncthreads();
            }
            const int nsteps = kcp / 32;
            const int s0 = wk * nsteps / WK, s1 = (wk + 1) * nsteps / WK;
            WL wa[U][R][NW], wb[U][R][NW];
            auto load = [&](WL (&w)[U][R][NW], int sb) {
                if constexpr (PAIR) {
                    static_assert(U % 2 == 0, "whole pairs of k-steps per stage");
#pragma unroll
                    for (int q = 0; q < U / 2; ++q) {
                        const int sp = sb + 2 * q;
                        const int k = k0 + sp * 32 + kq * 16;
                        const bool kok = sp + (kq >> 1) < s1 && k < K;   // the step these codes belong to
                        const int kc = kok ? k : 0;
#pragma unroll
                        for (int rb = 0; rb < R; ++rb)
#pragma unroll
                            for (int n = 0; n < NW; ++n) {
                                const uint4 v = load_or_zero<uint4>(wrow[rb][n] + kc, kok && rok[rb]);
                                w[2 * q][rb][n] = WL{v.x, v.y};
                                w[2 * q + 1][rb][n] = WL{v.z, v.w};
                            }
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int s = sb + u;
                        const int k = k0 + s * 32 + kq * 8;
                        const bool kok = s < s1 && k < K;
                        const int kc = kok ? k : 0;
#pragma unroll
                        for (int rb = 0; rb < R; ++rb)
#pragma unroll
                            for (int n = 0; n < NW; ++n)
                                w[u][rb][n] = load_or_zero<WL>(wrow[rb][n] + kc, kok && rok[rb]);
                    }
                }
            };
            auto mma = [&](const WL (&w)[U][R][NW], int sb) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int s = sb + u, sp = sb + (u & ~1);   // (PAIR: the pair's first step)
                    if (PAIR ? sp >= s1 : s >= s1) break;
                    // (PAIR: a lane whose codes lie past the range holds zeros; it reads group 0)
                    const int grp = PAIR ? (sp + (kq >> 1) < s1 ? 4 * sp + 2 * kq + (u & 1) : 0) : s * 4 + kq;
                    const g16_bf16x8 bh = g16_frag(xhi[grp * 16 + col]);
                    const g16_bf16x8 bl = g16_frag(xlo[grp * 16 + col]);
#pragma unroll
                    for (int rb = 0; rb < R; ++rb)
#pragma unroll
                        for (int n = 0; n < NW; ++n) {
                            const g16_bf16x8 af = g16_frag(G16W<WT>::frag(w[u][rb][n]));
                            acc[rb][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bh, acc[rb][n], 0, 0, 0);
                            acc[rb][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bl, acc[rb][n], 0, 0, 0);
                        }
                }
            };
            int s = s0;
            if (s < s1) load(wa, s);
            while (s < s1) {
                load(wb, s + U);
                mma(wa, s);
                s += U;
                if (s >= s1) break;
                load(wa, s + U);
                mma(wb, s);
                s += U;
            }
        }

        if (!have_rs) {            // every thread reaches this on the first tile
            if (a.gain) {
                const float t = strided_sum<16>(ss);
                if (lane < 16) ssum[wave][lane] = t;
                __syncthreads();
                rs = 1.0f / sqrtf((ssum[0][col] + ssum[1][col] + ssum[2][col] + ssum[3][col]) / (float)K + a.eps);
            }
            have_rs = true;
        }

        if (WK > 1) {
            if (wk > 0)
#pragma unroll
                for (int rb = 0; rb < R; ++rb)
#pragma unroll
                    for (int n = 0; n < NW; ++n) red[wk - 1][wr][rb][n][lane] = acc[rb][n];
            __syncthreads();
            if (wk == 0)
#pragma unroll
                for (int q = 0; q < WK - 1; ++q)
#pragma unroll
                    for (int rb = 0; rb < R; ++rb)
#pragma unroll
                        for (int n = 0; n < NW; ++n) acc[rb][n] += red[q][wr][rb][n][lane];
            __syncthreads();
        }

        if (wk == 0 && col < B) {
            float* yrow = a.y + (long)col * N;
#pragma unroll
            for (int rb = 0; rb < R; ++rb) {
                const int rbase = tile * TR + (wr * R + rb) * 16 + kq * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = rbase + e;
                    if (r >= N) break;
                    const float v0 = acc[rb][0][e] * rs * g16_scale<WT, EPI>(a, r, 0);
                    if (EPI == EPI_STORE) {
                        const bool s0 = r < a.seg_end[0], s1 = r < a.seg_end[1];
                        const void* bsel = s0 ? a.bias[0] : (s1 ? a.bias[1] : a.bias[2]);
                        const int base = s0 ? 0 : (s1 ? a.seg_end[0] : a.seg_end[1]);
                        yrow[r] = bsel ? v0 + load_scalar<uint16_t>(bsel, r - base) : v0;
                    } else if (EPI == EPI_RESID) {
                        yrow[r] = yrow[r] + v0;
                    } else if (EPI == EPI_SWIGLU) {
                        yrow[r] = silu(v0) * (acc[rb][NW - 1][e] * rs * g16_scale<WT, EPI>(a, r, NW - 1));
                    } else {
                        yrow[r] = v0;
                        if (better(v0, r, best_v, best_i)) { best_v = v0; best_i = r; }
                    }
                }
            }
        }
    }

    if (EPI == EPI_LOGITS) {
        argmax_across_rows(best_v, best_i);
        if (lane < 16) { bv_s[wave][lane] = best_v; bi_s[wave][lane] = best_i; }
        __syncthreads();
        if (tid < B) {
            float v = bv_s[0][tid];
            int i = bi_s[0][tid];
            for (int w = 1; w < WR; ++w)            // waves 0 .. WR-1 hold the wk == 0 results
                if (better(bv_s[w][tid], bi_s[w][tid], v, i)) { v = bv_s[w][tid]; i = bi_s[w][tid]; }
            a.part_val[(long)tid * gridDim.x + blockIdx.x] = v;
            a.part_idx[(long)tid * gridDim.x + blockIdx.x] = i;
        }
    }
}

// One 16-row block per wave-row, activations straight from memory: with a
// single row block per workgroup a staged copy of the activation would be read
// once, so each lane loads its own B fragment (8 float32 of one token) from
// L2 in the same pipeline as the weights and splits it into hi/lo in
// registers. No LDS staging, no barrier before the first MFMA. The gain, when
// present, must be 16-byte aligned.
template <typename WT, int EPI, int WK>
__global__ __launch_bounds__(64 * WK) void gemm16_direct_kernel(GemvArgs a) {
    using WL = typename G16W<WT>::L;
    constexpr bool GAIN = EPI != EPI_RESID;       // every normed projection; residual ones have none
    constexpr int NW = (EPI == EPI_SWIGLU) ? 2 : 1;
    constexpr int TR = 16;
    constexpr int U = kG16U;
    __shared__ float ssum[WK][16];
    __shared__ g16_f32x4 red[WK - 1][NW][kWave];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int wk = wave;
    const int col = lane & 15, kq = lane >> 4;
    const int B = a.B, K = a.K, N = a.N;
    const int tile = blockIdx.x;
    const bool tok = col < B;
    const float* xrow = a.x + (long)(tok ? col : 0) * K;
    const uint16_t* gain = (const uint16_t*)a.gain;

    if (a.zero_ptr && blockIdx.x == 0)
        for (int i = tid; i < a.zero_n; i += 64 * WK) a.zero_ptr[i] = 0u;

    const WT* wrow[NW];         // a row past N reads row 0 (masked)
    const int r_own = tile * TR + col;
    const bool rok = r_own < N;
    {
        const int r = r_own;
#pragma unroll
        for (int n = 0; n < NW; ++n) {
            const WT* p = (const WT*)a.w[n];
            if (r < N) {
                if (EPI == EPI_SWIGLU) {
                    p = (const WT*)a.w[n] + (long)r * K;
                } else {
                    const bool s0 = r < a.seg_end[0], s1 = r < a.seg_end[1];
                    const void* w = s0 ? a.w[0] : (s1 ? a.w[1] : a.w[2]);
                    const int base = s0 ? 0 : (s1 ? a.seg_end[0] : a.seg_end[1]);
                    p = (const WT*)w + (long)(r - base) * K;
                }
            }
            wrow[n] = p;
        }
    }
    g16_f32x4 acc[NW];
#pragma unroll
    for (int n = 0; n < NW; ++n) acc[n] = g16_f32x4{0.f, 0.f, 0.f, 0.f};
    float ss = 0.f;

    const int nsteps = (K + 31) / 32;
    const int s0 = wk * nsteps / WK, s1 = (wk + 1) * nsteps / WK;
    struct Stage {
        WL w[U][NW];
        float4 x0[U], x1[U];
        uint4 g[U];
    };
    Stage sa, sb;
    auto load = [&](Stage& st, int sbase) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = sbase + u;
            const int k = s * 32 + kq * 8;
            const bool ok = s < s1 && k < K;
            const int kc = ok ? k : 0;
#pragma unroll
            for (int n = 0; n < NW; ++n) st.w[u][n] = load_or_zero<WL>(wrow[n] + kc, ok && rok);
            st.x0[u] = load_or_zero<float4>(xrow + kc, ok && tok);
            st.x1[u] = load_or_zero<float4>(xrow + kc + 4, ok && tok);
            if (GAIN) st.g[u] = load_or_zero<uint4>(gain + kc, ok);
        }
    };
    auto mma = [&](const Stage& st, int sbase) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (sbase + u >= s1) break;
            float v[8] = {st.x0[u].x, st.x0[u].y, st.x0[u].z, st.x0[u].w,
                          st.x1[u].x, st.x1[u].y, st.x1[u].z, st.x1[u].w};
            if (GAIN) {
                float gf[8];
                widen16(st.g[u], gf);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ss += v[e] * v[e];
                    v[e] *= gf[e];
                }
            }
            uint4 hu, lu;
            split_hi_lo(v, hu, lu);
            const g16_bf16x8 bh = g16_frag(hu);
            const g16_bf16x8 bl = g16_frag(lu);
#pragma unroll
            for (int n = 0; n < NW; ++n) {
                const g16_bf16x8 af = g16_frag(G16W<WT>::frag(st.w[u][n]));
                acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bh, acc[n], 0, 0, 0);
                acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bl, acc[n], 0, 0, 0);
            }
        }
    };
    int s = s0;
    if (s < s1) load(sa, s);
    while (s < s1) {
        load(sb, s + U);
        mma(sa, s);
        s += U;
        if (s >= s1) break;
        load(sa, s + U);
        mma(sb, s);
        s += U;
    }

    // sum of squares of token `col` over this wave's K range, then over the WK waves
    // of this wave-row (fixed order); partial products likewise
    if (GAIN) {
        const float t = strided_sum<16>(ss);
        if (lane < 16) ssum[wave][lane] = t;
    }
    if (wk > 0)
#pragma unroll
        for (int n = 0; n < NW; ++n) red[wk - 1][n][lane] = acc[n];
    __syncthreads();
    float rs = 1.0f;
    if (wk == 0) {
#pragma unroll
        for (int q = 0; q < WK - 1; ++q)
#pragma unroll
            for (int n = 0; n < NW; ++n) acc[n] += red[q][n][lane];
        if (GAIN) {
            float t = 0.f;
#pragma unroll
            for (int q = 0; q < WK; ++q) t += ssum[q][col];
            rs = 1.0f / sqrtf(t / (float)K + a.eps);
        }
    }

    float best_v = -INFINITY;
    int best_i = 0x7fffffff;
    if (wk == 0 && tok) {
        float* yrow = a.y + (long)col * N;
        const int rbase = tile * TR + kq * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rbase + e;
            if (r >= N) break;
            const float v0 = acc[0][e] * rs * g16_scale<WT, EPI>(a, r, 0);
            if (EPI == EPI_STORE) {
                const bool q0 = r < a.seg_end[0], q1 = r < a.seg_end[1];
                const void* bsel = q0 ? a.bias[0] : (q1 ? a.bias[1] : a.bias[2]);
                const int base = q0 ? 0 : (q1 ? a.seg_end[0] : a.seg_end[1]);
                yrow[r] = bsel ? v0 + load_scalar<uint16_t>(bsel, r - base) : v0;
            } else if (EPI == EPI_RESID) {
                yrow[r] = yrow[r] + v0;
            } else if (EPI == EPI_SWIGLU) {
                yrow[r] = silu(v0) * (acc[NW - 1][e] * rs * g16_scale<WT, EPI>(a, r, NW - 1));
            } else {
                yrow[r] = v0;
                if (better(v0, r, best_v, best_i)) { best_v = v0; best_i = r; }
            }
        }
    }
    if (EPI == EPI_LOGITS) {           // wave 0 holds the block's 16 rows for every token
        argmax_across_rows(best_v, best_i);
        if (wk == 0 && lane < B) {
            a.part_val[(long)lane * gridDim.x + blockIdx.x] = best_v;
            a.part_idx[(long)lane * gridDim.x + blockIdx.x] = best_i;
        }
    }
}

// Normed products with more 16-row blocks than the chip has CUs (gate|up at the
// 0.5B shape: 304 blocks of gate and up rows). With one block per workgroup some
// CUs take two workgroups and others one, and every workgroup loads the whole
// activation (16 tokens x K float32) as well. Here the grid is two workgroups per
// CU and workgroup w takes rows [N w / G, N (w + 1) / G) in RB MFMA blocks of 16
// starting at its first row (rows past its range read the zero block), so every
// CU loads an equal share of the weights: the tokens' rows (zeros past B) and the
// gain go into LDS by DMA, ahead of the weights, then every wave issues its
// weight loads for all of its k-steps
// at once (RB blocks x NW matrices), waits only for the DMA, and runs each
// step's MFMAs as its weights land. The four waves split K and meet in LDS in a
// fixed order. LDS layout of the activation: one 128-byte line per (k-step s,
// token t) at (16 s + t) * 128, holding x[t][32 s .. 32 s + 32) as 16-byte granules
// with granule g at position g ^ sw(t), sw(t) = 2 ((t / 2) % 4): each DMA
// instruction then fetches 8 whole lines (a layout with 32-byte pieces of 32
// lines per instruction fetched every line twice), and the 8 lanes of a 16-byte
// LDS read phase (tokens 0..7 or 8..15) land on distinct banks.
template <typename WT, int EPI, int RB, int SPW, int NWV>
__global__ __launch_bounds__(NWV * 64) void gemm16_rows_kernel(GemvArgs a) {
    using WL = typename G16W<WT>::L;
    constexpr int NW = (EPI == EPI_SWIGLU) ? 2 : 1;
    constexpr int NLD = SPW * RB * NW;      // weight loads per lane
    static_assert(NLD <= 63, "vmcnt range");
    extern __shared__ __align__(16) char g16r_smem[];
    __shared__ float ssum[NWV][16];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int col = lane & 15, kq = lane >> 4;
    const int B = a.B, K = a.K, N = a.N;
    const int nsteps = K / 32;
    const int r0 = (int)((long)N * blockIdx.x / gridDim.x), r1 = (int)((long)N * (blockIdx.x + 1) / gridDim.x);
    float* xs = (float*)g16r_smem;
    const uint16_t* gs = (const uint16_t*)(g16r_smem + nsteps * 2048);

    // 1. activation and gain by DMA (each 1 KB instruction fills 32 units)
    {
        const uint32_t xl = lds_addr(xs), gl = lds_addr(gs);
        for (int c = wave; c < nsteps * 2; c += NWV) {   // lines (c / 2, 8 (c % 2) + lane / 8)
            const int t = (c & 1) * 8 + (lane >> 3);
            const int k = (c >> 1) * 32 + ((lane & 7) ^ (((t >> 1) & 3) << 1)) * 4;
            const void* src = t < B ? (const void*)(a.x + (long)t * K + k) : (const void*)kG16Zeros;
            lds_dma16(src, __builtin_amdgcn_readfirstlane(xl + c * 1024));
        }
        for (int c = wave; c < (K * 2 + 1023) / 1024; c += NWV) {
            const int e = min(c * 512 + lane * 8, K - 8);       // what lands past K is never read
            lds_dma16((const uint16_t*)a.gain + e, __builtin_amdgcn_readfirstlane(gl + c * 1024));
        }
    }
    // 2. this wave's weights: steps s0 + u (past s1, and rows past r1, read the zero block)
    const int s0 = wave * nsteps / NWV, s1 = (wave + 1) * nsteps / NWV;
    const WT* wrow[RB][NW];
    bool rok[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r = r0 + rb * 16 + col;
        rok[rb] = r < r1;
#pragma unroll
        for (int n = 0; n < NW; ++n) {
            const WT* p = (const WT*)a.w[n];
            if (r < r1) {
                if (EPI == EPI_SWIGLU) {
                    p = (const WT*)a.w[n] + (long)r * K;
                } else {
                    const bool q0 = r < a.seg_end[0], q1 = r < a.seg_end[1];
                    const void* w = q0 ? a.w[0] : (q1 ? a.w[1] : a.w[2]);
                    const int base = q0 ? 0 : (q1 ? a.seg_end[0] : a.seg_end[1]);
                    p = (const WT*)w + (long)(r - base) * K;
                }
            }
            wrow[rb][n] = p;
        }
    }
    WL wv[SPW][RB][NW];
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
        const int st = s0 + u;
        const bool ok = st < s1;
        const int k = ok ? st * 32 + kq * 8 : 0;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int n = 0; n < NW; ++n) wv[u][rb][n] = load_or_zero<WL>(wrow[rb][n] + k, ok && rok[rb]);
    }
    __builtin_amdgcn_s_waitcnt(wait_vm(NLD));   // this wave's DMA landed (loads retire in issue order)
    lds_barrier();                              // ... and every wave's
    if (a.zero_ptr && blockIdx.x == 0)
        for (int i = tid; i < a.zero_n; i += NWV * 64) a.zero_ptr[i] = 0u;

    // 3. MFMAs, step by step
    g16_f32x4 acc[RB][NW];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int n = 0; n < NW; ++n) acc[rb][n] = g16_f32x4{0.f, 0.f, 0.f, 0.f};
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
        const int st = s0 + u;
        if (st >= s1) break;
        const float* xp = xs + (st * 16 + col) * 32 + ((2 * kq) ^ (((col >> 1) & 3) << 1)) * 4;
        const float4 p0 = *(const float4*)xp, p1 = *(const float4*)(xp + 4);
        float gf[8];
        widen16(*(const uint4*)(gs + st * 32 + kq * 8), gf);
        float v[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ss += v[e] * v[e];
            v[e] *= gf[e];
        }
        uint4 hu, lu;
        split_hi_lo(v, hu, lu);
        const g16_bf16x8 bh = g16_frag(hu), bl = g16_frag(lu);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int n = 0; n < NW; ++n) {
                const g16_bf16x8 af = g16_frag(G16W<WT>::frag(wv[u][rb][n]));
                acc[rb][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bh, acc[rb][n], 0, 0, 0);
                acc[rb][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bl, acc[rb][n], 0, 0, 0);
            }
    }

    // 4. the waves' partial products and sums of squares meet in wave 0 (the
    //    activation's LDS holds the partials once every wave is done reading it)
    {
        const float t = strided_sum<16>(ss);
        if (lane < 16) ssum[wave][lane] = t;
    }
    g16_f32x4* red = (g16_f32x4*)g16r_smem;     // [NWV - 1][RB][NW][64]
    lds_barrier();
    if (wave > 0)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int n = 0; n < NW; ++n) red[(((wave - 1) * RB + rb) * NW + n) * kWave + lane] = acc[rb][n];
    lds_barrier();
    if (wave != 0 || col >= B) return;
#pragma unroll
    for (int q = 0; q < NWV - 1; ++q)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int n = 0; n < NW; ++n) acc[rb][n] += red[((q * RB + rb) * NW + n) * kWave + lane];
    float sst = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) sst += ssum[w][col];
    const float rs = 1.0f / sqrtf(sst / (float)K + a.eps);
    float* yrow = a.y + (long)col * N;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int rbase = r0 + rb * 16 + kq * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rbase + e;
            if (r >= r1) break;
            const float v0 = acc[rb][0][e] * rs * g16_scale<WT, EPI>(a, r, 0);
            if (EPI == EPI_SWIGLU) {
                yrow[r] = silu(v0) * (acc[rb][NW - 1][e] * rs * g16_scale<WT, EPI>(a, r, NW - 1));
            } else {
                const bool q0 = r < a.seg_end[0], q1 = r < a.seg_end[1];
                const void* bsel = q0 ? a.bias[0] : (q1 ? a.bias[1] : a.bias[2]);
                const int base = q0 ? 0 : (q1 ? a.seg_end[0] : a.seg_end[1]);
                yrow[r] = bsel ? v0 + load_scalar<uint16_t>(bsel, r - base) : v0;
            }
        }
    }
}

// Single-shot form for matrices whose K range fits the workgroup's registers:
// every wave issues all of its k-steps' loads (weights, activation, gain) at
// once, then runs its MFMAs. The grid is (groups of R 16-row blocks, K splits);
// K is cut into `splits` ranges of 32-wide steps and each range over the 4
// waves, at most SPW steps per wave; the R blocks of a group share each
// activation fragment. A residual product with several K ranges adds its
// partial sums into y with float atomics (each range's sum is complete and
// fixed; only the order of the final few additions varies from run to run);
// every other epilogue takes one range (splits = 1), so its output is formed
// once.
template <typename WT, int EPI, int SPW, int R>
__global__ __launch_bounds__(256) void gemm16_split_kernel(GemvArgs a, int splits) {
    using WL = typename G16W<WT>::L;
    constexpr bool GAIN = EPI != EPI_RESID;
    constexpr int NW = (EPI == EPI_SWIGLU) ? 2 : 1;
    constexpr int WK = 4;
    __shared__ float ssum[WK][16];
    __shared__ g16_f32x4 red[WK - 1][R][NW][kWave];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int col = lane & 15, kq = lane >> 4;
    const int B = a.B, K = a.K, N = a.N;
    const int tile = blockIdx.x, ks = blockIdx.y;
    const bool tok = col < B;
    const float* xrow = a.x + (long)(tok ? col : 0) * K;
    const uint16_t* gain = (const uint16_t*)a.gain;
    const int nsteps = (K + 31) / 32;
    const int a0 = ks * nsteps / splits, a1 = (ks + 1) * nsteps / splits;
    const int s0 = a0 + wave * (a1 - a0) / WK, s1 = a0 + (wave + 1) * (a1 - a0) / WK;

    const WT* wrow[R][NW];     // a row past N reads row 0 (masked)
    bool rok[R];
#pragma unroll
    for (int rb = 0; rb < R; ++rb) {
        const int r_own = (tile * R + rb) * 16 + col;
        rok[rb] = r_own < N;
#pragma unroll
        for (int n = 0; n < NW; ++n) {
            const WT* p = (const WT*)a.w[n];
            if (rok[rb]) {
                if (EPI == EPI_SWIGLU) {
                    p = (const WT*)a.w[n] + (long)r_own * K;
                } else {
                    const bool q0 = r_own < a.seg_end[0], q1 = r_own < a.seg_end[1];
                    const void* w = q0 ? a.w[0] : (q1 ? a.w[1] : a.w[2]);
                    const int base = q0 ? 0 : (q1 ? a.seg_end[0] : a.seg_end[1]);
                    p = (const WT*)w + (long)(r_own - base) * K;
                }
            }
            wrow[rb][n] = p;
        }
    }
    WL wv[SPW][R][NW];
    float4 x0[SPW], x1[SPW];
    uint4 gv[SPW];
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
        const int st = s0 + u;
        const int k = st * 32 + kq * 8;
        const bool ok = st < s1 && k < K;
        const int kc = ok ? k : 0;
#pragma unroll
        for (int rb = 0; rb < R; ++rb)
#pragma unroll
            for (int n = 0; n < NW; ++n) wv[u][rb][n] = load_or_zero<WL>(wrow[rb][n] + kc, ok && rok[rb]);
        x0[u] = load_or_zero<float4>(xrow + kc, ok && tok);
        x1[u] = load_or_zero<float4>(xrow + kc + 4, ok && tok);
        if (GAIN) gv[u] = load_or_zero<uint4>(gain + kc, ok);
    }
    float yv[R][4] = {};                      // single-range residual: y read with the loads
    if (EPI == EPI_RESID && splits == 1) {
        const float* yrow = a.y + (long)(tok ? col : 0) * N;
#pragma unroll
        for (int rb = 0; rb < R; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = (tile * R + rb) * 16 + kq * 4 + e;
                const float t = yrow[r < N ? r : 0];
                yv[rb][e] = (tok && r < N) ? t : 0.f;
            }
    }
    g16_f32x4 acc[R][NW];
#pragma unroll
    for (int rb = 0; rb < R; ++rb)
#pragma unroll
        for (int n = 0; n < NW; ++n) acc[rb][n] = g16_f32x4{0.f, 0.f, 0.f, 0.f};
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
        float v[8] = {x0[u].x, x0[u].y, x0[u].z, x0[u].w, x1[u].x, x1[u].y, x1[u].z, x1[u].w};
        if (GAIN) {
            float gf[8];
            widen16(gv[u], gf);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ss += v[e] * v[e];
                v[e] *= gf[e];
            }
        }
        uint4 hu, lu;
        split_hi_lo(v, hu, lu);
        const g16_bf16x8 bh = g16_frag(hu);
        const g16_bf16x8 bl = g16_frag(lu);
#pragma unroll
        for (int rb = 0; rb < R; ++rb)
#pragma unroll
            for (int n = 0; n < NW; ++n) {
                const g16_bf16x8 af = g16_frag(G16W<WT>::frag(wv[u][rb][n]));
                acc[rb][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bh, acc[rb][n], 0, 0, 0);
                acc[rb][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bl, acc[rb][n], 0, 0, 0);
            }
    }
    // the four waves' partial products and sums of squares meet in wave 0, in a fixed order
    if (GAIN) {
        const float t = strided_sum<16>(ss);
        if (lane < 16) ssum[wave][lane] = t;
    }
    if (wave > 0)
#pragma unroll
        for (int rb = 0; rb < R; ++rb)
#pragma unroll
            for (int n = 0; n < NW; ++n) red[wave - 1][rb][n][lane] = acc[rb][n];
    __syncthreads();
    if (wave != 0 || !tok) return;
#pragma unroll
    for (int q = 0; q < WK - 1; ++q)
#pragma unroll
        for (int rb = 0; rb < R; ++rb)
#pragma unroll
            for (int n = 0; n < NW; ++n) acc[rb][n] += red[q][rb][n][lane];
    float rs = 1.0f;
    if (GAIN) {
        float t = 0.f;
#pragma unroll
        for (int q = 0; q < WK; ++q) t += ssum[q][col];
        rs = 1.0f / sqrtf(t / (float)K + a.eps);
        if (EPI == EPI_STORE && a.ss_out) {   // partial form: this range's products and sum of squares
            if (tile == 0 && kq == 0) a.ss_out[ks * B + col] = t;
            float* prow = a.y + ((long)ks * B + col) * N;
            const int rbase = tile * 16 + kq * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (rbase + e < N) prow[rbase + e] = acc[0][0][e];
            return;
        }
    }
    float* yrow = a.y + (long)col * N;
#pragma unroll
    for (int rb = 0; rb < R; ++rb) {
        const int rbase = (tile * R + rb) * 16 + kq * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = rbase + e;
            if (r >= N) break;
            const float v0 = acc[rb][0][e] * rs * g16_scale<WT, EPI>(a, r, 0);
            if (EPI == EPI_STORE) {
                const bool q0 = r < a.seg_end[0], q1 = r < a.seg_end[1];
                const void* bsel = q0 ? a.bias[0] : (q1 ? a.bias[1] : a.bias[2]);
                const int base = q0 ? 0 : (q1 ? a.seg_end[0] : a.seg_end[1]);
                yrow[r] = bsel ? v0 + load_scalar<uint16_t>(bsel, r - base) : v0;
            } else if (EPI == EPI_RESID) {
                if (splits == 1) yrow[r] = yv[rb][e] + v0;
                else unsafeAtomicAdd(yrow + r, v0);
            } else {
                yrow[r] = silu(v0) * (acc[rb][NW - 1][e] * rs * g16_scale<WT, EPI>(a, r, NW - 1));
            }
        }
    }
}

// Shape of the single-shot form for a matrix, or spw = 0 when it does not apply.
// A long residual product (K >= 2048: down) takes groups of two row blocks and
// as many K ranges as keep the grid within one workgroup per CU, so each CU
// loads its share of the weights and the matching activation slice once (with
// one block per workgroup and 4-step ranges the down product at batch 16 put
// three workgroups, each loading twice its weight bytes of activation, on a CU).
// Other residual products take k-steps per wave by K (2) and as many K ranges as
// that needs; a normed product must fit one range of at most 8 steps per wave
// (K <= 1024).
struct G16Split { int spw, splits, r; };
static G16Split gemm16_split_shape(int K, int N, int epi) {
    const int nsteps = (K + 31) / 32;
    if (epi == EPI_RESID) {
        if (K >= 2048) {
            const int groups = (N + 31) / 32;
            const int splits = std::max(1, std::min(kG16Cus / groups, nsteps / 8));
            const int spw = ((nsteps + splits - 1) / splits + 3) / 4;
            if (spw >= 2 && spw <= 6) return {spw, splits, 2};
        }
        const int spw = K >= 2048 ? 4 : 2;
        return {spw, (nsteps + 4 * spw - 1) / (4 * spw), 1};
    }
    if ((epi == EPI_STORE || epi == EPI_SWIGLU) && nsteps <= 32) return {8, 1, 1};
    return {0, 0, 0};
}

// K ranges of a normed store product in the partial form (GemvArgs::ss_out): as
// many as keep one workgroup per CU (at most 3, at least 4 k-steps each), for
// the matrices the single-shot form takes; with one range per workgroup the
// q|k|v product at the 0.5B shape ran on 72 of the 256 CUs, each loading the
// whole activation.
int gemm16_store_splits(int K, int N) {
    const int nsteps = (K + 31) / 32, nb = (N + 15) / 16;
    if (nsteps > 32) return 1;
    const int s = std::min(kGemm16MaxStoreSplits, std::min(kG16Cus / nb, nsteps / 4));
    if (s < 2 || (nsteps + s - 1) / s > 16) return 1;
    return s;
}

// Blocks per workgroup of the multi-block normed kernel (gemm16_rows_kernel: two
// 4-wave workgroups per CU for bf16 rows, what the staged activation's LDS allows;
// against one 4-wave workgroup per CU with twice the rows, 9.7 -> 9.0 us for
// gate|up at batch 16 although each CU then stages the activation twice: the load
// path wants the extra waves; int8 rows one 8-wave workgroup per CU), or 0
// when it does not apply: gate|up with more rows than 16 per CU (up to 48 per
// workgroup), K a multiple of 32 up to 1024 with a per-wave step count it is
// built for
template <typename WT>
static int gemm16_rows_shape(int K, int N, int epi, int* spw) {
    constexpr int nwv = g16_rows_waves<WT>(), wgs = g16_rows_wgs<WT>();
    if (epi != EPI_SWIGLU || K % 32 || K > 1024 || N <= 16 * kG16Cus || N > 48 * wgs) return 0;
    *spw = (K / 32 + nwv - 1) / nwv;
    if (*spw != 2 && *spw != 4 && *spw != 7 && *spw != 8) return 0;
    return ((N + wgs - 1) / wgs + 15) / 16;
}

// K split into the fewest chunks of at most kG16Chunk, evened out (multiples of 32)
int gemm16_chunk(int K) {
    const int kp = (K + 31) & ~31;
    const int n = (kp + kG16Chunk - 1) / kG16Chunk;
    return ((kp + n - 1) / n + 31) & ~31;
}

// Many-row matrices (the lm_head) take wide tiles and a capped, grid-strided
// grid with the activation staged once per workgroup; the rest take one 16-row
// block per workgroup with the four waves splitting K and the activation read
// directly, which spreads even the smallest decode matrix (896 rows) over 56
// workgroups.
template <typename WT>
static hipError_t gemm16_dispatch(const GemvArgs& a, int epi, int grid_cap, int* grid_out, hipStream_t s) {
    const bool wide = a.N >= 16 * 2048;
    const bool gain_ok = epi == EPI_RESID ? a.gain == nullptr
                                          : (a.gain != nullptr && ((uintptr_t)a.gain & 15u) == 0);
    // the partial form exists only as the single-shot store product below
    if (a.ss_out && (epi != EPI_STORE || wide || !gain_ok || gemm16_store_splits(a.K, a.N) < 2))
        return hipErrorInvalidValue;
    if (!wide && gain_ok) {
        int rspw = 0;
        const int rb = gemm16_rows_shape<WT>(a.K, a.N, epi, &rspw);
        constexpr int nwv = g16_rows_waves<WT>();
        if (rb) {
            const int grid = g16_rows_wgs<WT>();     // rows [N w / grid, N (w + 1) / grid) each
            if (grid > grid_cap) return hipErrorInvalidValue;
            if (grid_out) *grid_out = grid;
            // activation and gain; the waves' partial products reuse it ([waves - 1][rb][2][64] x 16 bytes)
            const size_t shm = std::max((size_t)(a.K / 32) * 2048 + (size_t)((a.K * 2 + 1023) / 1024) * 1024,
                                        (size_t)rb * (nwv - 1) * 2 * 1024);
            auto go = [&](auto kern) {
                if (shm > 65536 &&
                    hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm) != hipSuccess)
                    return hipErrorInvalidValue;
                hipLaunchKernelGGL(kern, dim3(grid), dim3(nwv * 64), shm, s, a);
                return hipGetLastError();
            };
#define QD_G16R(RB)                                                                         \
            switch (rspw) {                                                                 \
                case 2: return go(gemm16_rows_kernel<WT, EPI_SWIGLU, RB, 2, nwv>);  \
                case 4: return go(gemm16_rows_kernel<WT, EPI_SWIGLU, RB, 4, nwv>);  \
                case 7: return go(gemm16_rows_kernel<WT, EPI_SWIGLU, RB, 7, nwv>);  \
                default: return go(gemm16_rows_kernel<WT, EPI_SWIGLU, RB, 8, nwv>); \
            }
            if (rb == 1) { QD_G16R(1) } else if (rb == 2) { QD_G16R(2) } else { QD_G16R(3) }
#undef QD_G16R
        }
        G16Split sp = gemm16_split_shape(a.K, a.N, epi);
        if (epi == EPI_RESID && a.deterministic) sp = {0, 0, 0};   // one K range: the direct form
        if (a.ss_out) {                      // partial form: K ranges of at most 4 steps per wave
            const int sn = gemm16_store_splits(a.K, a.N);
            sp = {((((a.K + 31) / 32) + sn - 1) / sn + 3) / 4, sn, 1};
        }
        if (sp.spw) {
            const int grid = ((a.N + 15) / 16 + sp.r - 1) / sp.r;
            if (grid > grid_cap) return hipErrorInvalidValue;
            if (grid_out) *grid_out = grid;
            const dim3 g2(grid, sp.splits);
#define QD_G16S(E, S, R) hipLaunchKernelGGL((gemm16_split_kernel<WT, E, S, R>), g2, dim3(256), 0, s, a, sp.splits)
            if (epi == EPI_RESID) {
                if (sp.r == 2) {
                    switch (sp.spw) {
                        case 2: QD_G16S(EPI_RESID, 2, 2); break;
                        case 3: QD_G16S(EPI_RESID, 3, 2); break;
                        case 4: QD_G16S(EPI_RESID, 4, 2); break;
                        case 5: QD_G16S(EPI_RESID, 5, 2); break;
                        default: QD_G16S(EPI_RESID, 6, 2); break;
                    }
                } else if (sp.spw == 4) {
                    QD_G16S(EPI_RESID, 4, 1);
                } else {
                    QD_G16S(EPI_RESID, 2, 1);
                }
            } else if (epi == EPI_STORE) {
                if (sp.spw <= 2) QD_G16S(EPI_STORE, 2, 1);
                else if (sp.spw == 3) QD_G16S(EPI_STORE, 3, 1);
                else if (sp.spw == 4) QD_G16S(EPI_STORE, 4, 1);
                else QD_G16S(EPI_STORE, 8, 1);
            } else {
                QD_G16S(EPI_SWIGLU, 8, 1);
            }
#undef QD_G16S
            return hipGetLastError();
        }
        const int grid = (a.N + 15) / 16;
        if (grid > grid_cap) return hipErrorInvalidValue;
        if (grid_out) *grid_out = grid;
        const bool deep = a.K >= 2048;       // long K: eight waves split it
#define QD_G16D(E)                                                                                       \
    if (deep) hipLaunchKernelGGL((gemm16_direct_kernel<WT, E, 8>), dim3(grid), dim3(512), 0, s, a);          \
    else hipLaunchKernelGGL((gemm16_direct_kernel<WT, E, 4>), dim3(grid), dim3(256), 0, s, a);
        switch (epi) {
            case EPI_STORE: QD_G16D(EPI_STORE) break;
            case EPI_RESID: QD_G16D(EPI_RESID) break;
            case EPI_SWIGLU: QD_G16D(EPI_SWIGLU) break;
            default: QD_G16D(EPI_LOGITS) break;
        }
#undef QD_G16D
        return hipGetLastError();
    }
    const size_t shm = (size_t)a.kt * 64;    // hi + lo, 16 tokens, 2 bytes each
    auto go = [&](auto kern, int tr) {
        const int tiles = (a.N + tr - 1) / tr;
        int grid = tiles < grid_cap ? tiles : grid_cap;
        // wide tiles: as many workgroups as the LDS lets the CUs hold at once (two each),
        // so each stages its activation once for several tiles (the lm_head at batch 16:
        // 67 -> 62 us against one workgroup per tile)
        if (tr == 128 && grid > 2 * kG16Cus) grid = 2 * kG16Cus;
        if (grid_out) *grid_out = grid;
        hipLaunchKernelGGL(kern, dim3(grid), dim3(256), shm, s, a);
        return hipGetLastError();
    };
    switch (epi) {
        case EPI_STORE: return wide ? go(gemm16_kernel<WT, EPI_STORE, 2, 1>, 128) : go(gemm16_kernel<WT, EPI_STORE, 1, 4>, 16);
        case EPI_RESID: return wide ? go(gemm16_kernel<WT, EPI_RESID, 2, 1>, 128) : go(gemm16_kernel<WT, EPI_RESID, 1, 4>, 16);
        case EPI_SWIGLU: return go(gemm16_kernel<WT, EPI_SWIGLU, 1, 4>, 16);
        default: return wide ? go(gemm16_kernel<WT, EPI_LOGITS, 2, 1>, 128) : go(gemm16_kernel<WT, EPI_LOGITS, 1, 4>, 16);
    }
}

hipError_t launch_gemm16(const GemvArgs& a, int w_type, int epi, int grid_cap, int* grid_out, hipStream_t s) {
    if (a.B < 1 || a.B > 16 || a.K % 8 || a.kt != gemm16_chunk(a.K)) return hipErrorInvalidValue;
    if (w_type == 2) {   // int8 rows: row scales (the partial form leaves them to its consumer)
        if (a.K % 16 || !a.wscale[0] || (epi == EPI_SWIGLU && !a.wscale[1])) return hipErrorInvalidValue;
        return gemm16_dispatch<int8_t>(a, epi, grid_cap, grid_out, s);
    }
    if (w_type != 1) return hipErrorInvalidValue;
    return gemm16_dispatch<uint16_t>(a, epi, grid_cap, grid_out, s);
}

}  // namespace qd
