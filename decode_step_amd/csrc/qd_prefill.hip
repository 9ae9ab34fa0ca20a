// Prefill block kernels for gfx950: the multi-token projections are dense
// contractions, so they run as bf16 MFMA GEMMs with float32 accumulation
// (v_mfma_f32_32x32x16_bf16); their activation operands are rounded to bf16
// at the points the block stores them (normed input, attention context,
// SwiGLU output). The residual stream stays float32.
//
// GEMM: C[M][N] (op)= A[M][K] . W[N][K]^T with both operands K-contiguous, as
// the weights are stored row-major [out][in]. A workgroup of 4 waves owns a
// 128 x BN tile (BN = 128 or 256; 2 x 2 waves of 64 x BN/2, each a grid of
// 32 x 32 MFMA tiles) and walks K in steps of 64. Tiles are staged in LDS
// (double buffered, rows padded against bank conflicts) from two register
// stages, so a tile's global loads are issued two K steps before its MFMAs:
// at M = 512 the loads come mostly from L2 and the other cache levels, and two
// steps of MFMAs cover that latency. The wider tile keeps the LDS traffic per
// MFMA below the LDS bandwidth (a 64 x 128 wave tile reads 6 operand fragments
// per 8 MFMAs). Workgroups are numbered so that the M tiles sharing one weight
// tile are dispatched together onto one XCD (dispatch goes round-robin over
// the 8 XCDs) and read it from that XCD's L2. Epilogues (Tang page, section
// 2.3): store float32 (q|k|v, plus bias), add into the float32 residual
// (o_proj, down), or silu(gate) * up rounded to bf16 with the gate and up
// tiles of the same columns held by the same lane (sibling reductions merged).
#include "qd_device.h"
#include "qd_launch.h"

namespace qd {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int kGemmBM = 128, kGemmBK = 64;

// silu(z) = z / (1 + e^-z) from the hardware exp2 and reciprocal (each within
// about an ulp), for results rounded to bf16; z -> -inf gives e^-z = inf and 0.
__device__ __forceinline__ float silu_fast(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}
constexpr int kGemmLdsRow = kGemmBK + 8;   // bf16 elements per padded LDS row (144 bytes)
constexpr int kXcds = 8;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// W row of output column n (stacked segments, as in the decode GEMV)
__device__ __forceinline__ const uint16_t* gemm_wrow(const GemmArgs& a, int n) {
    const bool s0 = n < a.seg_end[0], s1 = n < a.seg_end[1];
    const void* w = s0 ? a.w[0] : (s1 ? a.w[1] : a.w[2]);
    const int base = s0 ? 0 : (s1 ? a.seg_end[0] : a.seg_end[1]);
    return (const uint16_t*)w + (long)(n - base) * a.K;
}

template <int EPI, int BN>
__global__ __launch_bounds__(256) void mfma_gemm_kernel(GemmArgs a, int ntn, int ntm) {
    constexpr int BM = kGemmBM, BK = kGemmBK, LR = kGemmLdsRow;
    constexpr int TJ = BN / 64;                 // 32-column MFMA tiles per wave
    constexpr int AL = BM * BK / 8 / 256;       // 16-byte A chunks per thread per K step
    constexpr int WL = BN * BK / 8 / 256;       // 16-byte W chunks per thread per K step
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LR];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[2][BN * LR];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int M = a.M, K = a.K;

    // tile of this workgroup: the ntm M tiles of an N tile are consecutive on one XCD
    int tileN, tileM;
    {
        const int id = blockIdx.x;
        if (ntn % kXcds == 0) {
            const int xcd = id % kXcds, slot = id / kXcds;
            tileM = slot % ntm;
            tileN = (slot / ntm) * kXcds + xcd;
        } else {
            tileN = id % ntn;
            tileM = id / ntn;
        }
    }
    const int m0 = tileM * BM;

    // chunk q of this thread: row idx / 8, 16-byte column idx % 8 of the tile's K step;
    // rows outside the matrix read row 0 and are zeroed
    const uint16_t* a_src[AL];
    bool a_ok[AL];
    const uint16_t* w_src[WL];
    bool w_ok[WL];
#pragma unroll
    for (int q = 0; q < AL; ++q) {
        const int m = m0 + (tid + 256 * q) / 8;
        a_ok[q] = m < M;
        a_src[q] = (const uint16_t*)a.A + (long)(a_ok[q] ? m : 0) * K;
    }
#pragma unroll
    for (int q = 0; q < WL; ++q) {
        const int r = (tid + 256 * q) / 8;
        if (EPI == GEMM_SWIGLU) {
            const int hcol = tileN * (BN / 2) + (r % (BN / 2));
            w_ok[q] = hcol < a.N;
            w_src[q] = (const uint16_t*)a.w[r / (BN / 2)] + (long)(w_ok[q] ? hcol : 0) * K;
        } else {
            const int n = tileN * BN + r;
            w_ok[q] = n < a.N;
            w_src[q] = w_ok[q] ? gemm_wrow(a, n) : (const uint16_t*)a.w[0];
        }
    }
    const int kc = (tid & 7) * 8;
    struct Stage {
        uint4 a[AL];
        uint4 w[WL];
    };
    auto load = [&](Stage& st, int kt) {
        const int k = kt * BK + kc;
        const bool kok = k < K;
        const int kk = kok ? k : 0;
#pragma unroll
        for (int q = 0; q < AL; ++q) {
            const uint4 v = *(const uint4*)(a_src[q] + kk);
            st.a[q] = (kok && a_ok[q]) ? v : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < WL; ++q) {
            const uint4 v = *(const uint4*)(w_src[q] + kk);
            st.w[q] = (kok && w_ok[q]) ? v : make_uint4(0, 0, 0, 0);
        }
    };
    auto store = [&](int buf, const Stage& st) {
#pragma unroll
        for (int q = 0; q < AL; ++q) *(uint4*)&As[buf][((tid + 256 * q) / 8) * LR + kc] = st.a[q];
#pragma unroll
        for (int q = 0; q < WL; ++q) *(uint4*)&Ws[buf][((tid + 256 * q) / 8) * LR + kc] = st.w[q];
    };

    f32x16_t acc[2][TJ];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // lane's operand row within a 32-row MFMA tile and k offset within a 16-wide step
    const int lrow = lane & 31, lk = (lane >> 5) * 8;
    auto wtile_row = [&](int j) {
        if (EPI == GEMM_SWIGLU)   // j < TJ/2: gate rows, else up rows, of h-columns wn*BN/4 ..
            return (j < TJ / 2 ? 0 : BN / 2) + wn * (BN / 4) + (j % (TJ / 2)) * 32 + lrow;
        return wn * (BN / 2) + j * 32 + lrow;
    };
    auto compute = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < BK; ks += 16) {
            bf16x8_t av[2], bv[TJ];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                av[i] = as_bf16x8(*(const uint4*)&As[buf][(wm * 64 + i * 32 + lrow) * LR + ks + lk]);
#pragma unroll
            for (int j = 0; j < TJ; ++j) bv[j] = as_bf16x8(*(const uint4*)&Ws[buf][wtile_row(j) * LR + ks + lk]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
    };

    // pipeline: LDS[kt & 1] holds step kt; register stages hold steps kt + 1 and kt + 2
    const int nk = (K + BK - 1) / BK;
    Stage s0, s1;
    load(s0, 0);
    if (nk > 1) load(s1, 1);
    store(0, s0);
    if (nk > 2) load(s0, 2);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
        compute(0);                       // step kt (even)
        if (kt + 1 < nk) store(1, s1);
        if (kt + 3 < nk) load(s1, kt + 3);
        __syncthreads();
        if (kt + 1 >= nk) break;
        compute(1);                       // step kt + 1
        if (kt + 2 < nk) store(0, s0);
        if (kt + 4 < nk) load(s0, kt + 4);
        __syncthreads();
    }

    // epilogue: lane holds column lrow of each 32 x 32 tile and rows
    // (e / 4) * 8 + (lane / 32) * 4 + (e % 4)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int m = m0 + wm * 64 + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
            if (m >= M) continue;
            if (EPI == GEMM_SWIGLU) {
#pragma unroll
                for (int j = 0; j < TJ / 2; ++j) {
                    const int hcol = tileN * (BN / 2) + wn * (BN / 4) + j * 32 + lrow;
                    if (hcol < a.N) {
                        const float g = acc[i][j][e], u = acc[i][j + TJ / 2][e];
                        ((uint16_t*)a.C)[(long)m * a.ldc + hcol] = f32_to_bf16(silu(g) * u);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < TJ; ++j) {
                    const int n = tileN * BN + wn * (BN / 2) + j * 32 + lrow;
                    if (n >= a.N) continue;
                    float* cp = (float*)a.C + (long)m * a.ldc + n;
                    if (EPI == GEMM_STORE) {
                        const bool s0b = n < a.seg_end[0], s1b = n < a.seg_end[1];
                        const void* bsel = s0b ? a.bias[0] : (s1b ? a.bias[1] : a.bias[2]);
                        const int base = s0b ? 0 : (s1b ? a.seg_end[0] : a.seg_end[1]);
                        *cp = bsel ? acc[i][j][e] + bf16_to_f32(((const uint16_t*)bsel)[n - base]) : acc[i][j][e];
                    } else {
                        *cp = *cp + acc[i][j][e];
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The same GEMM with the tiles fed by LDS DMA (global_load_lds_dwordx4): each
// lane's 16 bytes go from memory straight into LDS at the wave's base + 16 x
// lane, no register staging. At M = 512 the tiles come from L2 and the caches
// behind it with a latency of a microsecond or two, so what bounds a CU is the
// bytes it has in flight: K steps of 32 go through a ring of NS LDS stages
// (the LDS holds about 144 KB of them) and each step's loads are issued
// NS - 1 steps ahead. The DMA writes rows of 32 bf16 (64 bytes) back to back,
// so the rows are swizzled instead of padded: 16-byte chunk c of row r sits at
// position c ^ ((r / 4) % 4), which keeps 16 consecutive rows on distinct
// banks for the fragment reads; lane L of a load instruction (16 rows) reads
// chunk (L % 4) ^ ((L / 16) % 4) of row L / 4. Completion is counted with
// s_waitcnt vmcnt before one barrier per step, which also frees the stage read
// in the previous step. Rows outside the matrix read row 0 (their outputs are
// dropped); K must be a multiple of 32 (the DMA cannot zero a tail).
constexpr int kDmaBK = 32;
constexpr int kDmaLds = 147456;    // bytes of LDS the ring may take

template <int BM, int BN>
constexpr int dma_stages() { return kDmaLds / ((BM + BN) * kDmaBK * 2); }

// BM x BN tile, 2 x (NWV/2) waves of BM/2 x BN/(NWV/2) (TI x TJ MFMA tiles of 32 x 32)
template <int EPI, int BM, int BN, int NWV = 4>
__global__ __launch_bounds__(64 * NWV) void mfma_gemm_dma_kernel(GemmArgs a, int ntn, int ntm, int splits) {
    constexpr int BK = kDmaBK, RB = BK * 2;       // row bytes
    constexpr int WGN = NWV / 2;                  // waves along N
    constexpr int TI = BM / 64, TJ = BN / (32 * WGN);
    constexpr int QA = BM / (16 * NWV), QW = BN / (16 * NWV);   // load instructions (16 rows each) per wave per step
    constexpr int NQ = QA + QW;
    constexpr int NS = dma_stages<BM, BN>();
    constexpr int SA = BM * RB, SB = (BM + BN) * RB;            // A part, whole stage
    static_assert(NS >= 3 && (NS - 2) * NQ <= 63, "ring depth");
    __shared__ __attribute__((aligned(16))) uint8_t ring[NS * SB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int M = a.M, K = a.K;

    // tile and K range of this workgroup; the M tiles of an N tile (and K range) are
    // consecutive on one XCD
    int tileN, tileM, split;
    {
        const int id = blockIdx.x;
        if (ntn % kXcds == 0) {
            const int xcd = id % kXcds, slot = id / kXcds;
            tileM = slot % ntm;
            split = (slot / ntm) % splits;
            tileN = (slot / ntm / splits) * kXcds + xcd;
        } else {
            tileN = id % ntn;
            tileM = (id / ntn) % ntm;
            split = id / ntn / ntm;
        }
    }
    const int m0 = tileM * BM;

    // source of lane's chunk in load instruction q: row 16 (wave Q + q) + lane / 4,
    // chunk (lane % 4) ^ ((lane / 16) % 4)
    const int lchunk = ((lane & 3) ^ ((lane >> 4) & 3)) * 8;
    const uint16_t* asrc[QA];
    const uint16_t* wsrc[QW];
#pragma unroll
    for (int q = 0; q < QA; ++q) {
        const int m = m0 + 16 * (wave * QA + q) + (lane >> 2);
        asrc[q] = (const uint16_t*)a.A + (long)(m < M ? m : 0) * K + lchunk;
    }
#pragma unroll
    for (int q = 0; q < QW; ++q) {
        const int r = 16 * (wave * QW + q) + (lane >> 2);
        const uint16_t* p;
        if (EPI == GEMM_SWIGLU) {
            const int hcol = tileN * (BN / 2) + (r % (BN / 2));
            p = (const uint16_t*)a.w[r / (BN / 2)] + (long)(hcol < a.N ? hcol : 0) * K;
        } else {
            const int n = tileN * BN + r;
            p = n < a.N ? gemm_wrow(a, n) : (const uint16_t*)a.w[0];
        }
        wsrc[q] = p + lchunk;
    }
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(qd_lds_void*)ring;
    const int nk_all = K / BK;
    const int kt_begin = split * nk_all / splits;
    const int nk = (split + 1) * nk_all / splits - kt_begin;   // K steps of this range
    auto issue = [&](int stage, int kt) {
        const int k0 = (kt_begin + kt) * BK;
        const uint32_t base = ring_lds + stage * SB;
#pragma unroll
        for (int q = 0; q < QA; ++q)
            lds_dma16(asrc[q] + k0, __builtin_amdgcn_readfirstlane(base + 16 * (wave * QA + q) * RB));
#pragma unroll
        for (int q = 0; q < QW; ++q)
            lds_dma16(wsrc[q] + k0, __builtin_amdgcn_readfirstlane(base + SA + 16 * (wave * QW + q) * RB));
    };

    f32x16_t acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    const int lrow = lane & 31, lhalf = lane >> 5;
    auto wtile_row = [&](int j) {
        if (EPI == GEMM_SWIGLU)
            return (j < TJ / 2 ? 0 : BN / 2) + wn * (BN / (2 * WGN)) + (j % (TJ / 2)) * 32 + lrow;
        return wn * (BN / WGN) + j * 32 + lrow;
    };
    auto frag = [&](const uint8_t* base, int row, int ks) {
        const int c = 2 * ks + lhalf;
        return as_bf16x8(*(const uint4*)(base + row * RB + ((c ^ ((row >> 2) & 3)) << 4)));
    };
    auto compute = [&](const uint8_t* st) {
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8_t av[TI], bv[TJ];
#pragma unroll
            for (int i = 0; i < TI; ++i) av[i] = frag(st, wm * (BM / 2) + i * 32 + lrow, ks);
#pragma unroll
            for (int j = 0; j < TJ; ++j) bv[j] = frag(st + SA, wtile_row(j), ks);
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
    };
    // Every step issues exactly NQ loads per lane (past the end it reloads the last
    // step into the free stage, unused), so one constant wait count serves all steps.
    if (nk > 0) {
#pragma unroll
        for (int t = 0; t < NS - 1; ++t) issue(t, t < nk ? t : nk - 1);
        for (int t = 0; t < nk; ++t) {
            __builtin_amdgcn_s_waitcnt(wait_vm((NS - 2) * NQ));   // step t landed (this lane's part)
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);               // this lane's reads of step t-1 done
            __builtin_amdgcn_s_barrier();                         // ... and every lane's
            const int tn = t + NS - 1;
            issue((t + NS - 1) % NS, tn < nk ? tn : nk - 1);      // into the stage of step t-1
            compute(ring + (t % NS) * SB);
        }
        __builtin_amdgcn_s_waitcnt(wait_vm(0));   // no DMA into LDS outlives the loop
    }

#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int m = m0 + wm * (BM / 2) + i * 32 + (e >> 2) * 8 + lhalf * 4 + (e & 3);
            if (m >= M) continue;
            if (EPI == GEMM_SWIGLU) {
#pragma unroll
                for (int j = 0; j < TJ / 2; ++j) {
                    const int hcol = tileN * (BN / 2) + wn * (BN / (2 * WGN)) + j * 32 + lrow;
                    if (hcol < a.N) {
                        const float g = acc[i][j][e], u = acc[i][j + TJ / 2][e];
                        ((uint16_t*)a.C)[(long)m * a.ldc + hcol] = f32_to_bf16(silu(g) * u);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < TJ; ++j) {
                    const int n = tileN * BN + wn * (BN / WGN) + j * 32 + lrow;
                    if (n >= a.N) continue;
                    float* cp = (float*)a.C + (long)m * a.ldc + n;
                    float v = acc[i][j][e];
                    if (EPI == GEMM_STORE && split == 0) {
                        const bool s0b = n < a.seg_end[0], s1b = n < a.seg_end[1];
                        const void* bsel = s0b ? a.bias[0] : (s1b ? a.bias[1] : a.bias[2]);
                        const int base = s0b ? 0 : (s1b ? a.seg_end[0] : a.seg_end[1]);
                        if (bsel) v += bf16_to_f32(((const uint16_t*)bsel)[n - base]);
                    }
                    if (splits > 1) unsafeAtomicAdd(cp, v);
                    else if (EPI == GEMM_STORE) *cp = v;
                    else *cp = *cp + v;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Wide-tile GEMM (M > 128, K a multiple of 64). What bounds a GEMM of 512 rows
// here is the bytes each CU pulls from L2: about 50-60 GB/s per CU whatever the
// number of CUs loading (measured), so the tile is the one that spends the
// fewest bytes per MAC with one tile per CU: 256 x BN (BN = 192 or 128), four
// waves of 128 x BN/2 with their accumulators in AGPRs. K steps of 64 make each
// row's share of a step one whole 128-byte line (rows of 64 bytes measured 2.5x
// slower to load); they go through an LDS ring (2 stages at BN = 192, 3 at 128)
// by LDS DMA, rows XOR-swizzled in 16-byte chunks (chunk c of row r at
// c ^ ((r / 2) % 8), which keeps 16 consecutive rows on distinct banks for the
// fragment reads). Within a step the fragments of sub-step ks + 1 are read
// while the MFMAs of sub-step ks run; the one barrier per step sits after the
// first MFMAs of the last sub-step, so the next step's loads and first reads
// overlap the rest.
//
// Products too small for one tile per CU cut K into `splits` ranges; each range
// writes its float32 partial product to its own slab C + split * M * ldc (plain
// stores) and the consumer adds the slabs (no atomics: about 2.4e11 float
// atomics per second would cost more than the product). SwiGLU tiles hold BN/2
// gate and the matching BN/2 up columns; the up waves pass their accumulators
// to the gate waves through LDS, and all four waves form silu(g) * u for half of
// the rows at a time and store bf16 rows 16 bytes per lane.
constexpr int kV2BM = 256, kV2BK = 64, kV2RB = 128;
constexpr int kV2Lds = 159744;
constexpr int kV2MinWgs = 240;

template <int BN>
constexpr int v2_stages() { return kV2Lds / ((kV2BM + BN) * kV2RB); }
__device__ __forceinline__ int v2_swz(int r) { return (r >> 1) & 7; }

template <int EPI, int BN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_gemm_v2_kernel(GemmArgs a, int ntn, int ntm, int splits) {
    constexpr int BM = kV2BM, BK = kV2BK, RB = kV2RB, NWV = 4;
    constexpr int WM = BM / 2, WN = BN / 2, TI = WM / 32, TJ = WN / 32;
    constexpr int RPI = 8;                                      // rows per DMA instruction
    constexpr int QA = BM / (RPI * NWV), QW = BN / (RPI * NWV);
    constexpr int NQ = QA + QW;
    constexpr int SA = BM * RB, SB = (BM + BN) * RB;
    constexpr int NS = v2_stages<BN>();
    constexpr int KS = BK / 16;
    constexpr int NR = TI + TJ;                                 // fragment reads per sub-step
    constexpr int PRE = 2;                                      // last-sub-step MFMAs before the barrier
    constexpr int TP = BN + 8;                                  // floats per row of the SwiGLU tile
    static_assert(NS >= 2 && (NS - 1) * NQ <= 63, "ring depth");
    static_assert(EPI != GEMM_SWIGLU || 128 * TP * 4 <= NS * SB, "SwiGLU tile");
    __shared__ __attribute__((aligned(16))) uint8_t ring[NS * SB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int M = a.M, K = a.K;

    // tile and K range; the M tiles of one (N tile, K range) are consecutive on one XCD
    int tileN, tileM, split;
    {
        const int id = blockIdx.x, combos = ntn * splits;
        int c;
        if (combos % kXcds == 0) {
            const int slot = id / kXcds;
            tileM = slot % ntm;
            c = (slot / ntm) * kXcds + id % kXcds;
        } else {
            tileM = (id / combos) % ntm;
            c = id % combos;
        }
        tileN = c / splits;
        split = c % splits;
    }
    const int m0 = tileM * BM;

    // lane's source in DMA instruction q: row RPI (wave Q + q) + lane / 8, logical
    // chunk (lane % 8) ^ swz(row), landing at physical chunk lane % 8
    const uint16_t* asrc[QA];
    const uint16_t* wsrc[QW];
#pragma unroll
    for (int q = 0; q < QA; ++q) {
        const int r = RPI * (wave * QA + q) + (lane >> 3);
        const int m = m0 + r;
        asrc[q] = (const uint16_t*)a.A + (long)(m < M ? m : 0) * K + (((lane & 7) ^ v2_swz(r)) * 8);
    }
#pragma unroll
    for (int q = 0; q < QW; ++q) {
        const int r = RPI * (wave * QW + q) + (lane >> 3);
        const uint16_t* p;
        if (EPI == GEMM_SWIGLU) {
            const int f = tileN * (BN / 2) + (r % (BN / 2));
            p = (const uint16_t*)a.w[r / (BN / 2)] + (long)(f < a.N ? f : 0) * K;
        } else {
            const int n = tileN * BN + r;
            p = n < a.N ? gemm_wrow(a, n) : (const uint16_t*)a.w[0];
        }
        wsrc[q] = p + (((lane & 7) ^ v2_swz(r)) * 8);
    }
    const uint32_t ring_lds = lds_addr(ring);
    const int nk_all = K / BK;
    const int kt_begin = split * nk_all / splits;
    const int nk = (split + 1) * nk_all / splits - kt_begin;   // >= 1: the plan keeps splits <= nk_all
    if (nk < 1) return;
    auto issue = [&](int buf, int kt) {
        const int k0 = (kt_begin + kt) * BK;
        const uint32_t base = ring_lds + buf * SB;
#pragma unroll
        for (int q = 0; q < QA; ++q)
            lds_dma16(asrc[q] + k0, __builtin_amdgcn_readfirstlane(base + RPI * (wave * QA + q) * RB));
#pragma unroll
        for (int q = 0; q < QW; ++q)
            lds_dma16(wsrc[q] + k0, __builtin_amdgcn_readfirstlane(base + SA + RPI * (wave * QW + q) * RB));
    };
    // one DMA instruction of step kt: d < QA an A row group, else a W row group
    auto issue_one = [&](int buf, int kt, int d) {
        const int k0 = (kt_begin + kt) * BK;
        const uint32_t base = ring_lds + buf * SB;
        if (d < QA) lds_dma16(asrc[d] + k0, __builtin_amdgcn_readfirstlane(base + RPI * (wave * QA + d) * RB));
        else lds_dma16(wsrc[d - QA] + k0, __builtin_amdgcn_readfirstlane(base + SA + RPI * (wave * QW + d - QA) * RB));
    };

    const int lrow = lane & 31, lhalf = lane >> 5;
    f32x16_t acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    auto frag = [&](const uint8_t* base, int row, int ks) {
        const int c = 2 * ks + lhalf;
        return as_bf16x8(*(const uint4*)(base + row * RB + ((c ^ v2_swz(row)) << 4)));
    };
    bf16x8_t fa[2][TI], fb[2][TJ];
    auto rd = [&](int buf, int ks, bf16x8_t (&av)[TI], bf16x8_t (&bv)[TJ]) {
        const uint8_t* st = ring + buf * SB;
#pragma unroll
        for (int i = 0; i < TI; ++i) av[i] = frag(st, wm * WM + i * 32 + lrow, ks);
#pragma unroll
        for (int j = 0; j < TJ; ++j) bv[j] = frag(st + SA, wn * WN + j * 32 + lrow, ks);
    };
    auto mm = [&](const bf16x8_t (&av)[TI], const bf16x8_t (&bv)[TJ], int lo, int hi) {
#pragma unroll
        for (int q = 0; q < TI * TJ; ++q)
            if (q >= lo && q < hi)
                acc[q / TJ][q % TJ] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[q / TJ], bv[q % TJ], acc[q / TJ][q % TJ], 0, 0, 0);
    };

    // Ring: steps 0 .. NS-1 issued up front; at step t's barrier every wave has read
    // stage t (its fragments are in registers) and the DMA of step t + NS takes its
    // buffer (right after the barrier, or spread over step t + 1, below). Past the
    // end the last step is reloaded (unused), so every step issues NQ loads per lane
    // and one wait count serves all.
#pragma unroll
    for (int st = 0; st < NS; ++st) issue(st, st < nk ? st : nk - 1);
    __builtin_amdgcn_s_waitcnt(wait_vm((NS - 1) * NQ));
    __builtin_amdgcn_s_barrier();
    rd(0, 0, fa[0], fb[0]);
    // SPREAD (three or more stages): the stage freed at step t - 1's barrier is
    // refilled during step t, one DMA instruction after every second MFMA of the
    // first KS - 1 sub-steps. Issued back to back after the barrier, a step's DMA
    // held each wave's issue for about 0.3 us (the texture unit takes the CU's 1 KB
    // instructions one after another) with the matrix core idle; spread, that work
    // overlaps the MFMAs, and the data is needed only NS - 1 steps later. The wait
    // at the end of step t still leaves exactly one slot's loads outstanding (the
    // ones issued during step t).
    constexpr bool SPREAD = NS >= 3 && (KS - 1) * (TI * TJ / 2) >= NQ;
    for (int t = 0; t < nk; ++t) {
        const int buf = t % NS;
        if constexpr (SPREAD) {
            const bool pend = t >= 1;                                   // a stage to refill
            const int pbuf = (t + NS - 1) % NS;
            const int pkt = t - 1 + NS < nk ? t - 1 + NS : nk - 1;    // past the end: the last step again (unused)
#pragma unroll
            for (int ks = 0; ks < KS - 1; ++ks) {
                rd(buf, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int q = 0; q < TI * TJ; ++q) {
                    mm(fa[ks & 1], fb[ks & 1], q, q + 1);
                    if (q & 1) {
                        const int dd = ks * (TI * TJ / 2) + (q >> 1);
                        if (dd < NQ && pend) issue_one(pbuf, pkt, dd);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < KS - 1; ++ks) {
                rd(buf, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
                mm(fa[ks & 1], fb[ks & 1], 0, TI * TJ);
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
                }
                __builtin_amdgcn_sched_group_barrier(0x008, TI * TJ - NR, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        mm(fa[(KS - 1) & 1], fb[(KS - 1) & 1], 0, PRE);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(wait_vm((NS - 2) * NQ));     // step t + 1 landed (this lane's part)
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);                 // this lane's reads of step t done
        __builtin_amdgcn_s_barrier();                           // ... and every lane's
        if constexpr (!SPREAD) issue(buf, t + NS < nk ? t + NS : nk - 1);
        __builtin_amdgcn_sched_barrier(0);
        rd((t + 1) % NS, 0, fa[0], fb[0]);                      // past the last step: unused
        mm(fa[(KS - 1) & 1], fb[(KS - 1) & 1], PRE, TI * TJ);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if constexpr (TI * TJ - PRE - NR > 0) __builtin_amdgcn_sched_group_barrier(0x008, TI * TJ - PRE - NR, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(wait_vm(0));   // no DMA into LDS outlives the loop
    __syncthreads();

    if (EPI == GEMM_SWIGLU) {
        // rows 64 r .. 64 r + 63 of each wave's 128 go through T[128][TP]: gate
        // columns [0, WN), up columns [WN, 2 WN); then 8 h columns per item
        float* T = (float*)ring;
        constexpr int CPR = WN / 8;
        const int f0 = tileN * WN;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                for (int j = 0; j < TJ; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        T[(wm * 64 + ii * 32 + (e >> 2) * 8 + lhalf * 4 + (e & 3)) * TP + wn * WN + j * 32 + lrow] =
                            acc[2 * r + ii][j][e];
            lds_barrier();
            static_assert(128 * CPR % 256 == 0, "whole items per thread");
#pragma unroll
            for (int it = 0; it < 128 * CPR / 256; ++it) {   // unrolled: the LDS reads of all items go out together
                const int item = tid + it * 256;
                const int R = item / CPR, c = item - R * CPR;
                const int m = m0 + (R >> 6) * WM + r * 64 + (R & 63);
                const int f = f0 + c * 8;
                const float4* gp = (const float4*)(T + R * TP + c * 8);
                const float4* up = (const float4*)(T + R * TP + WN + c * 8);
                const float4 g0 = gp[0], g1 = gp[1], u0 = up[0], u1 = up[1];
                const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
                const float u[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
                float hv[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) hv[k] = silu_fast(g[k]) * u[k];
                if (m < M && f < a.N) *(uint4*)((uint16_t*)a.C + (long)m * a.ldc + f) = pack16<uint16_t>(hv);
            }
            lds_barrier();
        }
    } else {
        float* out = (float*)a.C + (long)split * M * a.ldc;
        if (m0 + BM <= M && (tileN + 1) * BN <= a.N) {
            // whole tile in range: one lane base, row offsets uniform over the wave
            // (per-element bounds checks and 64-bit index arithmetic had made this
            // epilogue instruction-bound: ~10 instructions per stored value)
            float* base = out + (long)(m0 + wm * WM + lhalf * 4) * a.ldc + tileN * BN + wn * WN + lrow;
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float* row = base + (long)(i * 32 + (e >> 2) * 8 + (e & 3)) * a.ldc;
#pragma unroll
                    for (int j = 0; j < TJ; ++j) row[j * 32] = acc[i][j][e];
                }
        } else {
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int m = m0 + wm * WM + i * 32 + (e >> 2) * 8 + lhalf * 4 + (e & 3);
                    if (m >= M) continue;
#pragma unroll
                    for (int j = 0; j < TJ; ++j) {
                        const int n = tileN * BN + wn * WN + j * 32 + lrow;
                        if (n < a.N) out[(long)m * a.ldc + n] = acc[i][j][e];
                    }
                }
        }
    }
}

// Wide-tile plan: use it when M > 128 and K % 64 == 0 (SwiGLU also needs N and
// ldc multiples of 8 for its 16-byte stores). BN = 192 unless the columns fit
// 128-wide tiles better; K ranges double while the tiles fill fewer than about
// one workgroup per CU and each range keeps at least 4 steps.
struct V2Plan { bool use; int bn, splits; };
static V2Plan v2_plan(int M, int N, int K, int ldc, int epi) {
    if (M <= 128 || K % kV2BK != 0 || K < kV2BK) return {false, 0, 0};
    const int ntm = (M + kV2BM - 1) / kV2BM;
    if (epi == GEMM_SWIGLU) {
        if (N % 8 || ldc % 8) return {false, 0, 0};
        const int bn = (N % 96 != 0 && N % 64 == 0) ? 128 : 192;
        return {true, bn, 1};
    }
    const int bn = (N % 192 != 0 && (N % 128 == 0 || N < 192)) ? 128 : 192;
    const long tiles = (long)ntm * ((N + bn - 1) / bn);
    const int nk = K / kV2BK;
    int s = 1;
    while (s < 8 && tiles * s < kV2MinWgs && nk / (2 * s) >= 4) s *= 2;
    return {true, bn, s};
}

int mfma_gemm_slabs(int M, int N, int K, int epi) {
    if (epi == GEMM_SWIGLU || N % 4) return 0;
    const V2Plan p = v2_plan(M, N, K, N, epi);
    return p.use ? p.splits : 0;
}

hipError_t launch_mfma_gemm_slabs(const GemmArgs& a, int slabs, hipStream_t s) {
    const V2Plan p = v2_plan(a.M, a.N, a.K, a.ldc, GEMM_STORE);
    if (!p.use || slabs != p.splits || a.ldc < a.N) return hipErrorInvalidValue;
    const int ntm = (a.M + kV2BM - 1) / kV2BM, ntn = (a.N + p.bn - 1) / p.bn;
    const dim3 grid(ntm * ntn * p.splits);
    if (p.bn == 192) hipLaunchKernelGGL((mfma_gemm_v2_kernel<GEMM_STORE, 192>), grid, dim3(256), 0, s, a, ntn, ntm, p.splits);
    else hipLaunchKernelGGL((mfma_gemm_v2_kernel<GEMM_STORE, 128>), grid, dim3(256), 0, s, a, ntn, ntm, p.splits);
    return hipGetLastError();
}

// x[i] += sum over s < nslab of part[s * stride + i], n a multiple of 4: the K
// ranges of a residual product added into the float32 residual stream.
__global__ __launch_bounds__(256) void add_slabs_kernel(float* x, const float* part, int nslab, long stride, long n4) {
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long)gridDim.x * 256) {
        float4 v = ((const float4*)x)[i];
        for (int sl = 0; sl < nslab; ++sl) {
            const float4 p = ((const float4*)(part + sl * stride))[i];
            v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
        }
        ((float4*)x)[i] = v;
    }
}

hipError_t launch_add_slabs(float* x, const float* part, int nslab, long stride, long n, hipStream_t s) {
    if (n % 4 || stride % 4 || nslab < 1) return hipErrorInvalidValue;
    long blocks = (n / 4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(add_slabs_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, part, nslab, stride, n / 4);
    return hipGetLastError();
}

constexpr int kGemmTargetWgs = 256;
#ifndef QD_GEMM256_WAVES
#define QD_GEMM256_WAVES 8     // waves of a 256 x 256 tile (2 x 4, 128 x 64 each)
#endif

// K a multiple of 32: LDS DMA kernel. Tile choice (measured at M = 512 on 256
// CUs): SwiGLU takes 256 x 256 tiles (two 128 x 128 operand blocks per wave
// halve the LDS and memory bytes per MFMA) and cannot split K (its epilogue is
// not linear). q|k|v takes 128 x 128 tiles (192 workgroups). The residual
// products take 128 x 128 tiles and at most two K ranges whose partial
// products meet in the float32 residual through float atomics: the atomics
// (about 2.4e11 per second) cost more than the arithmetic they spread past two
// ranges, and 256 x 256 tiles would need eight. Other K: the register-staged
// kernel with 128 x 128 tiles.
struct GemmPlan { int bm, bn, splits; };
static GemmPlan gemm_plan(const GemmArgs& a, int epi) {
    if (a.K % kDmaBK != 0) return {kGemmBM, 128, 1};
    if (epi == GEMM_SWIGLU) return {a.M <= 128 ? 128 : 256, 256, 1};
    if (epi == GEMM_STORE) return {128, 128, 1};
    const int nk = a.K / kDmaBK;
    const int tiles = ((a.M + 127) / 128) * ((a.N + 127) / 128);
    int s = 1;
    while (s < 2 && (long)tiles * (s + 1) <= kGemmTargetWgs && nk / (s + 1) >= 8) ++s;
    return {128, 128, s};
}
int mfma_gemm_splits(const GemmArgs& a, int epi) { return gemm_plan(a, epi).splits; }

hipError_t launch_mfma_gemm(const GemmArgs& a, int epi, int splits, hipStream_t s) {
    if (a.M < 1 || a.N < 1 || a.K < 8 || a.K % 8) return hipErrorInvalidValue;
    if (epi == GEMM_SWIGLU) {
        const V2Plan p = v2_plan(a.M, a.N, a.K, a.ldc, GEMM_SWIGLU);
        if (p.use) {
            if (splits > 1) return hipErrorInvalidValue;
            const int ntm = (a.M + kV2BM - 1) / kV2BM, ntn = (a.N + p.bn / 2 - 1) / (p.bn / 2);
            if (p.bn == 192) hipLaunchKernelGGL((mfma_gemm_v2_kernel<GEMM_SWIGLU, 192>), dim3(ntm * ntn), dim3(256), 0, s, a, ntn, ntm, 1);
            else hipLaunchKernelGGL((mfma_gemm_v2_kernel<GEMM_SWIGLU, 128>), dim3(ntm * ntn), dim3(256), 0, s, a, ntn, ntm, 1);
            return hipGetLastError();
        }
    }
    const GemmPlan pl = gemm_plan(a, epi);
    if (splits <= 0) splits = pl.splits;
    if (splits != pl.splits) return hipErrorInvalidValue;
    if (a.K % kDmaBK != 0) {
        const int ntm = (a.M + kGemmBM - 1) / kGemmBM;
        const int cols = epi == GEMM_SWIGLU ? 64 : 128, ntn = (a.N + cols - 1) / cols;
        switch (epi) {
            case GEMM_STORE: hipLaunchKernelGGL((mfma_gemm_kernel<GEMM_STORE, 128>), dim3(ntn * ntm), dim3(256), 0, s, a, ntn, ntm); break;
            case GEMM_RESID: hipLaunchKernelGGL((mfma_gemm_kernel<GEMM_RESID, 128>), dim3(ntn * ntm), dim3(256), 0, s, a, ntn, ntm); break;
            default: hipLaunchKernelGGL((mfma_gemm_kernel<GEMM_SWIGLU, 128>), dim3(ntn * ntm), dim3(256), 0, s, a, ntn, ntm); break;
        }
        return hipGetLastError();
    }
    const int ntm = (a.M + pl.bm - 1) / pl.bm;
    const int cols = epi == GEMM_SWIGLU ? pl.bn / 2 : pl.bn, ntn = (a.N + cols - 1) / cols;
    const dim3 grid(ntn * ntm * splits);
#define QD_GEMM_DMA(E)                                                                                                  \
    if (pl.bm == 256) hipLaunchKernelGGL((mfma_gemm_dma_kernel<E, 256, 256, QD_GEMM256_WAVES>), grid, dim3(64 * QD_GEMM256_WAVES), 0, s, a, ntn, ntm, splits); \
    else if (pl.bn == 256) hipLaunchKernelGGL((mfma_gemm_dma_kernel<E, 128, 256>), grid, dim3(256), 0, s, a, ntn, ntm, splits); \
    else hipLaunchKernelGGL((mfma_gemm_dma_kernel<E, 128, 128>), grid, dim3(256), 0, s, a, ntn, ntm, splits);
    switch (epi) {
        case GEMM_STORE: QD_GEMM_DMA(GEMM_STORE) break;
        case GEMM_RESID: QD_GEMM_DMA(GEMM_RESID) break;
        default: QD_GEMM_DMA(GEMM_SWIGLU) break;
    }
#undef QD_GEMM_DMA
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row RMSNorm to a bf16 GEMM operand: n = bf16(x * (1/sqrt(sum(x^2)/D + eps)) * g)
// (nanocompile page, phase 1: sum then divide, eps inside the root). With
// x_res set, the input row (bf16 or float) is also widened into the float32
// residual stream.
template <typename WT, int NSL>
__global__ __launch_bounds__(256) void prefill_norm_kernel(PrefillNormArgs a) {
    // One row per workgroup; each thread holds chunks of 8 consecutive elements
    // (16-byte loads and stores), the row read once.
    constexpr int kMaxChunks = 8;           // D <= 8 * 8 * 256 = 16384
    __shared__ float wsum[4];
    const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int D = a.D, nch = D / 8;
    if (a.zero) {   // this row's share of the buffer to clear
        const long per = (a.zero_n + gridDim.x - 1) / gridDim.x;
        const long z0 = (long)row * per, z1 = min(a.zero_n, z0 + per);
        for (long i = z0 + tid; i < z1; i += 256) a.zero[i] = 0.f;
    }
    float v[kMaxChunks][8];
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        const int ch = tid + 256 * c;
        if (ch >= nch) break;
        const long off = (long)row * D + 8 * ch;
        if (a.x_bf16) {
            widen16(*(const uint4*)((const uint16_t*)a.x_bf16 + off), v[c]);
        } else {
            const float4 p0 = *(const float4*)(a.x_f32 + off), p1 = *(const float4*)(a.x_f32 + off + 4);
            v[c][0] = p0.x; v[c][1] = p0.y; v[c][2] = p0.z; v[c][3] = p0.w;
            v[c][4] = p1.x; v[c][5] = p1.y; v[c][6] = p1.z; v[c][7] = p1.w;
#pragma unroll
            for (int sl = 0; sl < NSL; ++sl) {   // K ranges of the product feeding the residual (all loads issued together)
                const float* q = a.part + sl * a.slab_stride + off;
                const float4 q0 = *(const float4*)q, q1 = *(const float4*)(q + 4);
                v[c][0] += q0.x; v[c][1] += q0.y; v[c][2] += q0.z; v[c][3] += q0.w;
                v[c][4] += q1.x; v[c][5] += q1.y; v[c][6] += q1.z; v[c][7] += q1.w;
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += v[c][e] * v[c][e];
        if (a.x_res) {
            *(float4*)(a.x_res + off) = make_float4(v[c][0], v[c][1], v[c][2], v[c][3]);
            *(float4*)(a.x_res + off + 4) = make_float4(v[c][4], v[c][5], v[c][6], v[c][7]);
        }
    }
    ss = group_sum<kWave>(ss);
    if (lane == 0) wsum[wave] = ss;
    __syncthreads();
    const float r = 1.0f / sqrtf((wsum[0] + wsum[1] + wsum[2] + wsum[3]) / (float)D + a.eps);
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        const int ch = tid + 256 * c;
        if (ch >= nch) break;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = v[c][e] * r * load_scalar<WT>(a.gain, 8 * ch + e);
        *(uint4*)(a.out + (long)row * D + 8 * ch) = pack16<uint16_t>(o);
    }
}

hipError_t launch_prefill_norm(const PrefillNormArgs& a, int w_is_bf16, hipStream_t s) {
    const int nsl = a.part ? a.nslab : 0;
#define QD_PN(WT)                                                                                  \
    switch (nsl) {                                                                                 \
        case 0: hipLaunchKernelGGL((prefill_norm_kernel<WT, 0>), dim3(a.rows), dim3(256), 0, s, a); break; \
        case 1: hipLaunchKernelGGL((prefill_norm_kernel<WT, 1>), dim3(a.rows), dim3(256), 0, s, a); break; \
        case 2: hipLaunchKernelGGL((prefill_norm_kernel<WT, 2>), dim3(a.rows), dim3(256), 0, s, a); break; \
        case 4: hipLaunchKernelGGL((prefill_norm_kernel<WT, 4>), dim3(a.rows), dim3(256), 0, s, a); break; \
        case 8: hipLaunchKernelGGL((prefill_norm_kernel<WT, 8>), dim3(a.rows), dim3(256), 0, s, a); break; \
        default: return hipErrorInvalidValue;                                                      \
    }
    if (w_is_bf16) { QD_PN(uint16_t) } else { QD_PN(float) }
#undef QD_PN
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per (row i, head): optional per-head q/k RMSNorm, RoPE at position start + i
// (half-split, angle in double reduced mod 2*pi, sine/cosine in float), q to a
// float32 buffer, k and v stored into the cache slot of that position in the
// cache type (keys rotated once, on insert -- nanoinfer page, phase 4). One
// workgroup per row (its angles formed once); lane i rotates the pair
// (i, i + hd/2) of every 16th head.
constexpr int kRopeWaves = 16;
template <typename WT, typename KVT, int NSL>
__global__ __launch_bounds__(64 * kRopeWaves) void prefill_rope_append_kernel(PrefillRopeArgs a) {
    // One workgroup per row: the row's q|k|v into LDS (the sum of its NSL K-range
    // slabs plus the bias, or the one buffer when NSL = 0; 16-byte loads, all of a
    // thread's issued together) while the row's hd/2 angles are formed, then each
    // wave takes every 16th head, lane i the pair (i, i + hd/2).
    __shared__ float2 tab[64];
    extern __shared__ __align__(16) float rowv[];   // [(Hq + 2 Hkv) hd]
    const int row = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, i = tid & 63;
    const int hd = a.hd, half = hd >> 1;
    const int p = a.start + row;
    if (p < 0 || p >= a.capacity) return;
    const int qkvr = (a.Hq + 2 * a.Hkv) * hd;
    {
        const float* rowp = a.qkv + (long)row * qkvr;
        for (int i4 = tid; i4 < qkvr / 4; i4 += 64 * kRopeWaves) {
            float4 v = *(const float4*)(rowp + 4 * i4);
#pragma unroll
            for (int sl = 1; sl < NSL; ++sl) {
                const float4 t = *(const float4*)(rowp + sl * a.slab_stride + 4 * i4);
                v.x += t.x; v.y += t.y; v.z += t.z; v.w += t.w;
            }
            if (NSL > 0) {   // the segment's bias (segments end on multiples of 4)
                const int col = 4 * i4;
                const bool s0 = col < a.seg_end[0], s1 = col < a.seg_end[1];
                const void* b = s0 ? a.bias[0] : (s1 ? a.bias[1] : a.bias[2]);
                if (b) {
                    const int bc = col - (s0 ? 0 : (s1 ? a.seg_end[0] : a.seg_end[1]));
                    v.x += load_scalar<WT>(b, bc); v.y += load_scalar<WT>(b, bc + 1);
                    v.z += load_scalar<WT>(b, bc + 2); v.w += load_scalar<WT>(b, bc + 3);
                }
            }
            *(float4*)(rowv + 4 * i4) = v;
        }
    }
    if (tid < half) {
        const double inv = pow((double)a.theta, -2.0 * (double)tid / (double)hd);
        double ang = (double)p * inv;
        const double two_pi = 6.283185307179586476925286766559;
        ang -= two_pi * rint(ang / two_pi);
        float sn, cs;
        sincosf((float)ang, &sn, &cs);
        tab[tid] = make_float2(cs, sn);
    }
    __syncthreads();
    const bool act = i < half;
    const float2 cs = tab[act ? i : 0];
    const int page_id = a.block_table[p / a.page];
    auto qkv_at = [&](int col) -> float { return rowv[col]; };
    for (int h = wave; h < a.Hq + a.Hkv; h += kRopeWaves) {
        const bool is_q = h < a.Hq;
        const int c0 = is_q ? h * hd : a.Hq * hd + (h - a.Hq) * hd;
        float lo = act ? qkv_at(c0 + i) : 0.f, hi = act ? qkv_at(c0 + i + half) : 0.f;
        if (a.qk_norm) {
            const float ss = group_sum<kWave>(lo * lo + hi * hi);
            const float r = 1.0f / sqrtf(ss / (float)hd + a.eps);
            const void* g = is_q ? a.q_norm : a.k_norm;
            if (act) {
                lo = lo * r * load_scalar<WT>(g, i);
                hi = hi * r * load_scalar<WT>(g, i + half);
            }
        }
        if (!act) continue;
        const float lo2 = lo * cs.x - hi * cs.y, hi2 = hi * cs.x + lo * cs.y;
        if (is_q) {
            float* q = a.q_out + ((long)row * a.Hq + h) * hd;
            q[i] = lo2;
            q[i + half] = hi2;
        } else {
            const int g = h - a.Hq;
            if (page_id < 0 || page_id >= a.num_pages) continue;
            const long off = (((long)page_id * a.Hkv + g) * a.page + (p % a.page)) * hd;
            const int vcol = (a.Hq + a.Hkv) * hd + g * hd;
            KVT* kc = (KVT*)a.k_cache + off;
            KVT* vc = (KVT*)a.v_cache + off;
            kc[i] = from_f32<KVT>(lo2);
            kc[i + half] = from_f32<KVT>(hi2);
            vc[i] = from_f32<KVT>(qkv_at(vcol + i));
            vc[i + half] = from_f32<KVT>(qkv_at(vcol + i + half));
        }
    }
}

template <typename WT, typename KVT>
static hipError_t rope_append_nsl(const PrefillRopeArgs& a, size_t shm, hipStream_t s) {
    const dim3 grid(a.rows), block(64 * kRopeWaves);
    switch (a.nslab) {
        case 0: hipLaunchKernelGGL((prefill_rope_append_kernel<WT, KVT, 0>), grid, block, shm, s, a); break;
        case 1: hipLaunchKernelGGL((prefill_rope_append_kernel<WT, KVT, 1>), grid, block, shm, s, a); break;
        case 2: hipLaunchKernelGGL((prefill_rope_append_kernel<WT, KVT, 2>), grid, block, shm, s, a); break;
        case 4: hipLaunchKernelGGL((prefill_rope_append_kernel<WT, KVT, 4>), grid, block, shm, s, a); break;
        case 8: hipLaunchKernelGGL((prefill_rope_append_kernel<WT, KVT, 8>), grid, block, shm, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_prefill_rope_append(const PrefillRopeArgs& a, int w_is_bf16, int kv_is_bf16, hipStream_t s) {
    // the row's q|k|v stays in LDS: (Hq + 2 Hkv) hd floats, at most 64 KB
    const size_t shm = (size_t)(a.Hq + 2 * a.Hkv) * a.hd * sizeof(float);
    if (shm > 65536 || a.hd % 4) return hipErrorInvalidValue;
    if (w_is_bf16) return kv_is_bf16 ? rope_append_nsl<uint16_t, uint16_t>(a, shm, s) : rope_append_nsl<uint16_t, float>(a, shm, s);
    return kv_is_bf16 ? rope_append_nsl<float, uint16_t>(a, shm, s) : rope_append_nsl<float, float>(a, shm, s);
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
