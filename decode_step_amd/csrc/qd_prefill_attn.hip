// Causal prefill attention on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Query row i of the block (position start + i) attends over cached positions
// 0 .. start + i (the block's own K/V are already in the cache). A workgroup
// takes 32 query rows of one query head; its 4 waves take every 4th block of
// 32 keys, each keeping a running softmax (m, l) per row and rescaling its
// output on the way, and the four states merge at the end (Tang page, section
// 2.2: online softmax, the monoid that lets the key range be cut anywhere;
// section 2.5: the causal row sees keys up to its own position). Query tiles
// with the most keys are dispatched first. Query head h reads KV head h / group.
//
// Products, transposed so that a lane holds one query's scores: S^T = K Q^T with
// K straight from the paged cache as the A operand (a lane's 16-byte fragment is
// 8 consecutive dims of one key row) and Q^T as the B operand; the lane (query
// r32, half hi) then holds its query's scores for 16 of the block's 32 keys, so
// the block's row maximum is a max over registers and one swap with the other
// half, and the exponentials are formed once each. Those 16 probabilities are
// directly the lane's B fragments of P^T for O^T += V^T P^T (the contraction runs
// over keys in the order the lane holds them: 4 keys of each 8), and the V^T
// fragment (A operand) reads the same keys, two runs of 4, from the wave's LDS
// tile, which V is written into transposed ([dim][key]) as it is loaded. The
// matrix cores take bf16; q and P are float32 here, so each is split into bf16
// hi + lo and multiplied twice (K and V are bf16 in the cache and exact), which
// keeps the products at float32 accuracy. The next key block's K/V loads are
// issued as soon as the current block's K and V have been used (after S^T and the
// V transpose), so they land while its softmax and P V run.
//
// The output is the attention context rounded to bf16, the operand of the
// o_proj matrix product.
#include "qd_device.h"
#include "qd_launch.h"

namespace qd {

typedef __attribute__((ext_vector_type(8))) __bf16 pa_bf16x8;
typedef __attribute__((ext_vector_type(16))) float pa_f32x16;

constexpr int kPaRows = 32;   // query rows per wavefront
constexpr int kPaKeys = 32;   // keys per block

__device__ __forceinline__ pa_bf16x8 pa_frag(uint4 v) { return __builtin_bit_cast(pa_bf16x8, v); }

constexpr int kPaWaves = 4;   // waves per workgroup, each over every 4th key block

// The row a query past the block's rows reads instead of q (static device memory,
// zero from load time, never written; one head of the widest head dim).
__device__ __align__(16) float kPaZeros[128];

template <int HD>
__global__ __launch_bounds__(64 * kPaWaves) __attribute__((amdgpu_waves_per_eu(2))) void prefill_attn_mfma_kernel(PrefillAttnArgs a) {
    constexpr int NWV = kPaWaves;
    constexpr int KS = HD / 16;          // 16-dim slices of the score product
    constexpr int CB = HD / 32;          // 32-dim column blocks of the output
    constexpr int VL = HD / 16;          // 16-byte V loads per lane: 4 keys x DPL dims
    constexpr int DPL = HD / 8;          // dims of each of its 4 keys a lane loads
    constexpr int VTS = kPaKeys + 4;     // bf16 per transposed V row (8-byte aligned; 36 spreads the
                                         // 8 dim groups of a write over the banks)
    constexpr int VT_B = HD * VTS * 2;   // one wave's tile
    constexpr int TILES = NWV * VT_B;
    constexpr int MERGE = (NWV - 1) * kPaRows * HD * 4 + NWV * kPaRows * 8;
    __shared__ __align__(16) char smem[TILES > MERGE ? TILES : MERGE];
    __shared__ uint4 qfr[2][KS][64];     // Q fragments (bf16 hi, lo) of every lane, shared by the waves

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r32 = lane & 31, hi = lane >> 5;
    uint16_t (*vt)[VTS] = (uint16_t (*)[VTS])(smem + wave * VT_B);
    // (query tile, head) by rank of work (rank k: tile ntile-1 - k/Hq, head k%Hq): the
    // first half of the dispatch takes the heaviest ranks in order and the second
    // half the lightest first, so the two workgroups that share a CU (one from each
    // half, when the whole grid is resident) sum to about the mean work
    int q0, h;
    {
        const int ntile = gridDim.x, total = ntile * a.Hq, half = (total + 1) / 2;
        const int id = blockIdx.y * ntile + blockIdx.x;
        const int rank = id < half ? id : total - 1 - (id - half);
        q0 = (ntile - 1 - rank / a.Hq) * kPaRows;
        h = rank % a.Hq;
    }
    const int G = a.Hq / a.Hkv, g = h / G;
    const int N = a.rows, start = a.start;
    const int last_row = min(q0 + kPaRows, N) - 1;
    const int t_max = start + last_row;              // the last key any row of this tile sees
    const int nkb = t_max / kPaKeys + 1;
    const int* bt = a.block_table;

    // Page ids go out first, as the addresses of the first K/V loads: key 0's (the
    // fallback row) and the page of this lane's key (kb*32 + r32, clamped to t_max)
    // in the wave's first two blocks; each later block's id is loaded one block
    // ahead of its K/V loads, so no block waits for a page-table round trip.
    auto page_of = [&](int kb) -> int {
        const int t = kb * kPaKeys + r32;
        return bt[(t <= t_max ? t : t_max) / a.page];
    };
    const int pg_key0 = bt[0];
    int pg_cur = page_of(wave < nkb ? wave : 0);
    int pg_nxt = page_of(wave + NWV < nkb ? wave + NWV : 0);

    // Q fragments: row q0 + r32, dims 16 kk + 8 hi .. + 7, as bf16 hi + lo, formed
    // once (wave w takes slices kk of its quarter) and read from LDS at each block
    // (registers are the limit here); a row past N reads the zero row, so no load
    // waits on a select before the next one goes out
    {
        constexpr int KW = (KS + NWV - 1) / NWV;
        const int row = q0 + r32;
        const float* qp = row < N ? a.q + ((long)row * a.Hq + h) * HD + 8 * hi : kPaZeros + 8 * hi;
        float4 u[KW], w[KW];
#pragma unroll
        for (int i = 0; i < KW; ++i) {
            const int kk = wave * KW + i < KS ? wave * KW + i : KS - 1;
            u[i] = *(const float4*)(qp + 16 * kk);
            w[i] = *(const float4*)(qp + 16 * kk + 4);
        }
#pragma unroll
        for (int i = 0; i < KW; ++i) {
            const int kk = wave * KW + i;
            if (kk >= KS) break;
            const float v[8] = {u[i].x, u[i].y, u[i].z, u[i].w, w[i].x, w[i].y, w[i].z, w[i].w};
            uint4 qh, ql;
            split_hi_lo(v, qh, ql);
            qfr[0][kk][lane] = qh;
            qfr[1][kk][lane] = ql;
        }
    }

    // Lane's key of block kb: kb*32 + r32, in page pg. Keys past t_max, or whose page
    // is not in the pool, read the row of key 0 (a written row) and are masked out.
    const int pg_fallback = (pg_key0 >= 0 && pg_key0 < a.num_pages) ? pg_key0 : 0;
    auto key_row = [&](int kb, int pg, bool& ok) -> long {
        const int t = kb * kPaKeys + r32;
        ok = t <= t_max && pg >= 0 && pg < a.num_pages;
        const int pgu = ok ? pg : pg_fallback;
        const int tt = ok ? t : 0;
        return (((long)pgu * a.Hkv + g) * a.page + (tt % a.page)) * HD;
    };
    struct Blk {
        uint4 k[KS];
        uint4 v[VL];
        bool ok;
    };
    // K: lane's key r32, dims 16 kk + 8 hi (its A fragments). V: lane's keys 4 vq .. + 3
    // (one page: 4 | page), dims vdg*DPL .. + DPL - 1, so that the transposed tile takes
    // 4 keys of a dim per 8-byte write; the page of key 4 vq is lane 4 vq's.
    const int vq = lane & 7, vdg = lane >> 3;
    const long vrow0 = (((long)pg_fallback * a.Hkv + g) * a.page) * HD;   // key 0's row
    auto load = [&](Blk& b, int kb, int pg) {
        const long off = key_row(kb, pg, b.ok);
        const uint16_t* kp = (const uint16_t*)a.k_cache + off + 8 * hi;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) b.k[kk] = *(const uint4*)(kp + 16 * kk);
        const int pgv = __shfl(pg, 4 * vq);
        const bool pgok = pgv >= 0 && pgv < a.num_pages;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = kb * kPaKeys + 4 * vq + i;
            const long vo = (t <= t_max && pgok) ? (((long)pgv * a.Hkv + g) * a.page + (t % a.page)) * HD : vrow0;
            const uint16_t* vp = (const uint16_t*)a.v_cache + vo + vdg * DPL;
#pragma unroll
            for (int c = 0; c < DPL / 8; ++c) b.v[i * (DPL / 8) + c] = *(const uint4*)(vp + 8 * c);
        }
    };
    // this wave's LDS tiles are its own: ordering them needs only the wave itself
    auto wave_sync = [&]() {
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
    };

    // Lane (query r32, half hi) keeps the running softmax of its query: m in base-2
    // units (the same in both halves), l its half's share of the sum.
    float m = -INFINITY, l = 0.f;
    pa_f32x16 o[CB];                  // O^T: dims cb*32 + (e/4)*8 + hi*4 + e%4 of query r32
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[cb][e] = 0.f;
    const float scale2 = a.scale * 1.4426950408889634f;
    const int lim = min(start + q0 + r32, t_max);     // the last key query r32 sees

    // one block: V^T into LDS and S^T = K Q^T, then the next block's loads go into the
    // same registers (they land while this block's softmax and O^T += V^T P^T run)
    auto compute = [&](Blk& b, int kb, int next) {
        // V block into LDS, transposed: vt[dim][key], the lane's 4 keys of a dim packed
        // into one 8-byte write
#pragma unroll
        for (int c = 0; c < DPL / 8; ++c) {
            const uint4 k0 = b.v[c], k1 = b.v[DPL / 8 + c], k2 = b.v[2 * (DPL / 8) + c], k3 = b.v[3 * (DPL / 8) + c];
            const uint32_t w0[4] = {k0.x, k0.y, k0.z, k0.w}, w1[4] = {k1.x, k1.y, k1.z, k1.w};
            const uint32_t w2[4] = {k2.x, k2.y, k2.z, k2.w}, w3[4] = {k3.x, k3.y, k3.z, k3.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {   // word e holds dims 2e (low half) and 2e + 1
                const int d = vdg * DPL + 8 * c + 2 * e;
                *(uint2*)&vt[d][4 * vq] = make_uint2((w0[e] & 0xffffu) | (w1[e] << 16), (w2[e] & 0xffffu) | (w3[e] << 16));
                *(uint2*)&vt[d + 1][4 * vq] = make_uint2((w0[e] >> 16) | (w1[e] & 0xffff0000u), (w2[e] >> 16) | (w3[e] & 0xffff0000u));
            }
        }
        // S^T of the 32 x 32 tile: K as the A operand, Q^T as the B operand; the lane
        // then holds query r32's scores of keys (e/4)*8 + hi*4 + e%4
        pa_f32x16 sacc;
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa_frag(b.k[kk]), pa_frag(qfr[0][kk][lane]), sacc, 0, 0, 0);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa_frag(b.k[kk]), pa_frag(qfr[1][kk][lane]), sacc, 0, 0, 0);
        }
        // which of the block's keys were loaded from a real row: lane r32 loaded key
        // r32 (bit r32), while the scores this lane holds are other keys'
        const uint32_t okm = (uint32_t)__ballot(b.ok);
        if (next >= 0) {
            // the next block's K/V (its page id came a block ago), then the page id of
            // the block after it: issued in that order, nothing waits for the fresh one
            load(b, next, pg_nxt);
            pg_nxt = page_of(next + NWV < nkb ? next + NWV : 0);
        }
        // online softmax of the query over the block (Tang page, section 2.2), scores
        // in base-2 units so that e^(s - m) is the hardware exp2 of s' - m'
        float sv[16];
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int kk = (e >> 2) * 8 + hi * 4 + (e & 3);
            const bool valid = ((okm >> kk) & 1u) && kb * kPaKeys + kk <= lim;
            sv[e] = valid ? sacc[e] * scale2 : -INFINITY;
            mx = fmaxf(mx, sv[e]);
        }
        mx = swap32_max(mx);                          // with the other half's 16 keys
        const float mn = fmaxf(m, mx);
        const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mn);
        float pv[16];
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            pv[e] = sv[e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[e] - mn);
            psum += pv[e];
        }
        l = l * alpha + psum;
        m = mn;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[cb][e] *= alpha;
        // P^T as B fragments straight from the registers: k-step ks takes e = 8 ks .. + 7,
        // i.e. keys 16 ks + {hi*4 .. +3, 8 + hi*4 .. +3}; split hi + lo
        uint4 ph[2], pl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = pv[8 * ks + j];
            split_hi_lo(v, ph[ks], pl[ks]);
        }
        wave_sync();                                  // V^T written by every lane of the wave
        // O^T += V^T P^T: the V^T fragment of dim cb*32 + r32 takes the same keys, two
        // runs of 4 from the LDS tile
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const uint16_t* row = &vt[cb * 32 + r32][16 * ks + 4 * hi];
                const uint2 v0 = *(const uint2*)row;
                const uint2 v1 = *(const uint2*)(row + 8);
                const uint4 vf = make_uint4(v0.x, v0.y, v1.x, v1.y);
                o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa_frag(vf), pa_frag(ph[ks]), o[cb], 0, 0, 0);
                o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa_frag(vf), pa_frag(pl[ks]), o[cb], 0, 0, 0);
            }
        wave_sync();   // the tile is rewritten by this wave's next block
    };

    // this wave's blocks: wave, wave + NWV, ...; the first one's loads go out before
    // the wait for the Q fragments
    Blk b;
    int kb = wave;
    if (kb < nkb) load(b, kb, pg_cur);
    __syncthreads();                                  // the Q fragments are in LDS
    while (kb < nkb) {
        const int next = kb + NWV;
        compute(b, kb, next < nkb ? next : -1);
        kb = next;
    }
    l = swap32_sum(l);                                // the query's whole sum in both halves

    // the waves' (m, l, o) meet in LDS (the online-softmax merge); wave c (c < CB)
    // forms context = O / L in bf16 for the 32-dim column block c from its own o and
    // the other waves' (one wave doing all four blocks was a serial tail of ~1 us)
    __syncthreads();                                  // every wave is done with its tiles
    float* mo = (float*)smem;                         // [CB][NWV-1][32][32]: block c's partials of the other waves
    float2* mlw = (float2*)(mo + CB * (NWV - 1) * kPaRows * 32);   // [NWV][32] (m, l)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        if (cb == wave) continue;                     // uniform over the wave
        const int slot = wave < cb ? wave : wave - 1;
        float* dp = mo + ((cb * (NWV - 1) + slot) * kPaRows + r32) * 32 + hi * 4;
#pragma unroll
        for (int e = 0; e < 16; ++e) dp[(e >> 2) * 8 + (e & 3)] = o[cb][e];
    }
    if (hi == 0) mlw[wave * kPaRows + r32] = make_float2(m, l);
    __syncthreads();
    if (wave >= CB) return;
    const int row = q0 + r32;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWV; ++w) M = fmaxf(M, mlw[w * kPaRows + r32].x);   // finite: wave 0 holds key 0
    float wt[NWV];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
        const float2 ml = mlw[w * kPaRows + r32];
        wt[w] = ml.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml.x - M);   // a wave without keys: 0
        L = fmaf(ml.y, wt[w], L);
    }
    if (row >= N) return;
    const float inv = 1.0f / L;
    uint16_t* dst = a.out + (long)row * a.Hq * HD + h * HD;
#pragma unroll
    for (int c = 0; c < CB; ++c) {
        if (c != wave) continue;                      // uniform; c is a constant below
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {              // dims c*32 + e4*8 + hi*4 .. + 3
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = 4 * e4 + i, dl = e4 * 8 + hi * 4 + i;
                float t = o[c][e] * wt[c];
#pragma unroll
                for (int sl = 0; sl < NWV - 1; ++sl)
                    t = fmaf(mo[((c * (NWV - 1) + sl) * kPaRows + r32) * 32 + dl], wt[sl < c ? sl : sl + 1], t);
                v[i] = t * inv;
            }
            const uint2 pk = make_uint2(f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3]));
            *(uint2*)(dst + c * 32 + e4 * 8 + hi * 4) = pk;
        }
    }
}

hipError_t launch_prefill_attn_mfma(const PrefillAttnArgs& a, hipStream_t s) {
    if (a.rows < 1 || a.Hq % a.Hkv || a.page < 1 || (a.hd != 64 && a.hd != 128)) return hipErrorInvalidValue;
    const dim3 grid((a.rows + kPaRows - 1) / kPaRows, a.Hq);
    if (a.hd == 64) hipLaunchKernelGGL((prefill_attn_mfma_kernel<64>), grid, dim3(64 * kPaWaves), 0, s, a);
    else hipLaunchKernelGGL((prefill_attn_mfma_kernel<128>), grid, dim3(64 * kPaWaves), 0, s, a);
    return hipGetLastError();
}

}  // namespace qd
