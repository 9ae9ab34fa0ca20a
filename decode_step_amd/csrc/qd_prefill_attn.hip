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
// Products: S = Q K^T with Q as the A operand (rows = queries) and K straight
// from the paged cache as the B operand (a lane's 16-byte fragment is 8
// consecutive dims of one key row); O += P V with P as the A operand and V as
// the B operand. Both contractions need operands whose k index runs along
// memory: Q and K do (the head dim), P and V do not (the key index), so P goes
// through LDS as a [row][key] tile and V is written into LDS transposed,
// [dim][key], while it is loaded. The matrix cores take bf16; q and P are
// float32 here, so each is split into bf16 hi + lo and multiplied twice (K and
// V are bf16 in the cache and exact), which keeps the products at float32
// accuracy. The next key block's K/V loads are issued as soon as the current
// block's K and V have been used (after S = Q K^T and the V transpose), so they
// land while its softmax and P V run.
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

template <int HD>
__global__ __launch_bounds__(64 * kPaWaves) __attribute__((amdgpu_waves_per_eu(2))) void prefill_attn_mfma_kernel(PrefillAttnArgs a) {
    constexpr int NWV = kPaWaves;
    constexpr int KS = HD / 16;          // 16-dim slices of the score product
    constexpr int CB = HD / 32;          // 32-dim column blocks of the output
    constexpr int VL = HD / 16;          // 16-byte V loads per lane (half a key row)
    constexpr int VTS = kPaKeys + 8;     // bf16 per transposed V row (16-byte aligned, padded)
    constexpr int PSS = kPaKeys + 4;     // floats per P row
    constexpr int VT_B = HD * VTS * 2, PS_B = kPaRows * PSS * 4;   // one wave's tiles
    constexpr int TILES = NWV * (VT_B + PS_B);
    constexpr int MERGE = (NWV - 1) * (kPaRows * HD + 2 * kPaRows) * 4;
    __shared__ __align__(16) char smem[TILES > MERGE ? TILES : MERGE];
    __shared__ uint4 qfr[2][KS][64];     // Q fragments (bf16 hi, lo) of every lane, shared by the waves

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r32 = lane & 31, hi = lane >> 5;
    uint16_t (*vt)[VTS] = (uint16_t (*)[VTS])(smem + wave * (VT_B + PS_B));
    float (*ps)[PSS] = (float (*)[PSS])(smem + wave * (VT_B + PS_B) + VT_B);
    // the longest query tiles (most key blocks) are dispatched first
    const int q0 = (gridDim.x - 1 - blockIdx.x) * kPaRows, h = blockIdx.y;
    const int G = a.Hq / a.Hkv, g = h / G;
    const int N = a.rows, start = a.start;
    const int last_row = min(q0 + kPaRows, N) - 1;
    const int t_max = start + last_row;              // the last key any row of this tile sees
    const int nkb = t_max / kPaKeys + 1;
    const int* bt = a.block_table;

    // Q fragments: row q0 + r32, dims 16 kk + 8 hi .. + 7, as bf16 hi + lo, formed
    // once by wave 0 and read from LDS at each block (registers are the limit here)
    if (wave == 0) {
        uint4 qh[KS], ql[KS];
        const int row = q0 + r32;
        const bool ok = row < N;
        const float* qp = a.q + ((long)(ok ? row : 0) * a.Hq + h) * HD + 8 * hi;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const float4 u = *(const float4*)(qp + 16 * kk);
            const float4 w = *(const float4*)(qp + 16 * kk + 4);
            float v[8] = {u.x, u.y, u.z, u.w, w.x, w.y, w.z, w.w};
            if (!ok)
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = 0.f;
            split_hi_lo(v, qh[kk], ql[kk]);
            qfr[0][kk][lane] = qh[kk];
            qfr[1][kk][lane] = ql[kk];
        }
    }
    __syncthreads();

    // Lane's key of block kb: kb*32 + r32. Keys past t_max, or whose page is not in
    // the pool, read the row of key 0 (a written row) and are masked out.
    const int pg_key0 = bt[0];
    const int pg_fallback = (pg_key0 >= 0 && pg_key0 < a.num_pages) ? pg_key0 : 0;
    auto key_row = [&](int kb, bool& ok) -> long {
        const int t = kb * kPaKeys + r32;
        const int tc = t <= t_max ? t : t_max;
        const int pg = bt[tc / a.page];
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
    auto load = [&](Blk& b, int kb) {
        const long off = key_row(kb, b.ok);
        const uint16_t* kp = (const uint16_t*)a.k_cache + off + 8 * hi;
        const uint16_t* vp = (const uint16_t*)a.v_cache + off + hi * (HD / 2);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) b.k[kk] = *(const uint4*)(kp + 16 * kk);
#pragma unroll
        for (int j = 0; j < VL; ++j) b.v[j] = *(const uint4*)(vp + 8 * j);
    };
    // this wave's LDS tiles are its own: ordering them needs only the wave itself
    auto wave_sync = [&]() {
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
    };

    float m[16], l[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) { m[e] = -INFINITY; l[e] = 0.f; }
    pa_f32x16 o[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[cb][e] = 0.f;

    // one block: V^T into LDS and S = Q K^T, then the next block's loads go into the
    // same registers (they land while this block's softmax and P V run)
    auto compute = [&](Blk& b, int kb, int next) {
        // V block into LDS, transposed: vt[dim][key]
#pragma unroll
        for (int j = 0; j < VL; ++j) {
            const uint32_t w[4] = {b.v[j].x, b.v[j].y, b.v[j].z, b.v[j].w};
            const int d0 = hi * (HD / 2) + 8 * j;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vt[d0 + 2 * e][r32] = (uint16_t)(w[e] & 0xffffu);
                vt[d0 + 2 * e + 1][r32] = (uint16_t)(w[e] >> 16);
            }
        }
        // scores of the 32 x 32 tile; lane holds key r32 of rows (e/4)*8 + hi*4 + e%4
        pa_f32x16 sacc;
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa_frag(qfr[0][kk][lane]), pa_frag(b.k[kk]), sacc, 0, 0, 0);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa_frag(qfr[1][kk][lane]), pa_frag(b.k[kk]), sacc, 0, 0, 0);
        }
        const bool bok = b.ok;
        if (next >= 0) load(b, next);
        const int key = kb * kPaKeys + r32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = (e >> 2) * 8 + hi * 4 + (e & 3);
            const bool valid = bok && key <= start + q0 + row && key <= t_max;
            const float sv = valid ? sacc[e] * a.scale : -INFINITY;
            const float mb = group_max<32>(sv);
            const float mn = fmaxf(m[e], mb);
            const float alpha = mn == -INFINITY ? 1.f : expf(m[e] - mn);
            const float p = valid ? expf(sv - mn) : 0.f;
            l[e] = l[e] * alpha + group_sum<32>(p);
            m[e] = mn;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) o[cb][e] *= alpha;
            ps[row][r32] = p;
        }
        wave_sync();
        // P as A fragments (row r32, keys 16 ks + 8 hi .. + 7), split hi + lo
        uint4 ph[2], pl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const float4 u = *(const float4*)&ps[r32][16 * ks + 8 * hi];
            const float4 w = *(const float4*)&ps[r32][16 * ks + 8 * hi + 4];
            const float v[8] = {u.x, u.y, u.z, u.w, w.x, w.y, w.z, w.w};
            split_hi_lo(v, ph[ks], pl[ks]);
        }
        // O += P V: V^T fragments are dim cb*32 + r32, keys 16 ks + 8 hi .. + 7
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const uint4 vf = *(const uint4*)&vt[cb * 32 + r32][16 * ks + 8 * hi];
                o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa_frag(ph[ks]), pa_frag(vf), o[cb], 0, 0, 0);
                o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa_frag(pl[ks]), pa_frag(vf), o[cb], 0, 0, 0);
            }
        wave_sync();   // the tiles are rewritten by this wave's next block
    };

    // this wave's blocks: wave, wave + NWV, ...
    Blk b;
    int kb = wave;
    if (kb < nkb) load(b, kb);
    while (kb < nkb) {
        const int next = kb + NWV;
        compute(b, kb, next < nkb ? next : -1);
        kb = next;
    }

    // the waves' (m, l, o) meet in LDS (the online-softmax merge); wave 0 (which
    // always holds key 0, valid for every row) forms context = O / L in bf16
    __syncthreads();                                  // every wave is done with its tiles
    float* mo = (float*)smem;                         // [NWV-1][32][HD], then [NWV-1][32] (m, l)
    float2* mlw = (float2*)(mo + (NWV - 1) * kPaRows * HD);
    if (wave > 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = (e >> 2) * 8 + hi * 4 + (e & 3);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) mo[((wave - 1) * kPaRows + row) * HD + cb * 32 + r32] = o[cb][e];
            if (r32 == 0) mlw[(wave - 1) * kPaRows + row] = make_float2(m[e], l[e]);
        }
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int rl = (e >> 2) * 8 + hi * 4 + (e & 3);
        const int row = q0 + rl;
        float M = m[e];
#pragma unroll
        for (int w = 1; w < NWV; ++w) M = fmaxf(M, mlw[(w - 1) * kPaRows + rl].x);
        float wt[NWV];
        wt[0] = expf(m[e] - M);
        float L = l[e] * wt[0];
#pragma unroll
        for (int w = 1; w < NWV; ++w) {
            const float2 ml = mlw[(w - 1) * kPaRows + rl];
            wt[w] = ml.x == -INFINITY ? 0.f : expf(ml.x - M);
            L = fmaf(ml.y, wt[w], L);
        }
        if (row >= N) continue;
        const float inv = 1.0f / L;
        uint16_t* dst = a.out + (long)row * a.Hq * HD + h * HD + r32;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            float v = o[cb][e] * wt[0];
#pragma unroll
            for (int w = 1; w < NWV; ++w) v = fmaf(mo[((w - 1) * kPaRows + rl) * HD + cb * 32 + r32], wt[w], v);
            dst[cb * 32] = f32_to_bf16(v * inv);
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
