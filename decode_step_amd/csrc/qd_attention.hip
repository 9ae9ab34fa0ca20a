// Decode attention for gfx950: per-head q/k RMSNorm, RoPE, the KV append of the
// new token and split-K online-softmax attention over the paged cache, in one
// kernel per layer.
//
// One workgroup per (split, kv head g, sequence b) reads each cached K and V
// row of its split once for all `group` query heads sharing KV head g (query
// head h reads KV head h / group: repeat, not tile -- nanoinfer page, phase 3).
// A split keeps (o, m, l) = (sum exp(s - m) v, max s, sum exp(s - m)); the
// last split to finish merges them with weights exp(m_s - M), M = max m_s
// (Tang page, section 2.2: online softmax is a monoid; Table 1: split-K).
//
// The new token (position p) is not read from the cache: its k is projected,
// normed (8B-class shape), rotated, rounded to the cache type, written to its
// slot, and that stored value is what the scores use (nanoserve day 49: the
// step writes this token's K/V into its row before it attends; nanoinfer page,
// phase 4: keys are rotated once, on insert). The query rows are normed and
// rotated here too.
//
// RoPE (nanoinfer page, phase 3: half-split pairs i and i + hd/2): the angle
// p * theta^(-2i/hd) is formed and reduced modulo 2*pi in double, then its
// sine and cosine are taken in float. A lane holds CE consecutive elements of a
// head, so the partner of element i sits in lane li ^ (LPT/2) and arrives by one
// cross-lane shuffle.
#include "qd_device.h"
#include "qd_launch.h"

namespace qd {

constexpr int kAttnThreads = 256;
constexpr int kMaxGroup = 8;
constexpr int kMaxChunk = 256;
constexpr int kAttnIters = 8;   // token passes whose K/V rows a lane holds in registers

template <int HD, typename KVT>
constexpr int attn_tokens_per_pass() { return 4 * (kWave / (HD / VecN<KVT>::n)); }

int attn_max_chunk(int hd, int kv_is_bf16) {
    int tpb;
    if (hd == 64) tpb = kv_is_bf16 ? attn_tokens_per_pass<64, uint16_t>() : attn_tokens_per_pass<64, float>();
    else tpb = kv_is_bf16 ? attn_tokens_per_pass<128, uint16_t>() : attn_tokens_per_pass<128, float>();
    int c = tpb * kAttnIters;
    return c < kMaxChunk ? c : kMaxChunk;
}

__device__ __forceinline__ void load_f32xN(const float* p, float* f, int n) {
#pragma unroll
    for (int q = 0; q < n / 4; ++q) {
        float4 t = ((const float4*)p)[q];
        f[4 * q] = t.x; f[4 * q + 1] = t.y; f[4 * q + 2] = t.z; f[4 * q + 3] = t.w;
    }
}

// Half-split rotation of the CE elements this lane holds (lower half when li < LPT/2).
template <int CE, int LPT>
__device__ __forceinline__ void rope_lane(float (&u)[CE], const float (&c)[CE], const float (&sn)[CE], bool lower) {
#pragma unroll
    for (int e = 0; e < CE; ++e) {
        const float partner = __shfl_xor(u[e], LPT / 2, kWave);
        u[e] = lower ? u[e] * c[e] - partner * sn[e] : u[e] * c[e] + partner * sn[e];
    }
}

template <typename WT, typename KVT, int HD>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(AttnArgs a) {
    constexpr int CE = VecN<KVT>::n;
    constexpr int LPT = HD / CE;
    constexpr int TPW = kWave / LPT;
    constexpr int TPB = 4 * TPW;
    constexpr int NI = kAttnIters;
    __shared__ float sc[kMaxGroup][kMaxChunk];
    __shared__ float red[4][kMaxGroup][HD];
    __shared__ float ml[kMaxGroup][2];
    __shared__ int is_last;

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int G = a.Hq / a.Hkv;
    const int p = a.pos[b];
    if (p < 0 || p >= a.capacity || a.chunk > NI * TPB || a.chunk > kMaxChunk || G > kMaxGroup) return;
    const int T = p + 1;
    const int ns = min(a.S, (T + a.chunk - 1) / a.chunk);
    const int t_begin = s * a.chunk;
    if (t_begin >= T) return;
    const int t_end = min(T, t_begin + a.chunk);
    const int n = t_end - t_begin;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int li = lane % LPT, slot = lane / LPT;
    const bool lower = li < LPT / 2;
    const int* bt = a.block_table + (long)b * a.max_blocks;

    // cached K/V rows of this split (position p excluded: it is the new token)
    uint4 kraw[NI], vraw[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int t = t_begin + i * TPB + wave * TPW + slot;
        kraw[i] = make_uint4(0, 0, 0, 0);
        vraw[i] = make_uint4(0, 0, 0, 0);
        if (t < t_end && t != p) {
            const int page_id = bt[t / a.page];
            if (page_id >= 0 && page_id < a.num_pages) {
                const long off = (((long)page_id * a.Hkv + g) * a.page + (t % a.page)) * HD + li * CE;
                kraw[i] = *(const uint4*)((const KVT*)a.k_cache + off);
                vraw[i] = *(const uint4*)((const KVT*)a.v_cache + off);
            }
        }
    }
    // projected q of the group's heads and the new k, v of head g
    const int qkvr = (a.Hq + 2 * a.Hkv) * HD;
    const float* src = a.qkv + (long)b * qkvr;
    float q[kMaxGroup][CE];
#pragma unroll
    for (int hl = 0; hl < kMaxGroup; ++hl) {
        if (hl < G) load_f32xN(src + (g * G + hl) * HD + li * CE, q[hl], CE);
        else {
#pragma unroll
            for (int e = 0; e < CE; ++e) q[hl][e] = 0.f;
        }
    }
    float kn[CE], vn[CE];
    load_f32xN(src + a.Hq * HD + g * HD + li * CE, kn, CE);
    load_f32xN(src + (a.Hq + a.Hkv) * HD + g * HD + li * CE, vn, CE);

    // rotation angles of this lane's elements: i = (li mod LPT/2) * CE + e
    float cs[CE], sn[CE];
#pragma unroll
    for (int e = 0; e < CE; ++e) {
        const int i = (li % (LPT / 2)) * CE + e;
        const double inv = pow((double)a.theta, -2.0 * (double)i / (double)HD);
        double ang = (double)p * inv;
        const double two_pi = 6.283185307179586476925286766559;
        ang -= two_pi * rint(ang / two_pi);
        sincosf((float)ang, &sn[e], &cs[e]);
    }
    if (a.qk_norm) {
#pragma unroll
        for (int hl = 0; hl < kMaxGroup; ++hl) {
            if (hl >= G) break;
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < CE; ++e) ss += q[hl][e] * q[hl][e];
            ss = group_sum<LPT>(ss);
            const float r = 1.0f / sqrtf(ss / (float)HD + a.eps);
#pragma unroll
            for (int e = 0; e < CE; ++e) q[hl][e] = q[hl][e] * r * load_scalar<WT>(a.q_norm, li * CE + e);
        }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < CE; ++e) ss += kn[e] * kn[e];
        ss = group_sum<LPT>(ss);
        const float r = 1.0f / sqrtf(ss / (float)HD + a.eps);
#pragma unroll
        for (int e = 0; e < CE; ++e) kn[e] = kn[e] * r * load_scalar<WT>(a.k_norm, li * CE + e);
    }
#pragma unroll
    for (int hl = 0; hl < kMaxGroup; ++hl)
        if (hl < G) rope_lane<CE, LPT>(q[hl], cs, sn, lower);
    rope_lane<CE, LPT>(kn, cs, sn, lower);
    // stored form of the new K/V (rounded to the cache type) and the append
    const uint4 kst = pack16<KVT>(kn), vst = pack16<KVT>(vn);
    float kq[CE], vq[CE];
    widen16(kst, kq);
    widen16(vst, vq);
    if (p >= t_begin && p < t_end && wave == 0 && slot == 0) {
        const int page_id = bt[p / a.page];
        if (page_id >= 0 && page_id < a.num_pages) {
            const long off = (((long)page_id * a.Hkv + g) * a.page + (p % a.page)) * HD + li * CE;
            *(uint4*)((KVT*)a.k_cache + off) = kst;
            *(uint4*)((KVT*)a.v_cache + off) = vst;
        }
    }

    // scores s = q . k / sqrt(hd)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        if (i * TPB >= n) break;
        const int t = t_begin + i * TPB + wave * TPW + slot;
        float kf[CE];
        widen16(kraw[i], kf);
        if (t == p) {
#pragma unroll
            for (int e = 0; e < CE; ++e) kf[e] = kq[e];
        }
#pragma unroll
        for (int hl = 0; hl < kMaxGroup; ++hl) {
            if (hl >= G) break;
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < CE; ++e) d = fmaf(q[hl][e], kf[e], d);
            d = group_sum<LPT>(d);
            if (li == 0 && t < t_end) sc[hl][t - t_begin] = d * a.scale;
        }
    }
    __syncthreads();
    for (int hl = wave; hl < G; hl += 4) {
        float m = -INFINITY;
        for (int j = lane; j < n; j += kWave) m = fmaxf(m, sc[hl][j]);
        m = wave_max(m);
        float l = 0.f;
        for (int j = lane; j < n; j += kWave) {
            const float e = expf(sc[hl][j] - m);
            sc[hl][j] = e;
            l += e;
        }
        l = group_sum<kWave>(l);
        if (lane == 0) { ml[hl][0] = m; ml[hl][1] = l; }
    }
    __syncthreads();
    // o = sum_t exp(s_t - m) v_t
    float o[kMaxGroup][CE];
#pragma unroll
    for (int hl = 0; hl < kMaxGroup; ++hl)
#pragma unroll
        for (int e = 0; e < CE; ++e) o[hl][e] = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        if (i * TPB >= n) break;
        const int t = t_begin + i * TPB + wave * TPW + slot;
        if (t >= t_end) continue;
        float vf[CE];
        widen16(vraw[i], vf);
        if (t == p) {
#pragma unroll
            for (int e = 0; e < CE; ++e) vf[e] = vq[e];
        }
#pragma unroll
        for (int hl = 0; hl < kMaxGroup; ++hl) {
            if (hl >= G) break;
            const float pr = sc[hl][t - t_begin];
#pragma unroll
            for (int e = 0; e < CE; ++e) o[hl][e] = fmaf(pr, vf[e], o[hl][e]);
        }
    }
#pragma unroll
    for (int hl = 0; hl < kMaxGroup; ++hl) {
        if (hl >= G) break;
#pragma unroll
        for (int e = 0; e < CE; ++e) {
            float v = o[hl][e];
#pragma unroll
            for (int off = kWave / 2; off >= LPT; off >>= 1) v += __shfl_xor(v, off, kWave);
            if (slot == 0) red[wave][hl][li * CE + e] = v;
        }
    }
    __syncthreads();
    float* ctx = a.ctx + ((long)b * a.Hq + g * G) * HD;
    if (ns == 1) {
        for (int idx = tid; idx < G * HD; idx += kAttnThreads) {
            const int hl = idx / HD, d = idx - hl * HD;
            ctx[idx] = (red[0][hl][d] + red[1][hl][d] + red[2][hl][d] + red[3][hl][d]) / ml[hl][1];
        }
        return;
    }
    // several splits: publish the partial; the last split to arrive merges
    float* part = a.part + (((long)b * a.Hkv + g) * a.S) * G * (HD + 2);
    const long sstride = (long)G * (HD + 2);
    for (int idx = tid; idx < G * HD; idx += kAttnThreads) {
        const int hl = idx / HD, d = idx - hl * HD;
        part[s * sstride + hl * (HD + 2) + d] = red[0][hl][d] + red[1][hl][d] + red[2][hl][d] + red[3][hl][d];
    }
    if (tid < G) {
        part[s * sstride + tid * (HD + 2) + HD] = ml[tid][0];
        part[s * sstride + tid * (HD + 2) + HD + 1] = ml[tid][1];
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) is_last = atomicAdd(a.counters + (long)b * a.Hkv + g, 1u) == (unsigned)(ns - 1);
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    for (int idx = tid; idx < G * HD; idx += kAttnThreads) {
        const int hl = idx / HD, d = idx - hl * HD;
        const float* ps = part + hl * (HD + 2);
        float M = -INFINITY;
        for (int j = 0; j < ns; ++j) M = fmaxf(M, ps[j * sstride + HD]);
        float L = 0.f, O = 0.f;
        for (int j = 0; j < ns; ++j) {
            const float w = expf(ps[j * sstride + HD] - M);
            L = fmaf(ps[j * sstride + HD + 1], w, L);
            O = fmaf(ps[j * sstride + d], w, O);
        }
        ctx[idx] = O / L;
    }
}

hipError_t launch_attention(const AttnArgs& a, int w_is_bf16, int kv_is_bf16, hipStream_t s) {
    dim3 grid(a.S, a.Hkv, a.B);
    dim3 block(kAttnThreads);
#define QD_ATTN(WT, KVT, HD) hipLaunchKernelGGL((attn_kernel<WT, KVT, HD>), grid, block, 0, s, a)
    if (a.hd == 64) {
        if (w_is_bf16) { if (kv_is_bf16) QD_ATTN(uint16_t, uint16_t, 64); else QD_ATTN(uint16_t, float, 64); }
        else { if (kv_is_bf16) QD_ATTN(float, uint16_t, 64); else QD_ATTN(float, float, 64); }
    } else {
        if (w_is_bf16) { if (kv_is_bf16) QD_ATTN(uint16_t, uint16_t, 128); else QD_ATTN(uint16_t, float, 128); }
        else { if (kv_is_bf16) QD_ATTN(float, uint16_t, 128); else QD_ATTN(float, float, 128); }
    }
#undef QD_ATTN
    return hipGetLastError();
}

}  // namespace qd
