// Next-token sampling from a row of logits on the GPU (nanoinfer page, phase 5:
// temperature -> top-k -> top-p -> softmax -> inverse-CDF draw, in that order;
// temperature 0 is the argmax). One workgroup of 1024 threads per row; no
// device memory beyond the logits, the uniforms and the tokens.
//
// Per row, with T > 0 and 1 <= k <= 1024:
// 1. top-k: the k-th largest logit is found exactly by a three-digit radix
//    select over order-preserving 32-bit keys (11, 11 and 10 bits), with the
//    histograms in LDS. The first digit reads the row; when the logits in its
//    boundary bin and above fit the candidate space (the usual case: the top
//    bins of a vocabulary's logits are sparse), they are compacted into LDS and
//    the other two digits run there, else each digit reads the row again. Every
//    logit >= the k-th largest is a candidate, so ties at the boundary are all
//    kept (the transformers warper removes only scores below the k-th).
//    Dividing by T > 0 keeps the order, so the threshold is taken on the logits
//    themselves.
// 2. The candidates are compacted into LDS with z = logit / T (float32, IEEE
//    division), and sorted ascending by (z, token id): a stable ascending sort,
//    the order the page settles on (a tied pair keeps its index order). When more
//    than kSampleCand candidates tie at the k-th largest value, only the fewer
//    than k above it are stored and sorted; the tied ones share one z and one
//    probability and come first in that order (by id), so they are counted, and
//    when some of them stay, wave 0 draws over the row in token order itself.
// 3. top-p as the page's reference defines it: with probabilities
//    e_j / S (e_j = exp(z_j - max z), S their sum), the cumulative sum over the
//    ascending order is taken in float32, one term at a time, and every token
//    whose cumulative sum is <= 1 - p is removed; the largest always stays.
// 4. The kept tokens, back in token-id order, get probabilities e_j / S_kept;
//    their running sum, again one term at a time, is searched for the first
//    token whose cumulative value exceeds u * total (an inverse-CDF draw that
//    does not need the probabilities to sum to exactly one).
#include "qd_device.h"
#include "qd_launch.h"

namespace qd {

constexpr int kSampleThreads = 1024;
constexpr int kSampleCand = 2048;    // candidates a row may hold (k plus ties at the boundary)

// larger float -> larger key, for every non-NaN value
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t b = __float_as_uint(f);
    return b ^ ((b & 0x80000000u) ? 0xffffffffu : 0x80000000u);
}

// Radix-select step: in hist[0..nb), scanned from the top bin down, the bin where
// the running count reaches `need`; returns the bin and the count of the bins
// above it. Run by wave 0 (every lane returns the same).
__device__ __forceinline__ void top_bin(const int* hist, int nb, int need, int lane, int& bin, int& above) {
    const int per = nb / kWave;                // bins per lane, lane 0 holding the highest
    const int hi = nb - per * lane;            // this lane's bins: [hi - per, hi)
    int mine = 0;
    for (int j = hi - 1; j >= hi - per; --j) mine += hist[j];
    // exclusive prefix over lanes 0..lane-1 (the bins above this lane's)
    int incl = mine;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int t = __shfl_up(incl, d);
        if (lane >= d) incl += t;
    }
    const int excl = incl - mine;
    const bool here = excl < need && incl >= need;
    int b = -1, a = 0;
    if (here) {
        int run = excl;
        for (int j = hi - 1; j >= hi - per; --j) {
            if (run + hist[j] >= need) { b = j; a = run; break; }
            run += hist[j];
        }
    }
    // broadcast from the lane that found it (exactly one lane, as 1 <= need <= total)
    const unsigned long long m = __ballot(here);
    const int src = m ? __ffsll((long long)m) - 1 : 0;
    bin = __shfl(b, src);
    above = __shfl(a, src);
}

// Top-p over the whole vocabulary (top_k <= 0 or >= V), one workgroup per row,
// every step a pass over the row (no candidate list):
// A. max logit; z = logit / T keeps the order, so max z = (max logit) / T.
// B. S = sum_j e_j, e_j = exp(z_j - max z) (tree sum).
// C. the top-p cut, as a radix select by probability mass over the logits'
//    order keys (11, 11, 10 bits): each digit's bins hold the mass m_j = e_j / S
//    of their logits (LDS float adds), scanned from the lowest key up for the
//    first bin where the running mass passes 1 - p. This gives the boundary key,
//    the mass below it and the number of logits tied at it; the tied ones (equal
//    z, equal m) are removed one at a time, in token-id order (the stable
//    ascending order), while the running sum stays <= 1 - p, and the largest
//    always stays.
// D. S_kept over the kept tokens; the draw in token-id order: each wave runs over
//    its own contiguous range of ids in chunks of 64 (lane order = id order, a
//    wave prefix sum per chunk) for its range's total, then the wave whose range
//    holds the first running value > u * total finds the token in it.
// The masses are summed in a different order than one at a time, so a row whose
// cut or draw lies within that rounding of a boundary may fall on its other side.
template <typename Scan>
__device__ __forceinline__ void sample_whole_vocab(const SampleArgs& a, int row, const float* lg, Scan&& scan, int* hist,
                                                float* mass, unsigned long long* ids, float* s_red) {
    __shared__ uint32_t s_key;
    __shared__ float s_base;
    __shared__ int s_idcut, s_cnt2;
    __shared__ float s_wtot[kSampleThreads / kWave];
    __shared__ int s_tok;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    constexpr int NWV = kSampleThreads / kWave;
    const int V = a.V;
    const float T = a.temperature;
    auto block_red = [&](float v, bool is_max) {   // every thread returns the workgroup's sum or max
        v = is_max ? group_max<kWave>(v) : group_sum<kWave>(v);
        __syncthreads();
        if (lane == 0) s_red[wave] = v;
        __syncthreads();
        float t = is_max ? -INFINITY : 0.f;
        for (int w = 0; w < NWV; ++w) t = is_max ? fmaxf(t, s_red[w]) : t + s_red[w];
        return t;
    };
    // A, B
    float m = -INFINITY;
    scan([&](int, float v) { m = fmaxf(m, v); });
    const float lmax = block_red(m, true);
    if (!(lmax > -INFINITY)) {   // every logit NaN or -inf: no candidate
        if (tid == 0) a.tokens[row] = -1;
        return;
    }
    const float zmax = __fdiv_rn(lmax, T);
    auto e_of = [&](float v) { return expf(__fdiv_rn(v, T) - zmax); };
    float part = 0.f;
    scan([&](int, float v) { part += e_of(v); });
    const float S = block_red(part, false);
    // C
    const uint32_t kmax = order_key(lmax);
    if (tid == 0) { s_key = 0u; s_base = 0.f; s_idcut = 0; }
    if (a.top_p < 1.f) {
        const float thr = a.one_minus_p;
        uint32_t prefix = 0;
        float base = 0.f;
        int n_t = 0;
        for (int d = 0; d < 3; ++d) {
            const int width = d < 2 ? 11 : 10, sh = d == 0 ? 21 : (d == 1 ? 10 : 0), nb = 1 << width, hs = sh + width;
            for (int j = tid; j < nb; j += kSampleThreads) { mass[j] = 0.f; hist[j] = 0; }
            __syncthreads();
            scan([&](int, float v) {
                const uint32_t key = order_key(v);
                if (hs >= 32 || (key >> hs) == prefix) {
                    const int bin = (int)((key >> sh) & (uint32_t)(nb - 1));
                    atomicAdd(&mass[bin], __fdiv_rn(e_of(v), S));
                    atomicAdd(&hist[bin], 1);
                }
            });
            __syncthreads();
            if (wave == 0) {
                // lane l holds bins [l * per, (l + 1) * per); the first lane whose running
                // mass passes thr, then the first such bin in it (a nonempty one)
                const int per = nb / kWave, lo = lane * per;
                float mine = 0.f;
                int last_ne = -1;
                for (int j = lo; j < lo + per; ++j) { mine += mass[j]; if (hist[j]) last_ne = j; }
                float incl = mine;
#pragma unroll
                for (int o = 1; o < kWave; o <<= 1) {
                    const float t = __shfl_up(incl, o);
                    if (lane >= o) incl += t;
                }
                const float excl = incl - mine;
                const unsigned long long pass = __ballot(base + incl > thr);
                const unsigned long long ne = __ballot(last_ne >= 0);
                // no lane passes (rounding): the highest nonempty bin
                const int src = pass ? __ffsll((long long)pass) - 1 : 63 - __clzll((long long)ne);
                int bin = -1;
                float below = 0.f;
                if (lane == src) {
                    float c = base + excl;
                    for (int j = lo; j < lo + per; ++j) {
                        if (hist[j] && c + mass[j] > thr) { bin = j; below = c; break; }
                        c += mass[j];
                    }
                    if (bin < 0) {   // rounding: the last nonempty bin of the range
                        c = base + excl;
                        for (int j = lo; j < lo + per; ++j) { if (hist[j]) { bin = j; below = c; } c += mass[j]; }
                    }
                }
                bin = max(__shfl(bin, src), 0);
                below = __shfl(below, src);
                if (lane == 0) { s_key = (prefix << width) | (uint32_t)bin; s_base = below; s_cnt2 = hist[bin]; }
            }
            __syncthreads();
            prefix = s_key;
            base = s_base;
            n_t = s_cnt2;
            __syncthreads();
        }
        // the tied logits at the boundary key, removed one at a time while the running
        // sum stays <= thr; the largest always stays
        if (tid == 0) {
            const float vk = __uint_as_float(prefix ^ ((prefix & 0x80000000u) ? 0x80000000u : 0xffffffffu));
            const float mk = __fdiv_rn(e_of(vk), S);
            float c = base;
            int r = 0;
            while (r < n_t) {
                const float c2 = c + mk;
                if (!(c2 <= thr)) break;
                c = c2;
                ++r;
            }
            if (r == n_t && prefix == kmax) r = n_t - 1;
            s_cnt2 = r;        // tied tokens removed (the lowest ids)
            s_key = prefix;
        }
        __syncthreads();
        const int r = s_cnt2;
        const uint32_t kap = s_key;
        __syncthreads();   // every thread has read r before s_cnt2 counts the tied ids below
        // the id from which tied tokens stay: the r-th smallest tied id (V: none stays)
        if (r == 0) {
            if (tid == 0) s_idcut = 0;
        } else if (r >= n_t) {
            if (tid == 0) s_idcut = V;
        } else if (n_t <= kSampleCand) {
            if (tid == 0) s_cnt2 = 0;
            __syncthreads();
            scan([&](int i, float v) {
                if (order_key(v) == kap) ids[atomicAdd(&s_cnt2, 1)] = (unsigned long long)i;
            });
            __syncthreads();
            for (int j = tid; j < n_t; j += kSampleThreads) {
                const unsigned long long me = ids[j];
                int smaller = 0;
                for (int q = 0; q < n_t; ++q) smaller += ids[q] < me ? 1 : 0;
                if (smaller == r) s_idcut = (int)me;
            }
        } else if (wave == 0) {   // more tied logits than LDS holds: count them in id order
            int seen = 0, cut = V;
            for (int c0 = 0; c0 < V && cut == V; c0 += kWave) {
                const int i = c0 + lane;
                const bool tied = i < V && order_key(lg[i]) == kap;
                const unsigned long long mk = __ballot(tied);
                const int cnt = __popcll(mk);
                if (seen + cnt > r) {   // the (r - seen)-th set lane of this chunk
                    unsigned long long mm = mk;
                    for (int q = 0; q < r - seen; ++q) mm &= mm - 1ull;
                    cut = c0 + __ffsll((long long)mm) - 1;
                }
                seen += cnt;
            }
            if (lane == 0) s_idcut = cut;
        }
    }
    __syncthreads();
    const uint32_t kap = s_key;
    const int idcut = s_idcut;
    auto kept = [&](int i, float v) {
        const uint32_t key = order_key(v);
        return key > kap || (key == kap && i >= idcut);
    };
    // D
    float kp = 0.f;
    scan([&](int i, float v) { if (kept(i, v)) kp += e_of(v); });
    const float Sk = block_red(kp, false);
    const int seg = (((V + NWV - 1) / NWV) + kWave - 1) / kWave * kWave;   // ids per wave, whole chunks
    const int i0 = wave * seg, i1 = min(V, i0 + seg);
    // one pass over this wave's range in chunks of 64 (8 chunks of loads in flight);
    // fn(chunk start, lane's p, wave-inclusive prefix of p) per chunk; stops when fn
    // returns true
    auto walk = [&](auto&& fn) {
        for (int c0 = i0; c0 < i1; c0 += 8 * kWave) {
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int i = c0 + q * kWave + lane;
                v[q] = i < i1 ? lg[i] : 0.f;
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int cs = c0 + q * kWave, i = cs + lane;
                if (cs >= i1) break;
                const float p = (i < i1 && kept(i, v[q])) ? __fdiv_rn(e_of(v[q]), Sk) : 0.f;
                float incl = p;
#pragma unroll
                for (int o = 1; o < kWave; o <<= 1) {
                    const float t = __shfl_up(incl, o);
                    if (lane >= o) incl += t;
                }
                if (fn(cs, p, incl)) return;
            }
        }
    };
    float wt = 0.f;
    walk([&](int, float, float incl) { wt += __shfl(incl, kWave - 1); return false; });
    if (lane == 0) s_wtot[wave] = wt;
    if (tid == 0) s_tok = -1;
    __syncthreads();
    float tot = 0.f, before = 0.f;
    for (int w = 0; w < NWV; ++w) { if (w < wave) before += s_wtot[w]; tot += s_wtot[w]; }
    const float target = a.uniforms[row] * tot;
    // the wave whose range holds the first running value > target (none: rounding, the last)
    int wsel = NWV - 1;
    {
        float c = 0.f;
        for (int w = 0; w < NWV; ++w) {
            if (s_wtot[w] > 0.f && c + s_wtot[w] > target) { wsel = w; break; }
            c += s_wtot[w];
        }
    }
    if (wave == wsel) {
        float run = before;
        int last = -1;
        walk([&](int cs, float p, float incl) {
            const unsigned long long hit = __ballot(p > 0.f && run + incl > target);
            const unsigned long long km = __ballot(p > 0.f);
            if (km) last = cs + 63 - __clzll((long long)km);
            if (hit) {
                if (lane == 0) s_tok = cs + __ffsll((long long)hit) - 1;
                return true;
            }
            run += __shfl(incl, kWave - 1);
            return false;
        });
        if (lane == 0 && s_tok < 0) s_tok = last;
    }
    __syncthreads();
    if (tid == 0) {
        int t = s_tok;
        if (t < 0) {   // the selected range kept nothing (rounding): the last kept token of the row
            for (int i = V - 1; i >= 0; --i) if (kept(i, lg[i])) { t = i; break; }
        }
        a.tokens[row] = t;
    }
}

__global__ __launch_bounds__(kSampleThreads) void sample_kernel(SampleArgs a) {
    __shared__ int hist[2048];
    __shared__ unsigned long long ck[kSampleCand];   // (order key of z) << 32 | token
    __shared__ float ce[kSampleCand];                // e_j in ascending order
    __shared__ int s_bin, s_above, s_cnt, s_j0;
    __shared__ float s_red[kSampleThreads / kWave];
    const int row = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int V = a.V;
    const float* lg = a.logits + (long)row * V;

    if (a.temperature == 0.f) {   // greedy: the lowest index among the maxima
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        for (int i = tid; i < V; i += kSampleThreads) {
            const float v = lg[i];
            if (better(v, i, bv, bi)) { bv = v; bi = i; }
        }
        wave_argmax(bv, bi);
        __shared__ float wv[kSampleThreads / kWave];
        __shared__ int wi[kSampleThreads / kWave];
        if (lane == 0) { wv[wave] = bv; wi[wave] = bi; }
        __syncthreads();
        if (tid == 0) {
            for (int w = 1; w < kSampleThreads / kWave; ++w)
                if (better(wv[w], wi[w], wv[0], wi[0])) { wv[0] = wv[w]; wi[0] = wi[w]; }
            a.tokens[row] = wi[0];
        }
        return;
    }

    // Every element of the row through fn(index, value): float4 loads, four in flight
    // per thread, when the row is 16-byte aligned (scalar loads otherwise).
    const bool vec = (V % 4 == 0) && (((uintptr_t)lg & 15u) == 0);
    auto scan = [&](auto&& fn) {
        if (vec) {
            const int V4 = V / 4;
            const float4* l4 = (const float4*)lg;
            int i4 = tid;
            for (; i4 + 3 * kSampleThreads < V4; i4 += 4 * kSampleThreads) {
                float4 q[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) q[u] = l4[i4 + u * kSampleThreads];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int i = 4 * (i4 + u * kSampleThreads);
                    fn(i, q[u].x); fn(i + 1, q[u].y); fn(i + 2, q[u].z); fn(i + 3, q[u].w);
                }
            }
            for (; i4 < V4; i4 += kSampleThreads) {
                const float4 q = l4[i4];
                fn(4 * i4, q.x); fn(4 * i4 + 1, q.y); fn(4 * i4 + 2, q.z); fn(4 * i4 + 3, q.w);
            }
        } else {
            for (int i = tid; i < V; i += kSampleThreads) fn(i, lg[i]);
        }
    };
    // one radix-select digit: histogram of the keys whose bits above this digit equal
    // `prefix`, then the bin where the count from the top reaches `need`
    auto digit = [&](int sh, int width, uint32_t& prefix, int& need, auto&& for_each_key) {
        const int nb = 1 << width, hs = sh + width;
        for (int j = tid; j < 2048; j += kSampleThreads) hist[j] = 0;
        __syncthreads();
        for_each_key([&](uint32_t key) {
            if (hs >= 32 || (key >> hs) == prefix) atomicAdd(&hist[(key >> sh) & (nb - 1)], 1);
        });
        __syncthreads();
        if (wave == 0) {
            int bin, above;
            top_bin(hist, nb, need, lane, bin, above);
            if (lane == 0) { s_bin = bin; s_above = above; }
        }
        __syncthreads();
        prefix = (prefix << width) | (uint32_t)s_bin;
        need -= s_above;
        __syncthreads();
    };
    auto global_keys = [&](auto&& f) { scan([&](int, float v) { f(order_key(v)); }); };

    if (a.top_k <= 0 || a.top_k >= V) {   // no top-k: top-p over the whole vocabulary
        sample_whole_vocab(a, row, lg, scan, hist, ce, ck, s_red);
        return;
    }

    // 1. the k-th largest key, 11 + 11 + 10 bits. After the first digit, when the
    //    boundary bin and everything above it fit the candidate space, those logits
    //    are compacted into LDS once and the last two digits run there; otherwise
    //    they read the row again.
    const int k = a.top_k < V ? a.top_k : V;
    uint32_t thr_key = 0;                          // order key of the k-th largest logit
    uint32_t prefix = 0;
    int need = k;
    digit(21, 11, prefix, need, global_keys);
    const int n0 = (k - need) + hist[prefix];      // logits in the boundary bin or above
    const bool in_lds = n0 <= kSampleCand;
    // slots holding candidates (compacted in place: in LDS they stay among the n0)
    const int nsort = in_lds ? n0 : kSampleCand;
    if (tid == 0) s_cnt = 0;
    for (int j = tid; j < kSampleCand; j += kSampleThreads) ck[j] = ~0ull;
    __syncthreads();
    if (in_lds) {
        const uint32_t b0 = prefix;
        scan([&](int i, float v) {
            const uint32_t key = order_key(v);
            if ((key >> 21) >= b0) {
                const int slot = atomicAdd(&s_cnt, 1);
                ck[slot] = ((unsigned long long)key << 32) | (uint32_t)i;
            }
        });
        __syncthreads();
        auto lds_keys = [&](auto&& f) {
            for (int j = tid; j < n0; j += kSampleThreads) f((uint32_t)(ck[j] >> 32));
        };
        digit(10, 11, prefix, need, lds_keys);
        digit(0, 10, prefix, need, lds_keys);
        const uint32_t thresh = prefix;
        thr_key = thresh;
        // 2. the candidates, in place: keys at or above the threshold become (key of
        //    z = logit / T, token); the rest sort to the end
        if (tid == 0) s_cnt = 0;
        __syncthreads();
        for (int j = tid; j < n0; j += kSampleThreads) {
            const unsigned long long e = ck[j];
            const uint32_t key = (uint32_t)(e >> 32), i = (uint32_t)(e & 0xffffffffu);
            if (key >= thresh) {
                atomicAdd(&s_cnt, 1);
                const float z = __fdiv_rn(lg[i], a.temperature);
                ck[j] = ((unsigned long long)order_key(z) << 32) | i;
            } else {
                ck[j] = ~0ull;
            }
        }
        __syncthreads();
    } else {
        digit(10, 11, prefix, need, global_keys);
        digit(0, 10, prefix, need, global_keys);
        const uint32_t thresh = prefix;
        thr_key = thresh;
        // 2. candidates: every logit whose key reaches the threshold, with z = logit / T
        scan([&](int i, float v) {
            if (order_key(v) >= thresh) {
                const int slot = atomicAdd(&s_cnt, 1);
                if (slot < kSampleCand) {
                    const float z = __fdiv_rn(v, a.temperature);
                    ck[slot] = ((unsigned long long)order_key(z) << 32) | (uint32_t)i;
                }
            }
        });
        __syncthreads();
    }
    int C = s_cnt;
    __syncthreads();   // every thread has read the count before the tie path below reuses s_cnt
    if (C < 1) {   // no candidate: NaN keys
        if (tid == 0) a.tokens[row] = -1;
        return;
    }
    // bitonic sort of ck ascending (empty slots hold the largest key)
    // (the first n entries; every slot from n up holds the largest key, so the
    // network runs over the next power of two only)
    auto bitonic = [&](int n) {
        int n2 = 2;
        while (n2 < n) n2 <<= 1;
        for (int size = 2; size <= n2; size <<= 1)
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                __syncthreads();
                for (int t = tid; t < n2 / 2; t += kSampleThreads) {
                    const int i = 2 * t - (t & (stride - 1));
                    const int j = i + stride;
                    const bool up = (i & size) == 0;
                    const unsigned long long x = ck[i], y = ck[j];
                    if ((x > y) == up) { ck[i] = y; ck[j] = x; }
                }
            }
        __syncthreads();
    };
    auto zval = [&](unsigned long long key) {
        const uint32_t ok = (uint32_t)(key >> 32);
        return __uint_as_float(ok ^ ((ok & 0x80000000u) ? 0x80000000u : 0xffffffffu));
    };
    auto block_sum = [&](float v) {   // tree sum over the workgroup (every thread returns it)
        v = group_sum<kWave>(v);
        __syncthreads();
        if (lane == 0) s_red[wave] = v;
        __syncthreads();
        float t = 0.f;
        for (int w = 0; w < kSampleThreads / kWave; ++w) t += s_red[w];
        return t;
    };

    int j0;
    if (C <= kSampleCand) {
        bitonic(in_lds ? nsort : C);
        // 3. e_j = exp(z_j - max z) over the ascending order; S by a tree sum; the
        //    cumulative sum of e_j / S one term at a time; remove while it is <= 1 - p
        const float zmax = zval(ck[C - 1]);
        float part = 0.f;
        for (int j = tid; j < C; j += kSampleThreads) {
            const float e = expf(zval(ck[j]) - zmax);
            ce[j] = e;
            part += e;
        }
        const float S = block_sum(part);
        if (tid == 0) {
            int jj = C - 1;   // the largest always stays
            if (a.top_p < 1.f) {
                float cum = 0.f;
                for (int j = 0; j < C - 1; ++j) {
                    cum += __fdiv_rn(ce[j], S);
                    if (!(cum <= a.one_minus_p)) { jj = j; break; }
                }
            } else {
                jj = 0;
            }
            s_j0 = jj;
        }
        __syncthreads();
        j0 = s_j0;
    } else {
        // More candidates than LDS holds: fewer than k lie above the threshold and the
        // rest tie at the threshold value itself, so they share one z and one e. In
        // the ascending (z, id) order the tied ones come first, in id order. The
        // above ones are sorted in LDS; the tied ones are counted, not stored.
        if (tid == 0) s_cnt = 0;
        for (int j = tid; j < kSampleCand; j += kSampleThreads) ck[j] = ~0ull;
        __syncthreads();
        const uint32_t thresh = thr_key;
        scan([&](int i, float v) {
            const uint32_t key = order_key(v);
            if (key > thresh) {
                const int slot = atomicAdd(&s_cnt, 1);
                if (slot < kSampleCand) ck[slot] = ((unsigned long long)order_key(__fdiv_rn(v, a.temperature)) << 32) | (uint32_t)i;
            }
        });
        __syncthreads();
        const int ng = s_cnt, ne = C - ng;   // above (ng < k <= kSampleMaxK), tied
        bitonic(ng);
        const float vt = __uint_as_float(thresh ^ ((thresh & 0x80000000u) ? 0x80000000u : 0xffffffffu));
        const float zt = __fdiv_rn(vt, a.temperature);
        const float zmax = ng > 0 ? zval(ck[ng - 1]) : zt;
        const float et = expf(zt - zmax);
        float part = 0.f;
        for (int j = tid; j < ng; j += kSampleThreads) {
            const float e = expf(zval(ck[j]) - zmax);
            ce[j] = e;
            part += e;
        }
        const float S = block_sum(part) + (float)ne * et;
        if (tid == 0) {
            int jj = C - 1;
            if (a.top_p < 1.f) {
                float cum = 0.f;
                const float pt = __fdiv_rn(et, S);
                for (int j = 0; j < C - 1; ++j) {
                    cum += j < ne ? pt : __fdiv_rn(ce[j - ne], S);
                    if (!(cum <= a.one_minus_p)) { jj = j; break; }
                }
            } else {
                jj = 0;
            }
            s_j0 = jj;
        }
        __syncthreads();
        j0 = s_j0;
        if (j0 >= ne) {   // only above candidates stay: the LDS path below, over them
            C = ng;
            j0 -= ne;
        } else {
            // tied tokens of tie rank >= j0 and every above one stay; the draw runs over
            // them in token order, one term at a time, by wave 0 reading the row in
            // chunks of 64 ids (lane order = id order): once for the total, once for
            // the search
            const float Sk = block_sum(tid < ng ? ce[tid] : 0.f) + (float)(ne - j0) * et;
            if (wave != 0) return;
            const float pt = __fdiv_rn(et, Sk);
            // the row's logit for lane l of the chunk at c0 (0 past the row)
            auto load = [&](int c0) { return c0 + lane < V ? lg[c0 + lane] : 0.f; };
            auto chunk = [&](int c0, float v, int& rank_base, float& p, bool& kept) {
                const int i = c0 + lane;
                const uint32_t key = order_key(v);
                const bool tied = i < V && key == thresh, above = i < V && key > thresh;
                const unsigned long long m = __ballot(tied);
                const int rank = rank_base + __popcll(m & ((1ull << lane) - 1ull));
                kept = above || (tied && rank >= j0);
                p = !kept ? 0.f : (tied ? pt : __fdiv_rn(expf(__fdiv_rn(v, a.temperature) - zmax), Sk));
                rank_base += __popcll(m);
            };
            float cdf = 0.f;
            int rb = 0;
            float vn = load(0);
            for (int c0 = 0; c0 < V; c0 += kWave) {
                const float v = vn;
                vn = load(c0 + kWave);   // the next chunk's load goes out before this one's sum
                float p;
                bool kept;
                chunk(c0, v, rb, p, kept);
                for (int l = 0; l < kWave; ++l) cdf += __shfl(p, l);   // adding 0 leaves the sum as it is
            }
            const float target = a.uniforms[row] * cdf;
            float run = 0.f;
            int tok = -1, last = -1;
            rb = 0;
            vn = load(0);
            for (int c0 = 0; c0 < V && tok < 0; c0 += kWave) {
                const float v = vn;
                vn = load(c0 + kWave);
                float p;
                bool kept;
                chunk(c0, v, rb, p, kept);
                const unsigned long long km = __ballot(kept);
                for (int l = 0; l < kWave; ++l) {
                    if (!((km >> l) & 1ull)) continue;
                    run += __shfl(p, l);
                    last = c0 + l;
                    if (run > target) { tok = c0 + l; break; }
                }
            }
            if (lane == 0) a.tokens[row] = tok >= 0 ? tok : last;
            return;
        }
    }

    // 4. the kept tokens back in token order (removed ones sort to the end), their
    //    e values carried along; S_kept by a tree sum; the draw
    for (int j = tid; j < kSampleCand; j += kSampleThreads) {
        if (j < C && j >= j0) {
            const uint32_t tok = (uint32_t)(ck[j] & 0xffffffffu);
            ck[j] = ((unsigned long long)tok << 32) | (uint32_t)__float_as_uint(ce[j]);
        } else {
            ck[j] = ~0ull;
        }
    }
    bitonic(C);
    const int nk = C - j0;
    float kp = 0.f;
    for (int j = tid; j < nk; j += kSampleThreads) kp += __uint_as_float((uint32_t)(ck[j] & 0xffffffffu));
    kp = group_sum<kWave>(kp);
    if (lane == 0) s_red[wave] = kp;
    __syncthreads();
    if (tid == 0) {
        float Sk = 0.f;
        for (int w = 0; w < kSampleThreads / kWave; ++w) Sk += s_red[w];
        float cdf = 0.f;
        for (int j = 0; j < nk; ++j) cdf += __fdiv_rn(__uint_as_float((uint32_t)(ck[j] & 0xffffffffu)), Sk);
        const float target = a.uniforms[row] * cdf;
        int tok = (int)(ck[nk - 1] >> 32);
        float run = 0.f;
        for (int j = 0; j < nk; ++j) {
            run += __fdiv_rn(__uint_as_float((uint32_t)(ck[j] & 0xffffffffu)), Sk);
            if (run > target) { tok = (int)(ck[j] >> 32); break; }
        }
        a.tokens[row] = tok;
    }
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t s) {
    if (a.B < 1 || a.V < 1 || (a.temperature > 0.f && a.top_k > kSampleMaxK && a.top_k < a.V))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(sample_kernel, dim3(a.B), dim3(kSampleThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace qd
