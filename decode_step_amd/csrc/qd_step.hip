// Batch-1 decode step as one persistent launch (gfx950, bf16 weights and KV).
//
// The forward is the same as the multi-launch step (nanoinfer, phase 3: the
// pre-norm block; nanoserve day 49: the new token's K/V are stored before it
// attends; Tang section 2.2: split attention merged by the online-softmax
// monoid). What differs is how the 256 compute units meet. A kernel boundary
// costs about 2 us of dispatch on this chip and a small product about 4 us,
// while a batch-1 layer of the 0.5B shape is 5 dependent products. Here one
// workgroup per CU lives through the whole step:
//
//  - wave 0 of each workgroup (the loader) streams the workgroup's share of every
//    weight matrix, layer after layer, into a ring of 1 KB LDS slots by LDS DMA,
//    as far ahead as the ring allows. Weights do not depend on the activations,
//    so HBM keeps streaming while the compute waves wait for their inputs, and
//    the compute waves' waits never sit behind weight loads in a vmcnt queue.
//  - waves 1..4 (the compute waves) wait only for activations, two ways:
//    * within an XCD (q|k|v to the attention, split partials to the merge) each
//      element travels as one 64-bit word (float value, 32-bit tag naming the
//      layer and phase that wrote it) through that XCD's L2 (plain store;
//      non-temporal load, which skips the CU's L1), and consumers poll the words
//      themselves: a 64-bit store is single-copy atomic, so no flag is needed.
//    * across XCDs (x, y_g, h) the producers store plain floats with sc1
//      (through the per-XCD L2 to memory), wait for those stores to be
//      acknowledged and then add 1 to a counter of their XCD; a consumer polls
//      the 8 counters (one lane each) and then reads the vector once. Polling
//      the data itself from every workgroup took most of the bandwidth the
//      weights need.
//  - the q|k|v rows, attention splits and o_proj columns of KV head g run on the
//    workgroups b with b mod 8 = g, so those two hand-offs stay in one L2 (the
//    dispatcher deals consecutive workgroups round robin over the 8 XCDs, from a
//    starting XCD that varies between launches, so equal b mod 8 means one XCD);
//    three hand-offs per layer cross XCDs.
//
// Per layer l (tag T(l, ph) = 8 (l + 1) + ph):
//   P0 qkv   (XCD g < Hkv)          q|k|v rows of group g = r * (W (x * g_attn)) + b
//   P1 attn  (XCD g, slot s < S)    q/k norm, RoPE, append, keys of split s
//   P2 o     (XCD g)                merge the splits; y_g = W_o[:, group g] ctx_g
//   P3 up    (all)                  x_a = x + sum_g y_g; h = silu(gate) * up
//   P4 down  (all)                  x = x_a + W_d h
// then the final norm and the lm_head with per-workgroup argmax partials.
//
// Every wait is bounded: a workgroup that waits too long records where in the
// error words and raises a global abort that every other wait also polls, so
// the grid always drains.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qd_device.h"
#include "qd_launch.h"
#include "qd_step_sched.h"

namespace qd {
namespace {

using namespace qd::step;
typedef unsigned long long u64;

__device__ __forceinline__ uint32_t tag_of(int l, int ph) { return (uint32_t)(8 * (l + 1) + ph); }
__device__ __forceinline__ u64 pack(float v, uint32_t t) { return (u64)__float_as_uint(v) | ((u64)t << 32); }
__device__ __forceinline__ float val_of(u64 w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ uint32_t tg_of(u64 w) { return (uint32_t)(w >> 32); }

// tagged words: sc1 for words other XCDs read, the XCD's L2 for words read within it
__device__ __forceinline__ void st_far(u64* p, u64 v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_near(u64* p, u64 v) { *p = v; }
__device__ __forceinline__ u64 ld_far(const u64* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 ld_near(const u64* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint32_t ld_far32(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_far32(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_farf(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes from memory past the L2 (sc1): a vector another XCD wrote
__device__ __forceinline__ float4 ld_far16(const float* base, int i4) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, 0x7fffffff, 0x00020000);
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, i4 * 16, 0, 16));
}

typedef __attribute__((address_space(3))) uint32_t lds_u32;
__device__ __forceinline__ uint32_t lds_ld(const uint32_t* p) { return *(volatile const lds_u32*)p; }
__device__ __forceinline__ void lds_st(uint32_t* p, uint32_t v) { *(volatile lds_u32*)p = v; }


// ---------------------------------------------------------------- shared state
struct Smem {
    uint8_t ring[kRingSlots * 1024];
    uint32_t xs_h[kXs], xs_l[kXs];  // a product's split input (bf16 hi / lo pairs)
    float work[kWork];              // P1: q|k|v, scores, per-wave P.V; P2: the split partials
    float xa[1024];                 // x_a (P3 -> P4)
    float2 rope[64];
    float wts[8 * 32];              // P2: merge weight of head h, split s
    uint32_t filled;                // slots whose DMA has landed (loader)
    uint32_t consumed[kNcw];        // slots each compute wave is done with
    uint32_t bar, abort_;
    float ssp[kNcw];                // sums of squares per compute wave
    float red_v[kNcw];
    int red_i[kNcw];
};

// The workgroup's LDS, at namespace scope so that every access to it compiles
// to LDS instructions (through a generic pointer they became flat accesses,
// which also wait on vmcnt: each one then waited for every DMA in flight).
__shared__ __attribute__((aligned(16))) Smem g_sm;

struct Ctl {
    const StepArgs* a;
    uint32_t bar_gen;
};

__device__ __forceinline__ void raise_abort(Ctl& c, uint32_t code) {
    if (__lane_id() == 0) {
        st_far32(c.a->err + 1, code);
        st_far32(c.a->err + 0, 1u);
        lds_st(&g_sm.abort_, 1u);
    }
}
// true when a wait must stop: an abort seen, or its budget spent
__device__ __forceinline__ bool spin_check(Ctl& c, uint32_t& it, uint32_t code) {
    ++it;
    if ((it & 15) == 0 && lds_ld(&g_sm.abort_)) return true;
    if ((it & 4095) == 0 && ld_far32(c.a->err)) {   // rare: the load waits for this wave's stores
        lds_st(&g_sm.abort_, 1u);
        return true;
    }
    if (it > kSpinMax) {
        raise_abort(c, code);
        return true;
    }
    return false;
}

// barrier of the compute waves only (the loader runs free): an LDS arrival counter
__device__ __forceinline__ bool cw_barrier(Ctl& c, uint32_t code) {
    c.bar_gen += kNcw;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    if (__lane_id() == 0) __hip_atomic_fetch_add(&g_sm.bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    uint32_t it = 0;
    while (lds_ld(&g_sm.bar) < c.bar_gen)
        if (spin_check(c, it, code)) return false;
    asm volatile("" ::: "memory");
    return true;
}

__device__ __forceinline__ bool wait_filled(Ctl& c, uint32_t slot_end, uint32_t code) {
    uint32_t it = 0;
    while (lds_ld(&g_sm.filled) < slot_end) {
        __builtin_amdgcn_s_sleep(1);
        if (spin_check(c, it, code)) return false;
    }
    asm volatile("" ::: "memory");
    return true;
}

// this wave is done reading every slot before slot_end
__device__ __forceinline__ void release(Ctl& c, int wave, uint32_t slot_end) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    if (__lane_id() == 0) lds_st(&g_sm.consumed[wave], slot_end);
}

// ring byte offset of byte `off` (< the ring's size) of a block starting at slot s0
__device__ __forceinline__ uint32_t ring_off(uint32_t s0, uint32_t off) {
    const uint32_t o = (s0 % kRingSlots) * 1024u + off;
    return o >= (uint32_t)(kRingSlots * 1024) ? o - kRingSlots * 1024 : o;
}
// element e of a bf16 vector held in a block at slot s0
__device__ __forceinline__ float ring_bf16(uint32_t s0, int e) {
    return bf16_to_f32(*(const uint16_t*)(g_sm.ring + ring_off(s0, (uint32_t)(2 * e))));
}

// Poll n tagged words (elements ct + 256 i, i < PER) until each tag equals `tag`;
// values go to dst[] (times the bf16 gains mul[] when given); *ss (when given)
// gains this lane's sum of their squares.
template <int PER, bool FAR>
__device__ __forceinline__ bool poll_vec(Ctl& c, const u64* src, int n, uint32_t tag, float* dst, const uint16_t* mul,
                         float* ss, int ct, uint32_t code) {
    uint32_t it = 0;
    for (;;) {
        u64 w[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = ct + 256 * i;
            const u64* p = src + (e < n ? e : 0);
            asm volatile("" ::: "memory");
            w[i] = FAR ? ld_far(p) : ld_near(p);
        }
        bool ok = true;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = ct + 256 * i;
            ok = ok && (e >= n || tg_of(w[i]) == tag);
        }
        if (__all(ok)) {
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int e = ct + 256 * i;
                if (e < n) {
                    const float v = val_of(w[i]);
                    if (ss) *ss += v * v;
                    dst[e] = mul ? v * bf16_to_f32(mul[e]) : v;
                }
            }
            return true;
        }
        __builtin_amdgcn_s_sleep(1);
        if (spin_check(c, it, code)) return false;
    }
}

// Completion counter of vector kind k (0: x after down, 1: y after o_proj, 2: h)
// of layer l written by XCD x; each sits in a 128-byte line of its own.
enum { CNT_X = 0, CNT_Y = 1, CNT_H = 2 };
__device__ __forceinline__ uint32_t* cnt_ptr(const StepArgs& a, int k, int l, int x) {
    return a.cnt + (((size_t)k * kStepMaxLayers + l) * kXcd + x) * 32;
}

// Producer side: this workgroup's sc1 stores of vector kind k are acknowledged
// (each compute wave waits for its own), then one lane adds 1 to its XCD's counter.
__device__ __forceinline__ bool publish(Ctl& c, int k, int l, int xcd, int wave, uint32_t code) {
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    if (!cw_barrier(c, code)) return false;
    if (wave == 0 && __lane_id() == 0)
        __hip_atomic_fetch_add(cnt_ptr(*c.a, k, l, xcd), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// Consumer side, compute wave 0: poll until every XCD's counter of (k0, l0)
// reaches its producer count (n_lo for XCDs below nx, n_hi for the others) and,
// when k1 >= 0, those of (k1, l1) likewise. The caller's barrier then releases
// the other waves.
__device__ __forceinline__ bool wait_counts(Ctl& c, int k0, int l0, int nx0, int lo0, int hi0, int k1, int l1, int nx1,
                                            int lo1, int hi1, uint32_t code) {
    const int lane = __lane_id();
    const bool second = lane >= kXcd && lane < 2 * kXcd && k1 >= 0;
    const int x = lane & (kXcd - 1);
    uint32_t need = 0;
    const uint32_t* p = c.a->cnt;
    if (lane < kXcd && l0 >= 0) { p = cnt_ptr(*c.a, k0, l0, x); need = x < nx0 ? lo0 : hi0; }
    else if (second && l1 >= 0) { p = cnt_ptr(*c.a, k1, l1, x); need = x < nx1 ? lo1 : hi1; }
    uint32_t it = 0;
    for (;;) {
        asm volatile("" ::: "memory");
        const uint32_t v = need ? ld_far32(p) : 0u;
        if (__all(v >= need)) return true;
        __builtin_amdgcn_s_sleep(2);
        if (spin_check(c, it, code)) return false;
    }
}

// ---------------------------------------------------------------- products from the ring
// A product's input vector (x after its norm gains, the merged context, h) is held
// as two bf16 vectors, hi = bf16(v) and lo = bf16(v - hi), packed in pairs like
// the weights, so each pair of weights takes two v_dot2_f32_bf16 (the products of
// two bf16 are exact in float32; hi + lo carries v to about 2^-17 relative). A
// float32 FMA per weight would take an extra instruction to widen each weight.
typedef __bf16 qd_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2(uint32_t w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(qd_bf16x2, w), __builtin_bit_cast(qd_bf16x2, x), acc,
                                           false);
}
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = f32x2_to_bf16x2(a, b);
    lo = f32x2_to_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}
// elements 4 q .. 4 q + 3 of the split input
__device__ __forceinline__ void xs_store4(int q, float4 v) {
    uint32_t h0, l0, h1, l1;
    split2(v.x, v.y, h0, l0);
    split2(v.z, v.w, h1, l1);
    *(uint2*)&g_sm.xs_h[2 * q] = make_uint2(h0, h1);
    *(uint2*)&g_sm.xs_l[2 * q] = make_uint2(l0, l1);
}
// one 16-byte chunk (8 weights) times the matching split input chunk
__device__ __forceinline__ float dot_chunk(const uint4 w, const uint4 h, const uint4 l, float acc) {
    acc = dot2(w.x, h.x, acc);
    acc = dot2(w.y, h.y, acc);
    acc = dot2(w.z, h.z, acc);
    acc = dot2(w.w, h.w, acc);
    acc = dot2(w.x, l.x, acc);
    acc = dot2(w.y, l.y, acc);
    acc = dot2(w.z, l.z, acc);
    acc = dot2(w.w, l.w, acc);
    return acc;
}

// A product row is read by one wave at a time, lane i taking 16-byte chunks i,
// i + 64, ...: each LDS read is then 1 KB of consecutive bytes. (Rows are 1792 or
// 9728 bytes long, multiples of 256: with several rows per wave at once, the rows'
// lanes met in the same LDS banks and every read cost several times over.) The
// input's chunks of the lane stay in registers for the whole product; chunks at or
// past the row's end are zero.
template <int NJ>
struct XW {
    uint4 h[NJ], l[NJ];
};
template <int NJ>
__device__ __forceinline__ void load_xw(XW<NJ>& x, int lane, int nch) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int c = lane + 64 * j;
        x.h[j] = make_uint4(0u, 0u, 0u, 0u);
        x.l[j] = x.h[j];
        if (c < nch) {
            x.h[j] = *(const uint4*)&g_sm.xs_h[4 * c];
            x.l[j] = *(const uint4*)&g_sm.xs_l[4 * c];
        }
    }
}

constexpr uint32_t kRingBytes = kRingSlots * 1024u;

// ring byte offset of byte `off` of a block that starts at absolute slot s0
__device__ __forceinline__ uint32_t ring_at(uint32_t s0, uint32_t off) {
    const uint32_t o = (s0 % kRingSlots) * 1024u + off;
    return o >= kRingBytes ? o - kRingBytes : o;
}

// R rows (ring byte offsets rb[r], wave-uniform; rows whose bit of `mask` is clear
// are skipped) of nch chunks times the input: out[r] is the full sum in every lane.
// Every chunk load of the R rows is issued before the first product.
template <int NJ, int R>
__device__ __forceinline__ void rows_dot(const uint32_t (&rb)[R], uint32_t mask, int lane, int nch, const XW<NJ>& x,
                                         float (&out)[R]) {
    uint4 w[R][NJ];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint32_t b = __builtin_amdgcn_readfirstlane(rb[r]);
        const bool flat = b + (uint32_t)nch * 16u <= kRingBytes;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int c = lane + 64 * j;
            w[r][j] = make_uint4(0u, 0u, 0u, 0u);
            if (((mask >> r) & 1u) && c < nch) {
                uint32_t o = b + (uint32_t)c * 16u;
                if (!flat) o = o >= kRingBytes ? o - kRingBytes : o;
                w[r][j] = *(const uint4*)(g_sm.ring + o);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float acc = dot_chunk(w[r][0], x.h[0], x.l[0], 0.f);
#pragma unroll
        for (int j = 1; j < NJ; ++j) acc = dot_chunk(w[r][j], x.h[j], x.l[j], acc);
        out[r] = group_sum<64>(acc);
    }
}

// One row per wave with the input read from LDS beside each weight chunk, NG chunks
// at a time: for a product whose rows are used once per wave (the down product),
// holding the input in registers would not be repaid.
template <int NG>
__device__ __forceinline__ float row_dot_lds(uint32_t rb, int lane, int nch) {
    const uint32_t b = __builtin_amdgcn_readfirstlane(rb);
    const bool flat = b + (uint32_t)nch * 16u <= kRingBytes;
    float acc = 0.f;
    for (int c0 = 0; c0 < nch; c0 += 64 * NG) {
        uint4 w[NG], xh[NG], xl[NG];
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            const int c = c0 + lane + 64 * j;
            w[j] = make_uint4(0u, 0u, 0u, 0u);
            xh[j] = w[j];
            xl[j] = w[j];
            if (c < nch) {
                uint32_t o = b + (uint32_t)c * 16u;
                if (!flat) o = o >= kRingBytes ? o - kRingBytes : o;
                w[j] = *(const uint4*)(g_sm.ring + o);
                xh[j] = *(const uint4*)&g_sm.xs_h[4 * c];
                xl[j] = *(const uint4*)&g_sm.xs_l[4 * c];
            }
        }
#pragma unroll
        for (int j = 0; j < NG; ++j) acc = dot_chunk(w[j], xh[j], xl[j], acc);
    }
    return group_sum<64>(acc);
}

// Rows [0, nrows) of a packed bf16 block at slot s0 (row i at byte i * seg): wave
// w takes rows w R .. w R + R - 1, then the next 4 R, ...; fn(row, sum) runs on
// lane 0 of the wave.
template <int NJ, int R, typename Fn>
__device__ __forceinline__ void block_rows(uint32_t s0, int nrows, int seg, const XW<NJ>& x, int wave, int lane,
                                           Fn fn) {
    const int nch = seg >> 4;
    for (int r0 = wave * R; r0 < nrows; r0 += kNcw * R) {
        uint32_t rb[R];
#pragma unroll
        for (int r = 0; r < R; ++r) rb[r] = ring_at(s0, (uint32_t)((r0 + r) * seg));
        float out[R];
        const int nv = nrows - r0 < R ? nrows - r0 : R;
        rows_dot<NJ, R>(rb, (1u << nv) - 1u, lane, nch, x, out);
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (r0 + r < nrows) fn(r0 + r, out[r]);
        }
    }
}

// Far vector loads (another XCD wrote them): n floats (n a multiple of 4) as
// 16-byte chunks, chunk q to compute thread q % 256.
// RMSNorm input: x (times the bf16 gains of the block at ring slot gs) goes to
// the split input; the lane's sum of squares of x is returned.
__device__ __forceinline__ float load_norm_input(const float* src, int n, uint32_t gs, int ct) {
    float ss = 0.f;
    for (int q = ct; q < (n >> 2); q += 256) {
        const float4 v = ld_far16(src, q);
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        const uint2 gw = *(const uint2*)(g_sm.ring + ring_off(gs, (uint32_t)(8 * q)));
        xs_store4(q, make_float4(v.x * bf16_to_f32(gw.x & 0xffffu), v.y * bf16_to_f32(gw.x >> 16),
                                 v.z * bf16_to_f32(gw.y & 0xffffu), v.w * bf16_to_f32(gw.y >> 16)));
    }
    return ss;
}

// 1/sqrt(mean of squares + eps) from the four compute waves' partial sums (each
// wave publishes its lanes' sum before a barrier; every wave adds them in order)
__device__ __forceinline__ void ss_publish(float* part, int wave, float ss) {
    ss = group_sum<64>(ss);
    if (__lane_id() == 0) part[wave] = ss;
}
__device__ __forceinline__ float ss_scale(const float* part, int D, float eps) {
    const float ss = ((part[0] + part[1]) + part[2]) + part[3];
    return 1.0f / sqrtf(ss / (float)D + eps);
}

// s_waitcnt vmcnt(n) for a run-time n (the count is an immediate of the instruction)
template <int N>
__device__ __forceinline__ void wait_vm_case(uint32_t n) {
    if constexpr (N >= 0) {
        if (n == (uint32_t)N) __builtin_amdgcn_s_waitcnt(wait_vm(N));
        else wait_vm_case<N - 1>(n);
    }
}
__device__ __forceinline__ void wait_vm_at_most(uint32_t n) {
    if (n >= (uint32_t)kMaxOut) return;
    wait_vm_case<kMaxOut - 1>(n);
}

// ---------------------------------------------------------------- the loader wave
__device__ __forceinline__ void loader(const StepArgs& a, const Sched& S, Ctl& c) {
    const int lane = __lane_id();
    uint32_t slot = 0, outst = 0;
    // page ids of this workgroup's attention split (lane i: page i)
    int my_page = 0;
    if (S.npg > 0 && lane < S.npg) {
        my_page = a.block_table[S.pg0 + lane];
        if (my_page < 0 || my_page >= a.num_pages) my_page = -1;
    }
    if (__any(my_page < 0)) {
        raise_abort(c, 0x100u);
        return;
    }
    const uint32_t ring_lds = __builtin_amdgcn_readfirstlane(lds_addr(g_sm.ring));
    auto publish = [&]() { if (lane == 0) lds_st(&g_sm.filled, slot - outst); };
    auto free_slot = [&]() {   // lowest slot some compute wave still needs
        uint32_t m = lds_ld(&g_sm.consumed[0]);
#pragma unroll
        for (int w = 1; w < kNcw; ++w) m = min(m, lds_ld(&g_sm.consumed[w]));
        return m;
    };
    bool stop = false;
    uint32_t lim = kRingSlots;   // slots below lim are free to fill
    // One block: its slots go out in batches of kBatch DMAs (one per slot), progress
    // published every batch once at least kBatch DMAs have landed. Every count and
    // address but the lane's 16-byte offset is wave-uniform (scalar registers), so a
    // full batch is kBatch address adds and DMAs: with the counts in vector registers
    // and a lane mask around each DMA the loop issued at under half the rate one wave
    // can stream.
    const uint32_t lane16 = (uint32_t)lane * 16u;
    auto issue = [&](const Blk& b) {
        const uint32_t bytes = __builtin_amdgcn_readfirstlane((uint32_t)blk_bytes(b));
        const uint32_t ns = (bytes + 1023) >> 10;
        const bool flat = __builtin_amdgcn_readfirstlane(b.rows) == 1;
        // the block's address in scalar registers (sgpr_gptr joins the two 32-bit halves
        // as unsigned: readfirstlane returns int, and a sign-extended low half set the
        // upper 32 bits whenever bit 31 of an address was set)
        const char* src = (const char*)sgpr_gptr(b.src);
        uint32_t i = 0;
        while (i < ns && !stop) {
            slot = __builtin_amdgcn_readfirstlane(slot);
            outst = __builtin_amdgcn_readfirstlane(outst);
            lim = __builtin_amdgcn_readfirstlane(lim);
            if (slot + kBatch > lim) {   // slots may still be held by a compute wave
                lim = __builtin_amdgcn_readfirstlane(free_slot()) + kRingSlots;
                uint32_t it = 0;
                while (slot >= lim) {
                    // let the oldest DMAs land and publish them (the rest stay in flight)
                    if (outst > 0) {
                        const uint32_t keep = outst > kBatch ? outst - kBatch : 0;
                        wait_vm_at_most(keep);
                        outst = keep;
                        publish();
                    } else {
                        __builtin_amdgcn_s_sleep(2);
                    }
                    if (spin_check(c, it, 0x200u)) { stop = true; return; }
                    lim = __builtin_amdgcn_readfirstlane(free_slot()) + kRingSlots;
                }
            }
            const uint32_t n = __builtin_amdgcn_readfirstlane(min(min((uint32_t)kBatch, ns - i), lim - slot));
            const uint32_t d0 = __builtin_amdgcn_readfirstlane(slot % kRingSlots);
            const uint32_t lds0 = __builtin_amdgcn_readfirstlane(ring_lds + d0 * 1024u);
            if (flat && n == (uint32_t)kBatch && (i + kBatch) * 1024u <= bytes && d0 + kBatch <= (uint32_t)kRingSlots) {
                const char* p = src + (size_t)i * 1024 + lane16;
#pragma unroll
                for (int j = 0; j < kBatch; ++j) lds_dma16(p + j * 1024, __builtin_amdgcn_readfirstlane(lds0 + j * 1024u));
            } else {
                for (uint32_t j = 0; j < n; ++j) {
                    bool on;
                    const char* sp = dma_src(b, i + j, (uint32_t)lane, &on);
                    const uint32_t d = __builtin_amdgcn_readfirstlane(ring_lds + ((d0 + j) % kRingSlots) * 1024u);
                    if (on) lds_dma16(sp, d);   // lane 0 always: one DMA per slot
                }
            }
            slot += n;
            i += n;
            outst += n;
            if (outst > (uint32_t)(kMaxOut - kBatch)) {
                __builtin_amdgcn_s_waitcnt(wait_vm(kMaxOut - 2 * kBatch));
                outst = kMaxOut - 2 * kBatch;
                publish();
            }
        }
    };
    for (int l = 0; l < a.L && !stop; ++l) {
        for (int ph = PH_QKV; ph <= PH_DOWN && !stop; ++ph) {
            const int nb = n_blocks(a, S, ph);
            for (int k = 0; k < nb && !stop; ++k) {
                if (ph == PH_ATTN) {
                    int kk = k;
                    if (a.qk_norm) {
                        if (kk < 2) { issue(get_block(a, S, l, ph, kk)); continue; }
                        kk -= 2;
                    }
                    const int isv = kk >= S.npg, i = isv ? kk - S.npg : kk;
                    issue(page_block(a, l, S.xcd, __builtin_amdgcn_readlane(my_page, i), isv));
                } else {
                    issue(get_block(a, S, l, ph, k));
                }
            }
        }
    }
    const int nh = n_blocks(a, S, PH_HEAD);
    for (int k = 0; k < nh && !stop; ++k) issue(get_block(a, S, 0, PH_HEAD, k));
    __builtin_amdgcn_s_waitcnt(wait_vm(0));   // no DMA outlives the kernel
    outst = 0;
    publish();
}

// ---------------------------------------------------------------- the compute waves
// The thread index as a value the compiler cannot see through: each phase derives
// its LDS addresses and lane masks from it, so they are recomputed in the phase
// instead of being hoisted out of the layer loop, where the addresses and masks of
// every phase at once spilled.
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}
__device__ __forceinline__ uint32_t take(uint32_t& cur, const Blk& b) {
    const uint32_t s0 = cur;
    cur += blk_slots(b);
    return s0;
}

// P1's work buffer: q heads, k, v (G + 2 vectors of 64), then the scores of head h
// at kScOff + 256 h (keys of the split), then the per-wave P.V sums.
constexpr int kScOff = 640;
constexpr int kPvOff = kScOff + 8 * 256;
static_assert(kPvOff + kNcw * 512 <= kWork, "P1 work buffer");

__device__ __forceinline__ void compute(const StepArgs& a, const Sched& S, Ctl& c) {
    const int ct = threadIdx.x - 64;          // 0..255
    const int wave = ct >> 6, lane = ct & 63;
    const int D = a.D, hd = a.hd, G = a.G, F = a.F;
    const bool grp = S.xcd < a.Hkv;
    const int g = S.xcd;
    const int p = S.p;
    uint32_t cur = 0;   // absolute ring slot of the next block
    // The new token's k and v (lane d: dimension d) wait in registers from P1 to P3:
    // stored in P1 they held up the next load of the wave (loads and stores share
    // one in-order counter) until the cache had taken them.
    uint32_t app = 0;
    bool has_app = false;
    for (int i = ct; i < hd / 2; i += 256) g_sm.rope[i] = a.rope[i];
    float* const XB = a.xb;
    for (int l = 0; l < a.L; ++l) {
        const int par = l & 1, ppar = (l + 1) & 1;   // this layer's buffers, the previous layer's
        const StepLayer& L = a.layer[l];
        // ------------------------------------------------------------ P0: q|k|v of group g
        if (grp) {
            const Blk gb = get_block(a, S, l, PH_QKV, 0);
            const uint32_t gs = take(cur, gb);
            if (!wait_filled(c, gs + blk_slots(gb), 0x1000u | l)) return;
            if (l > 0) {   // layer 0 reads the prologue's x
                if (wave == 0 && !wait_counts(c, CNT_X, l - 1, kXcd, kSlotsPerXcd, kSlotsPerXcd, -1, 0, 0, 0, 0,
                                              0x1050u | l)) return;
                if (!cw_barrier(c, 0x1060u | l)) return;
            }
            ss_publish(g_sm.ssp, wave, load_norm_input(XB + (size_t)ppar * D, D, gs, ct));
            if (!cw_barrier(c, 0x1200u | l)) return;
            const float r = ss_scale(g_sm.ssp, D, a.eps);
            const int lno = opaque(lane);
            XW<2> x;
            load_xw<2>(x, lno, D >> 3);
            const int np = qkv_nparts(a, S.slot);
            u64* out = a.qkv + (size_t)par * a.qkvr;
            const uint32_t tg = tag_of(l, PH_QKV);
            for (int k = 0; k < np; ++k) {
                const QkvPart q = qkv_part(a, g, S.slot, k);
                uint32_t bs = 0;
                int boff = 0;
                if (a.has_bias) {
                    bs = take(cur, get_block(a, S, l, PH_QKV, 1 + 2 * k));
                    boff = (int)(((long)q.r0 * 2) & 15L);
                }
                const Blk wb = get_block(a, S, l, PH_QKV, a.has_bias ? 2 + 2 * k : 1 + k);
                const uint32_t ws = take(cur, wb);
                if (!wait_filled(c, ws + blk_slots(wb), 0x1300u | l)) return;
                const bool hb = a.has_bias;
                block_rows<2, 4>(ws, q.n, D * 2, x, wave, lno, [&](int row, float s) {
                    float v = r * s;
                    if (hb) v += bf16_to_f32(*(const uint16_t*)(g_sm.ring + ring_off(bs, (uint32_t)(boff + 2 * row))));
                    st_near(out + q.out0 + row, pack(v, tg));
                });
            }
            release(c, wave, cur);
        }
        // ------------------------------------------------------------ P1: attention over split s
        if (grp && S.slot < a.S) {
            const int s = S.slot;
            uint32_t qns = 0, kns = 0;
            if (a.qk_norm) {
                qns = take(cur, get_block(a, S, l, PH_ATTN, 0));
                kns = take(cur, get_block(a, S, l, PH_ATTN, 1));
            }
            // the split's K pages, then its V pages: 2 slots (16 rows of 128 bytes) each,
            // so 8 keys fill one slot
            const uint32_t kp0 = cur;
            cur += 2 * S.npg;
            const uint32_t vp0 = cur;
            cur += 2 * S.npg;
            float* qv = g_sm.work;   // q heads of group g, then k, then v
            const u64* qkvb = a.qkv + (size_t)par * a.qkvr;
            const int qn = G * 64;
            const uint32_t tg = tag_of(l, PH_QKV);
            if (!poll_vec<2, false>(c, qkvb + (size_t)g * qn, qn, tg, qv, nullptr, nullptr, ct, 0x2100u | l)) return;
            if (!poll_vec<1, false>(c, qkvb + (size_t)a.Hq * 64 + g * 64, 64, tg, qv + qn, nullptr, nullptr, ct,
                                    0x2101u | l)) return;
            if (!poll_vec<1, false>(c, qkvb + (size_t)(a.Hq + a.Hkv) * 64 + g * 64, 64, tg, qv + qn + 64, nullptr,
                                    nullptr, ct, 0x2102u | l)) return;
            if (!wait_filled(c, cur, 0x2103u | l)) return;   // norms and K/V pages landed
            if (!cw_barrier(c, 0x2200u | l)) return;
            // ring position of row t's bytes of page block `p0` (rows 0-7 in its first slot)
            auto row_off = [&](uint32_t p0, int t) {
                const int pi = t / 16 - S.pg0, rr = t % 16;
                return ring_off(p0 + 2 * pi + (rr >> 3), (uint32_t)((rr & 7) * 128));
            };
            // vectors 0..G-1 (q heads) and G (k): per-head RMSNorm with the shared gains,
            // then the half-split rotation (element i pairs with i + 32). q, scaled by
            // 1/sqrt(hd) log2(e) so scores come out in base 2, goes to the split input
            // (head h at word 32 h); the new k and v, rounded to bf16, go to the cache and
            // into the ring rows of position p.
            const float qscale = a.scale * 1.4426950408889634f;
            for (int v = wave; v <= G; v += kNcw) {
                float e0 = qv[v * 64 + lane];
                if (a.qk_norm) {
                    const float ss = group_sum<64>(e0 * e0);
                    const float rr = 1.0f / sqrtf(ss / 64.0f + a.eps);
                    e0 = e0 * rr * ring_bf16(v < G ? qns : kns, lane);
                }
                const float partner = __shfl_xor(e0, 32);
                const float2 cs = g_sm.rope[lane & 31];
                const float o0 = lane < 32 ? e0 * cs.x - partner * cs.y : e0 * cs.x + partner * cs.y;
                if (v < G) {
                    const float qs = o0 * qscale;
                    const float nb = dpp_f<kDppQuadXor1>(qs);   // element lane ^ 1
                    if ((lane & 1) == 0) {
                        uint32_t hi, lo;
                        split2(qs, nb, hi, lo);
                        g_sm.xs_h[v * 32 + (lane >> 1)] = hi;
                        g_sm.xs_l[v * 32 + (lane >> 1)] = lo;
                    }
                } else if (p / a.C == s) {   // the split holding p appends the new K/V
                    const uint16_t kb = f32_to_bf16(o0), vb16 = f32_to_bf16(qv[qn + 64 + lane]);
                    *(uint16_t*)(g_sm.ring + row_off(kp0, p) + 2 * lane) = kb;
                    *(uint16_t*)(g_sm.ring + row_off(vp0, p) + 2 * lane) = vb16;
                    app = (uint32_t)kb | ((uint32_t)vb16 << 16);   // stored to the cache in P3
                    has_app = true;
                }
            }
            if (!cw_barrier(c, 0x2400u | l)) return;
            const int t0 = s * a.C, nk = min(a.C, p + 1 - t0), ngr = (nk + 7) >> 3;
            float* sc = g_sm.work + kScOff;
            // scores: key group i (8 keys, one ring slot) to wave i % 4; lane (key kk,
            // chunk cc) takes 16 bytes of key kk's row and chunk cc of every q head
            {
                const int lno = opaque(lane);
                const int kk = lno >> 3, cc = lno & 7;
                for (int gi = wave; gi < ngr; gi += kNcw) {
                    const uint4 kv = *(const uint4*)(g_sm.ring + ring_off(kp0 + gi, (uint32_t)lno * 16u));
                    float mine = 0.f;
#pragma unroll
                    for (int h = 0; h < 8; ++h) {
                        if (h < G) {
                            const uint4 qh = *(const uint4*)&g_sm.xs_h[h * 32 + cc * 4];
                            const uint4 ql = *(const uint4*)&g_sm.xs_l[h * 32 + cc * 4];
                            const float sh = group_sum<8>(dot_chunk(kv, qh, ql, 0.f));
                            mine = cc == h ? sh : mine;
                        }
                    }
                    const int t = gi * 8 + kk;
                    if (cc < G) sc[cc * 256 + t] = t < nk ? mine : -INFINITY;
                }
            }
            if (!cw_barrier(c, 0x2500u | l)) return;
            // softmax of head h (wave h % 4): max, 2^(s - max) in place, sum
            for (int h = wave; h < G; h += kNcw) {
                float* sr = sc + h * 256;
                float v4[4];
                float m = -INFINITY;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = lane + 64 * i;
                    v4[i] = t < nk ? sr[t] : -INFINITY;
                    m = fmaxf(m, v4[i]);
                }
                m = wave_max(m);
                float ls = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = lane + 64 * i;
                    const float pe = t < nk ? exp2f(v4[i] - m) : 0.f;
                    if (t < ngr * 8) sr[t] = pe;
                    ls += pe;
                }
                ls = group_sum<64>(ls);
                if (lane == 0) {
                    g_sm.wts[2 * h] = m;
                    g_sm.wts[2 * h + 1] = ls;
                }
            }
            if (!cw_barrier(c, 0x2600u | l)) return;
            // P.V: lane (head hh, chunk cc) sums its 8 output dimensions over the key
            // groups of its wave
            {
                const int lno = opaque(lane);
                const int hh = lno >> 3, cc = lno & 7;
                float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                if (hh < G) {
                    for (int gi = wave; gi < ngr; gi += kNcw) {
                        const float4 p0 = *(const float4*)&sc[hh * 256 + gi * 8];
                        const float4 p1 = *(const float4*)&sc[hh * 256 + gi * 8 + 4];
                        const float pk[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
                        const uint32_t vb = ring_off(vp0 + gi, (uint32_t)cc * 16u);
                        uint4 vv[8];
#pragma unroll
                        for (int k = 0; k < 8; ++k) vv[k] = *(const uint4*)(g_sm.ring + vb + k * 128);
#pragma unroll
                        for (int k = 0; k < 8; ++k) {
                            float f[8];
                            widen16(vv[k], f);
#pragma unroll
                            for (int j = 0; j < 8; ++j) o[j] += pk[k] * f[j];
                        }
                    }
                    float* pv = g_sm.work + kPvOff + wave * 512 + hh * 64 + cc * 8;
                    *(float4*)pv = make_float4(o[0], o[1], o[2], o[3]);
                    *(float4*)(pv + 4) = make_float4(o[4], o[5], o[6], o[7]);
                }
            }
            if (!cw_barrier(c, 0x2700u | l)) return;
            // the split's partial of head h: the sum over the waves (fixed order), then
            // its max and sum of exponentials
            u64* part = a.part + (size_t)par * a.part_stride + ((size_t)g * a.S + s) * G * 66;
            const uint32_t ta = tag_of(l, PH_ATTN);
            for (int e = ct; e < G * 64; e += 256) {
                const float* pv = g_sm.work + kPvOff + e;
                const float sum = ((pv[0] + pv[512]) + pv[1024]) + pv[1536];
                st_near(part + (e >> 6) * 66 + (e & 63), pack(sum, ta));
            }
            if (ct < G) {
                st_near(part + ct * 66 + 64, pack(g_sm.wts[2 * ct], ta));
                st_near(part + ct * 66 + 65, pack(g_sm.wts[2 * ct + 1], ta));
            }
            release(c, wave, cur);
            if (!cw_barrier(c, 0x2800u | l)) return;   // the work buffer is free again
        }
        // ------------------------------------------------------------ P2: split merge, o_proj (group columns)
        if (grp) {
            const Blk ob = get_block(a, S, l, PH_O, 0);
            const uint32_t os = take(cur, ob);
            float* pin = g_sm.work;
            const int stride_s = G * (hd + 2);
            const u64* part = a.part + (size_t)par * a.part_stride + (size_t)g * a.S * stride_s;
            if (!poll_vec<20, false>(c, part, a.S * stride_s, tag_of(l, PH_ATTN), pin, nullptr, nullptr, ct,
                                     0x3100u | l)) return;
            if (!cw_barrier(c, 0x3200u | l)) return;
            // weight of split s for head h: 2^(m_s - M) / sum_s 2^(m_s - M) l_s
            for (int h = wave; h < G; h += kNcw) {
                const bool on = lane < a.S;
                const float ms = on ? pin[lane * stride_s + h * (hd + 2) + hd] : -INFINITY;
                const float M = wave_max(ms);
                const float w = on ? exp2f(ms - M) : 0.f;
                const float lt = group_sum<64>(on ? w * pin[lane * stride_s + h * (hd + 2) + hd + 1] : 0.f);
                if (on) g_sm.wts[h * 32 + lane] = w / lt;
            }
            if (!cw_barrier(c, 0x3300u | l)) return;
            // ctx[h][d] = sum_s w[h][s] o_s[h][d], two elements per thread, into the split input
            for (int e2 = ct; e2 < G * 32; e2 += 256) {
                const int h = e2 >> 5, d = 2 * (e2 & 31);
                float c0 = 0.f, c1 = 0.f;
                const float* ps = pin + h * (hd + 2) + d;
                for (int s = 0; s < a.S; ++s) {
                    const float w = g_sm.wts[h * 32 + s];
                    const float2 o2 = *(const float2*)(ps + s * stride_s);
                    c0 += w * o2.x;
                    c1 += w * o2.y;
                }
                uint32_t hi, lo;
                split2(c0, c1, hi, lo);
                g_sm.xs_h[e2] = hi;
                g_sm.xs_l[e2] = lo;
            }
            if (!wait_filled(c, os + blk_slots(ob), 0x3400u | l)) return;
            if (!cw_barrier(c, 0x3500u | l)) return;
            const int lno = opaque(lane);
            XW<1> x;
            load_xw<1>(x, lno, G * 8);
            const int r0 = S.slot * D / kSlotsPerXcd;
            float* y = a.y + ((size_t)par * a.Hkv + g) * D + r0;
            block_rows<1, 4>(os, ob.rows, ob.seg, x, wave, lno, [&](int row, float v) { st_farf(y + row, v); });
            release(c, wave, cur);
            if (!publish(c, CNT_Y, l, S.xcd, wave, 0x3600u | l)) return;
        }
        // ------------------------------------------------------------ P3: x_a, RMSNorm, gate|up, SwiGLU
        {
            const Blk gb = get_block(a, S, l, PH_UP, 0);
            const uint32_t gs = take(cur, gb);
            if (!wait_filled(c, gs + blk_slots(gb), 0x4120u | l)) return;
            // x of the previous layer (all XCDs) and y_g of this one (XCDs < Hkv)
            if (wave == 0 && !wait_counts(c, CNT_X, l - 1, kXcd, l > 0 ? kSlotsPerXcd : 0, l > 0 ? kSlotsPerXcd : 0,
                                          CNT_Y, l, a.Hkv, kSlotsPerXcd, 0, 0x4100u | l)) return;
            if (!cw_barrier(c, 0x4200u | l)) return;
            // x_a = x + sum_g y_g (fixed order) into xa; x_a * g_mlp into the split input
            {
                float ss = 0.f;
                const float* xs = XB + (size_t)ppar * D;
                const float* ys = a.y + (size_t)par * a.Hkv * D;
                for (int q = ct; q < D / 4; q += 256) {
                    float4 v = ld_far16(xs, q);
                    for (int gg = 0; gg < a.Hkv; ++gg) {
                        const float4 yv = ld_far16(ys + (size_t)gg * D, q);
                        v.x += yv.x; v.y += yv.y; v.z += yv.z; v.w += yv.w;
                    }
                    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
                    *(float4*)&g_sm.xa[4 * q] = v;
                    const uint2 gw = *(const uint2*)(g_sm.ring + ring_off(gs, (uint32_t)(8 * q)));
                    xs_store4(q, make_float4(v.x * bf16_to_f32(gw.x & 0xffffu), v.y * bf16_to_f32(gw.x >> 16),
                                             v.z * bf16_to_f32(gw.y & 0xffffu), v.w * bf16_to_f32(gw.y >> 16)));
                }
                ss_publish(g_sm.ssp, wave, ss);
            }
            if (has_app) {
                if (S.pid_p >= 0) {
                    const long off = (((long)S.pid_p * a.Hkv + g) * 16 + (p % 16)) * 64;
                    ((uint16_t*)L.kc)[off + lane] = (uint16_t)(app & 0xffffu);
                    ((uint16_t*)L.vc)[off + lane] = (uint16_t)(app >> 16);
                }
                has_app = false;
            }
            if (!cw_barrier(c, 0x4300u | l)) return;
            const float r = ss_scale(g_sm.ssp, D, a.eps);
            const int lno = opaque(lane);
            XW<2> x;
            load_xw<2>(x, lno, D >> 3);
            const int nblk = (S.f1 - S.f0 + kP3Rows - 1) / kP3Rows;
            float* hout = a.h + (size_t)par * F;
            // block pair k (8 gate rows, then the same 8 up rows): wave w takes rows 2 w
            // and 2 w + 1 of both
            const int row = 2 * wave;
            for (int k = 0; k < nblk; ++k) {
                const Blk bg = get_block(a, S, l, PH_UP, 1 + 2 * k);
                const uint32_t sg = take(cur, bg);
                const Blk bu = get_block(a, S, l, PH_UP, 2 + 2 * k);
                const uint32_t su = take(cur, bu);
                if (!wait_filled(c, su + blk_slots(bu), 0x4500u | l)) return;
                const int n = bg.seg / (D * 2);
                const uint32_t rb[4] = {ring_at(sg, (uint32_t)(row * D * 2)), ring_at(sg, (uint32_t)((row + 1) * D * 2)),
                                        ring_at(su, (uint32_t)(row * D * 2)), ring_at(su, (uint32_t)((row + 1) * D * 2))};
                const uint32_t m2 = row + 1 < n ? 3u : row < n ? 1u : 0u;
                float o[4];
                rows_dot<2, 4>(rb, m2 | (m2 << 2), lno, D >> 3, x, o);
                if (lno == 0) {
                    if (row < n) st_farf(hout + S.f0 + k * kP3Rows + row, silu(r * o[0]) * (r * o[2]));
                    if (row + 1 < n) st_farf(hout + S.f0 + k * kP3Rows + row + 1, silu(r * o[1]) * (r * o[3]));
                }
                release(c, wave, cur);
            }
            release(c, wave, cur);
            if (!publish(c, CNT_H, l, S.xcd, wave, 0x4600u | l)) return;
        }
        // ------------------------------------------------------------ P4: down + residual
        {
            const Blk db = get_block(a, S, l, PH_DOWN, 0);
            const uint32_t ds = take(cur, db);
            if (wave == 0 && !wait_counts(c, CNT_H, l, kXcd, kSlotsPerXcd, kSlotsPerXcd, -1, 0, 0, 0, 0, 0x5100u | l))
                return;
            if (!cw_barrier(c, 0x5150u | l)) return;
            {
                const float* hs = a.h + (size_t)par * F;
                float4 v[5];
#pragma unroll
                for (int i = 0; i < 5; ++i) {
                    const int q = ct + 256 * i;
                    v[i] = ld_far16(hs, q < F / 4 ? q : 0);
                }
#pragma unroll
                for (int i = 0; i < 5; ++i) {
                    const int q = ct + 256 * i;
                    if (q < F / 4) xs_store4(q, v[i]);
                }
            }
            if (!wait_filled(c, ds + blk_slots(db), 0x5200u | l)) return;
            if (!cw_barrier(c, 0x5300u | l)) return;
            const int lno = opaque(lane);
            float* xo = XB + (size_t)par * D + S.d0;
            const bool last = l == a.L - 1;
            const int d0 = S.d0;
            for (int row = wave; row < S.d1 - S.d0; row += kNcw) {
                const float v = row_dot_lds<5>(ring_at(ds, (uint32_t)(row * F * 2)), lno, F >> 3);
                if (lno == 0) {
                    const float xn = g_sm.xa[d0 + row] + v;
                    st_farf(xo + row, xn);
                    if (a.layer_out) a.layer_out[(size_t)l * D + d0 + row] = xn;
                    if (last && a.x_out) a.x_out[d0 + row] = xn;
                }
            }
            release(c, wave, cur);
            if (!publish(c, CNT_X, l, S.xcd, wave, 0x5500u | l)) return;
        }
    }
    // ---------------------------------------------------------------- final norm, lm_head, argmax partials
    if (a.lm_head) {
        const int nb = n_blocks(a, S, PH_HEAD);
        const Blk gb = get_block(a, S, 0, PH_HEAD, 0);
        const uint32_t gs = take(cur, gb);
        if (!wait_filled(c, gs + blk_slots(gb), 0x6000u)) return;
        const int lp = (a.L - 1) & 1;
        if (wave == 0 && !wait_counts(c, CNT_X, a.L - 1, kXcd, kSlotsPerXcd, kSlotsPerXcd, -1, 0, 0, 0, 0, 0x6050u))
            return;
        if (!cw_barrier(c, 0x6060u)) return;
        ss_publish(g_sm.ssp, wave, load_norm_input(XB + (size_t)lp * D, D, gs, ct));
        if (!cw_barrier(c, 0x6200u)) return;
        const float r = ss_scale(g_sm.ssp, D, a.eps);
        const int lno = opaque(lane);
        XW<2> x;
        load_xw<2>(x, lno, D >> 3);
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        for (int k = 1; k < nb; ++k) {
            const Blk b = get_block(a, S, 0, PH_HEAD, k);
            const uint32_t s0 = take(cur, b);
            if (!wait_filled(c, s0 + blk_slots(b), 0x6300u)) return;
            const int rbase = S.v0 + (k - 1) * kLmRows;
            block_rows<2, 4>(s0, b.seg / (D * 2), D * 2, x, wave, lno, [&](int row, float v) {
                const float lg = r * v;
                a.logits[rbase + row] = lg;
                if (better(lg, rbase + row, bv, bi)) { bv = lg; bi = rbase + row; }
            });
            release(c, wave, cur);
        }
        wave_argmax(bv, bi);
        if (lane == 0) { g_sm.red_v[wave] = bv; g_sm.red_i[wave] = bi; }
        if (!cw_barrier(c, 0x6500u)) return;
        if (ct == 0) {
            float v = g_sm.red_v[0];
            int i = g_sm.red_i[0];
            for (int w = 1; w < kNcw; ++w)
                if (better(g_sm.red_v[w], g_sm.red_i[w], v, i)) { v = g_sm.red_v[w]; i = g_sm.red_i[w]; }
            a.argmax_val[S.wg] = v;
            a.argmax_idx[S.wg] = i;
        }
    }
    release(c, wave, cur);
}

__global__ __launch_bounds__(kThreads) void step_kernel(StepArgs a) {
    const int wg = blockIdx.x;
    Sched S;
    S.wg = wg;
    S.xcd = wg % kXcd;
    S.slot = wg / kXcd;
    init_rows(a, S);
    Ctl c{&a, 0};
    if (threadIdx.x == 0) {
        g_sm.filled = 0;
        for (int w = 0; w < kNcw; ++w) g_sm.consumed[w] = 0;
        g_sm.bar = 0;
        g_sm.abort_ = 0;
    }
    __syncthreads();
    const int p = a.pos[0];
    S.p = p;
    S.pg0 = 0;
    S.npg = 0;
    bool bad = p < 0 || p + 1 > a.S * a.C || p / 16 >= a.max_blocks;
    S.pid_p = -1;
    if (!bad && S.xcd < a.Hkv && S.slot < a.S) {
        split_pages(S.slot, a.C, p, &S.pg0, &S.npg);
        if (p / a.C == S.slot) {   // the page of the new token's K/V (read once per step)
            const int pid = a.block_table[p / 16];
            S.pid_p = pid >= 0 && pid < a.num_pages ? pid : -1;
        }
    }
    if (bad) {
        if (threadIdx.x == 0) {
            st_far32(a.err + 1, 0x10u);
            st_far32(a.err, 1u);
        }
        return;
    }
    if (threadIdx.x < 64) loader(a, S, c);
    else compute(a, S, c);
}

// Prologue: x = the embedding row (or x_in) in the parity-1 residual buffer, the
// RoPE table of the step's position (the angle formed and reduced modulo 2 pi in
// double, then sincosf), and the tagged words and counters cleared, so no word
// or count of an earlier step satisfies a wait of this one.
__global__ __launch_bounds__(256) void step_prologue_kernel(StepArgs a, const int* tokens, const void* embed,
                                                            const float* x_in, float theta) {
    const int tid = threadIdx.x, b = blockIdx.x;
    if (b == 0) {
        float* xb1 = a.xb + a.D;   // x of "layer -1": parity 1
        if (tokens) {
            const int tok = tokens[0];
            const bool ok = tok >= 0 && tok < a.V;
            const uint16_t* row = (const uint16_t*)embed + (ok ? (long)tok * a.D : 0L);
            for (int d = tid; d < a.D; d += 256) xb1[d] = ok ? bf16_to_f32(row[d]) : 0.f;
        } else {
            for (int d = tid; d < a.D; d += 256) xb1[d] = x_in[d];
        }
        const int half = a.hd / 2;
        if (tid < half) {
            const int p = a.pos[0];
            const double inv = pow((double)theta, -2.0 * (double)tid / (double)a.hd);
            double ang = (double)p * inv;
            const double two_pi = 6.283185307179586476925286766559;
            ang -= two_pi * rint(ang / two_pi);
            float sv, cv;
            sincosf((float)ang, &sv, &cv);
            a.rope[tid] = make_float2(cv, sv);
        }
        if (tid < 4) a.err[tid] = 0u;
    }
    for (long i = (long)b * 256 + tid; i < a.clear_n; i += (long)gridDim.x * 256) a.clear_from[i] = 0ull;
}

}  // namespace

hipError_t launch_step_prologue(const StepArgs& a, const int* tokens, const void* embed, const float* x_in,
                                float theta, hipStream_t s) {
    hipLaunchKernelGGL(step_prologue_kernel, dim3(64), dim3(256), 0, s, a, tokens, embed, x_in, theta);
    return hipGetLastError();
}

hipError_t launch_step_kernel(const StepArgs& a, hipStream_t s) {
    void* args[] = {(void*)&a};
    return hipLaunchCooperativeKernel((const void*)step_kernel, dim3(kWgs), dim3(kThreads), args, 0, s);
}

}  // namespace qd
