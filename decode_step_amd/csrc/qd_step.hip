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
//  - the q|k|v rows, attention splits and o_proj columns of KV head g run on XCD
//    g, so those two hand-offs stay in one L2; three hand-offs per layer cross
//    XCDs.
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

__device__ __forceinline__ uint32_t hw_xcc_id() {
    return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 0xF;   // HW_REG_XCC_ID [3:0]
}

// ---------------------------------------------------------------- shared state
struct Smem {
    uint8_t ring[kRingSlots * 1024];
    float vin[2][kVin];
    float xa[1024];          // x_a (P3 -> P4); the merged context (P2); x (P0, head); new k, v (P1)
    float2 rope[64];
    uint32_t filled;                // slots whose DMA has landed (loader)
    uint32_t consumed[kNcw];        // slots each compute wave is done with
    uint32_t bar, abort_;
    float ssp[2][kNcw];             // sums of squares per compute wave (two parities)
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
    if ((it & 255) == 0 && ld_far32(c.a->err)) {
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

// Read n floats (n a multiple of 4) that other XCDs wrote: dst[e] = src[e] (times
// element e of the bf16 gain block at ring slot gain_slot when >= 0); *ss (when given) gains the lane's sum of
// squares. Chunk q of 16 bytes goes to lane q % 256; every load of a lane is in
// flight together (out-of-range chunks reread chunk 0 and are dropped).
template <int PER>
__device__ __forceinline__ void load_far(const float* src, int n, float* dst, int gain_slot, float* ss, int ct) {
    const int nq = n >> 2;
    float4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int q = ct + 256 * i;
        v[i] = ld_far16(src, q < nq ? q : 0);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int q = ct + 256 * i;
        if (q < nq) {
            float f[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
            if (ss) *ss += f[0] * f[0] + f[1] * f[1] + f[2] * f[2] + f[3] * f[3];
            if (gain_slot >= 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) f[e] *= ring_bf16((uint32_t)gain_slot, 4 * q + e);
            }
            *(float4*)(dst + 4 * q) = make_float4(f[0], f[1], f[2], f[3]);
        }
    }
}

// Rows [0, nrows) of a packed bf16 block (row r at byte r * seg, in one lap of the
// ring) times x (seg / 2 floats in LDS); LPR lanes per row. fn(row, sum) runs on the
// first lane of each row's group.
template <int LPR, typename Fn>
__device__ __forceinline__ void block_dots(uint32_t s0, int nrows, int seg, const float* x, int ct,
                                           Fn fn) {
    constexpr int RPP = 256 / LPR;
    const int nch = seg >> 4, lr = ct % LPR;
    for (int r0 = 0; r0 < nrows; r0 += RPP) {
        const int row = r0 + ct / LPR;
        float acc = 0.f;
        if (row < nrows) {
            for (int ch = lr; ch < nch; ch += LPR) {
                const uint4 wv = *(const uint4*)(g_sm.ring + ring_off(s0, (uint32_t)(row * seg + ch * 16)));
                const float4 x0 = *(const float4*)(x + ch * 8), x1 = *(const float4*)(x + ch * 8 + 4);
                float f[8];
                widen16(wv, f);
                acc += f[0] * x0.x + f[1] * x0.y + f[2] * x0.z + f[3] * x0.w + f[4] * x1.x + f[5] * x1.y +
                       f[6] * x1.z + f[7] * x1.w;
            }
        }
        acc = group_sum<LPR>(acc);
        if (lr == 0 && row < nrows) fn(row, acc);
    }
}

__device__ __forceinline__ float rms_scale(const float* x, int D, float eps, int lane) {
    float ss = 0.f;
    for (int d = lane; d < D; d += 64) ss += x[d] * x[d];
    ss = group_sum<64>(ss);
    return 1.0f / sqrtf(ss / (float)D + eps);
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
__device__ __forceinline__ uint32_t take(uint32_t& cur, const Blk& b) {
    const uint32_t s0 = cur;
    cur += blk_slots(b);
    return s0;
}

__device__ __forceinline__ void compute(const StepArgs& a, const Sched& S, Ctl& c) {
    const int ct = threadIdx.x - 64;          // 0..255
    const int wave = ct >> 6, lane = ct & 63;
    const int D = a.D, hd = a.hd, G = a.G, F = a.F;
    const bool grp = S.xcd < a.Hkv;
    const int g = S.xcd;
    const int p = S.p;
    uint32_t cur = 0;   // absolute ring slot of the next block
    uint32_t vb = 0;    // input buffer parity
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
            float* xin = g_sm.vin[vb];
            float ss = 0.f;
            if (l > 0) {   // layer 0 reads the prologue's x
                if (wave == 0 && !wait_counts(c, CNT_X, l - 1, kXcd, kSlotsPerXcd, kSlotsPerXcd, -1, 0, 0, 0, 0,
                                              0x1050u | l)) return;
                if (!cw_barrier(c, 0x1060u | l)) return;
            }
            load_far<1>(XB + (size_t)ppar * D, D, xin, (int)gs, &ss, ct);
            ss_publish(g_sm.ssp[vb], wave, ss);
            if (!cw_barrier(c, 0x1200u | l)) return;
            const float r = ss_scale(g_sm.ssp[vb], D, a.eps);
            const int np = qkv_nparts(a, S.slot);
            u64* out = a.qkv + (size_t)par * a.qkvr;
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
                const uint32_t tg = tag_of(l, PH_QKV);
                block_dots<16>(ws, q.n, D * 2, xin, ct, [&](int row, float s) {
                    float v = r * s;
                    if (hb) v += bf16_to_f32(*(const uint16_t*)(g_sm.ring + ring_off(bs, (uint32_t)(boff + 2 * row))));
                    st_near(out + q.out0 + row, pack(v, tg));
                });
            }
            release(c, wave, cur);
            vb ^= 1;
        }
        // ------------------------------------------------------------ P1: attention over split s
        // (head_dim 64: lane d of a wave holds dimension d)
        if (grp && S.slot < a.S) {
            const int s = S.slot;
            uint32_t qns = 0, kns = 0;
            if (a.qk_norm) {
                qns = take(cur, get_block(a, S, l, PH_ATTN, 0));
                kns = take(cur, get_block(a, S, l, PH_ATTN, 1));
            }
            // the split's K pages, then its V pages: 2 slots (16 rows of 128 bytes) each
            const uint32_t kp0 = cur;
            cur += 2 * S.npg;
            const uint32_t vp0 = cur;
            cur += 2 * S.npg;
            float* qv = g_sm.vin[vb];   // q heads of group g, then k, then v
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
                const int pi = t / 16 - S.pg0, r = t % 16;
                return ring_off(p0 + 2 * pi + (r >> 3), (uint32_t)((r & 7) * 128));
            };
            // vectors 0..G-1 (q heads) and G (k): per-head RMSNorm with the shared gains,
            // then the half-split rotation (element i pairs with i + 32); the new k and v,
            // rounded to bf16, go to the cache and into the ring rows of position p
            for (int v = wave; v <= G; v += kNcw) {
                float* vec = qv + v * 64;
                float e0 = vec[lane];
                if (a.qk_norm) {
                    const float ss = group_sum<64>(e0 * e0);
                    const float rr = 1.0f / sqrtf(ss / 64.0f + a.eps);
                    e0 = e0 * rr * ring_bf16(v < G ? qns : kns, lane);
                }
                const float partner = __shfl_xor(e0, 32);
                const float2 cs = g_sm.rope[lane & 31];
                const float o0 = lane < 32 ? e0 * cs.x - partner * cs.y : e0 * cs.x + partner * cs.y;
                if (v < G) {
                    vec[lane] = o0;
                } else if (p / a.C == s) {   // the split holding p appends the new K/V
                    const uint16_t kb = f32_to_bf16(o0), vb16 = f32_to_bf16(qv[qn + 64 + lane]);
                    *(uint16_t*)(g_sm.ring + row_off(kp0, p) + 2 * lane) = kb;
                    *(uint16_t*)(g_sm.ring + row_off(vp0, p) + 2 * lane) = vb16;
                    const int pid = a.block_table[p / 16];
                    if (pid >= 0 && pid < a.num_pages) {
                        const long off = (((long)pid * a.Hkv + g) * 16 + (p % 16)) * 64;
                        ((uint16_t*)L.kc)[off + lane] = kb;
                        ((uint16_t*)L.vc)[off + lane] = vb16;
                    }
                }
            }
            if (!cw_barrier(c, 0x2400u | l)) return;
            // scores (base 2), softmax and P.V; wave w takes heads w and w + 4 together
            const int t0 = s * a.C, t1 = min(t0 + a.C, p + 1);
            const float scl = a.scale * 1.4426950408889634f;
            u64* part = a.part + (size_t)par * a.part_stride + ((size_t)g * a.S + s) * G * 66;
            const uint32_t ta = tag_of(l, PH_ATTN);
            const int hA = wave, hB = wave + kNcw;
            const bool has_b = hB < G;
            if (hA < G) {
                constexpr int KPL = 4;   // keys per lane (C <= 256)
                float sa[KPL], sb[KPL];
                float ma = -INFINITY, mb = -INFINITY;
                const float* qa = qv + hA * 64;
                const float* qb = qv + (has_b ? hB : hA) * 64;
#pragma unroll
                for (int i = 0; i < KPL; ++i) {
                    sa[i] = -INFINITY;
                    sb[i] = -INFINITY;
                    if (i * 64 < a.C) {
                        const int t = t0 + lane + 64 * i;
                        const bool ok = t < t1;
                        const uint8_t* kr = g_sm.ring + row_off(kp0, ok ? t : t0);
                        float acc_a = 0.f, acc_b = 0.f;
#pragma unroll
                        for (int d8 = 0; d8 < 64; d8 += 8) {
                            float f[8];
                            widen16(*(const uint4*)(kr + d8 * 2), f);
                            const float4 a0 = *(const float4*)(qa + d8), a1 = *(const float4*)(qa + d8 + 4);
                            const float4 b0 = *(const float4*)(qb + d8), b1 = *(const float4*)(qb + d8 + 4);
                            acc_a += f[0] * a0.x + f[1] * a0.y + f[2] * a0.z + f[3] * a0.w + f[4] * a1.x + f[5] * a1.y +
                                     f[6] * a1.z + f[7] * a1.w;
                            acc_b += f[0] * b0.x + f[1] * b0.y + f[2] * b0.z + f[3] * b0.w + f[4] * b1.x + f[5] * b1.y +
                                     f[6] * b1.z + f[7] * b1.w;
                        }
                        if (ok) {
                            sa[i] = acc_a * scl;
                            sb[i] = acc_b * scl;
                            ma = fmaxf(ma, sa[i]);
                            mb = fmaxf(mb, sb[i]);
                        }
                    }
                }
                ma = wave_max(ma);
                mb = wave_max(mb);
                float la = 0.f, lb = 0.f;
#pragma unroll
                for (int i = 0; i < KPL; ++i) {
                    sa[i] = sa[i] == -INFINITY ? 0.f : exp2f(sa[i] - ma);
                    sb[i] = sb[i] == -INFINITY ? 0.f : exp2f(sb[i] - mb);
                    la += sa[i];
                    lb += sb[i];
                }
                la = group_sum<64>(la);
                lb = group_sum<64>(lb);
                // o[d] = sum_t p_t V_t[d], a page (16 keys) at a time; the 16 keys of a page
                // sit in lanes ln0 .. ln0 + 15 of key group i
                float oa = 0.f, ob = 0.f;
                for (int pi = 0; pi < S.npg; ++pi) {
                    const int tp = (S.pg0 + pi) * 16, rel = tp - t0;
                    const int i = rel >> 6, ln0 = rel & 63;
                    const float pa = i == 0 ? sa[0] : i == 1 ? sa[1] : i == 2 ? sa[2] : sa[3];
                    const float pb = i == 0 ? sb[0] : i == 1 ? sb[1] : i == 2 ? sb[2] : sb[3];
                    const uint32_t v0 = ring_off(vp0 + 2 * pi, (uint32_t)(2 * lane));
                    const uint32_t v1 = ring_off(vp0 + 2 * pi + 1, (uint32_t)(2 * lane));
                    const int nk = min(16, t1 - tp);
                    if (nk == 16) {
                        float vv[16];
#pragma unroll
                        for (int k = 0; k < 16; ++k)
                            vv[k] = bf16_to_f32(*(const uint16_t*)(g_sm.ring + (k < 8 ? v0 : v1) + (k & 7) * 128));
#pragma unroll
                        for (int k = 0; k < 16; ++k) {
                            oa += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pa), ln0 + k)) * vv[k];
                            ob += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pb), ln0 + k)) * vv[k];
                        }
                    } else {
                        for (int k = 0; k < nk; ++k) {
                            const float vk = bf16_to_f32(*(const uint16_t*)(g_sm.ring + (k < 8 ? v0 : v1) + (k & 7) * 128));
                            oa += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pa), ln0 + k)) * vk;
                            ob += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pb), ln0 + k)) * vk;
                        }
                    }
                }
                u64* pa_out = part + (size_t)hA * 66;
                st_near(pa_out + lane, pack(oa, ta));
                if (lane == 0) {
                    st_near(pa_out + 64, pack(ma, ta));
                    st_near(pa_out + 65, pack(la, ta));
                }
                if (has_b) {
                    u64* pb_out = part + (size_t)hB * 66;
                    st_near(pb_out + lane, pack(ob, ta));
                    if (lane == 0) {
                        st_near(pb_out + 64, pack(mb, ta));
                        st_near(pb_out + 65, pack(lb, ta));
                    }
                }
            }
            release(c, wave, cur);
            vb ^= 1;
        }
        // ------------------------------------------------------------ P2: split merge, o_proj (group columns)
        if (grp) {
            const Blk ob = get_block(a, S, l, PH_O, 0);
            const uint32_t os = take(cur, ob);
            float* pin = g_sm.vin[vb];
            const int stride_s = G * (hd + 2);
            const u64* part = a.part + (size_t)par * a.part_stride + (size_t)g * a.S * stride_s;
            if (!poll_vec<20, false>(c, part, a.S * stride_s, tag_of(l, PH_ATTN), pin, nullptr, nullptr, ct,
                                     0x3100u | l)) return;
            if (!cw_barrier(c, 0x3200u | l)) return;
            // ctx[h][d] = sum_s 2^(m_s - M) o_s[d] / sum_s 2^(m_s - M) l_s
            float* ctx = g_sm.xa;
            for (int e = ct; e < G * hd; e += 256) {
                const int h = e / hd, d = e % hd;
                float M = -INFINITY;
                for (int s = 0; s < a.S; ++s) M = fmaxf(M, pin[s * stride_s + h * (hd + 2) + hd]);
                float lt = 0.f, ot = 0.f;
                for (int s = 0; s < a.S; ++s) {
                    const float* ps = pin + s * stride_s + h * (hd + 2);
                    const float w = ps[hd] == -INFINITY ? 0.f : exp2f(ps[hd] - M);
                    lt += w * ps[hd + 1];
                    ot += w * ps[d];
                }
                ctx[e] = ot / lt;
            }
            if (!wait_filled(c, os + blk_slots(ob), 0x3300u | l)) return;
            if (!cw_barrier(c, 0x3400u | l)) return;
            const int r0 = S.slot * D / kSlotsPerXcd;
            float* y = a.y + ((size_t)par * a.Hkv + g) * D + r0;
            block_dots<16>(os, ob.rows, ob.seg, ctx, ct, [&](int row, float v) { st_farf(y + row, v); });
            release(c, wave, cur);
            if (!publish(c, CNT_Y, l, S.xcd, wave, 0x3500u | l)) return;
            vb ^= 1;
        }
        // ------------------------------------------------------------ P3: x_a, RMSNorm, gate|up, SwiGLU
        {
            const Blk gb = get_block(a, S, l, PH_UP, 0);
            const uint32_t gs = take(cur, gb);
            float* xin = g_sm.vin[vb];
            if (!wait_filled(c, gs + blk_slots(gb), 0x4120u | l)) return;
            // x of the previous layer (all XCDs) and y_g of this one (XCDs < Hkv)
            if (wave == 0 && !wait_counts(c, CNT_X, l - 1, kXcd, l > 0 ? kSlotsPerXcd : 0, l > 0 ? kSlotsPerXcd : 0,
                                          CNT_Y, l, a.Hkv, kSlotsPerXcd, 0, 0x4100u | l)) return;
            if (!cw_barrier(c, 0x4200u | l)) return;
            // x_a = x + sum_g y_g (fixed order) into xa; x_a * g_mlp into xin; the sum of squares
            {
                float ss = 0.f;
                const float* xs = XB + (size_t)ppar * D;
                const float* ys = a.y + (size_t)par * a.Hkv * D;
                for (int q = ct; q < D / 4; q += 256) {
                    const float4 xv = ld_far16(xs, q);
                    float f[4] = {xv.x, xv.y, xv.z, xv.w};
                    for (int gg = 0; gg < a.Hkv; ++gg) {
                        const float4 yv = ld_far16(ys + (size_t)gg * D, q);
                        f[0] += yv.x; f[1] += yv.y; f[2] += yv.z; f[3] += yv.w;
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        ss += f[e] * f[e];
                        g_sm.xa[4 * q + e] = f[e];
                        xin[4 * q + e] = f[e] * ring_bf16(gs, 4 * q + e);
                    }
                }
                ss_publish(g_sm.ssp[vb], wave, ss);
            }
            if (!cw_barrier(c, 0x4300u | l)) return;
            const float r = ss_scale(g_sm.ssp[vb], D, a.eps);
            int f0, f1;
            weighted_range(S.wg, F, a.Hkv, a.up_wa, a.up_wb, &f0, &f1);
            const int nblk = (f1 - f0 + kP3Rows - 1) / kP3Rows;
            float* hout = a.h + (size_t)par * F;
            for (int k = 0; k < nblk; ++k) {
                const Blk bg = get_block(a, S, l, PH_UP, 1 + 2 * k);
                const uint32_t sg = take(cur, bg);
                const Blk bu = get_block(a, S, l, PH_UP, 2 + 2 * k);
                const uint32_t su = take(cur, bu);
                if (!wait_filled(c, su + blk_slots(bu), 0x4500u | l)) return;
                const int n = bg.seg / (D * 2);
                // 16 lanes per row; wave w, lane group q: row 2w + (q & 1) of gate (q < 2) or up (q >= 2)
                const int q = lane >> 4, row = 2 * wave + (q & 1), isup = q >> 1, lr = lane & 15;
                float acc = 0.f;
                if (row < n) {
                    const uint32_t s0 = isup ? su : sg;
                    for (int ch = lr; ch < D / 8; ch += 16) {
                        const uint4 wv = *(const uint4*)(g_sm.ring + ring_off(s0, (uint32_t)(row * D * 2 + ch * 16)));
                        const float4 x0 = *(const float4*)(xin + ch * 8), x1 = *(const float4*)(xin + ch * 8 + 4);
                        float f[8];
                        widen16(wv, f);
                        acc += f[0] * x0.x + f[1] * x0.y + f[2] * x0.z + f[3] * x0.w + f[4] * x1.x + f[5] * x1.y +
                               f[6] * x1.z + f[7] * x1.w;
                    }
                }
                acc = group_sum<16>(acc);
                // the up sum of a row sits 32 lanes above its gate sum
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(acc), __float_as_int(acc), false, false);
                const float upv = __int_as_float(sw[1]);
                if (lr == 0 && !isup && row < n)
                    st_farf(hout + f0 + k * kP3Rows + row, silu(r * acc) * (r * upv));
                release(c, wave, cur);
            }
            release(c, wave, cur);
            if (!publish(c, CNT_H, l, S.xcd, wave, 0x4600u | l)) return;
            vb ^= 1;
        }
        // ------------------------------------------------------------ P4: down + residual
        {
            const Blk db = get_block(a, S, l, PH_DOWN, 0);
            const uint32_t ds = take(cur, db);
            float* hin = g_sm.vin[vb];
            if (wave == 0 && !wait_counts(c, CNT_H, l, kXcd, kSlotsPerXcd, kSlotsPerXcd, -1, 0, 0, 0, 0, 0x5100u | l))
                return;
            if (!cw_barrier(c, 0x5150u | l)) return;
            load_far<5>(a.h + (size_t)par * F, F, hin, -1, nullptr, ct);
            if (!wait_filled(c, ds + blk_slots(db), 0x5200u | l)) return;
            if (!cw_barrier(c, 0x5300u | l)) return;
            int d0, d1;
            weighted_range(S.wg, D, a.Hkv, a.down_wa, a.down_wb, &d0, &d1);
            float* xo = XB + (size_t)par * D + d0;
            const bool last = l == a.L - 1;
            block_dots<64>(ds, d1 - d0, F * 2, hin, ct, [&](int row, float v) {
                const float xn = g_sm.xa[d0 + row] + v;
                st_farf(xo + row, xn);
                if (a.layer_out) a.layer_out[(size_t)l * D + d0 + row] = xn;
                if (last && a.x_out) a.x_out[d0 + row] = xn;
            });
            release(c, wave, cur);
            if (!publish(c, CNT_X, l, S.xcd, wave, 0x5500u | l)) return;
            vb ^= 1;
        }
    }
    // ---------------------------------------------------------------- final norm, lm_head, argmax partials
    if (a.lm_head) {
        const int nb = n_blocks(a, S, PH_HEAD);
        const Blk gb = get_block(a, S, 0, PH_HEAD, 0);
        const uint32_t gs = take(cur, gb);
        float* xin = g_sm.vin[vb];
        if (!wait_filled(c, gs + blk_slots(gb), 0x6000u)) return;
        float ss = 0.f;
        const int lp = (a.L - 1) & 1;
        if (wave == 0 && !wait_counts(c, CNT_X, a.L - 1, kXcd, kSlotsPerXcd, kSlotsPerXcd, -1, 0, 0, 0, 0, 0x6050u))
            return;
        if (!cw_barrier(c, 0x6060u)) return;
        load_far<1>(XB + (size_t)lp * D, D, xin, (int)gs, &ss, ct);
        ss_publish(g_sm.ssp[vb], wave, ss);
        if (!cw_barrier(c, 0x6200u)) return;
        const float r = ss_scale(g_sm.ssp[vb], D, a.eps);
        const int v0 = (int)((long)a.V * S.wg / kWgs);
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        for (int k = 1; k < nb; ++k) {
            const Blk b = get_block(a, S, 0, PH_HEAD, k);
            const uint32_t s0 = take(cur, b);
            if (!wait_filled(c, s0 + blk_slots(b), 0x6300u)) return;
            const int rbase = v0 + (k - 1) * kLmRows;
            block_dots<16>(s0, b.seg / (D * 2), D * 2, xin, ct, [&](int row, float v) {
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
    if (!bad && S.xcd < a.Hkv && S.slot < a.S) split_pages(S.slot, a.C, p, &S.pg0, &S.npg);
    if (hw_xcc_id() != (uint32_t)S.xcd) bad = true;   // the XCD layout the schedule assumes
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

int step_max_vin() { return kVin; }

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
