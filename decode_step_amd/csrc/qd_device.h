// Device-side helpers shared by the gfx950 kernels of libqd: number formats,
// 128-bit loads and 64-lane wavefront reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qd {

constexpr int kWave = 64;

// bf16 is the top half of a float32: widening appends 16 zero bits (exact for
// every pattern); narrowing rounds half to even (nanoinfer page, phase 1), here
// by the hardware conversion v_cvt_pk_bf16_f32 (two values per instruction; a
// NaN stays a NaN). The integer form of the rounding (add 0x7fff plus the kept
// low bit, test for NaN) cost about 8 instructions per value.
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    typedef __attribute__((ext_vector_type(2))) float f2;
    typedef __attribute__((ext_vector_type(2))) __bf16 b2;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{lo, hi}, b2));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)f32x2_to_bf16x2(f, 0.f); }

// Elements per 16-byte vector for a storage type.
template <typename T> struct VecN;
template <> struct VecN<uint16_t> { static constexpr int n = 8; };
template <> struct VecN<float> { static constexpr int n = 4; };
template <> struct VecN<int8_t> { static constexpr int n = 16; };

// Type of the norm gains and biases that go with a weight type: int8 matrices
// keep their gains and biases in bf16.
template <typename WT> struct GainT { using type = WT; };
template <> struct GainT<int8_t> { using type = uint16_t; };

// Widen one 16-byte vector of T into floats.
__device__ __forceinline__ void widen16(const uint4 v, float (&f)[8]) {
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}
__device__ __forceinline__ void widen16(const uint4 v, float (&f)[16]) {   // int8, sign-extended
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int b = 0; b < 4; ++b) f[4 * i + b] = (float)(int8_t)(w[i] >> (8 * b));
}
__device__ __forceinline__ void widen16(const uint4 v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}

// Round floats to the storage type and pack them into one 16-byte vector.
template <typename T> __device__ __forceinline__ uint4 pack16(const float (&f)[VecN<T>::n]);
template <> __device__ __forceinline__ uint4 pack16<uint16_t>(const float (&f)[8]) {
    return make_uint4(f32x2_to_bf16x2(f[0], f[1]), f32x2_to_bf16x2(f[2], f[3]),
                      f32x2_to_bf16x2(f[4], f[5]), f32x2_to_bf16x2(f[6], f[7]));
}
template <> __device__ __forceinline__ uint4 pack16<float>(const float (&f)[4]) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
}

template <typename T> __device__ __forceinline__ float load_scalar(const void* p, int i);
template <> __device__ __forceinline__ float load_scalar<uint16_t>(const void* p, int i) {
    return bf16_to_f32(((const uint16_t*)p)[i]);
}
template <> __device__ __forceinline__ float load_scalar<float>(const void* p, int i) {
    return ((const float*)p)[i];
}

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float f) { return f32_to_bf16(f); }
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }

// Cross-lane reductions on 64-lane wavefronts. Within a 16-lane row they use
// DPP operand modifiers (quad_perm, row_half_mirror, row_mirror, row_ror), which
// fold into the VALU op; across rows they use gfx950's permlane16/permlane32
// swaps. Every lane of a group ends with the same bits (each step adds a pair
// in both lanes, and a + b == b + a exactly).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;       // lane i <-> 15 - i within 16
constexpr int kDppRor8 = 0x128;         // lane i <- (i + 8) mod 16, i.e. i ^ 8

// the other half of a permlane swap pair: (lane's own value, partner's value) summed
__device__ __forceinline__ float swap16_sum(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}
__device__ __forceinline__ float swap32_sum(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}
__device__ __forceinline__ float swap16_max(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
    return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float swap32_max(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
    return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

// Sum over aligned groups of W lanes (W a power of two <= 64); every lane of a
// group ends with the group's total.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
    if (W >= 2) v += dpp_f<kDppQuadXor1>(v);
    if (W >= 4) v += dpp_f<kDppQuadXor2>(v);
    if (W >= 8) v += dpp_f<kDppHalfMirror>(v);
    if (W >= 16) v += dpp_f<kDppMirror>(v);
    if (W >= 32) v = swap16_sum(v);
    if (W >= 64) v = swap32_sum(v);
    return v;
}

template <int W>
__device__ __forceinline__ float group_max(float v) {
    if (W >= 2) v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
    if (W >= 4) v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
    if (W >= 8) v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    if (W >= 16) v = fmaxf(v, dpp_f<kDppMirror>(v));
    if (W >= 32) v = swap16_max(v);
    if (W >= 64) v = swap32_max(v);
    return v;
}

__device__ __forceinline__ float wave_max(float v) { return group_max<kWave>(v); }

// Sum over the lanes that share lane % FROM (FROM in {8, 16, 32}): adds lanes
// i ^ FROM, i ^ 2*FROM, ... up to i ^ 32.
template <int FROM>
__device__ __forceinline__ float strided_sum(float v) {
    if (FROM <= 8) v += dpp_f<kDppRor8>(v);
    if (FROM <= 16) v = swap16_sum(v);
    v = swap32_sum(v);
    return v;
}

// (value, index) pair that wins an argmax: larger value, lower index on a tie.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
    const float ov = dpp_f<CTRL>(v);
    const int oi = dpp_i<CTRL>(i);
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
}

// Whole-wave argmax: every lane ends with the best (value, index) of the wave.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
    argmax_step<kDppQuadXor1>(v, i);
    argmax_step<kDppQuadXor2>(v, i);
    argmax_step<kDppHalfMirror>(v, i);
    argmax_step<kDppMirror>(v, i);
    const int lane = __lane_id();
    {
        auto rv = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
        auto ri = __builtin_amdgcn_permlane16_swap(i, i, false, false);
        const bool odd_row = (lane >> 4) & 1;
        const float ov = __int_as_float(odd_row ? rv[0] : rv[1]);
        const int oi = odd_row ? ri[0] : ri[1];
        if (better(ov, oi, v, i)) { v = ov; i = oi; }
    }
    {
        auto rv = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
        auto ri = __builtin_amdgcn_permlane32_swap(i, i, false, false);
        const bool upper = lane >= 32;
        const float ov = __int_as_float(upper ? rv[0] : rv[1]);
        const int oi = upper ? ri[0] : ri[1];
        if (better(ov, oi, v, i)) { v = ov; i = oi; }
    }
}

// A kernel-argument pointer pinned to scalar registers, as a global-memory
// (address space 1) byte pointer. Choosing among several such pointers with a
// per-lane condition could otherwise be compiled as a per-lane load from the
// argument block (a memory round trip the weight loads behind it would wait
// for); pinned values are chosen with plain selects, and the explicit address
// space keeps the loads through them global loads rather than flat ones.
typedef __attribute__((address_space(1))) const char gbyte;
__device__ __forceinline__ gbyte* sgpr_gptr(const void* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (gbyte*)(((uint64_t)hi << 32) | lo);
}
typedef unsigned int qd_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 gld16(gbyte* p) {
    const qd_u32x4 v = *(const __attribute__((address_space(1))) qd_u32x4*)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
template <typename T> __device__ __forceinline__ float gld_scalar(gbyte* p, long i) {
    if constexpr (sizeof(T) == 2) return bf16_to_f32(*(const __attribute__((address_space(1))) uint16_t*)(p + 2 * i));
    else return *(const __attribute__((address_space(1))) float*)(p + 4 * i);
}

// LDS address (offset within the workgroup's LDS) of a __shared__ object.
typedef __attribute__((address_space(3))) void qd_lds_void;
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const qd_lds_void*)p;
}

// One wave-wide LDS DMA of 16 bytes per lane: lane i's global source lands at
// lds + 16 i. Issued as inline asm so the compiler does not see an LDS write it
// would have to order against later LDS reads (left to itself it waits for every
// outstanding load before the next LDS access). Completion is the caller's
// business (s_waitcnt vmcnt); the compiler's own vmcnt waits stay correct, as
// extra outstanding loads only make a wait stricter.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "memory", "m0");
}

// s_waitcnt immediates (vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int wait_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x70 | 0xF00; }
constexpr int kWaitLgkm0 = 0xF | (0x3 << 14) | 0x70;

// Workgroup barrier for LDS traffic: this wave's LDS accesses complete, then
// s_barrier; compiler-only fences keep LDS accesses on their side. Unlike
// __syncthreads it does not wait for outstanding global loads, so prefetched
// weights stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// v -> (hi, lo) with hi = bf16(v) and lo = bf16(v - hi), both round-to-nearest-even
// through v_cvt_pk_bf16_f32; a pair's first element sits in the low half-word.
__device__ __forceinline__ void split_hi_lo(const float (&v)[8], uint4& hi, uint4& lo) {
    typedef __attribute__((ext_vector_type(2))) float f2;
    typedef __attribute__((ext_vector_type(2))) __bf16 b2;
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t hu = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{v[2 * i], v[2 * i + 1]}, b2));
        const float h0 = __uint_as_float(hu << 16), h1 = __uint_as_float(hu & 0xffff0000u);
        h[i] = hu;
        l[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{v[2 * i] - h0, v[2 * i + 1] - h1}, b2));
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// (value, index) argmax over the lanes that share lane % 16
__device__ __forceinline__ void argmax_across_rows(float& v, int& i) {
    const int lane = __lane_id();
    {
        auto rv = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
        auto ri = __builtin_amdgcn_permlane16_swap(i, i, false, false);
        const bool odd_row = (lane >> 4) & 1;
        const float ov = __int_as_float(odd_row ? rv[0] : rv[1]);
        const int oi = odd_row ? ri[0] : ri[1];
        if (better(ov, oi, v, i)) { v = ov; i = oi; }
    }
    {
        auto rv = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
        auto ri = __builtin_amdgcn_permlane32_swap(i, i, false, false);
        const bool upper = lane >= 32;
        const float ov = __int_as_float(upper ? rv[0] : rv[1]);
        const int oi = upper ? ri[0] : ri[1];
        if (better(ov, oi, v, i)) { v = ov; i = oi; }
    }
}

// SiLU with the sigmoid taken from e = exp(-|z|): 1/(1+e) for z >= 0 and
// e/(1+e) otherwise (nanoinfer page, phase 7).
__device__ __forceinline__ float silu(float z) {
    float e = expf(-fabsf(z));
    float s = (z >= 0.f) ? 1.f / (1.f + e) : e / (1.f + e);
    return z * s;
}

}  // namespace qd
