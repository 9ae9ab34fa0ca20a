// Device-side helpers shared by the gfx950 kernels of libqd: number formats,
// 128-bit loads and 64-lane wavefront reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qd {

constexpr int kWave = 64;

// bf16 is the top half of a float32: widening appends 16 zero bits (exact for
// every pattern); narrowing rounds half to even (nanoinfer page, phase 1).
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Elements per 16-byte vector for a storage type.
template <typename T> struct VecN;
template <> struct VecN<uint16_t> { static constexpr int n = 8; };
template <> struct VecN<float> { static constexpr int n = 4; };

// Widen one 16-byte vector of T into floats.
__device__ __forceinline__ void widen16(const uint4 v, float (&f)[8]) {
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}
__device__ __forceinline__ void widen16(const uint4 v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}

// Round floats to the storage type and pack them into one 16-byte vector.
template <typename T> __device__ __forceinline__ uint4 pack16(const float (&f)[VecN<T>::n]);
template <> __device__ __forceinline__ uint4 pack16<uint16_t>(const float (&f)[8]) {
    uint4 v;
    v.x = (uint32_t)f32_to_bf16(f[0]) | ((uint32_t)f32_to_bf16(f[1]) << 16);
    v.y = (uint32_t)f32_to_bf16(f[2]) | ((uint32_t)f32_to_bf16(f[3]) << 16);
    v.z = (uint32_t)f32_to_bf16(f[4]) | ((uint32_t)f32_to_bf16(f[5]) << 16);
    v.w = (uint32_t)f32_to_bf16(f[6]) | ((uint32_t)f32_to_bf16(f[7]) << 16);
    return v;
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

// Sum over groups of W consecutive lanes (W a power of two <= 64); every lane
// of the group ends with the group's total.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int off = W / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// (value, index) pair that wins an argmax: larger value, lower index on a tie.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        float ov = __shfl_xor(v, off, kWave);
        int oi = __shfl_xor(i, off, kWave);
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
