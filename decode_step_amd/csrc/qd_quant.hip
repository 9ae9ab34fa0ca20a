// Per-output-channel symmetric int8 quantization of a weight matrix (nanoinfer
// page, phase 6: one scale per row, no zero point, range [-127, 127], rounding
// half away from zero). An offline conversion, not part of a decode step.
//
// Row r: scale = max_k |w[r][k]| / 127 and q[r][k] = round(w[r][k] / scale),
// both quotients float32 with IEEE rounding (HIP's default float division). The
// integer rounding is exact on the float32 quotient v: with t = trunc(|v|), the
// fraction |v| - t is exact, and the code is sign(v) * (t + (|v| - t >= 0.5)).
// (Adding 0.5 and truncating would round v just below 0.5 up to 1 once the sum
// rounds to 1.0.) A zero row has scale 0 and codes 0.
#include "qd_device.h"
#include "qd_launch.h"

namespace qd {

constexpr int kQuantThreads = 256;

template <typename WT>
__global__ __launch_bounds__(kQuantThreads) void quantize_rows_kernel(const WT* w, long rows, int cols,
                                                                       int8_t* q, float* scale) {
    __shared__ float wmax[kQuantThreads / kWave];
    const long r = blockIdx.x;
    if (r >= rows) return;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const WT* row = w + r * (long)cols;
    float m = 0.f;
    for (int k = tid; k < cols; k += kQuantThreads) m = fmaxf(m, fabsf(load_scalar<WT>(row, k)));
    m = group_max<kWave>(m);
    if (lane == 0) wmax[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float s = __fdiv_rn(m, 127.0f);
    if (tid == 0) scale[r] = s;
    int8_t* qr = q + r * (long)cols;
    for (int k = tid; k < cols; k += kQuantThreads) {
        int c = 0;
        if (s > 0.f) {
            const float v = __fdiv_rn(load_scalar<WT>(row, k), s);
            const float a = fabsf(v);
            const float t = truncf(a);
            int mag = (int)t + (a - t >= 0.5f ? 1 : 0);
            mag = mag > 127 ? 127 : mag;
            c = v < 0.f ? -mag : mag;
        }
        qr[k] = (int8_t)c;
    }
}

hipError_t launch_quantize_rows(const void* w, int w_is_bf16, long rows, int cols, int8_t* q, float* scale,
                                hipStream_t s) {
    if (rows < 1 || cols < 1 || rows > 0x7fffffffL) return hipErrorInvalidValue;
    if (w_is_bf16)
        hipLaunchKernelGGL(quantize_rows_kernel<uint16_t>, dim3((unsigned)rows), dim3(kQuantThreads), 0, s,
                           (const uint16_t*)w, rows, cols, q, scale);
    else
        hipLaunchKernelGGL(quantize_rows_kernel<float>, dim3((unsigned)rows), dim3(kQuantThreads), 0, s,
                           (const float*)w, rows, cols, q, scale);
    return hipGetLastError();
}

}  // namespace qd
