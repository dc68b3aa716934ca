// quantize.hip -- fused Q8_0 activation quantisation (8-bit activations of the
// W4A8 decode path, Dutch technical summary "Methodologie 1" and
// "Methodologie 2" of "A 35B Hybrid-Attention Mixture-of-Experts Model on a
// 6GB 2011 GPU").
//
// One wave per row.  Each pass covers 256 columns: lane l loads the float4 at
// columns 4l..4l+3, so a 32-wide block is held by 8 consecutive lanes and its
// amax is a 3-step xor-shuffle max inside the wave.  d = amax / 127 and
// q = rint(x / d) use correctly rounded fp32 division (no fast-math), so the
// codes match any IEEE implementation of the same rule bit for bit.
// Optional pre-norm: x <- x * (1 / sqrt(mean(x^2) + 1e-6)), the factor in fp64.
// HBM-bound: 4 bytes in, 1 + 1/8 bytes out per element.
#include "device.h"

namespace moeq4 {

constexpr int QA_WAVES = 4;

template <bool RMSNORM>
__global__ __launch_bounds__(QA_WAVES* WAVE) void quantize_act_kernel(const float* __restrict__ x, int64_t rows,
                                                                       int cols, int8_t* __restrict__ xq,
                                                                       float* __restrict__ xd)
{
    const int lane = threadIdx.x % WAVE;
    const int64_t row = (int64_t)blockIdx.x * QA_WAVES + threadIdx.x / WAVE;
    if (row >= rows) return;
    const float* xr = x + row * cols;
    double inv = 1.0;
    if (RMSNORM) {
        double ss = 0.0;
        for (int c = lane * 4; c < cols; c += WAVE * 4) {
            const float4 v = *reinterpret_cast<const float4*>(xr + c);
            ss += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
        }
        ss = sum_wave_f64(ss);
        inv = 1.0 / sqrt(ss / (double)cols + 1e-6);
    }
    for (int c = lane * 4; c < cols; c += WAVE * 4) {
        float4 v = *reinterpret_cast<const float4*>(xr + c);
        if (RMSNORM) {
            v.x = (float)((double)v.x * inv);
            v.y = (float)((double)v.y * inv);
            v.z = (float)((double)v.z * inv);
            v.w = (float)((double)v.w * inv);
        }
        float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        // the 8 lanes of a block are aligned groups of 8 (cols % 32 == 0)
        amax = max_xor<8>(amax);
        const float d = amax / 127.0f;
        const uint32_t q0 = (uint32_t)(q8_code(v.x, d) & 0xFF);
        const uint32_t q1 = (uint32_t)(q8_code(v.y, d) & 0xFF);
        const uint32_t q2 = (uint32_t)(q8_code(v.z, d) & 0xFF);
        const uint32_t q3 = (uint32_t)(q8_code(v.w, d) & 0xFF);
        *reinterpret_cast<uint32_t*>(xq + row * cols + c) = q0 | (q1 << 8) | (q2 << 16) | (q3 << 24);
        if ((lane & 7) == 0) xd[row * (cols / 32) + c / 32] = d;
    }
}

hipError_t launch_quantize_act(const float* x, int64_t rows, int cols, bool rmsnorm, int8_t* xq, float* xd,
                               hipStream_t s)
{
    if (rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((rows + QA_WAVES - 1) / QA_WAVES));
    if (rmsnorm)
        quantize_act_kernel<true><<<grid, QA_WAVES * WAVE, 0, s>>>(x, rows, cols, xq, xd);
    else
        quantize_act_kernel<false><<<grid, QA_WAVES * WAVE, 0, s>>>(x, rows, cols, xq, xd);
    return hipGetLastError();
}

} // namespace moeq4
