// quantize.hip -- fused Q8_0 activation quantisation (8-bit activations of the
// W4A8 decode path, Dutch technical summary "Methodologie 1" and
// "Methodologie 2" of "A 35B Hybrid-Attention Mixture-of-Experts Model on a
// 6GB 2011 GPU").
//
// Each thread owns float4s of a row; a 32-wide block is held by 8 consecutive
// lanes and its amax is a 3-step DPP max inside the wave.  Every
// thread issues all of its loads before any arithmetic.  d = amax / 127 and
// q = rint(x / d) use correctly rounded fp32 division (no fast-math), so the
// codes match any IEEE implementation of the same rule bit for bit.
// Optional pre-norm: x <- x * (1 / sqrt(mean(x^2) + 1e-6)), the factor in
// fp64 from a workgroup-wide fp64 sum of squares.
// HBM-bound: 4 bytes in, 1 + 1/8 bytes out per element.
//
// Layouts: rows of >= 1024 columns (or with the pre-norm) take one
// 256-thread workgroup each, F = ceil(cols / 1024) float4s per thread; shorter
// rows are packed several to a workgroup, one float4 per thread.
#include "device.h"

namespace moeq4 {

constexpr int QA_THREADS = 256;

__device__ __forceinline__ void quant4(float4 v, float d, int8_t* dst)
{
    const uint32_t q0 = (uint32_t)(q8_code(v.x, d) & 0xFF);
    const uint32_t q1 = (uint32_t)(q8_code(v.y, d) & 0xFF);
    const uint32_t q2 = (uint32_t)(q8_code(v.z, d) & 0xFF);
    const uint32_t q3 = (uint32_t)(q8_code(v.w, d) & 0xFF);
    *reinterpret_cast<uint32_t*>(dst) = q0 | (q1 << 8) | (q2 << 16) | (q3 << 24);
}

__device__ __forceinline__ float amax4(float4 v)
{
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// one row per workgroup, F float4s per thread (thread t owns float4s t, t+256, ...)
template <bool RMSNORM, int F>
__global__ __launch_bounds__(QA_THREADS) void quantize_row_kernel(const float* __restrict__ x, int cols,
                                                                  int8_t* __restrict__ xq, float* __restrict__ xd)
{
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    const int n4 = cols / 4;
    const float* xr = x + row * cols;
    float4 v[F];
#pragma unroll
    for (int f = 0; f < F; ++f) {
        const int i = tid + QA_THREADS * f;
        v[f] = i < n4 ? *reinterpret_cast<const float4*>(xr + 4 * i) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (RMSNORM) {
        __shared__ double s_part[QA_THREADS / WAVE];
        double ss = 0.0;
#pragma unroll
        for (int f = 0; f < F; ++f)
            ss += (double)v[f].x * v[f].x + (double)v[f].y * v[f].y + (double)v[f].z * v[f].z +
                  (double)v[f].w * v[f].w;
        ss = sum_wave_f64(ss);
        if (tid % WAVE == 0) s_part[tid / WAVE] = ss;
        __syncthreads();
        double tot = 0.0;
#pragma unroll
        for (int w = 0; w < QA_THREADS / WAVE; ++w) tot += s_part[w];
        const double inv = 1.0 / sqrt(tot / (double)cols + 1e-6);
#pragma unroll
        for (int f = 0; f < F; ++f) {
            v[f].x = (float)((double)v[f].x * inv);
            v[f].y = (float)((double)v[f].y * inv);
            v[f].z = (float)((double)v[f].z * inv);
            v[f].w = (float)((double)v[f].w * inv);
        }
    }
#pragma unroll
    for (int f = 0; f < F; ++f) {
        const int i = tid + QA_THREADS * f;
        // the 8 lanes of a block share `i < n4` (n4 is a multiple of 8)
        const float amax = max_group<8>(amax4(v[f]));
        const float d = amax / 127.0f;
        if (i < n4) {
            quant4(v[f], d, xq + row * cols + 4 * i);
            if ((tid & 7) == 0) xd[row * (cols / 32) + i / 8] = d;
        }
    }
}

// several short rows per workgroup (cols < 1024), one float4 per thread
__global__ __launch_bounds__(QA_THREADS) void quantize_short_kernel(const float* __restrict__ x, int64_t rows,
                                                                    int cols, int8_t* __restrict__ xq,
                                                                    float* __restrict__ xd)
{
    const int tpr = cols / 4; // threads per row: a multiple of 8
    const int rpw = QA_THREADS / tpr;
    const int lr = threadIdx.x / tpr, i = threadIdx.x % tpr;
    const int64_t row = (int64_t)blockIdx.x * rpw + lr;
    const bool live = lr < rpw && row < rows;
    const float4 v = live ? *reinterpret_cast<const float4*>(x + row * cols + 4 * i) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float amax = max_group<8>(amax4(v));
    const float d = amax / 127.0f;
    if (live) {
        quant4(v, d, xq + row * cols + 4 * i);
        if ((i & 7) == 0) xd[row * (cols / 32) + i / 8] = d;
    }
}

hipError_t launch_quantize_act(const float* x, int64_t rows, int cols, bool rmsnorm, int8_t* xq, float* xd,
                               hipStream_t s)
{
    if (rows == 0) return hipSuccess;
    if (cols < 1024 && !rmsnorm) {
        const int rpw = QA_THREADS / (cols / 4);
        quantize_short_kernel<<<dim3((unsigned)((rows + rpw - 1) / rpw)), QA_THREADS, 0, s>>>(x, rows, cols, xq, xd);
        return hipGetLastError();
    }
    const int f = (cols / 4 + QA_THREADS - 1) / QA_THREADS;
    const dim3 grid((unsigned)rows);
#define MOEQ4_QROW(FV)                                                                                  \
    if (f <= FV) {                                                                                      \
        if (rmsnorm) quantize_row_kernel<true, FV><<<grid, QA_THREADS, 0, s>>>(x, cols, xq, xd);        \
        else quantize_row_kernel<false, FV><<<grid, QA_THREADS, 0, s>>>(x, cols, xq, xd);               \
        return hipGetLastError();                                                                       \
    }
    MOEQ4_QROW(1)
    MOEQ4_QROW(2)
    MOEQ4_QROW(4)
    MOEQ4_QROW(8)
    MOEQ4_QROW(16)
#undef MOEQ4_QROW
    return hipErrorInvalidValue;
}

} // namespace moeq4
