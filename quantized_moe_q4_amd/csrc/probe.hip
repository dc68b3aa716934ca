// Measurement probes: the two "achievable" ceilings that the decode and
// prefill kernels are set against, next to the published peaks.
//
//   probe_read_kernel   a plain streaming read of a device buffer: 16-byte
//                       non-temporal loads, consecutive lanes on consecutive
//                       addresses, every byte read once, two workgroups per
//                       CU (of the shapes tried, with plain or non-temporal
//                       loads and 2 to 32 workgroups per CU, the fastest).
//                       Its rate is the HBM read bandwidth a
//                       weight-streaming kernel can reach.
//   probe_mfma_kernel   back-to-back v_mfma_i32_32x32x32_i8 on register
//                       operands (four independent accumulators per wave):
//                       the int8 matrix-core rate with no memory traffic and
//                       no epilogue.
//   probe_w4a8_step_kernel  the W4A8 prefill's inner step on registers: per
//                       step two v_mfma_i32_32x32x32_i8 (one Q4_0 block of two
//                       32x32 tiles) and, per output, the two fp32 FMAs that
//                       apply the weight and activation block scales, at the
//                       prefill kernels' occupancy (two workgroups of 4 waves
//                       per CU).  No memory traffic: the int8 rate this
//                       per-block-scaled formulation can reach at most.
//
// Neither kernel's result means anything; each ends in a store whose
// condition depends on every value computed, so no load or product can be
// dropped by the compiler.
#include "device.h"

#include "moe_q4.h"

namespace moeq4 {

constexpr int PR_THREADS = 256;
constexpr int PR_UNROLL = 4;
constexpr uint32_t PR_NEVER = 0x9E3779B9u; // a value the probes' results take with negligible chance

__global__ __launch_bounds__(PR_THREADS) void probe_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                                uint32_t* __restrict__ sink)
{
    const int64_t stride = (int64_t)gridDim.x * PR_THREADS;
    int64_t i = (int64_t)blockIdx.x * PR_THREADS + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (PR_UNROLL - 1) * stride < n16; i += PR_UNROLL * stride) {
        uint4 v[PR_UNROLL];
#pragma unroll
        for (int u = 0; u < PR_UNROLL; ++u) v[u] = ld_stream16(reinterpret_cast<const uint8_t*>(p + i + u * stride));
#pragma unroll
        for (int u = 0; u < PR_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = ld_stream16(reinterpret_cast<const uint8_t*>(p + i));
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == PR_NEVER) sink[0] = acc;
}

constexpr int PM_THREADS = 256;

__global__ __launch_bounds__(PM_THREADS) void probe_mfma_kernel(int iters, int32_t* __restrict__ sink)
{
    const int lane = threadIdx.x;
    const v4i a = {lane, lane * 3 + 1, lane ^ 0x5a, (int)blockIdx.x};
    const v4i b = {lane * 7, lane + 0x11, (int)blockIdx.x * 5, lane ^ 0x33};
    v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    }
    int r = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) r ^= c0[q] ^ c1[q] ^ c2[q] ^ c3[q];
    if ((uint32_t)r == PR_NEVER) sink[0] = r;
}

constexpr int PS_MAGIC = 0x4B400000; // 1.5 * 2^23, as the prefill kernels' MFMA C operand

__global__ __launch_bounds__(PM_THREADS, 2) void probe_w4a8_step_kernel(int iters, float* __restrict__ sink)
{
    const int lane = threadIdx.x;
    v4i a = {lane, lane * 3 + 1, lane ^ 0x5a, (int)blockIdx.x};
    const v4i b0 = {lane * 7, lane + 0x11, (int)blockIdx.x * 5, lane ^ 0x33};
    const v4i b1 = {lane * 5, lane + 0x23, (int)blockIdx.x * 3, lane ^ 0x1c};
    v16i c;
#pragma unroll
    for (int r = 0; r < 16; ++r) c[r] = PS_MAGIC;
    float acc0[16], acc1[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        acc0[r] = 0.0f;
        acc1[r] = 0.0f;
    }
    const float da = 1.0f + lane * 1e-5f, dw0 = 1e-3f * (lane + 1), dw1 = 2e-3f * (lane + 1);
    const float nw0 = -12582912.0f * dw0, nw1 = -12582912.0f * dw1;
    for (int it = 0; it < iters; ++it) {
        const v16i d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b0, c, 0, 0, 0);
        const v16i d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b1, c, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc0[r] = fmaf(fmaf(__int_as_float(d0[r]), dw0, nw0), da, acc0[r]);
            acc1[r] = fmaf(fmaf(__int_as_float(d1[r]), dw1, nw1), da, acc1[r]);
        }
        a.x += 1; // a new product every step
    }
    float r = 0.0f;
#pragma unroll
    for (int q = 0; q < 16; ++q) r += acc0[q] + acc1[q];
    if (__float_as_uint(r) == PR_NEVER) sink[0] = r;
}

static int device_cus()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    return n;
}

} // namespace moeq4

using namespace moeq4;

extern "C" {

int moe_q4_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream)
{
    if (!buf || !sink || bytes < 16 || bytes % 16 != 0 || ((uintptr_t)buf % 16) != 0 || ((uintptr_t)sink % 4) != 0)
        return MOE_Q4_ERR_INVALID_ARG;
    const int64_t n16 = (int64_t)(bytes / 16);
    // two workgroups per CU, each thread with PR_UNROLL loads in flight
    const int64_t want = (n16 + PR_THREADS - 1) / PR_THREADS;
    const int64_t cap = (int64_t)device_cus() * 2;
    const unsigned grid = (unsigned)(want < cap ? want : cap);
    probe_read_kernel<<<grid, PR_THREADS, 0, (hipStream_t)stream>>>(reinterpret_cast<const uint4*>(buf), n16, sink);
    return hipGetLastError() == hipSuccess ? MOE_Q4_OK : MOE_Q4_ERR_HIP;
}

int moe_q4_probe_mfma_i8(int32_t iters, int32_t workgroups, int32_t* sink, void* stream)
{
    if (iters < 1 || workgroups < 1 || !sink || ((uintptr_t)sink % 4) != 0) return MOE_Q4_ERR_INVALID_ARG;
    probe_mfma_kernel<<<(unsigned)workgroups, PM_THREADS, 0, (hipStream_t)stream>>>(iters, sink);
    return hipGetLastError() == hipSuccess ? MOE_Q4_OK : MOE_Q4_ERR_HIP;
}

int moe_q4_probe_w4a8_step(int32_t iters, int32_t workgroups, float* sink, void* stream)
{
    if (iters < 1 || workgroups < 1 || !sink || ((uintptr_t)sink % 4) != 0) return MOE_Q4_ERR_INVALID_ARG;
    probe_w4a8_step_kernel<<<(unsigned)workgroups, PM_THREADS, 0, (hipStream_t)stream>>>(iters, sink);
    return hipGetLastError() == hipSuccess ? MOE_Q4_OK : MOE_Q4_ERR_HIP;
}

} // extern "C"
