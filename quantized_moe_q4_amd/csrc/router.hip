// router.hip -- the router projection in front of the routing step:
// logits[T][E] = x_n W_r^T in fp32, W_r [E][H] (Dutch technical summary
// "Methodologie 1" of "A 35B Hybrid-Attention Mixture-of-Experts Model on a
// 6GB 2011 GPU" names the MoE routing ahead of the grouped expert GEMM; the
// pages give no router arithmetic, so the plain reading is a dense fp32
// projection of the layer input).  With the pre-norm flag, x_n is the row
// scaled by 1/sqrt(mean(x^2) + 1e-6), the factor summed in fp64 as the
// activation quantiser does; here it multiplies the finished dot product
// (fp64 product, one rounding), which differs from scaling every element
// first by rounding only.
//
//   router_gemv_kernel  (T <= RL_GEMV_T) one wave per expert: lanes stride
//                       the row in float4, a fixed-order fma chain per lane,
//                       then a wave sum; the rows of x come from L1/L2 shared
//                       by the workgroup's four experts.
//   router_gemm_kernel  (larger T) 64 tokens x 64 experts per workgroup, 4 x 4
//                       outputs per thread (32 x 32 or 16 x 32 tiles when that
//                       would leave CUs idle); K in LDS-staged chunks (64 or
//                       128) whose next chunk is loaded into registers while
//                       the current one is multiplied, read back 16 bytes
//                       along k at a time.
// Both sum in a fixed order, so results are deterministic.
#include "device.h"

#include "moe_q4.h"

namespace moeq4 {

constexpr int RL_THREADS = 256;
constexpr int RL_GEMV_T = 16;

__device__ __forceinline__ float4 live4(float4 v, bool live)
{
    return make_float4(live ? v.x : 0.f, live ? v.y : 0.f, live ? v.z : 0.f, live ? v.w : 0.f);
}

__device__ __forceinline__ float rl_norm(float acc, double ss, int H)
{
    return (float)((double)acc * (1.0 / sqrt(ss / (double)H + 1e-6)));
}

__global__ __launch_bounds__(RL_THREADS) void router_gemv_kernel(const float* __restrict__ x, int T, int H,
                                                                 const float* __restrict__ wr, int E, bool rmsnorm,
                                                                 float* __restrict__ logits)
{
    const int lane = threadIdx.x % WAVE;
    const int e = blockIdx.x * (RL_THREADS / WAVE) + threadIdx.x / WAVE;
    if (e >= E) return; // whole waves
    const float4* w4 = reinterpret_cast<const float4*>(wr + (int64_t)e * H);
    const int n4 = H / 4;
    for (int t = 0; t < T; ++t) {
        const float4* x4 = reinterpret_cast<const float4*>(x + (int64_t)t * H);
        float acc = 0.0f;
        double ss = 0.0;
        for (int q = lane; q < n4; q += WAVE) {
            const float4 a = x4[q], b = w4[q];
            acc = fmaf(a.x, b.x, acc);
            acc = fmaf(a.y, b.y, acc);
            acc = fmaf(a.z, b.z, acc);
            acc = fmaf(a.w, b.w, acc);
            if (rmsnorm) ss += (double)a.x * a.x + (double)a.y * a.y + (double)a.z * a.z + (double)a.w * a.w;
        }
        acc = sum_group<WAVE>(acc);
        if (rmsnorm) ss = sum_wave_f64(ss);
        if (lane == 0) logits[(int64_t)t * E + e] = rmsnorm ? rl_norm(acc, ss, H) : acc;
    }
}

template <int TM, int TN, int KC>
__global__ __launch_bounds__(RL_THREADS) void router_gemm_kernel(const float* __restrict__ x, int T, int H,
                                                                 const float* __restrict__ wr, int E, bool rmsnorm,
                                                                 float* __restrict__ logits)
{
    constexpr int RPT = TM / 16, CPT = TN / 16; // outputs per thread: RPT tokens x CPT experts
    constexpr int XP = TM * KC / 4;          // float4 pieces of a staged x chunk
    constexpr int WP = TN * KC / 4;          // float4 pieces of a staged W chunk
    constexpr int XPT = (XP + RL_THREADS - 1) / RL_THREADS, WPT = (WP + RL_THREADS - 1) / RL_THREADS;
    constexpr int PITCH = KC + 4; // floats per staged row: 16-byte reads along k stay aligned
    constexpr int PPR = KC / 4;   // float4 pieces per staged row
    // the caller picks KC dividing H: every chunk lies inside its rows
    __shared__ __align__(16) float s_x[TM][PITCH];
    __shared__ __align__(16) float s_w[TN][PITCH];
    __shared__ double s_ss[TM];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.y * TM, e0 = blockIdx.x * TN;
    const int ty = tid / 16, tx = tid % 16;
    float acc[RPT][CPT] = {};
    // staging: piece idx of a chunk is row idx / PPR, floats 4 * (idx % PPR) .. + 3
    const float* xp[XPT];
    bool xlive[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int idx = tid + RL_THREADS * i;
        xlive[i] = idx < XP && t0 + idx / PPR < T;
        xp[i] = x + (int64_t)(xlive[i] ? t0 + idx / PPR : 0) * H + 4 * (idx % PPR);
    }
    const float* wp[WPT];
    bool wlive[WPT];
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
        const int idx = tid + RL_THREADS * i;
        wlive[i] = idx < WP && e0 + idx / PPR < E;
        wp[i] = wr + (int64_t)(wlive[i] ? e0 + idx / PPR : 0) * H + 4 * (idx % PPR);
    }
    // the next chunk's pieces are loaded into registers while the current one is multiplied; the
    // addresses are always valid (dead pieces read row 0) and dead values are zeroed after the load
    float4 xv[XPT], wv[WPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) xv[i] = live4(*reinterpret_cast<const float4*>(xp[i]), xlive[i]);
#pragma unroll
    for (int i = 0; i < WPT; ++i) wv[i] = live4(*reinterpret_cast<const float4*>(wp[i]), wlive[i]);
    double ss[XPT] = {}; // this thread's parts of the sums of squares of its staged x rows
    for (int k0 = 0; k0 < H; k0 += KC) {
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int idx = tid + RL_THREADS * i;
            if (idx < XP) {
                if (rmsnorm)
                    ss[i] += (double)xv[i].x * xv[i].x + (double)xv[i].y * xv[i].y + (double)xv[i].z * xv[i].z +
                             (double)xv[i].w * xv[i].w;
                *reinterpret_cast<float4*>(&s_x[idx / PPR][4 * (idx % PPR)]) = xv[i];
            }
        }
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int idx = tid + RL_THREADS * i;
            if (idx < WP) *reinterpret_cast<float4*>(&s_w[idx / PPR][4 * (idx % PPR)]) = wv[i];
        }
        __syncthreads();
        if (k0 + KC < H) { // uniform
#pragma unroll
            for (int i = 0; i < XPT; ++i) xv[i] = live4(*reinterpret_cast<const float4*>(xp[i] + k0 + KC), xlive[i]);
#pragma unroll
            for (int i = 0; i < WPT; ++i) wv[i] = live4(*reinterpret_cast<const float4*>(wp[i] + k0 + KC), wlive[i]);
        }
#pragma unroll
        for (int k = 0; k < KC; k += 4) {
            float4 a[RPT], bw[CPT];
#pragma unroll
            for (int i = 0; i < RPT; ++i) a[i] = *reinterpret_cast<const float4*>(&s_x[RPT * ty + i][k]);
#pragma unroll
            for (int j = 0; j < CPT; ++j) bw[j] = *reinterpret_cast<const float4*>(&s_w[CPT * tx + j][k]);
#pragma unroll
            for (int i = 0; i < RPT; ++i)
#pragma unroll
                for (int j = 0; j < CPT; ++j) { // k, k+1, k+2, k+3 in order: the same chain as one k at a time
                    acc[i][j] = fmaf(a[i].x, bw[j].x, acc[i][j]);
                    acc[i][j] = fmaf(a[i].y, bw[j].y, acc[i][j]);
                    acc[i][j] = fmaf(a[i].z, bw[j].z, acc[i][j]);
                    acc[i][j] = fmaf(a[i].w, bw[j].w, acc[i][j]);
                }
        }
        __syncthreads();
    }
    if (rmsnorm) { // the PPR threads of a staged row are PPR consecutive lanes (PPR divides 64)
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int idx = tid + RL_THREADS * i;
            double v = ss[i];
#pragma unroll
            for (int m = 1; m < PPR; m <<= 1) v += __shfl_xor(v, m, WAVE);
            if (idx < XP && idx % PPR == 0) s_ss[idx / PPR] = v;
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int t = t0 + RPT * ty + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int e = e0 + CPT * tx + j;
            if (e < E) logits[(int64_t)t * E + e] = rmsnorm ? rl_norm(acc[i][j], s_ss[RPT * ty + i], H) : acc[i][j];
        }
    }
}

static int rl_cus()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    return n;
}

} // namespace moeq4

using namespace moeq4;

extern "C" int moe_q4_router_logits(const float* x, int32_t T, int32_t H, const float* wr, int32_t E, uint32_t flags,
                                    float* logits, void* stream)
{
    if (T < 0 || E < 1 || H < 32 || H % 32) return MOE_Q4_ERR_INVALID_ARG;
    if (flags & ~(uint32_t)MOE_Q4_QUANT_RMSNORM) return MOE_Q4_ERR_INVALID_ARG;
    if (H > 16384 || E > MOE_Q4_MAX_EXPERTS) return MOE_Q4_ERR_UNSUPPORTED;
    if (T == 0) return MOE_Q4_OK;
    if (!x || !wr || !logits) return MOE_Q4_ERR_INVALID_ARG;
    if (((uintptr_t)x % 16) || ((uintptr_t)wr % 16) || ((uintptr_t)logits % 4)) return MOE_Q4_ERR_INVALID_ARG;
    const bool rms = (flags & MOE_Q4_QUANT_RMSNORM) != 0;
    const hipStream_t s = (hipStream_t)stream;
    if (T <= RL_GEMV_T) {
        const unsigned grid = (unsigned)((E + RL_THREADS / WAVE - 1) / (RL_THREADS / WAVE));
        router_gemv_kernel<<<grid, RL_THREADS, 0, s>>>(x, T, H, wr, E, rms, logits);
    } else if ((int64_t)((T + 63) / 64) * ((E + 63) / 64) >= 2 * rl_cus()) {
        const dim3 grid((unsigned)((E + 63) / 64), (unsigned)((T + 63) / 64));
        if (H % 64 == 0) router_gemm_kernel<64, 64, 64><<<grid, RL_THREADS, 0, s>>>(x, T, H, wr, E, rms, logits);
        else router_gemm_kernel<64, 64, 32><<<grid, RL_THREADS, 0, s>>>(x, T, H, wr, E, rms, logits);
    } else if ((int64_t)((T + 31) / 32) * ((E + 31) / 32) >= 2 * rl_cus()) {
        const dim3 grid((unsigned)((E + 31) / 32), (unsigned)((T + 31) / 32));
        if (H % 128 == 0) router_gemm_kernel<32, 32, 128><<<grid, RL_THREADS, 0, s>>>(x, T, H, wr, E, rms, logits);
        else router_gemm_kernel<32, 32, 32><<<grid, RL_THREADS, 0, s>>>(x, T, H, wr, E, rms, logits);
    } else { // smaller tiles, so that a mid-sized batch still fills the chip
        const dim3 grid((unsigned)((E + 31) / 32), (unsigned)((T + 15) / 16));
        if (H % 128 == 0) router_gemm_kernel<16, 32, 128><<<grid, RL_THREADS, 0, s>>>(x, T, H, wr, E, rms, logits);
        else router_gemm_kernel<16, 32, 32><<<grid, RL_THREADS, 0, s>>>(x, T, H, wr, E, rms, logits);
    }
    return hipGetLastError() == hipSuccess ? MOE_Q4_OK : MOE_Q4_ERR_HIP;
}
