// route.hip -- MoE router: softmax, top-k, renormalisation and a stable
// counting sort of (token, slot) pairs by expert.  The routing feeds the
// grouped 4-bit GEMM of the prefill and the W4A8 decode GEMV (Dutch technical
// summary "Methodologie 1" of "A 35B Hybrid-Attention Mixture-of-Experts Model
// on a 6GB 2011 GPU"); the pages give no router arithmetic, so the plain
// reading is used: renormalised top-k of the softmax, which equals
// exp(l_j - l_max) / sum over the kept k (the full denominator cancels).
//
// Kernel 1 (route_topk): one wave per token.  Lane l holds logits
// l, l+64, ...; k rounds of a wave arg-max over (logit, -id) pick the experts
// in (logit descending, id ascending) order, which is also selection by
// softmax probability.  Weights are computed in fp64.
//
// Kernel 2 (route_group): one workgroup per expert e.  It walks all P = T*k
// pair ids in order, counts pairs of experts < e (its offset) and writes its
// own pairs in ascending pair id, ranked by wave ballots, so the permutation
// is a deterministic stable counting sort with no atomics.
#include "device.h"

namespace moeq4 {

constexpr int TOPK_WAVES = 4;

template <int LPL>
__global__ __launch_bounds__(TOPK_WAVES* WAVE) void route_topk_kernel(const float* __restrict__ logits, int T, int E,
                                                                       int k, int32_t* __restrict__ ids,
                                                                       float* __restrict__ wts)
{
    const int lane = threadIdx.x % WAVE;
    const int t = blockIdx.x * TOPK_WAVES + threadIdx.x / WAVE;
    if (t >= T) return;
    const float* lr = logits + (int64_t)t * E;
    float v[LPL];
    bool live[LPL];
#pragma unroll
    for (int i = 0; i < LPL; ++i) {
        const int e = lane + i * WAVE;
        live[i] = e < E;
        v[i] = live[i] ? lr[e] : 0.0f;
    }
    float lmax = 0.0f;
    double psum = 0.0;
    double my_p = 0.0; // lane j keeps slot j
    int my_id = 0;
    for (int j = 0; j < k; ++j) {
        // local best: largest logit, lowest id on ties (ids grow with i)
        float bv = 0.0f;
        int bid = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < LPL; ++i) {
            const int e = lane + i * WAVE;
            if (live[i] && (bid == 0x7FFFFFFF || v[i] > bv)) { bv = v[i]; bid = e; }
        }
        // wave arg-max on (value desc, id asc); lanes without candidates carry id = INT_MAX
#pragma unroll
        for (int m = WAVE / 2; m >= 1; m >>= 1) {
            const float ov = __shfl_xor(bv, m, WAVE);
            const int oid = __shfl_xor(bid, m, WAVE);
            const bool take = (oid != 0x7FFFFFFF) &&
                              (bid == 0x7FFFFFFF || ov > bv || (ov == bv && oid < bid));
            if (take) { bv = ov; bid = oid; }
        }
        // the owner retires the chosen expert
#pragma unroll
        for (int i = 0; i < LPL; ++i)
            if (lane + i * WAVE == bid) live[i] = false;
        if (j == 0) lmax = bv;
        const double p = exp((double)bv - (double)lmax);
        psum += p;
        if (lane == j) { my_p = p; my_id = bid; }
    }
    if (lane < k) {
        ids[(int64_t)t * k + lane] = my_id;
        wts[(int64_t)t * k + lane] = (float)(my_p / psum);
    }
}

constexpr int GROUP_THREADS = 256;

__global__ __launch_bounds__(GROUP_THREADS) void route_group_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                                     int32_t* __restrict__ offsets,
                                                                     int32_t* __restrict__ sorted)
{
    __shared__ int s_wave[GROUP_THREADS / WAVE];
    __shared__ int s_lt[GROUP_THREADS / WAVE];
    const int e = blockIdx.x;
    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;

    // pass 1: number of pairs routed to experts below e
    int lt = 0;
    for (int p = tid; p < P; p += GROUP_THREADS) lt += ids[p] < e;
#pragma unroll
    for (int m = WAVE / 2; m >= 1; m >>= 1) lt += __shfl_xor(lt, m, WAVE);
    if (lane == 0) s_lt[wv] = lt;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < GROUP_THREADS / WAVE; ++w) base += s_lt[w];
    if (tid == 0) {
        offsets[e] = base;
        if (e == E - 1) offsets[E] = P;
    }

    // pass 2: write this expert's pairs in ascending pair id
    int run = base;
    for (int p0 = 0; p0 < P; p0 += GROUP_THREADS) {
        const int p = p0 + tid;
        const bool mine = p < P && ids[p] == e;
        const uint64_t bal = __ballot(mine);
        const int before = __popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (WAVE - lane))));
        if (lane == 0) s_wave[wv] = __popcll(bal);
        __syncthreads();
        int wbase = run;
        for (int w = 0; w < wv; ++w) wbase += s_wave[w];
        if (mine) sorted[wbase + before] = p;
        int tot = 0;
        for (int w = 0; w < GROUP_THREADS / WAVE; ++w) tot += s_wave[w];
        run += tot;
        __syncthreads();
    }
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* wts, int32_t* offsets,
                        int32_t* sorted, hipStream_t s)
{
    if (T > 0) {
        const dim3 grid((unsigned)((T + TOPK_WAVES - 1) / TOPK_WAVES));
        const int lpl = (E + WAVE - 1) / WAVE;
        if (lpl <= 1)
            route_topk_kernel<1><<<grid, TOPK_WAVES * WAVE, 0, s>>>(logits, T, E, k, ids, wts);
        else if (lpl <= 2)
            route_topk_kernel<2><<<grid, TOPK_WAVES * WAVE, 0, s>>>(logits, T, E, k, ids, wts);
        else if (lpl <= 4)
            route_topk_kernel<4><<<grid, TOPK_WAVES * WAVE, 0, s>>>(logits, T, E, k, ids, wts);
        else if (lpl <= 8)
            route_topk_kernel<8><<<grid, TOPK_WAVES * WAVE, 0, s>>>(logits, T, E, k, ids, wts);
        else
            route_topk_kernel<16><<<grid, TOPK_WAVES * WAVE, 0, s>>>(logits, T, E, k, ids, wts);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    route_group_kernel<<<dim3((unsigned)E), GROUP_THREADS, 0, s>>>(ids, T * k, E, offsets, sorted);
    return hipGetLastError();
}

} // namespace moeq4
