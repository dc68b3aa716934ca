// route.hip -- MoE router: softmax, top-k, renormalisation and a stable
// counting sort of (token, slot) pairs by expert.  The routing feeds the
// grouped 4-bit GEMM of the prefill and the W4A8 decode GEMV (Dutch technical
// summary "Methodologie 1" of "A 35B Hybrid-Attention Mixture-of-Experts Model
// on a 6GB 2011 GPU"); the pages give no router arithmetic, so the plain
// reading is used: renormalised top-k of the softmax, which equals
// exp(l_j - l_max) / sum over the kept k (the full denominator cancels).
//
// Top-k: one wave per token.  Lane l holds logits l, l+64, ...; k rounds of a
// wave arg-max over (logit, -id) pick the experts in (logit descending, id
// ascending) order, which is also selection by softmax probability.  Weights
// are computed in fp64.
//
// Grouping, two shapes:
//   T <= 64 (decode): route_small, a single workgroup, top-k then a counting
//     sort in LDS: each expert keeps a 64-bit mask of the tokens that chose it,
//     so a pair's stable position is offset[e] + popcount(mask_e below t).
// The wave arg-max packs (logit, id) into one 64-bit key and reduces it with
// DPP row exchanges plus four readlanes.
//   larger T (prefill): route_topk then route_group; a route_group workgroup
//     owns 4 experts; its 16 waves own contiguous segments of the pair ids.
//     Pass 1 counts, per wave, pairs of experts below / equal to each owned
//     expert; pass 2 ranks pairs inside each segment by wave ballots and
//     writes them in ascending pair id.
// Both are deterministic: no result depends on the order of atomics.
#include "device.h"
#include "topk.h"

namespace moeq4 {

constexpr int TOPK_WAVES = 4;
constexpr int RS_THREADS = 1024; // one wave per token up to 16 tokens
constexpr int RS_MAX_T = 64;
constexpr int RS_MAX_E = 1024;
constexpr int RS_MAX_K = 16;
constexpr int GROUP_THREADS = 1024;
constexpr int GROUP_EPW = 4; // experts per route_group workgroup

template <int LPL>
__global__ __launch_bounds__(TOPK_WAVES* WAVE) void route_topk_kernel(const float* __restrict__ logits, int T, int E,
                                                                       int k, int32_t* __restrict__ ids,
                                                                       float* __restrict__ wts)
{
    const int lane = threadIdx.x % WAVE;
    const int t = blockIdx.x * TOPK_WAVES + threadIdx.x / WAVE;
    if (t >= T) return;
    int id;
    float w;
    select_topk<LPL>(logits + (int64_t)t * E, E, k, lane, id, w);
    if (lane < k) {
        ids[(int64_t)t * k + lane] = id;
        wts[(int64_t)t * k + lane] = w;
    }
}

// ------------------------------------------------------------------ T <= 64: one workgroup
template <int LPL>
__global__ __launch_bounds__(RS_THREADS) void route_small_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                                 int32_t* __restrict__ ids, float* __restrict__ wts,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ sorted)
{
    constexpr int EPT = RS_MAX_E / RS_THREADS; // experts per thread in the scan
    __shared__ uint32_t s_mask[RS_MAX_E][2];   // bit t: token t chose expert e
    __shared__ int s_ids[RS_MAX_T * RS_MAX_K];
    __shared__ int s_off[RS_MAX_E];
    __shared__ int s_wave[RS_THREADS / WAVE];
    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    for (int e = tid; e < E; e += RS_THREADS) s_mask[e][0] = s_mask[e][1] = 0u;
    __syncthreads();
    for (int t = wv; t < T; t += RS_THREADS / WAVE) {
        int id;
        float w;
        select_topk<LPL>(logits + (int64_t)t * E, E, k, lane, id, w);
        if (lane < k) {
            ids[t * k + lane] = id;
            wts[t * k + lane] = w;
            s_ids[t * k + lane] = id;
            atomicOr(&s_mask[id][t >> 5], 1u << (t & 31));
        }
    }
    __syncthreads();
    // per-expert counts and their exclusive scan; thread t owns experts EPT*t .. EPT*t+EPT-1
    int c[EPT], local = 0;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = EPT * tid + i;
        c[i] = e < E ? __popc(s_mask[e][0]) + __popc(s_mask[e][1]) : 0;
        local += c[i];
    }
    int inc = local;
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
        const int o = __shfl_up(inc, d, WAVE);
        if (lane >= d) inc += o;
    }
    if (lane == WAVE - 1) s_wave[wv] = inc;
    __syncthreads();
    int run = inc - local;
    for (int w = 0; w < wv; ++w) run += s_wave[w];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = EPT * tid + i;
        if (e < E) {
            s_off[e] = run;
            offsets[e] = run;
        }
        run += c[i];
    }
    if (tid == 0) offsets[E] = T * k;
    __syncthreads();
    const int P = T * k;
    for (int p = tid; p < P; p += RS_THREADS) {
        const int t = p / k, e = s_ids[p];
        const uint32_t m0 = s_mask[e][0], m1 = s_mask[e][1];
        const int below = t < 32 ? __popc(m0 & ((1u << t) - 1u)) : __popc(m0) + __popc(m1 & ((1u << (t - 32)) - 1u));
        sorted[s_off[e] + below] = p;
    }
}

// ------------------------------------------------------------------ larger T: per-expert grouping
__global__ __launch_bounds__(GROUP_THREADS) void route_group_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                                     int32_t* __restrict__ offsets,
                                                                     int32_t* __restrict__ sorted)
{
    constexpr int NW = GROUP_THREADS / WAVE;
    __shared__ int s_lt[NW][GROUP_EPW];
    __shared__ int s_eq[NW][GROUP_EPW];
    const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
    const int e0 = blockIdx.x * GROUP_EPW;
    const int seg = (P + NW - 1) / NW;
    const int p_beg = min(P, wv * seg), p_end = min(P, p_beg + seg);

    // pass 1: this wave's counts of pairs with expert < e and == e
    int lt[GROUP_EPW], eq[GROUP_EPW];
#pragma unroll
    for (int q = 0; q < GROUP_EPW; ++q) lt[q] = eq[q] = 0;
    for (int p = p_beg + lane; p < p_end; p += WAVE) {
        const int id = ids[p];
#pragma unroll
        for (int q = 0; q < GROUP_EPW; ++q) {
            lt[q] += id < e0 + q;
            eq[q] += id == e0 + q;
        }
    }
#pragma unroll
    for (int q = 0; q < GROUP_EPW; ++q) {
#pragma unroll
        for (int m = WAVE / 2; m >= 1; m >>= 1) {
            lt[q] += __shfl_xor(lt[q], m, WAVE);
            eq[q] += __shfl_xor(eq[q], m, WAVE);
        }
    }
    if (lane == 0)
#pragma unroll
        for (int q = 0; q < GROUP_EPW; ++q) { s_lt[wv][q] = lt[q]; s_eq[wv][q] = eq[q]; }
    __syncthreads();
    int run[GROUP_EPW];
#pragma unroll
    for (int q = 0; q < GROUP_EPW; ++q) {
        int off_q = 0, before = 0;
        for (int w = 0; w < NW; ++w) {
            off_q += s_lt[w][q];
            if (w < wv) before += s_eq[w][q];
        }
        run[q] = off_q + before;
        if (wv == 0 && lane == 0 && e0 + q < E) offsets[e0 + q] = off_q;
    }
    if (wv == 0 && lane == 0 && e0 + GROUP_EPW >= E) offsets[E] = P;

    // pass 2: stable scatter of this wave's segment
    const uint64_t below_mask = lane == 0 ? 0ull : (~0ull >> (WAVE - lane));
    for (int p0 = p_beg; p0 < p_end; p0 += WAVE) {
        const int p = p0 + lane;
        const int id = p < p_end ? ids[p] : -1;
#pragma unroll
        for (int q = 0; q < GROUP_EPW; ++q) {
            const bool mine = id == e0 + q;
            const uint64_t bal = __ballot(mine);
            if (mine) sorted[run[q] + __popcll(bal & below_mask)] = p;
            run[q] += __popcll(bal);
        }
    }
}

#define MOEQ4_LPL_DISPATCH(E, ...)                                  \
    do {                                                            \
        const int lpl_ = ((E) + WAVE - 1) / WAVE;                   \
        if (lpl_ <= 1) { constexpr int L = 1; __VA_ARGS__; }        \
        else if (lpl_ <= 2) { constexpr int L = 2; __VA_ARGS__; }   \
        else if (lpl_ <= 4) { constexpr int L = 4; __VA_ARGS__; }   \
        else if (lpl_ <= 8) { constexpr int L = 8; __VA_ARGS__; }   \
        else { constexpr int L = 16; __VA_ARGS__; }                 \
    } while (0)

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* wts, int32_t* offsets,
                        int32_t* sorted, hipStream_t s)
{
    if (T <= RS_MAX_T) {
        MOEQ4_LPL_DISPATCH(E, route_small_kernel<L><<<1, RS_THREADS, 0, s>>>(logits, T, E, k, ids, wts, offsets,
                                                                             sorted));
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((T + TOPK_WAVES - 1) / TOPK_WAVES));
    MOEQ4_LPL_DISPATCH(E, route_topk_kernel<L><<<grid, TOPK_WAVES * WAVE, 0, s>>>(logits, T, E, k, ids, wts));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    route_group_kernel<<<dim3((unsigned)((E + GROUP_EPW - 1) / GROUP_EPW)), GROUP_THREADS, 0, s>>>(ids, T * k, E,
                                                                                                   offsets, sorted);
    return hipGetLastError();
}

} // namespace moeq4
