// topk.h -- per-token top-k selection of router logits by one wave, shared
// by the router kernels and the fused decode kernel (Dutch technical summary
// "Methodologie 1" of "A 35B Hybrid-Attention Mixture-of-Experts Model on a
// 6GB 2011 GPU": the MoE routing; the pages give no router arithmetic, so the
// plain reading is used: renormalised top-k of the softmax, which equals
// exp(l_j - l_max) / sum over the kept k, the full denominator cancelling).
#pragma once
#include "device.h"

namespace moeq4 {

// Candidate key: an order-preserving map of the fp32 logit in the high word
// and ~id in the low word, so the largest key is the largest logit and, among
// equal logits, the lowest expert id.  0 marks "no candidate".
// Order-preserving image of an fp32 value as an unsigned integer (finite
// values map above 0), and its inverse.  -0.0 and +0.0 are equal logits, so
// -0.0 is first made +0.0: both get one image, and the tie goes to the lower
// expert id like any other tie.
__device__ __forceinline__ uint32_t logit_ord(float v)
{
    uint32_t b = __float_as_uint(v);
    b = b == 0x80000000u ? 0u : b;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float ord_value(uint32_t ord)
{
    return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

__device__ __forceinline__ uint64_t topk_key(float v, int id)
{
    return ((uint64_t)logit_ord(v) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)id);
}

__device__ __forceinline__ float key_value(uint64_t key) { return ord_value((uint32_t)(key >> 32)); }

template <int CTRL>
__device__ __forceinline__ uint64_t max_key_step(uint64_t k)
{
    const uint32_t hi = (uint32_t)dpp<CTRL>((int)(uint32_t)(k >> 32));
    const uint32_t lo = (uint32_t)dpp<CTRL>((int)(uint32_t)k);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    return o > k ? o : k;
}

// Largest key of the wave: DPP inside each 16-lane row, then the four row
// maxima through readlane (uniform result).
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k)
{
    k = max_key_step<DPP_QUAD_1032>(k);
    k = max_key_step<DPP_QUAD_2301>(k);
    k = max_key_step<DPP_ROW_HALF_MIRROR>(k);
    k = max_key_step<DPP_ROW_MIRROR>(k);
    const uint32_t hi = (uint32_t)(k >> 32), lo = (uint32_t)k;
    uint64_t best = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint64_t v = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, 16 * r) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)lo, 16 * r);
        best = v > best ? v : best;
    }
    return best;
}

// Top-k keys of one token's logits by one wave: k rounds of a wave arg-max;
// lane j < k receives the key of slot j.
template <int LPL>
__device__ __forceinline__ uint64_t select_topk_keys(const float* __restrict__ lr, int E, int k, int lane)
{
    uint64_t key[LPL];
#pragma unroll
    for (int i = 0; i < LPL; ++i) {
        const int e = lane + i * WAVE;
        key[i] = e < E ? topk_key(lr[e], e) : 0ull;
    }
    uint64_t mine = 0;
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < LPL; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_key(best);
        // the owner retires the chosen expert
#pragma unroll
        for (int i = 0; i < LPL; ++i)
            if (key[i] == best) key[i] = 0ull;
        if (lane == j) mine = best;
    }
    return mine;
}

// Renormalised weight of slot `lane` (< k) from the kept logits, slot 0 being
// the largest: p_j = exp(l_j - l_0) in fp64, summed in slot order (j = 0..k-1)
// from the lanes' values, w_j = p_j / sum.  Every lane of the wave calls it;
// lane j < k passes its slot's logit.
__device__ __forceinline__ float topk_weight(float my_logit, int k, int lane)
{
    const float lmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_logit), 0)); // slot 0
    const double my_p = lane < k ? exp((double)my_logit - (double)lmax) : 0.0;
    double psum = 0.0;
    const int lo = __double2loint(my_p), hi = __double2hiint(my_p);
    for (int j = 0; j < k; ++j)
        psum += __hiloint2double(__builtin_amdgcn_readlane(hi, j), __builtin_amdgcn_readlane(lo, j));
    return (float)(my_p / psum);
}

// Top-k of one token's logits by one wave.  Lane j < k receives slot j.
template <int LPL>
__device__ __forceinline__ void select_topk(const float* __restrict__ lr, int E, int k, int lane, int& my_id,
                                            float& my_w)
{
    const uint64_t mine = select_topk_keys<LPL>(lr, E, k, lane);
    my_id = (int)(0xFFFFFFFFu - (uint32_t)mine);
    my_w = topk_weight(key_value(mine), k, lane);
}

} // namespace moeq4
