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
__device__ __forceinline__ uint64_t topk_key(float v, int id)
{
    const uint32_t b = __float_as_uint(v);
    const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)id);
}

__device__ __forceinline__ float key_value(uint64_t key)
{
    const uint32_t ord = (uint32_t)(key >> 32);
    return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

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

// Top-k of one token's logits by one wave.  Lane j < k receives slot j.
// The k selection rounds only move keys; the fp64 weights are computed after
// them, every lane its own exp in parallel, and summed in slot order
// (j = 0..k-1) from the lanes' values, the same operations in the same order
// as a sequential loop.
template <int LPL>
__device__ __forceinline__ void select_topk(const float* __restrict__ lr, int E, int k, int lane, int& my_id,
                                            float& my_w)
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
    my_id = (int)(0xFFFFFFFFu - (uint32_t)mine);
    const float lmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(key_value(mine)), 0)); // slot 0
    const double my_p = lane < k ? exp((double)key_value(mine) - (double)lmax) : 0.0;
    double psum = 0.0;
    const int2 pb = make_int2(__double2loint(my_p), __double2hiint(my_p));
    for (int j = 0; j < k; ++j)
        psum += __hiloint2double(__builtin_amdgcn_readlane(pb.y, j), __builtin_amdgcn_readlane(pb.x, j));
    my_w = (float)(my_p / psum);
}

} // namespace moeq4
