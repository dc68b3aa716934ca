// device.h -- gfx950 device helpers shared by the library's kernels.
//
// Formats (readings of the Q4_0 family and of 8-bit activations, Dutch
// technical summary "Methodologie 2" of "A 35B Hybrid-Attention
// Mixture-of-Experts Model on a 6GB 2011 GPU"): a Q4_0 block is 16 nibble
// bytes plus one fp16 scale; byte i holds element i (low nibble) and element
// i + 16 (high nibble); weight = (q - 8) * d.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeq4 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int WAVE = 64;

// fp16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float half_to_float(uint16_t h)
{
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return (float)v;
}

// Four nibbles per byte-lane -> signed int8 (q - 8), one byte each.
// For a byte x in 0..15: (x + 0x78) ^ 0x80 == x - 8 in two's complement, and
// the add never carries into the next byte.
__device__ __forceinline__ int nib_lo_s8(uint32_t w)
{
    return (int)(((w & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
}
__device__ __forceinline__ int nib_hi_s8(uint32_t w)
{
    return (int)((((w >> 4) & 0x0F0F0F0Fu) + 0x78787878u) ^ 0x80808080u);
}

// A whole Q4_0 block (16 nibble bytes) -> 32 signed int8 in element order:
// out[0..3] = elements 0..15, out[4..7] = elements 16..31.
__device__ __forceinline__ void unpack_block(const uint4 w, int out[8])
{
    out[0] = nib_lo_s8(w.x); out[1] = nib_lo_s8(w.y); out[2] = nib_lo_s8(w.z); out[3] = nib_lo_s8(w.w);
    out[4] = nib_hi_s8(w.x); out[5] = nib_hi_s8(w.y); out[6] = nib_hi_s8(w.z); out[7] = nib_hi_s8(w.w);
}

// Exact int32 dot of one unpacked weight block with one int8 activation block
// (8 dwords, element order), on v_dot4_i32_i8.
__device__ __forceinline__ int block_dot(const int w[8], const int a[8])
{
    int s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s = __builtin_amdgcn_sdot4(w[i], a[i], s, false);
    return s;
}

// ---------------------------------------------------------------- reductions
template <int WIDTH>
__device__ __forceinline__ float sum_xor(float v)
{
#pragma unroll
    for (int m = WIDTH / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
    return v;
}

template <int WIDTH>
__device__ __forceinline__ float max_xor(float v)
{
#pragma unroll
    for (int m = WIDTH / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, WAVE));
    return v;
}

__device__ __forceinline__ double sum_wave_f64(double v)
{
#pragma unroll
    for (int m = WAVE / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
    return v;
}

// Q8_0 of one value given its block's amax (the same rule as the activation
// quantiser): d = amax / 127, q = rint(v / d) clamped to [-127, 127].
__device__ __forceinline__ int q8_code(float v, float d)
{
    if (d == 0.0f) return 0;
    float q = rintf(v / d);
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    return (int)q;
}

// ---------------------------------------------------------------- expert lookup
// Block-wide search over the per-expert pair counts c_e = off[e+1] - off[e].
// value(c_e) is a non-negative tile count for expert e; the call finds the
// expert e whose half-open range [prefix_e, prefix_e + value_e) contains
// `target` and returns e and target - prefix_e, or false when target lies
// beyond the total.  All threads of the block must call it (it synchronises).
template <int NT, typename F>
__device__ bool locate_expert(const int32_t* __restrict__ off, int E, int target, F value, int& e_out, int& rel_out)
{
    constexpr int NWAVES = NT / WAVE;
    __shared__ int s_wave[NWAVES];
    __shared__ int s_res[2];
    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    const int ept = (E + NT - 1) / NT; // experts per thread, contiguous
    const int e0 = tid * ept;
    int local = 0;
    for (int i = 0; i < ept; ++i) {
        const int e = e0 + i;
        if (e < E) local += value(off[e + 1] - off[e]);
    }
    // inclusive scan within the wave
    int inc = local;
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
        const int o = __shfl_up(inc, d, WAVE);
        if (lane >= d) inc += o;
    }
    if (tid == 0) { s_res[0] = -1; s_res[1] = 0; }
    if (lane == WAVE - 1) s_wave[wv] = inc;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wv; ++w) base += s_wave[w];
    int run = base + inc - local; // exclusive prefix of this thread
    if (target >= run && target < run + local) {
        for (int i = 0; i < ept; ++i) {
            const int e = e0 + i;
            if (e >= E) break;
            const int v = value(off[e + 1] - off[e]);
            if (target < run + v) { s_res[0] = e; s_res[1] = target - run; break; }
            run += v;
        }
    }
    __syncthreads();
    e_out = s_res[0];
    rel_out = s_res[1];
    __syncthreads();
    return e_out >= 0;
}

} // namespace moeq4
