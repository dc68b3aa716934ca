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

typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// Decode weight loads.  A decode call reads each touched expert's matrices
// exactly once (every token that chose the expert is served by the same
// load), so its weight loads are non-temporal: streamed rather than kept in
// the caches, which on this part also raises the rate of a plain streaming
// read by about a tenth.
__device__ __forceinline__ uint4 ld_stream16(const uint8_t* p)
{
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint16_t ld_stream_u16(const uint16_t* p)
{
    return __builtin_nontemporal_load(p);
}

// The same loads with the default cache policy: a lone small read (one GEMV call, 576 KB) finishes sooner with
// them than with the non-temporal hint.
template <bool NT>
__device__ __forceinline__ uint4 ld_w16(const uint8_t* p)
{
    if constexpr (NT) return ld_stream16(p);
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    return v;
}

template <bool NT>
__device__ __forceinline__ uint16_t ld_w_u16(const uint16_t* p)
{
    if constexpr (NT) return ld_stream_u16(p);
    return *p;
}

typedef unsigned v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint2 ld_stream8(const uint16_t* p) // 8-byte aligned
{
    const v2u v = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p));
    return make_uint2(v.x, v.y);
}

__device__ __forceinline__ uint32_t ld_stream4(const uint16_t* p) // 4-byte aligned
{
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// fp16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float half_to_float(uint16_t h)
{
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return (float)v;
}

// Nibbles -> int8 operands, scaled by 16.  With x' = w ^ 0x88888888 the high
// nibble field of every byte, x' & 0xF0F0F0F0, read as a signed int8 equals
// 16 * (q_hi - 8), and (x' << 4) & 0xF0F0F0F0 gives 16 * (q_lo - 8) (the shift
// moves each low nibble to the top of its own byte).  So a dot product over
// these operands is exactly 16 * sum (q - 8) * a; the 16 is folded into the
// weight scale (d / 16 is exact in fp32).  Two VALU ops per output dword.
__device__ __forceinline__ uint32_t nib_flip(uint32_t w) { return w ^ 0x88888888u; }
__device__ __forceinline__ int nib_lo16(uint32_t flipped) { return (int)((flipped << 4) & 0xF0F0F0F0u); }
__device__ __forceinline__ int nib_hi16(uint32_t flipped) { return (int)(flipped & 0xF0F0F0F0u); }

// A whole Q4_0 block (16 nibble bytes) -> 32 int8 = 16 (q - 8) in element
// order: out[0..3] = elements 0..15, out[4..7] = elements 16..31.
__device__ __forceinline__ void unpack_block16(const uint4 w, int out[8])
{
    const uint32_t a = nib_flip(w.x), b = nib_flip(w.y), c = nib_flip(w.z), d = nib_flip(w.w);
    out[0] = nib_lo16(a); out[1] = nib_lo16(b); out[2] = nib_lo16(c); out[3] = nib_lo16(d);
    out[4] = nib_hi16(a); out[5] = nib_hi16(b); out[6] = nib_hi16(c); out[7] = nib_hi16(d);
}

// 16 x the exact int32 dot of one unpacked weight block with one int8
// activation block (8 dwords, element order), on v_dot4_i32_i8.
// |16 isum| <= 16 * 32512 < 2^20: no overflow.
__device__ __forceinline__ int block_dot16(const int w[8], const int a[8])
{
    int s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s = __builtin_amdgcn_sdot4(w[i], a[i], s, false);
    return s;
}

constexpr float INV16 = 0.0625f;

// A workgroup barrier that orders LDS accesses only.  __syncthreads() also
// waits for every global load in flight (its workgroup-scope fence covers
// global memory), which would land prefetched weights at the first barrier
// after their issue; with this one they stay in flight until their registers
// are read.  Use it where the barrier has no global memory to order.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------- reductions
// Lane exchanges on DPP (a VALU operand modifier, a few cycles) rather than
// ds_bpermute (an LDS round trip).  gfx9 DPP controls used: quad_perm
// [1,0,3,2] and [2,3,0,1], row_half_mirror (lane i <-> 7-i within 8),
// row_mirror (i <-> 15-i within 16), row_ror:8, row_shl:4 and row_shr:4.
// Every lane must be active.
constexpr int DPP_QUAD_1032 = 0xB1;
constexpr int DPP_QUAD_2301 = 0x4E;
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_ROR8 = 0x128;
constexpr int DPP_ROW_SHL4 = 0x104; // lane i reads lane i + 4 of its 16-lane row (0 past the row end)
constexpr int DPP_ROW_SHR4 = 0x114; // lane i reads lane i - 4 of its 16-lane row (0 before the row start)

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// Sum / max over aligned groups of WIDTH lanes (WIDTH in {8, 16, 32, 64});
// every lane of a group receives the group's result.
template <int WIDTH>
__device__ __forceinline__ float sum_group(float v)
{
    static_assert(WIDTH == 8 || WIDTH == 16 || WIDTH == 32 || WIDTH == 64, "group width");
    v += dpp<DPP_QUAD_1032>(v);
    v += dpp<DPP_QUAD_2301>(v);
    v += dpp<DPP_ROW_HALF_MIRROR>(v);
    if (WIDTH >= 16) v += dpp<DPP_ROW_MIRROR>(v);
    if (WIDTH >= 32) v += __shfl_xor(v, 16, WAVE);
    if (WIDTH >= 64) v += __shfl_xor(v, 32, WAVE);
    return v;
}

template <int WIDTH>
__device__ __forceinline__ float max_group(float v)
{
    static_assert(WIDTH == 8 || WIDTH == 16 || WIDTH == 32 || WIDTH == 64, "group width");
    v = fmaxf(v, dpp<DPP_QUAD_1032>(v));
    v = fmaxf(v, dpp<DPP_QUAD_2301>(v));
    v = fmaxf(v, dpp<DPP_ROW_HALF_MIRROR>(v));
    if (WIDTH >= 16) v = fmaxf(v, dpp<DPP_ROW_MIRROR>(v));
    if (WIDTH >= 32) v = fmaxf(v, __shfl_xor(v, 16, WAVE));
    if (WIDTH >= 64) v = fmaxf(v, __shfl_xor(v, 32, WAVE));
    return v;
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const int lo = dpp<CTRL>(__double2loint(v)), hi = dpp<CTRL>(__double2hiint(v));
    return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double readlane_f64(double v, int lane)
{
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), lane),
                            __builtin_amdgcn_readlane(__double2loint(v), lane));
}

// Sum over the wave in fp64, the same value in every lane: pairs, quads,
// halves and whole 16-lane rows by DPP (after the quad steps every lane of a
// quad holds the quad's sum, so the mirrors add the partner group's sum),
// then the four row sums as (r0 + r1) + (r2 + r3).  Every lane must be active.
__device__ __forceinline__ double sum_wave_f64(double v)
{
    v += dpp_f64<DPP_QUAD_1032>(v);
    v += dpp_f64<DPP_QUAD_2301>(v);
    v += dpp_f64<DPP_ROW_HALF_MIRROR>(v);
    v += dpp_f64<DPP_ROW_MIRROR>(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
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
__device__ bool locate_expert(const int32_t* __restrict__ off, int E, int target, F value, int& e_out, int& rel_out,
                              int* total_out = nullptr)
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
    int base = 0, total = 0;
    for (int w = 0; w < NWAVES; ++w) {
        if (w < wv) base += s_wave[w];
        total += s_wave[w];
    }
    if (total_out) *total_out = total;
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

// Writes the ids of experts with at least one pair, ascending, to s_list and
// returns their number U; s_beg[a] receives off[s_list[a]] and s_beg[U] =
// off[E], so the pairs of active expert a occupy sorted positions
// [s_beg[a], s_beg[a+1]).  All threads of the block must call it (it
// synchronises); s_list needs room for E entries and s_beg for E + 1.
template <int NT>
__device__ int compact_active(const int32_t* __restrict__ off, int E, int* s_list, int* s_beg)
{
    __shared__ int s_cwave[NT / WAVE];
    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    const int ept = (E + NT - 1) / NT;
    const int e0 = tid * ept;
    int local = 0;
    for (int i = 0; i < ept; ++i) {
        const int e = e0 + i;
        if (e < E) local += off[e + 1] > off[e];
    }
    int inc = local;
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
        const int o = __shfl_up(inc, d, WAVE);
        if (lane >= d) inc += o;
    }
    if (lane == WAVE - 1) s_cwave[wv] = inc;
    __syncthreads();
    int base = 0, total = 0;
    for (int w = 0; w < NT / WAVE; ++w) {
        if (w < wv) base += s_cwave[w];
        total += s_cwave[w];
    }
    int pos = base + inc - local;
    for (int i = 0; i < ept; ++i) {
        const int e = e0 + i;
        if (e < E) {
            const int b = off[e];
            if (off[e + 1] > b) {
                s_list[pos] = e;
                s_beg[pos] = b;
                ++pos;
            }
        }
    }
    if (tid == 0) s_beg[total] = off[E];
    __syncthreads();
    return total;
}

} // namespace moeq4
