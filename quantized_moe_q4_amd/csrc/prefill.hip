// prefill.hip -- top-k routed W4A8 grouped GEMM over resident Q4_0 experts
// (Dutch technical summary "Methodologie 1" of "A 35B Hybrid-Attention
// Mixture-of-Experts Model on a 6GB 2011 GPU": the prefill runs a grouped
// 4-bit GEMM for the MoE; "Methodologie 4": the whole prompt goes through in
// one pass, so each touched expert is read once per tile column and the GEMM
// batch is as large as the prompt allows).
//
// Work decomposition.  Pairs are grouped by expert (moe_q4_route's counting
// sort).  Expert e with c_e pairs owns ceil(c_e / 64) row tiles of up to 64
// rows (two 32-row MFMA tiles; a tile with at most 32 live rows runs a
// one-MFMA-row body).  The grid's y index enumerates row tiles across experts
// (an upper bound is launched; surplus workgroups exit after a block-wide scan
// of the per-expert counts); x enumerates column tiles.  A workgroup is 4
// waves; each wave owns 32 columns of each B matrix it multiplies.
//
// Inner product on int8 MFMA.  v_mfma_i32_32x32x32_i8 multiplies a 32x32 int8
// A (rows m = activation rows) by a 32x32 int8 B (columns n = weight rows) over
// K = 32, exactly one Q4_0/Q8_0 block, so each MFMA yields one block's exact
// int32 dot for a 32x32 tile.  Nibbles are unpacked in registers to 16 (q - 8)
// (device.h), so the MFMA produces 16 isum.  Operand K order: lane half h
// (lane / 32) carries block elements 8h..8h+7 (bytes 0..7 of its 16-byte
// operand) and 16+8h..16+8h+7 (bytes 8..15); A and B use the same order, and
// an integer sum over the block does not depend on it.  D layout: lane l holds
// column l % 32 and, in register r, row 8*(r/4) + 4*(l/32) + (r%4).
//
// Scales in fp32.  The MFMA's C operand is the bit pattern of 1.5 * 2^23
// (0x4B400000); since |16 isum| < 2^22, D read as fp32 is exactly
// 1.5*2^23 + 16 isum.  With dw = d_w / 16: t = fma(D, dw, -1.5*2^23*dw) =
// fl(isum * d_w) (1.5*2^23*dw is exact: 2 + 11 significant bits) and
// acc = fma(t, d_a, acc).  Two VALU ops per output per block: on gfx950
// without packed fp32 math that VALU work, not the MFMA, bounds the kernel.
//
// Pipelining: each wave loads its A and B operands PF blocks ahead into a
// register ring; activation scales d_a of the workgroup's rows are staged in
// LDS once.
//
// gate/up kernel: a wave's B columns are 32 gate rows and the same 32 up rows;
// the epilogue forms h = silu(g) * u and re-quantises it to Q8_0 across the 32
// columns (one block of I per row), writing hq/hd in sorted-pair order, and
// the kernel clears y for the scatter-add.  down kernel: a wave's B columns are
// 64 rows of W_down; the epilogue scatter-adds topk_w * o into y with fp32
// atomics.
#include "device.h"

namespace moeq4 {

constexpr int PF_THREADS = 256;
constexpr int PF_TM = 64;               // rows per workgroup tile (two MFMA m-tiles)
constexpr int PF_GU_BN = 128;           // gate/up: columns of I per workgroup (4 waves x 32)
constexpr int PF_DN_BN = 256;           // down: columns of H per workgroup (4 waves x 64)
constexpr int MAGIC_BITS = 0x4B400000;  // 1.5 * 2^23
constexpr float MAGIC_F = 12582912.0f;
constexpr int PF_MAX_NB = 64;           // K blocks (K <= 2048)

__device__ __forceinline__ int mfma_row(int r, int lane)
{
    return 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
}

// 16-byte B operand (16 (q - 8) in the operand K order) from the 8 nibble bytes of half h.
__device__ __forceinline__ v4i b_operand(uint2 w)
{
    const uint32_t a = nib_flip(w.x), b = nib_flip(w.y);
    v4i r;
    r.x = nib_lo16(a);
    r.y = nib_lo16(b);
    r.z = nib_hi16(a);
    r.w = nib_hi16(b);
    return r;
}

// 16-byte A operand from an int8 activation block (32 bytes), half h.
__device__ __forceinline__ v4i a_load(const int8_t* __restrict__ blk32)
{
    const uint2 lo = *reinterpret_cast<const uint2*>(blk32);
    const uint2 hi = *reinterpret_cast<const uint2*>(blk32 + 16);
    v4i a;
    a.x = (int)lo.x;
    a.y = (int)lo.y;
    a.z = (int)hi.x;
    a.w = (int)hi.y;
    return a;
}

__device__ __forceinline__ v16i magic_c()
{
    v16i c;
#pragma unroll
    for (int r = 0; r < 16; ++r) c[r] = MAGIC_BITS;
    return c;
}

struct TileRows {
    int e, beg, m0, mcount;
};

// Locate this workgroup's (expert, row tile); false for surplus workgroups.
__device__ __forceinline__ bool pf_locate(const int32_t* __restrict__ off, int E, TileRows& tr)
{
    int e, mt;
    if (!locate_expert<PF_THREADS>(off, E, (int)blockIdx.y, [](int c) { return (c + PF_TM - 1) / PF_TM; }, e, mt))
        return false;
    tr.e = e;
    tr.beg = off[e];
    tr.m0 = mt * PF_TM;
    const int left = off[e + 1] - tr.beg - tr.m0;
    tr.mcount = left < PF_TM ? left : PF_TM;
    return true;
}

// One wave's share of a grouped-GEMM tile: MW 32-row m-tiles of A times two
// 32-column B tiles, over NB K-blocks, into fp32 accumulators.
//
// Pipelining: four operand buffers hold blocks b .. b+3; a buffer is refilled
// with block b+4 right after the MFMAs that consume it have been issued (so
// the refill reuses its registers and the loop needs no register copies), and
// the fp16 weight scales arrive four blocks per 8-byte load, two groups ahead.
// `dump(mi, t, r, b, isum)` receives every exact block dot (a no-op outside
// the inspection variant).
template <int MW>
struct OpBuf {
    v4i a[MW];
    uint2 b[2];
};

template <int MW>
__device__ __forceinline__ void load_ops(OpBuf<MW>& X, const int8_t* const (&arow)[2],
                                         const uint8_t* __restrict__ bq0, const uint8_t* __restrict__ bq1, int b)
{
#pragma unroll
    for (int mi = 0; mi < MW; ++mi) X.a[mi] = a_load(arow[mi] + 32 * b);
    X.b[0] = *reinterpret_cast<const uint2*>(bq0 + 16 * b);
    X.b[1] = *reinterpret_cast<const uint2*>(bq1 + 16 * b);
}

template <int MW, typename Dump>
__device__ __forceinline__ void gemm_step(OpBuf<MW>& X, int b, int NB, const uint2 (&S)[2], int u,
                                          const int8_t* const (&arow)[2], const uint8_t* __restrict__ bq0,
                                          const uint8_t* __restrict__ bq1, const float (*s_da)[PF_TM], int h,
                                          const v16i& cmag, float (&acc)[MW][2][16], Dump& dump)
{
    v16i D[MW][2];
    {
        const v4i B0 = b_operand(X.b[0]), B1 = b_operand(X.b[1]);
#pragma unroll
        for (int mi = 0; mi < MW; ++mi) {
            D[mi][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(X.a[mi], B0, cmag, 0, 0, 0);
            D[mi][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(X.a[mi], B1, cmag, 0, 0, 0);
        }
    }
    load_ops<MW>(X, arow, bq0, bq1, min(b + 4, NB - 1)); // refill: block b+4 (clamped at the end)
    __builtin_amdgcn_sched_barrier(0);
    float dw[2], nw[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const uint32_t pair = (u & 2) ? S[t].y : S[t].x;
        dw[t] = half_to_float((uint16_t)(pair >> (16 * (u & 1)))) * INV16;
        nw[t] = -MAGIC_F * dw[t];
    }
#pragma unroll
    for (int mi = 0; mi < MW; ++mi) {
        float da[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 v = *reinterpret_cast<const float4*>(&s_da[b][32 * mi + 8 * q + 4 * h]);
            da[4 * q + 0] = v.x;
            da[4 * q + 1] = v.y;
            da[4 * q + 2] = v.z;
            da[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc[mi][t][r] = fmaf(fmaf(__int_as_float(D[mi][t][r]), dw[t], nw[t]), da[r], acc[mi][t][r]);
                dump(mi, t, r, b, (D[mi][t][r] - MAGIC_BITS) >> 4);
            }
    }
}

template <int MW, typename Dump>
__device__ __forceinline__ void wave_gemm(const int8_t* const (&arow)[2], const uint8_t* __restrict__ bq0,
                                          const uint8_t* __restrict__ bq1, const uint16_t* __restrict__ bd0,
                                          const uint16_t* __restrict__ bd1, int NB, const float (*s_da)[PF_TM],
                                          float (&acc)[MW][2][16], Dump dump)
{
    const int h = (threadIdx.x % WAVE) / 32;
    const v16i cmag = magic_c();
#pragma unroll
    for (int mi = 0; mi < MW; ++mi)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][t][r] = 0.0f;
    OpBuf<MW> X0, X1, X2, X3;
    load_ops<MW>(X0, arow, bq0, bq1, 0);
    load_ops<MW>(X1, arow, bq0, bq1, 1);
    load_ops<MW>(X2, arow, bq0, bq1, 2);
    load_ops<MW>(X3, arow, bq0, bq1, 3);
    uint2 S0[2], S1[2]; // fp16 weight scales of blocks g..g+3, per B tile
    S0[0] = *reinterpret_cast<const uint2*>(bd0);
    S0[1] = *reinterpret_cast<const uint2*>(bd1);
    S1[0] = *reinterpret_cast<const uint2*>(bd0 + 4);
    S1[1] = *reinterpret_cast<const uint2*>(bd1 + 4);
    for (int b0 = 0; b0 < NB; b0 += 8) {
        gemm_step<MW>(X0, b0 + 0, NB, S0, 0, arow, bq0, bq1, s_da, h, cmag, acc, dump);
        gemm_step<MW>(X1, b0 + 1, NB, S0, 1, arow, bq0, bq1, s_da, h, cmag, acc, dump);
        gemm_step<MW>(X2, b0 + 2, NB, S0, 2, arow, bq0, bq1, s_da, h, cmag, acc, dump);
        gemm_step<MW>(X3, b0 + 3, NB, S0, 3, arow, bq0, bq1, s_da, h, cmag, acc, dump);
        const int g0 = min(b0 + 8, NB - 4);
        S0[0] = *reinterpret_cast<const uint2*>(bd0 + g0);
        S0[1] = *reinterpret_cast<const uint2*>(bd1 + g0);
        gemm_step<MW>(X0, b0 + 4, NB, S1, 0, arow, bq0, bq1, s_da, h, cmag, acc, dump);
        gemm_step<MW>(X1, b0 + 5, NB, S1, 1, arow, bq0, bq1, s_da, h, cmag, acc, dump);
        gemm_step<MW>(X2, b0 + 6, NB, S1, 2, arow, bq0, bq1, s_da, h, cmag, acc, dump);
        gemm_step<MW>(X3, b0 + 7, NB, S1, 3, arow, bq0, bq1, s_da, h, cmag, acc, dump);
        const int g1 = min(b0 + 12, NB - 4);
        S1[0] = *reinterpret_cast<const uint2*>(bd0 + g1);
        S1[1] = *reinterpret_cast<const uint2*>(bd1 + g1);
    }
}

// ------------------------------------------------------------------ gate/up
template <int MW, bool DUMP>
__device__ __forceinline__ void gateup_body(const uint8_t* __restrict__ gq, const uint8_t* __restrict__ uq,
                                            const uint16_t* __restrict__ gdr, const uint16_t* __restrict__ udr,
                                            const int8_t* const (&arow)[2], int NB, const float (*s_da)[PF_TM],
                                            const TileRows& tr, int n, int I, int8_t* __restrict__ hq,
                                            float* __restrict__ hd, int32_t* __restrict__ dump)
{
    const int lane = threadIdx.x % WAVE, col = lane % 32;
    float acc[MW][2][16];
    wave_gemm<MW>(arow, gq, uq, gdr, udr, NB, s_da, acc, [&](int mi, int t, int r, int b, int isum) {
        if (DUMP) {
            const int m = 32 * mi + mfma_row(r, lane);
            if (m < tr.mcount) dump[(((int64_t)(tr.beg + tr.m0 + m) * 2 + t) * I + n) * NB + b] = isum;
        }
    });

    // SwiGLU + Q8_0 re-quantisation across the wave's 32 columns (one block of I)
#pragma unroll
    for (int mi = 0; mi < MW; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 32 * mi + mfma_row(r, lane);
            const float g = acc[mi][0][r];
            const float hv = g / (1.0f + expf(-g)) * acc[mi][1][r];
            const float amax = max_group<32>(fabsf(hv));
            const float d = amax / 127.0f;
            if (m < tr.mcount) {
                const int64_t pos = tr.beg + tr.m0 + m;
                hq[pos * I + n] = (int8_t)q8_code(hv, d);
                if (col == 0) hd[pos * (I / 32) + n / 32] = d;
            }
        }
}

template <bool DUMP>
__global__ __launch_bounds__(PF_THREADS, 2) void prefill_gateup_kernel(
    const uint8_t* __restrict__ gate_qs, const uint8_t* __restrict__ up_qs, const uint16_t* __restrict__ gate_d,
    const uint16_t* __restrict__ up_d, int E, int H, int I, const int8_t* __restrict__ xq,
    const float* __restrict__ xd, int T, int k, const int32_t* __restrict__ off, const int32_t* __restrict__ sorted,
    int8_t* __restrict__ hq, float* __restrict__ hd, float* __restrict__ y_zero, int32_t* __restrict__ dump)
{
    __shared__ __align__(16) float s_da[PF_MAX_NB][PF_TM]; // activation scales of the tile, [block][row]
    __shared__ int s_tok[PF_TM];

    if (y_zero) { // y = 0 ahead of the down kernel's scatter-add
        const int64_t total = (int64_t)T * H;
        const int64_t stride = (int64_t)gridDim.x * gridDim.y * PF_THREADS;
        for (int64_t i = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * PF_THREADS + threadIdx.x; i < total;
             i += stride)
            y_zero[i] = 0.0f;
    }
    TileRows tr;
    if (!pf_locate(off, E, tr)) return;
    const int NB = H / 32;
    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    const int col = lane % 32;

    if (tid < PF_TM) {
        int t = 0;
        if (tid < tr.mcount) t = sorted[tr.beg + tr.m0 + tid] / k;
        s_tok[tid] = t < T ? t : T - 1;
    }
    __syncthreads();
    for (int i = tid; i < NB * PF_TM; i += PF_THREADS) {
        const int b = i / PF_TM, m = i % PF_TM;
        s_da[b][m] = m < tr.mcount ? xd[(int64_t)s_tok[m] * NB + b] : 0.0f;
    }
    __syncthreads();

    const int h8 = 8 * (lane / 32); // this lane's half of every 32-wide block
    const int n = blockIdx.x * PF_GU_BN + wv * 32 + col;
    const int8_t* const arow[2] = {xq + (int64_t)s_tok[col] * H + h8, xq + (int64_t)s_tok[32 + col] * H + h8};
    const int64_t wrow = (int64_t)tr.e * I + n;
    const uint8_t* gq = gate_qs + wrow * (H / 2) + h8;
    const uint8_t* uq = up_qs + wrow * (H / 2) + h8;
    const uint16_t* gdr = gate_d + wrow * NB;
    const uint16_t* udr = up_d + wrow * NB;
    if (tr.mcount > 32)
        gateup_body<2, DUMP>(gq, uq, gdr, udr, arow, NB, s_da, tr, n, I, hq, hd, dump);
    else
        gateup_body<1, DUMP>(gq, uq, gdr, udr, arow, NB, s_da, tr, n, I, hq, hd, dump);
}

// ------------------------------------------------------------------ down + scatter-add
template <int MW, bool DUMP>
__device__ __forceinline__ void down_body(const uint8_t* __restrict__ dq0, const uint16_t* __restrict__ ddr0,
                                          const uint8_t* __restrict__ dq1, const uint16_t* __restrict__ ddr1,
                                          const int8_t* const (&arow)[2], int NB, const float (*s_da)[PF_TM],
                                          const TileRows& tr, int n0, int H, int T, int k,
                                          const float* __restrict__ topk_w, const int32_t* __restrict__ sorted,
                                          float* __restrict__ y, int32_t* __restrict__ dump)
{
    const int lane = threadIdx.x % WAVE, col = lane % 32;
    float acc[MW][2][16];
    wave_gemm<MW>(arow, dq0, dq1, ddr0, ddr1, NB, s_da, acc, [&](int mi, int t, int r, int b, int isum) {
        if (DUMP) {
            const int m = 32 * mi + mfma_row(r, lane);
            if (m < tr.mcount) dump[((int64_t)(tr.beg + tr.m0 + m) * H + n0 + 32 * t + col) * NB + b] = isum;
        }
    });
    if (DUMP) return; // the dump variant leaves y alone

#pragma unroll
    for (int mi = 0; mi < MW; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = 32 * mi + mfma_row(r, lane);
            if (m < tr.mcount) {
                const int pair = sorted[tr.beg + tr.m0 + m];
                const int t = pair / k;
                if (t < T) {
                    const float w = topk_w[pair];
                    float* yr = y + (int64_t)t * H + n0 + col;
                    atomicAdd(yr, w * acc[mi][0][r]);
                    atomicAdd(yr + 32, w * acc[mi][1][r]);
                }
            }
        }
}

template <bool DUMP>
__global__ __launch_bounds__(PF_THREADS, 2) void prefill_down_kernel(
    const uint8_t* __restrict__ down_qs, const uint16_t* __restrict__ down_d, int E, int H, int I,
    const int8_t* __restrict__ hq, const float* __restrict__ hd, int T, int k, const float* __restrict__ topk_w,
    const int32_t* __restrict__ off, const int32_t* __restrict__ sorted, float* __restrict__ y,
    int32_t* __restrict__ dump)
{
    __shared__ __align__(16) float s_da[PF_MAX_NB / 2][PF_TM];
    TileRows tr;
    if (!pf_locate(off, E, tr)) return;
    const int NB = I / 32;
    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    const int col = lane % 32;
    const int64_t pos0 = tr.beg + tr.m0;

    for (int i = tid; i < NB * PF_TM; i += PF_THREADS) {
        const int b = i / PF_TM, m = i % PF_TM;
        s_da[b][m] = m < tr.mcount ? hd[(pos0 + m) * NB + b] : 0.0f;
    }
    __syncthreads();

    const int h8 = 8 * (lane / 32); // this lane's half of every 32-wide block
    const int n0 = blockIdx.x * PF_DN_BN + wv * 64; // this wave's 64 columns: two 32-wide B tiles
    const int8_t* const arow[2] = {hq + (pos0 + (col < tr.mcount ? col : 0)) * I + h8,
                                   hq + (pos0 + (32 + col < tr.mcount ? 32 + col : 0)) * I + h8};
    const int64_t wrow0 = (int64_t)tr.e * H + n0 + col;
    const uint8_t* dq0 = down_qs + wrow0 * (I / 2) + h8;
    const uint8_t* dq1 = down_qs + (wrow0 + 32) * (I / 2) + h8;
    const uint16_t* dd0 = down_d + wrow0 * NB;
    const uint16_t* dd1 = down_d + (wrow0 + 32) * NB;
    if (tr.mcount > 32)
        down_body<2, DUMP>(dq0, dd0, dq1, dd1, arow, NB, s_da, tr, n0, H, T, k, topk_w, sorted, y, dump);
    else
        down_body<1, DUMP>(dq0, dd0, dq1, dd1, arow, NB, s_da, tr, n0, H, T, k, topk_w, sorted, y, dump);
}

// ------------------------------------------------------------------ launchers
static unsigned pf_tiles_bound(int P, int E)
{
    const int nonempty = P < E ? P : E;
    return (unsigned)((P + PF_TM - 1) / PF_TM + nonempty);
}

hipError_t launch_prefill(const uint8_t* gate_qs, const uint8_t* up_qs, const uint8_t* down_qs,
                          const uint16_t* gate_d, const uint16_t* up_d, const uint16_t* down_d, int E, int H, int I,
                          const int8_t* xq, const float* xd, int T, int k, const float* topk_w, const int32_t* off,
                          const int32_t* sorted, bool accumulate, float* y, int8_t* hq, float* hd, hipStream_t s)
{
    if (T == 0) return hipSuccess;
    const int P = T * k;
    const unsigned mt = pf_tiles_bound(P, E);
    prefill_gateup_kernel<false><<<dim3((unsigned)(I / PF_GU_BN), mt), PF_THREADS, 0, s>>>(
        gate_qs, up_qs, gate_d, up_d, E, H, I, xq, xd, T, k, off, sorted, hq, hd, accumulate ? nullptr : y, nullptr);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    prefill_down_kernel<false><<<dim3((unsigned)(H / PF_DN_BN), mt), PF_THREADS, 0, s>>>(
        down_qs, down_d, E, H, I, hq, hd, T, k, topk_w, off, sorted, y, nullptr);
    return hipGetLastError();
}

hipError_t launch_prefill_dots(const uint8_t* gate_qs, const uint8_t* up_qs, const uint8_t* down_qs,
                               const uint16_t* gate_d, const uint16_t* up_d, const uint16_t* down_d, int E, int H,
                               int I, const int8_t* xq, const float* xd, int T, int k, const int32_t* off,
                               const int32_t* sorted, int which, int8_t* hq, float* hd, int32_t* dump, hipStream_t s)
{
    if (T == 0) return hipSuccess;
    const int P = T * k;
    const unsigned mt = pf_tiles_bound(P, E);
    if (which == 0) {
        // writes hq/hd as a side effect, exactly as the production launch does
        prefill_gateup_kernel<true><<<dim3((unsigned)(I / PF_GU_BN), mt), PF_THREADS, 0, s>>>(
            gate_qs, up_qs, gate_d, up_d, E, H, I, xq, xd, T, k, off, sorted, hq, hd, nullptr, dump);
    } else {
        // y is not touched: topk_w and y are not needed by the dump epilogue
        prefill_down_kernel<true><<<dim3((unsigned)(H / PF_DN_BN), mt), PF_THREADS, 0, s>>>(
            down_qs, down_d, E, H, I, hq, hd, T, k, nullptr, off, sorted, nullptr, dump);
    }
    return hipGetLastError();
}

} // namespace moeq4
