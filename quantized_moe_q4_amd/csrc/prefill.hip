// prefill.hip -- top-k routed W4A8 grouped GEMM over resident Q4_0 experts
// (Dutch technical summary "Methodologie 1" of "A 35B Hybrid-Attention
// Mixture-of-Experts Model on a 6GB 2011 GPU": the prefill runs a grouped
// 4-bit GEMM for the MoE; "Methodologie 4": the whole prompt goes through in
// one pass, so each touched expert is read once and the GEMM batch is as
// large as the prompt allows).
//
// Work decomposition.  Pairs are grouped by expert (moe_q4_route's counting
// sort).  Expert e with c_e pairs owns ceil(c_e / 32) m-tiles of 32 rows; the
// grid's y index enumerates m-tiles across experts (an upper bound is launched,
// surplus workgroups exit after a block-wide scan of the per-expert counts),
// x enumerates n-tiles.  A workgroup is 4 waves; each wave owns 32 output
// columns of the tile.
//
// Inner product on int8 MFMA.  v_mfma_i32_32x32x32_i8 multiplies a 32x32 int8
// A (rows m = activation rows) by a 32x32 int8 B (columns n = weight rows) over
// K = 32, exactly one Q4_0/Q8_0 block, so each MFMA yields the exact int32 block
// dot isum[m][n] for one block.  The nibbles are sign-unpacked to int8 in
// registers (q - 8).  Operand K order: lane half h (lane / 32) carries block
// elements 8h..8h+7 (bytes 0..7 of its 16-byte operand) and 16+8h..16+8h+7
// (bytes 8..15); A and B use the same order, and an integer sum over the block
// does not depend on it.  D layout: lane l holds column l % 32 and, in
// register r, row 8*(r/4) + 4*(l/32) + (r%4).
//
// Scales in fp32.  The MFMA's C operand is the bit pattern of 1.5 * 2^23
// (0x4B400000); since |isum| <= 32512 < 2^22, D read as fp32 is exactly
// 1.5*2^23 + isum.  Then t = fma(D, d_w, -1.5*2^23*d_w) = fl(isum * d_w)
// (the product 1.5*2^23*d_w is exact: 2 + 11 significant bits) and
// acc = fma(t, d_a, acc): two VALU ops per output per block.
//
// gate/up kernel: B columns are 32 gate rows and the same 32 up rows per wave;
// the epilogue forms h = silu(g) * u and re-quantises it to Q8_0 across the 32
// columns of a wave (one block of I per row), writing hq/hd in sorted-pair
// order.  down kernel: B columns are rows of W_down; the epilogue scatter-adds
// topk_w * o into y with fp32 atomics.
#include "device.h"

namespace moeq4 {

constexpr int PF_THREADS = 256;
constexpr int PF_BM = 32;   // rows of an m-tile
constexpr int PF_WN = 32;   // columns per wave (one MFMA tile)
constexpr int PF_BN = PF_WN * (PF_THREADS / WAVE);
constexpr int MAGIC_BITS = 0x4B400000; // 1.5 * 2^23
constexpr float MAGIC_F = 12582912.0f;
constexpr int PF_MAX_NB = 64;          // K blocks staged for the activation scales (K <= 2048)

__device__ __forceinline__ int mfma_row(int r, int lane)
{
    return 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
}

// 16-byte B operand from the 8 nibble bytes of half h of a weight block.
__device__ __forceinline__ v4i b_operand(const uint8_t* __restrict__ blk16, int h)
{
    const uint2 w = *reinterpret_cast<const uint2*>(blk16 + 8 * h);
    v4i b;
    b.x = nib_lo_s8(w.x);
    b.y = nib_lo_s8(w.y);
    b.z = nib_hi_s8(w.x);
    b.w = nib_hi_s8(w.y);
    return b;
}

// 16-byte A operand from an int8 activation block (32 bytes), half h.
__device__ __forceinline__ v4i a_operand(const int8_t* __restrict__ blk32, int h)
{
    const uint2 lo = *reinterpret_cast<const uint2*>(blk32 + 8 * h);
    const uint2 hi = *reinterpret_cast<const uint2*>(blk32 + 16 + 8 * h);
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

// Locate this workgroup's (expert, m-tile); false for surplus workgroups.
__device__ __forceinline__ bool pf_locate(const int32_t* __restrict__ off, int E, TileRows& tr)
{
    int e, mt;
    if (!locate_expert<PF_THREADS>(off, E, (int)blockIdx.y, [](int c) { return (c + PF_BM - 1) / PF_BM; }, e, mt))
        return false;
    tr.e = e;
    tr.beg = off[e];
    tr.m0 = mt * PF_BM;
    const int left = off[e + 1] - tr.beg - tr.m0;
    tr.mcount = left < PF_BM ? left : PF_BM;
    return true;
}

// ------------------------------------------------------------------ gate/up
template <bool DUMP>
__global__ __launch_bounds__(PF_THREADS) void prefill_gateup_kernel(
    const uint8_t* __restrict__ gate_qs, const uint8_t* __restrict__ up_qs, const uint16_t* __restrict__ gate_d,
    const uint16_t* __restrict__ up_d, int E, int H, int I, const int8_t* __restrict__ xq,
    const float* __restrict__ xd, int T, int k, const int32_t* __restrict__ off, const int32_t* __restrict__ sorted,
    int8_t* __restrict__ hq, float* __restrict__ hd, float* __restrict__ y_zero, int32_t* __restrict__ dump)
{
    __shared__ __align__(16) float s_da[PF_MAX_NB][PF_BM]; // activation scales of the tile, [block][row]
    __shared__ int s_tok[PF_BM];

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
    const int h = lane / 32, col = lane % 32;

    if (tid < PF_BM) {
        int t = 0;
        if (tid < tr.mcount) t = sorted[tr.beg + tr.m0 + tid] / k;
        s_tok[tid] = t < T ? t : T - 1;
    }
    __syncthreads();
    for (int i = tid; i < NB * PF_BM; i += PF_THREADS) {
        const int b = i / PF_BM, m = i % PF_BM;
        s_da[b][m] = m < tr.mcount ? xd[(int64_t)s_tok[m] * NB + b] : 0.0f;
    }
    __syncthreads();

    const int n = blockIdx.x * PF_BN + wv * PF_WN + col;
    const int8_t* arow = xq + (int64_t)s_tok[col] * H;
    const int64_t wrow = (int64_t)tr.e * I + n;
    const uint8_t* gq = gate_qs + wrow * (H / 2);
    const uint8_t* uq = up_qs + wrow * (H / 2);
    const uint16_t* gdr = gate_d + wrow * NB;
    const uint16_t* udr = up_d + wrow * NB;

    const v16i cmag = magic_c();
    float accg[16], accu[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) accg[r] = accu[r] = 0.0f;

    for (int b = 0; b < NB; ++b) {
        const v4i A = a_operand(arow + 32 * b, h);
        const v4i Bg = b_operand(gq + 16 * b, h);
        const v4i Bu = b_operand(uq + 16 * b, h);
        const float dwg = half_to_float(gdr[b]);
        const float dwu = half_to_float(udr[b]);
        const v16i Dg = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, Bg, cmag, 0, 0, 0);
        const v16i Du = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, Bu, cmag, 0, 0, 0);
        const float ng = -MAGIC_F * dwg, nu = -MAGIC_F * dwu;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 da = *reinterpret_cast<const float4*>(&s_da[b][8 * q + 4 * h]);
            const float dav[4] = {da.x, da.y, da.z, da.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * q + i;
                accg[r] = fmaf(fmaf(__int_as_float(Dg[r]), dwg, ng), dav[i], accg[r]);
                accu[r] = fmaf(fmaf(__int_as_float(Du[r]), dwu, nu), dav[i], accu[r]);
            }
        }
        if (DUMP) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = mfma_row(r, lane);
                if (m < tr.mcount) {
                    const int64_t pos = tr.beg + tr.m0 + m;
                    dump[((pos * 2 + 0) * I + n) * NB + b] = Dg[r] - MAGIC_BITS;
                    dump[((pos * 2 + 1) * I + n) * NB + b] = Du[r] - MAGIC_BITS;
                }
            }
        }
    }

    // SwiGLU + Q8_0 re-quantisation across the wave's 32 columns (one block of I)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int m = mfma_row(r, lane);
        const float g = accg[r];
        const float hv = g / (1.0f + expf(-g)) * accu[r];
        const float amax = max_xor<32>(fabsf(hv));
        const float d = amax / 127.0f;
        if (m < tr.mcount) {
            const int64_t pos = tr.beg + tr.m0 + m;
            hq[pos * I + n] = (int8_t)q8_code(hv, d);
            if (col == 0) hd[pos * (I / 32) + n / 32] = d;
        }
    }
}

// ------------------------------------------------------------------ down + scatter-add
template <bool DUMP>
__global__ __launch_bounds__(PF_THREADS) void prefill_down_kernel(
    const uint8_t* __restrict__ down_qs, const uint16_t* __restrict__ down_d, int E, int H, int I,
    const int8_t* __restrict__ hq, const float* __restrict__ hd, int T, int k, const float* __restrict__ topk_w,
    const int32_t* __restrict__ off, const int32_t* __restrict__ sorted, float* __restrict__ y,
    int32_t* __restrict__ dump)
{
    __shared__ __align__(16) float s_da[PF_MAX_NB][PF_BM];
    TileRows tr;
    if (!pf_locate(off, E, tr)) return;
    const int NB = I / 32;
    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    const int h = lane / 32, col = lane % 32;
    const int64_t pos0 = tr.beg + tr.m0;

    for (int i = tid; i < NB * PF_BM; i += PF_THREADS) {
        const int b = i / PF_BM, m = i % PF_BM;
        s_da[b][m] = m < tr.mcount ? hd[(pos0 + m) * NB + b] : 0.0f;
    }
    __syncthreads();

    const int n = blockIdx.x * PF_BN + wv * PF_WN + col;
    const int8_t* arow = hq + (pos0 + (col < tr.mcount ? col : 0)) * I;
    const int64_t wrow = (int64_t)tr.e * H + n;
    const uint8_t* dq = down_qs + wrow * (I / 2);
    const uint16_t* ddr = down_d + wrow * NB;

    const v16i cmag = magic_c();
    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    for (int b = 0; b < NB; ++b) {
        const v4i A = a_operand(arow + 32 * b, h);
        const v4i B = b_operand(dq + 16 * b, h);
        const float dw = half_to_float(ddr[b]);
        const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B, cmag, 0, 0, 0);
        const float nw = -MAGIC_F * dw;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 da = *reinterpret_cast<const float4*>(&s_da[b][8 * q + 4 * h]);
            const float dav[4] = {da.x, da.y, da.z, da.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * q + i;
                acc[r] = fmaf(fmaf(__int_as_float(D[r]), dw, nw), dav[i], acc[r]);
            }
        }
        if (DUMP) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = mfma_row(r, lane);
                if (m < tr.mcount) dump[((pos0 + m) * H + n) * NB + b] = D[r] - MAGIC_BITS;
            }
        }
    }

    if (DUMP) return; // the dump variant leaves y alone
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int m = mfma_row(r, lane);
        if (m < tr.mcount) {
            const int pair = sorted[pos0 + m];
            const int t = pair / k;
            if (t < T) atomicAdd(y + (int64_t)t * H + n, topk_w[pair] * acc[r]);
        }
    }
}

// ------------------------------------------------------------------ launchers
static unsigned pf_mtiles_bound(int P, int E)
{
    const int nonempty = P < E ? P : E;
    return (unsigned)((P + PF_BM - 1) / PF_BM + nonempty);
}

hipError_t launch_prefill(const uint8_t* gate_qs, const uint8_t* up_qs, const uint8_t* down_qs,
                          const uint16_t* gate_d, const uint16_t* up_d, const uint16_t* down_d, int E, int H, int I,
                          const int8_t* xq, const float* xd, int T, int k, const float* topk_w, const int32_t* off,
                          const int32_t* sorted, bool accumulate, float* y, int8_t* hq, float* hd, hipStream_t s)
{
    if (T == 0) return hipSuccess;
    const int P = T * k;
    const unsigned mt = pf_mtiles_bound(P, E);
    prefill_gateup_kernel<false><<<dim3((unsigned)(I / PF_BN), mt), PF_THREADS, 0, s>>>(
        gate_qs, up_qs, gate_d, up_d, E, H, I, xq, xd, T, k, off, sorted, hq, hd, accumulate ? nullptr : y, nullptr);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    prefill_down_kernel<false><<<dim3((unsigned)(H / PF_BN), mt), PF_THREADS, 0, s>>>(
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
    const unsigned mt = pf_mtiles_bound(P, E);
    if (which == 0) {
        // writes hq/hd as a side effect, exactly as the production launch does
        prefill_gateup_kernel<true><<<dim3((unsigned)(I / PF_BN), mt), PF_THREADS, 0, s>>>(
            gate_qs, up_qs, gate_d, up_d, E, H, I, xq, xd, T, k, off, sorted, hq, hd, nullptr, dump);
    } else {
        // y is not touched: topk_w and y are not needed by the dump epilogue
        prefill_down_kernel<true><<<dim3((unsigned)(H / PF_BN), mt), PF_THREADS, 0, s>>>(
            down_qs, down_d, E, H, I, hq, hd, T, k, nullptr, off, sorted, nullptr, dump);
    }
    return hipGetLastError();
}

} // namespace moeq4
