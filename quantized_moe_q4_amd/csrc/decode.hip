// decode.hip -- W4A8 decode GEMV over resident Q4_0 experts (Dutch technical
// summary "Methodologie 1" and "Methodologie 2" of "A 35B Hybrid-Attention
// Mixture-of-Experts Model on a 6GB 2011 GPU": a W4A8 integer kernel whose
// integer multiply-adds consume 4-bit weights and 8-bit activations; the
// "Resultaten" section names thin-M GEMM a structural bottleneck, and at
// decode batch sizes this path is a bandwidth-bound matvec, so it runs on
// v_dot4_i32_i8 and no MFMA).
//
// Row walks (one Q4_0 row = K/32 blocks of 16 nibble bytes + fp16 scales):
//   gate/up walk (K = hidden): 8 lanes per row, lane j owns blocks j, j+8, ...;
//     each load instruction of a wave reads 8 rows x 128 contiguous bytes.
//   down walk (K = inter): LPR = min(K/32, 16) lanes per row, lane j owns
//     blocks j, j+LPR, ...; a wave reads 64/LPR rows per instruction.
// Each block dot is an exact int32 sum (8 x v_dot4 on sign-unpacked nibbles),
// scaled in fp32 by d_w * d_a and summed over the row's lanes.
//
// Kernels:
//   decode_gateup: one workgroup per (touched expert, 32 outputs of I); its
//     64 rows (32 gate + the 32 matching up rows) are read once and applied
//     to every token routed to the expert; SwiGLU and the Q8_0 re-quantisation
//     of h (32 values = one block) are fused into the epilogue.
//   decode_down: one workgroup per group of output rows of H; it walks every
//     touched expert's down rows for those outputs, keeps o per pair in LDS and
//     finishes with the fixed-order routing-weighted sum into y.
#include "device.h"

namespace moeq4 {

// ------------------------------------------------------------------ row walks
template <int BPL> // blocks per lane = K / 256
struct GuRow {
    int wq[BPL][8];
    float dw[BPL];

    __device__ __forceinline__ void load(const uint8_t* __restrict__ qrow, const uint16_t* __restrict__ drow, int j)
    {
        uint4 raw[BPL];
#pragma unroll
        for (int i = 0; i < BPL; ++i) raw[i] = *reinterpret_cast<const uint4*>(qrow + (j + 8 * i) * 16);
#pragma unroll
        for (int i = 0; i < BPL; ++i) dw[i] = half_to_float(drow[j + 8 * i]);
#pragma unroll
        for (int i = 0; i < BPL; ++i) unpack_block(raw[i], wq[i]);
    }

    __device__ __forceinline__ int isum(int i, const int8_t* __restrict__ arow, int j) const
    {
        const int4* ap = reinterpret_cast<const int4*>(arow + (j + 8 * i) * 32);
        const int4 a0 = ap[0], a1 = ap[1];
        const int a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        return block_dot(wq[i], a);
    }

    // this lane's share of one output: sum over its blocks of d_w d_a isum
    __device__ __forceinline__ float partial(const int8_t* __restrict__ arow, const float* __restrict__ adr,
                                             int j) const
    {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < BPL; ++i) part = fmaf((float)isum(i, arow, j), dw[i] * adr[j + 8 * i], part);
        return part;
    }
};

template <int NBR> // blocks per row = K / 32
struct DnRow {
    static constexpr int LPR = NBR < 16 ? NBR : 16;
    static constexpr int BPL = NBR / LPR;
    int wq[BPL][8];
    float dw[BPL];

    __device__ __forceinline__ void load(const uint8_t* __restrict__ qrow, const uint16_t* __restrict__ drow, int j)
    {
        uint4 raw[BPL];
#pragma unroll
        for (int i = 0; i < BPL; ++i) raw[i] = *reinterpret_cast<const uint4*>(qrow + (j + LPR * i) * 16);
#pragma unroll
        for (int i = 0; i < BPL; ++i) dw[i] = half_to_float(drow[j + LPR * i]);
#pragma unroll
        for (int i = 0; i < BPL; ++i) unpack_block(raw[i], wq[i]);
    }

    __device__ __forceinline__ int isum(int i, const int8_t* __restrict__ arow, int j) const
    {
        const int4* ap = reinterpret_cast<const int4*>(arow + (j + LPR * i) * 32);
        const int4 a0 = ap[0], a1 = ap[1];
        const int a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        return block_dot(wq[i], a);
    }

    __device__ __forceinline__ float partial(const int8_t* __restrict__ arow, const float* __restrict__ adr,
                                             int j) const
    {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < BPL; ++i) part = fmaf((float)isum(i, arow, j), dw[i] * adr[j + LPR * i], part);
        return part;
    }
};

// ------------------------------------------------------------------ active-expert compaction
// Writes the ids of experts with at least one pair, ascending, to s_list and
// returns their number.  All threads of the block must call it.
template <int NT>
__device__ int compact_active(const int32_t* __restrict__ off, int E, int* s_list)
{
    __shared__ int s_wave[NT / WAVE];
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
    if (lane == WAVE - 1) s_wave[wv] = inc;
    __syncthreads();
    int base = 0, total = 0;
    for (int w = 0; w < NT / WAVE; ++w) {
        if (w < wv) base += s_wave[w];
        total += s_wave[w];
    }
    int pos = base + inc - local;
    for (int i = 0; i < ept; ++i) {
        const int e = e0 + i;
        if (e < E && off[e + 1] > off[e]) s_list[pos++] = e;
    }
    __syncthreads();
    return total;
}

// ------------------------------------------------------------------ gate/up + SwiGLU + requant
constexpr int DG_THREADS = 512; // 8 waves x 8 rows: 32 gate rows + 32 up rows
constexpr int DG_N = 32;        // outputs of I per workgroup (one Q8_0 block of h)
constexpr int MAX_DEC_T = 64;

template <int BPL>
__global__ __launch_bounds__(DG_THREADS) void decode_gateup_kernel(
    const uint8_t* __restrict__ gate_qs, const uint8_t* __restrict__ up_qs, const uint16_t* __restrict__ gate_d,
    const uint16_t* __restrict__ up_d, int E, int H, int I, const int8_t* __restrict__ xq,
    const float* __restrict__ xd, int k, const int32_t* __restrict__ off, const int32_t* __restrict__ sorted,
    int8_t* __restrict__ hq, float* __restrict__ hd)
{
    __shared__ float s_h[MAX_DEC_T][DG_N];
    int e, rel;
    if (!locate_expert<DG_THREADS>(off, E, (int)blockIdx.y, [](int c) { return c > 0 ? 1 : 0; }, e, rel)) return;
    const int beg = off[e];
    const int cnt = min(off[e + 1] - beg, MAX_DEC_T); // a token picks an expert at most once: cnt <= T <= 64
    const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
    const int rs = lane / 8, j = lane % 8;
    const int nl = wv * 4 + (rs & 3); // output within the workgroup's 32
    const int n = blockIdx.x * DG_N + nl;
    const bool is_up = rs >= 4;
    const int64_t row = (int64_t)e * I + n;
    GuRow<BPL> w;
    w.load((is_up ? up_qs : gate_qs) + row * (H / 2), (is_up ? up_d : gate_d) + row * (H / 32), j);

    for (int c = 0; c < cnt; ++c) {
        const int t = sorted[beg + c] / k;
        float part = w.partial(xq + (int64_t)t * H, xd + (int64_t)t * (H / 32), j);
        part = sum_xor<8>(part);
        const float up = __shfl_xor(part, 32, WAVE); // row slot rs ^ 4 holds the matching up row
        if (!is_up && j == 0) {
            const float g = part;
            s_h[c][nl] = g / (1.0f + expf(-g)) * up;
        }
    }
    __syncthreads();
    for (int c = wv; c < cnt; c += DG_THREADS / WAVE) {
        const float v = lane < DG_N ? s_h[c][lane] : 0.0f;
        const float amax = max_xor<32>(fabsf(v));
        const float d = amax / 127.0f;
        if (lane < DG_N) hq[(int64_t)(beg + c) * I + blockIdx.x * DG_N + lane] = (int8_t)q8_code(v, d);
        if (lane == 0) hd[(int64_t)(beg + c) * (I / 32) + blockIdx.x] = d;
    }
}

// ------------------------------------------------------------------ down + combine
constexpr int DD_THREADS = 128;
constexpr int MAX_DEC_P = MAX_DEC_T * 16;

template <int NBR>
__global__ __launch_bounds__(DD_THREADS) void decode_down_kernel(
    const uint8_t* __restrict__ down_qs, const uint16_t* __restrict__ down_d, int E, int H, int I,
    const int8_t* __restrict__ hq, const float* __restrict__ hd, int T, int k, const float* __restrict__ topk_w,
    const int32_t* __restrict__ off, const int32_t* __restrict__ sorted, bool accumulate, float* __restrict__ y)
{
    using Row = DnRow<NBR>;
    constexpr int SLOTS = DD_THREADS / Row::LPR; // output rows per workgroup
    __shared__ int s_list[1024];
    __shared__ float s_o[MAX_DEC_P][SLOTS];
    const int U = compact_active<DD_THREADS>(off, E, s_list);
    const int rs = threadIdx.x / Row::LPR, j = threadIdx.x % Row::LPR;
    const int n = blockIdx.x * SLOTS + rs;

    for (int a = 0; a < U; ++a) {
        const int e = s_list[a];
        const int beg = off[e], cnt = off[e + 1] - beg;
        const int64_t row = (int64_t)e * H + n;
        Row w;
        w.load(down_qs + row * (I / 2), down_d + row * (I / 32), j);
        for (int c = 0; c < cnt; ++c) {
            const int pos = beg + c;
            float part = w.partial(hq + (int64_t)pos * I, hd + (int64_t)pos * (I / 32), j);
            part = sum_xor<Row::LPR>(part);
            if (j == 0) s_o[sorted[pos]][rs] = part;
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < T * SLOTS; i += DD_THREADS) {
        const int t = i / SLOTS, r = i % SLOTS;
        float acc = 0.0f;
        for (int jj = 0; jj < k; ++jj) acc = fmaf(topk_w[t * k + jj], s_o[t * k + jj][r], acc);
        float* yp = y + (int64_t)t * H + blockIdx.x * SLOTS + r;
        *yp = accumulate ? *yp + acc : acc;
    }
}

// ------------------------------------------------------------------ single-matrix GEMV
constexpr int GV_THREADS = 256; // 4 waves x 8 rows

template <int BPL>
__global__ __launch_bounds__(GV_THREADS) void gemv_kernel(const uint8_t* __restrict__ qs, const uint16_t* __restrict__ d,
                                                          int N, int K, const int8_t* __restrict__ xq,
                                                          const float* __restrict__ xd, int T, float* __restrict__ y)
{
    const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
    const int j = lane % 8;
    const int n = (blockIdx.x * (GV_THREADS / WAVE) + wv) * 8 + lane / 8;
    if (n >= N) return; // whole 8-lane row groups exit together
    GuRow<BPL> w;
    w.load(qs + (int64_t)n * (K / 2), d + (int64_t)n * (K / 32), j);
    for (int t = 0; t < T; ++t) {
        float part = w.partial(xq + (int64_t)t * K, xd + (int64_t)t * (K / 32), j);
        part = sum_xor<8>(part);
        if (j == 0) y[(int64_t)t * N + n] = part;
    }
}

template <int BPL>
__global__ __launch_bounds__(GV_THREADS) void block_dots_gu_kernel(const uint8_t* __restrict__ qs, int N, int K,
                                                                   const int8_t* __restrict__ xq, int T,
                                                                   int32_t* __restrict__ out)
{
    const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
    const int j = lane % 8;
    const int n = (blockIdx.x * (GV_THREADS / WAVE) + wv) * 8 + lane / 8;
    if (n >= N) return;
    GuRow<BPL> w; // integer dots only: the scales are not read
    uint4 raw[BPL];
#pragma unroll
    for (int i = 0; i < BPL; ++i) raw[i] = *reinterpret_cast<const uint4*>(qs + (int64_t)n * (K / 2) + (j + 8 * i) * 16);
#pragma unroll
    for (int i = 0; i < BPL; ++i) unpack_block(raw[i], w.wq[i]);
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < BPL; ++i)
            out[((int64_t)t * N + n) * (K / 32) + j + 8 * i] = w.isum(i, xq + (int64_t)t * K, j);
}

template <int NBR>
__global__ __launch_bounds__(DD_THREADS) void block_dots_dn_kernel(const uint8_t* __restrict__ qs, int N,
                                                                   const int8_t* __restrict__ xq, int T,
                                                                   int32_t* __restrict__ out)
{
    using Row = DnRow<NBR>;
    constexpr int SLOTS = DD_THREADS / Row::LPR;
    constexpr int K = NBR * 32;
    const int rs = threadIdx.x / Row::LPR, j = threadIdx.x % Row::LPR;
    const int n = blockIdx.x * SLOTS + rs;
    if (n >= N) return;
    Row w;
    uint4 raw[Row::BPL];
#pragma unroll
    for (int i = 0; i < Row::BPL; ++i)
        raw[i] = *reinterpret_cast<const uint4*>(qs + (int64_t)n * (K / 2) + (j + Row::LPR * i) * 16);
#pragma unroll
    for (int i = 0; i < Row::BPL; ++i) unpack_block(raw[i], w.wq[i]);
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < Row::BPL; ++i)
            out[((int64_t)t * N + n) * NBR + j + Row::LPR * i] = w.isum(i, xq + (int64_t)t * K, j);
}

// ------------------------------------------------------------------ launchers
#define MOEQ4_GU_DISPATCH(BPLV, ...)                    \
    switch (BPLV) {                                     \
    case 1: { constexpr int B = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int B = 2; __VA_ARGS__; } break; \
    case 4: { constexpr int B = 4; __VA_ARGS__; } break; \
    case 8: { constexpr int B = 8; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;               \
    }

#define MOEQ4_DN_DISPATCH(NBRV, ...)                      \
    switch (NBRV) {                                       \
    case 8: { constexpr int R = 8; __VA_ARGS__; } break;   \
    case 16: { constexpr int R = 16; __VA_ARGS__; } break; \
    case 32: { constexpr int R = 32; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;                 \
    }

hipError_t launch_decode(const uint8_t* gate_qs, const uint8_t* up_qs, const uint8_t* down_qs, const uint16_t* gate_d,
                         const uint16_t* up_d, const uint16_t* down_d, int E, int H, int I, const int8_t* xq,
                         const float* xd, int T, int k, const float* topk_w, const int32_t* off,
                         const int32_t* sorted, bool accumulate, float* y, int8_t* hq, float* hd, hipStream_t s)
{
    if (T == 0) return hipSuccess;
    const int P = T * k;
    const int umax = P < E ? P : E;
    {
        const dim3 grid((unsigned)(I / DG_N), (unsigned)umax);
        MOEQ4_GU_DISPATCH(H / 256, decode_gateup_kernel<B><<<grid, DG_THREADS, 0, s>>>(
                                       gate_qs, up_qs, gate_d, up_d, E, H, I, xq, xd, k, off, sorted, hq, hd));
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    MOEQ4_DN_DISPATCH(I / 32, {
        constexpr int SLOTS = DD_THREADS / DnRow<R>::LPR;
        decode_down_kernel<R><<<dim3((unsigned)(H / SLOTS)), DD_THREADS, 0, s>>>(
            down_qs, down_d, E, H, I, hq, hd, T, k, topk_w, off, sorted, accumulate, y);
    });
    return hipGetLastError();
}

hipError_t launch_gemv(const uint8_t* qs, const uint16_t* d, int N, int K, const int8_t* xq, const float* xd, int T,
                       float* y, hipStream_t s)
{
    if (N == 0 || T == 0) return hipSuccess;
    const int rows_per_wg = (GV_THREADS / WAVE) * 8;
    const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg));
    MOEQ4_GU_DISPATCH(K / 256, gemv_kernel<B><<<grid, GV_THREADS, 0, s>>>(qs, d, N, K, xq, xd, T, y));
    return hipGetLastError();
}

hipError_t launch_block_dots(const uint8_t* qs, int N, int K, const int8_t* xq, int T, bool down_walk, int32_t* out,
                             hipStream_t s)
{
    if (N == 0 || T == 0) return hipSuccess;
    if (!down_walk) {
        const int rows_per_wg = (GV_THREADS / WAVE) * 8;
        const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg));
        MOEQ4_GU_DISPATCH(K / 256, block_dots_gu_kernel<B><<<grid, GV_THREADS, 0, s>>>(qs, N, K, xq, T, out));
    } else {
        MOEQ4_DN_DISPATCH(K / 32, {
            constexpr int SLOTS = DD_THREADS / DnRow<R>::LPR;
            block_dots_dn_kernel<R><<<dim3((unsigned)((N + SLOTS - 1) / SLOTS)), DD_THREADS, 0, s>>>(qs, N, xq, T,
                                                                                                    out);
        });
    }
    return hipGetLastError();
}

} // namespace moeq4
