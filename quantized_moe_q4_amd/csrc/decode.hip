// decode.hip -- W4A8 decode GEMV over resident Q4_0 experts (Dutch technical
// summary "Methodologie 1" and "Methodologie 2" of "A 35B Hybrid-Attention
// Mixture-of-Experts Model on a 6GB 2011 GPU": a W4A8 integer kernel whose
// integer multiply-adds consume 4-bit weights and 8-bit activations; the
// "Resultaten" section names thin-M GEMM a structural bottleneck, and at
// decode batch sizes this path is a bandwidth-bound matvec, so it runs on
// v_dot4_i32_i8 and no MFMA).
//
// Row walks, the SwiGLU row and the down walk live in rows.h (shared with
// the fused one-launch decode).
//
// Kernels (every touched expert's weights are read once per call):
//   decode_gateup: one workgroup per (touched expert, 32 outputs of I); its
//     64 rows (32 gate + the 32 matching up rows) are applied to every token
//     routed to the expert; SwiGLU and the Q8_0 re-quantisation of h (32 values
//     = one block) are fused into the epilogue.
//   decode_down: one workgroup per group of output rows of H; it walks every
//     touched expert's down rows for those outputs, keeps o per pair in LDS
//     and ends with y[t] (+)= sum_j w[t][j] o[t*k+j], a fixed-order sum, so
//     decode results are deterministic and need no cross-workgroup exchange
//     (a device-scope release per workgroup, which a cross-workgroup combine
//     would need, writes back the L2 on this multi-XCD part).
#include "device.h"
#include "rows.h"

namespace moeq4 {

// ------------------------------------------------------------------ gate/up + SwiGLU + requant
constexpr int DG_THREADS = 512; // 8 waves x 8 rows: 32 gate rows + 32 up rows
constexpr int DG_N = 32;        // outputs of I per workgroup (one Q8_0 block of h)
constexpr int MAX_DEC_T = 64;
constexpr int DD_THREADS = 128;

constexpr int DG_TCHUNK = 16; // tokens staged in LDS at a time

template <int BPL>
__global__ __launch_bounds__(DG_THREADS, 4) void decode_gateup_kernel(
    const uint8_t* __restrict__ gate_qs, const uint8_t* __restrict__ up_qs, const uint16_t* __restrict__ gate_d,
    const uint16_t* __restrict__ up_d, int E, int H, int I, const int8_t* __restrict__ xq,
    const float* __restrict__ xd, int T, int k, const int32_t* __restrict__ off, const int32_t* __restrict__ sorted,
    int8_t* __restrict__ hq, float* __restrict__ hd)
{
    constexpr int HMAX = 256 * BPL; // hidden size of this instantiation
    __shared__ float s_h[MAX_DEC_T][DG_N];
    __shared__ __align__(16) int8_t s_act[DG_TCHUNK][HMAX];
    __shared__ float s_ad[DG_TCHUNK][HMAX / 32];
    __shared__ int s_tok[MAX_DEC_T];
    int e, rel;
    if (!locate_expert<DG_THREADS>(off, E, (int)blockIdx.y, [](int c) { return c > 0 ? 1 : 0; }, e, rel)) return;
    const int beg = off[e];
    const int cnt = min(off[e + 1] - beg, MAX_DEC_T); // a token picks an expert at most once: cnt <= T <= 64
    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    // a 16-lane DPP row per output: lanes 0-7 walk the gate row, 8-15 the up row
    const int j = lane % 8;
    const int nl = wv * 4 + lane / 16; // output within the workgroup's 32
    const int n = blockIdx.x * DG_N + nl;
    const bool is_up = (lane & 8) != 0;
    const int64_t row = (int64_t)e * I + n;
    // weight loads go out first; the token ids and activations follow while they are in flight
    uint4 raw[BPL];
    GuScales<BPL> dh;
    GuRow<BPL>::issue((is_up ? up_qs : gate_qs) + row * (H / 2), (is_up ? up_d : gate_d) + row * (H / 32), j, raw,
                      dh);
    if (tid < cnt) s_tok[tid] = min(sorted[beg + tid] / k, T - 1);
    __syncthreads();
    GuRow<BPL> w;
    bool unpacked = false;

    for (int c0 = 0; c0 < cnt; c0 += DG_TCHUNK) {
        const int nc = min(DG_TCHUNK, cnt - c0);
        // stage this chunk's activation rows (16-byte pieces) and their scales
        for (int i = tid; i < nc * (H / 16); i += DG_THREADS) {
            const int c = i / (H / 16), q = i % (H / 16);
            *reinterpret_cast<int4*>(&s_act[c][16 * q]) =
                *reinterpret_cast<const int4*>(xq + (int64_t)s_tok[c0 + c] * H + 16 * q);
        }
        for (int i = tid; i < nc * (H / 32); i += DG_THREADS) {
            const int c = i / (H / 32), q = i % (H / 32);
            s_ad[c][q] = xd[(int64_t)s_tok[c0 + c] * (H / 32) + q];
        }
        __syncthreads();
        if (!unpacked) { // first chunk: the weights are needed from here on
            w.finish(raw, dh, j);
            unpacked = true;
        }
        for (int c = 0; c < nc; ++c) {
            const float h = swiglu_row(w, s_act[c], s_ad[c], j);
            if (!is_up && j == 0) s_h[c0 + c][nl] = h;
        }
        __syncthreads();
    }
    for (int c = wv; c < cnt; c += DG_THREADS / WAVE) {
        const float v = lane < DG_N ? s_h[c][lane] : 0.0f;
        const float amax = max_group<32>(fabsf(v));
        const float d = amax / 127.0f;
        if (lane < DG_N) hq[(int64_t)(beg + c) * I + blockIdx.x * DG_N + lane] = (int8_t)q8_code(v, d);
        if (lane == 0) hd[(int64_t)(beg + c) * (I / 32) + blockIdx.x] = d;
    }
}

// ------------------------------------------------------------------ down + combine
// One workgroup per SLOTS rows of H: it walks the down rows of every touched
// expert for those outputs (rows.h), keeps o per pair in LDS and ends with the
// fixed-order routing-weighted sum, so no other workgroup's data is needed.
// When hq fits (P * I <= 64 KB) it is staged in LDS once.
constexpr int DD_STAGE_BYTES = 64 * 1024; // hq staged in LDS up to this size
constexpr int MAX_DEC_P = MAX_DEC_T * 16;
constexpr int DD_ROW_MAJOR_MAX_EXPERTS = 8; // beyond this many possible experts: expert-major down + combine
                                              // (measured faster from 16 possible experts on)

template <int NBR, bool STAGE>
__global__ __launch_bounds__(DD_THREADS) void decode_down_kernel(
    const uint8_t* __restrict__ down_qs, const uint16_t* __restrict__ down_d, int E, int H, int I,
    const int8_t* __restrict__ hq, const float* __restrict__ hd, int T, int k, const float* __restrict__ topk_w,
    const int32_t* __restrict__ off, const int32_t* __restrict__ sorted, bool accumulate, float* __restrict__ y)
{
    using Row = DnRow<NBR>;
    constexpr int SLOTS = DD_THREADS / Row::LPR; // output rows per workgroup
    constexpr int SP = STAGE ? DD_STAGE_BYTES / (32 * NBR) : 1; // pairs that fit the staging area
    __shared__ int s_list[1024];
    __shared__ int s_beg[1025];
    __shared__ int s_pair[MAX_DEC_P];
    __shared__ float s_o[MAX_DEC_P * SLOTS];
    __shared__ __align__(16) int8_t s_hq[STAGE ? SP : 1][STAGE ? 32 * NBR : 16];
    __shared__ float s_hd[STAGE ? SP : 1][STAGE ? NBR : 1];
    const int tid = threadIdx.x;
    const int P = T * k;
    DnWalk c;
    c.qs = down_qs;
    c.d = down_d;
    c.H = H;
    c.I = I;
    c.list = s_list;
    c.beg = s_beg;
    c.pair = s_pair;
    c.U = compact_active<DD_THREADS>(off, E, s_list, s_beg);
    c.rs = tid / Row::LPR;
    c.j = tid % Row::LPR;
    c.n = blockIdx.x * SLOTS + c.rs;
    c.slots = SLOTS;
    c.s_o = s_o;

    DnBatch<NBR> A, B;
    dn_issue<NBR>(A, c, 0);
    for (int p = tid; p < P; p += DD_THREADS) s_pair[p] = sorted[p];
    if (STAGE) {
        for (int i = tid; i < P * (I / 16); i += DD_THREADS)
            *reinterpret_cast<int4*>(&s_hq[i / (I / 16)][16 * (i % (I / 16))]) =
                *reinterpret_cast<const int4*>(hq + (int64_t)16 * i);
        for (int i = tid; i < P * (I / 32); i += DD_THREADS) s_hd[i / (I / 32)][i % (I / 32)] = hd[i];
    }
    __syncthreads();
    if (STAGE)
        dn_walk<NBR>(A, B, c, [&](int pos, const int8_t*& arow, const float*& adr) {
            arow = s_hq[pos];
            adr = s_hd[pos];
        });
    else
        dn_walk<NBR>(A, B, c, [&](int pos, const int8_t*& arow, const float*& adr) {
            arow = hq + (int64_t)pos * I;
            adr = hd + (int64_t)pos * (I / 32);
        });
    __syncthreads();
    dn_combine(s_o, SLOTS, T, k, topk_w, accumulate, y, H, blockIdx.x * SLOTS, tid, DD_THREADS);
}

// ------------------------------------------------------------------ down, expert-major + combine
// For larger batches the row-major walk above visits many experts one batch
// after another and is bound by load latency.  Here every (touched expert,
// DE_ROWS rows of H) is its own workgroup, as in gate/up: the expert's h rows
// are staged in LDS and o = W_down h is written per pair to the workspace;
// decode_combine_kernel then forms y with the same fixed-order sum.  Same
// row walk and reductions as the row-major walk, so o and y are bit-identical.
constexpr int DE_THREADS = 256;
constexpr int DE_RPL = 4; // rows per lane group

template <int NBR>
__global__ __launch_bounds__(DE_THREADS) void decode_down_em_kernel(
    const uint8_t* __restrict__ down_qs, const uint16_t* __restrict__ down_d, int E, int H, int I,
    const int8_t* __restrict__ hq, const float* __restrict__ hd, const int32_t* __restrict__ off,
    const int32_t* __restrict__ sorted, float* __restrict__ o)
{
    using Row = DnRow<NBR>;
    constexpr int GROUPS = DE_THREADS / Row::LPR;
    constexpr int ROWS = GROUPS * DE_RPL; // rows of H per workgroup
    extern __shared__ __align__(16) uint8_t de_dyn[];
    __shared__ int s_pair[MAX_DEC_T];
    int e, rel;
    if (!locate_expert<DE_THREADS>(off, E, (int)blockIdx.y, [](int c) { return c > 0 ? 1 : 0; }, e, rel)) return;
    const int beg = off[e];
    const int cnt = min(off[e + 1] - beg, MAX_DEC_T); // a token picks an expert at most once: cnt <= T <= 64
    const int tid = threadIdx.x, grp = tid / Row::LPR, j = tid % Row::LPR;
    const int n0 = blockIdx.x * ROWS;
    int8_t* s_hq = reinterpret_cast<int8_t*>(de_dyn);                 // [cnt][I]
    float* s_hd = reinterpret_cast<float*>(de_dyn + (size_t)cnt * I);   // [cnt][I/32]

    // weight loads go out first; the expert's h rows are staged while they are in flight
    uint4 raw[DE_RPL][Row::BPL];
    uint16_t dh[DE_RPL][Row::BPL];
    {
        Row wr;
#pragma unroll
        for (int r = 0; r < DE_RPL; ++r) {
            const int64_t row = (int64_t)e * H + n0 + grp + GROUPS * r;
            wr.issue(down_qs + row * (I / 2), down_d + row * (I / 32), j, raw[r], dh[r]);
        }
    }
    for (int i = tid; i < cnt * (I / 16); i += DE_THREADS)
        *reinterpret_cast<int4*>(s_hq + 16 * i) = *reinterpret_cast<const int4*>(hq + (int64_t)beg * I + 16 * i);
    for (int i = tid; i < cnt * NBR; i += DE_THREADS) s_hd[i] = hd[(int64_t)beg * NBR + i];
    if (tid < cnt) s_pair[tid] = sorted[beg + tid];
    __syncthreads();
    Row w[DE_RPL];
#pragma unroll
    for (int r = 0; r < DE_RPL; ++r) w[r].finish(raw[r], dh[r]);
    for (int c = 0; c < cnt; ++c) {
        typename Row::Act act;
        Row::load_act(s_hq + (size_t)c * I, s_hd + c * NBR, j, act);
        float part[DE_RPL];
#pragma unroll
        for (int r = 0; r < DE_RPL; ++r) part[r] = w[r].dot(act);
#pragma unroll
        for (int r = 0; r < DE_RPL; ++r) part[r] = sum_group<Row::LPR>(part[r]);
        if (j == 0) {
            float* orow = o + (int64_t)s_pair[c] * H + n0 + grp;
#pragma unroll
            for (int r = 0; r < DE_RPL; ++r) orow[GROUPS * r] = part[r];
        }
    }
}

// y[t][n] (+)= sum_j topk_w[t][j] * o[t*k + j][n], j = 0..k-1 in order; 4 outputs per thread
__global__ __launch_bounds__(256) void decode_combine_kernel(const float* __restrict__ o,
                                                             const float* __restrict__ topk_w, int T, int k, int H,
                                                             bool accumulate, float* __restrict__ y)
{
    const int H4 = H / 4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * H4) return;
    const int t = (int)(i / H4), n4 = (int)(i % H4);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // the token's k rows, loaded 8 at a time before they are summed (in slot order)
    for (int j0 = 0; j0 < k; j0 += 8) {
        float4 v[8];
        float wv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int jj = j0 + u < k ? j0 + u : j0;
            v[u] = reinterpret_cast<const float4*>(o + (int64_t)(t * k + jj) * H)[n4];
            wv[u] = topk_w[t * k + jj];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (j0 + u < k) {
                acc.x = fmaf(wv[u], v[u].x, acc.x);
                acc.y = fmaf(wv[u], v[u].y, acc.y);
                acc.z = fmaf(wv[u], v[u].z, acc.z);
                acc.w = fmaf(wv[u], v[u].w, acc.w);
            }
        }
    }
    float4* yp = reinterpret_cast<float4*>(y + (int64_t)t * H) + n4;
    if (accumulate) {
        const float4 yv = *yp;
        acc.x = yv.x + acc.x;
        acc.y = yv.y + acc.y;
        acc.z = yv.z + acc.z;
        acc.w = yv.w + acc.w;
    }
    *yp = acc;
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
    w.template load<false>(qs + (int64_t)n * (K / 2), d + (int64_t)n * (K / 32), j); // (default cache policy)
    for (int t = 0; t < T; ++t) {
        float part = w.partial(xq + (int64_t)t * K, xd + (int64_t)t * (K / 32), j);
        part = sum_group<8>(part);
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
    w.unpack_only(qs + (int64_t)n * (K / 2), j);
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < BPL; ++i)
            out[((int64_t)t * N + n) * (K / 32) + j + 8 * i] = w.isum16(i, xq + (int64_t)t * K, j) >> 4;
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
    for (int i = 0; i < Row::BPL; ++i) unpack_block16(raw[i], w.wq[i]);
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < Row::BPL; ++i)
            out[((int64_t)t * N + n) * NBR + j + Row::LPR * i] = w.isum16(i, xq + (int64_t)t * K, j) >> 4;
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

// y (+)= sum_j w[t][j] * o[t*k + j] for every token, in slot order (also the prefill's combine)
hipError_t launch_combine(const float* o, const float* topk_w, int T, int k, int H, bool accumulate, float* y,
                          hipStream_t s)
{
    const int64_t n4 = (int64_t)T * (H / 4);
    if (n4 == 0) return hipSuccess;
    decode_combine_kernel<<<dim3((unsigned)((n4 + 255) / 256)), 256, 0, s>>>(o, topk_w, T, k, H, accumulate, y);
    return hipGetLastError();
}

hipError_t launch_decode(const uint8_t* gate_qs, const uint8_t* up_qs, const uint8_t* down_qs, const uint16_t* gate_d,
                         const uint16_t* up_d, const uint16_t* down_d, int E, int H, int I, const int8_t* xq,
                         const float* xd, int T, int k, const float* topk_w, const int32_t* off,
                         const int32_t* sorted, bool accumulate, float* y, int8_t* hq, float* hd, float* o,
                         hipStream_t s)
{
    if (T == 0) return hipSuccess;
    const int P = T * k;
    const int umax = P < E ? P : E;
    {
        const dim3 grid((unsigned)(I / DG_N), (unsigned)umax);
        MOEQ4_GU_DISPATCH(H / 256, decode_gateup_kernel<B><<<grid, DG_THREADS, 0, s>>>(
                                       gate_qs, up_qs, gate_d, up_d, E, H, I, xq, xd, T, k, off, sorted, hq, hd));
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (umax > DD_ROW_MAJOR_MAX_EXPERTS) { // many touched experts: expert-major down, then the combine
        MOEQ4_DN_DISPATCH(I / 32, {
            constexpr int ROWS = (DE_THREADS / DnRow<R>::LPR) * DE_RPL;
            const size_t lds = (size_t)T * I + (size_t)T * (I / 32) * 4;
            if (lds > 64 * 1024) {
                hipError_t e2 = hipFuncSetAttribute((const void*)decode_down_em_kernel<R>,
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
                if (e2 != hipSuccess) return e2;
            }
            decode_down_em_kernel<R><<<dim3((unsigned)(H / ROWS), (unsigned)umax), DE_THREADS, lds, s>>>(
                down_qs, down_d, E, H, I, hq, hd, off, sorted, o);
        });
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        const int64_t n4 = (int64_t)T * (H / 4);
        decode_combine_kernel<<<dim3((unsigned)((n4 + 255) / 256)), 256, 0, s>>>(o, topk_w, T, k, H, accumulate, y);
        return hipGetLastError();
    }
    const bool stage = (int64_t)P * I <= DD_STAGE_BYTES;
    MOEQ4_DN_DISPATCH(I / 32, {
        constexpr int SLOTS = DD_THREADS / DnRow<R>::LPR;
        const dim3 grid((unsigned)(H / SLOTS));
        if (stage)
            decode_down_kernel<R, true><<<grid, DD_THREADS, 0, s>>>(down_qs, down_d, E, H, I, hq, hd, T, k, topk_w,
                                                                     off, sorted, accumulate, y);
        else
            decode_down_kernel<R, false><<<grid, DD_THREADS, 0, s>>>(down_qs, down_d, E, H, I, hq, hd, T, k, topk_w,
                                                                      off, sorted, accumulate, y);
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
