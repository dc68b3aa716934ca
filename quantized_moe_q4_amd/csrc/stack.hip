// stack.hip -- one-launch decode of a stack of MoE layers for one token
// (Dutch technical summary "Methodologie 1" and "Methodologie 2" of "A 35B
// Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU": the W4A8
// decode over resident 4-bit experts, here layer after layer).
//
// Each layer computes h_{l+1} = [h_l +] MoE_l(Q8_0([RMSNorm] h_l)) with the
// arithmetic of the single-layer fused decode (fused.h, rows.h, topk.h), so
// the stack's hidden states are bit-identical to a chain of single-layer
// fused calls updating h in place.  What one launch adds is overlap across
// layers: the router logits of every layer are inputs, so a workgroup selects
// layer l+1's experts and issues its weight loads as soon as it has finished
// its part of layer l.  The weights then stream while layer l's h and y
// travel between workgroups, instead of after a kernel boundary.
//
// Roles, fixed for the whole launch (T = 1, k <= 8 experts per layer):
//   gate/up workgroups g < k * I/32: the a-th selected expert (ascending ids;
//     its sorted position, since each expert has one pair at T = 1) and one
//     slice of 32 outputs of I: 64 weight rows, SwiGLU and the Q8_0 block of
//     h of that slice;
//   down workgroups: 16 output rows of H over the k experts (one quad of
//     lanes per (row, expert)), the routing-weighted combine and the residual.
// Exchanges go through 64-bit words that carry a 32-bit payload in the low
// half and a tag in the high half (single-copy atomic, so a word that shows
// the expected tag carries this layer's payload): h of layer l as nine words
// per 32-value block (32 codes, then the scale), y of layer l as one word per
// element.  Layer l uses tag base + l, where base follows the last tag that
// the previous call on the workspace stored, so stale words never match.
// Each exchange has two buffers, by layer parity; a writer cannot reach a
// buffer's next use before every reader of its previous use is done, because
// each layer's y needs every gate/up workgroup's h and each layer's h needs
// every down workgroup's previous y.
//
// Forward progress: the launch is cooperative (every workgroup resident at
// once), every wait is bounded, and a wait that gives up sets the workspace's
// sticky error word, which makes every later wait of the launch give up too.
#include "fused.h"

namespace moeq4 {

constexpr int SK_MAX_LAYERS = 48;
constexpr int SK_MAX_K = 8;           // one quad per (row, expert): 8 experts x 16 rows x 4 lanes = 512 threads
constexpr int SK_ROWS = 16;           // output rows of H per down workgroup
constexpr int SK_XH_WORDS = 2560;     // h exchange words per buffer: k * I/32 * FD_XW <= 8 * 32 * 9 = 2304
constexpr int SK_XH_PER_THREAD = SK_XH_WORDS / FD_THREADS;
constexpr uint32_t SK_ERR_POLL = 64;  // polls between looks at the error word
// the stack's exchanges follow the single-layer decode's sync area and exchange (20 KB)
constexpr size_t SK_XH_OFFSET = FD_XCH_OFFSET + FD_XCH_WORDS * 8;
constexpr size_t SK_XY_OFFSET = SK_XH_OFFSET + 2 * SK_XH_WORDS * 8;

size_t stack_workspace_bytes(int H) { return SK_XY_OFFSET + 2 * (size_t)H * 8; }
int stack_max_layers() { return SK_MAX_LAYERS; }

struct SkLayers { // device pointers of every layer's experts, passed by value
    const uint8_t* gq[SK_MAX_LAYERS];
    const uint8_t* uq[SK_MAX_LAYERS];
    const uint8_t* dq[SK_MAX_LAYERS];
    const uint16_t* gd[SK_MAX_LAYERS];
    const uint16_t* ud[SK_MAX_LAYERS];
    const uint16_t* dd[SK_MAX_LAYERS];
};

// Wait until this thread's exchange words (indices first + stride * m < n,
// m < M) show `tag`, and return their payloads.  Bounded: gives up after
// FD_SPIN_LIMIT polls, or as soon as another wait of the launch has.
template <int M>
__device__ __forceinline__ void sk_wait_words(const uint64_t* __restrict__ src, int first, int stride, int n,
                                              uint32_t tag, uint32_t (&val)[M], FdCtl* __restrict__ ctl)
{
    uint32_t pend = 0;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        val[m] = 0u;
        if (first + stride * m < n) pend |= 1u << m;
    }
    uint32_t it = 0;
    while (pend) {
        uint64_t v[M];
#pragma unroll
        for (int m = 0; m < M; ++m)
            v[m] = (pend >> m) & 1u
                       ? __hip_atomic_load(src + first + stride * m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                       : 0ull;
#pragma unroll
        for (int m = 0; m < M; ++m)
            if (((pend >> m) & 1u) && (uint32_t)(v[m] >> 32) == tag) {
                val[m] = (uint32_t)v[m];
                pend &= ~(1u << m);
            }
        if (!pend) break;
        if (++it % SK_ERR_POLL == 0) {
            if (it >= FD_SPIN_LIMIT) {
                __hip_atomic_store(&ctl->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            if (__hip_atomic_load(&ctl->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

template <int BPL, int NBR, int LPL>
__global__ __launch_bounds__(FD_THREADS) void decode_stack_kernel(
    const SkLayers lp, int L, int E, int H, int I, float* h, const float* __restrict__ logits, int k, bool rmsnorm,
    bool accumulate, int G_gu, float* __restrict__ h_all, int8_t* __restrict__ hq_all, float* __restrict__ hd_all,
    FdCtl* __restrict__ ctl)
{
    __shared__ FdRoute R;
    __shared__ double s_part[FD_WAVES];
    __shared__ double s_inv;
    __shared__ float s_h[32];
    __shared__ __align__(16) int8_t s_act[2048];                  // Q8_0 codes of h_l (H <= 2048)
    __shared__ float s_ad[2048 / 32];                             // their scales
    __shared__ __align__(16) int8_t s_hq[SK_MAX_K * HQ_ROW_PADDED_MAX]; // h codes of the k pairs, padded rows
    __shared__ float s_hd[SK_MAX_K * 32];                         // their scales
    __shared__ float s_o[SK_MAX_K * SK_ROWS];                     // down outputs per (pair, row)

    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    const int g = blockIdx.x;
    const int NS = I / 32;
    const int RS = hq_row_padded(NS);
    uint64_t* xh = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ctl) + SK_XH_OFFSET); // [2][SK_XH_WORDS]
    uint64_t* xy = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ctl) + SK_XY_OFFSET); // [2][H]
    // tags base .. base + L - 1 follow the last tag stored on this workspace (0 is never a tag)
    const uint32_t ep_prev = __hip_atomic_load(&ctl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t base = ep_prev > 0xFFFFFFFEu - (uint32_t)L ? 1u : ep_prev + 1u;

    if (g < G_gu) {
        // ---------------------------------------------------------- gate/up role
        const int a = g / NS, slice = g % NS;
        const int j = lane % 8;
        const int nl = wv * 4 + lane / 16;
        const bool is_up = (lane & 8) != 0;
        const int n4 = H / 4; // float4 of h_l: thread tid holds float4 tid
        uint4 raw[BPL];
        GuScales<BPL> dh;
        // this workgroup's expert of layer l (at T = 1 the k selected experts are distinct: a < k is active)
        // and its weight loads, which stay in flight until the layer's activations are ready
        auto issue = [&](int l) {
            fd_select<LPL>(logits + (int64_t)l * E, 1, E, k, R);
            int e = fd_nth_active(R, E, a);
            if (e < 0) e = 0; // cannot happen (k distinct experts are selected); keeps the loads in bounds
            const int64_t row = (int64_t)e * I + slice * 32 + nl;
            GuRow<BPL>::issue((is_up ? lp.uq[l] : lp.gq[l]) + row * (H / 2),
                              (is_up ? lp.ud[l] : lp.gd[l]) + row * (H / 32), j, raw, dh);
        };
        issue(0);
        for (int l = 0; l < L; ++l) {
            float4 xv = make_float4(0.f, 0.f, 0.f, 0.f);
            if (l == 0) {
                if (tid < n4) xv = reinterpret_cast<const float4*>(h)[tid];
            } else { // y of the previous layer, from the tagged exchange
                uint32_t v[4];
                sk_wait_words<4>(xy + (size_t)((l - 1) & 1) * H, 4 * tid, 1, tid < n4 ? H : 0, base + l - 1, v, ctl);
                if (tid < n4)
                    xv = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                                     __uint_as_float(v[3]));
            }
            if (rmsnorm) { // the fused decode's fp64 row factor, in its order: per wave, then waves in order
                double ss = (double)xv.x * xv.x + (double)xv.y * xv.y + (double)xv.z * xv.z + (double)xv.w * xv.w;
                ss = sum_wave_f64(ss);
                if (lane == 0) s_part[wv] = ss;
                __syncthreads();
                if (tid == 0) {
                    double tot = 0.0;
                    for (int w8 = 0; w8 < FD_WAVES; ++w8)
                        if (WAVE * w8 < n4) tot += s_part[w8];
                    s_inv = 1.0 / sqrt(tot / (double)H + 1e-6);
                }
                __syncthreads();
            }
            if (tid < n4) { // whole 8-lane blocks are in or out together (H is a multiple of 32)
                float4 v = xv;
                if (rmsnorm) {
                    const double inv = s_inv;
                    v.x = (float)((double)v.x * inv);
                    v.y = (float)((double)v.y * inv);
                    v.z = (float)((double)v.z * inv);
                    v.w = (float)((double)v.w * inv);
                }
                const float amax = max_group<8>(amax4f(v));
                const float d = amax / 127.0f;
                quant4_lds(v, d, s_act + 4 * tid);
                if ((tid & 7) == 0) s_ad[tid / 8] = d;
            }
            __syncthreads();

            GuRow<BPL> w;
            w.finish(raw, dh, j);
            const float hv = swiglu_row(w, s_act, s_ad, j);
            if (!is_up && j == 0) s_h[nl] = hv;
            __syncthreads();
            if (wv == 0) { // re-quantise the slice (one Q8_0 block) and publish it
                const float v = lane < 32 ? s_h[lane] : 0.0f;
                const float amax = max_group<32>(fabsf(v));
                const float d = amax / 127.0f;
                const int code = q8_code(v, d) & 0xFF;
                uint32_t word = 0; // lane m < 8 packs the codes of outputs 4m .. 4m+3
#pragma unroll
                for (int b = 0; b < 4; ++b) word |= (uint32_t)__shfl(code, 4 * (lane % 8) + b) << (8 * b);
                if (lane < FD_XW) {
                    const uint32_t pay = lane < 8 ? word : __float_as_uint(d);
                    __hip_atomic_store(xh + (size_t)(l & 1) * SK_XH_WORDS + (a * NS + slice) * FD_XW + lane,
                                       ((uint64_t)(base + l) << 32) | pay, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
                if (hq_all) { // the layer's h codes and scales for the caller, rows in sorted-pair order
                    const int64_t pos = (int64_t)l * k + a;
                    if (lane < 8) reinterpret_cast<uint32_t*>(hq_all + pos * I + slice * 32)[lane] = word;
                    if (lane == 0) hd_all[pos * NS + slice] = d;
                }
            }
            if (l + 1 < L) issue(l + 1); // the next layer's weights stream while this layer's h travels
        }
    } else {
        // -------------------------------------------------------------- down role
        const int n0 = (g - G_gu) * SK_ROWS;
        const int qd = tid / 4, li = tid % 4, a = qd % SK_MAX_K, rs = qd / SK_MAX_K; // rs < SK_ROWS
        float resid = 0.0f; // thread tid < SK_ROWS: h_l of output row n0 + tid
        if (tid < SK_ROWS) resid = h[n0 + tid];
        for (int l = 0; l < L; ++l) {
            fd_select<LPL>(logits + (int64_t)l * E, 1, E, k, R);
            fd_sort(k, R);
            fd_weights(1, k, R);
            const bool live = a < R.U;
            DnQuad<NBR> W;
            if (live) {
                const int64_t row = (int64_t)R.list[a] * H + n0 + rs;
                W.issue(lp.dq[l] + row * (I / 2), lp.dd[l] + row * (I / 32), li);
            }
            { // h of this layer from the tagged exchange, into LDS
                const int nw = k * NS * FD_XW;
                uint32_t v[SK_XH_PER_THREAD];
                sk_wait_words<SK_XH_PER_THREAD>(xh + (size_t)(l & 1) * SK_XH_WORDS, tid, FD_THREADS, nw, base + l, v,
                                                ctl);
#pragma unroll
                for (int m = 0; m < SK_XH_PER_THREAD; ++m) {
                    const int i = tid + FD_THREADS * m;
                    if (i < nw) {
                        const int b = i / FD_XW, wd = i % FD_XW, pos = b / NS, blk = b % NS;
                        if (wd < 8)
                            *reinterpret_cast<uint32_t*>(s_hq + pos * RS + blk * 32 + (blk / 4) * 16 + wd * 4) = v[m];
                        else
                            s_hd[b] = __uint_as_float(v[m]);
                    }
                }
            }
            __syncthreads();
            if (live) {
                const int pos = R.beg[a]; // T = 1: one pair per active expert
                const float o = W.template dot<true>(s_hq + pos * RS, s_hd + pos * NS, li);
                if (li == 0) s_o[R.sorted[pos] * SK_ROWS + rs] = o;
            }
            __syncthreads();
            if (tid < SK_ROWS) { // the routing-weighted sum in slot order, then the residual
                float acc = 0.0f;
                for (int jj = 0; jj < k; ++jj) acc = fmaf(R.w[jj], s_o[jj * SK_ROWS + tid], acc);
                const float y = accumulate ? resid + acc : acc;
                resid = y;
                __hip_atomic_store(xy + (size_t)(l & 1) * H + n0 + tid,
                                   ((uint64_t)(base + l) << 32) | __float_as_uint(y), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                if (h_all) h_all[(int64_t)l * H + n0 + tid] = y;
                if (l == L - 1) h[n0 + tid] = y;
            }
        }
    }
    // departure: the last workgroup out stores the last tag used (every workgroup has read the old one)
    __syncthreads();
    if (tid == 0 &&
        __hip_atomic_fetch_add(&ctl->stack_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1) {
        __hip_atomic_store(&ctl->stack_done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctl->epoch, base + (uint32_t)L - 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ------------------------------------------------------------------ launcher
bool stack_supported(int E, int H, int I, int k)
{
    (void)E;
    return k >= 1 && k <= SK_MAX_K && H >= 256 && H <= 2048 && (I == 512 || I == 1024);
}

hipError_t launch_decode_stack(const uint8_t* const* gq, const uint8_t* const* uq, const uint8_t* const* dq,
                               const uint16_t* const* gd, const uint16_t* const* ud, const uint16_t* const* dd, int L,
                               int E, int H, int I, float* h, const float* logits, int k, bool rmsnorm,
                               bool accumulate, float* h_all, int8_t* hq_all, float* hd_all, void* ws,
                               bool* too_large, hipStream_t s)
{
    *too_large = false;
    if (L < 1 || L > SK_MAX_LAYERS || !stack_supported(E, H, I, k)) return hipErrorInvalidValue;
    SkLayers lp = {};
    for (int l = 0; l < L; ++l) {
        lp.gq[l] = gq[l];
        lp.uq[l] = uq[l];
        lp.dq[l] = dq[l];
        lp.gd[l] = gd[l];
        lp.ud[l] = ud[l];
        lp.dd[l] = dd[l];
    }
    int G_gu = k * (I / 32); // non-const: its address goes into the argument array
    const int G = G_gu + H / SK_ROWS;
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    FdCtl* ctl = reinterpret_cast<FdCtl*>(ws);
    MOEQ4_FD_BPL(H / 256, MOEQ4_FD_NBR(I / 32, MOEQ4_FD_LPL(E, {
        auto kern = decode_stack_kernel<B, R, LP>;
        err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, FD_THREADS, 0);
        if (err != hipSuccess) return err;
        if ((int64_t)per_cu * cus < G) { // every workgroup must be resident at once
            *too_large = true;
            return hipErrorInvalidValue;
        }
        void* args[] = {&lp, &L, &E, &H, &I, &h, &logits, &k, &rmsnorm, &accumulate, &G_gu, &h_all, &hq_all,
                        &hd_all, &ctl};
        err = hipLaunchCooperativeKernel((const void*)kern, dim3((unsigned)G), dim3(FD_THREADS), args, 0, s);
        if (err != hipSuccess) return err;
    })));
    return hipGetLastError();
}

} // namespace moeq4
