// stack.hip -- one-launch decode of a stack of MoE layers for one token
// (Dutch technical summary "Methodologie 1" and "Methodologie 2" of "A 35B
// Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU": the W4A8
// decode over resident 4-bit experts, here layer after layer).
//
// Each layer computes h_{l+1} = [h_l +] MoE_l(Q8_0([RMSNorm] h_l)) with the
// arithmetic of the single-layer fused decode (fused.h, rows.h, topk.h), so
// the stack's hidden states are bit-identical to a chain of single-layer
// fused calls updating h in place.  What one launch adds is overlap across
// layers: the router logits of every layer are inputs, so the routing of all
// layers is computed first (the router kernel over the [L][E] logits, one row
// per layer: the same selection and weights as the fused decode's), and a
// workgroup issues layer l+1's weight loads as soon as it has finished its
// part of layer l.  The weights then stream while layer l's h and y travel
// between workgroups, instead of after a kernel boundary.
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
// Forward progress: the grid is no larger than the device holds at once (the
// occupancy query), so on an otherwise idle device every workgroup is resident
// together; every wait is bounded, and a wait that gives up sets the
// workspace's sticky error word, which makes every later wait of the launch
// give up too (the outputs are then invalid, nothing hangs).
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

// then the routing of every layer, as the router writes it for L one-token rows
constexpr size_t SK_RT_OFFSET = SK_XY_OFFSET + 2 * 2048 * 8;
constexpr size_t SK_RT_IDS = SK_RT_OFFSET;                                // int32 [L][k]
constexpr size_t SK_RT_W = SK_RT_IDS + SK_MAX_LAYERS * SK_MAX_K * 4;      // fp32 [L][k]
constexpr size_t SK_RT_SORTED = SK_RT_W + SK_MAX_LAYERS * SK_MAX_K * 4;   // int32 [L * k] (not read)
constexpr size_t SK_RT_OFFS = SK_RT_SORTED + SK_MAX_LAYERS * SK_MAX_K * 4; // int32 [E + 1] (not read)
constexpr size_t SK_WS_BYTES = SK_RT_OFFS + (1024 + 1) * 4;

size_t stack_workspace_bytes(int H)
{
    (void)H;
    return (SK_WS_BYTES + 255) & ~(size_t)255;
}
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

template <int BPL, int NBR>
__global__ __launch_bounds__(FD_THREADS) void decode_stack_kernel(
    const SkLayers lp, int L, int H, int I, float* h, const int32_t* __restrict__ rt_ids,
    const float* __restrict__ rt_w, int k, bool rmsnorm, bool accumulate, int G_gu, float* __restrict__ h_all,
    int8_t* __restrict__ hq_all, float* __restrict__ hd_all, FdCtl* __restrict__ ctl)
{
    __shared__ float s_w[SK_MAX_LAYERS * SK_MAX_K];     // routing of every layer: weight of slot j
    __shared__ int s_list[SK_MAX_LAYERS * SK_MAX_K];    // the a-th smallest expert id (sorted position a)
    __shared__ int s_slot[SK_MAX_LAYERS * SK_MAX_K];    // and its slot
    __shared__ double s_part[FD_WAVES];
    __shared__ float s_h[32];
    __shared__ __align__(16) int8_t s_act[2048];                        // Q8_0 codes of h_l (H <= 2048)
    __shared__ float s_ad[2048 / 32];                                   // their scales
    __shared__ __align__(16) int8_t s_hq[SK_MAX_K * HQ_ROW_PADDED_MAX]; // h codes of the k pairs, padded rows
    __shared__ float s_hd[SK_MAX_K * 32];                               // their scales
    __shared__ float s_o[SK_MAX_K * SK_ROWS];                           // down outputs per (pair, row)

    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    const int g = blockIdx.x;
    const int NS = I / 32;
    const int RS = hq_row_padded(NS);
    uint64_t* xh = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ctl) + SK_XH_OFFSET); // [2][SK_XH_WORDS]
    uint64_t* xy = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ctl) + SK_XY_OFFSET); // [2][H]
    // tags base .. base + L - 1 follow the last tag stored on this workspace (0 is never a tag)
    const uint32_t ep_prev = __hip_atomic_load(&ctl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t base = ep_prev > 0xFFFFFFFEu - (uint32_t)L ? 1u : ep_prev + 1u;
    // every layer's experts in ascending order (T = 1: sorted position = rank among the k distinct ids)
    for (int i = tid; i < L * k; i += FD_THREADS) {
        const int l = i / k, j = i % k;
        const int e = rt_ids[i];
        int pos = 0;
        for (int jj = 0; jj < k; ++jj) pos += rt_ids[l * k + jj] < e;
        s_list[l * k + pos] = e;
        s_slot[l * k + pos] = j;
        s_w[i] = rt_w[i];
    }
    __syncthreads();

    if (g < G_gu) {
        // ---------------------------------------------------------- gate/up role
        // After publishing h_l the workgroup issues layer l+1's weights and unpacks them as they land, all
        // before y_l lands.  Nothing is in flight while a layer is computed (the compiler's waits at
        // control-flow joins would land it there).
        const int a = g / NS, slice = g % NS;
        const int j = lane % 8;
        const int nl = wv * 4 + lane / 16;
        const bool is_up = (lane & 8) != 0;
        const int n4 = H / 4; // float4 of h_l: thread tid holds float4 tid
        uint4 raw[BPL];
        GuScales<BPL> dh;
        GuRowUnpacked<BPL> wu; // the current layer's weights, unpacked ahead of its activations
        // layer m's weights: the a-th smallest of its k distinct experts (a < k is always active at T = 1)
        auto issue = [&](int m) {
            const int64_t row = (int64_t)s_list[m * k + a] * I + slice * 32 + nl;
            // both matrices' pointers are read uniformly (scalar loads of the argument block) and the up rows
            // taken as an offset from the gate rows: a per-lane choice of pointer would be a vector load of
            // the argument block, waited for behind the stores issued before it
            const uint8_t* qg = lp.gq[m];
            const uint16_t* dg = lp.gd[m];
            const int64_t qo = is_up ? lp.uq[m] - qg : 0, dof = is_up ? lp.ud[m] - dg : 0;
            GuRow<BPL>::issue(qg + qo + row * (H / 2), dg + dof + row * (H / 32), j, raw, dh);
        };
        auto land = [&]() { // waits for the loads of `raw`
            GuRow<BPL> w;
            w.finish(raw, dh, j);
            wu.unpack(w);
        };
        // steps l = -1 .. L-1: step l computes layer l (l >= 0), then issues and unpacks layer l+1's weights,
        // so each routine has one call site
        for (int l = -1; l < L; ++l) {
            if (l >= 0) {
                float4 xv = make_float4(0.f, 0.f, 0.f, 0.f);
                if (l == 0) {
                    if (tid < n4) xv = reinterpret_cast<const float4*>(h)[tid];
                } else { // y of the previous layer, from the tagged exchange
                    uint32_t v[4];
                    sk_wait_words<4>(xy + (size_t)((l - 1) & 1) * H, 4 * tid, 1, tid < n4 ? H : 0, base + l - 1, v,
                                     ctl);
                    // every load is back by now (the polls waited for them); said explicitly, the compiler's
                    // wait tracking knows it and puts no wait (which would include store acknowledgements,
                    // counted by the same counter here) in front of later register uses
                    __builtin_amdgcn_s_waitcnt(0);
                    if (tid < n4)
                        xv = make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                                         __uint_as_float(v[3]));
                }
                double inv = 1.0;
                if (rmsnorm) { // the fused decode's fp64 row factor, in its order: per wave, then waves in order
                    double ss = (double)xv.x * xv.x + (double)xv.y * xv.y + (double)xv.z * xv.z +
                                (double)xv.w * xv.w;
                    ss = sum_wave_f64(ss);
                    if (lane == 0) s_part[wv] = ss;
                    lds_barrier();
                    double tot = 0.0; // every thread sums the wave parts in order (no second barrier)
                    for (int w8 = 0; w8 < FD_WAVES; ++w8)
                        if (WAVE * w8 < n4) tot += s_part[w8];
                    inv = 1.0 / sqrt(tot / (double)H + 1e-6);
                }
                if (tid < n4) { // whole 8-lane blocks are in or out together (H is a multiple of 32)
                    float4 v = xv;
                    if (rmsnorm) {
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
                lds_barrier();

                const float hv = swiglu_row(wu, s_act, s_ad, j);
                if (!is_up && j == 0) s_h[nl] = hv;
                lds_barrier();
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
            } // layer l
            if (l + 1 < L) { // while h_l travels: layer l+1's weights
                issue(l + 1);
                land();
            }
        }
    } else {
        // -------------------------------------------------------------- down role
        // While waiting for h_l the workgroup holds layer l's down rows unpacked and layer l+1's in flight;
        // after publishing y_l it unpacks layer l+1 and issues layer l+2's weights, all before h_{l+1} lands.
        const int n0 = (g - G_gu) * SK_ROWS;
        const int qd = tid / 4, li = tid % 4, a = qd % SK_MAX_K, rs = qd / SK_MAX_K; // rs < SK_ROWS
        const bool live = a < k; // T = 1: the k selected experts are distinct
        DnQuad<NBR> Wq;        // packed rows of the next layer (loads in flight)
        DnQuadUnpacked<NBR> W; // unpacked rows of the current layer
        auto issue = [&](int m) {
            if (live) {
                const int64_t row = (int64_t)s_list[m * k + a] * H + n0 + rs;
                Wq.issue(lp.dq[m] + row * (I / 2), lp.dd[m] + row * (I / 32), li);
            }
        };
        float resid = 0.0f; // thread tid < SK_ROWS: h_l of output row n0 + tid
        if (tid < SK_ROWS) resid = h[n0 + tid];
        // steps l = -2 .. L-1: layer l (l >= 0), then unpack layer l+1 and issue layer l+2's weights
        for (int l = -2; l < L; ++l) {
            if (l >= 0) {
                { // h of this layer from the tagged exchange, into LDS
                    const int nw = k * NS * FD_XW;
                    uint32_t v[SK_XH_PER_THREAD];
                    sk_wait_words<SK_XH_PER_THREAD>(xh + (size_t)(l & 1) * SK_XH_WORDS, tid, FD_THREADS, nw,
                                                    base + l, v, ctl);
                    __builtin_amdgcn_s_waitcnt(0); // as in the gate/up role: everything has landed
#pragma unroll
                    for (int m = 0; m < SK_XH_PER_THREAD; ++m) {
                        const int i = tid + FD_THREADS * m;
                        if (i < nw) {
                            const int b = i / FD_XW, wd = i % FD_XW, pos = b / NS, blk = b % NS;
                            if (wd < 8)
                                *reinterpret_cast<uint32_t*>(s_hq + pos * RS + blk * 32 + (blk / 4) * 16 + wd * 4) =
                                    v[m];
                            else
                                s_hd[b] = __uint_as_float(v[m]);
                        }
                    }
                }
                lds_barrier();
                if (live) { // T = 1: the a-th active expert's pair is at sorted position a
                    const float o = W.template dot<true>(s_hq + a * RS, s_hd + a * NS, li);
                    if (li == 0) s_o[s_slot[l * k + a] * SK_ROWS + rs] = o;
                }
                lds_barrier();
                if (tid < SK_ROWS) { // the routing-weighted sum in slot order, then the residual
                    float acc = 0.0f;
                    for (int jj = 0; jj < k; ++jj) acc = fmaf(s_w[l * k + jj], s_o[jj * SK_ROWS + tid], acc);
                    const float y = accumulate ? resid + acc : acc;
                    resid = y;
                    __hip_atomic_store(xy + (size_t)(l & 1) * H + n0 + tid,
                                       ((uint64_t)(base + l) << 32) | __float_as_uint(y), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                    if (h_all) h_all[(int64_t)l * H + n0 + tid] = y;
                    if (l == L - 1) h[n0 + tid] = y;
                }
            } // layer l
            // while y_l travels: unpack layer l+1, issue layer l+2's weights
            if (l >= -1 && l + 1 < L) W.unpack(Wq);
            if (l + 2 < L) issue(l + 2);
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

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* wts, int32_t* offsets,
                        int32_t* sorted, hipStream_t s);

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
    const int G_gu = k * (I / 32);
    const int G = G_gu + H / SK_ROWS;
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    FdCtl* ctl = reinterpret_cast<FdCtl*>(ws);
    char* wsb = reinterpret_cast<char*>(ws);
    int32_t* rt_ids = reinterpret_cast<int32_t*>(wsb + SK_RT_IDS);
    float* rt_w = reinterpret_cast<float*>(wsb + SK_RT_W);
    MOEQ4_FD_BPL(H / 256, MOEQ4_FD_NBR(I / 32, {
        auto kern = decode_stack_kernel<B, R>;
        err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, FD_THREADS, 0);
        if (err != hipSuccess) return err;
        if ((int64_t)per_cu * cus < G) { // every workgroup must be resident at once
            *too_large = true;
            return hipErrorInvalidValue;
        }
        // the routing of every layer: the router over the [L][E] logits, one row per layer
        err = launch_route(logits, L, E, k, rt_ids, rt_w, reinterpret_cast<int32_t*>(wsb + SK_RT_OFFS),
                           reinterpret_cast<int32_t*>(wsb + SK_RT_SORTED), s);
        if (err != hipSuccess) return err;
        // an ordinary launch: the grid is no larger than the device holds at once, so on an otherwise idle
        // device every workgroup is resident together (and the bounded waits catch the case where it is not)
        kern<<<dim3((unsigned)G), dim3(FD_THREADS), 0, s>>>(lp, L, H, I, h, rt_ids, rt_w, k, rmsnorm, accumulate,
                                                           G_gu, h_all, hq_all, hd_all, ctl);
    }));
    return hipGetLastError();
}

} // namespace moeq4
