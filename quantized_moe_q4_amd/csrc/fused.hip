// fused.hip -- one-launch MoE decode for small batches: Q8_0 activation
// quantisation, routing, gate/up + SwiGLU + re-quantisation, down and the
// routing-weighted combine (Dutch technical summary "Methodologie 1" and
// "Methodologie 2" of "A 35B Hybrid-Attention Mixture-of-Experts Model on a
// 6GB 2011 GPU": the W4A8 decode over resident 4-bit experts).
//
// At decode batch sizes the layer moves a few MB of weights, which the chip
// reads in about a microsecond; four dependent launches would cost several
// microseconds each.  This kernel runs the layer in one launch with two roles:
//   gate/up workgroups (ids 0 .. G_gu-1): items (touched expert, 32 outputs
//     of I), as the standalone gate/up kernel, workgroup g taking items g,
//     g + G_gu, ...; G_gu is capped so that the whole grid is resident at
//     once (a second round of workgroups would wait for the first to end);
//   down workgroups (ids G_gu ..): one per group of output rows of H, as the
//     standalone down kernel.
// Every workgroup selects the T <= 8 tokens' experts itself (all threads rank
// the logits in parallel) and sorts the pairs, so no launch is needed for
// routing; a gate/up workgroup reads its expert off the selection's bitmask
// and issues its weight loads before the sort, then quantises the
// activations into LDS while they are in flight.  Down
// workgroups issue their weight loads first, compute the routing weights, and
// only then wait until every active gate/up workgroup has published its slice
// of h: the down weights stream while gate/up runs.  A down workgroup is two
// expert groups of 256 threads over the same output rows, each walking every
// other active expert.
//
// Exchange of h between workgroups (they run on different XCDs, whose L2
// caches are not coherent with each other): gate/up writes hq/hd with
// device-scope atomic stores, waits for them to complete, and bumps an arrival
// counter with a device-scope atomic add; down polls the counter with
// device-scope atomic loads and reads hq/hd with device-scope atomic loads.
// None of these go through a full-L2 writeback or invalidate.
// Forward progress: gate/up workgroups never wait and have the lower ids, so
// each one is dispatched before any down workgroup of the same dispatch queue
// can occupy its slot; the wait is also bounded (a sticky error word records a
// timeout).  The last down workgroup to pass the wait resets the counters, so
// every call leaves them at zero for the next one on the same workspace.
//
// The arithmetic is the standalone kernels' (rows.h, topk.h, the same Q8_0
// rounding), so fused and standalone decode agree bit for bit.
#include "fused.h"

namespace moeq4 {

template <int BPL, int NBR, int LPL>
__global__ __launch_bounds__(FD_THREADS) void decode_fused_kernel(
    const uint8_t* __restrict__ gate_qs, const uint8_t* __restrict__ up_qs, const uint8_t* __restrict__ down_qs,
    const uint16_t* __restrict__ gate_d, const uint16_t* __restrict__ up_d, const uint16_t* __restrict__ down_d,
    int E, int H, int I, const float* x, const float* __restrict__ logits, int T, int k, bool rmsnorm,
    bool accumulate, int G_gu, int G_dn, int32_t* __restrict__ ids_out, float* __restrict__ w_out,
    int32_t* __restrict__ off_out, int32_t* __restrict__ sorted_out, float* y, int8_t* __restrict__ hq,
    float* __restrict__ hd, FdCtl* __restrict__ ctl, bool tagged)
{
    using Dn = DnRow<NBR>;
    constexpr int SLOTS = FD_GROUP / Dn::LPR;     // down output rows per workgroup
    constexpr int EGROUPS = FD_THREADS / FD_GROUP; // expert groups of a down workgroup
    __shared__ FdRoute R;
    __shared__ double s_inv[FD_MAX_T];
    __shared__ double s_part[FD_MAX_T][FD_WAVES];
    __shared__ float s_h[FD_MAX_T][32];
    extern __shared__ __align__(16) uint8_t fd_dyn[];

    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    const int g = blockIdx.x;
    const int P = T * k;
    const int NS = I / 32; // gate/up slices of I (one Q8_0 block of h each)
    uint64_t* xch = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ctl) + FD_XCH_OFFSET);
    // this call's epoch (the previous call on the workspace stored its own before it ended)
    const uint32_t ep_prev = __hip_atomic_load(&ctl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t ep = ep_prev >= 0xFFFFFFFEu ? 1u : ep_prev + 1u;

    // gate/up workgroups load the activations before routing (they do not depend on it)
    const int n4 = H / 4, nx = T * n4;
    float4 xv[FD_MAX_T]; // thread tid holds float4 tid + FD_THREADS*m of x
    if (g < G_gu) {
#pragma unroll
        for (int m = 0; m < FD_MAX_T; ++m) {
            const int i = tid + FD_THREADS * m;
            xv[m] = i < nx ? reinterpret_cast<const float4*>(x)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    fd_select<LPL>(logits, T, E, k, R);

    if (g < G_gu) {
        // ---------------------------------------------------------- gate/up role
        // Items are (active expert a, slice of 32 outputs of I), item a * NS + slice; this workgroup takes items
        // g, g + G_gu, ...  The first item's expert comes from the bitmask of the selection, so its weight loads
        // go out before the pairs are sorted; a later item's loads go out as soon as the previous item's weights
        // are in registers, while that item's SwiGLU and re-quantisation run.
        const int e0 = fd_nth_active(R, E, g / NS);
        if (e0 < 0) return; // no such active expert: this workgroup takes no part
        const int j = lane % 8;
        const int nl = wv * 4 + lane / 16;
        const bool is_up = (lane & 8) != 0;
        uint4 raw[BPL];
        GuScales<BPL> dh;
        auto issue = [&](int e, int slice) {
            const int64_t row = (int64_t)e * I + slice * 32 + nl;
            GuRow<BPL>::issue((is_up ? up_qs : gate_qs) + row * (H / 2), (is_up ? up_d : gate_d) + row * (H / 32),
                              j, raw, dh);
        };
        issue(e0, g % NS);
        fd_sort(P, R);
        if (g == 0) fd_write_route(R, T, E, k, ids_out, off_out, sorted_out);

        // Q8_0 rows of the T tokens in LDS while the weights are in flight.  A
        // wave's 64 float4 of one m lie in one row (n4 is a multiple of 64), and
        // 8 consecutive lanes hold one 32-block.
        int8_t* s_act = reinterpret_cast<int8_t*>(fd_dyn);                         // [T][H]
        float* s_ad = reinterpret_cast<float*>(fd_dyn + (size_t)T * H);             // [T][H/32]
        if (rmsnorm) { // row sums of squares in fp64: per (m, wave), then per row in a fixed order
#pragma unroll
            for (int m = 0; m < FD_MAX_T; ++m) {
                if (FD_THREADS * m >= nx) break;
                const float4 v = xv[m];
                double ss = (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
                ss = sum_wave_f64(ss);
                if (lane == 0) s_part[m][wv] = ss;
            }
            lds_barrier(); // LDS only: the weight loads stay in flight
            if (tid < T) {
                double tot = 0.0;
                for (int m = 0; m < FD_MAX_T; ++m)
                    for (int w8 = 0; w8 < FD_WAVES; ++w8) {
                        const int i0 = FD_THREADS * m + WAVE * w8;
                        if (i0 < nx && i0 / n4 == tid) tot += s_part[m][w8];
                    }
                s_inv[tid] = 1.0 / sqrt(tot / (double)H + 1e-6);
            }
            lds_barrier(); // LDS only: the weight loads stay in flight
        }
#pragma unroll
        for (int m = 0; m < FD_MAX_T; ++m) {
            const int i = tid + FD_THREADS * m;
            if (FD_THREADS * m >= nx) break; // whole waves stop together (nx is a multiple of 64)
            if (i < nx) {
                const int t = i / n4, q = i % n4;
                float4 v = xv[m];
                if (rmsnorm) {
                    const double inv = s_inv[t];
                    v.x = (float)((double)v.x * inv);
                    v.y = (float)((double)v.y * inv);
                    v.z = (float)((double)v.z * inv);
                    v.w = (float)((double)v.w * inv);
                }
                const float amax = max_group<8>(amax4f(v));
                const float d = amax / 127.0f;
                quant4_lds(v, d, s_act + (int64_t)t * H + 4 * q);
                if ((q & 7) == 0) s_ad[t * (H / 32) + q / 8] = d;
            }
        }
        lds_barrier(); // LDS only: the weight loads stay in flight

        const int NI = R.U * NS;
        uint32_t items = 0; // items this workgroup has published
        // one item; multi: more may follow (the straight path, at most one item per workgroup, has no
        // look-ahead to test)
        auto run = [&](int item, auto multi) {
            const int a = item / NS, slice = item % NS;
            const int beg = R.beg[a], cnt = R.beg[a + 1] - beg;
            GuRow<BPL> w;
            w.finish(raw, dh, j);
            if constexpr (decltype(multi)::value)
                if (item + G_gu < NI) issue(R.list[(item + G_gu) / NS], (item + G_gu) % NS);
            for (int c = 0; c < cnt; ++c) {
                const int t = R.sorted[beg + c] / k;
                const float h = swiglu_row(w, s_act + (int64_t)t * H, s_ad + t * (H / 32), j);
                if (!is_up && j == 0) s_h[c][nl] = h;
            }
            lds_barrier(); // LDS only: the weight loads stay in flight
            // re-quantise (one block of 32 per token) and publish with device-scope stores
            for (int c = wv; c < cnt; c += FD_WAVES) {
                const float v = lane < 32 ? s_h[c][lane] : 0.0f;
                const float amax = max_group<32>(fabsf(v));
                const float d = amax / 127.0f;
                const int code = q8_code(v, d) & 0xFF;
                uint32_t word = 0; // lane m < 8 packs the codes of outputs 4m .. 4m+3
#pragma unroll
                for (int b = 0; b < 4; ++b) word |= (uint32_t)__shfl(code, 4 * (lane % 8) + b) << (8 * b);
                const int64_t pos = beg + c;
                if (tagged) {
                    // hq/hd keep the call's values for the caller; the tagged words carry them to the down side
                    if (lane < 8) reinterpret_cast<uint32_t*>(hq + pos * I + slice * 32)[lane] = word;
                    if (lane == 0) hd[pos * NS + slice] = d;
                    if (lane < FD_XW) {
                        const uint32_t pay = lane < 8 ? word : __float_as_uint(d);
                        __hip_atomic_store(xch + (pos * NS + slice) * FD_XW + lane, ((uint64_t)ep << 32) | pay,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                } else if (lane < 8) {
                    __hip_atomic_store(reinterpret_cast<uint32_t*>(hq + pos * I + slice * 32) + lane, word,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (lane == 0)
                        __hip_atomic_store(hd + pos * NS + slice, d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            if constexpr (decltype(multi)::value)
                if (item + G_gu < NI) lds_barrier(); // the next item rewrites s_h
        };
        if (G_gu >= NI) {
            run(g, std::false_type());
            items = 1;
        } else {
            for (int item = g; item < NI; item += G_gu, ++items) run(item, std::true_type());
        }
        if (tagged) return; // the data is its own flag
        __builtin_amdgcn_s_waitcnt(0); // this wave's stores are complete
        __syncthreads();
        if (tid == 0)
            __hip_atomic_fetch_add(&ctl->line[g % FD_NCTR].arrive, items, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    // -------------------------------------------------------------- down role
    fd_sort(P, R);
    const int dg = g - G_gu;
    // the quad walk on the tagged exchange stages h rows padded (fused.h), spreading its LDS reads over the banks
    const bool padded = tagged && Dn::LPR == 16 && R.U <= 8;
    const int RS = padded ? hq_row_padded(NS) : I;                            // bytes per staged h row
    int8_t* s_hq = reinterpret_cast<int8_t*>(fd_dyn);                        // [P][RS]
    float* s_hd = reinterpret_cast<float*>(fd_dyn + (size_t)P * RS);          // [P][I/32]
    float* s_o = s_hd + (size_t)P * NS;                                       // [P][SLOTS]
    const int grp = dg % FD_NCTR;
    uint32_t prev1 = 0;
    // the routing weights (only the combine needs them), while the down weights stream
    auto weights = [&]() {
        fd_weights(T, k, R);
        if (dg == 0)
            for (int p = tid; p < P; p += FD_THREADS) w_out[p] = R.w[p];
    };
    // wait for h and stage it in LDS
    auto receive_h = [&]() {
        if (tagged) {
            // every thread polls its (at most four) words of the exchange until they show this call's epoch,
            // and moves their payload into LDS
            constexpr int M = FD_XCH_WORDS / FD_THREADS;
            const int nw = P * NS * FD_XW;
            uint32_t pend = 0;
#pragma unroll
            for (int m = 0; m < M; ++m)
                if (tid + FD_THREADS * m < nw) pend |= 1u << m;
            uint32_t* s_hq32 = reinterpret_cast<uint32_t*>(s_hq);
            uint32_t it = 0;
            while (pend) {
                uint64_t v[M];
#pragma unroll
                for (int m = 0; m < M; ++m)
                    v[m] = (pend >> m) & 1u ? __hip_atomic_load(xch + tid + FD_THREADS * m, __ATOMIC_RELAXED,
                                                                 __HIP_MEMORY_SCOPE_AGENT)
                                            : 0ull;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    if (((pend >> m) & 1u) && (uint32_t)(v[m] >> 32) == ep) {
                        const int i = tid + FD_THREADS * m, b = i / FD_XW, w = i % FD_XW;
                        if (w >= 8) s_hd[b] = __uint_as_float((uint32_t)v[m]);
                        else if (!padded) s_hq32[b * 8 + w] = (uint32_t)v[m];
                        else { // block blk of row pos at 32 blk + 16 (blk / 4)
                            const int pos = b / NS, blk = b % NS;
                            *reinterpret_cast<uint32_t*>(s_hq + pos * RS + blk * 32 + (blk / 4) * 16 + w * 4) =
                                (uint32_t)v[m];
                        }
                        pend &= ~(1u << m);
                    }
                }
                if (!pend) break;
                if (++it >= FD_SPIN_LIMIT) {
                    __hip_atomic_store(&ctl->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            __syncthreads();
            if (tid == 0)
                prev1 = __hip_atomic_fetch_add(&ctl->line[grp].done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            if (wv == 0) { // wave 0 polls the arrival lines: lane j < FD_NCTR loads line j
                const uint32_t target = (uint32_t)(R.U * NS);
                uint32_t it = 0;
                for (;;) {
                    const uint32_t v =
                        lane < FD_NCTR
                            ? __hip_atomic_load(&ctl->line[lane].arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                            : 0u;
                    uint32_t total = 0;
#pragma unroll
                    for (int j = 0; j < FD_NCTR; ++j) total += (uint32_t)__builtin_amdgcn_readlane((int)v, j);
                    if (total >= target) break;
                    if (++it >= FD_SPIN_LIMIT) {
                        if (lane == 0) __hip_atomic_store(&ctl->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            __syncthreads();
            // departure: every down workgroup is past the wait once all lines are complete
            if (tid == 0)
                prev1 = __hip_atomic_fetch_add(&ctl->line[grp].done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            {
                // rounds of four loads per thread in flight, then their LDS stores (a plain loop would wait
                // for each load before issuing the next)
                const uint64_t* src = reinterpret_cast<const uint64_t*>(hq);
                uint64_t* dst = reinterpret_cast<uint64_t*>(s_hq);
                const int n8 = P * I / 8, nd = P * NS;
                for (int i0 = 0; i0 < n8 || i0 < nd; i0 += 4 * FD_THREADS) {
                    uint64_t v[4];
                    float dv[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int i = i0 + tid + FD_THREADS * m;
                        v[m] = i < n8 ? __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
                        dv[m] = i < nd ? __hip_atomic_load(hd + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.0f;
                    }
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int i = i0 + tid + FD_THREADS * m;
                        if (i < n8) dst[i] = v[m];
                        if (i < nd) s_hd[i] = dv[m];
                    }
                }
            }
            __syncthreads();
        } // counter protocol
    };
    if (Dn::LPR == 16 && R.U <= 8) {
        // at most 8 active experts: one quad of lanes per (output row, expert), a quarter of the row each
        const int qd = tid / 4, li = tid % 4, a = qd % 8, rs = qd / 8; // rs < SLOTS = 16
        const bool live = a < R.U;
        DnQuad<NBR> W;
        weights(); // first, so the down loads do not compete with the gate/up weights arriving now
        if (live) {
            const int64_t row = (int64_t)R.list[a] * H + dg * SLOTS + rs;
            W.issue(down_qs + row * (I / 2), down_d + row * (I / 32), li);
        }
        receive_h();
        if (live) {
            const int beg = R.beg[a], cnt = R.beg[a + 1] - beg;
            for (int c = 0; c < cnt; ++c) {
                const int pos = beg + c;
                const float o = padded ? W.template dot<true>(s_hq + pos * RS, s_hd + pos * NS, li)
                                       : W.dot(s_hq + (int64_t)pos * I, s_hd + pos * NS, li);
                if (li == 0) s_o[R.sorted[pos] * SLOTS + rs] = o;
            }
        }
    } else {
        DnWalk c;
        c.qs = down_qs;
        c.d = down_d;
        c.H = H;
        c.I = I;
        c.list = R.list;
        c.beg = R.beg;
        c.pair = R.sorted;
        const int eg = tid / FD_GROUP; // this thread's expert group walks active experts eg, eg + EGROUPS, ...
        c.U = (R.U - eg + EGROUPS - 1) / EGROUPS;
        c.a_first = eg;
        c.a_step = EGROUPS;
        c.rs = (tid % FD_GROUP) / Dn::LPR;
        c.j = tid % Dn::LPR;
        c.n = dg * SLOTS + c.rs;
        c.slots = SLOTS;
        c.s_o = s_o;
        DnBatch<NBR, DD_CH / Dn::BPL> A, B; // batches of 8 experts (4 at two blocks per lane: registers)
        dn_issue<NBR>(A, c, 0); // the first two batches of down weights stream during the wait
        dn_issue<NBR>(B, c, DnBatch<NBR, DD_CH / Dn::BPL>::N);
        weights();
        receive_h();
        dn_walk<NBR, Dn::BPL == 1 ? 4 : 2>(
            A, B, c,
            [&](int pos, const int8_t*& arow, const float*& adr) {
                arow = s_hq + (int64_t)pos * I;
                adr = s_hd + pos * NS;
            },
            true);
    }
    __syncthreads();
    dn_combine(s_o, SLOTS, T, k, R.w, accumulate, y, H, dg * SLOTS, tid, FD_THREADS);
    if (tid == 0) { // the last departure of the last line resets every counter for the next call
        const uint32_t in_line = (uint32_t)((G_dn - grp + FD_NCTR - 1) / FD_NCTR);
        if (prev1 == in_line - 1) {
            const uint32_t lines = (uint32_t)(G_dn < FD_NCTR ? G_dn : FD_NCTR);
            if (__hip_atomic_fetch_add(&ctl->done2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == lines - 1) {
                for (int j = 0; j < FD_NCTR; ++j) {
                    __hip_atomic_store(&ctl->line[j].arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(&ctl->line[j].done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                __hip_atomic_store(&ctl->done2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                // every workgroup of this call has read the epoch (all have started): the next call takes the next
                __hip_atomic_store(&ctl->epoch, ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// ------------------------------------------------------------------ launcher
int fused_max_tokens() { return FD_MAX_T; }

bool fused_supported(int T, int k, int I) { return T <= FD_MAX_T && (int64_t)T * k * I <= FD_MAX_HQ; }

hipError_t launch_decode_fused(const uint8_t* gate_qs, const uint8_t* up_qs, const uint8_t* down_qs,
                               const uint16_t* gate_d, const uint16_t* up_d, const uint16_t* down_d, int E, int H,
                               int I, const float* x, const float* logits, int T, int k, bool rmsnorm,
                               bool accumulate, int32_t* ids, float* wts, int32_t* offsets, int32_t* sorted,
                               float* y, int8_t* hq, float* hd, void* ctl, hipStream_t s)
{
    if (T == 0 || !fused_supported(T, k, I)) return hipErrorInvalidValue;
    const int P = T * k;
    const int umax = P < E ? P : E;
    const int lpr = (I / 32) < 16 ? (I / 32) : 16;
    const int slots = FD_GROUP / lpr;
    const int G_dn = H / slots;
    const size_t lds_gu = (size_t)T * H + (size_t)T * (H / 32) * 4;
    const bool tagged = (int64_t)P * (I / 32) * FD_XW <= FD_XCH_WORDS;
    const size_t row = tagged ? (size_t)hq_row_padded(I / 32) : (size_t)I; // staged h row (padded: quad walk)
    const size_t lds_dn = (size_t)P * row + (size_t)P * (I / 32) * 4 + (size_t)P * slots * 4;
    const size_t lds = lds_gu > lds_dn ? lds_gu : lds_dn;
    hipError_t err = hipSuccess;
    MOEQ4_FD_BPL(H / 256, MOEQ4_FD_NBR(I / 32, MOEQ4_FD_LPL(E, {
        auto kern = decode_fused_kernel<B, R, LP>;
        if (lds > 64 * 1024) {
            err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (err != hipSuccess) return err;
        }
        // one gate/up workgroup per item, unless that would not leave the whole grid resident at once: then
        // fewer workgroups, each taking several items (the down workgroups' wait needs only that gate/up
        // workgroups have the lower ids, so this is a matter of speed, not of progress)
        int G_gu = (I / 32) * umax;
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kern, FD_THREADS, lds) == hipSuccess) {
            const int room = per_cu * cus - G_dn;
            if (G_gu > room) G_gu = room > I / 32 ? room : I / 32;
        }
        kern<<<dim3((unsigned)(G_gu + G_dn)), FD_THREADS, lds, s>>>(
            gate_qs, up_qs, down_qs, gate_d, up_d, down_d, E, H, I, x, logits, T, k, rmsnorm, accumulate, G_gu, G_dn,
            ids, wts, offsets, sorted, y, hq, hd, reinterpret_cast<FdCtl*>(ctl), tagged);
    })));
    return hipGetLastError();
}

} // namespace moeq4
