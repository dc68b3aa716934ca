// bstack.hip -- one-launch decode of a stack of MoE layers for a batch of up
// to 16 tokens (Dutch technical summary "Methodologie 1" and "Methodologie 2"
// of "A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011 GPU": the
// W4A8 decode over resident 4-bit experts, here layer after layer; "Resultaten"
// names the thin-M GEMM a structural bottleneck, and at these batch sizes each
// expert matrix is a bandwidth-bound matvec over the tokens that chose it).
//
// Each layer computes h_{l+1} = [h_l +] MoE_l(Q8_0([RMSNorm] h_l)) for the T
// tokens with the arithmetic of the three-call decode (rows.h: the same block
// dots, scale products, row reductions, SwiGLU and Q8_0 re-quantisation; the
// combine sums each token's k outputs in slot order), so without the pre-norm
// every hidden state is bit-identical to that chain.  With the pre-norm too:
// the fp64 sum of squares of every layer's input is formed in quantize_act's
// order (threads of 4 values, a wave sum, the waves in order).
//
// Two launches per call:
//   bstack_prep_kernel: one workgroup per layer routes that layer's T tokens
//     (the router's selection and stable counting sort, bit-identical to
//     moe_q4_route) and lists its active experts; ceil(T / 4) more workgroups
//     quantise h_0 into the exchange, four rows each (quantize_act's arithmetic
//     and order).
//   bstack_kernel: persistent; every workgroup resident at once.
//
// Work of layer l, a flat list: gate/up tasks (active expert a, 32 outputs of
// I: 64 weight rows, SwiGLU and one Q8_0 block of h per token of the expert),
// then down tasks (active expert a, DR rows of H: o of each of the expert's
// pairs for those rows), 73.7 KB of weights each at H = 2048, I = 512.  Task q
// goes to worker workgroup q mod GW.  The last T workgroups own one token each
// and keep its row of the residual stream in registers: for every layer they
// gather o of the token's k pairs, form y in slot order and the residual, and
// quantise the token's input to the next layer (the whole row is in the
// workgroup, so the pre-norm needs no exchange).
//
// A worker workgroup is 8 compute waves and two I/O waves.  The vector memory
// counter of a wave retires in issue order and counts stores as well as
// loads: a wave that waits for one load waits for every load it issued
// before and for the acknowledgement of every store.  So the compute waves
// issue nothing but weight loads (two tasks' weights in two register slots,
// the next task's streaming while the current one computes) and read every
// other input from LDS (the routing tables, staged once; the layer's x rows;
// a down task's h rows); the publisher wave issues only the exchange stores
// (a task's results) and never waits for memory; the gatherer wave issues
// only the exchange loads (the next down task's h rows).  Owners issue no
// weight loads at all, so their waits end as soon as the data arrives.
//
// Exchanges between workgroups (different XCDs, L2 caches not coherent with
// each other) are 64-bit words written and read with device-scope atomics: a
// 32-bit payload in the low half and a tag in the high half, so a word that
// shows the expected tag carries this layer's payload (64-bit accesses are
// single-copy atomic) and the data is its own flag: no producer waits for its
// stores to complete.  Tags: the call's base + l for what layer l produces and
// consumes (x of layer 0 from the pre-pass carries base); base follows the
// last tag stored on the workspace, so stale words never match.  Every
// exchange buffer alternates by layer parity; a writer reaches a buffer's next
// use only after every reader of its previous use is done (each layer's x
// needs every down task of the layer before, each down task needs its
// expert's h, which needs that layer's x).
//
// Forward progress: every workgroup is resident at once (the host sizes the
// grid from the occupancy query: one workgroup per CU); a workgroup waits
// only after publishing all it has computed, and gate/up tasks never wait
// within a layer, so no wait is part of a cycle; every wait is bounded and a
// wait that gives up sets the workspace's sticky error word, after which
// every later wait gives up too.
#include <type_traits>

#include "device.h"
#include "rows.h"
#include "topk.h"

namespace moeq4 {

constexpr int BS_MAX_T = 16;
constexpr int BS_MAX_K = 8;
constexpr int BS_MAX_P = BS_MAX_T * BS_MAX_K;
constexpr int BS_MAX_LAYERS = 48;
constexpr int BS_XW = 9;             // words per 32-value block of h: 8 x 4 codes, then the scale
constexpr int BS_MAX_TASKS = 2048;   // tasks of one worker over all layers (the task table in LDS)
constexpr uint32_t BS_SPIN = 1u << 20;
constexpr uint32_t BS_ERR_POLL = 64;
constexpr int BS_PREP_THREADS = 1024;

// Workspace: [0, 4096) control words (error word at byte 2112, the last tag
// used at byte 2176, a departure counter at 2240), then per layer 4 KB of
// routing (BsMeta), then the exchanges.
struct BsCtl {
    uint32_t pad0[528];
    uint32_t error; // byte 2112
    uint32_t pad1[15];
    uint32_t epoch; // byte 2176
    uint32_t pad2[15];
    uint32_t done;  // byte 2240
};
static_assert(offsetof(BsCtl, error) == 2112 && offsetof(BsCtl, epoch) == 2176, "control word offsets");

struct BsMeta {
    int32_t ids[BS_MAX_P];    // [T][k] chosen experts, slot order
    float w[BS_MAX_P];        // [T][k] renormalised weights
    int32_t sorted[BS_MAX_P]; // pair at each sorted position
    int32_t list[BS_MAX_P];   // active experts, ascending
    int32_t beg[BS_MAX_P + 1];// first sorted position of each active expert; beg[U] = P
    int32_t order[BS_MAX_P];  // active experts by falling token count (ties: ascending), as indexes into list
    int32_t U;
};
static_assert(sizeof(BsMeta) <= 4096, "one layer's routing in 4 KB");

constexpr size_t BS_META_OFFSET = 4096;
__host__ __device__ constexpr size_t bs_align(size_t v) { return (v + 255) & ~(size_t)255; }

struct BsLayout { // byte offsets of the exchanges (all 64-bit words, two buffers each by layer parity)
    size_t xx, xh, xo, total;
    int xx_words, xh_words, xo_words; // words per buffer
};

__host__ __device__ inline BsLayout bs_layout(int L, int T, int k, int H, int I)
{
    BsLayout s;
    const int P = T * k;
    s.xx_words = T * (H / 4 + H / 32);                 // x of a layer: [T][H/4 code words + H/32 scales]
    s.xh_words = P * (I / 32) * BS_XW;                 // h: [sorted position][slice][9]
    s.xo_words = P * H;                                // o: [pair][H]
    s.xx = BS_META_OFFSET + (size_t)L * 4096;
    s.xh = s.xx + bs_align((size_t)2 * s.xx_words * 8);
    s.xo = s.xh + bs_align((size_t)2 * s.xh_words * 8);
    s.total = s.xo + bs_align((size_t)2 * s.xo_words * 8);
    return s;
}

struct BsLayers { // device pointers of every layer's experts, passed by value
    const uint8_t* gq[BS_MAX_LAYERS];
    const uint8_t* uq[BS_MAX_LAYERS];
    const uint8_t* dq[BS_MAX_LAYERS];
    const uint16_t* gd[BS_MAX_LAYERS];
    const uint16_t* ud[BS_MAX_LAYERS];
    const uint16_t* dd[BS_MAX_LAYERS];
};

__device__ __forceinline__ uint32_t bs_base(const BsCtl* ctl, int L)
{
    const uint32_t ep = __hip_atomic_load(&ctl->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return ep > 0xFFFFFFFEu - (uint32_t)(L + 1) ? 1u : ep + 1u;
}

__device__ __forceinline__ void bs_put(uint64_t* p, uint32_t tag, uint32_t pay)
{
    __hip_atomic_store(p, ((uint64_t)tag << 32) | pay, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll this thread's words src[idx[m]] (m < M, live where bit m of `live` is set) until each shows `tag`;
// payloads to val[m].  Bounded: gives up after BS_SPIN polls, or once another wait of the launch has.
template <int M, int SLEEP>
__device__ __forceinline__ void bs_poll(const uint64_t* src, const int (&idx)[M], uint32_t live, uint32_t tag,
                                        uint32_t (&val)[M], BsCtl* ctl)
{
    uint32_t pend = live;
#pragma unroll
    for (int m = 0; m < M; ++m) val[m] = 0u;
    uint32_t it = 0;
    while (pend) {
        uint64_t v[M];
#pragma unroll
        for (int m = 0; m < M; ++m)
            v[m] = (pend >> m) & 1u ? __hip_atomic_load(src + idx[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                    : 0ull;
#pragma unroll
        for (int m = 0; m < M; ++m)
            if (((pend >> m) & 1u) && (uint32_t)(v[m] >> 32) == tag) {
                val[m] = (uint32_t)v[m];
                pend &= ~(1u << m);
            }
        if (!pend) break;
        if (++it % BS_ERR_POLL == 0) {
            if (it >= BS_SPIN) {
                __hip_atomic_store(&ctl->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            if (__hip_atomic_load(&ctl->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
        }
        __builtin_amdgcn_s_sleep(SLEEP);
    }
}

// Pairs of exchange words in one 16-byte access: buffer loads and stores with the sc1 cache bit, the level at
// which the device-scope atomics above are coherent (a volatile access would give the same bits but be followed
// by a wait for its completion, which would serialise a round of polls).  Each 8-byte half is written and read
// whole, and its tag decides for it alone.  base is wave-uniform; offsets are below 2 GB.
typedef unsigned bs_v4u32 __attribute__((ext_vector_type(4)));
constexpr int BS_SC1 = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t bs_rsrc(const uint64_t* base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint64_t*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}

// words p[0] = (tag, a) and p[1] = (tag, b) of the buffer at r, p = base + w (w even)
__device__ __forceinline__ void bs_put2(__amdgpu_buffer_rsrc_t r, int w, uint32_t tag, uint32_t a, uint32_t b)
{
    __builtin_amdgcn_raw_buffer_store_b128(bs_v4u32{a, tag, b, tag}, r, w * 8, 0, BS_SC1);
}

// bs_poll over pairs of words: src[idx[m]] and src[idx[m] + 1] (idx[m] even) in one 16-byte load, half the
// requests of two 8-byte ones

template <int M, int SLEEP>
__device__ __forceinline__ void bs_poll2(const uint64_t* src, const int (&idx)[M], uint32_t live, uint32_t tag,
                                         uint32_t (&val)[M][2], BsCtl* ctl)
{
    static_assert(M <= 16, "two pending bits per pair in 32 bits");
    uint32_t pend = 0; // bit 2m + h: half h of pair m still expected
#pragma unroll
    for (int m = 0; m < M; ++m) {
        if ((live >> m) & 1u) pend |= 3u << (2 * m);
        val[m][0] = val[m][1] = 0u;
    }
    const __amdgpu_buffer_rsrc_t r = bs_rsrc(src);
    uint32_t it = 0;
    while (pend) {
        bs_v4u32 v[M]; // payload, tag, payload, tag
#pragma unroll
        for (int m = 0; m < M; ++m)
            v[m] = (pend >> (2 * m)) & 3u ? __builtin_amdgcn_raw_buffer_load_b128(r, idx[m] * 8, 0, BS_SC1)
                                          : bs_v4u32{0u, 0u, 0u, 0u};
#pragma unroll
        for (int m = 0; m < M; ++m) {
            if (((pend >> (2 * m)) & 1u) && v[m].y == tag) {
                val[m][0] = v[m].x;
                pend &= ~(1u << (2 * m));
            }
            if (((pend >> (2 * m + 1)) & 1u) && v[m].w == tag) {
                val[m][1] = v[m].z;
                pend &= ~(2u << (2 * m));
            }
        }
        if (!pend) break;
        if (++it % BS_ERR_POLL == 0) {
            if (it >= BS_SPIN) {
                __hip_atomic_store(&ctl->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            if (__hip_atomic_load(&ctl->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
        }
        __builtin_amdgcn_s_sleep(SLEEP);
    }
}

// ------------------------------------------------------------------ pre-pass: routing of every layer, x of layer 0
template <int LPL>
__global__ __launch_bounds__(BS_PREP_THREADS) void bstack_prep_kernel(const float* __restrict__ logits, int L, int T,
                                                                      int E, int k, const float* __restrict__ h0,
                                                                      int H, bool rmsnorm, BsMeta* __restrict__ meta,
                                                                      uint64_t* __restrict__ xx, BsCtl* ctl)
{
    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    if ((int)blockIdx.x < L) {
        // ---- routing of layer l: the router's selection (one wave per token) and its stable counting sort
        constexpr int EPT = 1024 / BS_PREP_THREADS;
        __shared__ uint32_t s_mask[1024]; // bit t: token t chose expert e (T <= 16)
        __shared__ int s_ids[BS_MAX_P];
        __shared__ int s_off[1024];
        __shared__ int s_wave[BS_PREP_THREADS / WAVE];
        __shared__ int s_cnt[BS_PREP_THREADS / WAVE];
        __shared__ int s_lbeg[BS_MAX_P + 1];
        const int l = blockIdx.x;
        BsMeta& M = meta[l];
        for (int e = tid; e < E; e += BS_PREP_THREADS) s_mask[e] = 0u;
        __syncthreads();
        if (wv < T) {
            int id;
            float w;
            select_topk<LPL>(logits + ((int64_t)l * T + wv) * E, E, k, lane, id, w);
            if (lane < k) {
                M.ids[wv * k + lane] = id;
                M.w[wv * k + lane] = w;
                s_ids[wv * k + lane] = id;
                atomicOr(&s_mask[id], 1u << wv);
            }
        }
        __syncthreads();
        // per-expert counts, their exclusive scan (offsets) and the active-expert ranks
        int c[EPT], act[EPT], local = 0, alocal = 0;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = EPT * tid + i;
            c[i] = e < E ? __popc(s_mask[e]) : 0;
            act[i] = c[i] > 0;
            local += c[i];
            alocal += act[i];
        }
        int inc = local, ainc = alocal;
#pragma unroll
        for (int d = 1; d < WAVE; d <<= 1) {
            const int o = __shfl_up(inc, d, WAVE), ao = __shfl_up(ainc, d, WAVE);
            if (lane >= d) {
                inc += o;
                ainc += ao;
            }
        }
        if (lane == WAVE - 1) {
            s_wave[wv] = inc;
            s_cnt[wv] = ainc;
        }
        __syncthreads();
        int run = inc - local, arun = ainc - alocal, utot = 0;
        for (int w8 = 0; w8 < BS_PREP_THREADS / WAVE; ++w8) {
            if (w8 < wv) {
                run += s_wave[w8];
                arun += s_cnt[w8];
            }
            utot += s_cnt[w8];
        }
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = EPT * tid + i;
            if (e < E) {
                s_off[e] = run;
                if (act[i]) {
                    M.list[arun] = e;
                    M.beg[arun] = run;
                    s_lbeg[arun] = run;
                    ++arun;
                }
            }
            run += c[i];
        }
        const int P = T * k;
        if (tid == 0) {
            M.U = utot;
            M.beg[utot] = P;
            s_lbeg[utot] = P;
        }
        __syncthreads();
        // the order in which the workers' task lists take the active experts: by falling token count, so that
        // the dealing below spreads equal costs evenly
        for (int a = tid; a < utot; a += BS_PREP_THREADS) {
            const int ca = s_lbeg[a + 1] - s_lbeg[a];
            int r = 0;
            for (int b = 0; b < utot; ++b) {
                const int cb = s_lbeg[b + 1] - s_lbeg[b];
                r += cb > ca || (cb == ca && b < a);
            }
            M.order[r] = a;
        }
        for (int p = tid; p < P; p += BS_PREP_THREADS) {
            const int t = p / k, e = s_ids[p];
            M.sorted[s_off[e] + __popc(s_mask[e] & ((1u << t) - 1u))] = p;
        }
        return;
    }
    // ---- x of layer 0, rows 4 (g - L) .. 4 (g - L) + 3: quantize_act's arithmetic, a row of H in a 256-thread
    // group (its order of the fp64 sums)
    __shared__ double s_part[BS_PREP_THREADS / WAVE];
    const uint32_t tag = bs_base(ctl, L);
    const int grp = tid / 256, gt = tid % 256; // 4 rows at a time
    const int n4 = H / 4;
    const int F = (n4 + 255) / 256;            // float4 per thread (<= 2 at H <= 2048)
    {
        const int t0 = 4 * ((int)blockIdx.x - L);
        const int t = t0 + grp;
        const bool row = t < T;
        float4 v[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const int i = gt + 256 * f;
            v[f] = (row && f < F && i < n4) ? reinterpret_cast<const float4*>(h0 + (int64_t)t * H)[i]
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (rmsnorm) {
            double ss = 0.0;
#pragma unroll
            for (int f = 0; f < 2; ++f)
                ss += (double)v[f].x * v[f].x + (double)v[f].y * v[f].y + (double)v[f].z * v[f].z +
                      (double)v[f].w * v[f].w;
            ss = sum_wave_f64(ss);
            if (lane == 0) s_part[wv] = ss;
            __syncthreads();
            double tot = 0.0;
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) tot += s_part[grp * 4 + w4];
            const double inv = 1.0 / sqrt(tot / (double)H + 1e-6);
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                v[f].x = (float)((double)v[f].x * inv);
                v[f].y = (float)((double)v[f].y * inv);
                v[f].z = (float)((double)v[f].z * inv);
                v[f].w = (float)((double)v[f].w * inv);
            }
            __syncthreads();
        }
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const int i = gt + 256 * f;
            const float amax = max_group<8>(fmaxf(fmaxf(fabsf(v[f].x), fabsf(v[f].y)), fmaxf(fabsf(v[f].z), fabsf(v[f].w))));
            const float d = amax / 127.0f;
            if (row && f < F && i < n4) {
                const uint32_t q0 = (uint32_t)(q8_code(v[f].x, d) & 0xFF), q1 = (uint32_t)(q8_code(v[f].y, d) & 0xFF);
                const uint32_t q2 = (uint32_t)(q8_code(v[f].z, d) & 0xFF), q3 = (uint32_t)(q8_code(v[f].w, d) & 0xFF);
                uint64_t* xr = xx + (int64_t)t * (H / 4 + H / 32);
                bs_put(xr + i, tag, q0 | (q1 << 8) | (q2 << 16) | (q3 << 24));
                if ((i & 7) == 0) bs_put(xr + H / 4 + i / 8, tag, __float_as_uint(d));
            }
        }
    }
}

// ------------------------------------------------------------------ the persistent kernel
constexpr int BS_CW = 8;                  // compute waves of a worker workgroup
constexpr int BS_CT = BS_CW * WAVE;       // their threads: the row walks' lane mappings
constexpr int BS_PW = BS_CW;              // the publisher wave
constexpr int BS_GW = BS_CW + 1;          // the gatherer wave
constexpr int BS_BLOCK = BS_CT + 2 * WAVE;
constexpr uint32_t BS_OWNER_SLEEP = 2;    // owners poll more slowly (they wait most of a layer)

// One task's weights in registers: 8 x 16 bytes of nibbles and 8 fp16 scales (zero-extended) per lane, 16
// load instructions whatever the task, so that the compiler's wait before a task's registers covers its own
// loads only (later tasks' loads are issued after them and retire after them).
typedef unsigned bs_v4u __attribute__((ext_vector_type(4)));
struct BsSlot {
    bs_v4u q[8]; // one register tuple each, kept whole
    uint32_t s[8];
};

template <int BPL, int NBR>
struct BsShape {
    using Dn = DnRow<NBR>;
    static constexpr int LPR = Dn::LPR, BPLD = Dn::BPL;
    static constexpr int GROUPS = BS_CT / LPR;
    static constexpr int RPL = 8 / BPLD;             // down rows per lane group
    static constexpr int DR = GROUPS * RPL;          // rows of H per down task
    static constexpr int HMAX = 256 * BPL, IMAX = 32 * NBR;
    static_assert(RPL * BPLD == 8 && BPL <= 8, "8 nibble pieces per lane and task");
    // dynamic LDS of a workgroup (bytes)
    static constexpr size_t META = BS_MAX_LAYERS * (2 + 2 * BS_MAX_P + (BS_MAX_P + 1) + 2 * BS_MAX_P);
    static constexpr size_t O_META = 0;
    static constexpr size_t O_XQ = (META + 15) & ~(size_t)15;                      // x rows [T][H] int8
    static constexpr size_t O_XD = O_XQ + (size_t)BS_MAX_T * HMAX;                 // [T][H/32] fp32
    static constexpr size_t O_XC = O_XD + (size_t)BS_MAX_T * (HMAX / 32) * 4;      // [T][H/32] int32
    static constexpr size_t O_HQ = O_XC + (size_t)BS_MAX_T * (HMAX / 32) * 4;      // 2 x [T][I] int8
    static constexpr size_t O_HD = O_HQ + (size_t)2 * BS_MAX_T * IMAX;             // 2 x [T][I/32] fp32
    static constexpr size_t O_SH = O_HD + (size_t)2 * BS_MAX_T * (IMAX / 32) * 4;  // 2 x [T][64] fp32
    static constexpr size_t O_SO = O_SH + (size_t)2 * BS_MAX_T * 64 * 4;           // 2 x [T][DR] fp32
    static constexpr size_t O_SS = O_SO + (size_t)2 * BS_MAX_T * DR * 4;           // 4 fp64 wave sums (owners)
    static constexpr size_t O_TASK = O_SS + 4 * 8;                                  // [BS_MAX_TASKS] task words
    static constexpr size_t O_CUM = O_TASK + (size_t)BS_MAX_TASKS * 4;              // [L + 1] task counts
    static constexpr size_t BYTES = O_CUM + (size_t)(BS_MAX_LAYERS + 1) * 4;
    // the 8 pieces of a task's weights: piece i's byte offset from the lane's first piece (gate/up: the lane's
    // row, blocks j, j + 8, ...; down: DnRow's walk over rows gid + GROUPS r) and its scale's element offset
    static constexpr int H = 256 * BPL, I = 32 * NBR;
    __device__ static constexpr int gu_q(int i) { return (i < BPL ? i : 0) * 128; }
    __device__ static constexpr int gu_d(int i) { return (i < BPL ? i : 0) * 8; }
    __device__ static constexpr int dn_q(int i) { return (i / BPLD) * GROUPS * (I / 2) + (i % BPLD) * LPR * 16; }
    __device__ static constexpr int dn_d(int i) { return (i / BPLD) * GROUPS * (I / 32) + (i % BPLD) * LPR; }
};

// Nibbles with fewer operations than unpack_block16: the low nibbles as they are (q, 0..15), the high ones as
// 16 (q - 8) (the high nibble field with its top bit flipped, read as a signed int8), one operation per dword each.  Then 16 isum = 16 sum_lo q a - 128 sum_lo a + sum_hi 16 (q - 8) a:
// the dot of the low half is shifted by 4 and the block's -128 sum_lo a (its activation codes 0..15, the same for
// every weight row) starts the high half's chain.  The integers are those of block_dot16, so every result is.
struct BsBlk {
    uint32_t lo[4], hi[4];
};

__device__ __forceinline__ BsBlk bs_unpack(const bs_v4u w)
{
    BsBlk b;
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        b.lo[i] = v[i] & 0x0F0F0F0Fu;
        b.hi[i] = (v[i] & 0xF0F0F0F0u) ^ 0x80808080u;
    }
    return b;
}

// 16 isum of one block with activations a0 (codes 0..15), a1 (16..31) and c = -128 sum(a0)
__device__ __forceinline__ int bs_dot16(const BsBlk& b, const int4 a0, const int4 a1, int c)
{
    int lo = __builtin_amdgcn_sdot4((int)b.lo[0], a0.x, 0, false);
    lo = __builtin_amdgcn_sdot4((int)b.lo[1], a0.y, lo, false);
    lo = __builtin_amdgcn_sdot4((int)b.lo[2], a0.z, lo, false);
    lo = __builtin_amdgcn_sdot4((int)b.lo[3], a0.w, lo, false);
    int hi = __builtin_amdgcn_sdot4((int)b.hi[0], a1.x, c, false);
    hi = __builtin_amdgcn_sdot4((int)b.hi[1], a1.y, hi, false);
    hi = __builtin_amdgcn_sdot4((int)b.hi[2], a1.z, hi, false);
    hi = __builtin_amdgcn_sdot4((int)b.hi[3], a1.w, hi, false);
    return (lo << 4) + hi;
}

// -128 x the sum of an activation block's codes 0..15
__device__ __forceinline__ int bs_corr(const int4 a0)
{
    int s = __builtin_amdgcn_sdot4(a0.x, 0x01010101, 0, false);
    s = __builtin_amdgcn_sdot4(a0.y, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4(a0.z, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4(a0.w, 0x01010101, s, false);
    return -128 * s;
}

// The gate/up row of one token from a slot: GuRow::partial's arithmetic (blocks j, j + 8, ... in order, one fmaf
// each with d_w / 16 times d_a) on bs_dot16's block sums.  x row: codes xq, scales xd, corrections xc.
template <int BPL>
__device__ __forceinline__ float bs_gu_row(BsSlot& S, const float (&dw)[BPL], const int8_t* __restrict__ xq,
                                           const float* __restrict__ xd, const int* __restrict__ xc, int j)
{
#pragma unroll
    for (int i = 0; i < BPL; ++i) // opaque: the blocks are unpacked again for each token, not kept unpacked
        asm volatile("" : "+v"(S.q[i]));
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
        const int b = j + 8 * i;
        const int4* ap = reinterpret_cast<const int4*>(xq + b * 32);
        part = fmaf((float)bs_dot16(bs_unpack(S.q[i]), ap[0], ap[1], xc[b]), dw[i] * xd[b], part);
        __builtin_amdgcn_sched_barrier(0); // one block at a time (registers)
    }
    return part;
}

// A worker's task n (its n-th over all layers) and its word from the task table: expert id (bits 0-9), index in the
// layer's active list (10-16), slice of I or row chunk of H (17-21), layer (22-27), gate/up (28), a down task whose
// inputs allow the overlapped gather (29), the first task of its layer (30).  d = 0 with n = N: no task.
struct BsTask {
    int n;
    uint32_t d;
    __device__ int e() const { return (int)(d & 1023u); }
    __device__ int a() const { return (int)((d >> 10) & 127u); }
    __device__ int sub() const { return (int)((d >> 17) & 31u); }
    __device__ int l() const { return (int)((d >> 22) & 63u); }
    __device__ bool gu() const { return (d >> 28) & 1u; }
    __device__ bool safe() const { return (d >> 29) & 1u; }
    __device__ bool first() const { return (d >> 30) & 1u; }
};

// The weight loads are buffer loads: a wave-uniform descriptor, a lane offset (one register for all of a task's
// pieces) and a uniform piece offset in a scalar register, so no 64-bit address is formed per lane.
// Cache policy of the weight loads: the default one.  Measured against the non-temporal hint (2), sc0 (1), sc0 + nt
// (3), sc1 (16) and sc0 + sc1 (17) at batch 16, it was the fastest by about 1.7% over the non-temporal hint.
constexpr int BS_WPOL = 0;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bs_wrsrc(const void* base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}

__device__ __forceinline__ bs_v4u bs_ld16o(__amdgpu_buffer_rsrc_t r, uint32_t off, int piece)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, piece, BS_WPOL);
}

__device__ __forceinline__ uint32_t bs_ld4o(__amdgpu_buffer_rsrc_t r, uint32_t off, int piece)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, piece, BS_WPOL);
}

// A wave-uniform pointer as a scalar value (its two halves through readfirstlane).
template <typename P>
__device__ __forceinline__ P* bs_scalar(P* p)
{
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return reinterpret_cast<P*>(((uint64_t)hi << 32) | lo);
}

// v made opaque to the optimiser: index arithmetic on it is redone where it is used instead of being hoisted
// out of the task loop into registers of its own, which the loop's two weight slots cannot spare
__device__ __forceinline__ int bs_opaque(int v)
{
    asm volatile("" : "+v"(v));
    return v;
}

template <int BPL, int NBR>
__global__ __launch_bounds__(BS_BLOCK) void bstack_kernel(
    const BsLayers lp, int L, int T, int k, int H, int I, bool rmsnorm, bool accumulate, float* __restrict__ h,
    float* __restrict__ h_all, int8_t* __restrict__ hq_all, float* __restrict__ hd_all,
    const BsMeta* __restrict__ meta, uint64_t* __restrict__ xxb, uint64_t* __restrict__ xhb,
    uint64_t* __restrict__ xob, int xx_words, int xh_words, int xo_words,
    BsCtl* __restrict__ ctl)
{
    using Sh = BsShape<BPL, NBR>;
    using Dn = DnRow<NBR>;
    constexpr int LPR = Sh::LPR, BPLD = Sh::BPLD, GROUPS = Sh::GROUPS, RPL = Sh::RPL, DR = Sh::DR;
    constexpr int HMAX = Sh::HMAX, IMAX = Sh::IMAX;
    extern __shared__ __align__(16) uint8_t bs_lds[];
    int16_t* mU = reinterpret_cast<int16_t*>(bs_lds + Sh::O_META);                   // [L]
    int16_t* mlist = mU + BS_MAX_LAYERS;                                              // [L][P]
    uint8_t* mbeg = reinterpret_cast<uint8_t*>(mlist + BS_MAX_LAYERS * BS_MAX_P);     // [L][P+1]
    uint8_t* msorted = mbeg + BS_MAX_LAYERS * (BS_MAX_P + 1);                         // [L][P]
    uint8_t* morder = msorted + BS_MAX_LAYERS * BS_MAX_P;                             // [L][P]
    int8_t(*s_xq)[HMAX] = reinterpret_cast<int8_t(*)[HMAX]>(bs_lds + Sh::O_XQ);
    float(*s_xd)[HMAX / 32] = reinterpret_cast<float(*)[HMAX / 32]>(bs_lds + Sh::O_XD);
    int(*s_xc)[HMAX / 32] = reinterpret_cast<int(*)[HMAX / 32]>(bs_lds + Sh::O_XC); // -128 sum of codes 0..15
    int8_t(*s_hq)[BS_MAX_T][IMAX] = reinterpret_cast<int8_t(*)[BS_MAX_T][IMAX]>(bs_lds + Sh::O_HQ);
    float(*s_hd)[BS_MAX_T][IMAX / 32] = reinterpret_cast<float(*)[BS_MAX_T][IMAX / 32]>(bs_lds + Sh::O_HD);
    float(*s_gu)[BS_MAX_T][64] = reinterpret_cast<float(*)[BS_MAX_T][64]>(bs_lds + Sh::O_SH); // gate 0-31, up 32-63
    float(*s_o)[BS_MAX_T][DR] = reinterpret_cast<float(*)[BS_MAX_T][DR]>(bs_lds + Sh::O_SO);

    const int tid = threadIdx.x, wv = tid / WAVE;
    const int g = blockIdx.x, G = gridDim.x;
    const int NS = I / 32, ND = H / DR;
    const int GW = G - T; // worker workgroups; the last T own one token each
    const int P = T * k;
    const uint32_t base = bs_base(ctl, L);

    if (g >= GW) {
        // ============================================================ owner of token ot
        // thread tid < H / 4: rows 4 tid .. 4 tid + 3 of the token; it keeps them of the residual stream in
        // registers
        const int ot = g - GW, orow = 4 * tid;
        const bool olive = tid < H / 4;
        float4* s_y = reinterpret_cast<float4*>(bs_lds + Sh::O_XQ); // [H / 4] the token's y (pre-norm only)
        double* s_part = reinterpret_cast<double*>(bs_lds + Sh::O_SS);
        float resid[4] = {0.f, 0.f, 0.f, 0.f};
        if (olive) {
            const float4 v = *reinterpret_cast<const float4*>(h + (int64_t)ot * H + orow);
            resid[0] = v.x;
            resid[1] = v.y;
            resid[2] = v.z;
            resid[3] = v.w;
        }
        for (int l = 0; l < L; ++l) {
            const uint32_t tag = base + (uint32_t)l;
            float wt[BS_MAX_K];
#pragma unroll
            for (int j = 0; j < BS_MAX_K; ++j) wt[j] = olive && j < k ? meta[l].w[ot * k + j] : 0.0f;
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
            if (olive) {
                const uint64_t* src = xob + (size_t)(l & 1) * xo_words;
                // o of the token's k pairs for the thread's 4 rows in one round of polls (two rows per 16-byte
                // load), then the sums in slot order
                int idx[2 * BS_MAX_K];
                uint32_t live = 0, val[2 * BS_MAX_K][2];
#pragma unroll
                for (int m = 0; m < 2 * BS_MAX_K; ++m) {
                    const int jj = m / 2;
                    idx[m] = (ot * k + (jj < k ? jj : 0)) * H + orow + 2 * (m % 2);
                    if (jj < k) live |= 1u << m;
                }
                bs_poll2<2 * BS_MAX_K, BS_OWNER_SLEEP>(src, idx, live, tag, val, ctl);
#pragma unroll
                for (int m = 0; m < 2 * BS_MAX_K; ++m) { // fixed slot order per row: 0, 1, ...
                    const int jj = m / 2;
                    if (jj < k) {
                        acc[2 * (m % 2)] = fmaf(wt[jj], __uint_as_float(val[m][0]), acc[2 * (m % 2)]);
                        acc[2 * (m % 2) + 1] = fmaf(wt[jj], __uint_as_float(val[m][1]), acc[2 * (m % 2) + 1]);
                    }
                }
            }
            float y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = accumulate ? resid[i] + acc[i] : acc[i];
            if (olive) {
#pragma unroll
                for (int i = 0; i < 4; ++i) resid[i] = y[i];
                if (h_all)
                    *reinterpret_cast<float4*>(h_all + ((int64_t)l * T + ot) * H + orow) = make_float4(y[0], y[1], y[2], y[3]);
                if (l == L - 1) *reinterpret_cast<float4*>(h + (int64_t)ot * H + orow) = make_float4(y[0], y[1], y[2], y[3]);
            }
            if (l == L - 1) break;
            const uint32_t ntag = tag + 1u;
            double inv = 1.0;
            if (rmsnorm) {
                // quantize_act's fp64 sum of squares in its order: thread i < 256 of the row takes float4s i and
                // i + 256 in turn, then a wave sum, then the four waves in order
                if (olive) s_y[tid] = make_float4(y[0], y[1], y[2], y[3]);
                lds_barrier();
                if (tid < 256) {
                    double ss = 0.0;
#pragma unroll
                    for (int f = 0; f < 2; ++f) {
                        const int i = tid + 256 * f;
                        const float4 v = i < H / 4 ? s_y[i] : make_float4(0.f, 0.f, 0.f, 0.f);
                        ss += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
                    }
                    ss = sum_wave_f64(ss);
                    if (tid % WAVE == 0) s_part[tid / WAVE] = ss;
                }
                lds_barrier();
                double tot = 0.0;
#pragma unroll
                for (int w = 0; w < 4; ++w) tot += s_part[w];
                inv = 1.0 / sqrt(tot / (double)H + 1e-6); // (s_y and s_part are next written after the next
                                                            // layer's poll, past this layer's second barrier)
            }
            // the owner's rows of x for layer l + 1: 8 threads hold one 32-row block
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = rmsnorm ? (float)((double)y[i] * inv) : y[i];
            const float amax = max_group<8>(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
            const float d = amax / 127.0f;
            if (olive) {
                uint64_t* xr = xxb + (size_t)((l + 1) & 1) * xx_words + (size_t)ot * (H / 4 + H / 32);
                const uint32_t q0 = (uint32_t)(q8_code(v[0], d) & 0xFF), q1 = (uint32_t)(q8_code(v[1], d) & 0xFF);
                const uint32_t q2 = (uint32_t)(q8_code(v[2], d) & 0xFF), q3 = (uint32_t)(q8_code(v[3], d) & 0xFF);
                bs_put(xr + orow / 4, ntag, q0 | (q1 << 8) | (q2 << 16) | (q3 << 24));
                if ((tid % 8) == 0) bs_put(xr + H / 4 + orow / 32, ntag, __float_as_uint(d));
            }
        }
    } else {
        // ============================================================ worker
        // every layer's routing into LDS (read-only from here on): the layers' U first, then their arrays, whose
        // loads do not wait on one another (entries past U are read and dropped), so that they are in flight together
        for (int l = tid; l < L; l += BS_BLOCK) mU[l] = (int16_t)meta[l].U;
        __syncthreads();
        {
            constexpr int MI = (BS_MAX_LAYERS * (BS_MAX_P + 1) + BS_BLOCK - 1) / BS_BLOCK;
            int vl[MI], vb[MI], vs[MI], vo[MI];
#pragma unroll
            for (int m = 0; m < MI; ++m) {
                const int i = tid + BS_BLOCK * m;
                const int l = i / (BS_MAX_P + 1), a = i % (BS_MAX_P + 1), ac = a < BS_MAX_P ? a : BS_MAX_P - 1;
                if (l < L) {
                    const BsMeta& M = meta[l];
                    vl[m] = M.list[ac];
                    vb[m] = M.beg[a];
                    vs[m] = M.sorted[ac];
                    vo[m] = M.order[ac];
                }
            }
#pragma unroll
            for (int m = 0; m < MI; ++m) {
                const int i = tid + BS_BLOCK * m;
                const int l = i / (BS_MAX_P + 1), a = i % (BS_MAX_P + 1);
                if (l < L) {
                    const int U = mU[l];
                    if (a < U) mlist[l * BS_MAX_P + a] = (int16_t)vl[m];
                    if (a <= U) mbeg[l * (BS_MAX_P + 1) + a] = (uint8_t)vb[m];
                    if (a < P) msorted[l * BS_MAX_P + a] = (uint8_t)vs[m];
                    if (a < U) morder[l * BS_MAX_P + a] = (uint8_t)vo[m];
                }
            }
        }
        __syncthreads();
        // Task lists.  Layer l's gate/up tasks are positions q = r NS + slice, its down tasks positions
        // U NS + r ND + chunk, where r ranks the active experts by falling token count (morder); each kind is
        // dealt to the workers round by round in alternating directions (round m goes to workers 0 .. GW - 1 for
        // even m, GW - 1 .. 0 for odd m), so equal costs are spread evenly and the heaviest experts come first.
        auto deal = [&](int m) { return (m & 1) ? GW - 1 - g : g; }; // this workgroup's position in round m
        auto rounds = [&](int n) { // how many of the positions 0 .. n - 1 are this workgroup's
            const int F = n / GW;
            return F + (deal(F) < n - F * GW ? 1 : 0);
        };
        auto nloc = [&](int l) { const int U = mU[l]; return rounds(U * NS) + rounds(U * ND); };
        // the active expert (index into the layer's list) of a gate/up or down position
        auto expert_of = [&](int l, int r) { return (int)morder[l * BS_MAX_P + r]; };
        // The task table: the worker's tasks in order, layer after layer (its gate/up tasks of a layer, then its
        // down tasks), one word each, built once so that a step reads one word instead of a chain of lookups.
        uint32_t* s_task = reinterpret_cast<uint32_t*>(bs_lds + Sh::O_TASK);
        int* s_cum = reinterpret_cast<int*>(bs_lds + Sh::O_CUM);
        if (tid < L) s_cum[tid + 1] = nloc(tid); // each layer's count, then their running sum (one wave)
        __syncthreads();
        if (tid < WAVE) {
            int c = 0;
            for (int l0 = 0; l0 < L; l0 += WAVE) {
                const int l = l0 + tid;
                int v = l < L ? s_cum[l + 1] : 0;
#pragma unroll
                for (int d = 1; d < WAVE; d <<= 1) {
                    const int o = __shfl_up(v, d, WAVE);
                    if (tid >= d) v += o;
                }
                if (l < L) s_cum[l + 1] = c + v;
                c += __shfl(v, WAVE - 1, WAVE);
            }
            if (tid == 0) s_cum[0] = 0;
        }
        __syncthreads();
        const int N = s_cum[L]; // tasks of this workgroup (the host bounds it by BS_MAX_TASKS)
        for (int n = tid; n < N; n += BS_BLOCK) {
            int l = 0;
            while (s_cum[l + 1] <= n) ++l;
            const int i = n - s_cum[l];
            const int nG = (int)mU[l] * NS, cg = rounds(nG);
            const bool gu = i < cg;
            const int m = gu ? i : i - cg, q = m * GW + deal(m); // position among the layer's tasks of its kind
            const int r = gu ? q / NS : q / ND, sub = gu ? q % NS : q % ND;
            const int a = expert_of(l, r), e = mlist[l * BS_MAX_P + a];
            // a down task's gather may overlap the gate/up task before it when every gate/up slice of its expert
            // lies in the dealing's rounds 0 .. F - 2 (F = nG / GW, the rounds every worker has in full): each of
            // those is followed, on its worker, by another gate/up task, which never waits, so it is published
            // within one step whatever any gatherer waits for
            const int F = nG / GW;
            const bool safe = !gu && F >= 2 && r * NS + NS - 1 < (F - 1) * GW;
            s_task[n] = (uint32_t)e | ((uint32_t)a << 10) | ((uint32_t)sub << 17) | ((uint32_t)l << 22) |
                        ((uint32_t)gu << 28) | ((uint32_t)safe << 29) | ((uint32_t)(i == 0) << 30);
        }
        __syncthreads();
        auto task = [&](int n) { // uniform: the word travels in a scalar register
            return n < N ? BsTask{n, (uint32_t)__builtin_amdgcn_readfirstlane((int)s_task[n])} : BsTask{N, 0u};
        };
        auto next_of = [&](BsTask t) { return task(t.n < N ? t.n + 1 : N); };
        auto is_gu = [&](BsTask t) { return t.gu(); };
        const bool cw = wv < BS_CW; // compute wave (else the I/O wave)

        // ---- compute waves: weights of a task into a slot: 8 pieces of 16 bytes and 8 scales per lane, the same
        // 16 load instructions in the same order for every task (for no task, task 0's), so that the compiler's
        // wait before a slot's registers counts the other slot's loads as later ones.  The scales are reloaded
        // once the current task's have been read, each piece once the current task's last token has unpacked it,
        // so the loads leave while the slot's last token is computed.
        // Gate/up walk: 8 lanes (j8) per row, rows nl of the gate (lanes 0-7 of a 16-lane row) and up matrix;
        // down walk: LPR lanes (jd) per row, row group gid.  A scale comes in the aligned 4-byte pair holding it.
        struct BsRef { // where a task's weights are: scalar buffer descriptors, and its kind
            __amdgpu_buffer_rsrc_t qr, dr;
            bool gu;
        };
        auto refill_addr = [&](BsTask t) {
            const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
            const BsTask u = t.n < N ? t : task(0); // (no task: task 0's loads)
            const int l = u.l(), sub = u.sub(); // sub: slice of I, or row chunk of H
            const bool gu = u.gu();
            const int64_t e = u.e();
            // the layer's matrix pointers as scalars (a per-lane choice of pointer would make the pointer load
            // itself a vector load, queued behind the other slot's weights); gate rows in waves 0-3, up rows in
            // waves 4-7, so each wave's rows start at a uniform address: the lane adds a 32-bit byte offset
            const bool up = w >= BS_CW / 2;
            const int64_t r0 = gu ? e * I + sub * 32 + 8 * (w % (BS_CW / 2)) : e * H + (int64_t)sub * DR;
            const uint8_t* qbase = gu ? bs_scalar(up ? lp.uq[l] : lp.gq[l]) + r0 * (H / 2)
                                      : bs_scalar(lp.dq[l]) + r0 * (I / 2);
            const uint8_t* dbase = reinterpret_cast<const uint8_t*>(
                gu ? bs_scalar(up ? lp.ud[l] : lp.gd[l]) + r0 * (H / 32) : bs_scalar(lp.dd[l]) + r0 * (I / 32));
            return BsRef{bs_wrsrc(qbase), bs_wrsrc(dbase), gu};
        };
        auto load_q = [&](const BsRef& R, int i) { // piece i
            const int lane = bs_opaque(threadIdx.x % WAVE), tid = bs_opaque(threadIdx.x);
            const uint32_t qoff = R.gu ? (uint32_t)((lane / 8) * (H / 2) + (lane % 8) * 16)
                                       : (uint32_t)((tid / LPR) * (I / 2) + (tid % LPR) * 16);
            return bs_ld16o(R.qr, qoff, R.gu ? Sh::gu_q(i) : Sh::dn_q(i));
        };
        auto load_s = [&](BsSlot& S, const BsRef& R) { // the 8 scales
            const int lane = bs_opaque(threadIdx.x % WAVE), tid = bs_opaque(threadIdx.x);
            const uint32_t doff = R.gu ? (uint32_t)(2 * ((lane / 8) * (H / 32) + ((lane % 8) & ~1)))
                                       : (uint32_t)(2 * ((tid / LPR) * (I / 32) + ((tid % LPR) & ~1)));
#pragma unroll
            for (int i = 0; i < 8; ++i) S.s[i] = bs_ld4o(R.dr, doff, 2 * (R.gu ? Sh::gu_d(i) : Sh::dn_d(i)));
        };
        auto issue = [&](BsSlot& S, BsTask t) { // a whole slot at once (the pipeline's start)
            const BsRef R = refill_addr(t);
            load_s(S, R);
#pragma unroll
            for (int i = 0; i < 8; ++i) S.q[i] = load_q(R, i);
        };

        // ---- compute waves: a task's arithmetic, results to LDS parity p.  With `refill` the slot is reloaded from
        // R meanwhile: the pieces during the last token (gate/up) or pair (down), each once it is unpacked, by the
        // same load instructions for both kinds, then the scales.  A task has at least one token.
        auto compute = [&](BsSlot& S, BsTask t, int p, const BsRef& R, auto refill) {
            constexpr bool RF = decltype(refill)::value;
            const int lane = bs_opaque(threadIdx.x % WAVE), tid = bs_opaque(threadIdx.x);
            const int w = tid / WAVE, j8 = lane % 8, gid = tid / LPR, jd = tid % LPR;
            const int orow = 8 * w + lane / 8; // gate/up: rows 0-31 gate, 32-63 up (waves 0-3, 4-7)
            const int l = t.l();
            const uint8_t* beg_l = mbeg + l * (BS_MAX_P + 1);
            const uint8_t* sorted_l = msorted + l * BS_MAX_P;
            const bool gu = t.gu();
            const int a = t.a(), beg = beg_l[a], cnt = beg_l[a + 1] - beg;
            const int cl = cnt > 0 ? cnt - 1 : 0; // the last token or pair
            // d_w / 16 of each piece: gate/up block j8 + 8 i of the lane's row; down row gid + GROUPS (i / BPLD),
            // block jd + LPR (i % BPLD)
            float dw[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) dw[i] = half_to_float((uint16_t)(S.s[i] >> (16 * ((gu ? j8 : jd) & 1)))) * INV16;
            // a down pair's activations: codes of its blocks, their scales and corrections
            auto dn_act = [&](int c, int4 (&a0)[BPLD], int4 (&a1)[BPLD], float (&da)[BPLD], int (&cc)[BPLD]) {
#pragma unroll
                for (int i = 0; i < BPLD; ++i) {
                    const int4* ap = reinterpret_cast<const int4*>(s_hq[p][c] + (jd + LPR * i) * 32);
                    a0[i] = ap[0];
                    a1[i] = ap[1];
                    da[i] = s_hd[p][c][jd + LPR * i];
                    cc[i] = bs_corr(a0[i]);
                }
            };
            // a down pair's rows to s_o: each row's sum over its LPR lanes; lane jd < RPL of the row group stores
            // row gid + GROUPS jd
            auto dn_out = [&](int c, float (&part)[RPL]) {
#pragma unroll
                for (int r = 0; r < RPL; ++r) part[r] = sum_group<LPR>(part[r]);
                float mine = part[0];
#pragma unroll
                for (int r = 1; r < RPL; ++r) mine = jd == r ? part[r] : mine;
                if (jd < RPL) s_o[p][c][gid + GROUPS * jd] = mine;
            };
            if (gu) {
                float dg[BPL];
#pragma unroll
                for (int i = 0; i < BPL; ++i) dg[i] = dw[i];
                for (int c = 0; c < cl; ++c) { // swiglu_row's reduction (the publisher applies SwiGLU)
                    const int tok = sorted_l[beg + c] / k;
                    const float part = sum_group<8>(bs_gu_row<BPL>(S, dg, s_xq[tok], s_xd[tok], s_xc[tok], j8));
                    if (j8 == 0) s_gu[p][c][orow] = part;
                }
            } else {
                for (int c = 0; c < cl; ++c) { // DnRow::dot's arithmetic on bs_dot16's block sums
#pragma unroll
                    for (int i = 0; i < 8; ++i) // opaque: the pieces are unpacked again for each pair
                        asm volatile("" : "+v"(S.q[i]));
                    int4 a0[BPLD], a1[BPLD];
                    float da[BPLD];
                    int cc[BPLD];
                    dn_act(c, a0, a1, da, cc);
                    float part[RPL];
#pragma unroll
                    for (int r = 0; r < RPL; ++r) {
                        float pr = 0.0f;
#pragma unroll
                        for (int i = 0; i < BPLD; ++i)
                            pr = fmaf((float)bs_dot16(bs_unpack(S.q[r * BPLD + i]), a0[i], a1[i], cc[i]),
                                      dw[r * BPLD + i] * da[i], pr);
                        part[r] = pr;
                        __builtin_amdgcn_sched_barrier(0); // one row at a time (registers)
                    }
                    dn_out(c, part);
                }
            }
            // the last token or pair, piece by piece, with the same arithmetic in the same order
#pragma unroll
            for (int i = 0; i < 8; ++i)
                asm volatile("" : "+v"(S.q[i]));
            const int tok = gu ? sorted_l[beg + cl] / k : 0;
            const int8_t* xq = s_xq[tok];
            const float* xd = s_xd[tok];
            const int* xc = s_xc[tok];
            int4 a0[BPLD], a1[BPLD];
            float da[BPLD];
            int cc[BPLD];
            if (!gu) dn_act(cl, a0, a1, da, cc);
            float gpart = 0.0f, dpart[RPL];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const BsBlk blk = bs_unpack(S.q[i]);
                if constexpr (RF) {
                    __builtin_amdgcn_sched_barrier(0); // the piece is unpacked before its registers are reloaded
                    S.q[i] = load_q(R, i);
                }
                if (gu) {
                    if (i < BPL) {
                        const int b = j8 + 8 * i;
                        const int4* ap = reinterpret_cast<const int4*>(xq + b * 32);
                        gpart = fmaf((float)bs_dot16(blk, ap[0], ap[1], xc[b]), dw[i] * xd[b], gpart);
                    }
                } else {
                    const int r = i / BPLD, ii = i % BPLD;
                    dpart[r] = fmaf((float)bs_dot16(blk, a0[ii], a1[ii], cc[ii]), dw[i] * da[ii],
                                    ii == 0 ? 0.0f : dpart[r]);
                }
                __builtin_amdgcn_sched_barrier(0); // one piece at a time (registers)
            }
            if (gu) {
                const float part = sum_group<8>(gpart);
                if (j8 == 0 && cnt > 0) s_gu[p][cl][orow] = part;
            } else if (cnt > 0) {
                dn_out(cl, dpart);
            }
            if constexpr (RF) load_s(S, R);
        };

        // ---- I/O wave: inputs of a down task (h rows of its expert's pairs) into stage parity p
        auto gather_h = [&](BsTask t, int p) {
            const int lane = bs_opaque(threadIdx.x % WAVE);
            const int l = t.l();
            const uint8_t* beg_l = mbeg + l * (BS_MAX_P + 1);
            const int a = t.a(), beg = beg_l[a], cnt = beg_l[a + 1] - beg;
            const uint64_t* src = xhb + (size_t)(l & 1) * xh_words + (size_t)beg * NS * BS_XW;
            const uint32_t tag = base + (uint32_t)l;
            const int total = cnt * NS * BS_XW;
            for (int w0 = 0; w0 < total; w0 += 8 * WAVE) {
                int idx[8];
                uint32_t live = 0, val[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const int w = w0 + lane + WAVE * m;
                    idx[m] = w < total ? w : 0;
                    if (w < total) live |= 1u << m;
                }
                bs_poll<8, 1>(src, idx, live, tag, val, ctl);
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const int w = w0 + lane + WAVE * m;
                    if (w < total) {
                        const int c = w / (NS * BS_XW), b = (w / BS_XW) % NS, wd = w % BS_XW;
                        if (wd < 8) reinterpret_cast<uint32_t*>(s_hq[p][c])[b * 8 + wd] = val[m];
                        else s_hd[p][c][b] = __uint_as_float(val[m]);
                    }
                }
            }
        };

        // ---- I/O wave: publish a task's results from LDS parity p
        auto publish = [&](BsTask t, int p) {
            const int lane = bs_opaque(threadIdx.x % WAVE);
            const int l = t.l();
            const uint8_t* beg_l = mbeg + l * (BS_MAX_P + 1);
            const uint8_t* sorted_l = msorted + l * BS_MAX_P;
            const uint32_t tag = base + (uint32_t)l;
            if (t.gu()) { // re-quantise one block of h per token (two tokens per pass) and publish it
                const int a = t.a(), slice = t.sub(), beg = beg_l[a], cnt = beg_l[a + 1] - beg;
                uint64_t* dst = xhb + (size_t)(l & 1) * xh_words;
                const int half = lane / 32, li = lane % 32;
                for (int c0 = 0; c0 < cnt; c0 += 2) {
                    const int c = c0 + half;
                    const bool live = c < cnt;
                    float v = 0.0f; // SwiGLU as swiglu_row forms it
                    if (live) {
                        const float gs = s_gu[p][c][li], us = s_gu[p][c][32 + li];
                        v = gs / (1.0f + expf(-gs)) * us;
                    }
                    const float amax = max_group<32>(fabsf(v));
                    const float d = amax / 127.0f;
                    const int code = q8_code(v, d) & 0xFF;
                    uint32_t word = 0; // lane m < 8 of each half packs the codes of outputs 4m .. 4m+3
#pragma unroll
                    for (int b = 0; b < 4; ++b) word |= (uint32_t)__shfl(code, 32 * half + 4 * (li % 8) + b) << (8 * b);
                    if (live) {
                        const int pos = beg + c;
                        if (li < BS_XW) bs_put(dst + ((size_t)pos * NS + slice) * BS_XW + li, tag, li < 8 ? word : __float_as_uint(d));
                        if (hq_all) {
                            const int64_t gpos = (int64_t)l * P + pos;
                            if (li < 8) reinterpret_cast<uint32_t*>(hq_all + gpos * I + slice * 32)[li] = word;
                            if (li == 0) hd_all[gpos * NS + slice] = d;
                        }
                    }
                }
            } else { // o of every pair of the expert for the task's DR rows, two rows per store
                const int a = t.a(), rc = t.sub(), beg = beg_l[a], cnt = beg_l[a + 1] - beg;
                const __amdgpu_buffer_rsrc_t dst = bs_rsrc(xob + (size_t)(l & 1) * xo_words);
                for (int i = lane; i < cnt * (DR / 2); i += WAVE) {
                    const int c = i / (DR / 2), r = 2 * (i % (DR / 2));
                    bs_put2(dst, sorted_l[beg + c] * H + rc * DR + r, tag, __float_as_uint(s_o[p][c][r]),
                            __float_as_uint(s_o[p][c][r + 1]));
                }
            }
        };

        // ---- x rows of layer l for the tokens of this workgroup's gate/up tasks of the layer (polled by the
        // compute waves and the gatherer; the compute waves' polls also wait for their weights in flight), with their
        // blocks' corrections; every wave meets the barrier
        auto gather_x = [&](int l) {
            const int tid = bs_opaque(threadIdx.x);
            const int WPR = H / 4 + H / 32, WPR2 = WPR / 2;
            const int nG = (int)mU[l] * NS;
            const uint8_t* beg_l = mbeg + l * (BS_MAX_P + 1);
            const uint8_t* sorted_l = msorted + l * BS_MAX_P;
            uint32_t mask = 0;
            for (int m = 0, cg = rounds(nG); m < cg; ++m) {
                const int a = expert_of(l, (m * GW + deal(m)) / NS);
                for (int c = beg_l[a]; c < beg_l[a + 1]; ++c) mask |= 1u << (sorted_l[c] / k);
            }
            mask = (uint32_t)__builtin_amdgcn_readfirstlane((int)mask);
            uint64_t lst = 0; // the listed tokens, 4 bits each
            int nt = 0;
            for (uint32_t mm = mask; mm; mm &= mm - 1u) lst |= (uint64_t)(__ffs(mm) - 1) << (4 * nt++);
            constexpr int NPT = BS_CT + WAVE; // polling threads: compute waves and the gatherer
            if (tid / WAVE != BS_PW) {
                // a thread takes 8 consecutive words of a row (4 word pairs): a block's 32 codes, which give its
                // correction for bs_dot16 (-128 x the sum of codes 0..15) at once, or 8 of the row's scales
                const int pt = tid / WAVE == BS_GW ? tid - WAVE : tid;
                const uint64_t* src = xxb + (size_t)(l & 1) * xx_words;
                const uint32_t tag = base + (uint32_t)l;
                const int QPR = WPR / 8; // H / 32 blocks of codes, then H / 256 runs of scales
                const int total = nt * QPR;
                for (int q = pt; q < total; q += NPT) {
                    const int n = q / QPR, o = q % QPR;
                    const int t = (int)((lst >> (4 * n)) & 15u);
                    int idx[4];
                    uint32_t val[4][2];
#pragma unroll
                    for (int m = 0; m < 4; ++m) idx[m] = t * WPR + 8 * o + 2 * m;
                    bs_poll2<4, 1>(src, idx, 15u, tag, val, ctl);
                    {
                        if (o < H / 32) {
                            const int4 a0 = make_int4((int)val[0][0], (int)val[0][1], (int)val[1][0], (int)val[1][1]);
                            const int4 a1 = make_int4((int)val[2][0], (int)val[2][1], (int)val[3][0], (int)val[3][1]);
                            int4* xq = reinterpret_cast<int4*>(s_xq[t] + 32 * o);
                            xq[0] = a0;
                            xq[1] = a1;
                            s_xc[t][o] = bs_corr(a0);
                        } else {
                            float4* xd = reinterpret_cast<float4*>(s_xd[t] + 8 * (o - H / 32));
                            xd[0] = make_float4(__uint_as_float(val[0][0]), __uint_as_float(val[0][1]),
                                                __uint_as_float(val[1][0]), __uint_as_float(val[1][1]));
                            xd[1] = make_float4(__uint_as_float(val[2][0]), __uint_as_float(val[2][1]),
                                                __uint_as_float(val[3][0]), __uint_as_float(val[3][1]));
                        }
                    }
                }
            }
            lds_barrier();
        };

        // ---- the pipeline.  Step i: the compute waves compute task i (slot i % 2, LDS stages of parity i % 2)
        // and refill the slot with task i + 2; meanwhile the publisher publishes task i - 1 if it is still pending
        // and the gatherer gathers the input of task i + 1 (a down task's h rows).  The publisher never waits for
        // memory, so every result a workgroup has computed gets published whatever its gatherer waits for.  Where
        // the input of task i + 1 may depend on task i's result (a gate/up task followed by a down task, and the
        // last task of a layer, whose layer the owners wait for) the step is serial: the publisher publishes task
        // i once it is computed, the gatherer gathers only then, and the compute waves wait for both at a second
        // barrier.  Within a layer the gate/up tasks precede the down tasks, so no wait is part of a cycle.  The
        // three roles run loops of their own that meet at the same barriers: one per step, a second in a serial
        // step, two where a layer's x rows are gathered.  Without a second barrier, LDS stays consistent: results
        // of parity p are published during the next step, before the compute waves can write parity p again, and
        // inputs of parity p are gathered during the step that computes parity 1 - p.
        // A gate/up task followed by a down task needs no serial step when the down task's inputs allow it (its
        // task word says so: see the task table).
        auto serial = [&](BsTask t, BsTask nxt) {
            if (nxt.n >= N || nxt.l() != t.l()) return true;
            return is_gu(t) && !is_gu(nxt) && !nxt.safe();
        };
        BsTask t0 = task(0);
        BsTask t1 = next_of(t0);
        // layer 0's x rows, when the first task needs them, are gathered before any weight load is issued: the
        // compute waves' polls would otherwise wait for the two slots' loads in flight
        const bool x0 = N > 0 && t0.first() && is_gu(t0) && t0.l() == 0;
        if (cw) {
            BsSlot A, B;
            // task t of step i from slot S (the task after it: tn), then the slot refilled with task tr (a
            // compile-time choice: the last task of an odd count is not refilled).  Every pass of the loop computes
            // and refills slot A, then slot B, and the loop has one exit, so the wait before a slot's registers
            // counts the other slot's loads as later ones.
            auto stepc = [&](BsSlot& S, BsTask t, BsTask tn, BsTask tr, int i, auto refill) {
                if (t.first() && is_gu(t) && !(t.n == 0 && x0)) gather_x(t.l()); // a layer's first task, gate/up
                const BsRef R = refill_addr(tr); // (its scalar loads are in flight while the task starts)
                compute(S, t, i & 1, R, refill);
                lds_barrier();
                if (serial(t, tn)) lds_barrier();
            };
            if (x0) gather_x(0);
            issue(A, t0);
            issue(B, t1);
            lds_barrier();
            int i = 0;
            for (; i + 1 < N; i += 2) {
                const BsTask t2 = next_of(t1);
                stepc(A, t0, t1, t2, i, std::true_type{});
                const BsTask t3 = next_of(t2);
                stepc(B, t1, t2, t3, i + 1, std::true_type{});
                t0 = t2;
                t1 = t3;
            }
            if (i < N) stepc(A, t0, t1, t0, i, std::false_type{});
        } else if (wv == BS_PW) {
            if (x0) gather_x(0); // (only its barrier)
            lds_barrier();
            bool pending = false; // task i - 1 computed, not yet published
            BsTask prev = t0;
            for (int i = 0; i < N; ++i) {
                if (t0.first() && is_gu(t0) && !(i == 0 && x0)) gather_x(t0.l()); // (only its barrier)
                if (pending) {
                    publish(prev, (i - 1) & 1);
                    pending = false;
                }
                lds_barrier(); // the compute waves are done with task i
                if (serial(t0, t1)) {
                    publish(t0, i & 1);
                    lds_barrier();
                } else {
                    pending = true;
                }
                prev = t0;
                t0 = t1;
                t1 = next_of(t1);
            }
        } else {
            if (x0) gather_x(0);
            if (N > 0 && !is_gu(t0)) gather_h(t0, 0);
            lds_barrier();
            for (int i = 0; i < N; ++i) {
                if (t0.first() && is_gu(t0) && !(i == 0 && x0)) gather_x(t0.l());
                const bool ser = serial(t0, t1);
                if (!ser && !is_gu(t1)) gather_h(t1, (i + 1) & 1);
                lds_barrier(); // the compute waves are done with task i
                if (ser) {
                    if (t1.n < N && !is_gu(t1)) gather_h(t1, (i + 1) & 1);
                    lds_barrier();
                }
                t0 = t1;
                t1 = next_of(t1);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
    }

    // departure: the last workgroup out stores the last tag used (every workgroup has read the old one)
    __syncthreads();
    if (tid == 0 &&
        __hip_atomic_fetch_add(&ctl->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)G - 1) {
        __hip_atomic_store(&ctl->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctl->epoch, base + (uint32_t)L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ------------------------------------------------------------------ launcher
bool stack_batch_supported(int E, int H, int I, int T, int k)
{
    return T >= 1 && T <= BS_MAX_T && k >= 1 && k <= BS_MAX_K && k <= E && E <= 1024 && (H == 1024 || H == 2048) &&
           (I == 256 || I == 512 || I == 1024);
}

size_t stack_batch_workspace_bytes(int L, int T, int k, int H, int I)
{
    return bs_layout(L, T, k, H, I).total;
}

int stack_batch_max_layers() { return BS_MAX_LAYERS; }

hipError_t launch_decode_stack_batch(const uint8_t* const* gq, const uint8_t* const* uq, const uint8_t* const* dq,
                                     const uint16_t* const* gd, const uint16_t* const* ud,
                                     const uint16_t* const* dd, int L, int T, int E, int H, int I, float* h,
                                     const float* logits, int k, bool rmsnorm, bool accumulate, float* h_all,
                                     int8_t* hq_all, float* hd_all, void* ws, bool* too_large, hipStream_t s)
{
    *too_large = false;
    if (L < 1 || L > BS_MAX_LAYERS || !stack_batch_supported(E, H, I, T, k)) return hipErrorInvalidValue;
    BsLayers lp = {};
    for (int l = 0; l < L; ++l) {
        lp.gq[l] = gq[l];
        lp.uq[l] = uq[l];
        lp.dq[l] = dq[l];
        lp.gd[l] = gd[l];
        lp.ud[l] = ud[l];
        lp.dd[l] = dd[l];
    }
    const BsLayout lay = bs_layout(L, T, k, H, I);
    char* wsb = reinterpret_cast<char*>(ws);
    BsCtl* ctl = reinterpret_cast<BsCtl*>(ws);
    BsMeta* meta = reinterpret_cast<BsMeta*>(wsb + BS_META_OFFSET);
    uint64_t* xx = reinterpret_cast<uint64_t*>(wsb + lay.xx);
    uint64_t* xh = reinterpret_cast<uint64_t*>(wsb + lay.xh);
    uint64_t* xo = reinterpret_cast<uint64_t*>(wsb + lay.xo);
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
#define MOEQ4_BS_LPL(E, ...)                                        \
    if ((E) <= 64) { constexpr int LP = 1; __VA_ARGS__; }            \
    else if ((E) <= 128) { constexpr int LP = 2; __VA_ARGS__; }      \
    else if ((E) <= 256) { constexpr int LP = 4; __VA_ARGS__; }      \
    else { constexpr int LP = 16; __VA_ARGS__; }
    // the routing of every layer and x of layer 0 (L + ceil(T / 4) workgroups; the x buffer of parity 0)
    MOEQ4_BS_LPL(E, bstack_prep_kernel<LP><<<dim3((unsigned)(L + (T + 3) / 4)), BS_PREP_THREADS, 0, s>>>(
                        logits, L, T, E, k, h, H, rmsnorm, meta, xx, ctl));
#undef MOEQ4_BS_LPL
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    auto go = [&](auto kern, size_t lds, int DR) -> hipError_t {
        hipError_t e2 = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e2 != hipSuccess) return e2;
        e2 = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)kern, BS_BLOCK, lds);
        if (e2 != hipSuccess) return e2;
        const int G = per_cu * cus;
        if (G < T + 1) {
            *too_large = true;
            return hipErrorInvalidValue;
        }
        // the task table: a worker's tasks over all layers, at most ceil(P NS / GW) + ceil(P ND / GW) per layer
        const int64_t GW = G - T, P = (int64_t)T * k, per_layer = (P * (I / 32) + GW - 1) / GW + (P * (H / DR) + GW - 1) / GW;
        if ((int64_t)L * per_layer > BS_MAX_TASKS) {
            *too_large = true;
            return hipErrorInvalidValue;
        }
        kern<<<dim3((unsigned)G), BS_BLOCK, lds, s>>>(lp, L, T, k, H, I, rmsnorm, accumulate, h, h_all, hq_all,
                                                      hd_all, meta, xx, xh, xo, lay.xx_words, lay.xh_words,
                                                      lay.xo_words, ctl);
        return hipGetLastError();
    };
#define MOEQ4_BS_GO(B_, R_) go(bstack_kernel<B_, R_>, BsShape<B_, R_>::BYTES, BsShape<B_, R_>::DR)
    switch (H / 256 * 100 + I / 32) {
    case 808: return MOEQ4_BS_GO(8, 8);
    case 816: return MOEQ4_BS_GO(8, 16);
    case 832: return MOEQ4_BS_GO(8, 32);
    case 408: return MOEQ4_BS_GO(4, 8);
    case 416: return MOEQ4_BS_GO(4, 16);
    case 432: return MOEQ4_BS_GO(4, 32);
    default: return hipErrorInvalidValue;
    }
#undef MOEQ4_BS_GO
}

} // namespace moeq4
