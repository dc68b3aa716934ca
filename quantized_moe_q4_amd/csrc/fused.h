// fused.h -- routing and control state shared by the one-launch decode
// kernels (the single-layer fused decode and the multi-layer stack decode):
// the sync area at the start of the workspace, the per-workgroup routing state
// in LDS, and the routing steps every workgroup runs itself (top-k selection,
// the stable counting sort of the pairs, the renormalised weights).  Dutch
// technical summary "Methodologie 1" of "A 35B Hybrid-Attention
// Mixture-of-Experts Model on a 6GB 2011 GPU": routed experts over resident
// 4-bit weights.
#pragma once
#include <cstddef>

#include "device.h"
#include "rows.h"
#include "topk.h"

namespace moeq4 {

constexpr int FD_THREADS = 512;
constexpr int FD_WAVES = FD_THREADS / WAVE;
constexpr int FD_GROUP = 256; // threads of one expert group in a down workgroup
constexpr int FD_MAX_T = 8; // one wave per token in the routing step
constexpr int FD_MAX_P = FD_MAX_T * 16;
constexpr int FD_MAX_HQ = 64 * 1024; // P * I bytes a down workgroup stages in LDS
constexpr uint32_t FD_SPIN_LIMIT = 1u << 20;

// Synchronisation words at the start of the workspace.  Same-address atomics
// are serialised where they are performed (memory side), so arrivals and
// departures are spread over FD_NCTR counters, each on its own 256-byte line:
// gate/up workgroup g counts on line g % FD_NCTR, down workgroup d departs on
// line d % FD_NCTR, and the last departure of a line bumps `done2`.
constexpr int FD_NCTR = 8;
struct FdLine {
    uint32_t arrive; // gate/up workgroups of this line that have published h
    uint32_t pad0[15];
    uint32_t done;   // down workgroups of this line past the wait
    uint32_t pad1[47];
};
struct FdCtl {
    FdLine line[FD_NCTR];
    uint32_t done2;  // lines whose down workgroups have all departed
    uint32_t pad[15];
    uint32_t error;  // sticky: nonzero after a wait gave up
    uint32_t pad2[15];
    uint32_t epoch;  // last exchange tag used on this workspace (skips 0; wraps below 2^32 - 1)
    uint32_t pad3[15];
    uint32_t stack_done; // workgroups of a stack decode that have finished (the last one resets it)
};
static_assert(sizeof(FdLine) == 256, "one counter line per 256 bytes");
static_assert(offsetof(FdCtl, error) == 2112, "error word offset is part of the ABI");
static_assert(offsetof(FdCtl, stack_done) == 2240, "stack departure counter on its own line");
static_assert(sizeof(FdCtl) <= 4096, "the control words fit their 4 KB");

// Tagged exchange of h (small batches): block b = (sorted position, slice of
// 32 outputs) of h is published as FD_XW 64-bit words at xch[b * FD_XW + w]:
// words 0..7 carry its 32 codes (4 per word, output 4w in the low byte),
// word 8 the bit pattern of its scale, each in the low half and the call's
// epoch in the high half.  64-bit stores and loads are single-copy atomic, so
// a word that shows the current epoch carries this call's payload: the down
// workgroups poll the data itself, one memory round trip instead of an
// arrival counter followed by a load of h.  Epochs start at 1 and skip 0, so
// the zero-filled area never matches.
constexpr size_t FD_XCH_OFFSET = 4096; // bytes from the start of the workspace
constexpr int FD_XCH_WORDS = 2048;     // 16 KB: four words per thread of a down workgroup
constexpr int FD_XW = 9;               // words per block of h

constexpr int FD_RANK_KEYS = 2048; // logits of one token up to which selection ranks them all in parallel (16 KB of keys)

// Padded staging of h rows for the quad down walk (DnQuad::dot<true>): block b at 32 b + 16 (b / 4) (16 bytes of
// padding after every 4 blocks), and a row stride of 16 (8 r + 2) bytes, so
// the 16-byte reads of the 8 experts' quads (lanes i, blocks 4 i + jj) spread
// evenly over the LDS banks instead of all landing on the same ones.
__host__ __device__ constexpr int hq_row_padded(int NS)
{
    const int u = (NS * 32 + (NS / 4) * 16 + 15) / 16; // 16-byte units of a padded row
    return 16 * (u + (10 - u % 8) % 8);                 // the next count = 2 (mod 8)
}
constexpr int HQ_ROW_PADDED_MAX = hq_row_padded(32);
static_assert(hq_row_padded(16) == 672 && HQ_ROW_PADDED_MAX == 1184, "padded h rows");

struct FdRoute {
    __align__(16) int e[FD_MAX_P]; // expert of pair p = t*k + j
    float v[FD_MAX_P];      // its logit
    float w[FD_MAX_P];      // renormalised weight of pair p (down workgroups only)
    int sorted[FD_MAX_P];   // pair at sorted position r
    int se[FD_MAX_P];       // expert at sorted position r
    int list[FD_MAX_P];     // active experts, ascending
    int beg[FD_MAX_P + 1];  // first sorted position of each active expert; beg[U] = P
    __align__(16) uint64_t key[FD_RANK_KEYS]; // (logit image, ~id) keys, [T][EP], 0-padded
    uint32_t active[1024 / 32];               // bit e: expert e has a pair (more than 64 pairs)
    int U;
};

// Top-k selection of every token, slot j = the j-th largest logit (equal
// logits: lower expert id first), the order of the router's wave arg-max.
// One token with up to FD_RANK_KEYS logits: every thread takes part, the
// router's 64-bit (logit image, ~id) keys (unique) go to LDS, 4 threads per
// key count the larger keys (a quad sum gives its rank), and rank j < k fills
// slot j.  Otherwise one wave per token runs the router's selection rounds
// (the tokens in parallel; ranking every token's keys would take a pass per
// token).  Every
// selected expert also sets its bit in R.active, from which a workgroup finds
// the a-th active expert without waiting for the sort of the pairs.
// REGS (one token, E <= 1024): the logits come from registers instead of
// `logits`, thread tid holding logits tid (r0) and tid + FD_THREADS (r1).
template <int LPL, bool REGS = false>
__device__ void fd_select(const float* __restrict__ logits, int T, int E, int k, FdRoute& R, float r0 = 0.0f,
                          float r1 = 0.0f)
{
    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    if (tid < 1024 / 32) R.active[tid] = 0u; // ordered before the atomics by the barrier below
    constexpr int QP = 4;                // threads per key
    const int EP = (E + 7) & ~7;         // padded row: QP parts of whole 16-byte pairs of keys
    const int C2 = EP / QP / 2;          // 16-byte reads per part
    if (T == 1 && EP <= FD_RANK_KEYS) {
        for (int i = tid; i < T * EP; i += FD_THREADS) { // 0 is below every real key
            const int t = i / EP, e = i % EP;
            if constexpr (REGS) R.key[i] = e < E ? topk_key(i < FD_THREADS ? r0 : r1, e) : 0ull;
            else R.key[i] = e < E ? topk_key(logits[t * E + e], e) : 0ull;
        }
        lds_barrier();
        const int items = T * E * QP;
        const int items_pad = (items + WAVE - 1) / WAVE * WAVE; // whole waves iterate together
        for (int it = tid; it < items_pad; it += FD_THREADS) {
            const bool live = it < items;
            const int q = it % QP, te = live ? it / QP : 0;
            const int t = te / E, e = te % E;
            const uint64_t* kr = R.key + t * EP;
            const uint64_t ke = kr[e];
            const ulonglong2* part = reinterpret_cast<const ulonglong2*>(kr) + q * C2;
            int cnt = 0;
#pragma unroll 8
            for (int c = 0; c < C2; ++c) {
                const ulonglong2 ko = part[c];
                cnt += ko.x > ke;
                cnt += ko.y > ke;
            }
            cnt += dpp<DPP_QUAD_1032>(cnt);
            cnt += dpp<DPP_QUAD_2301>(cnt);
            if (live && q == 0 && cnt < k) { // rank = slot
                R.e[t * k + cnt] = e;
                R.v[t * k + cnt] = key_value(ke);
                atomicOr(&R.active[e >> 5], 1u << (e & 31));
            }
        }
    } else if (wv < T) {
        const uint64_t mine = select_topk_keys<LPL>(logits + (int64_t)wv * E, E, k, lane);
        if (lane < k) {
            const int e = (int)(0xFFFFFFFFu - (uint32_t)mine);
            R.e[wv * k + lane] = e;
            R.v[wv * k + lane] = key_value(mine);
            atomicOr(&R.active[e >> 5], 1u << (e & 31));
        }
    }
    lds_barrier();
}

// The a-th active expert (ascending ids) from the bitmask R.active, or -1 when
// fewer than a + 1 experts are active.  Every thread computes it (uniform).
__device__ __forceinline__ int fd_nth_active(const FdRoute& R, int E, int a)
{
    for (int w = 0; w < (E + 31) / 32; ++w) {
        uint32_t m = R.active[w];
        const int c = __popc(m);
        if (a < c) {
            for (int i = 0; i < a; ++i) m &= m - 1u; // drop the a lowest set bits
            return 32 * w + __ffs(m) - 1;
        }
        a -= c;
    }
    return -1;
}

// The stable counting sort of the pairs by expert (rank of each pair among
// pairs with a lower expert, or the same expert and a lower pair id), and the
// list of active experts with their first sorted positions.  Up to 16 pairs,
// wave 0 holds pair p in lane p and reads every pair's expert with broadcast
// 16-byte LDS reads; up to 64, every wave counts over its own 8 pairs and
// wave 0 adds the counts; beyond that, every thread takes one pair.  The
// bitmask of active experts (filled by fd_select) gives each expert's list
// index (the active experts below it) where the start flags are not all in
// one wave.
__device__ inline void fd_sort(int P, FdRoute& R)
{
    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    if (P > 16 && P <= WAVE) {
        // wave w counts, for pair p = lane, the pairs q = 8w .. 8w + 7 that sort before it; the keys of the
        // selection are dead by now, so their LDS holds the partial counts (rank | before << 8)
        static_assert(FD_THREADS / WAVE * 8 >= WAVE, "the waves' shares cover 64 pairs");
        int* s_cnt = reinterpret_cast<int*>(R.key); // [FD_THREADS / WAVE][WAVE]
        const int ep = lane < P ? R.e[lane] : INT32_MAX;
        int part = 0;
        if (8 * wv < P) {
            const int4 e0 = reinterpret_cast<const int4*>(R.e)[2 * wv], e1 = reinterpret_cast<const int4*>(R.e)[2 * wv + 1];
            const int es[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
            int rank = 0, before = 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int q = 8 * wv + u;
                const bool in = q < P; // entries past P in the last group are masked out
                rank += in && ((es[u] < ep) || (es[u] == ep && q < lane));
                before += in && es[u] == ep && q < lane;
            }
            part = rank | (before << 8);
        }
        s_cnt[wv * WAVE + lane] = part;
        lds_barrier();
        if (wv == 0) {
            int rank = 0, before = 0;
#pragma unroll
            for (int w = 0; w < FD_THREADS / WAVE; ++w) {
                const int c = s_cnt[w * WAVE + lane];
                rank += c & 0xFF;
                before += c >> 8;
            }
            const bool start = lane < P && before == 0; // the expert's first pair
            if (lane < P) {
                R.sorted[rank] = lane;
                R.se[rank] = ep;
            }
            if (start) { // its list entry: the active experts below it, from the selection's bitmask
                int idx = __popc(R.active[ep >> 5] & ((1u << (ep & 31)) - 1u));
                for (int w = 0; w < (ep >> 5); ++w) idx += __popc(R.active[w]);
                R.list[idx] = ep;
                R.beg[idx] = rank;
            }
            const int U = __popcll(__ballot(start));
            if (lane == 0) {
                R.U = U;
                R.beg[U] = P;
            }
        }
        lds_barrier();
        return;
    }
    if (P <= WAVE) {
        if (wv == 0) {
            // every lane reads all slots' experts with broadcast 16-byte LDS reads
            const int ep = lane < P ? R.e[lane] : INT32_MAX;
            const int P4 = (P + 3) / 4;
            int rank = 0, before = 0;
#pragma unroll 4
            for (int c = 0; c < P4; ++c) {
                const int4 e4 = reinterpret_cast<const int4*>(R.e)[c];
                const int es[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int q = 4 * c + u;
                    const bool in = q < P; // entries past P in the last group are masked out
                    rank += in && ((es[u] < ep) || (es[u] == ep && q < lane));
                    before += in && es[u] == ep && q < lane;
                }
            }
            const bool start = lane < P && before == 0; // the expert's first pair
            const uint64_t starts = __ballot(start);
            int idx = 0; // active experts below this one
#pragma unroll 4
            for (int c = 0; c < P4; ++c) {
                const int4 e4 = reinterpret_cast<const int4*>(R.e)[c];
                const int es[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int q = 4 * c + u;
                    idx += q < P && ((starts >> q) & 1ull) && es[u] < ep;
                }
            }
            if (lane < P) {
                R.sorted[rank] = lane;
                R.se[rank] = ep;
            }
            if (start) {
                R.list[idx] = ep;
                R.beg[idx] = rank;
            }
            const int U = __popcll(__ballot(start));
            if (lane == 0) {
                R.U = U;
                R.beg[U] = P;
            }
        }
        lds_barrier();
        return;
    }
    int rank = 0, before = 0, ep = 0;
    if (tid < P) {
        ep = R.e[tid];
        const int P4 = (P + 3) / 4;
#pragma unroll 4
        for (int c = 0; c < P4; ++c) { // entries at or beyond P in the last int4 are masked out
            const int4 eq = reinterpret_cast<const int4*>(R.e)[c];
            const int q0 = 4 * c;
            const int es[4] = {eq.x, eq.y, eq.z, eq.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool in = q0 + u < P;
                rank += in && ((es[u] < ep) || (es[u] == ep && q0 + u < tid));
                before += in && es[u] == ep && q0 + u < tid;
            }
        }
        R.sorted[rank] = tid;
        R.se[rank] = ep;
    }
    const int U = __syncthreads_count(tid < P && before == 0); // active experts
    if (tid < P && before == 0) { // the expert's first pair: its list entry
        int idx = __popc(R.active[ep >> 5] & ((1u << (ep & 31)) - 1u));
        for (int w = 0; w < (ep >> 5); ++w) idx += __popc(R.active[w]);
        R.list[idx] = ep;
        R.beg[idx] = rank;
    }
    if (tid == 0) {
        R.U = U;
        R.beg[U] = P;
    }
    lds_barrier();
}

// Renormalised weights, wave t for token t: the router's own arithmetic.
__device__ inline void fd_weights(int T, int k, FdRoute& R)
{
    const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
    if (wv < T) {
        const float v = lane < k ? R.v[wv * k + lane] : 0.0f;
        const float w = topk_weight(v, k, lane);
        if (lane < k) R.w[wv * k + lane] = w;
    }
    lds_barrier();
}

// The router's outputs, as moe_q4_route writes them (the weights separately).
__device__ inline void fd_write_route(const FdRoute& R, int T, int E, int k, int32_t* __restrict__ ids,
                               int32_t* __restrict__ offsets, int32_t* __restrict__ sorted)
{
    const int tid = threadIdx.x, P = T * k;
    for (int p = tid; p < P; p += FD_THREADS) {
        ids[p] = R.e[p];
        sorted[p] = R.sorted[p];
    }
    for (int e = tid; e <= E; e += FD_THREADS) { // offsets[e] = pairs with a lower expert
        int lo = 0, hi = P;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (R.se[mid] < e) lo = mid + 1;
            else hi = mid;
        }
        offsets[e] = lo;
    }
}

__device__ __forceinline__ void quant4_lds(float4 v, float d, int8_t* dst)
{
    const uint32_t q0 = (uint32_t)(q8_code(v.x, d) & 0xFF);
    const uint32_t q1 = (uint32_t)(q8_code(v.y, d) & 0xFF);
    const uint32_t q2 = (uint32_t)(q8_code(v.z, d) & 0xFF);
    const uint32_t q3 = (uint32_t)(q8_code(v.w, d) & 0xFF);
    *reinterpret_cast<uint32_t*>(dst) = q0 | (q1 << 8) | (q2 << 16) | (q3 << 24);
}

__device__ __forceinline__ float amax4f(float4 v)
{
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// Launch-time dispatch over the kernels' template parameters: B = blocks per
// gate/up lane (H / 256), R = blocks per down row (I / 32), LP = logits per
// lane of the router's selection rounds.
#define MOEQ4_FD_BPL(BPLV, ...)                          \
    switch (BPLV) {                                      \
    case 1: { constexpr int B = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int B = 2; __VA_ARGS__; } break; \
    case 4: { constexpr int B = 4; __VA_ARGS__; } break; \
    case 8: { constexpr int B = 8; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;                \
    }
#define MOEQ4_FD_NBR(NBRV, ...)                            \
    switch (NBRV) {                                        \
    case 8: { constexpr int R = 8; __VA_ARGS__; } break;   \
    case 16: { constexpr int R = 16; __VA_ARGS__; } break; \
    case 32: { constexpr int R = 32; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;                  \
    }
#define MOEQ4_FD_LPL(E, ...)                                          \
    if ((E) <= 128) { constexpr int LP = 2; __VA_ARGS__; }             \
    else if ((E) <= 256) { constexpr int LP = 4; __VA_ARGS__; }        \
    else { constexpr int LP = 16; __VA_ARGS__; }

} // namespace moeq4
