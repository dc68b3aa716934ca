// rows.h -- Q4_0 row walks of the W4A8 decode GEMV (Dutch technical summary
// "Methodologie 1" and "Methodologie 2" of "A 35B Hybrid-Attention
// Mixture-of-Experts Model on a 6GB 2011 GPU": integer multiply-adds over 4-bit
// weights and 8-bit activations), shared by the standalone decode kernels and
// the fused one-launch decode, so both produce bit-identical results.
//
// Row walks (one Q4_0 row = K/32 blocks of 16 nibble bytes + fp16 scales):
//   gate/up walk (K = hidden): 8 lanes per row, lane j owns blocks j, j+8, ...;
//     each load instruction of a wave reads 8 rows x 128 contiguous bytes.
//   down walk (K = inter): LPR = min(K/32, 16) lanes per row, lane j owns
//     blocks j, j+LPR, ...; a wave reads 64/LPR rows per instruction.
// Nibbles are unpacked to 16 (q - 8) (device.h), so 8 v_dot4 give 16 x the
// exact int32 block dot; the 16 is folded into d_w.  The fp32 contribution
// d_w d_a isum of each block is summed over the row's lanes.
#pragma once
#include "device.h"

namespace moeq4 {

// The fp16 scales of a lane's blocks j, j + 8, ..., j + 8 (BPL - 1), as loaded.
// At BPL = 8 the lane instead loads the 8 consecutive scales 8j .. 8j + 7 with
// one 16-byte load (a row's 64 scales are 8 such pieces), and GuRow::finish
// transposes them across the row's 8 lanes: one load instead of eight, which
// is most of the load instructions a row walk issues.
template <int BPL>
struct GuScales {
    uint16_t h[BPL];
};
template <>
struct GuScales<8> {
    uint4 w;
};

// 8 x 8 transpose of 16-bit values across the 8 lanes j of an aligned lane
// group: lane j holds w = values (8j .. 8j + 7) (value 2k in the low half of
// word k) and receives values (j, j + 8, ..., j + 56), in the same packing.
// Three exchange stages (partner distance 4, 2, 1) by DPP inside 16-lane rows.
// Every DPP move is made by all lanes and every choice is a bit-mask select:
// a DPP read from a lane that a branch has switched off returns the old value.
__device__ __forceinline__ uint32_t sel32(uint32_t m, uint32_t a, uint32_t b) { return (a & m) | (b & ~m); }

__device__ __forceinline__ uint4 transpose8x8_u16(uint4 v, int j)
{
    uint32_t W[4] = {v.x, v.y, v.z, v.w};
    { // distance 4: lanes 0-3 trade their elements 4-7 for the elements 0-3 of lanes 4-7
        const uint32_t m = (j & 4) ? 0xFFFFFFFFu : 0u;
        const uint32_t x0 = sel32(m, W[0], W[2]), x1 = sel32(m, W[1], W[3]);
        const uint32_t dn0 = (uint32_t)dpp<DPP_ROW_SHL4>((int)x0), up0 = (uint32_t)dpp<DPP_ROW_SHR4>((int)x0); // from j + 4, j - 4
        const uint32_t dn1 = (uint32_t)dpp<DPP_ROW_SHL4>((int)x1), up1 = (uint32_t)dpp<DPP_ROW_SHR4>((int)x1);
        const uint32_t r0 = sel32(m, up0, dn0), r1 = sel32(m, up1, dn1); // lane j - 4 or lane j + 4
        W[0] = sel32(m, r0, W[0]);
        W[1] = sel32(m, r1, W[1]);
        W[2] = sel32(m, W[2], r0);
        W[3] = sel32(m, W[3], r1);
    }
    { // distance 2
        const uint32_t m = (j & 2) ? 0xFFFFFFFFu : 0u;
        const uint32_t x0 = sel32(m, W[0], W[1]), x1 = sel32(m, W[2], W[3]);
        const uint32_t r0 = (uint32_t)dpp<DPP_QUAD_2301>((int)x0), r1 = (uint32_t)dpp<DPP_QUAD_2301>((int)x1);
        W[0] = sel32(m, r0, W[0]);
        W[1] = sel32(m, W[1], r0);
        W[2] = sel32(m, r1, W[2]);
        W[3] = sel32(m, W[3], r1);
    }
    { // distance 1: 16-bit halves
        const uint32_t m = (j & 1) ? 0xFFFFFFFFu : 0u;
        const uint32_t s0 = sel32(m, (W[0] & 0xFFFFu) | (W[1] << 16), (W[0] >> 16) | (W[1] & 0xFFFF0000u));
        const uint32_t s1 = sel32(m, (W[2] & 0xFFFFu) | (W[3] << 16), (W[2] >> 16) | (W[3] & 0xFFFF0000u));
        const uint32_t r0 = (uint32_t)dpp<DPP_QUAD_1032>((int)s0), r1 = (uint32_t)dpp<DPP_QUAD_1032>((int)s1);
        W[0] = sel32(m, (W[0] & 0xFFFF0000u) | (r0 & 0xFFFFu), (W[0] & 0xFFFFu) | (r0 << 16));
        W[1] = sel32(m, (W[1] & 0xFFFF0000u) | (r0 >> 16), (W[1] & 0xFFFFu) | (r0 & 0xFFFF0000u));
        W[2] = sel32(m, (W[2] & 0xFFFF0000u) | (r1 & 0xFFFFu), (W[2] & 0xFFFFu) | (r1 << 16));
        W[3] = sel32(m, (W[3] & 0xFFFF0000u) | (r1 >> 16), (W[3] & 0xFFFFu) | (r1 & 0xFFFF0000u));
    }
    return make_uint4(W[0], W[1], W[2], W[3]);
}

template <int BPL> // blocks per lane = K / 256
struct GuRow {
    // Nibbles stay packed (4 registers per block) and are unpacked block by
    // block inside the dot product: at BPL = 8 this keeps a 512-thread gate/up
    // workgroup under 128 registers per lane, two workgroups per CU.
    uint4 raw[BPL];
    float dw[BPL]; // d_w / 16
    static constexpr int G = BPL < 4 ? BPL : 4; // blocks whose activations are loaded together

    // loads in flight until finish(): nothing here waits on memory (NT: the non-temporal hint)
    template <bool NT = true>
    __device__ __forceinline__ static void issue(const uint8_t* __restrict__ qrow, const uint16_t* __restrict__ drow,
                                                 int j, uint4 (&r)[BPL], GuScales<BPL>& dh)
    {
#pragma unroll
        for (int i = 0; i < BPL; ++i) r[i] = ld_w16<NT>(qrow + (j + 8 * i) * 16);
        if constexpr (BPL == 8) {
            dh.w = ld_w16<NT>(reinterpret_cast<const uint8_t*>(drow + 8 * j));
        } else {
#pragma unroll
            for (int i = 0; i < BPL; ++i) dh.h[i] = ld_w_u16<NT>(drow + j + 8 * i);
        }
    }

    // j: the lane's index in its row's aligned group of 8 lanes (all 8 take part)
    __device__ __forceinline__ void finish(const uint4 (&r)[BPL], const GuScales<BPL>& dh, int j)
    {
        if constexpr (BPL == 8) {
            const uint4 t = transpose8x8_u16(dh.w, j);
            const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int i = 0; i < BPL; ++i) dw[i] = half_to_float((uint16_t)(w[i / 2] >> (16 * (i % 2)))) * INV16;
        } else {
#pragma unroll
            for (int i = 0; i < BPL; ++i) dw[i] = half_to_float(dh.h[i]) * INV16;
        }
#pragma unroll
        for (int i = 0; i < BPL; ++i) raw[i] = r[i];
    }

    template <bool NT = true>
    __device__ __forceinline__ void load(const uint8_t* __restrict__ qrow, const uint16_t* __restrict__ drow, int j)
    {
        uint4 r[BPL];
        GuScales<BPL> dh;
        issue<NT>(qrow, drow, j, r, dh);
        finish(r, dh, j);
    }

    __device__ __forceinline__ void unpack_only(const uint8_t* __restrict__ qrow, int j)
    {
#pragma unroll
        for (int i = 0; i < BPL; ++i) raw[i] = ld_stream16(qrow + (j + 8 * i) * 16);
    }

    // 16 x isum of block j + 8i against an activation row
    __device__ __forceinline__ int isum16(int i, const int8_t* __restrict__ arow, int j) const
    {
        const int4* ap = reinterpret_cast<const int4*>(arow + (j + 8 * i) * 32);
        const int4 a0 = ap[0], a1 = ap[1];
        const int a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        int wq[8];
        unpack_block16(raw[i], wq);
        return block_dot16(wq, a);
    }

    // this lane's share of one output: sum over its blocks (in order) of
    // d_w d_a isum; each group's activation loads are issued before its dots
    __device__ __forceinline__ float partial(const int8_t* __restrict__ arow, const float* __restrict__ adr,
                                             int j) const
    {
        float part = 0.0f;
#pragma unroll
        for (int g0 = 0; g0 < BPL; g0 += G) {
            int4 a[G][2];
            float da[G];
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const int4* ap = reinterpret_cast<const int4*>(arow + (j + 8 * (g0 + i)) * 32);
                a[i][0] = ap[0];
                a[i][1] = ap[1];
            }
#pragma unroll
            for (int i = 0; i < G; ++i) da[i] = adr[j + 8 * (g0 + i)];
            __builtin_amdgcn_sched_barrier(0); // keep the group's loads ahead of its dot products
#pragma unroll
            for (int i = 0; i < G; ++i) {
                int wq[8];
                unpack_block16(raw[g0 + i], wq);
                const int av[8] = {a[i][0].x, a[i][0].y, a[i][0].z, a[i][0].w,
                                   a[i][1].x, a[i][1].y, a[i][1].z, a[i][1].w};
                part = fmaf((float)block_dot16(wq, av), dw[g0 + i] * da[i], part);
            }
        }
        return part;
    }
};

// A gate/up row walk whose nibbles are unpacked ahead of the dot products:
// where the weights arrive well before the activations they wait for, the
// unpacking (most of the walk's VALU work) leaves the critical path.  The
// arithmetic of partial() is GuRow's, operation for operation.
template <int BPL>
struct GuRowUnpacked {
    int wq[BPL][8]; // 16 (q - 8) per byte
    float dw[BPL];  // d_w / 16
    static constexpr int G = GuRow<BPL>::G;

    __device__ __forceinline__ void unpack(const GuRow<BPL>& w)
    {
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            dw[i] = w.dw[i];
            unpack_block16(w.raw[i], wq[i]);
            // pinned here: the unpacked operands are not re-derived inside the dot products
#pragma unroll
            for (int m = 0; m < 8; ++m) asm volatile("" : "+v"(wq[i][m]));
        }
    }

    __device__ __forceinline__ float partial(const int8_t* __restrict__ arow, const float* __restrict__ adr,
                                             int j) const
    {
        float part = 0.0f;
#pragma unroll
        for (int g0 = 0; g0 < BPL; g0 += G) {
            int4 a[G][2];
            float da[G];
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const int4* ap = reinterpret_cast<const int4*>(arow + (j + 8 * (g0 + i)) * 32);
                a[i][0] = ap[0];
                a[i][1] = ap[1];
            }
#pragma unroll
            for (int i = 0; i < G; ++i) da[i] = adr[j + 8 * (g0 + i)];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const int av[8] = {a[i][0].x, a[i][0].y, a[i][0].z, a[i][0].w,
                                   a[i][1].x, a[i][1].y, a[i][1].z, a[i][1].w};
                part = fmaf((float)block_dot16(wq[g0 + i], av), dw[g0 + i] * da[i], part);
            }
        }
        return part;
    }
};

template <int NBR> // blocks per row = K / 32
struct DnRow {
    static constexpr int LPR = NBR < 16 ? NBR : 16;
    static constexpr int BPL = NBR / LPR;
    int wq[BPL][8];
    float dw[BPL]; // d_w / 16

    __device__ __forceinline__ void issue(const uint8_t* __restrict__ qrow, const uint16_t* __restrict__ drow, int j,
                                          uint4 raw[BPL], uint16_t dh[BPL]) const
    {
#pragma unroll
        for (int i = 0; i < BPL; ++i) raw[i] = ld_stream16(qrow + (j + LPR * i) * 16);
#pragma unroll
        for (int i = 0; i < BPL; ++i) dh[i] = ld_stream_u16(drow + j + LPR * i);
    }

    __device__ __forceinline__ void finish(const uint4 raw[BPL], const uint16_t dh[BPL])
    {
#pragma unroll
        for (int i = 0; i < BPL; ++i) dw[i] = half_to_float(dh[i]) * INV16;
#pragma unroll
        for (int i = 0; i < BPL; ++i) unpack_block16(raw[i], wq[i]);
    }

    __device__ __forceinline__ int isum16(int i, const int8_t* __restrict__ arow, int j) const
    {
        const int4* ap = reinterpret_cast<const int4*>(arow + (j + LPR * i) * 32);
        const int4 a0 = ap[0], a1 = ap[1];
        const int a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        return block_dot16(wq[i], a);
    }

    // one h row's operands for this lane's blocks
    struct Act {
        int4 a[BPL][2];
        float da[BPL];
    };

    __device__ __forceinline__ static void load_act(const int8_t* __restrict__ arow, const float* __restrict__ adr,
                                                    int j, Act& A)
    {
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            const int4* ap = reinterpret_cast<const int4*>(arow + (j + LPR * i) * 32);
            A.a[i][0] = ap[0];
            A.a[i][1] = ap[1];
        }
#pragma unroll
        for (int i = 0; i < BPL; ++i) A.da[i] = adr[j + LPR * i];
    }

    // this lane's share of one output: sum over its blocks of d_w d_a isum
    __device__ __forceinline__ float dot(const Act& A) const
    {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
            const int av[8] = {A.a[i][0].x, A.a[i][0].y, A.a[i][0].z, A.a[i][0].w,
                               A.a[i][1].x, A.a[i][1].y, A.a[i][1].z, A.a[i][1].w};
            part = fmaf((float)block_dot16(wq[i], av), dw[i] * A.da[i], part);
        }
        return part;
    }

    __device__ __forceinline__ float partial(const int8_t* __restrict__ arow, const float* __restrict__ adr,
                                             int j) const
    {
        Act A;
        load_act(arow, adr, j, A);
        __builtin_amdgcn_sched_barrier(0); // keep every load ahead of the dot products
        return dot(A);
    }
};

// ------------------------------------------------------------------ down row by a quad of lanes
// One output row of one expert by 4 lanes instead of LPR: lane i of the quad
// takes the blocks of DnRow lanes i*JPL .. i*JPL + JPL - 1.  Each of those
// lanes' values is formed exactly as DnRow::dot forms it (its blocks j,
// j + LPR, ... in order, one fmaf each), the lane adds its JPL values as the
// first levels of sum_group<LPR> would ((v0 + v1) + (v2 + v3)), and two quad
// steps finish the tree.  fp32 addition is commutative, so every addition
// has the same operands as in the LPR-lane walk: the result is bit-identical,
// with far fewer instructions per lane when a workgroup has few experts.
template <int NBR>
struct DnQuad {
    static constexpr int LPR = NBR < 16 ? NBR : 16;
    static constexpr int BPL = NBR / LPR;
    static constexpr int JPL = LPR / 4; // DnRow lanes folded into one quad lane
    static_assert(JPL == 2 || JPL == 4, "quad walk: 8, 16 or 32 blocks per row");
    uint4 raw[BPL][JPL];
    uint2 dpk[BPL]; // the JPL consecutive scales of each block row, one 8- (JPL 4) or 4-byte (JPL 2) load

    __device__ __forceinline__ void issue(const uint8_t* __restrict__ qrow, const uint16_t* __restrict__ drow, int i)
    {
#pragma unroll
        for (int b = 0; b < BPL; ++b)
#pragma unroll
            for (int jj = 0; jj < JPL; ++jj) raw[b][jj] = ld_stream16(qrow + (i * JPL + jj + LPR * b) * 16);
#pragma unroll
        for (int b = 0; b < BPL; ++b)
            dpk[b] = JPL == 4 ? ld_stream8(drow + i * JPL + LPR * b)
                              : make_uint2(ld_stream4(drow + i * JPL + LPR * b), 0u);
    }

    __device__ __forceinline__ uint16_t dh(int b, int jj) const
    {
        const uint32_t w = jj < 2 ? dpk[b].x : dpk[b].y;
        return (uint16_t)(w >> (16 * (jj % 2)));
    }

    // the row's output against one h row (int8 [I] and its scales), in all 4 lanes of the quad.  PAD: the
    // row is staged with 16 bytes of padding after every 4 blocks (block b at 32 b + 16 (b / 4)), which
    // spreads the quad's lanes over the LDS banks
    template <bool PAD = false>
    __device__ __forceinline__ float dot(const int8_t* __restrict__ arow, const float* __restrict__ adr, int i) const
    {
        float v[JPL];
#pragma unroll
        for (int jj = 0; jj < JPL; ++jj) {
            float part = 0.0f;
#pragma unroll
            for (int b = 0; b < BPL; ++b) {
                const int blk = i * JPL + jj + LPR * b;
                const int4* ap = reinterpret_cast<const int4*>(arow + blk * 32 + (PAD ? (blk / 4) * 16 : 0));
                const int4 a0 = ap[0], a1 = ap[1];
                const int av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                int wq[8];
                unpack_block16(raw[b][jj], wq);
                const float dw = half_to_float(dh(b, jj)) * INV16;
                part = fmaf((float)block_dot16(wq, av), dw * adr[blk], part);
            }
            v[jj] = part;
        }
        float s = JPL == 4 ? (v[0] + v[1]) + (v[2] + v[JPL - 1]) : v[0] + v[JPL - 1];
        s += dpp<DPP_QUAD_1032>(s);
        s += dpp<DPP_QUAD_2301>(s);
        return s;
    }
};

// DnQuad with its nibbles unpacked and scales converted ahead of the dot
// products (same arithmetic as DnQuad::dot<PAD>, operation for operation).
template <int NBR>
struct DnQuadUnpacked {
    using Q = DnQuad<NBR>;
    static constexpr int BPL = Q::BPL, JPL = Q::JPL;
    int wq[BPL][JPL][8];
    float dw[BPL][JPL]; // d_w / 16

    __device__ __forceinline__ void unpack(const Q& w)
    {
#pragma unroll
        for (int b = 0; b < BPL; ++b)
#pragma unroll
            for (int jj = 0; jj < JPL; ++jj) {
                dw[b][jj] = half_to_float(w.dh(b, jj)) * INV16;
                unpack_block16(w.raw[b][jj], wq[b][jj]);
#pragma unroll
                for (int m = 0; m < 8; ++m) asm volatile("" : "+v"(wq[b][jj][m]));
            }
    }

    template <bool PAD = false>
    __device__ __forceinline__ float dot(const int8_t* __restrict__ arow, const float* __restrict__ adr, int i) const
    {
        float v[JPL];
#pragma unroll
        for (int jj = 0; jj < JPL; ++jj) {
            float part = 0.0f;
#pragma unroll
            for (int b = 0; b < BPL; ++b) {
                const int blk = i * JPL + jj + Q::LPR * b;
                const int4* ap = reinterpret_cast<const int4*>(arow + blk * 32 + (PAD ? (blk / 4) * 16 : 0));
                const int4 a0 = ap[0], a1 = ap[1];
                const int av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                part = fmaf((float)block_dot16(wq[b][jj], av), dw[b][jj] * adr[blk], part);
            }
            v[jj] = part;
        }
        float s = JPL == 4 ? (v[0] + v[1]) + (v[2] + v[JPL - 1]) : v[0] + v[JPL - 1];
        s += dpp<DPP_QUAD_1032>(s);
        s += dpp<DPP_QUAD_2301>(s);
        return s;
    }
};

// ------------------------------------------------------------------ gate/up + SwiGLU for one output
// Lanes 0-7 of a 16-lane DPP row walk the gate row, lanes 8-15 the matching up
// row; the result h = silu(g) * u is valid in lane 0 of the row.
template <class Row> // GuRow or GuRowUnpacked
__device__ __forceinline__ float swiglu_row(const Row& w, const int8_t* arow, const float* adr, int j)
{
    float part = w.partial(arow, adr, j);
    part = sum_group<8>(part);
    const float up = dpp<DPP_ROW_ROR8>(part); // the other half of the 16-lane row
    const float g = part;
    return g / (1.0f + expf(-g)) * up;
}

// ------------------------------------------------------------------ down walk over the touched experts
// A workgroup owns `slots` output rows of H; each row is walked by LPR lanes.
// It visits every touched expert's down rows for those outputs, DD_CH experts
// per load batch in two named register batches (static indexing), the next
// batch issued before the current one is used, and keeps o per pair in LDS.
constexpr int DD_CH = 8; // experts per load batch

template <int NBR, int CH = DD_CH> // CH experts per batch
struct DnBatch {
    static constexpr int N = CH;
    uint4 raw[CH][DnRow<NBR>::BPL];
    uint16_t dh[CH][DnRow<NBR>::BPL];
};

struct DnWalk {
    const uint8_t* __restrict__ qs; // down_qs
    const uint16_t* __restrict__ d; // down_d
    int H, I;
    const int* list; // active experts, ascending (LDS)
    const int* beg;  // first sorted position of each active expert; beg[U] = number of pairs (LDS)
    const int* pair; // pair id at each sorted position (LDS)
    int U;           // experts this walk visits: list entries a_first + a_step * i, i < U
    int a_first = 0, a_step = 1;
    int n, rs, j;  // output row, its slot in the workgroup, lane within the row
    int slots;     // output rows per workgroup
    float* s_o;    // [pairs][slots] (LDS)
};

template <int NBR, int CH>
__device__ __forceinline__ void dn_issue(DnBatch<NBR, CH>& B, const DnWalk& c, int a0)
{
    DnRow<NBR> wr;
#pragma unroll
    for (int q = 0; q < CH; ++q) {
        // slots past the walk's last expert load nothing (their registers are never read)
        if (a0 + q >= c.U) break;
        const int e = c.list[c.a_first + c.a_step * (a0 + q)];
        const int64_t row = (int64_t)e * c.H + c.n;
        wr.issue(c.qs + row * (c.I / 2), c.d + row * (c.I / 32), c.j, B.raw[q], B.dh[q]);
    }
}

// o of every pair routed to the batch's experts.  The experts' pairs are
// visited in rounds (round r takes the r-th pair of every expert), IW experts
// at a time, so their h loads, dot products and row reductions overlap instead
// of running one expert after another.  hsrc(pos, arow, adr) gives the h row
// at sorted position pos.
// IW: experts in flight per group (register budget); 0 picks CH (CH / 2 at two blocks per lane)
template <int NBR, int IW_ = 0, int CH, typename HSrc>
__device__ __forceinline__ void dn_consume(const DnBatch<NBR, CH>& B, const DnWalk& c, int a0, HSrc hsrc)
{
    using Row = DnRow<NBR>;
    constexpr int IW = IW_ > 0 ? IW_ : (Row::BPL == 1 ? CH : CH / 2);
    static_assert(CH % IW == 0, "interleave width divides the batch");
    int beg[CH], cnt[CH];
    int maxc = 0;
#pragma unroll
    for (int q = 0; q < CH; ++q) {
        const bool live = a0 + q < c.U;
        const int a = c.a_first + c.a_step * (a0 + q);
        beg[q] = live ? c.beg[a] : 0;
        cnt[q] = live ? c.beg[a + 1] - beg[q] : 0;
        maxc = max(maxc, cnt[q]);
    }
    for (int r = 0; r < maxc; ++r) {
#pragma unroll
        for (int q0 = 0; q0 < CH; q0 += IW) {
            if (a0 + q0 >= c.U) break; // a group of slots past the last expert: nothing loaded, nothing to do
            typename Row::Act act[IW];
#pragma unroll
            for (int q = 0; q < IW; ++q) { // clamped to a valid position; unused results are dropped
                const int pos = beg[q0 + q] + min(r, max(cnt[q0 + q] - 1, 0));
                const int8_t* arow;
                const float* adr;
                hsrc(pos, arow, adr);
                Row::load_act(arow, adr, c.j, act[q]);
            }
            __builtin_amdgcn_sched_barrier(0); // every h load of the group goes out first
            float part[IW];
#pragma unroll
            for (int q = 0; q < IW; ++q) {
                // unpack here, every round: an empty asm makes the packed words opaque so the
                // unpacked copies (twice the registers) are not hoisted out of the round loop
                uint4 r4[Row::BPL];
#pragma unroll
                for (int i = 0; i < Row::BPL; ++i) {
                    r4[i] = B.raw[q0 + q][i];
                    asm volatile("" : "+v"(r4[i].x), "+v"(r4[i].y), "+v"(r4[i].z), "+v"(r4[i].w));
                }
                Row w;
                w.finish(r4, B.dh[q0 + q]);
                part[q] = w.dot(act[q]);
            }
#pragma unroll
            for (int q = 0; q < IW; ++q) part[q] = sum_group<Row::LPR>(part[q]);
            if (c.j == 0) {
#pragma unroll
                for (int q = 0; q < IW; ++q)
                    if (r < cnt[q0 + q]) c.s_o[c.pair[beg[q0 + q] + r] * c.slots + c.rs] = part[q];
            }
        }
    }
}

// A holds the loads of the first batch (issued by the caller); so does B of
// the second when b_issued.
template <int NBR, int IW = 0, int CH, typename HSrc>
__device__ __forceinline__ void dn_walk(DnBatch<NBR, CH>& A, DnBatch<NBR, CH>& B, const DnWalk& c, HSrc hsrc,
                                        bool b_issued = false)
{
    for (int a0 = 0; a0 < c.U; a0 += 2 * CH) {
        if (a0 + CH < c.U && !(a0 == 0 && b_issued)) dn_issue<NBR>(B, c, a0 + CH);
        __builtin_amdgcn_sched_barrier(0);
        dn_consume<NBR, IW>(A, c, a0, hsrc);
        if (a0 + 2 * CH < c.U) dn_issue<NBR>(A, c, a0 + 2 * CH);
        __builtin_amdgcn_sched_barrier(0);
        if (a0 + CH < c.U) dn_consume<NBR, IW>(B, c, a0 + CH, hsrc);
    }
}

// y[t][n0 + r] (+)= sum_j wt[t*k + j] * s_o[t*k + j][r], a fixed-order sum (j = 0..k-1)
__device__ __forceinline__ void dn_combine(const float* s_o, int slots, int T, int k, const float* wt,
                                           bool accumulate, float* y, int H, int n0, int tid, int nthreads)
{
    for (int i = tid; i < T * slots; i += nthreads) {
        const int t = i / slots, r = i % slots;
        float acc = 0.0f;
        for (int jj = 0; jj < k; ++jj) acc = fmaf(wt[t * k + jj], s_o[(t * k + jj) * slots + r], acc);
        float* yp = y + (int64_t)t * H + n0 + r;
        *yp = accumulate ? *yp + acc : acc;
    }
}

} // namespace moeq4
