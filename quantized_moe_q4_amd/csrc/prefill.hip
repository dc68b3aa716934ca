// prefill.hip -- top-k routed W4A8 grouped GEMM over resident Q4_0 experts
// (Dutch technical summary "Methodologie 1" of "A 35B Hybrid-Attention
// Mixture-of-Experts Model on a 6GB 2011 GPU": the prefill runs a grouped
// 4-bit GEMM for the MoE; "Methodologie 4": the whole prompt goes through in
// one pass, so each touched expert is read once per tile column and the GEMM
// batch is as large as the prompt allows).
//
// Work decomposition.  Pairs are grouped by expert (moe_q4_route's counting
// sort).  Expert e with c_e pairs owns ceil(c_e / 64) row tiles of up to 64
// rows (two 32-row MFMA m-tiles; a tile with at most 32 live rows runs a
// one-m-tile body).  Row tiles are numbered across experts (an upper bound is
// launched; surplus workgroups exit after a block-wide scan of the per-expert
// counts) and combined with column tiles in an XCD-aware order (pf_tile).  A
// workgroup is 4 waves; each wave multiplies the tile's rows by two 32-column
// B tiles.
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
// acc = fma(t, d_a, acc): two VALU ops per output per block.
//
// Data movement (K in chunks of 4 blocks = 128 columns):
//   A (activation rows, shared by the 4 waves) is staged in LDS, double
//     buffered, with coalesced 16-byte global loads (8 lanes per 128-byte row
//     piece); the next chunk's loads are in flight while the current chunk is
//     multiplied, and are written to the other LDS buffer afterwards.
//   B (weight nibbles, private to a wave) goes straight to registers: per
//     block, lane half h loads the 8 nibble bytes 8h..8h+7 of its row, which
//     are exactly the bytes of its operand.  Two named register batches (even /
//     odd chunk) alternate, so a batch is reloaded right after its last use and
//     no register copies (which would force a wait on the loads) are needed.
//     The weight scales of a chunk (4 fp16 per row) travel in the same batch.
//     (The W4A16 kernels below load 16 bytes per lane and exchange halves with
//     v_permlane32_swap.)
//   d_a of the tile's rows for all K blocks is staged in LDS once.
//
// gate/up kernel: a wave's B tiles are 32 gate rows and the same 32 up rows;
// the epilogue forms h = silu(g) * u, transposes it through LDS so that each
// lane owns one row's 32 values (one Q8_0 block of I) and re-quantises it with
// no cross-lane traffic, writing hq/hd in sorted-pair order.  down kernel: a
// wave's B tiles are 64 rows of W_down; the epilogue stores each pair's row of
// o (unweighted, plain coalesced stores) into the caller's buffer, and the
// combine kernel then forms y = sum over slots of topk_w * o in slot order, so
// y is the same on every run (no atomics).
#include "device.h"

namespace moeq4 {

constexpr int PF_THREADS = 256;
constexpr int PF_TM = 64;               // rows per workgroup tile (two MFMA m-tiles)
constexpr int PF_GU_TM = 96;            // W4A8 gate/up: rows per workgroup tile (three MFMA m-tiles)
constexpr int PF_GU_BN = 128;           // gate/up: columns of I per workgroup (4 waves x 32)
constexpr int PF_DN_BN = 256;           // down: columns of H per workgroup (4 waves x 64)
constexpr int PF_DN_TM = 96;            // W4A8 down: rows per workgroup tile (three MFMA m-tiles)
constexpr int PF_KC = 4;                // K blocks per chunk
constexpr int PF_AROW = PF_KC * 32 + 8; // LDS bytes per staged A row (padding: 2-way bank conflicts)
constexpr int PF_HROW = 33;             // floats per row of the epilogue transpose (conflict-free)
constexpr int MAGIC_BITS = 0x4B400000;  // 1.5 * 2^23
constexpr float MAGIC_F = 12582912.0f;
constexpr int PF_MAX_NB = 64;           // K blocks (K <= 2048)

// SwiGLU of the prefill epilogues, silu(g) * u = g * u / (1 + e^-g), with
// e^-g taken as 2^(-g log2 e) on the hardware base-2 exponential and the
// quotient on the hardware reciprocal: a few ulp in fp32, against two
// correctly rounded library calls per element.  The Q8_0 codes of h that it
// feeds can differ from those of the exact SwiGLU only next to a rounding
// boundary, as any fp32 evaluation of h does.  For g below about -88 the
// exponential overflows to +inf and the result is the limit, -0 * u.
__device__ __forceinline__ float pf_swiglu(float g, float u)
{
    const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

__device__ __forceinline__ int mfma_row(int r, int lane)
{
    return 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
}

// 16-byte B operand (16 (q - 8) in the operand K order) from the 8 nibble bytes of half h.
__device__ __forceinline__ v4i b_operand(uint32_t lo, uint32_t hi)
{
    const uint32_t a = nib_flip(lo), b = nib_flip(hi);
    v4i r;
    r.x = nib_lo16(a);
    r.y = nib_lo16(b);
    r.z = nib_hi16(a);
    r.w = nib_hi16(b);
    return r;
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

// XCD-aware tile order.  Workgroups are dispatched to the 8 XCDs round-robin
// by linear id, and each XCD has its own L2.  The grid is 1D; workgroup L
// takes XCD slot L % 8 and sequence s = L / 8 on it, and row tile
// rt = 8 * (s / ncol) + L % 8 with column tile ct = s % ncol, so all column
// tiles of a row tile (which stage the same activation rows) share one L2,
// and consecutive row tiles spread over the XCDs.  Short launches number the
// row tiles costliest first (pf_locate).  Surplus ids (rt beyond the launched
// bound) exit.
struct TileId {
    int rt, ct;
};

__device__ __forceinline__ TileId pf_tile(int ncol)
{
    const int L = (int)blockIdx.x;
    const int s = L / 8;
    TileId t;
    t.rt = 8 * (s / ncol) + L % 8;
    t.ct = s % ncol;
    return t;
}

static unsigned pf_grid(int ncol, unsigned mt) { return 8u * ((mt + 7u) / 8u) * (unsigned)ncol; }

// Row tiles in falling order of their MFMA m-tiles (a tile of c rows has ceil(c / 32)), so that the costliest come
// first: the first row tiles take the first workgroup slot of every CU, and two of the costliest do not share one
// while lighter ones are left.  Class 0 holds an expert's full tiles, then its partial tile if that has TM / 32
// m-tiles too (row tile mt of the expert is its mt-th in the class); classes 1 and 2 hold the partial tiles with
// one and two m-tiles fewer (row tile n / TM).  Within a class, experts in ascending order.  One block-wide
// scan of the three class counts, as locate_expert does for one.
template <int TM>
__device__ __forceinline__ int pf_class_count(int n, int k)
{
    constexpr int MWX = TM / 32;
    const int full = n / TM, mwp = (n % TM + 31) / 32; // m-tiles of the partial tile (0: none)
    if (k == 0) return full + (mwp == MWX ? 1 : 0);
    return (mwp > 0 && mwp == MWX - k) ? 1 : 0;
}

template <int NT, int TM>
__device__ bool pf_locate_sorted(const int32_t* __restrict__ off, int E, int target, int& e_out, int& mt_out)
{
    constexpr int NWAVES = NT / WAVE;
    __shared__ int s_wave[NWAVES][3];
    __shared__ int s_res[2];
    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    const int ept = (E + NT - 1) / NT; // experts per thread, contiguous
    const int e0 = tid * ept;
    int local[3] = {0, 0, 0};
    for (int i = 0; i < ept; ++i) {
        const int e = e0 + i;
        if (e < E) {
            const int n = off[e + 1] - off[e];
#pragma unroll
            for (int k = 0; k < 3; ++k) local[k] += pf_class_count<TM>(n, k);
        }
    }
    int inc[3] = {local[0], local[1], local[2]}; // inclusive scans within the wave
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int o = __shfl_up(inc[k], d, WAVE);
            if (lane >= d) inc[k] += o;
        }
    }
    if (tid == 0) {
        s_res[0] = -1;
        s_res[1] = 0;
    }
    if (lane == WAVE - 1)
#pragma unroll
        for (int k = 0; k < 3; ++k) s_wave[wv][k] = inc[k];
    __syncthreads();
    int base[3] = {0, 0, 0}, total[3] = {0, 0, 0};
    for (int w = 0; w < NWAVES; ++w)
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            if (w < wv) base[k] += s_wave[w][k];
            total[k] += s_wave[w][k];
        }
    int t = target, k = 0; // the class holding the target, and its index there (k = 3: a surplus workgroup)
    while (k < 3 && t >= total[k]) t -= total[k++];
    if (k < 3) {
        int run = base[k] + inc[k] - local[k]; // exclusive prefix of this thread in class k
        if (t >= run && t < run + local[k]) {
            for (int i = 0; i < ept; ++i) {
                const int e = e0 + i;
                if (e >= E) break;
                const int n = off[e + 1] - off[e];
                const int v = pf_class_count<TM>(n, k);
                if (t < run + v) {
                    s_res[0] = e;
                    s_res[1] = k == 0 ? t - run : n / TM;
                    break;
                }
                run += v;
            }
        }
    }
    __syncthreads();
    e_out = s_res[0];
    mt_out = s_res[1];
    return e_out >= 0;
}

// Launches of up to PF_LPT_MAX_WG workgroups (four rounds of two per CU on 256 CUs) number the row tiles costliest
// first, since there the slowest CU sets the time.  Longer launches balance themselves as workgroups finish, and
// keep the experts' order, in which an expert's tiles (reading the same weights) run close together in time.
constexpr unsigned PF_LPT_MAX_WG = 2048;

// Locate this workgroup's (expert, row tile of TM rows); false for surplus workgroups.
template <int TM = PF_TM>
__device__ __forceinline__ bool pf_locate(const int32_t* __restrict__ off, int E, int rt, TileRows& tr)
{
    int e, mt;
    const bool found = gridDim.x <= PF_LPT_MAX_WG
                           ? pf_locate_sorted<PF_THREADS, TM>(off, E, rt, e, mt)
                           : locate_expert<PF_THREADS>(off, E, rt, [](int c) { return (c + TM - 1) / TM; }, e, mt);
    if (!found) return false;
    tr.e = e;
    tr.beg = off[e];
    tr.m0 = mt * TM;
    const int left = off[e + 1] - tr.beg - tr.m0;
    tr.mcount = left < TM ? left : TM;
    return true;
}

// The down kernels' output rows: offset pair * H of each tile row's row of o
// (-1: padding), read once per tile by the first PF_TM threads.  The caller's
// K loop starts with a barrier, so the epilogue sees them.  Offsets rather
// than pointers: an address read back from LDS loses its address space, and
// the stores would become flat ones.
template <int TM = PF_TM>
__device__ __forceinline__ void pf_out_rows(const TileRows& tr, const int32_t* __restrict__ sorted, int T, int k,
                                            int H, int64_t* s_ooff)
{
    const int tid = threadIdx.x;
    if (tid >= TM) return;
    int64_t oo = -1;
    if (tid < tr.mcount) {
        const int pair = sorted[tr.beg + tr.m0 + tid];
        if (pair / k < T) oo = (int64_t)pair * H;
    }
    s_ooff[tid] = oo;
}

// ------------------------------------------------------------------ operand staging
// One chunk (4 blocks) of the wave's two B tiles: per tile two 16-byte pieces
// (block pairs, lane half h holding block 2p+h) and the 4 fp16 scales.
struct BChunk {
    uint4 q[2][2]; // [tile][pair]
    uint2 s[2];    // [tile]
};

struct BRows {
    const uint8_t* q[2];  // nibble row of each tile, + 16 bytes for lane half 1
    const uint16_t* d[2]; // scale row of each tile
};

__device__ __forceinline__ void load_b(BChunk& X, const BRows& br, int c)
{
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int p = 0; p < 2; ++p) X.q[t][p] = *reinterpret_cast<const uint4*>(br.q[t] + 64 * c + 32 * p);
        X.s[t] = *reinterpret_cast<const uint2*>(br.d[t] + PF_KC * c);
    }
}

// The W4A8 kernels' batch: per tile and block the 8 nibble bytes 8h..8h+7 of
// the lane's row (lane half h), which are exactly its B operand bytes, so no
// cross-lane exchange (whose in-place operands would force copies of the
// loop-carried batch, and with them early waits on the prefetch) is needed.
struct BChunk8 {
    uint2 q[2][PF_KC]; // [tile][block]
    uint2 s[2];        // [tile]: the 4 fp16 scales
};

// br.q[t] points at byte 8h of the row (lane half h)
__device__ __forceinline__ void load_b8(BChunk8& X, const BRows& br, int c)
{
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int u = 0; u < PF_KC; ++u) X.q[t][u] = *reinterpret_cast<const uint2*>(br.q[t] + 64 * c + 16 * u);
        X.s[t] = *reinterpret_cast<const uint2*>(br.d[t] + PF_KC * c);
    }
}

// The tile's A rows, coalesced: 8 lanes per 128-byte row piece of a chunk,
// NP = TM * 8 / PF_THREADS 16-byte pieces per thread (64 rows: 2, 96 rows: 3).
template <int NP>
struct AChunk {
    int4 v[NP];
};

template <int NP>
__device__ __forceinline__ void load_a(AChunk<NP>& X, const int8_t* const (&aptr)[NP], int c)
{
#pragma unroll
    for (int i = 0; i < NP; ++i) X.v[i] = *reinterpret_cast<const int4*>(aptr[i] + PF_KC * 32 * c);
}

// aoff: LDS offset of the thread's first piece; piece i lies 32 * i rows below
// it (thread t takes row t / 8 + 32 i, piece t % 8), a constant the stores
// carry as an immediate.
template <int NP>
__device__ __forceinline__ void store_a(const AChunk<NP>& X, uint8_t* s_a, int aoff)
{
    // opaque to the optimiser: the few address adds are redone at each store
    // rather than hoisted out of the K loop into registers of their own, which
    // the three-m-tile body cannot spare
    asm volatile("" : "+v"(aoff));
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        // 8-byte stores: the padded row pitch is 8- but not 16-byte aligned
        uint8_t* d = s_a + aoff + i * (PF_THREADS / 8) * PF_AROW;
        *reinterpret_cast<int2*>(d) = make_int2(X.v[i].x, X.v[i].y);
        *reinterpret_cast<int2*>(d + 8) = make_int2(X.v[i].z, X.v[i].w);
    }
}

// Multiply one chunk: MW m-tiles of the LDS A stage x the wave's two B tiles,
// 4 blocks, accumulated in fp32.  `dump(mi, t, r, b, isum)` receives every
// exact block dot (a no-op outside the inspection variant).
//
// The chunk is a sequence of 4 * MW steps (block u, m-tile mi), u-major, each
// two MFMAs (tiles 0 and 1) and their 2 x 16 scale FMAs per lane.  The steps
// are software-pipelined in source order: a tile's MFMA for step s + 1 follows
// that tile's FMAs of step s, so it runs while the other tile's FMAs issue
// and its result is ready when needed.  Same registers: each tile's product
// is overwritten only after its last read.
template <int MW, int TM, typename Dump>
__device__ __forceinline__ void mma_chunk(const uint8_t* s_a, const BChunk8& X, int c, const float (*s_da)[TM],
                                          const v16i& cmag, float (&acc)[MW][2][16], Dump& dump)
{
    const int lane = threadIdx.x % WAVE, h = lane / 32, col = lane % 32;
    constexpr int S = PF_KC * MW;
    auto a_op = [&](int st) {
        const int u = st / MW, mi = st % MW;
        const uint8_t* ap = s_a + (32 * mi + col) * PF_AROW + 32 * u + 8 * h;
        const int2 a0 = *reinterpret_cast<const int2*>(ap);
        const int2 a1 = *reinterpret_cast<const int2*>(ap + 16);
        return v4i{a0.x, a0.y, a1.x, a1.y};
    };
    auto prep = [&](int u, v4i (&Bo)[2], float (&dwo)[2], float (&nwo)[2]) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            Bo[t] = b_operand(X.q[t][u].x, X.q[t][u].y);
            const uint32_t pr = u < 2 ? X.s[t].x : X.s[t].y;
            dwo[t] = half_to_float((uint16_t)(pr >> (16 * (u % 2)))) * INV16;
            nwo[t] = -MAGIC_F * dwo[t];
        }
    };
    v4i B[2], Bn[2];
    float dw[2], nw[2], dwn[2], nwn[2];
    prep(0, B, dw, nw);
    v4i A = a_op(0);
    v16i D0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B[0], cmag, 0, 0, 0);
    v16i D1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B[1], cmag, 0, 0, 0);
#pragma unroll
    for (int st = 0; st < S; ++st) {
        const int u = st / MW, mi = st % MW, b = PF_KC * c + u;
        const bool more = st + 1 < S, turn = more && (st + 1) % MW == 0; // next step starts a new block
        float da[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 v = *reinterpret_cast<const float4*>(&s_da[b][32 * mi + 8 * g + 4 * h]);
            da[4 * g + 0] = v.x;
            da[4 * g + 1] = v.y;
            da[4 * g + 2] = v.z;
            da[4 * g + 3] = v.w;
        }
        if (more) A = a_op(st + 1);
        if (turn) prep(u + 1, Bn, dwn, nwn);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc[mi][0][r] = fmaf(fmaf(__int_as_float(D0[r]), dw[0], nw[0]), da[r], acc[mi][0][r]);
            dump(mi, 0, r, b, (D0[r] - MAGIC_BITS) >> 4);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (more) D0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, turn ? Bn[0] : B[0], cmag, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            acc[mi][1][r] = fmaf(fmaf(__int_as_float(D1[r]), dw[1], nw[1]), da[r], acc[mi][1][r]);
            dump(mi, 1, r, b, (D1[r] - MAGIC_BITS) >> 4);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (more) D1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, turn ? Bn[1] : B[1], cmag, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (turn) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                B[t] = Bn[t];
                dw[t] = dwn[t];
                nw[t] = nwn[t];
            }
        }
    }
}

// The whole K loop for one wave: chunks alternate between the two LDS A
// buffers and the two register B batches (see the header comment).  The
// loop's last statement is a barrier that follows every read of the A stages
// and of s_da, so the caller may reuse that memory afterwards.
template <int MW, int TM, int NP, typename Dump>
__device__ __forceinline__ void gemm_loop(int NC, const int8_t* const (&aptr)[NP], int aoff,
                                          uint8_t* s_a0, uint8_t* s_a1, const BRows& br,
                                          const float (*s_da)[TM], float (&acc)[MW][2][16], Dump dump)
{
    const v16i cmag = magic_c();
#pragma unroll
    for (int mi = 0; mi < MW; ++mi)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][t][r] = 0.0f;
    AChunk<NP> ar;
    BChunk8 Bx, By;
    load_a(ar, aptr, 0);
    load_b8(Bx, br, 0);
    store_a(ar, s_a0, aoff);
    __syncthreads();
    for (int c = 0; c < NC; c += 2) {
        load_a(ar, aptr, min(c + 1, NC - 1));
        load_b8(By, br, min(c + 1, NC - 1));
        __builtin_amdgcn_sched_barrier(0); // the next chunk's loads stay ahead of this chunk's math
        mma_chunk<MW, TM>(s_a0, Bx, c, s_da, cmag, acc, dump);
        store_a(ar, s_a1, aoff);
        __syncthreads();
        load_a(ar, aptr, min(c + 2, NC - 1)); // clamped: a repeated load at the end is harmless
        load_b8(Bx, br, min(c + 2, NC - 1));
        __builtin_amdgcn_sched_barrier(0);
        mma_chunk<MW, TM>(s_a1, By, c + 1, s_da, cmag, acc, dump);
        store_a(ar, s_a0, aoff);
        __syncthreads();
    }
}

// ------------------------------------------------------------------ gate/up
template <bool DUMP>
__global__ __launch_bounds__(PF_THREADS, 2) void prefill_gateup_kernel(
    const uint8_t* __restrict__ gate_qs, const uint8_t* __restrict__ up_qs, const uint16_t* __restrict__ gate_d,
    const uint16_t* __restrict__ up_d, int E, int H, int I, const int8_t* __restrict__ xq,
    const float* __restrict__ xd, int T, int k, const int32_t* __restrict__ off, const int32_t* __restrict__ sorted,
    int8_t* __restrict__ hq, float* __restrict__ hd, int32_t* __restrict__ dump)
{
    constexpr int TM = PF_GU_TM, NP = TM * 8 / PF_THREADS;
    // The K loop's stages (activation scales [block][row] and the two A
    // buffers) and the epilogue's h transpose share one LDS region: the loop
    // ends with a barrier after its last read of the stages.
    constexpr int STAGE_BYTES = PF_MAX_NB * TM * 4 + 2 * TM * PF_AROW;
    constexpr int H_BYTES = PF_THREADS / WAVE * TM * PF_HROW * 4;
    __shared__ __align__(16) uint8_t s_mem[STAGE_BYTES > H_BYTES ? STAGE_BYTES : H_BYTES];
    float(*s_da)[TM] = reinterpret_cast<float(*)[TM]>(s_mem);
    uint8_t* s_a0 = s_mem + PF_MAX_NB * TM * 4;
    uint8_t* s_a1 = s_a0 + TM * PF_AROW;
    float(*s_h)[TM][PF_HROW] = reinterpret_cast<float(*)[TM][PF_HROW]>(s_mem);
    __shared__ int s_tok[TM];

    const TileId ti = pf_tile(I / PF_GU_BN);
    TileRows tr;
    if (!pf_locate<TM>(off, E, ti.rt, tr)) return;
    const int NB = H / 32;
    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    const int h = lane / 32, col = lane % 32;

    if (tid < TM) {
        int t = 0;
        if (tid < tr.mcount) t = sorted[tr.beg + tr.m0 + tid] / k;
        s_tok[tid] = t < T ? t : T - 1;
    }
    __syncthreads();
    for (int i = tid; i < NB * TM; i += PF_THREADS) {
        const int b = i / TM, m = i % TM;
        s_da[b][m] = m < tr.mcount ? xd[(int64_t)s_tok[m] * NB + b] : 0.0f;
    }
    // this thread's NP 16-byte pieces of every staged A chunk
    const int8_t* aptr[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int idx = tid + PF_THREADS * i, row = idx / 8, piece = idx % 8;
        aptr[i] = xq + (int64_t)s_tok[row] * H + 16 * piece;
    }
    const int aoff = (tid / 8) * PF_AROW + 16 * (tid % 8);

    const int n = ti.ct * PF_GU_BN + wv * 32 + col;
    const int64_t wrow = (int64_t)tr.e * I + n;
    BRows br;
    br.q[0] = gate_qs + wrow * (H / 2) + 8 * h;
    br.q[1] = up_qs + wrow * (H / 2) + 8 * h;
    br.d[0] = gate_d + wrow * NB;
    br.d[1] = up_d + wrow * NB;
    const int NC = NB / PF_KC;

    auto body = [&](auto mw) {
        constexpr int MW = decltype(mw)::value;
        float acc[MW][2][16];
        gemm_loop<MW, TM, NP>(NC, aptr, aoff, s_a0, s_a1, br, s_da, acc, [&](int mi, int t, int r, int b, int isum) {
            if (DUMP) {
                const int m = 32 * mi + mfma_row(r, lane);
                if (m < tr.mcount) dump[(((int64_t)(tr.beg + tr.m0 + m) * 2 + t) * I + n) * NB + b] = isum;
            }
        });
        // h = silu(g) * u, transposed through LDS: lane `row` then owns row `row`
#pragma unroll
        for (int mi = 0; mi < MW; ++mi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float g = acc[mi][0][r];
                s_h[wv][32 * mi + mfma_row(r, lane)][col] = pf_swiglu(g, acc[mi][1][r]);
            }
    };
    if (tr.mcount > 64)
        body(std::integral_constant<int, 3>());
    else if (tr.mcount > 32)
        body(std::integral_constant<int, 2>());
    else
        body(std::integral_constant<int, 1>());
    __syncthreads();

    // Q8_0 re-quantisation: one row of the wave's 32 columns (one block of I) per lane and pass
    for (int m = lane; m < tr.mcount; m += WAVE) {
        float v[32];
        float amax = 0.0f;
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            v[c] = s_h[wv][m][c];
            amax = fmaxf(amax, fabsf(v[c]));
        }
        // d = amax / 127 as everywhere; the codes take one correctly rounded
        // 1/d per row and a product per element (within an ulp of v / d, so a
        // code can differ from rint(v / d) only next to a rounding boundary)
        const float d = amax / 127.0f;
        const float inv = d > 0.0f ? 1.0f / d : 0.0f;
        auto code = [&](float x) {
            return (uint32_t)((int)fminf(fmaxf(rintf(x * inv), -127.0f), 127.0f) & 0xFF);
        };
        uint32_t pk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            pk[i] = code(v[4 * i]) | (code(v[4 * i + 1]) << 8) | (code(v[4 * i + 2]) << 16) | (code(v[4 * i + 3]) << 24);
        const int64_t pos = tr.beg + tr.m0 + m;
        const int n0 = ti.ct * PF_GU_BN + wv * 32;
        uint4* dst = reinterpret_cast<uint4*>(hq + pos * I + n0);
        dst[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        dst[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
        hd[pos * (I / 32) + n0 / 32] = d;
    }
}

// ------------------------------------------------------------------ down (rows of o)
template <bool DUMP>
__global__ __launch_bounds__(PF_THREADS, 2) void prefill_down_kernel(
    const uint8_t* __restrict__ down_qs, const uint16_t* __restrict__ down_d, int E, int H, int I,
    const int8_t* __restrict__ hq, const float* __restrict__ hd, int T, int k, const int32_t* __restrict__ off,
    const int32_t* __restrict__ sorted, float* __restrict__ o, int32_t* __restrict__ dump)
{
    constexpr int TM = PF_DN_TM, NP = TM * 8 / PF_THREADS;
    __shared__ __align__(16) float s_da[PF_MAX_NB / 2][TM];
    __shared__ __align__(16) uint8_t s_a[2][TM * PF_AROW];
    __shared__ int64_t s_ooff[TM]; // offset of each tile row's row of o (-1: no output)
    const TileId ti = pf_tile(H / PF_DN_BN);
    TileRows tr;
    if (!pf_locate<TM>(off, E, ti.rt, tr)) return;
    const int NB = I / 32;
    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    const int h = lane / 32, col = lane % 32;
    const int64_t pos0 = tr.beg + tr.m0;

    if (!DUMP) pf_out_rows<TM>(tr, sorted, T, k, H, s_ooff);
    for (int i = tid; i < NB * TM; i += PF_THREADS) {
        const int b = i / TM, m = i % TM;
        s_da[b][m] = m < tr.mcount ? hd[(pos0 + m) * NB + b] : 0.0f;
    }
    const int8_t* aptr[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int idx = tid + PF_THREADS * i, row = idx / 8, piece = idx % 8;
        aptr[i] = hq + (pos0 + (row < tr.mcount ? row : 0)) * I + 16 * piece;
    }
    const int aoff = (tid / 8) * PF_AROW + 16 * (tid % 8);

    const int n0 = ti.ct * PF_DN_BN + wv * 64; // this wave's 64 columns: two 32-wide B tiles
    const int64_t wrow = (int64_t)tr.e * H + n0 + col;
    BRows br;
    br.q[0] = down_qs + wrow * (I / 2) + 8 * h;
    br.q[1] = down_qs + (wrow + 32) * (I / 2) + 8 * h;
    br.d[0] = down_d + wrow * NB;
    br.d[1] = down_d + (wrow + 32) * NB;
    const int NC = NB / PF_KC;

    auto body = [&](auto mw) {
        constexpr int MW = decltype(mw)::value;
        float acc[MW][2][16];
        gemm_loop<MW, TM, NP>(NC, aptr, aoff, s_a[0], s_a[1], br, s_da, acc, [&](int mi, int t, int r, int b, int isum) {
            if (DUMP) {
                const int m = 32 * mi + mfma_row(r, lane);
                if (m < tr.mcount) dump[((int64_t)(tr.beg + tr.m0 + m) * H + n0 + 32 * t + col) * NB + b] = isum;
            }
        });
        if (DUMP) return; // the inspection variant writes no o
        // the pair's row of o, plain stores (s_ooff was written before the K loop's first barrier); the combine
        // sums each token's k rows in slot order
#pragma unroll
        for (int mi = 0; mi < MW; ++mi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 32 * mi + mfma_row(r, lane);
                const int64_t oo = s_ooff[m];
                if (oo >= 0) {
                    float* orow = o + oo + n0 + col;
                    orow[0] = acc[mi][0][r];
                    orow[32] = acc[mi][1][r];
                }
            }
    };
    if (tr.mcount > 64)
        body(std::integral_constant<int, 3>());
    else if (tr.mcount > 32)
        body(std::integral_constant<int, 2>());
    else
        body(std::integral_constant<int, 1>());
}

// ------------------------------------------------------------------ launchers
// The K loop takes chunks in pairs and the column tiles must cover I and H.
static bool pf_shape_ok(int H, int I)
{
    return H % (2 * PF_KC * 32) == 0 && I % (2 * PF_KC * 32) == 0 && H / 32 <= PF_MAX_NB &&
           I / 32 <= PF_MAX_NB / 2 && I % PF_GU_BN == 0 && H % PF_DN_BN == 0;
}

// An upper bound on the row tiles of TM rows over all experts: sum ceil(c_e / TM) <= P / TM + (experts with pairs).
template <int TM = PF_TM>
static unsigned pf_tiles_bound(int P, int E)
{
    const int nonempty = P < E ? P : E;
    return (unsigned)((P + TM - 1) / TM + nonempty);
}

hipError_t launch_combine(const float* o, const float* topk_w, int T, int k, int H, bool accumulate, float* y,
                          hipStream_t s);

hipError_t launch_prefill(const uint8_t* gate_qs, const uint8_t* up_qs, const uint8_t* down_qs,
                          const uint16_t* gate_d, const uint16_t* up_d, const uint16_t* down_d, int E, int H, int I,
                          const int8_t* xq, const float* xd, int T, int k, const float* topk_w, const int32_t* off,
                          const int32_t* sorted, bool accumulate, float* y, int8_t* hq, float* hd, float* o,
                          hipStream_t s)
{
    if (T == 0) return hipSuccess;
    if (!pf_shape_ok(H, I)) return hipErrorInvalidValue;
    const int P = T * k;
    const unsigned mt = pf_tiles_bound<PF_DN_TM>(P, E), mt_gu = pf_tiles_bound<PF_GU_TM>(P, E);
    if (!o) return hipErrorInvalidValue;
    // the down kernel stores each pair's row of o and the combine forms y in slot order (no atomics, the same y
    // on every run)
    prefill_gateup_kernel<false><<<dim3(pf_grid(I / PF_GU_BN, mt_gu)), PF_THREADS, 0, s>>>(
        gate_qs, up_qs, gate_d, up_d, E, H, I, xq, xd, T, k, off, sorted, hq, hd, nullptr);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    prefill_down_kernel<false><<<dim3(pf_grid(H / PF_DN_BN, mt)), PF_THREADS, 0, s>>>(
        down_qs, down_d, E, H, I, hq, hd, T, k, off, sorted, o, nullptr);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_combine(o, topk_w, T, k, H, accumulate, y, s);
}

hipError_t launch_prefill_dots(const uint8_t* gate_qs, const uint8_t* up_qs, const uint8_t* down_qs,
                               const uint16_t* gate_d, const uint16_t* up_d, const uint16_t* down_d, int E, int H,
                               int I, const int8_t* xq, const float* xd, int T, int k, const int32_t* off,
                               const int32_t* sorted, int which, int8_t* hq, float* hd, int32_t* dump, hipStream_t s)
{
    if (T == 0) return hipSuccess;
    if (!pf_shape_ok(H, I)) return hipErrorInvalidValue;
    const int P = T * k;
    const unsigned mt = pf_tiles_bound<PF_DN_TM>(P, E), mt_gu = pf_tiles_bound<PF_GU_TM>(P, E);
    if (which == 0) {
        // writes hq/hd as a side effect, exactly as the production launch does
        prefill_gateup_kernel<true><<<dim3(pf_grid(I / PF_GU_BN, mt_gu)), PF_THREADS, 0, s>>>(
            gate_qs, up_qs, gate_d, up_d, E, H, I, xq, xd, T, k, off, sorted, hq, hd, dump);
    } else {
        // no o: the dump epilogue writes only the dots
        prefill_down_kernel<true><<<dim3(pf_grid(H / PF_DN_BN, mt)), PF_THREADS, 0, s>>>(
            down_qs, down_d, E, H, I, hq, hd, T, k, off, sorted, nullptr, dump);
    }
    return hipGetLastError();
}

// ================================================================== W4A16 prefill
// The same packed experts with 16-bit activations: the layer input and h stay
// fp16 instead of Q8_0 (the pages tie 8-bit activations to decode; this is the
// prefill variant whose activations are not quantised).  The weights are
// dequantised in registers to fp16 with the scale folded in,
// w = fl16((q - 8) * d) (q - 8 is exact in fp16, one rounding for the product),
// and v_mfma_f32_32x32x16_f16 accumulates in fp32 across all of K, so there is no
// per-block scaling epilogue: two MFMAs (K = 16 each) cover one Q4_0 block.
//
// K order.  A lane's 8-element fp16 operand for k-slice s (0: elements 0-15 of
// the block, 1: 16-31) and lane half h holds elements 16s + 8h + j.  B is built
// from the lane's 8 nibble bytes 8h..8h+7 (low nibbles for s = 0, high for
// s = 1) two bytes at a time ((w & 0x000F000F) | 0x64006400 is the fp16 pair
// 1024 + q of bytes 0 and 2), so within every group of 8 the operand carries
// elements 0,2,1,3,4,6,5,7 (a16_pos swaps bits 0 and 1 of the index).  The
// activations are stored in HBM (x16, h16) and LDS in that same order; the
// MFMA's sum over K does not depend on the order, only on A and B agreeing.
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));

constexpr int PF_A16ROW = PF_KC * 32 + 8; // halves per staged A row (272 bytes: 16-byte aligned, banks spread)

__device__ __forceinline__ int a16_pos(int i) // position of element i within the stored order
{
    return (i & ~3) | ((i & 1) << 1) | ((i >> 1) & 1);
}

// x [T][H] fp32 -> x16 [T][H] fp16 (nearest, ties to even) in the stored order; 8 elements per thread
__global__ __launch_bounds__(256) void a16_convert_kernel(const float* __restrict__ x, int64_t n8,
                                                          _Float16* __restrict__ x16)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const float4 a = reinterpret_cast<const float4*>(x)[2 * i];
    const float4 b = reinterpret_cast<const float4*>(x)[2 * i + 1];
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    v8h o;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[a16_pos(j)] = (_Float16)v[j];
    reinterpret_cast<v8h*>(x16)[i] = o;
}

// fp16 pair (q - 8) * d of the nibbles in bits 0-3 and 16-19 of w
__device__ __forceinline__ uint32_t a16_pair(uint32_t w, h2v d2)
{
    const h2v t = __builtin_bit_cast(h2v, (w & 0x000F000Fu) | 0x64006400u); // 1024 + q, exact
    const h2v m = {(_Float16)1032.0f, (_Float16)1032.0f};
    return __builtin_bit_cast(uint32_t, (h2v)((t - m) * d2));
}

// the lane's B operands of one block: lo/hi = its nibble bytes 8h..8h+3 / 8h+4..8h+7
__device__ __forceinline__ void a16_b_operands(uint32_t lo, uint32_t hi, h2v d2, v8h (&B)[2])
{
    const uint32_t w0[4] = {a16_pair(lo, d2), a16_pair(lo >> 8, d2), a16_pair(hi, d2), a16_pair(hi >> 8, d2)};
    const uint32_t w1[4] = {a16_pair(lo >> 4, d2), a16_pair(lo >> 12, d2), a16_pair(hi >> 4, d2),
                            a16_pair(hi >> 12, d2)};
    B[0] = __builtin_bit_cast(v8h, make_uint4(w0[0], w0[1], w0[2], w0[3]));
    B[1] = __builtin_bit_cast(v8h, make_uint4(w1[0], w1[1], w1[2], w1[3]));
}

// One chunk (4 blocks) of the A stage times the wave's two B tiles, MW m-tiles, fp32 accumulation.
template <int MW>
__device__ __forceinline__ void mma_chunk_a16(const _Float16* s_a, const BChunk& X, v16f (&acc)[MW][2])
{
    const int lane = threadIdx.x % WAVE, h = lane / 32, col = lane % 32;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        uint32_t lo[2][2], hi[2][2]; // [tile][block of the pair]: bytes 8h..8h+7 of blocks 2p, 2p+1
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const auto s0 = __builtin_amdgcn_permlane32_swap(X.q[t][p].x, X.q[t][p].z, false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(X.q[t][p].y, X.q[t][p].w, false, false);
            lo[t][0] = s0[0];
            lo[t][1] = s0[1];
            hi[t][0] = s1[0];
            hi[t][1] = s1[1];
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int u = 2 * p + q; // block within the chunk
            v8h B[2][2];             // [tile][k-slice]
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint32_t pr = p == 0 ? X.s[t].x : X.s[t].y;
                const uint16_t dbits = (uint16_t)(pr >> (16 * q));
                const _Float16 d = __builtin_bit_cast(_Float16, dbits);
                const h2v d2 = {d, d};
                a16_b_operands(lo[t][q], hi[t][q], d2, B[t]);
            }
#pragma unroll
            for (int mi = 0; mi < MW; ++mi)
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) {
                    const v8h A =
                        *reinterpret_cast<const v8h*>(s_a + (32 * mi + col) * PF_A16ROW + 32 * u + 16 * sl + 8 * h);
                    acc[mi][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B[0][sl], acc[mi][0], 0, 0, 0);
                    acc[mi][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B[1][sl], acc[mi][1], 0, 0, 0);
                }
        }
    }
}

// The tile's A rows for one chunk: 64 rows x 256 bytes = 1024 pieces of 16 bytes, 4 per thread.
struct AChunk16 {
    uint4 v[4];
};

__device__ __forceinline__ void load_a16(AChunk16& X, const _Float16* const (&aptr)[4], int c)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) X.v[i] = *reinterpret_cast<const uint4*>(aptr[i] + PF_KC * 32 * c);
}

__device__ __forceinline__ void store_a16(const AChunk16& X, _Float16* s_a, const int (&aoff)[4])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(s_a + aoff[i]) = X.v[i];
}

template <int MW>
__device__ __forceinline__ void gemm_loop_a16(int NC, const _Float16* const (&aptr)[4], const int (&aoff)[4],
                                              _Float16* s_a0, _Float16* s_a1, const BRows& br, v16f (&acc)[MW][2])
{
#pragma unroll
    for (int mi = 0; mi < MW; ++mi)
#pragma unroll
        for (int t = 0; t < 2; ++t) acc[mi][t] = v16f{};
    AChunk16 ar;
    BChunk Bx, By;
    load_a16(ar, aptr, 0);
    load_b(Bx, br, 0);
    store_a16(ar, s_a0, aoff);
    __syncthreads();
    for (int c = 0; c < NC; c += 2) {
        load_a16(ar, aptr, min(c + 1, NC - 1));
        load_b(By, br, min(c + 1, NC - 1));
        __builtin_amdgcn_sched_barrier(0); // the next chunk's loads stay ahead of this chunk's math
        mma_chunk_a16<MW>(s_a0, Bx, acc);
        store_a16(ar, s_a1, aoff);
        __syncthreads();
        load_a16(ar, aptr, min(c + 2, NC - 1)); // clamped: a repeated load at the end is harmless
        load_b(Bx, br, min(c + 2, NC - 1));
        __builtin_amdgcn_sched_barrier(0);
        mma_chunk_a16<MW>(s_a1, By, acc);
        store_a16(ar, s_a0, aoff);
        __syncthreads();
    }
}

__global__ __launch_bounds__(PF_THREADS, 2) void prefill_a16_gateup_kernel(
    const uint8_t* __restrict__ gate_qs, const uint8_t* __restrict__ up_qs, const uint16_t* __restrict__ gate_d,
    const uint16_t* __restrict__ up_d, int E, int H, int I, const _Float16* __restrict__ x16, int T, int k,
    const int32_t* __restrict__ off, const int32_t* __restrict__ sorted, _Float16* __restrict__ h16)
{
    __shared__ __align__(16) _Float16 s_a[2][PF_TM * PF_A16ROW];
    __shared__ int s_tok[PF_TM];
    const TileId ti = pf_tile(I / PF_GU_BN);
    TileRows tr;
    if (!pf_locate(off, E, ti.rt, tr)) return;
    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    const int h = lane / 32, col = lane % 32;
    if (tid < PF_TM) {
        int t = 0;
        if (tid < tr.mcount) t = sorted[tr.beg + tr.m0 + tid] / k;
        s_tok[tid] = t < T ? t : T - 1;
    }
    __syncthreads();
    const _Float16* aptr[4];
    int aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + PF_THREADS * i, row = idx / 16, piece = idx % 16;
        aptr[i] = x16 + (int64_t)s_tok[row] * H + 8 * piece;
        aoff[i] = row * PF_A16ROW + 8 * piece;
    }
    const int n = ti.ct * PF_GU_BN + wv * 32 + col;
    const int64_t wrow = (int64_t)tr.e * I + n;
    BRows br;
    br.q[0] = gate_qs + wrow * (H / 2) + 16 * h;
    br.q[1] = up_qs + wrow * (H / 2) + 16 * h;
    br.d[0] = gate_d + wrow * (H / 32);
    br.d[1] = up_d + wrow * (H / 32);
    const int NC = H / (PF_KC * 32);
    const int nst = (n & ~7) | a16_pos(n & 7); // h16 is stored in the operand order
    auto body = [&](auto mw) {
        constexpr int MW = decltype(mw)::value;
        v16f acc[MW][2];
        gemm_loop_a16<MW>(NC, aptr, aoff, s_a[0], s_a[1], br, acc);
#pragma unroll
        for (int mi = 0; mi < MW; ++mi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 32 * mi + mfma_row(r, lane);
                if (m < tr.mcount) {
                    const float g = acc[mi][0][r], u = acc[mi][1][r];
                    h16[(int64_t)(tr.beg + tr.m0 + m) * I + nst] = (_Float16)pf_swiglu(g, u);
                }
            }
    };
    if (tr.mcount > 32)
        body(std::integral_constant<int, 2>());
    else
        body(std::integral_constant<int, 1>());
}

__global__ __launch_bounds__(PF_THREADS, 2) void prefill_a16_down_kernel(
    const uint8_t* __restrict__ down_qs, const uint16_t* __restrict__ down_d, int E, int H, int I,
    const _Float16* __restrict__ h16, int T, int k, const int32_t* __restrict__ off,
    const int32_t* __restrict__ sorted, float* __restrict__ o)
{
    __shared__ __align__(16) _Float16 s_a[2][PF_TM * PF_A16ROW];
    __shared__ int64_t s_ooff[PF_TM];
    const TileId ti = pf_tile(H / PF_DN_BN);
    TileRows tr;
    if (!pf_locate(off, E, ti.rt, tr)) return;
    const int tid = threadIdx.x, lane = tid % WAVE, wv = tid / WAVE;
    const int h = lane / 32, col = lane % 32;
    const int64_t pos0 = tr.beg + tr.m0;
    pf_out_rows(tr, sorted, T, k, H, s_ooff);
    const _Float16* aptr[4];
    int aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + PF_THREADS * i, row = idx / 16, piece = idx % 16;
        aptr[i] = h16 + (pos0 + (row < tr.mcount ? row : 0)) * I + 8 * piece;
        aoff[i] = row * PF_A16ROW + 8 * piece;
    }
    const int n0 = ti.ct * PF_DN_BN + wv * 64; // this wave's 64 columns: two 32-wide B tiles
    const int64_t wrow = (int64_t)tr.e * H + n0 + col;
    BRows br;
    br.q[0] = down_qs + wrow * (I / 2) + 16 * h;
    br.q[1] = down_qs + (wrow + 32) * (I / 2) + 16 * h;
    br.d[0] = down_d + wrow * (I / 32);
    br.d[1] = down_d + (wrow + 32) * (I / 32);
    const int NC = I / (PF_KC * 32);
    auto body = [&](auto mw) {
        constexpr int MW = decltype(mw)::value;
        v16f acc[MW][2];
        gemm_loop_a16<MW>(NC, aptr, aoff, s_a[0], s_a[1], br, acc);
        // the pair's row of o, as in the W4A8 down kernel (s_ooff was written before the K loop's first barrier)
#pragma unroll
        for (int mi = 0; mi < MW; ++mi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 32 * mi + mfma_row(r, lane);
                const int64_t oo = s_ooff[m];
                if (oo >= 0) {
                    float* orow = o + oo + n0 + col;
                    orow[0] = acc[mi][0][r];
                    orow[32] = acc[mi][1][r];
                }
            }
    };
    if (tr.mcount > 32)
        body(std::integral_constant<int, 2>());
    else
        body(std::integral_constant<int, 1>());
}

hipError_t launch_prefill_a16(const uint8_t* gate_qs, const uint8_t* up_qs, const uint8_t* down_qs,
                              const uint16_t* gate_d, const uint16_t* up_d, const uint16_t* down_d, int E, int H,
                              int I, const float* x, int T, int k, const float* topk_w, const int32_t* off,
                              const int32_t* sorted, bool accumulate, float* y, _Float16* x16, _Float16* h16,
                              float* o, hipStream_t s)
{
    if (T == 0) return hipSuccess;
    if (!pf_shape_ok(H, I) || !o) return hipErrorInvalidValue;
    const int P = T * k;
    const int64_t n8 = (int64_t)T * H / 8;
    a16_convert_kernel<<<dim3((unsigned)((n8 + 255) / 256)), 256, 0, s>>>(x, n8, x16);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const unsigned mt = pf_tiles_bound(P, E);
    prefill_a16_gateup_kernel<<<dim3(pf_grid(I / PF_GU_BN, mt)), PF_THREADS, 0, s>>>(
        gate_qs, up_qs, gate_d, up_d, E, H, I, x16, T, k, off, sorted, h16);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    prefill_a16_down_kernel<<<dim3(pf_grid(H / PF_DN_BN, mt)), PF_THREADS, 0, s>>>(
        down_qs, down_d, E, H, I, h16, T, k, off, sorted, o);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_combine(o, topk_w, T, k, H, accumulate, y, s);
}

} // namespace moeq4
