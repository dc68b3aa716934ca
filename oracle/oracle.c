/*
 * oracle.c -- plain, slow, single-threaded CPU reference of the Q4_0 W4A8
 * mixture-of-experts expert matmul.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the bench's
 * CPU-baseline leg may load this file's library.  It shares no code, header,
 * table or helper with the GPU library; the two meet only in the bytes that
 * the seeded input generator produces.
 *
 * Source pages: "A 35B Hybrid-Attention Mixture-of-Experts Model on a 6GB 2011
 * GPU: Hand-Written 4-bit CUDA Inference for Fermi" (gist.science 2606.24031).
 * Citations below use the page language and its section:
 *   [nl Methodologie 1]  Dutch technical summary, Methodologie, item 1
 *                        (GPU prefill runs a grouped 4-bit GEMM for the MoE;
 *                        CPU decode runs a W4A8 integer kernel whose integer
 *                        multiply-adds consume 4-bit weights and 8-bit
 *                        activations)
 *   [nl Methodologie 2]  same page, item 2 "Kwantisatie" (group-wise symmetric
 *                        4-bit weights of the Q4_0 family, 8-bit activations)
 *   [nl Methodologie 4]  same page, item 4 (single-pass prefill: the whole
 *                        prompt in one pass)
 *   [nl Resultaten]      same page, results (thin-M GEMM named a structural
 *                        bottleneck)
 *
 * The pages name the scheme but fix none of its numbers.  Readings taken
 * here (each one is restated where it is used):
 *   R1  Q4_0 block = 32 weights, 16 bytes of nibbles and one fp16 scale d;
 *       weight value = (q - 8) * d, q in 0..15 ("symmetric": no zero point).
 *       Byte i of a block holds element i in its low nibble and element
 *       i + 16 in its high nibble.
 *   R2  8-bit activations use the same 32-wide blocks: d = amax / 127 with a
 *       correctly rounded fp32 divide, q = round-half-even(x / d) (again a
 *       correctly rounded fp32 divide), clamped to [-127, 127]; amax = 0
 *       gives d = 0 and q = 0.  The scale stays fp32.
 *   R3  A block's dot product is an exact int32 sum of (q_w - 8) * q_a; the
 *       matvec output is the fp64 sum over blocks of d_w * d_a * isum, which
 *       equals the dequantised fp64 matvec up to the final rounding to fp32.
 *   R4  Router: softmax over the E logits, keep the k largest, renormalise
 *       over the kept k.  Selection compares logits (softmax is strictly
 *       monotone), larger first, equal logits broken by the lower expert id;
 *       slots are stored in that order.  Weights in fp64, stored as fp32.
 *   R5  Grouping: pair id p = t*k + j; expert_offsets is the exclusive prefix
 *       sum of per-expert pair counts; sorted_pairs lists each expert's pairs
 *       in ascending p (a stable counting sort).
 *   R6  Expert FFN (SwiGLU): g = W_gate x, u = W_up x, h = silu(g) * u with
 *       silu(z) = z / (1 + exp(-z)); h is rounded to fp32 and re-quantised
 *       with R2 before the down projection o = W_down h_q (W4A8 throughout).
 *   R7  Combine: y_t = sum_j w_{t,j} o_{t,j} in fp64, one rounding to fp32;
 *       with the ACCUMULATE flag the sum is added to the incoming y_t.
 *   R8  Optional pre-norm for stacked layers: x <- x / sqrt(mean(x^2) + 1e-6)
 *       per row, the factor in fp64, each element rounded to fp32.
 *   R9  Prefill and decode compute the same function; only the schedule
 *       differs [nl Methodologie 4].
 *   R11 W4A16 variant of the expert FFN (prefill): the same packed experts
 *       dequantised to 16-bit operands, w = fp16((q - 8) * d), and
 *       activations not quantised but carried in 16 bits: the layer input
 *       and h are rounded to the nearest fp16 (ties to even); every sum is
 *       exact (fp64) over those 16-bit values.  The pages tie 8-bit
 *       activations to decode only [nl Methodologie 2], so this is the plain
 *       reading of a prefill whose operands are all 16-bit.  With
 *       ORC_FLAG_EXACT_ACT nothing is rounded (exact weights and activations:
 *       the fp64 FFN itself), the yardstick both variants are measured
 *       against.
 *   R10 Router projection (the step in front of R4): logits = x_n W_r^T with
 *       W_r [E][H] fp32 and x_n the input row, pre-normed with R8 when the
 *       flag is set; each logit is the fp64 sum of fp64 products, rounded
 *       once to fp32.  The pages name MoE routing [nl Methodologie 1] but
 *       give no router arithmetic; a dense fp32 projection is the plain
 *       reading.
 *
 * Compiled with -O2 -fno-fast-math -ffp-contract=off.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ENOMEM (-2)

#define ORC_FLAG_RMSNORM 1u
#define ORC_FLAG_ACCUMULATE 2u
#define ORC_FLAG_EXACT_ACT 4u

/* Exact value of an IEEE binary16 bit pattern (R1: fp16 scale). */
double orc_half_to_double(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int ex = (h >> 10) & 31;
    const int man = h & 1023;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + man), ex - 25);
    return sign ? -v : v;
}

/* Nibble q (0..15) of element `i` (0..K-1) of a Q4_0 row (R1). */
static int q4_nibble(const uint8_t* row_qs, int64_t i)
{
    const int64_t b = i / 32, e = i % 32;
    const uint8_t byte = row_qs[b * 16 + (e % 16)];
    return e < 16 ? (byte & 15) : (byte >> 4);
}

/* --------------------------------------------------------------------------
 * Q4_0 dequantisation [nl Methodologie 2], R1.
 * qs [rows][K/2], d [rows][K/32] -> w [rows][K] in fp64 (exact).
 */
int orc_q4_dequant(const uint8_t* qs, const uint16_t* d, int64_t rows, int64_t K, double* w)
{
    if (!qs || !d || !w || rows < 0 || K <= 0 || K % 32) return ORC_EINVAL;
    for (int64_t r = 0; r < rows; ++r) {
        const uint8_t* rq = qs + r * (K / 2);
        for (int64_t i = 0; i < K; ++i) {
            const double scale = orc_half_to_double(d[r * (K / 32) + i / 32]);
            w[r * K + i] = (double)(q4_nibble(rq, i) - 8) * scale;
        }
    }
    return ORC_OK;
}

/* --------------------------------------------------------------------------
 * Q8_0 activation quantisation [nl Methodologie 2] ("8-bit activations"), R2,
 * with the optional per-row pre-norm R8.
 * x [rows][cols] -> xq [rows][cols] int8, xd [rows][cols/32] fp32.
 */
int orc_q8_quantize(const float* x, int64_t rows, int64_t cols, uint32_t flags, int8_t* xq, float* xd)
{
    if (!x || !xq || !xd || rows < 0 || cols <= 0 || cols % 32) return ORC_EINVAL;
    float* xn = (float*)malloc((size_t)cols * sizeof(float));
    if (!xn) return ORC_ENOMEM;
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * cols;
        if (flags & ORC_FLAG_RMSNORM) {
            double ss = 0.0;
            for (int64_t i = 0; i < cols; ++i) ss += (double)xr[i] * (double)xr[i];
            const double inv = 1.0 / sqrt(ss / (double)cols + 1e-6);
            for (int64_t i = 0; i < cols; ++i) xn[i] = (float)((double)xr[i] * inv);
        } else {
            memcpy(xn, xr, (size_t)cols * sizeof(float));
        }
        for (int64_t b = 0; b < cols / 32; ++b) {
            const float* blk = xn + b * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                const float a = fabsf(blk[i]);
                if (a > amax) amax = a;
            }
            const float dq = amax / 127.0f;
            xd[r * (cols / 32) + b] = dq;
            for (int i = 0; i < 32; ++i) {
                int q = 0;
                if (dq != 0.0f) {
                    const float v = rintf(blk[i] / dq);
                    q = v > 127.0f ? 127 : (v < -127.0f ? -127 : (int)v);
                }
                xq[r * cols + b * 32 + i] = (int8_t)q;
            }
        }
    }
    free(xn);
    return ORC_OK;
}

/* --------------------------------------------------------------------------
 * Exact int32 block dot products (R3) [nl Methodologie 1] (integer
 * multiply-adds of 4-bit weights with 8-bit activations).
 * qs [rows][K/2] (one Q4_0 matrix), xq [T][K]  ->  out [T][rows][K/32]:
 *     out[t][r][b] = sum_{i<32} (q[r][32b+i] - 8) * xq[t][32b+i].
 */
int orc_block_dots(const uint8_t* qs, int64_t rows, int64_t K, const int8_t* xq, int64_t T, int32_t* out)
{
    if (!qs || !xq || !out || rows < 0 || T < 0 || K <= 0 || K % 32) return ORC_EINVAL;
    const int64_t nb = K / 32;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t r = 0; r < rows; ++r) {
            const uint8_t* rq = qs + r * (K / 2);
            for (int64_t b = 0; b < nb; ++b) {
                int32_t s = 0;
                for (int i = 0; i < 32; ++i)
                    s += (q4_nibble(rq, b * 32 + i) - 8) * (int32_t)xq[t * K + b * 32 + i];
                out[(t * rows + r) * nb + b] = s;
            }
        }
    return ORC_OK;
}

/* One output of a W4A8 matvec in fp64 (R3): sum_b d_w * d_a * isum.  When
 * abs_sum is given it also receives sum_b |d_w * d_a * isum|, the sum of the
 * magnitudes of the same block terms (not part of the method: the quantity
 * that bounds the rounding error of any fp32 evaluation of this sum). */
static double w4a8_dot(const uint8_t* row_qs, const uint16_t* row_d, int64_t K, const int8_t* a,
                       const float* ad, double* abs_sum)
{
    double acc = 0.0, mag = 0.0;
    for (int64_t b = 0; b < K / 32; ++b) {
        int32_t s = 0;
        for (int i = 0; i < 32; ++i) s += (q4_nibble(row_qs, b * 32 + i) - 8) * (int32_t)a[b * 32 + i];
        const double term = orc_half_to_double(row_d[b]) * (double)ad[b] * (double)s;
        acc += term;
        mag += fabs(term);
    }
    if (abs_sum) *abs_sum = mag;
    return acc;
}

/* --------------------------------------------------------------------------
 * W4A8 matvec of one Q4_0 matrix against T quantised activation rows
 * [nl Methodologie 1] (W4A8 integer decode kernel), R3.
 * qs [N][K/2], d [N][K/32], xq [T][K], xd [T][K/32]  ->  y [T][N] fp32.
 */
int orc_gemv(const uint8_t* qs, const uint16_t* d, int64_t N, int64_t K, const int8_t* xq, const float* xd,
             int64_t T, float* y)
{
    if (!qs || !d || !xq || !xd || !y || N < 0 || T < 0 || K <= 0 || K % 32) return ORC_EINVAL;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < N; ++n)
            y[t * N + n] = (float)w4a8_dot(qs + n * (K / 2), d + n * (K / 32), K, xq + t * K, xd + t * (K / 32), NULL);
    return ORC_OK;
}

/* --------------------------------------------------------------------------
 * Router [nl Methodologie 1] ("grouped 4-bit GEMM for the MoE routing"),
 * R4 + R5.
 * logits [T][E] -> topk_ids [T][k], topk_w [T][k], expert_offsets [E+1],
 * sorted_pairs [T*k].
 */
int orc_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids, float* topk_w,
              int32_t* expert_offsets, int32_t* sorted_pairs)
{
    if (!logits || !topk_ids || !topk_w || !expert_offsets || !sorted_pairs) return ORC_EINVAL;
    if (T < 0 || E < 1 || k < 1 || k > E) return ORC_EINVAL;
    char* taken = (char*)malloc((size_t)E);
    double* p = (double*)malloc((size_t)E * sizeof(double));
    int32_t* fill = (int32_t*)malloc((size_t)E * sizeof(int32_t));
    if (!taken || !p || !fill) { free(taken); free(p); free(fill); return ORC_ENOMEM; }

    for (int32_t t = 0; t < T; ++t) {
        const float* l = logits + (int64_t)t * E;
        /* softmax over all E experts, fp64 */
        double lmax = l[0];
        for (int32_t e = 1; e < E; ++e) if (l[e] > lmax) lmax = l[e];
        double den = 0.0;
        for (int32_t e = 0; e < E; ++e) { p[e] = exp((double)l[e] - lmax); den += p[e]; }
        for (int32_t e = 0; e < E; ++e) p[e] /= den;
        /* top-k: repeatedly take the largest logit not yet taken, lower id on ties */
        memset(taken, 0, (size_t)E);
        double kept = 0.0;
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
            taken[best] = 1;
            topk_ids[(int64_t)t * k + j] = best;
            kept += p[best];
        }
        /* renormalise over the kept experts */
        for (int32_t j = 0; j < k; ++j)
            topk_w[(int64_t)t * k + j] = (float)(p[topk_ids[(int64_t)t * k + j]] / kept);
    }

    /* stable counting sort of pair ids by expert */
    const int64_t P = (int64_t)T * k;
    for (int32_t e = 0; e <= E; ++e) expert_offsets[e] = 0;
    for (int64_t q = 0; q < P; ++q) expert_offsets[topk_ids[q] + 1] += 1;
    for (int32_t e = 0; e < E; ++e) expert_offsets[e + 1] += expert_offsets[e];
    for (int32_t e = 0; e < E; ++e) fill[e] = expert_offsets[e];
    for (int64_t q = 0; q < P; ++q) sorted_pairs[fill[topk_ids[q]]++] = (int32_t)q;

    free(taken); free(p); free(fill);
    return ORC_OK;
}

/* --------------------------------------------------------------------------
 * One MoE layer on quantised activations: expert FFNs (R6) and the
 * routing-weighted combine (R7) [nl Methodologie 1] [nl Methodologie 2].
 *
 * Experts use the library's structure-of-arrays layout:
 *   gate_qs/up_qs [E][I][H/2], down_qs [E][H][I/2],
 *   gate_d/up_d [E][I][H/32], down_d [E][H][I/32] (fp16 bits).
 * xq [T][H], xd [T][H/32]: the Q8_0 activations (R2); topk_ids/topk_w [T][k].
 * tokens / n_tokens: the tokens to compute (NULL = all T); other rows of y
 *   and of the optional outputs are left untouched.
 * y [T][H]: overwritten, or accumulated into with ORC_FLAG_ACCUMULATE.
 * Optional outputs, indexed by pair id p = t*k + j (NULL = skip):
 *   g_out, u_out, h_out [P][I] fp32; hq_out [P][I] int8, hd_out [P][I/32];
 *   sg_out, su_out [P][I] fp64: sum_b |d_w d_a isum| over the blocks of each
 *   gate and up output (see w4a8_dot).
 * Optional conditioning inputs hq_in/hd_in [P][I]: when both are given, the
 *   down projection uses them in place of the oracle's own re-quantised h.
 */
typedef struct {
    int32_t E, H, I;
    const uint8_t *gate_qs, *up_qs, *down_qs;
    const uint16_t *gate_d, *up_d, *down_d;
} orc_experts;

int orc_moe_layer(const orc_experts* w, const int8_t* xq, const float* xd, int32_t T, int32_t k,
                  const int32_t* topk_ids, const float* topk_w, const int32_t* tokens, int32_t n_tokens,
                  uint32_t flags, float* y, float* g_out, float* u_out, float* h_out, int8_t* hq_out,
                  float* hd_out, const int8_t* hq_in, const float* hd_in, double* sg_out, double* su_out)
{
    if (!w || !xq || !xd || !topk_ids || !topk_w || !y) return ORC_EINVAL;
    const int64_t E = w->E, H = w->H, I = w->I;
    if (E < 1 || H <= 0 || I <= 0 || H % 32 || I % 32 || T < 0 || k < 1 || k > E) return ORC_EINVAL;
    const int32_t nt = tokens ? n_tokens : T;

    float* hf = (float*)malloc((size_t)I * sizeof(float));
    int8_t* hq = (int8_t*)malloc((size_t)I);
    float* hd = (float*)malloc((size_t)(I / 32) * sizeof(float));
    double* acc = (double*)malloc((size_t)H * sizeof(double));
    if (!hf || !hq || !hd || !acc) { free(hf); free(hq); free(hd); free(acc); return ORC_ENOMEM; }

    for (int32_t it = 0; it < nt; ++it) {
        const int64_t t = tokens ? tokens[it] : it;
        if (t < 0 || t >= T) { free(hf); free(hq); free(hd); free(acc); return ORC_EINVAL; }
        const int8_t* a = xq + t * H;
        const float* ad = xd + t * (H / 32);
        for (int64_t n = 0; n < H; ++n) acc[n] = 0.0;

        for (int32_t j = 0; j < k; ++j) {
            const int64_t p = t * k + j;
            const int64_t e = topk_ids[p];
            if (e < 0 || e >= E) { free(hf); free(hq); free(hd); free(acc); return ORC_EINVAL; }
            const uint8_t* gq = w->gate_qs + e * I * (H / 2);
            const uint8_t* uq = w->up_qs + e * I * (H / 2);
            const uint16_t* gd = w->gate_d + e * I * (H / 32);
            const uint16_t* ud = w->up_d + e * I * (H / 32);
            /* gate/up projections and SwiGLU (R6) */
            for (int64_t n = 0; n < I; ++n) {
                const double g = w4a8_dot(gq + n * (H / 2), gd + n * (H / 32), H, a, ad, sg_out ? sg_out + p * I + n : NULL);
                const double u = w4a8_dot(uq + n * (H / 2), ud + n * (H / 32), H, a, ad, su_out ? su_out + p * I + n : NULL);
                const double h = g / (1.0 + exp(-g)) * u;
                hf[n] = (float)h;
                if (g_out) g_out[p * I + n] = (float)g;
                if (u_out) u_out[p * I + n] = (float)u;
                if (h_out) h_out[p * I + n] = hf[n];
            }
            /* re-quantise h (R2) */
            int rc = orc_q8_quantize(hf, 1, I, 0u, hq, hd);
            if (rc) { free(hf); free(hq); free(hd); free(acc); return rc; }
            if (hq_out) memcpy(hq_out + p * I, hq, (size_t)I);
            if (hd_out) memcpy(hd_out + p * (I / 32), hd, (size_t)(I / 32) * sizeof(float));
            const int8_t* hqu = (hq_in && hd_in) ? hq_in + p * I : hq;
            const float* hdu = (hq_in && hd_in) ? hd_in + p * (I / 32) : hd;
            /* down projection and routing-weighted combine (R7) */
            const uint8_t* dq = w->down_qs + e * H * (I / 2);
            const uint16_t* dd = w->down_d + e * H * (I / 32);
            const double wt = (double)topk_w[p];
            for (int64_t n = 0; n < H; ++n)
                acc[n] += wt * w4a8_dot(dq + n * (I / 2), dd + n * (I / 32), I, hqu, hdu, NULL);
        }
        float* yr = y + t * H;
        for (int64_t n = 0; n < H; ++n)
            yr[n] = (flags & ORC_FLAG_ACCUMULATE) ? (float)((double)yr[n] + acc[n]) : (float)acc[n];
    }
    free(hf); free(hq); free(hd); free(acc);
    return ORC_OK;
}

/* --------------------------------------------------------------------------
 * Router logits, R10 (with R8 when ORC_FLAG_RMSNORM is set).
 * x [T][H] fp32, wr [E][H] fp32  ->  logits [T][E] fp32.
 */
int orc_router_logits(const float* x, int64_t T, int64_t H, const float* wr, int64_t E, uint32_t flags,
                      float* logits)
{
    if (!x || !wr || !logits || T < 0 || H <= 0 || E <= 0) return ORC_EINVAL;
    float* xn = (float*)malloc((size_t)H * sizeof(float));
    if (!xn) return ORC_ENOMEM;
    for (int64_t t = 0; t < T; ++t) {
        const float* xr = x + t * H;
        if (flags & ORC_FLAG_RMSNORM) {
            double ss = 0.0;
            for (int64_t i = 0; i < H; ++i) ss += (double)xr[i] * (double)xr[i];
            const double inv = 1.0 / sqrt(ss / (double)H + 1e-6);
            for (int64_t i = 0; i < H; ++i) xn[i] = (float)((double)xr[i] * inv);
        } else {
            memcpy(xn, xr, (size_t)H * sizeof(float));
        }
        for (int64_t e = 0; e < E; ++e) {
            const float* we = wr + e * H;
            double acc = 0.0;
            for (int64_t i = 0; i < H; ++i) acc += (double)xn[i] * (double)we[i];
            logits[t * E + e] = (float)acc;
        }
    }
    free(xn);
    return ORC_OK;
}

/* --------------------------------------------------------------------------
 * The nearest IEEE binary16 value of v, ties to even (R11), returned in fp64:
 * the spacing of fp16 values is 2^(e-10) in the binade [2^e, 2^(e+1)) for
 * e >= -14 and 2^-24 below it; magnitudes from 65520 up round to infinity.
 */
static double round_to_half(double v)
{
    if (v == 0.0 || v != v) return v;
    const double a = fabs(v);
    if (a >= 65520.0) return v > 0 ? INFINITY : -INFINITY;
    int e;
    frexp(a, &e); /* a in [2^(e-1), 2^e) */
    int lead = e - 1;
    if (lead < -14) lead = -14;
    const double quantum = ldexp(1.0, lead - 10);
    const double r = nearbyint(a / quantum) * quantum; /* default mode: nearest, ties to even */
    return v < 0 ? -r : r;
}

double orc_round_to_half(double v) { return round_to_half(v); }

/* One output of a matvec over a dequantised Q4_0 row and fp64 activations (R1, R11): each weight
 * (q - 8) * d exactly, or rounded to fp16 when w16 is set. */
static double w4_dot(const uint8_t* row_qs, const uint16_t* row_d, int64_t K, const double* a, int w16)
{
    double acc = 0.0;
    for (int64_t b = 0; b < K / 32; ++b) {
        const double d = orc_half_to_double(row_d[b]);
        for (int i = 0; i < 32; ++i) {
            const double wv = (double)(q4_nibble(row_qs, b * 32 + i) - 8) * d;
            acc += (w16 ? round_to_half(wv) : wv) * a[b * 32 + i];
        }
    }
    return acc;
}

/* --------------------------------------------------------------------------
 * One MoE layer, W4A16 (R11 with R4-R7): x [T][H] fp32 input rows; routing
 * as orc_moe_layer; y [T][H] overwritten or accumulated (ORC_FLAG_ACCUMULATE).
 * h_out [P][I] (optional, pair order): h as carried to the down projection.
 */
int orc_moe_layer_a16(const orc_experts* w, const float* x, int32_t T, int32_t k, const int32_t* topk_ids,
                      const float* topk_w, const int32_t* tokens, int32_t n_tokens, uint32_t flags, float* y,
                      float* h_out)
{
    if (!w || !x || !topk_ids || !topk_w || !y) return ORC_EINVAL;
    const int64_t E = w->E, H = w->H, I = w->I;
    if (E < 1 || H <= 0 || I <= 0 || H % 32 || I % 32 || T < 0 || k < 1 || k > E) return ORC_EINVAL;
    const int exact = (flags & ORC_FLAG_EXACT_ACT) != 0;
    const int32_t nt = tokens ? n_tokens : T;
    double* a = (double*)malloc((size_t)H * sizeof(double));
    double* h = (double*)malloc((size_t)I * sizeof(double));
    double* acc = (double*)malloc((size_t)H * sizeof(double));
    if (!a || !h || !acc) { free(a); free(h); free(acc); return ORC_ENOMEM; }
    for (int32_t it = 0; it < nt; ++it) {
        const int64_t t = tokens ? tokens[it] : it;
        if (t < 0 || t >= T) { free(a); free(h); free(acc); return ORC_EINVAL; }
        for (int64_t i = 0; i < H; ++i) a[i] = exact ? (double)x[t * H + i] : round_to_half((double)x[t * H + i]);
        for (int64_t n = 0; n < H; ++n) acc[n] = 0.0;
        for (int32_t j = 0; j < k; ++j) {
            const int64_t p = t * k + j;
            const int64_t e = topk_ids[p];
            if (e < 0 || e >= E) { free(a); free(h); free(acc); return ORC_EINVAL; }
            const uint8_t* gq = w->gate_qs + e * I * (H / 2);
            const uint8_t* uq = w->up_qs + e * I * (H / 2);
            const uint16_t* gd = w->gate_d + e * I * (H / 32);
            const uint16_t* ud = w->up_d + e * I * (H / 32);
            for (int64_t n = 0; n < I; ++n) {
                const double g = w4_dot(gq + n * (H / 2), gd + n * (H / 32), H, a, !exact);
                const double u = w4_dot(uq + n * (H / 2), ud + n * (H / 32), H, a, !exact);
                const double v = g / (1.0 + exp(-g)) * u;
                h[n] = exact ? v : round_to_half(v);
                if (h_out) h_out[p * I + n] = (float)h[n];
            }
            const uint8_t* dq = w->down_qs + e * H * (I / 2);
            const uint16_t* dd = w->down_d + e * H * (I / 32);
            const double wt = (double)topk_w[p];
            for (int64_t n = 0; n < H; ++n) acc[n] += wt * w4_dot(dq + n * (I / 2), dd + n * (I / 32), I, h, !exact);
        }
        float* yr = y + t * H;
        for (int64_t n = 0; n < H; ++n)
            yr[n] = (flags & ORC_FLAG_ACCUMULATE) ? (float)((double)yr[n] + acc[n]) : (float)acc[n];
    }
    free(a); free(h); free(acc);
    return ORC_OK;
}
