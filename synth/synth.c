/*
 * synth.c -- seeded, counter-based generator of the synthetic inputs.
 *
 * This module holds no arithmetic of the quantized MoE method: it only turns
 * (seed, tensor id, element index) into bytes.  Both the CPU oracle and the
 * GPU path consume exactly the bytes produced here, so any tensor slice (one
 * expert of one layer, a few tokens) can be regenerated on demand without
 * materialising the whole tensor twice.
 *
 * Generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014).  A stream is keyed by (seed, tid); its
 * i-th output (i = 0, 1, ...) is the SplitMix64 finaliser applied to
 * key + (i + 1) * GAMMA, i.e. the (i+1)-th output of a SplitMix64 generator
 * whose state starts at `key`.
 *
 * Derived draws:
 *   uniform  u  = (r >> 11) * 2^-53                       in [0, 1)
 *   normal   z  = Box-Muller on the pair (u[2j], u[2j+1]) in fp64,
 *                 element 2j takes the cosine, 2j+1 the sine, rounded to fp32
 *   nibbles     : byte b of the stream is byte (b % 8) of r[b / 8]
 *                 (little-endian), so every nibble is uniform on 0..15
 *   fp16 scale  : d = fp16_RNE(lo + (hi - lo) * u[i])
 *   Zipf bias   : element (t, e) of a biased logit tensor is
 *                 fp32(z(t*E+e) + s_bias * log(e + 1)), all in fp64
 *
 * Built with -O2 -ffp-contract=off so the bytes do not depend on FMA fusion.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tid)
{
    return mix64(seed * GAMMA + mix64(tid + 0x632BE59BD9B4E019ULL));
}

static inline uint64_t draw(uint64_t key, uint64_t i)
{
    return mix64(key + (i + 1) * GAMMA);
}

static inline double unit(uint64_t r)
{
    return (double)(r >> 11) * (1.0 / 9007199254740992.0); /* 2^-53 */
}

static double normal_at(uint64_t key, uint64_t i)
{
    const uint64_t j = i >> 1;
    const double u1 = unit(draw(key, 2 * j));
    const double u2 = unit(draw(key, 2 * j + 1));
    const double rad = sqrt(-2.0 * log(1.0 - u1)); /* 1 - u1 is in (0, 1] */
    const double ang = 6.283185307179586476925 * u2;
    return (i & 1) ? rad * sin(ang) : rad * cos(ang);
}

/* IEEE binary16 from a finite double, round-to-nearest-even. */
static uint16_t half_from_double(double v)
{
    uint16_t sign = 0;
    if (v < 0) { sign = 0x8000u; v = -v; }
    if (v == 0.0) return sign;
    int e;
    const double m = frexp(v, &e);       /* v = m * 2^e, m in [0.5, 1) */
    int E = e + 14;                      /* biased fp16 exponent of v  */
    if (E <= 0) {                        /* subnormal: multiple of 2^-24 */
        const double n = nearbyint(v * 16777216.0);
        return (uint16_t)(sign | (uint16_t)n); /* n == 1024 becomes the smallest normal */
    }
    double r = nearbyint(m * 2048.0);    /* 11 significant bits */
    if (r == 2048.0) { r = 1024.0; E += 1; }
    if (E >= 31) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)(E << 10) | (uint16_t)((int)r - 1024));
}

/* ---- exported: raw and derived streams over the index range [start, start+n) ---- */

void synth_u64(uint64_t seed, uint64_t tid, uint64_t start, int64_t n, uint64_t* out)
{
    const uint64_t key = stream_key(seed, tid);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = draw(key, start + (uint64_t)i);
}

void synth_uniform_f64(uint64_t seed, uint64_t tid, uint64_t start, int64_t n, double* out)
{
    const uint64_t key = stream_key(seed, tid);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = unit(draw(key, start + (uint64_t)i));
}

void synth_normal_f32(uint64_t seed, uint64_t tid, uint64_t start, int64_t n, float* out)
{
    const uint64_t key = stream_key(seed, tid);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (float)normal_at(key, start + (uint64_t)i);
}

/* logits[t][e] = fp32(z + s_bias * log(e + 1)) for the flat index t*E + e */
void synth_biased_logits_f32(uint64_t seed, uint64_t tid, int64_t T, int64_t E, double s_bias,
                             float* out)
{
    const uint64_t key = stream_key(seed, tid);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < T * E; ++i) {
        const int64_t e = i % E;
        out[i] = (float)(normal_at(key, (uint64_t)i) + s_bias * log((double)(e + 1)));
    }
}

void synth_nibble_bytes(uint64_t seed, uint64_t tid, uint64_t start_byte, int64_t nbytes,
                        uint8_t* out)
{
    const uint64_t key = stream_key(seed, tid);
    /* process whole 8-byte words in parallel, then the ragged ends */
    const uint64_t first_word = (start_byte + 7) / 8;
    const uint64_t end_byte = start_byte + (uint64_t)nbytes;
    const uint64_t last_word = end_byte / 8; /* exclusive */
    uint64_t b = start_byte;
    for (; b < end_byte && b < first_word * 8; ++b) {
        const uint64_t r = draw(key, b / 8);
        out[b - start_byte] = (uint8_t)(r >> (8 * (b % 8)));
    }
    if (last_word > first_word) {
#pragma omp parallel for schedule(static)
        for (int64_t w = (int64_t)first_word; w < (int64_t)last_word; ++w) {
            const uint64_t r = draw(key, (uint64_t)w);
            uint8_t* dst = out + ((uint64_t)w * 8 - start_byte);
            for (int k = 0; k < 8; ++k) dst[k] = (uint8_t)(r >> (8 * k));
        }
        b = last_word * 8;
    }
    for (; b < end_byte; ++b) {
        const uint64_t r = draw(key, b / 8);
        out[b - start_byte] = (uint8_t)(r >> (8 * (b % 8)));
    }
}

void synth_scales_f16(uint64_t seed, uint64_t tid, uint64_t start, int64_t n, double lo, double hi,
                      uint16_t* out)
{
    const uint64_t key = stream_key(seed, tid);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = half_from_double(lo + (hi - lo) * unit(draw(key, start + (uint64_t)i)));
}
