/*
 * synth.c — seeded synthetic inputs for the NVFP4 projection.
 *
 * Shared by the tests, the benchmark and the smoke check, and fed to both the
 * HIP library and the CPU oracle.  It contains only random-number generation
 * and *encoders* (real value -> bf16 / e4m3 / e2m1 bytes); it has no decoder,
 * no value table and none of the projection's arithmetic.
 *
 * Generator.  Counter-based SplitMix64: the i-th draw of stream (seed, stream)
 * is  mix(key + (i+1) * 0x9E3779B97F4A7C15)  with
 *     key = mix(mix(seed + 0x9E3779B97F4A7C15) ^ (stream * 0xD1B54A32D192ED03)),
 * where mix is the SplitMix64 output function (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014, with the constants
 * of Vigna's public-domain splitmix64.c).  Being counter-based, any element can
 * be produced alone, so work can be split over threads freely.
 *
 * Normal draws: Box-Muller on draws 2i and 2i+1,
 *     u1 = (hi53(r0) + 1) * 2^-53 in (0,1],  u2 = hi53(r1) * 2^-53 in [0,1),
 *     z  = sqrt(-2 ln u1) * cos(2 pi u2).
 *
 * Encoders (round to nearest, ties to even):
 *   bf16: round the double to 8 significant bits;
 *   e4m3 (OCP "fn"): quantum 2^(E-3) with E >= -6, saturating at 448;
 *   e2m1: nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code,
 *         clamped to 6, sign taken from the input (so -0.1 -> code 0x8).
 *
 * Two-level NVFP4 quantiser for the N(0, 0.02) weight configs (the configs
 * state "amax/6 scale in e4m3" per 16-element block and a global scale of
 * amax/(448*6)):  g = fp32(amax_tensor / 2688);  per block b of row n,
 * s_b = e4m3((amax_b / 6) / g);  q = e2m1(w / (s_b * g)), q = 0 when s_b = 0.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static uint64_t stream_key(uint64_t seed, uint64_t stream)
{
    return mix64(mix64(seed + GOLDEN) ^ (stream * 0xD1B54A32D192ED03ULL));
}

uint64_t syn_u64(uint64_t seed, uint64_t stream, uint64_t i)
{
    return mix64(stream_key(seed, stream) + (i + 1) * GOLDEN);
}

static double normal_at(uint64_t key, uint64_t i)
{
    uint64_t r0 = mix64(key + (2 * i + 1) * GOLDEN);
    uint64_t r1 = mix64(key + (2 * i + 2) * GOLDEN);
    double u1 = (double)((r0 >> 11) + 1) * 0x1.0p-53;
    double u2 = (double)(r1 >> 11) * 0x1.0p-53;
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

double syn_normal(uint64_t seed, uint64_t stream, uint64_t i)
{
    return normal_at(stream_key(seed, stream), i);
}

/* Round to 8 significant bits, ties to even (bf16 precision, normal range). */
static double round_bf16(double v)
{
    if (v == 0.0 || !isfinite(v))
        return v;
    int e;
    double f = frexp(v, &e);                 /* v = f * 2^e, 0.5 <= |f| < 1 */
    return ldexp(nearbyint(ldexp(f, 8)), e - 8);
}

static uint16_t bf16_bits(double rounded)
{
    float f = (float)rounded;                /* exact: 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* e4m3 encode of v >= 0, RNE, saturating; *value receives the rounded value. */
static uint8_t e4m3_encode(double v, double *value)
{
    if (!(v > 0.0)) {
        *value = 0.0;
        return 0;
    }
    if (v >= 448.0) {
        *value = 448.0;
        return 0x7E;
    }
    int e;
    frexp(v, &e);
    int E = e - 1;                           /* 2^E <= v < 2^(E+1) */
    if (E < -6)
        E = -6;                              /* subnormal quantum 2^-9 */
    double r = nearbyint(ldexp(v, 3 - E));   /* v in units of 2^(E-3) */
    *value = ldexp(r, E - 3);
    if (r < 8.0)
        return (uint8_t)r;                   /* subnormal, exponent field 0 */
    if (r >= 16.0) {
        r = 8.0;
        E += 1;
    }
    unsigned code = ((unsigned)(E + 7) << 3) | ((unsigned)r - 8u);
    if (code > 0x7Eu) {
        *value = 448.0;
        return 0x7E;
    }
    return (uint8_t)code;
}

/* e2m1 encode, RNE with ties to the even code, magnitude clamped to 6. */
static unsigned e2m1_encode(double v)
{
    double a = fabs(v);
    unsigned m;
    if (a <= 0.25) m = 0;
    else if (a < 0.75) m = 1;
    else if (a <= 1.25) m = 2;
    else if (a < 1.75) m = 3;
    else if (a <= 2.5) m = 4;
    else if (a < 3.5) m = 5;
    else if (a <= 5.0) m = 6;
    else m = 7;
    return m | (signbit(v) ? 8u : 0u);
}

/* out[j] = bf16(stddev * N(0,1)_{i0+j}) as bit patterns. */
void syn_normal_bf16(uint64_t seed, uint64_t stream, double stddev, int64_t i0,
                     int64_t count, uint16_t *out)
{
    uint64_t key = stream_key(seed, stream);
    for (int64_t j = 0; j < count; ++j)
        out[j] = bf16_bits(round_bf16(stddev * normal_at(key, (uint64_t)(i0 + j))));
}

/* max_j |bf16(stddev * N(0,1)_{i0+j})| over [i0, i0+count). */
double syn_normal_bf16_amax(uint64_t seed, uint64_t stream, double stddev,
                            int64_t i0, int64_t count)
{
    uint64_t key = stream_key(seed, stream);
    double amax = 0.0;
    for (int64_t j = 0; j < count; ++j) {
        double a = fabs(round_bf16(stddev * normal_at(key, (uint64_t)(i0 + j))));
        if (a > amax)
            amax = a;
    }
    return amax;
}

/* fp32 global scale from the tensor amax: g = fp32(amax / (448 * 6)). */
float syn_global_scale(double amax)
{
    return (float)(amax / 2688.0);
}

/*
 * Quantise rows [n0, n1) of the [N][K] matrix W[n][k] = bf16(stddev *
 * N(0,1)_{n*K+k}) with global scale g.  codes/scales point at row n0 of the
 * canonical [N][K/2] and [N][K/16] arrays.  K % 16 == 0.
 */
void syn_quantize_rows(uint64_t seed, uint64_t stream, double stddev, int64_t K,
                       int64_t n0, int64_t n1, float g, uint8_t *codes,
                       uint8_t *scales)
{
    uint64_t key = stream_key(seed, stream);
    double gd = (double)g;
    double w[16];
    for (int64_t n = n0; n < n1; ++n) {
        uint8_t *crow = codes + (n - n0) * (K / 2);
        uint8_t *srow = scales + (n - n0) * (K / 16);
        for (int64_t b = 0; b < K / 16; ++b) {
            double amax = 0.0;
            for (int t = 0; t < 16; ++t) {
                uint64_t i = (uint64_t)(n * K + b * 16 + t);
                w[t] = round_bf16(stddev * normal_at(key, i));
                if (fabs(w[t]) > amax)
                    amax = fabs(w[t]);
            }
            double sval;
            srow[b] = e4m3_encode(amax / 6.0 / gd, &sval);
            double unit = sval * gd;
            for (int t = 0; t < 16; t += 2) {
                unsigned lo = unit > 0.0 ? e2m1_encode(w[t] / unit) : 0u;
                unsigned hi = unit > 0.0 ? e2m1_encode(w[t + 1] / unit) : 0u;
                crow[(b * 16 + t) / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
}

/* Packed codes drawn uniformly over all 16 e2m1 codes: element i gets
 * syn_u64(seed, stream, i) & 15; bytes [byte0, byte0+count). */
void syn_uniform_codes(uint64_t seed, uint64_t stream, int64_t byte0,
                       int64_t count, uint8_t *out)
{
    uint64_t key = stream_key(seed, stream);
    for (int64_t j = 0; j < count; ++j) {
        uint64_t i = (uint64_t)(2 * (byte0 + j));
        unsigned lo = (unsigned)(mix64(key + (i + 1) * GOLDEN) & 15u);
        unsigned hi = (unsigned)(mix64(key + (i + 2) * GOLDEN) & 15u);
        out[j] = (uint8_t)(lo | (hi << 4));
    }
}

/* Block scales e4m3(|N(0, sd)| + offset) for elements [i0, i0+count). */
void syn_abs_normal_e4m3(uint64_t seed, uint64_t stream, double sd,
                         double offset, int64_t i0, int64_t count, uint8_t *out)
{
    uint64_t key = stream_key(seed, stream);
    double unused;
    for (int64_t j = 0; j < count; ++j)
        out[j] = e4m3_encode(fabs(sd * normal_at(key, (uint64_t)(i0 + j))) + offset,
                             &unused);
}

/* Encoders exposed for the generator's own tests. */
uint16_t syn_encode_bf16(double v) { return bf16_bits(round_bf16(v)); }
uint8_t syn_encode_e4m3(double v) { double u; return e4m3_encode(v, &u); }
unsigned syn_encode_e2m1(double v) { return e2m1_encode(v); }
