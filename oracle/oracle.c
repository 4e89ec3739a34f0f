/*
 * oracle.c — CPU oracle for the NVFP4 weight-only projection  y = x · dequant(W)^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (plain definition, fp64 throughout):
 *
 *     W[n,k] = e2m1(code[n,k]) * e4m3(scale[n, floor(k/16)]) * g
 *     y[m,n] = sum_k  bf16(x[m,k]) * W[n,k]
 *     S[m,n] = sum_k |bf16(x[m,k]) * W[n,k]|        (tolerance base)
 *
 * Sources.  The weight format is the NVFP4 checkpoint format named on the
 * FlashRT "Qwen3.6 NVFP4 usage" page (constructor argument table: a
 * compressed-tensors "nvfp4-pack-quantized" checkpoint) and on the Qwen3x-Orin
 * README (repository map: FP8 and NVFP4 format primitives).  Neither page gives
 * bit layouts, so:
 *   - e2m1 follows the OCP Microscaling Formats (MX) v1.0 spec, FP4 E2M1
 *     element: 1 sign, 2 exponent (bias 1), 1 mantissa bit, E=0 subnormal,
 *     no Inf/NaN;
 *   - e4m3 follows the OCP 8-bit Floating Point spec, E4M3 ("fn"): bias 7,
 *     subnormals m/8 * 2^-6, S.1111.111 = NaN, no Inf (not the FNUZ variant);
 *   - codes are packed two per byte, element 2j in the low nibble (bits 3:0),
 *     element 2j+1 in the high nibble;
 *   - canonical layouts: codes u8 [N][K/2], scales u8 [N][K/16], x bf16 bits
 *     [M][K] row-major, y [M][N];
 *   - the fp32 global scale g multiplies.
 * Row dequantisation into an fp64 buffer is exact: q*s has at most 6
 * significant bits and g 24, so q*s*g fits in 53 bits.
 *
 * Parity pins (see tests/): the e2m1 table against the OCP table fixture, all
 * 256 e4m3 encodings against torch.float8_e4m3fn, bf16 against torch.bfloat16,
 * and the projection against exact rational arithmetic on tiny inputs.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- element formats (closed forms) ----------------------------------- */

/* e2m1 code (low 4 bits of c) -> value.  OCP MX v1.0 FP4 E2M1. */
double orc_e2m1(unsigned c)
{
    unsigned sign = (c >> 3) & 1u;
    unsigned e = (c >> 1) & 3u;
    unsigned m = c & 1u;
    double mag;
    if (e == 0)
        mag = 0.5 * (double)m;                       /* subnormal: m/2 * 2^(1-1) */
    else
        mag = ldexp(1.0 + 0.5 * (double)m, (int)e - 1); /* 2^(e-1) * (1 + m/2) */
    return sign ? -mag : mag;
}

/* e4m3 byte -> value.  OCP OFP8 E4M3 ("fn"): bias 7, NaN = S.1111.111. */
double orc_e4m3(unsigned b)
{
    unsigned sign = (b >> 7) & 1u;
    unsigned e = (b >> 3) & 15u;
    unsigned m = b & 7u;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);                  /* m/8 * 2^-6 */
    else
        mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return sign ? -mag : mag;
}

/* bf16 bit pattern -> value: the upper half of an IEEE binary32. */
double orc_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ---- one weight row ----------------------------------------------------- */

/* w[k] = e2m1(code[n,k]) * e4m3(scale[n,k/16]) * g for one row n, k in [0,K). */
void orc_dequant_row(const uint8_t *codes_row, const uint8_t *scales_row,
                     int64_t K, double g, double *w)
{
    for (int64_t k = 0; k < K; ++k) {
        uint8_t byte = codes_row[k / 2];
        unsigned code = (k % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4);
        double s = orc_e4m3(scales_row[k / 16]);
        w[k] = orc_e2m1(code) * s * g;
    }
}

/* ---- the projection ----------------------------------------------------- */

typedef struct {
    int64_t M, N, K;
    const uint8_t *codes, *scales;
    double g;
    const uint16_t *x;
    const int64_t *rows;   /* NULL: all rows; else row indices to evaluate */
    int64_t nrows;
    double *y, *S;         /* [M][nrows] */
    int64_t r0, r1;        /* this worker's slice of [0,nrows) */
    int status;
} orc_job;

static void *orc_worker(void *arg)
{
    orc_job *j = (orc_job *)arg;
    double *w = (double *)malloc((size_t)j->K * sizeof(double));
    double *xd = (double *)malloc((size_t)(j->M * j->K) * sizeof(double));
    if (!w || !xd) {
        free(w);
        free(xd);
        j->status = -1;
        return NULL;
    }
    for (int64_t i = 0; i < j->M * j->K; ++i)
        xd[i] = orc_bf16(j->x[i]);
    for (int64_t r = j->r0; r < j->r1; ++r) {
        int64_t n = j->rows ? j->rows[r] : r;
        orc_dequant_row(j->codes + n * (j->K / 2), j->scales + n * (j->K / 16),
                        j->K, j->g, w);
        for (int64_t m = 0; m < j->M; ++m) {
            const double *xm = xd + m * j->K;
            double acc = 0.0, absacc = 0.0;
            for (int64_t k = 0; k < j->K; ++k) {
                double t = xm[k] * w[k];
                acc += t;
                absacc += fabs(t);
            }
            j->y[m * j->nrows + r] = acc;
            j->S[m * j->nrows + r] = absacc;
        }
    }
    free(w);
    free(xd);
    j->status = 0;
    return NULL;
}

/*
 * y[m][r], S[m][r] for the weight rows listed in rows[0..nrows) (rows == NULL:
 * every row, nrows must equal N).  Work is split over rows on nthreads POSIX
 * threads.  Returns 0, or -1 on a bad argument or allocation failure.
 */
int orc_proj_rows(int64_t M, int64_t N, int64_t K, const uint8_t *codes,
                  const uint8_t *scales, double g, const uint16_t *x,
                  const int64_t *rows, int64_t nrows, double *y, double *S,
                  int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0 || nrows < 0)
        return -1;
    if (!rows && nrows != N)
        return -1;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= N)
                return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nrows == 0 || M == 0)
        return 0;
    if (nthreads > nrows)
        nthreads = (int)nrows;
    orc_job *jobs = (orc_job *)calloc((size_t)nthreads, sizeof(orc_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !tid) {
        free(jobs);
        free(tid);
        return -1;
    }
    int rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        orc_job *j = &jobs[t];
        j->M = M; j->N = N; j->K = K;
        j->codes = codes; j->scales = scales; j->g = g; j->x = x;
        j->rows = rows; j->nrows = nrows; j->y = y; j->S = S;
        j->r0 = nrows * t / nthreads;
        j->r1 = nrows * (t + 1) / nthreads;
        j->status = -1;
        if (pthread_create(&tid[t], NULL, orc_worker, j) != 0) {
            orc_worker(j);   /* run inline if a thread cannot start */
            tid[t] = 0;
        }
    }
    for (int t = 0; t < nthreads; ++t) {
        if (tid[t])
            pthread_join(tid[t], NULL);
        if (jobs[t].status != 0)
            rc = -1;
    }
    free(jobs);
    free(tid);
    return rc;
}

/* Full projection: y[M][N], S[M][N]. */
int orc_proj(int64_t M, int64_t N, int64_t K, const uint8_t *codes,
             const uint8_t *scales, double g, const uint16_t *x, double *y,
             double *S, int nthreads)
{
    return orc_proj_rows(M, N, K, codes, scales, g, x, NULL, N, y, S, nthreads);
}

/* ---- the acceptance test ------------------------------------------------ */

/*
 * Element test against the projection's stated tolerance:
 *     |y_gpu - y_ref| <= rtol * S      (S = sum_k |x_k * w_k|, fp64)
 * with the special cases: S == 0 requires y_gpu == 0 exactly; a NaN y_ref
 * requires a NaN y_gpu; a finite y_ref requires a finite y_gpu.
 * Returns the number of failing elements; *max_ratio receives the largest
 * |y_gpu - y_ref| / S over elements with S > 0 (diagnostic).
 */
int64_t orc_check(int64_t count, const double *yref, const double *S,
                  const float *ygpu, double rtol, double *max_ratio)
{
    int64_t bad = 0;
    double worst = 0.0;
    for (int64_t i = 0; i < count; ++i) {
        double r = yref[i], s = S[i], v = (double)ygpu[i];
        if (isnan(r)) {
            if (!isnan(v))
                ++bad;
            continue;
        }
        if (!isfinite(v)) {
            ++bad;
            continue;
        }
        double d = fabs(v - r);
        if (s == 0.0) {
            if (v != 0.0)
                ++bad;
            continue;
        }
        double q = d / s;
        if (q > worst)
            worst = q;
        if (d > rtol * s)
            ++bad;
    }
    if (max_ratio)
        *max_ratio = worst;
    return bad;
}

/* ---- fused gate/up: h = silu(gate) * up ---------------------------------
 *
 * The FlashRT "Qwen3.6 NVFP4 usage" page, environment table (the fused MLP
 * gate/up and fused silu(gate)*up entries): when gate and up share one global
 * scale they run as one NVFP4 projection, followed by silu(gate) * up, with
 * silu(z) = z * sigmoid(z) = z / (1 + exp(-z)) (the SwiGLU gate).
 *
 * This library's fused weight (a reading; the page gives no layout) stacks
 * gate and up rows interleaved in groups of 8: rows 16p..16p+7 are gate rows
 * 8p..8p+7 and rows 16p+8..16p+15 are up rows 8p..8p+7, so gate row f sits
 * at 16*(f/8) + f%8 and up row f 8 rows later.  The row selection is
 * done by the Python wrapper; this file supplies the fp64 arithmetic.
 */
void orc_silu_mul(int64_t count, const double *gate, const double *up, double *h)
{
    for (int64_t i = 0; i < count; ++i)
        h[i] = gate[i] / (1.0 + exp(-gate[i])) * up[i];
}

/*
 * Error bound for h computed from gate' = gate + da and up' = up + db with
 * |da| <= rtol*Sg, |db| <= rtol*Su (the projection's acceptance test):
 *   |silu(gate') up' - silu(gate) up|
 *       <= max|silu'| |da| (|up| + |db|) + |silu(gate)| |db|,
 * and max over z of |silu'(z)| = |sigmoid(z) (1 + z (1 - sigmoid(z)))| is
 * 1.0998 (at z ~ 2.40), taken as 1.1.  The bf16 rounding of the result is
 * added by orc_check_bf16.
 */
void orc_silu_mul_bound(int64_t count, const double *gate, const double *up, const double *Sg,
                        const double *Su, double rtol, double *bound)
{
    for (int64_t i = 0; i < count; ++i) {
        double da = rtol * Sg[i], db = rtol * Su[i];
        double sg = gate[i] / (1.0 + exp(-gate[i]));
        bound[i] = 1.1 * da * (fabs(up[i]) + db) + fabs(sg) * db;
    }
}

/*
 * Acceptance test of bf16 results (bit patterns) against fp64 references:
 *   |h_gpu - h_ref| <= bound + 2^-8 (|h_ref| + bound),
 * the second term covering the round-to-nearest-even to bf16 (relative error
 * at most 2^-9) and the fp32 arithmetic before it.  A NaN h_ref requires a
 * NaN h_gpu; a finite h_ref requires a finite h_gpu.  Returns the number of
 * failing elements; *max_ratio receives the largest |h_gpu - h_ref| over its
 * allowance (diagnostic).
 */
int64_t orc_check_bf16(int64_t count, const double *href, const double *bound,
                       const uint16_t *hgpu, double *max_ratio)
{
    int64_t bad = 0;
    double worst = 0.0;
    for (int64_t i = 0; i < count; ++i) {
        double r = href[i], v = orc_bf16(hgpu[i]);
        if (isnan(r)) {
            if (!isnan(v))
                ++bad;
            continue;
        }
        if (!isfinite(v)) {
            ++bad;
            continue;
        }
        double allow = bound[i] + ldexp(fabs(r) + bound[i], -8);
        double d = fabs(v - r);
        if (allow > 0.0 && d / allow > worst)
            worst = d / allow;
        if (d > allow)
            ++bad;
    }
    if (max_ratio)
        *max_ratio = worst;
    return bad;
}

/* ---- the NVFP4 quantizer: bf16 W -> (codes, e4m3 block scales, g) ---------
 *
 * The FlashRT "Qwen3.6 NVFP4 usage" page (environment-variable table, the MTP
 * checkpoint entry) converts weights to NVFP4 at load time (FP8 -> BF16 ->
 * NVFP4).  The page gives no formula; the reading here is the two-level
 * NVFP4 recipe: a per-tensor fp32 global scale that maps the tensor's largest
 * magnitude to the largest representable product 6 * 448, an e4m3 scale per
 * 16 consecutive k that maps the block's largest magnitude to the largest
 * e2m1 magnitude 6, and each element rounded to the nearest e2m1 value:
 *
 *     amax = max |w|                       (exact; bf16 values)
 *     g    = fp32(amax / 2688)             (one IEEE division; 1 when amax == 0)
 *   per 16-element block b, with amax_b = max over the block of |w|:
 *     s_b  = the e4m3 code in 0..0x7E whose value is nearest to the exact
 *            quotient amax_b / (6 g), ties to the even code (a quotient past
 *            448 therefore gets 448, code 0x7E)
 *   per element, with unit = e4m3(s_b) * g (exact real product):
 *     code = the e2m1 magnitude code in 0..7 whose value is nearest to the
 *            exact quotient |w| / unit, ties to the even code (past 6: 6);
 *            bit 3 = the sign bit of w (so small negatives give code 8, -0)
 *   and every code of a block is 0 when unit == 0 (scale code 0).
 *
 * The quotients are never formed.  The code values v_0 < v_1 < ... are
 * increasing in code order, so the nearest value is found by walking the
 * midpoints (v_c + v_{c+1}) / 2 upward while the quotient lies above them
 * (at a quotient equal to a midpoint: to the even one of c, c+1).  Comparing
 * a / d with a midpoint mu, d > 0, is comparing a with d * mu, and both
 * products below are exact in fp64: 6 * g * mu has at most 2 + 24 + 5 = 31
 * significant bits (g is an fp32 value, an e4m3 midpoint has at most 5) and
 * e4m3(s) * g * mu at most 4 + 24 + 3 = 31 (an e2m1 midpoint has at most 3),
 * far inside fp64's 53 bits and its exponent range, while a (a bf16 value)
 * is exact in fp64 too.  So every decision is exact: no rounding step of the
 * kernel's arithmetic takes part in what the result is.
 */

/* e4m3 code (0..0x7E) nearest to a / (6 g), a >= 0, g > 0, ties to the even code */
static unsigned quant_scale(double a, double g)
{
    unsigned c = 0;
    while (c < 0x7Eu) {
        const double lim = 6.0 * g * ((orc_e4m3(c) + orc_e4m3(c + 1)) / 2.0);
        if (a > lim || (a == lim && ((c + 1) & 1u) == 0))
            ++c;
        else
            break;
    }
    return c;
}

/* e2m1 magnitude code (0..7) nearest to a / unit, a >= 0, unit > 0, ties to
 * the even code */
static unsigned quant_code(double a, double unit)
{
    unsigned c = 0;
    while (c < 7u) {
        const double lim = unit * ((orc_e2m1(c) + orc_e2m1(c + 1)) / 2.0);
        if (a > lim || (a == lim && ((c + 1) & 1u) == 0))
            ++c;
        else
            break;
    }
    return c;
}

/* single-value forms of the two rounding steps (for the tests):
 * the scale code for a block maximum amax_b under global scale g, and the
 * magnitude code of |w| = a under scale code s and global scale g */
unsigned orc_quant_scale(float amax_b, float g) { return quant_scale((double)amax_b, (double)g); }

unsigned orc_quant_code(float a, unsigned s, float g)
{
    const double unit = orc_e4m3(s) * (double)g;
    return unit == 0.0 ? 0u : quant_code((double)a, unit);
}

static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* The global scale of a bf16 tensor of `count` elements. */
float orc_quant_global_scale(int64_t count, const uint16_t *w)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < count; ++i) {
        const float a = fabsf(bf16_to_float(w[i]));
        if (a > amax)
            amax = a;
    }
    return amax == 0.0f ? 1.0f : amax / 2688.0f;
}

/* Quantise rows of w (bf16 [N][K], K % 16 == 0) with global scale g into
 * canonical codes [N][K/2] and scales [N][K/16]. */
void orc_quantize(int64_t N, int64_t K, const uint16_t *w, float g, uint8_t *codes,
                  uint8_t *scales)
{
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < K / 16; ++b) {
            const uint16_t *wb = w + n * K + 16 * b;
            double amax_b = 0.0;
            for (int i = 0; i < 16; ++i) {
                const double a = fabs((double)bf16_to_float(wb[i]));
                if (a > amax_b)
                    amax_b = a;
            }
            const unsigned s = quant_scale(amax_b, (double)g);
            const double unit = orc_e4m3(s) * (double)g;
            scales[n * (K / 16) + b] = (uint8_t)s;
            for (int i = 0; i < 16; i += 2) {
                unsigned q[2];
                for (int j = 0; j < 2; ++j) {
                    const uint16_t bits = wb[i + j];
                    const double a = fabs((double)bf16_to_float(bits));
                    q[j] = unit == 0.0 ? 0u : quant_code(a, unit) | ((bits >> 15) << 3);
                }
                codes[n * (K / 2) + 8 * b + i / 2] = (uint8_t)(q[0] | (q[1] << 4));
            }
        }
    }
}

/* ---- greedy argmax of a logits row --------------------------------------
 *
 * The FlashRT "Qwen3.6 NVFP4 usage" page decodes greedily: each next token is
 * the argmax of the logits row (per-step forward example; the speculative
 * path is greedy-only).  The GPU decides on its fp32 logits, which may order
 * two logits differently from the exact values when they lie within the
 * projection tolerance of each other, so several indices can be correct.
 * For row m with exact logits yref and tolerance bases S (orc_proj):
 *   - a row holding a NaN must return its first NaN column, with a NaN value
 *     (NaN positions are exact: they come from NaN block scales);
 *   - otherwise index i is accepted when yref[i] + rtol*S[i] >= max over j of
 *     (yref[j] - rtol*S[j])  (i can be the largest within tolerance), and the
 *     returned value v when |v - yref[i]| <= rtol*S[i].
 * Returns the number of rejected rows.
 */
int64_t orc_argmax_check(int64_t M, int64_t N, const double *yref, const double *S,
                         double rtol, const int64_t *idx, const float *val)
{
    int64_t bad = 0;
    for (int64_t m = 0; m < M; ++m) {
        const double *yr = yref + m * N, *sr = S + m * N;
        const int64_t i = idx[m];
        const double v = (double)val[m];
        int64_t first_nan = -1;
        double floor_max = -INFINITY;
        for (int64_t j = 0; j < N; ++j) {
            if (isnan(yr[j])) {
                if (first_nan < 0)
                    first_nan = j;
                continue;
            }
            const double lo = yr[j] - rtol * sr[j];
            if (lo > floor_max)
                floor_max = lo;
        }
        if (i < 0 || i >= N) {
            ++bad;
            continue;
        }
        if (first_nan >= 0) {
            if (i != first_nan || !isnan(v))
                ++bad;
            continue;
        }
        const double tol = rtol * sr[i];
        if (!(yr[i] + tol >= floor_max) || !(fabs(v - yr[i]) <= tol))
            ++bad;
    }
    return bad;
}
