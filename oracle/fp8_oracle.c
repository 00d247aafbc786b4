/*
 * fp8_oracle.c -- plain, slow, scalar CPU oracle of per-tensor FP8 delayed scaling.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU
 * baseline may load this library.  It shares no code, header, table or constant with the
 * HIP library; the product never calls it.
 *
 * Sources.  The method is the FP8 linear-layer path discussed on three TransformerEngine
 * pull-request pages:
 *   [UB]   "[PyTorch] Userbuffers support in operation-based API" (PR 1142)
 *   [WS]   "[PyTorch] Refactor FP8 workspaces in linear modules" (PR 820)
 *   [CG]   "[PyTorch] cuda graph support" (PR 575)
 * The pages never define the FP8 bit formats; those follow the OCP "8-bit Floating Point
 * Specification (OFP8)" E4M3 and E5M2 encodings.  Every reading taken where the pages are
 * silent is listed in the design notes and repeated at the function that uses it.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC (no FTZ/DAZ,
 * so float32 subnormals are kept exactly as IEEE 754 defines them).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORC_E4M3 0
#define ORC_E5M2 1

/* ---------------------------------------------------------------------------------------
 * Formats (OCP OFP8).  E4M3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent
 * 1..15 are normal, exponent 0 subnormal; S.1111.111 is NaN and there is no infinity.
 * E5M2: 1 sign, 5 exponent bits (bias 15), 2 mantissa bits, IEEE-like: exponent 31 is
 * infinity (mantissa 0) or NaN.
 * ------------------------------------------------------------------------------------- */
static int fmt_mbits(int fmt) { return fmt == ORC_E4M3 ? 3 : 2; }
static int fmt_ebits(int fmt) { return fmt == ORC_E4M3 ? 4 : 5; }
static int fmt_bias(int fmt) { return fmt == ORC_E4M3 ? 7 : 15; }

/* Value of an FP8 code, by the closed form of its bit fields. */
double orc_fp8_decode(uint8_t code, int fmt)
{
    int mb = fmt_mbits(fmt), eb = fmt_ebits(fmt), bias = fmt_bias(fmt);
    int sign = code >> 7;
    int e = (code >> mb) & ((1 << eb) - 1);
    int m = code & ((1 << mb) - 1);
    double v;
    if (fmt == ORC_E4M3) {
        if (e == 15 && m == 7) return NAN;
    } else if (e == 31) {
        if (m != 0) return NAN;
        return sign ? -INFINITY : INFINITY;
    }
    if (e == 0)
        v = ldexp((double)m, 1 - bias - mb);                 /* m / 2^mb * 2^(1-bias) */
    else
        v = ldexp((double)((1 << mb) + m), e - bias - mb);   /* (1 + m/2^mb) * 2^(e-bias) */
    return sign ? -v : v;
}

/* Largest finite code of a format (positive sign). */
static uint8_t fmt_maxcode(int fmt) { return fmt == ORC_E4M3 ? 0x7E : 0x7B; }

/* Largest finite magnitude: 448 (E4M3) or 57344 (E5M2), read off the decoder. */
double orc_fp8_max(int fmt) { return orc_fp8_decode(fmt_maxcode(fmt), fmt); }

/* Smallest normal exponent, 1 - bias: -6 (E4M3) or -14 (E5M2). */
static int fmt_emin(int fmt) { return 1 - fmt_bias(fmt); }

/*
 * Encode a float32 into FP8, saturating, round-to-nearest-even.
 *   NaN              -> 0x7F, the positive all-ones NaN code of both formats, whatever the
 *                       NaN's sign bit (IEEE 754 leaves the sign of a NaN made by an invalid
 *                       operation such as inf * 0 unspecified, so it carries no information);
 *   |f| > max finite -> the largest finite code with the input's sign (also for +-inf);
 *   otherwise        -> |f| rounded to the nearest point of the format's grid, ties to the
 *                       point with an even significand; a zero result keeps the sign.
 * All grid arithmetic is in float64, where it is exact: the quantum q is a power of two and
 * |f| / q has at most 24 significant bits.
 */
uint8_t orc_fp8_encode(float f, int fmt)
{
    int mb = fmt_mbits(fmt), bias = fmt_bias(fmt), emin = fmt_emin(fmt);
    uint8_t sign = signbit(f) ? 0x80 : 0x00;
    double a, maxv, q, r, v;
    int ex, e, ebits, mant;

    if (isnan(f)) return 0x7F;
    a = fabs((double)f);
    maxv = orc_fp8_max(fmt);
    if (a > maxv) return (uint8_t)(fmt_maxcode(fmt) | sign);
    if (a == 0.0) return sign;

    (void)frexp(a, &ex);                      /* a = fr * 2^ex, fr in [0.5, 1) */
    e = ex - 1;                               /* floor(log2 a) */
    if (e < emin) e = emin;                   /* below the normal range: subnormal quantum */
    q = ldexp(1.0, e - mb);
    r = nearbyint(a / q);                     /* default rounding mode: to nearest, ties even */
    v = r * q;
    if (v == 0.0) return sign;

    (void)frexp(v, &ex);                      /* rounding may have carried into the next binade */
    e = ex - 1;
    if (e < emin) {                           /* subnormal: exponent field 0 */
        ebits = 0;
        mant = (int)(v / ldexp(1.0, emin - mb));
    } else {
        ebits = e + bias;
        mant = (int)(v / ldexp(1.0, e - mb)) - (1 << mb);
    }
    return (uint8_t)(sign | (ebits << mb) | mant);
}

/*
 * An independent second encoder, for cross-checking orc_fp8_encode: the nearest of all
 * finite non-negative codes by direct search (ties to the code whose last mantissa bit is
 * 0), with the same NaN and saturation rules.
 */
uint8_t orc_fp8_encode_search(float f, int fmt)
{
    uint8_t sign = signbit(f) ? 0x80 : 0x00;
    double a, best_d = INFINITY;
    int c, best = 0;
    if (isnan(f)) return 0x7F;
    a = fabs((double)f);
    if (a > orc_fp8_max(fmt)) return (uint8_t)(fmt_maxcode(fmt) | sign);   /* saturation, incl. inf */
    for (c = 0; c < 0x80; ++c) {
        double v = orc_fp8_decode((uint8_t)c, fmt), d;
        if (!isfinite(v)) continue;
        d = fabs(v - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best_d = d;
            best = c;
        }
    }
    return (uint8_t)(sign | best);
}

/* Bulk helpers over arrays, for the tests. */
void orc_fp8_encode_n(const float *x, int64_t n, int fmt, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_encode(x[i], fmt);
}
void orc_fp8_encode_search_n(const float *x, int64_t n, int fmt, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_encode_search(x[i], fmt);
}
void orc_fp8_decode_n(const uint8_t *c, int64_t n, int fmt, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_decode(c[i], fmt);
}

/* bfloat16 is the top half of a float32: exact widening. */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * Amax: the largest magnitude of the high-precision input, before scaling ([WS] Motivations,
 * first bullet, names the recipe's amax; [CG] feature list: amaxes are reduced per iteration).
 * A NaN input makes the amax NaN.  The result folds into *amax by the same rule.
 */
static float amax_fold(float acc, float v)
{
    float a = fabsf(v);
    if (isnan(acc) || isnan(a)) return NAN;
    return a > acc ? a : acc;
}

/*
 * Cast to FP8 with amax capture ([CG] transpose-cache thread: Float8Tensor.to_float8; [WS]
 * Motivations, first bullet: the cast uses the current scale).  Per element the scaled value
 * is one float32 IEEE product, y = float(x) * scale, then y is encoded as above: two
 * roundings in all.  The private inverse scale the cast records is 1/scale (see
 * orc_scale_inv).  *amax_slot accumulates the largest |x| (it is read and written).
 */
void orc_cast_amax(const uint16_t *x, int64_t n, float scale, int fmt, uint8_t *out, float *amax_slot)
{
    float amax = *amax_slot;
    for (int64_t i = 0; i < n; ++i) {
        float f = bf16_to_f32(x[i]);
        float y = f * scale;
        out[i] = orc_fp8_encode(y, fmt);
        amax = amax_fold(amax, f);
    }
    *amax_slot = amax;
}

/*
 * Cast plus transpose: the row-major FP8 tensor and its transpose cache ([WS] "grown in
 * scope" first bullet, the Float8Tensor transpose cache; [CG] DbiasCastTranspose example,
 * cast_transpose creates an FP8 tensor with its transpose cache).
 * x is [rows, cols] row-major; out is [rows, cols]; out_t is [cols, rows], out_t[j][i] = out[i][j].
 */
void orc_cast_transpose(const uint16_t *x, int64_t rows, int64_t cols, float scale, int fmt,
                        uint8_t *out, uint8_t *out_t, float *amax_slot)
{
    orc_cast_amax(x, rows * cols, scale, fmt, out, amax_slot);
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j)
            out_t[j * rows + i] = out[i * cols + j];
}

/*
 * Transpose of an FP8 tensor that already exists: the lazy fill of a Float8Tensor's transpose
 * cache ([WS] "grown in scope" first bullet: transpose_2d(cache=True) and lazy transpose
 * caching; [CG] transpose-cache thread: dy.transpose() of an FP8 dy that carries no cached
 * transpose).  The codes are moved, never re-encoded: in is [rows, cols] row-major and out_t
 * is [cols, rows] with out_t[j][i] = in[i][j].
 */
void orc_fp8_transpose(const uint8_t *in, int64_t rows, int64_t cols, uint8_t *out_t)
{
    for (int64_t j = 0; j < cols; ++j)
        for (int64_t i = 0; i < rows; ++i)
            out_t[j * rows + i] = in[i * cols + j];
}

/*
 * Cast of a float32 tensor with amax capture: the quantisation of an FP8 GEMM's output
 * written straight into an FP8 tensor ([CG] transpose-cache thread: fp8_gemm(..., out=dx._data)
 * in FP8Linear.backward).  Same two roundings as orc_cast_amax: y = x * scale in float32,
 * then the saturating nearest-even encode; *amax_slot accumulates the largest |x|.
 */
void orc_cast_f32_amax(const float *x, int64_t n, float scale, int fmt, uint8_t *out, float *amax_slot)
{
    float amax = *amax_slot;
    for (int64_t i = 0; i < n; ++i) {
        float y = x[i] * scale;
        out[i] = orc_fp8_encode(y, fmt);
        amax = amax_fold(amax, x[i]);
    }
    *amax_slot = amax;
}

/*
 * Bias gradient: the column sum of dy ([CG] DbiasCastTranspose example: db = dy.sum(dim=0)),
 * taken from the bfloat16 dy before any cast, accumulated in float64.
 */
void orc_dbias(const uint16_t *dy, int64_t rows, int64_t cols, double *db)
{
    for (int64_t j = 0; j < cols; ++j) db[j] = 0.0;
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j)
            db[j] += (double)bf16_to_f32(dy[i * cols + j]);
}

/* The private inverse scale a cast records ([WS] Motivations, first and second bullets):
 * the correctly rounded float32 quotient 1/scale. */
float orc_scale_inv(float scale) { return 1.0f / scale; }

/*
 * Delayed-scaling update of T tensors' scales from their amax histories ([WS] Motivations,
 * first bullet: the scale-update kernel, and a fix for amaxes small enough to make the scale
 * infinite; [CG] feature list: amaxes reduced within the current iteration).
 *
 * hist is [L][T] float32, row 0 = the current iteration's amaxes.  For each tensor t:
 *   a      = max over the L rows of hist[.][t]          (the current amax and L-1 earlier ones)
 *   s      = (fp8_max / a) * 2^-margin                   (float32: one division, one exact
 *                                                         power-of-two product)
 *   guard  : keep the previous scale if a == 0, a is not finite, s is not finite, or 1/s is
 *            not finite (s == 0, or s so small that its float32 inverse overflows)
 *   scale[t] = s; scale_inv[t] = 1/s (float32)
 *   history: every row moves one place towards row 0 (row i takes row i+1), row L-1 takes
 *            the old row 0 (the amax just used), and row 0 is cleared for the next iteration.
 * fmt[t] selects fp8_max.  margin is an integer in [-126, 126].
 */
void orc_scale_update(float *hist, int64_t L, int64_t T, float *scale, float *scale_inv,
                      const int32_t *fmt, int32_t margin)
{
    float *old = hist;
    for (int64_t t = 0; t < T; ++t) {
        float a = 0.0f, s, fmax = (float)orc_fp8_max(fmt[t]);
        float p = (float)ldexp(1.0, -margin);
        float row0;
        int64_t i;
        for (i = 0; i < L; ++i) {
            float h = old[i * T + t];
            if (isnan(h) || isnan(a)) a = NAN;
            else if (h > a) a = h;
        }
        s = (fmax / a) * p;
        if (a == 0.0f || !isfinite(a) || !isfinite(s) || !isfinite(1.0f / s)) s = scale[t];
        scale[t] = s;
        scale_inv[t] = 1.0f / s;
        row0 = old[t];
        for (i = 0; i + 1 < L; ++i) hist[i * T + t] = old[(i + 1) * T + t];
        hist[(L - 1) * T + t] = row0;
        hist[t] = 0.0f;
    }
}

/*
 * Dequantise an [rows, k] FP8 operand with leading dimension ld into float64, one value per
 * code by the closed form (the contraction itself is done by the caller with a float64
 * matrix product; see the Python wrapper).
 */
void orc_dequant(const uint8_t *a, int64_t rows, int64_t k, int64_t ld, int fmt, double *out)
{
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < k; ++j)
            out[i * k + j] = orc_fp8_decode(a[i * ld + j], fmt);
}

/*
 * Scalar float64 FP8 GEMM with dequantisation and bias, the plain definition
 * ([CG] transpose-cache thread: fp8_gemm on FP8 data; [UB] each output chunk adds its own
 * chunk of the bias):
 *   R[m][n] = (sum_k dec(A[m][k]) * dec(B[n][k])) * a_sinv * b_sinv + bias[n]
 * A is [M, K] (leading dimension lda), B is [N, K] (ldb), bias is bfloat16 [N] or NULL,
 * R is [M, N] (ldr).  Used for small shapes and as a check of the matrix-product path.
 */
void orc_gemm_bias_scalar(const uint8_t *A, int fa, float a_sinv, int64_t lda,
                          const uint8_t *B, int fb, float b_sinv, int64_t ldb,
                          const uint16_t *bias, int64_t M, int64_t N, int64_t K,
                          double *R, int64_t ldr)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += orc_fp8_decode(A[m * lda + k], fa) * orc_fp8_decode(B[n * ldb + k], fb);
            acc = acc * (double)a_sinv * (double)b_sinv;
            if (bias) acc += (double)bf16_to_f32(bias[n]);
            R[m * ldr + n] = acc;
        }
}
