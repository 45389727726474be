/*
 * mxq_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 CPU statement of the online activation path of
 * "DuQuant++: block-aligned rotation quantization for MXFP4 activation
 * outliers" (the DuQuant++ page): smooth by a per-channel factor, rotate each
 * 32-element group by one shared 32x32 orthogonal matrix, then MXFP4-encode.
 * Only tests/, the package's smoke check and the bench's CPU-baseline leg
 * may load this library. It shares no code, header, table or helper with the
 * HIP library; it is written from the pages and the OCP MX v1.0 standard.
 *
 * Formulas, with their sources:
 *   smoothing      x'_c = x_c / lambda_c               DuQuant++ page, sec. 3.1
 *                                                       (Y = (X Lambda^-1)(Lambda W))
 *   rotation       y_n = sum_k x'_k * R[k][n]           DuQuant++ page, sec. 3.3
 *                  (row-vector form X * Lambda^-1 * R; R shared by all groups,
 *                  block-diagonal with block size 32: sec. 2.3 and 3.2 step 4)
 *   shared scale   amax of the group, then s = 2^e      DuQuant++ page, sec. 2.1
 *                  e = clamp(floor(log2 amax) - 2, -127, 127) with e = -127 for
 *                  amax = 0; "- 2" is emax of E2M1 (OCP MX v1.0 conversion rule)
 *   element code   nearest E2M1 value of y / 2^e        DuQuant++ page, sec. 2.1
 *                  and 5.1 item 5 (round-to-nearest); ties to the even code,
 *                  saturation at +-6, zero always emitted as +0 (code 0x0)
 *   packing        byte j = code(2j) | code(2j+1) << 4; codes [T][C/2],
 *                  scales [T][C/32] as E8M0 bytes (e + 127)
 *   dequant        (-1)^s * {0,.5,1,1.5,2,3,4,6}[m] * 2^(S-127)  (OCP MX v1.0
 *                  E2M1 and E8M0 tables; S = 255 is NaN)
 *   block size     DuQuant++ page, sec. 4.3 (ablation of the rotation block
 *                  size B in {16, 32, 64, 128}; MXFP4 groups stay 32 wide):
 *                  y_b = x'_b * R_B for every B-channel block b, then the
 *                  encoding of every 32-element group of y
 *   norm in front  DuQuant++ page, sec. 5.2 item 1: the per-channel 1/lambda
 *                  folds into the output of a preceding LayerNorm.  Textbook
 *                  definitions, per token row of C channels:
 *                  RMSNorm   n_c = x_c / sqrt(sum_c x_c^2 / C + eps)
 *                  LayerNorm n_c = (x_c - mu) / sqrt(sum_c (x_c - mu)^2 / C + eps),
 *                            mu = sum_c x_c / C (biased variance)
 *                  then a_c = n_c * gamma_c + beta_c (beta optional) and the
 *                  smoothing, rotation and encoding above applied to a.
 *
 * Parity status: every exported function is pinned by tests/test_oracle_pins.py
 * (worked example of sec. 2.1, brute-force nearest-code search, identity
 * rotation, dense block-diagonal product, norm preservation, scale and sign
 * equivariance, dequant exactness and idempotence); oracle_norm_rotate_quant
 * by the norm pins (closed forms of alternating rows, scale and shift
 * invariance, power-of-two refactoring of gamma and lambda, eps on zero rows,
 * reduction to oracle_rotate_quant); oracle_rotate_quant_block by the block
 * pins (B = 32 equals oracle_rotate_quant, block-diagonal embeddings of
 * smaller blocks, dense products, norm preservation).  No function is
 * unpinned.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no -ffast-math).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GROUP 32

enum { OR_BF16 = 0, OR_FP16 = 1, OR_FP32 = 2, OR_FP64 = 3 };

/* ---- exact upcast of the stored input element to double ---------------- */

static double decode_bf16(uint16_t bits) {
    /* bfloat16 is the upper half of an IEEE binary32 word. */
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

static double decode_fp16(uint16_t bits) {
    /* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
    int sign = (bits >> 15) & 1;
    int ex = (bits >> 10) & 0x1f;
    int fr = bits & 0x3ff;
    double mag;
    if (ex == 0)
        mag = ldexp((double)fr, -24); /* subnormal: fr * 2^-14 * 2^-10 */
    else if (ex == 31)
        mag = fr ? NAN : INFINITY;
    else
        mag = ldexp((double)(fr | 0x400), ex - 25); /* (1024 + fr) * 2^(ex-15-10) */
    return sign ? -mag : mag;
}

static double load_elem(const void *x, int dtype, int64_t i) {
    switch (dtype) {
    case OR_BF16: return decode_bf16(((const uint16_t *)x)[i]);
    case OR_FP16: return decode_fp16(((const uint16_t *)x)[i]);
    case OR_FP32: return (double)((const float *)x)[i];
    default: return ((const double *)x)[i];
    }
}

/* ---- E2M1 element encoding ---------------------------------------------- */

/* Magnitude code (0..7) of the E2M1 value nearest to a >= 0, from the table
 * of decision intervals.  E2M1 values by code: 0, .5, 1, 1.5, 2, 3, 4, 6.
 * A value exactly between two neighbours goes to the one whose code is even
 * (ties-to-even); everything above 5 saturates to 6 (code 7).              */
static int e2m1_magnitude_code(double a) {
    if (a <= 0.25) return 0; /* tie 0.25: 0 (code 0) vs 0.5 (code 1) -> 0   */
    if (a < 0.75) return 1;  /* tie 0.75: 0.5 (1) vs 1 (2)            -> 1  */
    if (a <= 1.25) return 2; /* tie 1.25: 1 (2) vs 1.5 (3)            -> 1  */
    if (a < 1.75) return 3;  /* tie 1.75: 1.5 (3) vs 2 (4)            -> 2  */
    if (a <= 2.5) return 4;  /* tie 2.5 : 2 (4) vs 3 (5)              -> 2  */
    if (a < 3.5) return 5;   /* tie 3.5 : 3 (5) vs 4 (6)              -> 4  */
    if (a <= 5.0) return 6;  /* tie 5   : 4 (6) vs 6 (7)              -> 4  */
    return 7;                /* (5, inf): 6, saturating                     */
}

/* Shared exponent of a group with largest magnitude m (m >= 0):
 * floor(log2 m) - 2, clamped to the E8M0 range [-127, 127]; m = 0 -> -127.
 * floor(log2 m) is taken exactly from frexp: m = f * 2^q with f in [0.5, 1). */
static int shared_exponent(double m) {
    if (!(m > 0.0)) return -127;
    int q;
    (void)frexp(m, &q);
    int e = (q - 1) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* Encode one group of 32 values: E8M0 scale byte and 16 packed code bytes.
 * DuQuant++ page sec. 2.1: find the group amax, derive its shared scale,
 * normalise every element by it and round to the nearest 4-bit float.     */
static void encode_group(const double *y, uint8_t *codes16, uint8_t *scale) {
    double m = 0.0;
    for (int n = 0; n < GROUP; ++n) {
        double a = fabs(y[n]);
        if (a > m) m = a;
    }
    int e = shared_exponent(m);
    *scale = (uint8_t)(e + 127);
    uint8_t c[GROUP];
    for (int n = 0; n < GROUP; ++n) {
        double v = ldexp(y[n], -e); /* exact: scaling by a power of two */
        int mag = e2m1_magnitude_code(fabs(v));
        int neg = signbit(v) && mag != 0; /* zero is always +0 (0x0) */
        c[n] = (uint8_t)((neg ? 8 : 0) | mag);
    }
    for (int j = 0; j < GROUP / 2; ++j)
        codes16[j] = (uint8_t)(c[2 * j] | (c[2 * j + 1] << 4));
}

/* ---- exported entry points ---------------------------------------------- */

/* Encode already-rotated values: y fp64 [n_groups][32] -> codes, scales. */
int oracle_encode_groups(const double *y, int64_t n_groups, uint8_t *codes, uint8_t *scales) {
    if (n_groups < 0) return 2;
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < n_groups; ++g)
        encode_group(y + g * GROUP, codes + g * (GROUP / 2), scales + g);
    return 0;
}

/* Plain MXFP4 quantization of x [tokens][stride] (first `channels` used). */
int oracle_quant(const void *x, int dtype, int64_t tokens, int64_t channels, int64_t stride,
                 uint8_t *codes, uint8_t *scales) {
    if (tokens < 0 || channels < 0 || channels % GROUP != 0 || stride < channels) return 2;
    const int64_t gpr = channels / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < tokens; ++t) {
        double y[GROUP];
        for (int64_t g = 0; g < gpr; ++g) {
            for (int k = 0; k < GROUP; ++k)
                y[k] = load_elem(x, dtype, t * stride + g * GROUP + k);
            encode_group(y, codes + (t * gpr + g) * (GROUP / 2), scales + t * gpr + g);
        }
    }
    return 0;
}

/* Smoothing of one element: x' = x / lambda_c (lambda NULL: all ones). */
static double smooth(double v, const float *lambda, int64_t c) {
    return lambda ? v / (double)lambda[c] : v;
}

/* y_n = sum_k x'_k R[k][n], n, k < B, for one block of B channels
 * (row-vector product; R holds the block in its top-left B x B corner). */
static void rotate_block(const double *xs, const double R[128][128], int B, double *y) {
    for (int n = 0; n < B; ++n) {
        double acc = 0.0;
        for (int k = 0; k < B; ++k)
            acc += xs[k] * R[k][n];
        y[n] = acc;
    }
}

/* Smooth + rotate + quantize (DuQuant++ page sec. 3.3 online side):
 *   x'  = x / lambda (lambda NULL means all ones)        sec. 3.1
 *   y_g = x'_g * R for every 32-channel group g           sec. 3.2 step 4, 3.3
 *   codes, scales = MXFP4(y)                              sec. 2.1
 * r is the shared 32x32 block, row-major, y_n = sum_k x'_k r[k][n]; r_dtype
 * is OR_BF16 (bits) or OR_FP64.  y_out (fp64 [tokens][channels]) may be NULL. */
int oracle_rotate_quant(const void *x, int dtype, int64_t tokens, int64_t channels, int64_t stride,
                        const float *lambda, const void *r, int r_dtype,
                        uint8_t *codes, uint8_t *scales, double *y_out) {
    if (tokens < 0 || channels < 0 || channels % GROUP != 0 || stride < channels) return 2;
    double R[128][128];
    for (int k = 0; k < GROUP; ++k)
        for (int n = 0; n < GROUP; ++n)
            R[k][n] = load_elem(r, r_dtype, k * GROUP + n);
    const int64_t gpr = channels / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < tokens; ++t) {
        double xs[GROUP], y[GROUP];
        for (int64_t g = 0; g < gpr; ++g) {
            for (int k = 0; k < GROUP; ++k) {
                int64_t c = g * GROUP + k;
                double v = load_elem(x, dtype, t * stride + c);
                xs[k] = smooth(v, lambda, c);
            }
            rotate_block(xs, R, GROUP, y);
            if (y_out)
                for (int n = 0; n < GROUP; ++n)
                    y_out[t * channels + g * GROUP + n] = y[n];
            encode_group(y, codes + (t * gpr + g) * (GROUP / 2), scales + t * gpr + g);
        }
    }
    return 0;
}

/* Rotation by a B x B block (B = 16, 32, 64 or 128; r is B x B, row-major,
 * y_n = sum_k x'_k r[k][n] within each block of B channels), then MXFP4 of
 * every 32-element group of the rotated row.  channels must be a multiple
 * of B and of 32.  y_out, when not NULL, receives the rotated values. */
int oracle_rotate_quant_block(const void *x, int dtype, int64_t tokens, int64_t channels, int64_t stride,
                              const float *lambda, const void *r, int r_dtype, int block,
                              uint8_t *codes, uint8_t *scales, double *y_out) {
    if (block != 16 && block != 32 && block != 64 && block != 128) return 3;
    if (tokens < 0 || channels < 0 || channels % block != 0 || channels % GROUP != 0 || stride < channels)
        return 2;
    double R[128][128];
    for (int k = 0; k < block; ++k)
        for (int n = 0; n < block; ++n)
            R[k][n] = load_elem(r, r_dtype, k * block + n);
    const int64_t gpr = channels / GROUP;
    int status = 0;
#pragma omp parallel
    {
        double *row = (double *)malloc((size_t)(channels > 0 ? channels : 1) * sizeof(double));
        if (!row) {
#pragma omp atomic write
            status = 4;
        }
#pragma omp for schedule(static)
        for (int64_t t = 0; t < tokens; ++t) {
            if (!row) continue;
            double xs[128];
            for (int64_t b0 = 0; b0 < channels; b0 += block) {
                for (int k = 0; k < block; ++k) {
                    int64_t c = b0 + k;
                    xs[k] = smooth(load_elem(x, dtype, t * stride + c), lambda, c);
                }
                rotate_block(xs, R, block, row + b0);
            }
            for (int64_t g = 0; g < gpr; ++g)
                encode_group(row + g * GROUP, codes + (t * gpr + g) * (GROUP / 2), scales + t * gpr + g);
            if (y_out)
                for (int64_t c = 0; c < channels; ++c) y_out[t * channels + c] = row[c];
        }
        free(row);
    }
    return status;
}

/* RMSNorm (norm_kind 0) or LayerNorm (norm_kind 1) of every row, then
 * gamma, beta, smoothing, rotation and encoding as in oracle_rotate_quant.
 * y_out, when not NULL, receives the rotated values [tokens][channels]. */
int oracle_norm_rotate_quant(const void *x, int dtype, int64_t tokens, int64_t channels, int64_t stride,
                             int norm_kind, const float *gamma, const float *beta, double eps,
                             const float *lambda, const void *r, int r_dtype,
                             uint8_t *codes, uint8_t *scales, double *y_out) {
    if (tokens < 0 || channels <= 0 || channels % GROUP != 0 || stride < channels) return 2;
    if (norm_kind != 0 && norm_kind != 1) return 3;
    if (!gamma) return 1;
    double R[128][128];
    for (int k = 0; k < GROUP; ++k)
        for (int n = 0; n < GROUP; ++n)
            R[k][n] = load_elem(r, r_dtype, k * GROUP + n);
    const int64_t gpr = channels / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < tokens; ++t) {
        /* row statistics */
        double mu = 0.0;
        if (norm_kind == 1) {
            double sum = 0.0;
            for (int64_t c = 0; c < channels; ++c) sum += load_elem(x, dtype, t * stride + c);
            mu = sum / (double)channels;
        }
        double sq = 0.0;
        for (int64_t c = 0; c < channels; ++c) {
            double d = load_elem(x, dtype, t * stride + c) - mu;
            sq += d * d;
        }
        const double inv = 1.0 / sqrt(sq / (double)channels + eps);
        double xs[GROUP], y[GROUP];
        for (int64_t g = 0; g < gpr; ++g) {
            for (int k = 0; k < GROUP; ++k) {
                int64_t c = g * GROUP + k;
                double n = (load_elem(x, dtype, t * stride + c) - mu) * inv;
                double a = n * (double)gamma[c] + (beta ? (double)beta[c] : 0.0);
                xs[k] = smooth(a, lambda, c);
            }
            rotate_block(xs, R, GROUP, y);
            if (y_out)
                for (int n = 0; n < GROUP; ++n)
                    y_out[t * channels + g * GROUP + n] = y[n];
            encode_group(y, codes + (t * gpr + g) * (GROUP / 2), scales + t * gpr + g);
        }
    }
    return 0;
}

/* Dequantize: value = (-1)^s * E2M1[m] * 2^(S - 127); S = 255 gives NaN. */
int oracle_dequant(const uint8_t *codes, const uint8_t *scales, int64_t tokens, int64_t channels,
                   double *out) {
    static const double e2m1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    if (tokens < 0 || channels < 0 || channels % GROUP != 0) return 2;
    const int64_t gpr = channels / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < tokens; ++t) {
        for (int64_t c = 0; c < channels; ++c) {
            uint8_t byte = codes[t * (channels / 2) + c / 2];
            int code = (c & 1) ? (byte >> 4) : (byte & 0xf);
            int S = scales[t * gpr + c / GROUP];
            double mag = e2m1[code & 7];
            double v = (S == 255) ? NAN : ldexp(mag, S - 127);
            out[t * channels + c] = (code & 8) ? -v : v;
        }
    }
    return 0;
}

/* Threads OpenMP would use (reported next to oracle timings). */
int oracle_num_threads(void) {
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
