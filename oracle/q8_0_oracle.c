/*
 * q8_0_oracle.c -- plain, slow, serial CPU oracle for the Q8_0 decode matvec.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table
 * or constant with the HIP library in q8_block_quantized_gemv_amd/csrc.
 *
 * What it computes (page "IV.4: One command buffer per token", section
 * "Eight kernels", the q8_matvec kernel and the prose after it; and the
 * exact-float reference in section "The correctness ladder", rung one):
 *
 *   A Q8_0 weight matrix W with p rows and n columns (n a multiple of 32) is
 *   stored as p rows of n/32 consecutive 34-byte blocks.  Block b of row r
 *   holds an IEEE binary16 scale d in bytes 0..1 (little endian) followed by
 *   32 two's-complement int8 quants q_0..q_31 in bytes 2..33.  The weight of
 *   column 32b+j is d * q_j.  The matvec is
 *
 *       y[r] = sum_b d(r,b) * sum_j q(r,b,j) * x[32b+j].
 *
 * The oracle evaluates that definition in the order it is written, in IEEE
 * double: per block, the inner sum S = sum_j q_j * x_j (each product exact in
 * double: 8 + 24 significant bits), then the block's share d * S is added to
 * the row sum, blocks in column order; y is rounded once to float at the end.
 * Scaling once per block, after the inner sum, is also how the page's kernel
 * is organised, so an infinite scale gives an infinite (not NaN) result when
 * the block's inner sum is finite and non-zero.  The oracle also returns
 * mag[r] = sum_b |d| * sum_j |q_j * x_j| = sum |w x|, the magnitude that
 * scales the parity tolerance.
 *
 * Pins (see tests/test_oracle_pins.py): brute force against a dense float64
 * dequantize-then-matmul built from numpy's own binary16 decoding, the page's
 * scale bytes 0x00 0x2c (= 0.0625), zero-scale and all-ones invariants, an
 * integer-exact case checked against exact rational arithmetic, and the
 * exhaustive binary16 table against numpy.
 *
 * The integer path (q8o_quantize_x, q8o_gemv_q8q8) follows the CPU kernel the
 * same page sets beside q8_matvec (section "Eight kernels", the note after the
 * kernel; and page "minfer Metal Backend Design", ADR-0013): the activations
 * are quantized to Q8_0 blocks too and each block's dot product is an integer
 * sum of quant products.  The pages do not print the quantization rule; the
 * reading taken is written at q8o_quantize_x.  Its pins: closed-form blocks
 * (scales that are powers of two, ties at .5, the all-zero block), the
 * dequantization error bound, numpy's binary16 cast for the scale encoding,
 * brute force for the integer dot, and the distance to the float matvec.
 */
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <math.h>

#define Q8O_BLOCK_QUANTS 32
#define Q8O_BLOCK_BYTES 34

/*
 * IEEE 754-2008 binary16 -> double, from the format definition:
 *   sign s (bit 15), biased exponent e (bits 14..10), fraction f (bits 9..0)
 *   e == 0      : (-1)^s * f * 2^-24            (zero and subnormals)
 *   1 <= e <= 30: (-1)^s * (1024 + f) * 2^(e-25)
 *   e == 31     : f == 0 ? (-1)^s * inf : NaN
 */
double q8o_f16_to_double(uint16_t bits)
{
    int s = (bits >> 15) & 1;
    int e = (bits >> 10) & 0x1f;
    int f = bits & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + f), e - 25);
    }
    return s ? -v : v;
}

/*
 * One row: returns the float64 sum and writes sum |t| to *mag.
 * row points at the row's first block; n is the column count.
 */
static double q8o_row(const uint8_t *row, const float *x, int64_t n, double *mag)
{
    double acc = 0.0;
    double m = 0.0;
    int64_t nblocks = n / Q8O_BLOCK_QUANTS;
    for (int64_t b = 0; b < nblocks; ++b) {
        const uint8_t *blk = row + b * Q8O_BLOCK_BYTES;
        uint16_t bits = (uint16_t)(blk[0] | ((uint16_t)blk[1] << 8));
        double d = q8o_f16_to_double(bits);
        double s = 0.0;
        double sa = 0.0;
        for (int j = 0; j < Q8O_BLOCK_QUANTS; ++j) {
            int q = (int)(int8_t)blk[2 + j];
            double t = (double)q * (double)x[b * Q8O_BLOCK_QUANTS + j];
            s += t;
            sa += fabs(t);
        }
        acc += d * s;
        m += fabs(d) * sa;
    }
    *mag = m;
    return acc;
}

/*
 * y[r] (float, rounded once from the double sum), y64[r] (the double sum)
 * and mag[r] (sum of |d*q*x|) for r < p.  Any of y, y64, mag may be NULL.
 * Returns 0, or -1 when n is not a positive multiple of 32 or p < 0.
 */
int q8o_gemv(const uint8_t *w, const float *x, int64_t n, int64_t p,
             float *y, double *y64, double *mag)
{
    if (n <= 0 || n % Q8O_BLOCK_QUANTS != 0 || p < 0)
        return -1;
    int64_t row_bytes = (n / Q8O_BLOCK_QUANTS) * Q8O_BLOCK_BYTES;
    for (int64_t r = 0; r < p; ++r) {
        double m;
        double acc = q8o_row(w + r * row_bytes, x, n, &m);
        if (y) y[r] = (float)acc;
        if (y64) y64[r] = acc;
        if (mag) mag[r] = m;
    }
    return 0;
}

/*
 * Small-batch product: m independent matvecs, X row-major m x n, Y row-major
 * m x p, Y[i][r] = the matvec of row r against X[i].  Outputs as in q8o_gemv.
 */
int q8o_gemm(const uint8_t *w, const float *X, int64_t m, int64_t n, int64_t p,
             float *Y, double *Y64, double *MAG)
{
    if (m < 0)
        return -1;
    for (int64_t i = 0; i < m; ++i) {
        int rc = q8o_gemv(w, X + i * n, n, p,
                          Y ? Y + i * p : NULL,
                          Y64 ? Y64 + i * p : NULL,
                          MAG ? MAG + i * p : NULL);
        if (rc != 0)
            return rc;
    }
    return 0;
}

/*
 * float -> IEEE binary16, rounding to nearest with ties to even, from the
 * format definition: a value a in [2^e, 2^(e+1)) with e >= -14 has the
 * spacing 2^(e-10); below 2^-14 the spacing is 2^-24 (subnormals).  Values at
 * or above 65520 (the midpoint between 65504 and 2^16) become infinity.
 */
uint16_t q8o_f32_to_f16(float vf)
{
    double v = (double)vf;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(a))
        return (uint16_t)(sign | 0x7e00);
    if (a >= 65520.0)
        return (uint16_t)(sign | 0x7c00);
    if (a == 0.0)
        return sign;
    int ex;
    frexp(a, &ex);
    int e = ex - 1;
    if (e < -14)
        e = -14;
    double ulp = ldexp(1.0, e - 10);
    double r = nearbyint(a / ulp) * ulp;   /* a / ulp is exact; ties go to even */
    if (r == 0.0)
        return sign;
    frexp(r, &ex);
    e = ex - 1;
    if (e < -14)
        return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(r / ldexp(1.0, e - 10) - 1024.0));
}

/*
 * x (n floats, n a positive multiple of 32) -> n/32 Q8_0 blocks of 34 bytes,
 * the layout of a weight row.  Reading of the pages' "quantize activations
 * to Q8_0" (the rule itself is not printed): per block of 32,
 *   amax = max_j |x_j|                                  (float32, exact)
 *   d    = amax / 127                                   (float32 division)
 *   q_j  = x_j / d rounded to the nearest integer, halves away from zero
 *          (float32 division; every q_j is 0 when d == 0)
 *   the stored scale is d rounded to binary16 (nearest, ties to even).
 * Every decision is a float32 operation, so an implementation doing the same
 * IEEE operations produces the same bytes.  x must be finite.
 * Returns 0, or -1 for a bad n.
 */
int q8o_quantize_x(const float *x, int64_t n, uint8_t *out)
{
    if (n <= 0 || n % Q8O_BLOCK_QUANTS != 0)
        return -1;
    for (int64_t b = 0; b < n / Q8O_BLOCK_QUANTS; ++b) {
        const float *xb = x + b * Q8O_BLOCK_QUANTS;
        uint8_t *o = out + b * Q8O_BLOCK_BYTES;
        float amax = 0.0f;
        for (int j = 0; j < Q8O_BLOCK_QUANTS; ++j) {
            float a = fabsf(xb[j]);
            if (a > amax)
                amax = a;
        }
        float d = amax / 127.0f;
        uint16_t db = q8o_f32_to_f16(d);
        o[0] = (uint8_t)(db & 0xff);
        o[1] = (uint8_t)(db >> 8);
        for (int j = 0; j < Q8O_BLOCK_QUANTS; ++j) {
            int q = 0;
            if (d != 0.0f) {
                float t = xb[j] / d;
                q = (int)roundf(t);
            }
            o[2 + j] = (uint8_t)(int8_t)q;
        }
    }
    return 0;
}

/*
 * The integer matvec: x quantized as q8o_quantize_x does, then per row
 *   y[r] = sum_b d_w(r,b) * d_x(b) * sum_j q_w(r,b,j) * q_x(b,j)
 * with the inner sum in integers (exact) and the blocks added in double, in
 * column order (each block's share is exact in double: 11 + 11 + 20 bits).
 * mag[r] = sum_b |d_w d_x| * sum_j |q_w q_x|.  Outputs as in q8o_gemv.
 * Returns 0, -1 for a bad shape, -2 if out of memory.
 */
int q8o_gemv_q8q8(const uint8_t *w, const float *x, int64_t n, int64_t p,
                  float *y, double *y64, double *mag)
{
    if (n <= 0 || n % Q8O_BLOCK_QUANTS != 0 || p < 0)
        return -1;
    int64_t nblocks = n / Q8O_BLOCK_QUANTS;
    int64_t row_bytes = nblocks * Q8O_BLOCK_BYTES;
    uint8_t *xq = (uint8_t *)malloc((size_t)row_bytes);
    if (!xq)
        return -2;
    q8o_quantize_x(x, n, xq);
    for (int64_t r = 0; r < p; ++r) {
        const uint8_t *row = w + r * row_bytes;
        double acc = 0.0;
        double m = 0.0;
        for (int64_t b = 0; b < nblocks; ++b) {
            const uint8_t *wb = row + b * Q8O_BLOCK_BYTES;
            const uint8_t *xb = xq + b * Q8O_BLOCK_BYTES;
            double dw = q8o_f16_to_double((uint16_t)(wb[0] | ((uint16_t)wb[1] << 8)));
            double dx = q8o_f16_to_double((uint16_t)(xb[0] | ((uint16_t)xb[1] << 8)));
            int64_t isum = 0;
            int64_t iabs = 0;
            for (int j = 0; j < Q8O_BLOCK_QUANTS; ++j) {
                int64_t prod = (int64_t)(int8_t)wb[2 + j] * (int64_t)(int8_t)xb[2 + j];
                isum += prod;
                iabs += prod < 0 ? -prod : prod;
            }
            acc += (dw * dx) * (double)isum;
            m += fabs(dw * dx) * (double)iabs;
        }
        if (y) y[r] = (float)acc;
        if (y64) y64[r] = acc;
        if (mag) mag[r] = m;
    }
    free(xq);
    return 0;
}
