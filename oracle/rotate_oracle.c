/*
 * Incoherent-processing oracle -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.
 *
 * Plain, slow CPU definitions of the step that precedes low-precision
 * attention on page "FlashAttention-3 (DE)", systems-analysis.ru, section 3
 * of the technical innovations (low precision with reduced quantisation
 * error): the feature vectors of Q and K are multiplied by a random
 * orthogonal matrix -- a Hadamard matrix with random signs -- which spreads
 * outlier features over all coordinates; the rotated tensors are then
 * quantised to FP8; since the matrix is orthogonal, Q K^T is unchanged.
 *
 * Readings of what the page leaves open (listed in the design notes):
 *   - the matrix is M = D H / sqrt(d): D = diag(sigma) with sigma_i = -1
 *     where bit i of the sign mask is set (+1 otherwise), H the d x d
 *     Sylvester-Hadamard matrix H[i][j] = (-1)^popcount(i & j); rows of the
 *     tensor are row vectors, so the rotated row is y = x M;
 *   - quantisation is per tensor: s = max|y| / 448 (s = 1 for an all-zero
 *     tensor), code = OCP E4M3 of y / s rounded to nearest, ties to even,
 *     saturated at +-448 (the same convention as the plain FP8 inputs).
 *
 * Everything here is IEEE double precision written from those definitions:
 * the dense product (d^2 multiply-adds per row, no fast transform) and an
 * encoder that picks the E4M3 value nearest to its argument.  No code is
 * shared with the GPU library.
 *
 * Build: compiled into the same liboracle.so as attn_oracle.c.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

enum { RO_BF16 = 0, RO_F64 = 2, RO_F32 = 3 };

static double ro_load(const void* x, int dtype, int64_t idx) {
    if (dtype == RO_BF16) {
        uint32_t bits = ((uint32_t)((const uint16_t*)x)[idx]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    if (dtype == RO_F32) return (double)((const float*)x)[idx];
    return ((const double*)x)[idx];
}

static int popcount64(uint64_t v) {
    int c = 0;
    while (v) { v &= v - 1; ++c; }
    return c;
}

/* Sylvester-Hadamard entry H[i][j] = (-1)^popcount(i & j). */
double oracle_hadamard_entry(int64_t i, int64_t j) {
    return (popcount64((uint64_t)(i & j)) & 1) ? -1.0 : 1.0;
}

/*
 * y[r, :] = x[r, :] D H / sqrt(d) for every row r (rotate != 0), or y = x
 * (rotate == 0).  sign_bits holds d bits (bit i of word i/32); NULL means no
 * sign flips.  d must be a power of two.  Returns 0, or -1 on invalid input.
 */
int oracle_rotate(const void* x, int dtype, int64_t rows, int64_t d, const uint32_t* sign_bits,
                  int rotate, double* y) {
    if (rows < 0 || d <= 0 || (d & (d - 1)) != 0) return -1;
    if (dtype != RO_BF16 && dtype != RO_F32 && dtype != RO_F64) return -1;
    const double norm = 1.0 / sqrt((double)d);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double* out = y + r * d;
        if (!rotate) {
            for (int64_t j = 0; j < d; ++j) out[j] = ro_load(x, dtype, r * d + j);
            continue;
        }
        for (int64_t j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int64_t i = 0; i < d; ++i) {
                double xi = ro_load(x, dtype, r * d + i);
                if (sign_bits && ((sign_bits[i >> 5] >> (i & 31)) & 1)) xi = -xi;
                acc += xi * oracle_hadamard_entry(i, j);
            }
            out[j] = acc * norm;
        }
    }
    return 0;
}

/* The finite E4M3 magnitudes in increasing order: code c (0..126) has
 * magnitude value_of(c); 127 is NaN.  Exponent field e (bias 7), mantissa m:
 * e == 0 -> m/8 * 2^-6 (subnormal), else (1 + m/8) * 2^(e-7). */
static double e4m3_mag(int c) {
    int e = c >> 3, m = c & 7;
    return e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
}

/* Encode v: the E4M3 value nearest to v, ties to the even code (mantissa
 * bit 0 clear), magnitudes above 448 saturate to 448.  NaN is not handled. */
uint8_t oracle_e4m3_encode(double v) {
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a >= 448.0) return sign | 126;
    /* the largest code lo with magnitude <= a (binary search over 0..126,
     * whose magnitudes increase with the code) */
    int lo = 0, top = 126;
    while (lo < top) {
        const int mid = (lo + top + 1) / 2;
        if (e4m3_mag(mid) <= a) lo = mid;
        else top = mid - 1;
    }
    if (e4m3_mag(lo) == a || lo == 126) return sign | (uint8_t)lo;
    const int hi = lo + 1;
    const double dlo = a - e4m3_mag(lo), dhi = e4m3_mag(hi) - a;
    int c;
    if (dlo < dhi) c = lo;
    else if (dhi < dlo) c = hi;
    else c = (lo & 1) ? hi : lo;   /* tie: the even code */
    return sign | (uint8_t)c;
}

/* codes[k] = E4M3(y[k] / s) for a given scale s (the encoding step of the
 * per-tensor quantisation below, for a subset of a tensor). */
void oracle_encode_scaled(const double* y, int64_t n, double s, uint8_t* codes) {
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < n; ++k) codes[k] = oracle_e4m3_encode(y[k] / s);
}

/*
 * Per-tensor quantisation of n values: amax = max |y|, s = amax / 448 (1 when
 * amax == 0), codes[k] = E4M3(y[k] / s).  *scale receives s.
 */
void oracle_quantize_e4m3(const double* y, int64_t n, double* scale, uint8_t* codes) {
    double amax = 0.0;
    for (int64_t k = 0; k < n; ++k) {
        double a = fabs(y[k]);
        if (a > amax) amax = a;
    }
    const double s = amax > 0.0 ? amax / 448.0 : 1.0;
    *scale = s;
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < n; ++k) codes[k] = oracle_e4m3_encode(y[k] / s);
}
