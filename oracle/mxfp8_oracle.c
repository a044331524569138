/*
 * CPU oracle for the low-bit KV cache: MXFP8 rows (E4M3 elements, one E8M0
 * power-of-two scale per block of 32 elements).
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this file's library.  It shares no code with the
 * GPU library and never calls it.
 *
 * "Understanding and Exploiting Diagonal Attention Sparsity in Autoregressive
 * Image Generation" (Section 6, related work on KV quantization) calls KV
 * quantization orthogonal to the diagonal selection and stackable with it; the
 * pages fix no format.  The format here is the OCP Microscaling (MX) v1.0
 * MXFP8 E4M3 format: per block of 32 values a shared exponent
 * X = floor(log2(max |v|)) - 8 (8 = the largest exponent of E4M3), stored as
 * the E8M0 byte X + 127, and each element the E4M3 value nearest to v / 2^X.
 *
 * Readings taken where the format leaves a step open:
 *   - rounding to nearest, ties to the even code (the even significand);
 *   - |v / 2^X| beyond 448 (the largest E4M3 value) saturates to +-448;
 *   - an all-zero block takes the smallest scale, X = -127 (byte 0);
 *   - X is clamped to [-127, 127] (never reached by bf16 inputs of normal size).
 * The quantisation is exact arithmetic: v / 2^X is exact, so the only decision
 * is the rounding, taken here by scanning the table of E4M3 values.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

/* Value of an E4M3 (OCP, "fn": no infinities, S.1111.111 is NaN) code. */
double oracle_e4m3_value(int code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = e == 0 ? m * ldexp(1.0, -9) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return s ? -mag : mag;
}

/* The E4M3 code nearest to y (ties to the even code), saturating at +-448. */
static int nearest_e4m3(double y) {
    int sign = y < 0 || (y == 0 && signbit(y));
    double a = fabs(y);
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) { /* non-negative finite codes, ascending */
        double err = fabs(oracle_e4m3_value(c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return best | (sign << 7);
}

/* Shared exponent of a block: floor(log2(amax)) - 8, clamped; -127 for an all-zero block. */
static int shared_exponent(const double* v, int n) {
    double amax = 0.0;
    for (int i = 0; i < n; ++i)
        if (fabs(v[i]) > amax) amax = fabs(v[i]);
    if (amax == 0.0) return -127;
    int x = (int)floor(log2(amax)) - 8;
    /* floor(log2()) of an exact power of two or of values just below one must not
     * be off by one: fix it against the definition 2^(x+8) <= amax < 2^(x+9) */
    while (ldexp(1.0, x + 8) > amax) --x;
    while (ldexp(1.0, x + 9) <= amax) ++x;
    if (x < -127) x = -127;
    if (x > 127) x = 127;
    return x;
}

/*
 * Quantise n_blocks blocks of 32 values: codes[32 * b + i], scales[b] = X_b + 127.
 * Returns 0.
 */
int oracle_mxfp8_quantize(const double* v, int n_blocks, uint8_t* codes, uint8_t* scales) {
    for (int b = 0; b < n_blocks; ++b) {
        const double* blk = v + (size_t)32 * b;
        int x = shared_exponent(blk, 32);
        scales[b] = (uint8_t)(x + 127);
        for (int i = 0; i < 32; ++i) codes[(size_t)32 * b + i] = (uint8_t)nearest_e4m3(ldexp(blk[i], -x));
    }
    return 0;
}

/* Dequantise: out[32 * b + i] = value(codes[32 * b + i]) * 2^(scales[b] - 127). */
int oracle_mxfp8_dequantize(const uint8_t* codes, const uint8_t* scales, int n_blocks, double* out) {
    for (int b = 0; b < n_blocks; ++b)
        for (int i = 0; i < 32; ++i)
            out[(size_t)32 * b + i] = ldexp(oracle_e4m3_value(codes[(size_t)32 * b + i]), (int)scales[b] - 127);
    return 0;
}
