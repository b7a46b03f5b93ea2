/*
 * CPU oracle for the segmented MXFP8 GEMM -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load or call this code.  The product (the HIP library) never does, and
 * this file shares no code, table or constant generator with it.
 *
 * What it computes, written out plainly and slowly:
 *
 *   C[m,n] = bf16_rne( sum_{r<R} sum_{k<kPerRank}
 *              deq(A_seg[r][m][k],  sA_seg[r][m][k/32])
 *            * deq(B[n][r*kPerRank+k], sB[n][(r*kPerRank+k)/32]) )
 *
 *   deq(q, s) = e4m3fn_value(q) * 2^(s - 127)
 *
 * Sources (cannbot-harness 0.1.5 package diff):
 *  - all_to_all_matmul.cpp, host buffer sizing: A is m*k FP8 bytes, B is
 *    k*n FP8 bytes, the scales hold CeilDiv(k,64)*2 bytes per row (one E8M0
 *    byte per 32 K-elements), the output is m*n two-byte elements.
 *  - all_to_all_comm_udma.h, PutSegmentToRank / PutScaleToRank: the sender's
 *    A is split into R segments [R][M][kPerRank], scales [R][M][kPerRank/32];
 *    the receiver keeps the piece from source rank r in slot r.
 *  - all_to_all_matmul_impl.h, SetupParams: every rank's segment is
 *    accumulated on-core (splitKNum = rankSize), i.e. the result is the sum
 *    over all R segments; kernel entry E4M3E4M3: A and B are fp8_e4m3fn,
 *    scales fp8_e8m0, C bfloat16, B transposed ([N][K], K contiguous).
 *  - verify_result.py: the output is compared as bfloat16.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - The sum is taken in double, r ascending then k ascending, and rounded
 *    once, directly from double, to bfloat16 with round-to-nearest-even.
 *  - E4M3 is the OCP "FN" variant: bias 7, no infinities, 0x7F/0xFF NaN,
 *    largest finite 448, subnormal step 2^-9.
 *  - Quantiser (the golden generator is not on the pages): per block of 32
 *    consecutive K-elements of one row, e = the smallest integer with
 *    448 * 2^e >= amax (that is 2^ceil(log2(amax/448))), clamped to
 *    [-127, 127], amax = 0 giving -127; the scale byte is e + 127 and each
 *    element is encoded as e4m3_rne(x * 2^-e), keeping the sign of zero.
 *  - Non-finite inputs.  A block holding a NaN has no exponent: its scale
 *    is the E8M0 NaN byte 0xFF and every code of the block is the NaN code
 *    0x7F (x divided by a NaN scale is NaN).  A block holding an infinity
 *    (and no NaN) has amax = +inf, for which no integer e satisfies the
 *    rule; the clamp gives e = 127 (byte 0xFE), infinities encode as the
 *    largest finite code of their sign (E4M3 has no infinity; the encoder
 *    saturates) and the finite elements encode as usual.
 *  - An E8M0 scale byte 0xFF in a GEMM input is NaN, so every output whose
 *    sum takes a product from that block is NaN.
 *
 * The other FP8 operand formats (all_to_all_matmul_impl.h, the sibling
 * kernel entries E5M2E5M2, E4M3E5M2 and E5M2E4M3): either operand may be
 * E5M2 instead, the OCP OFP8 format with bias 15, IEEE-style infinities
 * (0x7C / 0xFC) and NaNs (0x7D-0x7F, 0xFD-0xFF), largest finite 57344 and
 * subnormal step 2^-16.  Its quantiser uses 57344 in place of 448 and
 * saturates to 57344 (MX conversions saturate).  Format codes below: 0 =
 * E4M3, 1 = E5M2.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- E4M3 --- */

/* Value of an E4M3FN code (NaN for 0x7F / 0xFF). */
double oracle_e4m3_value(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int expo = (code >> 3) & 0xF;
    int mant = code & 0x7;
    double v;
    if (expo == 0xF && mant == 0x7)
        return NAN;
    if (expo == 0)
        v = ldexp((double)mant, -9);                /* mant/8 * 2^(1-7) */
    else
        v = ldexp(1.0 + (double)mant / 8.0, expo - 7);
    return sign ? -v : v;
}

/* E4M3FN code of v, round-to-nearest-even.  Magnitudes above 448 after
 * rounding, infinities included, saturate to 448 (the quantiser produces
 * them only from infinite inputs); NaN gives 0x7F. */
uint8_t oracle_e4m3_encode(double v)
{
    uint8_t sign;
    double a;
    if (isnan(v))
        return 0x7F;
    sign = signbit(v) ? 0x80 : 0x00;
    a = fabs(v);
    if (isinf(a))
        return (uint8_t)(sign | 0x7E);
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: multiples of 2^-9; q == 8 is the smallest
         * normal, whose code is also 8 */
        double q = rint(ldexp(a, 9));
        return (uint8_t)(sign | (uint8_t)q);
    } else {
        int E;
        double f = frexp(a, &E);        /* a = f * 2^E, f in [0.5, 1) */
        int e = E - 1;                  /* a in [2^e, 2^(e+1)) */
        double q = rint(ldexp(f, 4));   /* a / 2^(e-3), in [8, 16] */
        int iq = (int)q;
        if (iq == 16) {
            iq = 8;
            e += 1;
        }
        if (e > 8 || (e == 8 && iq > 14))
            return (uint8_t)(sign | 0x7E);          /* saturate at 448 */
        return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | (iq - 8)));
    }
}

/* ---------------------------------------------------------------- E5M2 --- */

/* Value of an E5M2 code (infinities at 0x7C / 0xFC, NaN above them). */
double oracle_e5m2_value(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int expo = (code >> 2) & 0x1F;
    int mant = code & 0x3;
    double v;
    if (expo == 0x1F)
        return mant == 0 ? (sign ? -INFINITY : INFINITY) : NAN;
    if (expo == 0)
        v = ldexp((double)mant, -16);               /* mant/4 * 2^(1-15) */
    else
        v = ldexp(1.0 + (double)mant / 4.0, expo - 15);
    return sign ? -v : v;
}

/* E5M2 code of v, round-to-nearest-even; magnitudes above 57344 after
 * rounding (infinities included) saturate to 57344, NaN gives 0x7F. */
uint8_t oracle_e5m2_encode(double v)
{
    uint8_t sign;
    double a;
    if (isnan(v))
        return 0x7F;
    sign = signbit(v) ? 0x80 : 0x00;
    a = fabs(v);
    if (isinf(a))
        return (uint8_t)(sign | 0x7B);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: multiples of 2^-16; q == 4 is the smallest
         * normal, whose code is also 4 */
        double q = rint(ldexp(a, 16));
        return (uint8_t)(sign | (uint8_t)q);
    } else {
        int E;
        double f = frexp(a, &E);        /* a = f * 2^E, f in [0.5, 1) */
        int e = E - 1;                  /* a in [2^e, 2^(e+1)) */
        double q = rint(ldexp(f, 3));   /* a / 2^(e-2), in [4, 8] */
        int iq = (int)q;
        if (iq == 8) {
            iq = 4;
            e += 1;
        }
        if (e > 15 || (e == 15 && iq > 7))
            return (uint8_t)(sign | 0x7B);          /* saturate at 57344 */
        return (uint8_t)(sign | (uint8_t)(((e + 15) << 2) | (iq - 4)));
    }
}

/* Value of a code of format fmt (0 = E4M3, 1 = E5M2). */
double oracle_fp8_value(uint8_t code, int fmt)
{
    return fmt ? oracle_e5m2_value(code) : oracle_e4m3_value(code);
}

/* --------------------------------------------------------------- E8M0 --- */

/* Smallest integer e with 448 * 2^e >= amax, clamped to [-127, 127]
 * (amax = 0 gives -127, amax = +inf the clamp 127).  A NaN amax has no such
 * e and gives 128, whose scale byte e + 127 is the E8M0 NaN 0xFF. */
int oracle_e8m0_exponent(double amax)
{
    int E, e;
    double f;
    if (isnan(amax))
        return 128;
    if (isinf(amax))
        return 127;
    if (!(amax > 0.0))
        return -127;
    f = frexp(amax, &E);                 /* amax = f * 2^E, f in [0.5, 1) */
    /* 448 = 0.875 * 2^9: amax <= 448 * 2^e  <=>  f * 2^E <= 0.875 * 2^(e+9) */
    e = (f <= 0.875) ? E - 9 : E - 8;
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return e;
}

/* Smallest integer e with 57344 * 2^e >= amax (the E5M2 largest finite),
 * clamped to [-127, 127]; non-finite amax as oracle_e8m0_exponent. */
int oracle_e8m0_exponent_e5m2(double amax)
{
    int E, e;
    double f;
    if (isnan(amax))
        return 128;
    if (isinf(amax))
        return 127;
    if (!(amax > 0.0))
        return -127;
    f = frexp(amax, &E);
    /* 57344 = 0.875 * 2^16: amax <= 57344 * 2^e <=> f * 2^E <= 0.875 * 2^(e+16) */
    e = (f <= 0.875) ? E - 16 : E - 15;
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return e;
}

/* Quantise a row-major [rows][cols] float32 matrix (cols % 32 == 0) into
 * codes [rows][cols] of format fmt and scale bytes [rows][cols/32]. */
void oracle_quantize_mx(const float* x, int64_t rows, int64_t cols,
                        uint8_t* q, uint8_t* s, int fmt)
{
    int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* blk = x + i * cols + b * 32;
            double amax = 0.0;
            int e, j, has_nan = 0;
            for (j = 0; j < 32; ++j) {
                double a = fabs((double)blk[j]);
                if (isnan(a))
                    has_nan = 1;
                else if (a > amax)
                    amax = a;
            }
            if (has_nan) {
                /* no exponent: NaN scale, every element NaN */
                s[i * nb + b] = 0xFF;
                for (j = 0; j < 32; ++j)
                    q[i * cols + b * 32 + j] = 0x7F;
                continue;
            }
            e = fmt ? oracle_e8m0_exponent_e5m2(amax) : oracle_e8m0_exponent(amax);
            s[i * nb + b] = (uint8_t)(e + 127);
            for (j = 0; j < 32; ++j) {
                double y = ldexp((double)blk[j], -e);
                q[i * cols + b * 32 + j] = fmt ? oracle_e5m2_encode(y) : oracle_e4m3_encode(y);
            }
        }
    }
}

/* --------------------------------------------------------------- BF16 --- */

/* bfloat16 bits of v, rounded once from double to nearest-even.
 * bfloat16 normals keep 8 significant bits; below 2^-126 the step is 2^-133;
 * magnitudes that round past the largest finite value become infinity. */
uint16_t oracle_bf16_from_double(double v)
{
    double a, r;
    float rf;
    uint32_t bits;
    int neg;
    if (isnan(v))
        return 0x7FC0;
    neg = signbit(v) ? 1 : 0;
    a = fabs(v);
    if (isinf(a)) {
        r = a;
    } else if (a < ldexp(1.0, -126)) {
        r = ldexp(rint(ldexp(a, 133)), -133);
    } else {
        int E;
        double f = frexp(a, &E);          /* a = f * 2^E, f in [0.5, 1) */
        r = ldexp(rint(ldexp(f, 8)), E - 8);
    }
    /* r is now a bfloat16 value (or >= 2^128, i.e. infinity): the float
     * conversion below is exact and its low 16 bits are zero */
    rf = (float)r;
    memcpy(&bits, &rf, 4);
    return (uint16_t)((bits >> 16) | (neg ? 0x8000u : 0u));
}

/* ------------------------------------------------------------- GEMM ----- */

/* Value of an E8M0 scale byte: 2^(s-127); 0xFF is NaN. */
static double e8m0_value(uint8_t s)
{
    if (s == 0xFF)
        return NAN;
    return ldexp(1.0, (int)s - 127);
}

/* One output element, summed in double, r ascending then k ascending. */
static double dot_entry(const double* lut_a, const double* lut_b,
                        const uint8_t* a_seg, const uint8_t* sa_seg,
                        const uint8_t* b, const uint8_t* sb,
                        int64_t R, int64_t M, int64_t kpr, int64_t m, int64_t n)
{
    int64_t K = R * kpr;
    int64_t nbs = kpr / 32, nbk = K / 32;
    double acc = 0.0;
    for (int64_t r = 0; r < R; ++r) {
        const uint8_t* arow = a_seg + (r * M + m) * kpr;
        const uint8_t* asrow = sa_seg + (r * M + m) * nbs;
        for (int64_t k = 0; k < kpr; ++k) {
            int64_t kg = r * kpr + k;
            double av = lut_a[arow[k]] * e8m0_value(asrow[k / 32]);
            double bv = lut_b[b[n * K + kg]] * e8m0_value(sb[n * nbk + kg / 32]);
            acc += av * bv;
        }
    }
    return acc;
}

static void fill_lut(double* lut, int fmt)
{
    for (int c = 0; c < 256; ++c)
        lut[c] = oracle_fp8_value((uint8_t)c, fmt);
}

/* Full C [M][N] as bfloat16 bits; A codes of format fmt_a, B of fmt_b.
 *   a_seg  [R][M][kpr]      sa_seg [R][M][kpr/32]
 *   b      [N][R*kpr]       sb     [N][R*kpr/32]          */
void oracle_mxgemm_seg(const uint8_t* a_seg, const uint8_t* sa_seg,
                       const uint8_t* b, const uint8_t* sb,
                       int64_t R, int64_t M, int64_t kpr, int64_t N,
                       uint16_t* c, int fmt_a, int fmt_b)
{
    double lut_a[256], lut_b[256];
    fill_lut(lut_a, fmt_a);
    fill_lut(lut_b, fmt_b);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            c[m * N + n] = oracle_bf16_from_double(
                dot_entry(lut_a, lut_b, a_seg, sa_seg, b, sb, R, M, kpr, m, n));
}

/* Selected entries only: c[i] = C[ms[i], ns[i]] as bfloat16 bits, and, if
 * exact != NULL, the unrounded double sum. */
void oracle_mxgemm_seg_entries(const uint8_t* a_seg, const uint8_t* sa_seg,
                               const uint8_t* b, const uint8_t* sb,
                               int64_t R, int64_t M, int64_t kpr, int64_t N,
                               const int64_t* ms, const int64_t* ns, int64_t count,
                               uint16_t* c, double* exact, int fmt_a, int fmt_b)
{
    double lut_a[256], lut_b[256];
    (void)N;
    fill_lut(lut_a, fmt_a);
    fill_lut(lut_b, fmt_b);
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < count; ++i) {
        double v = dot_entry(lut_a, lut_b, a_seg, sa_seg, b, sb, R, M, kpr, ms[i], ns[i]);
        c[i] = oracle_bf16_from_double(v);
        if (exact)
            exact[i] = v;
    }
}

/* Rows [m0, m1) of C, for a bounded timing sample. */
void oracle_mxgemm_seg_rows(const uint8_t* a_seg, const uint8_t* sa_seg,
                            const uint8_t* b, const uint8_t* sb,
                            int64_t R, int64_t M, int64_t kpr, int64_t N,
                            int64_t m0, int64_t m1, uint16_t* c, int fmt_a, int fmt_b)
{
    double lut_a[256], lut_b[256];
    fill_lut(lut_a, fmt_a);
    fill_lut(lut_b, fmt_b);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = m0; m < m1; ++m)
        for (int64_t n = 0; n < N; ++n)
            c[(m - m0) * N + n] = oracle_bf16_from_double(
                dot_entry(lut_a, lut_b, a_seg, sa_seg, b, sb, R, M, kpr, m, n));
}

/* Elementwise helpers exposed for the pins. */
void oracle_e4m3_encode_array(const double* v, int64_t n, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_encode(v[i]);
}

void oracle_e4m3_value_array(const uint8_t* codes, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_value(codes[i]);
}

void oracle_e8m0_exponent_array(const double* amax, int64_t n, int32_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e8m0_exponent(amax[i]);
}

void oracle_e5m2_encode_array(const double* v, int64_t n, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e5m2_encode(v[i]);
}

void oracle_e5m2_value_array(const uint8_t* codes, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e5m2_value(codes[i]);
}

void oracle_e8m0_exponent_e5m2_array(const double* amax, int64_t n, int32_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e8m0_exponent_e5m2(amax[i]);
}

void oracle_bf16_from_double_array(const double* v, int64_t n, uint16_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_from_double(v[i]);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
