/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the scaled_mm
 * hot path (per-token dynamic FP8 quantization, W8A8 INT8, FP8 with
 * per-token x per-channel scales, Block-FP8, bf16 GEMM, the MXFP4 quantizer
 * and GEMM, and the INT4 weight-only quantizer and GEMM).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header or table with the HIP path.
 *
 * Sources (the pages these definitions follow):
 *   - "Helion in vLLM: A Unified Route to Tunable Linear Kernels", section
 *     "What the integration changes": the three quantized formats (FP8 dynamic
 *     quantization, W8A8 INT8, Block-FP8) and the ordinary / Split-K / Swap-AB
 *     strategies, which all compute the same GEMM.
 *   - vLLM PR #53446 "Hopper (SM90) tuned config for batch-invariant
 *     persistent matmul", sections "Summary" and "Test Plan": a bf16 matmul
 *     whose output rows do not depend on the batch size.
 *   The pages give no formulas; the scale rule (absmax / 448, e4m3), the
 *   per-row / per-column / 128x128 / 1x128 scale shapes and the INT8 epilogue
 *   order (acc * sa[m] * sb[n] in fp32, then bf16) are the plainest reading of
 *   the workloads these pages describe, listed as readings in the design notes.
 *
 * Arithmetic rules:
 *   - integer sums in int64 (exact);
 *   - floating sums in double (fp64).  Products of two e4m3 values or two bf16
 *     values are exact in double, and for the sizes used here the fp8 sums are
 *     exact as well (at most 8+8 significant bits per product, |sum| < 2^31);
 *   - the quantizer and the INT8 epilogue are defined in fp32 and are computed
 *     in fp32 here (x86-64 SSE arithmetic, built with -ffp-contract=off so no
 *     multiply-add is fused).
 *
 * Layouts: A is [M][K] row-major, B (weights) is [N][K] row-major, outputs are
 * [rows][N] where rows is an explicit list of output rows (so that a sample of
 * a very large problem can be checked one row at a time).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent field 0 holds subnormals m * 2^-9; exponent field 15 with
 * mantissa 7 is NaN; there is no infinity; the largest finite value is
 * 2^8 * 1.75 = 448 (code 0x7E). */
double oracle_e4m3_decode(uint8_t c)
{
    int sign = c >> 7;
    int e = (c >> 3) & 15;
    int m = c & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* Round-to-nearest, ties-to-even encode of a finite value of magnitude at most
 * 448 into e4m3.  Definition: among the non-negative finite codes 0x00..0x7E
 * (whose values increase with the code), pick the one nearest to |v|; on an
 * exact tie pick the code whose last mantissa bit is 0.  The sign bit is the
 * sign of v, also when the magnitude rounds to zero.  Returns 0xFF (NaN) for
 * an input outside the domain, which callers treat as an error. */
uint8_t oracle_e4m3_encode_rne(float v)
{
    double a;
    int lo, hi, mid, best;
    double dlo, dhi;
    uint8_t sign;
    if (!(fabsf(v) <= 448.0f))
        return 0xFF;
    sign = signbit(v) ? 0x80 : 0x00;
    a = fabs((double)v);
    /* binary search: largest code in [0, 0x7E] whose value is <= a */
    lo = 0;
    hi = 0x7E;
    while (lo < hi) {
        mid = (lo + hi + 1) / 2;
        if (oracle_e4m3_decode((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    best = lo;
    if (lo < 0x7E) {
        dlo = a - oracle_e4m3_decode((uint8_t)lo);
        dhi = oracle_e4m3_decode((uint8_t)(lo + 1)) - a;
        if (dhi < dlo || (dhi == dlo && ((lo + 1) & 1) == 0))
            best = lo + 1;
    }
    return (uint8_t)(sign | best);
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
float oracle_bf16_decode(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round-to-nearest, ties-to-even of a finite binary32 to bfloat16.
 * Definition: the two bfloat16 neighbours of f are f with its low 16 bits
 * cleared (same sign, smaller or equal magnitude) and the next bfloat16 away
 * from zero; pick the nearer, on a tie the one with an even last bit.  A
 * magnitude that rounds past the largest finite bfloat16 gives infinity (the
 * infinity pattern is then taken to stand for 2^128, as IEEE 754 prescribes). */
uint16_t oracle_bf16_encode_rne(float f)
{
    uint32_t u, ulo, uhi;
    double a, vlo, vhi;
    memcpy(&u, &f, 4);
    if (isnan(f))
        return 0x7FC0;
    ulo = u & 0xFFFF0000u;
    if (ulo == u)
        return (uint16_t)(u >> 16);
    uhi = ulo + 0x10000u; /* next bfloat16 away from zero (same sign) */
    a = fabs((double)f);
    vlo = fabs((double)oracle_bf16_decode((uint16_t)(ulo >> 16)));
    if (((uhi >> 16) & 0x7FFF) == 0x7F80)
        vhi = ldexp(1.0, 128);
    else
        vhi = fabs((double)oracle_bf16_decode((uint16_t)(uhi >> 16)));
    if (vhi - a < a - vlo)
        return (uint16_t)(uhi >> 16);
    if (a - vlo < vhi - a)
        return (uint16_t)(ulo >> 16);
    return ((ulo >> 16) & 1) ? (uint16_t)(uhi >> 16) : (uint16_t)(ulo >> 16);
}

/* ------------------------------------------------------------------------ */
/* Dynamic FP8 quantization (FP8 dynamic quantization / Block-FP8 formats of  */
/* "What the integration changes")                                           */
/* ------------------------------------------------------------------------ */

/* Quantize one group of n bf16 values (stride 1) with the rule
 *   amax = max |x|;  s = amax / 448 (fp32);  q = e4m3_rne(clamp(x / s, +-448))
 * A group whose values are all zero gets s = 0 and all-zero codes.
 * Returns 0 on success, -1 on a non-finite input. */
static int quantize_group(const uint16_t* x, int64_t n, int64_t stride,
                          uint8_t* q, float* s_out)
{
    float amax = 0.0f, s, v;
    int64_t i;
    for (i = 0; i < n; ++i) {
        float xi = oracle_bf16_decode(x[i * stride]);
        if (!isfinite(xi))
            return -1;
        if (fabsf(xi) > amax)
            amax = fabsf(xi);
    }
    s = amax / 448.0f;
    *s_out = s;
    for (i = 0; i < n; ++i) {
        if (s == 0.0f) {
            q[i * stride] = 0x00;
            continue;
        }
        v = oracle_bf16_decode(x[i * stride]) / s;
        if (v > 448.0f)
            v = 448.0f;
        if (v < -448.0f)
            v = -448.0f;
        q[i * stride] = oracle_e4m3_encode_rne(v);
    }
    return 0;
}

/* Per-token (G == K) or per-1xG-group activation quantization.
 * x: bf16 [M][K]; q: e4m3 [M][K]; s: fp32 [M][K/G].  G must divide K. */
int oracle_quantize_fp8(const uint16_t* x, int64_t M, int64_t K, int64_t G,
                        uint8_t* q, float* s)
{
    int64_t m, g, ng;
    int bad = 0;
    if (G <= 0 || K % G != 0)
        return -2;
    ng = K / G;
#pragma omp parallel for private(g) reduction(| : bad) schedule(static)
    for (m = 0; m < M; ++m)
        for (g = 0; g < ng; ++g)
            bad |= quantize_group(x + m * K + g * G, G, 1, q + m * K + g * G,
                                  &s[m * ng + g]) != 0;
    return bad ? -1 : 0;
}

/* Weight quantization with one scale per BN x BK block of the [N][K] weight
 * (Block-FP8: 128 x 128).  s: fp32 [ceil(N/BN)][K/BK]; an N edge block holds
 * the rows that exist.  BK must divide K. */
int oracle_quantize_fp8_block(const uint16_t* w, int64_t N, int64_t K,
                              int64_t BN, int64_t BK, uint8_t* q, float* s)
{
    int64_t nb, kb, nnb, nkb;
    int bad = 0;
    if (BN <= 0 || BK <= 0 || K % BK != 0)
        return -2;
    nnb = (N + BN - 1) / BN;
    nkb = K / BK;
#pragma omp parallel for private(kb) reduction(| : bad) schedule(static)
    for (nb = 0; nb < nnb; ++nb) {
        for (kb = 0; kb < nkb; ++kb) {
            int64_t r0 = nb * BN, r1 = r0 + BN < N ? r0 + BN : N, r, i;
            float amax = 0.0f, sc;
            for (r = r0; r < r1; ++r)
                for (i = 0; i < BK; ++i) {
                    float xi = oracle_bf16_decode(w[r * K + kb * BK + i]);
                    if (!isfinite(xi))
                        bad = 1;
                    else if (fabsf(xi) > amax)
                        amax = fabsf(xi);
                }
            sc = amax / 448.0f;
            s[nb * nkb + kb] = sc;
            for (r = r0; r < r1; ++r)
                for (i = 0; i < BK; ++i) {
                    float v;
                    uint8_t* dst = &q[r * K + kb * BK + i];
                    if (sc == 0.0f) {
                        *dst = 0x00;
                        continue;
                    }
                    v = oracle_bf16_decode(w[r * K + kb * BK + i]) / sc;
                    if (v > 448.0f)
                        v = 448.0f;
                    if (v < -448.0f)
                        v = -448.0f;
                    *dst = oracle_e4m3_encode_rne(v);
                }
        }
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* GEMMs.  rows[r] names the output row of A that output row r holds.        */
/* ------------------------------------------------------------------------ */

/* W8A8 INT8 accumulators: acc[r][n] = sum_k A[rows[r]][k] * B[n][k], exact. */
void oracle_gemm_int8_acc(const int8_t* A, const int8_t* B, int64_t M, int64_t N,
                          int64_t K, const int64_t* rows, int64_t nrows,
                          int64_t* acc)
{
    int64_t r, n, k;
    (void)M;
#pragma omp parallel for private(n, k) collapse(2) schedule(static)
    for (r = 0; r < nrows; ++r)
        for (n = 0; n < N; ++n) {
            const int8_t* a = A + rows[r] * K;
            const int8_t* b = B + n * K;
            int64_t sum = 0;
            for (k = 0; k < K; ++k)
                sum += (int64_t)a[k] * (int64_t)b[k];
            acc[r * N + n] = sum;
        }
}

/* W8A8 INT8 epilogue, defined in fp32: y = (float(acc) * sa[m]) * sb[n], two
 * separately rounded multiplies, the left one first. */
void oracle_epilogue_int8(const int64_t* acc, const float* sa, const float* sb,
                          int64_t N, const int64_t* rows, int64_t nrows,
                          float* y)
{
    int64_t r, n;
#pragma omp parallel for private(n) schedule(static)
    for (r = 0; r < nrows; ++r)
        for (n = 0; n < N; ++n) {
            float a = (float)acc[r * N + n];
            float t = a * sa[rows[r]];
            y[r * N + n] = t * sb[n];
        }
}

/* (The fp8 GEMMs decode through a 256-entry table filled by
 * oracle_e4m3_decode, i.e. the same definition, evaluated once per code.)
 *
 * FP8 with per-token x per-channel scales:
 *   ref[r][n] = sa[m] * sb[n] * sum_k dec(A[m][k]) * dec(B[n][k])   (fp64)
 * absref[r][n] = |sa[m] * sb[n]| * sum_k |dec(A[m][k]) * dec(B[n][k])|
 * (absref feeds the a-priori error bound of any fp32 summation order). */
void oracle_gemm_fp8(const uint8_t* A, const uint8_t* B, const float* sa,
                     const float* sb, int64_t M, int64_t N, int64_t K,
                     const int64_t* rows, int64_t nrows, double* ref,
                     double* absref)
{
    int64_t r, n, k;
    double dec[256];
    (void)M;
    for (k = 0; k < 256; ++k)
        dec[k] = oracle_e4m3_decode((uint8_t)k);
#pragma omp parallel for private(n, k) collapse(2) schedule(static)
    for (r = 0; r < nrows; ++r)
        for (n = 0; n < N; ++n) {
            const uint8_t* a = A + rows[r] * K;
            const uint8_t* b = B + n * K;
            double sum = 0.0, asum = 0.0, sc;
            for (k = 0; k < K; ++k) {
                double p = dec[a[k]] * dec[b[k]];
                sum += p;
                asum += fabs(p);
            }
            sc = (double)sa[rows[r]] * (double)sb[n];
            ref[r * N + n] = sc * sum;
            if (absref)
                absref[r * N + n] = fabs(sc) * asum;
        }
}

/* Block-FP8: with G = 128 (one activation scale per 1 x 128 K-group of a row,
 * one weight scale per 128 x 128 block of [N][K]):
 *   P_g = sum_{k in group g} dec(A[m][k]) * dec(B[n][k])        (exact, fp64)
 *   ref[r][n] = sum_g sa[m][g] * sb[n / 128][g] * P_g           (fp64)
 * sa: [M][K/G]; sb: [ceil(N/G)][K/G]. */
void oracle_gemm_block_fp8(const uint8_t* A, const uint8_t* B, const float* sa,
                           const float* sb, int64_t M, int64_t N, int64_t K,
                           int64_t G, const int64_t* rows, int64_t nrows,
                           double* ref, double* absref)
{
    int64_t r, n, k, g, ng = K / G;
    double dec[256];
    (void)M;
    for (k = 0; k < 256; ++k)
        dec[k] = oracle_e4m3_decode((uint8_t)k);
#pragma omp parallel for private(n, k, g) collapse(2) schedule(static)
    for (r = 0; r < nrows; ++r)
        for (n = 0; n < N; ++n) {
            const int64_t m = rows[r];
            const uint8_t* a = A + m * K;
            const uint8_t* b = B + n * K;
            double sum = 0.0, asum = 0.0;
            for (g = 0; g < ng; ++g) {
                double pg = 0.0, apg = 0.0, sc;
                for (k = g * G; k < (g + 1) * G; ++k) {
                    double p = dec[a[k]] * dec[b[k]];
                    pg += p;
                    apg += fabs(p);
                }
                sc = (double)sa[m * ng + g] * (double)sb[(n / G) * ng + g];
                sum += sc * pg;
                asum += fabs(sc) * apg;
            }
            ref[r * N + n] = sum;
            if (absref)
                absref[r * N + n] = asum;
        }
}

/* bf16 GEMM: ref[r][n] = sum_k A[m][k] * B[n][k] in fp64. */
void oracle_gemm_bf16(const uint16_t* A, const uint16_t* B, int64_t M, int64_t N,
                      int64_t K, const int64_t* rows, int64_t nrows, double* ref,
                      double* absref)
{
    int64_t r, n, k;
    (void)M;
#pragma omp parallel for private(n, k) collapse(2) schedule(static)
    for (r = 0; r < nrows; ++r)
        for (n = 0; n < N; ++n) {
            const uint16_t* a = A + rows[r] * K;
            const uint16_t* b = B + n * K;
            double sum = 0.0, asum = 0.0;
            for (k = 0; k < K; ++k) {
                double p = (double)oracle_bf16_decode(a[k]) *
                           (double)oracle_bf16_decode(b[k]);
                sum += p;
                asum += fabs(p);
            }
            ref[r * N + n] = sum;
            if (absref)
                absref[r * N + n] = asum;
        }
}

/* ------------------------------------------------------------------------ */
/* MXFP4: 4-bit E2M1 elements sharing one power-of-two E8M0 scale per block  */
/* of 32 consecutive K elements.  The pages name 4-bit formats (INT4, NVFP4) */
/* among those vLLM serves (introduction of "Helion in vLLM: A Unified Route */
/* to Tunable Linear Kernels") but define none; MXFP4 is the block-scaled    */
/* 4-bit format the CDNA4 matrix cores take natively, and its element and    */
/* scale encodings and its conversion rule are those of the OCP Microscaling */
/* Formats (MX) v1.0 specification (sections on the E2M1 element type, the   */
/* E8M0 scale type and the conversion of a vector to an MX block).           */
/* Packing (a reading: the specification leaves it to the implementation):   */
/* element 2j of a row in bits 0-3 of byte j, element 2j+1 in bits 4-7.      */
/* ------------------------------------------------------------------------ */

/* E2M1: bit 3 sign, bits 2-1 exponent (bias 1), bit 0 mantissa.  Exponent
 * field 0 is subnormal (m * 2^-1).  No infinity, no NaN; largest value 6. */
double oracle_e2m1_decode(uint8_t c)
{
    int sign = (c >> 3) & 1;
    int e = (c >> 1) & 3;
    int m = c & 1;
    double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -mag : mag;
}

/* E8M0 scale: the power of two 2^(c - 127); code 0xFF is NaN. */
double oracle_e8m0_decode(uint8_t c)
{
    return c == 0xFF ? NAN : ldexp(1.0, (int)c - 127);
}

/* Nearest E2M1 code to v, ties to the code whose last bit is 0; magnitudes
 * above the largest value 6 give 6 (the MX conversion saturates to the
 * largest normal).  The sign bit is the sign of v, also for a magnitude that
 * rounds to zero.  Codes 0..7 have increasing magnitudes. */
uint8_t oracle_e2m1_encode_rne(double v)
{
    uint8_t sign = signbit(v) ? 8 : 0;
    double a = fabs(v);
    int lo = 0, best;
    if (isnan(v))
        return 0xFF;
    while (lo < 7 && oracle_e2m1_decode((uint8_t)(lo + 1)) <= a)
        ++lo;
    best = lo;
    if (lo < 7) {
        double dlo = a - oracle_e2m1_decode((uint8_t)lo);
        double dhi = oracle_e2m1_decode((uint8_t)(lo + 1)) - a;
        if (dhi < dlo || (dhi == dlo && ((lo + 1) & 1) == 0))
            best = lo + 1;
    }
    return (uint8_t)(sign | best);
}

/* MXFP4 quantization of bf16 x [M][K] (K a multiple of 32), one block of 32
 * consecutive elements of a row at a time:
 *   amax = max |x_i|;
 *   shared exponent E = floor(log2(amax)) - 2 (2 = the exponent of E2M1's
 *   largest normal, 6 = 1.5 * 2^2), clamped to the E8M0 range [-127, 127];
 *   an all-zero block has no logarithm and takes the lower end -127;
 *   scale code s = E + 127;
 *   element code = e2m1_rne(x_i / 2^E), saturating at 6.
 * q: packed codes [M][K/2]; s: [M][K/32].  Returns 0, or -1 on a non-finite
 * input, -2 when 32 does not divide K. */
int oracle_quantize_mxfp4(const uint16_t* x, int64_t M, int64_t K, uint8_t* q,
                          uint8_t* s)
{
    int64_t m, b, nb;
    int bad = 0;
    if (K % 32 != 0)
        return -2;
    nb = K / 32;
#pragma omp parallel for private(b) reduction(| : bad) schedule(static)
    for (m = 0; m < M; ++m)
        for (b = 0; b < nb; ++b) {
            const uint16_t* xb = x + m * K + b * 32;
            uint8_t codes[32];
            double amax = 0.0;
            int i, E;
            for (i = 0; i < 32; ++i) {
                double xi = (double)oracle_bf16_decode(xb[i]);
                if (!isfinite(xi))
                    bad = 1;
                else if (fabs(xi) > amax)
                    amax = fabs(xi);
            }
            if (amax == 0.0) {
                E = -127;
            } else {
                int p;
                (void)frexp(amax, &p); /* amax = f * 2^p, 0.5 <= f < 1 */
                E = (p - 1) - 2;
                if (E < -127)
                    E = -127;
                if (E > 127)
                    E = 127;
            }
            s[m * nb + b] = (uint8_t)(E + 127);
            for (i = 0; i < 32; ++i)
                codes[i] = oracle_e2m1_encode_rne(
                    ldexp((double)oracle_bf16_decode(xb[i]), -E));
            for (i = 0; i < 16; ++i)
                q[m * (K / 2) + b * 16 + i] =
                    (uint8_t)((codes[2 * i] & 15) | ((codes[2 * i + 1] & 15) << 4));
        }
    return bad ? -1 : 0;
}

/* MXFP4 GEMM in fp64: with A [M][K/2], B [N][K/2] packed codes and
 * sa [M][K/32], sb [N][K/32] scale codes,
 *   ref[r][n] = sum_k dec(A[m][k]) * 2^(sa[m][k/32]-127)
 *                     * dec(B[n][k]) * 2^(sb[n][k/32]-127),
 * absref the same sum of magnitudes. */
void oracle_gemm_mxfp4(const uint8_t* A, const uint8_t* B, const uint8_t* sa,
                       const uint8_t* sb, int64_t M, int64_t N, int64_t K,
                       const int64_t* rows, int64_t nrows, double* ref,
                       double* absref)
{
    int64_t r, n, k;
    double dec[16], sdec[256];
    (void)M;
    for (k = 0; k < 16; ++k)
        dec[k] = oracle_e2m1_decode((uint8_t)k);
    for (k = 0; k < 256; ++k)
        sdec[k] = oracle_e8m0_decode((uint8_t)k);
#pragma omp parallel for private(n, k) collapse(2) schedule(static)
    for (r = 0; r < nrows; ++r)
        for (n = 0; n < N; ++n) {
            const int64_t m = rows[r];
            const uint8_t* a = A + m * (K / 2);
            const uint8_t* b = B + n * (K / 2);
            double sum = 0.0, asum = 0.0;
            for (k = 0; k < K; ++k) {
                int ca = (a[k / 2] >> (4 * (k & 1))) & 15;
                int cb = (b[k / 2] >> (4 * (k & 1))) & 15;
                double p = dec[ca] * sdec[sa[m * (K / 32) + k / 32]] * dec[cb] *
                           sdec[sb[n * (K / 32) + k / 32]];
                sum += p;
                asum += fabs(p);
            }
            ref[r * N + n] = sum;
            if (absref)
                absref[r * N + n] = asum;
        }
}

void oracle_e2m1_encode_array(const double* v, int64_t n, uint8_t* out)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = oracle_e2m1_encode_rne(v[i]);
}

/* ------------------------------------------------------------------------ */
/* INT4 weight-only (W4A16): signed 4-bit weights with one fp32 scale per    */
/* output channel and 128-element K group, bf16 activations.  The pages name */
/* INT4 among vLLM's formats (introduction of "Helion in vLLM: A Unified     */
/* Route to Tunable Linear Kernels") without defining it; the reading here   */
/* is the symmetric per-group form of the FP8 rule above: scale = amax / 7,  */
/* codes in [-8, 7] (two's complement nibbles, packed like MXFP4: element 2j */
/* in bits 0-3 of byte j).                                                    */
/* ------------------------------------------------------------------------ */

/* Two's complement value of a 4-bit code. */
int oracle_int4_decode(uint8_t c)
{
    int v = c & 15;
    return v >= 8 ? v - 16 : v;
}

/* Weight quantization of bf16 w [N][K] (K a multiple of 128), one group of
 * 128 consecutive elements of a row at a time:
 *   amax = max |w|;  s = amax / 7 (fp32);  q = clamp(rne(w / s), -8, 7)
 * with w / s the correctly rounded fp32 quotient; an all-zero group gets
 * s = 0 and zero codes.  q: packed [N][K/2]; s: fp32 [N][K/128].
 * Returns 0, -1 on a non-finite input, -2 when 128 does not divide K. */
int oracle_quantize_int4(const uint16_t* w, int64_t N, int64_t K, uint8_t* q,
                         float* s)
{
    int64_t n, g, ng;
    int bad = 0;
    if (K % 128 != 0)
        return -2;
    ng = K / 128;
#pragma omp parallel for private(g) reduction(| : bad) schedule(static)
    for (n = 0; n < N; ++n)
        for (g = 0; g < ng; ++g) {
            const uint16_t* wg = w + n * K + g * 128;
            float amax = 0.0f, sc;
            int i;
            for (i = 0; i < 128; ++i) {
                float x = oracle_bf16_decode(wg[i]);
                if (!isfinite(x))
                    bad = 1;
                else if (fabsf(x) > amax)
                    amax = fabsf(x);
            }
            sc = amax / 7.0f;
            s[n * ng + g] = sc;
            for (i = 0; i < 128; i += 2) {
                int c[2], j;
                for (j = 0; j < 2; ++j) {
                    float v, r;
                    if (sc == 0.0f) {
                        c[j] = 0;
                        continue;
                    }
                    v = oracle_bf16_decode(wg[i + j]) / sc;
                    r = nearbyintf(v); /* default rounding: to nearest, ties to even */
                    if (r > 7.0f)
                        r = 7.0f;
                    if (r < -8.0f)
                        r = -8.0f;
                    c[j] = (int)r & 15;
                }
                q[n * (K / 2) + (g * 128 + i) / 2] = (uint8_t)(c[0] | (c[1] << 4));
            }
        }
    return bad ? -1 : 0;
}

/* W4A16 GEMM in fp64: with A bf16 [M][K], B packed int4 [N][K/2] and
 * s fp32 [N][K/128],
 *   P_g = sum_{k in group g} A[m][k] * q[n][k]        (exact)
 *   ref[r][n] = sum_g s[n][g] * P_g,
 * absref the same with magnitudes. */
void oracle_gemm_w4a16(const uint16_t* A, const uint8_t* B, const float* s,
                       int64_t M, int64_t N, int64_t K, const int64_t* rows,
                       int64_t nrows, double* ref, double* absref)
{
    int64_t r, n, k, g, ng = K / 128;
    (void)M;
#pragma omp parallel for private(n, k, g) collapse(2) schedule(static)
    for (r = 0; r < nrows; ++r)
        for (n = 0; n < N; ++n) {
            const uint16_t* a = A + rows[r] * K;
            const uint8_t* b = B + n * (K / 2);
            double sum = 0.0, asum = 0.0;
            for (g = 0; g < ng; ++g) {
                double pg = 0.0, apg = 0.0, sc = (double)s[n * ng + g];
                for (k = g * 128; k < (g + 1) * 128; ++k) {
                    double p = (double)oracle_bf16_decode(a[k]) *
                               (double)oracle_int4_decode((uint8_t)(b[k / 2] >> (4 * (k & 1))));
                    pg += p;
                    apg += fabs(p);
                }
                sum += sc * pg;
                asum += fabs(sc) * apg;
            }
            ref[r * N + n] = sum;
            if (absref)
                absref[r * N + n] = asum;
        }
}

/* Elementwise helpers exposed for tests: fp32 -> bf16 bits, fp32 -> e4m3. */
void oracle_bf16_encode_array(const float* f, int64_t n, uint16_t* out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        out[i] = oracle_bf16_encode_rne(f[i]);
}

void oracle_e4m3_encode_array(const float* f, int64_t n, uint8_t* out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        out[i] = oracle_e4m3_encode_rne(f[i]);
}

void oracle_e4m3_decode_array(const uint8_t* c, int64_t n, double* out)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = oracle_e4m3_decode(c[i]);
}

/* Threads the OpenMP loops use from now on (n >= 1); timing only. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}

int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
