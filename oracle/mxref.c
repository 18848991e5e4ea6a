/*
 * mxref.c - CPU oracle for the block-scaled ("MX") matrix multiply.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant with the
 * HIP library: every value below is derived here, from the format
 * definitions, in plain C and float64.
 *
 * What it computes, and the passages it follows:
 *   - The operand model: each operand is a data plane of low-precision codes
 *     plus a scale plane holding one FP8 E8M0 (UE8M0) power of two per block
 *     of 32 consecutive elements along the reduction axis.  Source: WWDC26
 *     session 330 summary "Metal tensors でカスタム機械学習オペレーションを
 *     最適化する", sections "多平面 tensor" and "Scale Factor 付き量子化
 *     tensor を作成する" (blockFactors {32, 1}); the same session's
 *     transcript "Metal 텐서로 맞춤형 머신 러닝 연산 최적화하기", chapter
 *     "Multi-plane tensors".
 *   - The check itself: a float64 reference computed from exactly the bytes
 *     the GPU consumed.  Source: "Resumo Técnico: RIGEL", section
 *     "Metodologia: O Harness RIGEL" (checksum-gated verification).
 *   - The product: a plain triple loop over rows, columns and the reduction
 *     index.  Source: "Treinar LLM em Swift: multiplicação de matrizes do
 *     Gflop/s ao Tflop/s", section "Passo 1 - Baseline: matmul ingênua".
 *   - E4M3 saturates to +-448 and has no infinity.  Source: "Resumo Técnico:
 *     RIGEL", section 3 "Semântica Numérica e Restrições Ocultas".
 *
 * Readings taken where the pages are silent (each is listed in the design
 * notes as well):
 *   - Scale selection is the OCP Microscaling rule: the block exponent is
 *     floor(log2(amax)) - emax_elem, emax_elem = 8 for E4M3 and 2 for E2M1,
 *     clamped to [-127, 127]; an all-zero block gets exponent -127.
 *   - Elements are rounded to nearest, ties to even, and saturated to the
 *     largest finite magnitude (448 for E4M3, 6 for E2M1).
 *   - A block holding a NaN or an infinity gets scale byte 255 (NaN) and
 *     element codes 0.
 *   - E2M1 codes are packed two per byte, the even K index in the low nibble.
 *   - UE8M0 byte e means 2^(e-127); e = 255 is NaN.
 *   - Integer elements (the 4-bit and 2-bit integer tensor types the WWDC26
 *     session 330 summary lists, section "量子化データ型のネイティブサポート",
 *     combined with a block-wise scale as its section "2-bit 量子化の限界圧縮
 *     を探る" suggests): two's complement codes, INT4 in -8..7 (two per byte,
 *     even K index in the low nibble) and INT2 in -2..1 (four per byte, K
 *     index k in bits 2(k mod 4)); the block exponent takes emax = the
 *     exponent of the largest power of two the range holds (2 for INT4, 0
 *     for INT2), as emax does for the float formats; elements are rounded to
 *     nearest, ties to even, and saturated to the range (+7 / -8, +1 / -2).
 *   - FP6 elements ("FP6" is the 6-bit float the scaled matrix unit takes
 *     beside E5M2, the other "E5M2 (and FP6)" operand; the pages name no FP6
 *     layout, so the OCP Microscaling definitions are taken, as for E2M1):
 *     E2M3 = sign, 2 exponent bits (bias 1), 3 mantissa bits, largest 7.5,
 *     emax 2; E3M2 = sign, 3 exponent bits (bias 3), 2 mantissa bits,
 *     largest 28, emax 4; exponent field 0 is subnormal; no NaN, no
 *     infinity.  Codes are packed little-endian, element k of a row at bits
 *     6k .. 6k+5 of the row's bytes (four elements in three bytes).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define MXREF_E4M3 0
#define MXREF_E5M2 1
#define MXREF_E2M3 2
#define MXREF_E3M2 3
#define MXREF_E2M1 4
#define MXREF_INT4 8
#define MXREF_INT2 9

static int known_elem(int elem)
{
    return elem == MXREF_E4M3 || elem == MXREF_E5M2 || elem == MXREF_E2M1 ||
           elem == MXREF_INT4 || elem == MXREF_INT2 || elem == MXREF_E2M3 ||
           elem == MXREF_E3M2;
}

/* Bytes of one operand row of K elements. */
static int64_t row_bytes(int elem, int64_t K)
{
    if (elem == MXREF_E2M1 || elem == MXREF_INT4)
        return K / 2;
    if (elem == MXREF_INT2)
        return K / 4;
    if (elem == MXREF_E2M3 || elem == MXREF_E3M2)
        return K / 4 * 3;
    return K;
}

static int is_fp6(int elem)
{
    return elem == MXREF_E2M3 || elem == MXREF_E3M2;
}

/* 6-bit code of element k of a packed row (bits 6k .. 6k+5). */
static unsigned get6(const uint8_t *row, int64_t k)
{
    int64_t bit = 6 * k;
    unsigned v = row[bit >> 3];
    if ((bit & 7) > 2) /* the code runs into the next byte */
        v |= (unsigned)row[(bit >> 3) + 1] << 8;
    return (v >> (bit & 7)) & 63u;
}

/* Store the 6-bit code c as element k of a packed row. */
static void put6(uint8_t *row, int64_t k, unsigned c)
{
    int64_t bit = 6 * k;
    int sh = (int)(bit & 7);
    unsigned mask = 63u << sh, v = (c & 63u) << sh;
    row[bit >> 3] = (uint8_t)((row[bit >> 3] & ~mask) | (v & 0xffu));
    if (sh > 2)
        row[(bit >> 3) + 1] = (uint8_t)((row[(bit >> 3) + 1] & ~(mask >> 8)) | (v >> 8));
}

/* ---------------------------------------------------------------- decode */

/* OCP E4M3 ("FN") code -> value: sign, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent field 0 is subnormal (m * 2^-9); the all-ones pattern
 * S.1111.111 is NaN; there is no infinity. */
double mxref_e4m3_value(uint8_t code)
{
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* OCP E5M2 code -> value: sign, 5 exponent bits (bias 15), 2 mantissa
 * bits; exponent field 0 is subnormal (m * 2^-16); exponent field 31 is
 * infinity (m = 0) or NaN (m != 0), as in IEEE binary formats. */
double mxref_e5m2_value(uint8_t code)
{
    int s = code >> 7, e = (code >> 2) & 31, m = code & 3;
    double v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -16);
    else
        v = ldexp(1.0 + m / 4.0, e - 15);
    return s ? -v : v;
}

/* OCP E2M1 nibble -> value: sign, 2 exponent bits (bias 1), 1 mantissa bit;
 * exponent field 0 is subnormal (m * 0.5); no NaN, no infinity. */
double mxref_e2m1_value(uint8_t nibble)
{
    int s = (nibble >> 3) & 1, e = (nibble >> 1) & 3, m = nibble & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + m / 2.0, e - 1);
    return s ? -v : v;
}

/* OCP E2M3 6-bit code -> value: sign, 2 exponent bits (bias 1), 3 mantissa
 * bits; exponent field 0 is subnormal (m * 2^-3); no NaN, no infinity. */
double mxref_e2m3_value(uint8_t code)
{
    int s = (code >> 5) & 1, e = (code >> 3) & 3, m = code & 7;
    double v = (e == 0) ? ldexp((double)m, -3) : ldexp(1.0 + m / 8.0, e - 1);
    return s ? -v : v;
}

/* OCP E3M2 6-bit code -> value: sign, 3 exponent bits (bias 3), 2 mantissa
 * bits; exponent field 0 is subnormal (m * 2^-4); no NaN, no infinity. */
double mxref_e3m2_value(uint8_t code)
{
    int s = (code >> 5) & 1, e = (code >> 2) & 7, m = code & 3;
    double v = (e == 0) ? ldexp((double)m, -4) : ldexp(1.0 + m / 4.0, e - 3);
    return s ? -v : v;
}

/* Two's complement 4-bit code (0..15) -> -8..7. */
double mxref_int4_value(uint8_t code)
{
    int c = code & 15;
    return (double)(c < 8 ? c : c - 16);
}

/* Two's complement 2-bit code (0..3) -> -2..1. */
double mxref_int2_value(uint8_t code)
{
    int c = code & 3;
    return (double)(c < 2 ? c : c - 4);
}

/* UE8M0 scale byte -> 2^(e-127); 255 is NaN. */
double mxref_ue8m0_value(uint8_t e)
{
    return e == 255 ? NAN : ldexp(1.0, (int)e - 127);
}

/* IEEE binary16 bits -> value. */
double mxref_fp16_value(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 31)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -24);
    else
        v = ldexp(1.0 + m / 1024.0, e - 15);
    return s ? -v : v;
}

/* -------------------------------------------------------------- quantize */

/* floor(log2(a)) for finite a > 0, exactly (no floating log2). */
static int floor_log2(double a)
{
    int e;
    frexp(a, &e); /* a = f * 2^e with f in [0.5, 1) */
    return e - 1;
}

/* Round |v| to the E4M3 grid (ties to even), saturate at 448, encode. */
static uint8_t encode_e4m3(double v)
{
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v), quantum, r;
    uint8_t code;
    /* normal binades [2^-6, ...) carry 3 fraction bits; below 2^-6 the
     * spacing is the subnormal step 2^-9 */
    quantum = (a >= ldexp(1.0, -6)) ? ldexp(1.0, floor_log2(a) - 3) : ldexp(1.0, -9);
    r = nearbyint(a / quantum) * quantum; /* default mode: nearest, ties even */
    if (r > 448.0)
        r = 448.0;
    if (r < ldexp(1.0, -6)) {
        code = (uint8_t)(r * 512.0); /* subnormal: m = r / 2^-9, 0..7 */
    } else {
        int e = floor_log2(r);
        int m = (int)((r / ldexp(1.0, e) - 1.0) * 8.0);
        code = (uint8_t)(((e + 7) << 3) | m);
    }
    return (uint8_t)(code | (neg << 7));
}

/* Round |v| to the E5M2 grid (ties to even), saturate at 57344, encode.
 * Reading: a plain cast to E5M2 overflows to +-infinity ("Resumo Técnico:
 * RIGEL", section 3), but inside a scaled block the quantizer maps values
 * the way it does for E4M3 and E2M1, saturating to the largest finite
 * magnitude (with the block exponent rule, only the block maximum can round
 * past it). */
static uint8_t encode_e5m2(double v)
{
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v), quantum, r;
    uint8_t code;
    /* normal binades [2^-14, ...) carry 2 fraction bits; below 2^-14 the
     * spacing is the subnormal step 2^-16 */
    quantum = (a >= ldexp(1.0, -14)) ? ldexp(1.0, floor_log2(a) - 2) : ldexp(1.0, -16);
    r = nearbyint(a / quantum) * quantum;
    if (r > 57344.0)
        r = 57344.0;
    if (r < ldexp(1.0, -14)) {
        code = (uint8_t)(r * 65536.0); /* subnormal: m = r / 2^-16, 0..3 */
    } else {
        int e = floor_log2(r);
        int m = (int)((r / ldexp(1.0, e) - 1.0) * 4.0);
        code = (uint8_t)(((e + 15) << 2) | m);
    }
    return (uint8_t)(code | (neg << 7));
}

/* Round |v| to the E2M1 grid (ties to even), saturate at 6, encode. */
static uint8_t encode_e2m1(double v)
{
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v), quantum, r;
    uint8_t code;
    quantum = (a >= 1.0) ? ldexp(1.0, floor_log2(a) - 1) : 0.5;
    r = nearbyint(a / quantum) * quantum;
    if (r > 6.0)
        r = 6.0;
    if (r < 1.0) {
        code = (uint8_t)(r * 2.0); /* subnormal: 0 or 0.5 */
    } else {
        int e = floor_log2(r);
        int m = (int)((r / ldexp(1.0, e) - 1.0) * 2.0);
        code = (uint8_t)(((e + 1) << 1) | m);
    }
    return (uint8_t)(code | (neg << 3));
}

/* Round |v| to the E2M3 grid (ties to even), saturate at 7.5, encode. */
static uint8_t encode_e2m3(double v)
{
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v), quantum, r;
    uint8_t code;
    /* normal binades [1, ...) carry 3 fraction bits; below 1 the spacing is
     * the subnormal step 2^-3 */
    quantum = (a >= 1.0) ? ldexp(1.0, floor_log2(a) - 3) : 0.125;
    r = nearbyint(a / quantum) * quantum;
    if (r > 7.5)
        r = 7.5;
    if (r < 1.0) {
        code = (uint8_t)(r * 8.0); /* subnormal: m = r / 2^-3, 0..7 */
    } else {
        int e = floor_log2(r);
        int m = (int)((r / ldexp(1.0, e) - 1.0) * 8.0);
        code = (uint8_t)(((e + 1) << 3) | m);
    }
    return (uint8_t)(code | (neg << 5));
}

/* Round |v| to the E3M2 grid (ties to even), saturate at 28, encode. */
static uint8_t encode_e3m2(double v)
{
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v), quantum, r;
    uint8_t code;
    /* normal binades [2^-2, ...) carry 2 fraction bits; below 2^-2 the
     * spacing is the subnormal step 2^-4 */
    quantum = (a >= 0.25) ? ldexp(1.0, floor_log2(a) - 2) : 0.0625;
    r = nearbyint(a / quantum) * quantum;
    if (r > 28.0)
        r = 28.0;
    if (r < 0.25) {
        code = (uint8_t)(r * 16.0); /* subnormal: m = r / 2^-4, 0..3 */
    } else {
        int e = floor_log2(r);
        int m = (int)((r / ldexp(1.0, e) - 1.0) * 4.0);
        code = (uint8_t)(((e + 3) << 2) | m);
    }
    return (uint8_t)(code | (neg << 5));
}

/* Round v to the nearest integer (ties to even), saturate to [qmin, qmax],
 * and return its two's complement code in `bits` bits. */
static uint8_t encode_int(double v, int qmin, int qmax, int bits)
{
    double r = nearbyint(v); /* default mode: nearest, ties even */
    int q;
    if (r > qmax)
        r = qmax;
    if (r < qmin)
        r = qmin;
    q = (int)r;
    return (uint8_t)(q & ((1 << bits) - 1));
}

/* Quantize X[rows][K] (fp32, K contiguous) to codes Q and scales S.
 *   E4M3, E5M2: Q is rows x K bytes.   E2M1, INT4: Q is rows x K/2 bytes, two
 *   per byte.   INT2: Q is rows x K/4 bytes, four per byte.   E2M3, E3M2: Q
 *   is rows x 3K/4 bytes, 6-bit codes packed little-endian.
 *   S is rows x K/32 UE8M0 bytes.
 * Returns 0, or -1 on a bad argument (K not a multiple of 32, unknown elem). */
int mxref_quantize(const float *x, int64_t rows, int64_t K, int elem,
                   uint8_t *q, uint8_t *s)
{
    int emax;
    int64_t nb = K / 32;
    if (K <= 0 || K % 32 != 0 || rows < 0)
        return -1;
    if (elem == MXREF_E4M3)
        emax = 8; /* 448 = 1.75 * 2^8 */
    else if (elem == MXREF_E5M2)
        emax = 15; /* 57344 = 1.75 * 2^15 */
    else if (elem == MXREF_E2M1)
        emax = 2; /* 6 = 1.5 * 2^2 */
    else if (elem == MXREF_INT4)
        emax = 2; /* 4 <= 7 < 8 */
    else if (elem == MXREF_INT2)
        emax = 0; /* 1 */
    else if (elem == MXREF_E2M3)
        emax = 2; /* 7.5 = 1.875 * 2^2 */
    else if (elem == MXREF_E3M2)
        emax = 4; /* 28 = 1.75 * 2^4 */
    else
        return -1;

#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t b = 0; b < nb; b++) {
            const float *blk = x + r * K + b * 32;
            double amax = 0.0;
            int bad = 0, e, i;
            for (i = 0; i < 32; i++) {
                double v = blk[i];
                if (isnan(v) || isinf(v))
                    bad = 1;
                else if (fabs(v) > amax)
                    amax = fabs(v);
            }
            if (bad) {
                s[r * nb + b] = 255;
                for (i = 0; i < 32; i++) {
                    int64_t k = b * 32 + i;
                    if (elem == MXREF_E4M3 || elem == MXREF_E5M2)
                        q[r * K + k] = 0;
                    else if (is_fp6(elem))
                        put6(q + r * row_bytes(elem, K), k, 0);
                    else if (elem == MXREF_INT2)
                        q[r * (K / 4) + k / 4] &= (uint8_t)~(3u << (2 * (k & 3)));
                    else
                        q[r * (K / 2) + k / 2] &= (uint8_t)((k & 1) ? 0x0F : 0xF0);
                }
                continue;
            }
            e = (amax == 0.0) ? -127 : floor_log2(amax) - emax;
            if (e < -127)
                e = -127;
            if (e > 127)
                e = 127;
            s[r * nb + b] = (uint8_t)(e + 127);
            for (i = 0; i < 32; i++) {
                int64_t k = b * 32 + i;
                double v = ldexp((double)blk[i], -e); /* exact */
                if (elem == MXREF_E4M3) {
                    q[r * K + k] = encode_e4m3(v);
                } else if (elem == MXREF_E5M2) {
                    q[r * K + k] = encode_e5m2(v);
                } else if (is_fp6(elem)) {
                    put6(q + r * row_bytes(elem, K), k,
                         elem == MXREF_E2M3 ? encode_e2m3(v) : encode_e3m2(v));
                } else if (elem == MXREF_INT2) {
                    uint8_t c = encode_int(v, -2, 1, 2);
                    uint8_t *p = q + r * (K / 4) + k / 4;
                    int sh = 2 * (int)(k & 3);
                    *p = (uint8_t)((*p & ~(3u << sh)) | (c << sh));
                } else {
                    uint8_t nib = (elem == MXREF_INT4) ? encode_int(v, -8, 7, 4) : encode_e2m1(v);
                    uint8_t *p = q + r * (K / 2) + k / 2;
                    if (k & 1)
                        *p = (uint8_t)((*p & 0x0F) | (nib << 4));
                    else
                        *p = (uint8_t)((*p & 0xF0) | nib);
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ GEMM */

static double tab_e4m3[256], tab_e5m2[256], tab_e2m1[16], tab_int4[16], tab_int2[4], tab_ue8m0[256];
static double tab_e2m3[64], tab_e3m2[64];
static int tabs_ready = 0;

static void make_tables(void)
{
    int i;
    if (tabs_ready)
        return;
    for (i = 0; i < 256; i++)
        tab_e4m3[i] = mxref_e4m3_value((uint8_t)i);
    for (i = 0; i < 256; i++)
        tab_e5m2[i] = mxref_e5m2_value((uint8_t)i);
    for (i = 0; i < 16; i++)
        tab_e2m1[i] = mxref_e2m1_value((uint8_t)i);
    for (i = 0; i < 16; i++)
        tab_int4[i] = mxref_int4_value((uint8_t)i);
    for (i = 0; i < 4; i++)
        tab_int2[i] = mxref_int2_value((uint8_t)i);
    for (i = 0; i < 64; i++) {
        tab_e2m3[i] = mxref_e2m3_value((uint8_t)i);
        tab_e3m2[i] = mxref_e3m2_value((uint8_t)i);
    }
    for (i = 0; i < 256; i++)
        tab_ue8m0[i] = mxref_ue8m0_value((uint8_t)i);
    tabs_ready = 1;
}

/* Value of element k of one operand row (codes only, no scale). */
static double element(const uint8_t *row, int elem, int64_t k)
{
    if (elem == MXREF_E4M3)
        return tab_e4m3[row[k]];
    if (elem == MXREF_E5M2)
        return tab_e5m2[row[k]];
    if (elem == MXREF_INT4)
        return tab_int4[(row[k >> 1] >> ((k & 1) * 4)) & 15];
    if (elem == MXREF_INT2)
        return tab_int2[(row[k >> 2] >> ((k & 3) * 2)) & 3];
    if (elem == MXREF_E2M3)
        return tab_e2m3[get6(row, k)];
    if (elem == MXREF_E3M2)
        return tab_e3m2[get6(row, k)];
    return tab_e2m1[(row[k >> 1] >> ((k & 1) * 4)) & 15];
}

/* One output element:
 *   C[i][j] = sum_b 2^(sA[i][b]-127) * 2^(sB[j][b]-127) * sum_{k in block b} a_ik * b_jk
 * A is M x K codes (K contiguous), B is N x K codes (K contiguous): both
 * scale planes run along K.  Each block partial is a sum of 32 products of
 * short significands, exact in float64; multiplying by a power of two is
 * exact; only the sum across blocks rounds (relative error below
 * (K/32) * 2^-53).  abs_out receives sum_k |a_ik * b_jk| * scales, the
 * magnitude that sets the accumulation-error bound.  When smax_out is not
 * NULL it receives, for the steps k = 128t .. 128t+127 of K (four blocks
 * each, the last step possibly shorter), the sum over the steps of the
 * largest |a_ik * b_jk| * scales inside the step: the magnitude a matrix
 * unit that adds one step's products in a single operation aligns them to
 * (a tolerance input only; the value of C does not depend on it). */
static void mx_point(const uint8_t *A, const uint8_t *sA, int elemA,
                     const uint8_t *B, const uint8_t *sB, int elemB,
                     int64_t K, int64_t i, int64_t j, double *out, double *abs_out,
                     double *smax_out)
{
    int64_t nb = K / 32;
    int64_t rowbytesA = row_bytes(elemA, K);
    int64_t rowbytesB = row_bytes(elemB, K);
    const uint8_t *ra = A + i * rowbytesA, *rb = B + j * rowbytesB;
    double acc = 0.0, acc_abs = 0.0, smax_sum = 0.0, step_max = 0.0;
    for (int64_t b = 0; b < nb; b++) {
        double part = 0.0, part_abs = 0.0, part_max = 0.0;
        double scale = tab_ue8m0[sA[i * nb + b]] * tab_ue8m0[sB[j * nb + b]];
        for (int64_t k = b * 32; k < b * 32 + 32; k++) {
            double p = element(ra, elemA, k) * element(rb, elemB, k);
            part += p;
            part_abs += fabs(p);
            if (!(fabs(p) <= part_max))
                part_max = fabs(p); /* NaN propagates */
        }
        acc += part * scale;
        acc_abs += part_abs * scale;
        if (!(part_max * scale <= step_max))
            step_max = part_max * scale;
        if (b % 4 == 3 || b == nb - 1) {
            smax_sum += step_max;
            step_max = 0.0;
        }
    }
    *out = acc;
    *abs_out = acc_abs;
    if (smax_out)
        *smax_out = smax_sum;
}

/* Full product: C and ABS (and SMAX unless NULL) are M x N float64,
 * row-major. */
int mxref_gemm(const uint8_t *A, const uint8_t *sA, int elemA,
               const uint8_t *B, const uint8_t *sB, int elemB,
               int64_t M, int64_t N, int64_t K, double *C, double *ABS,
               double *SMAX)
{
    if (K <= 0 || K % 32 != 0 || M < 0 || N < 0)
        return -1;
    if (!known_elem(elemA) || !known_elem(elemB))
        return -1;
    make_tables();
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; i++)
        for (int64_t j = 0; j < N; j++)
            mx_point(A, sA, elemA, B, sB, elemB, K, i, j,
                     &C[i * N + j], &ABS[i * N + j], SMAX ? &SMAX[i * N + j] : NULL);
    return 0;
}

/* Sampled product: only the npts points (I[p], J[p]); C, ABS and SMAX
 * (unless NULL) have npts entries.  Same arithmetic as mxref_gemm. */
int mxref_gemm_points(const uint8_t *A, const uint8_t *sA, int elemA,
                      const uint8_t *B, const uint8_t *sB, int elemB,
                      int64_t M, int64_t N, int64_t K,
                      const int64_t *I, const int64_t *J, int64_t npts,
                      double *C, double *ABS, double *SMAX)
{
    if (K <= 0 || K % 32 != 0)
        return -1;
    if (!known_elem(elemA) || !known_elem(elemB))
        return -1;
    for (int64_t p = 0; p < npts; p++)
        if (I[p] < 0 || I[p] >= M || J[p] < 0 || J[p] >= N)
            return -1;
    make_tables();
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t p = 0; p < npts; p++)
        mx_point(A, sA, elemA, B, sB, elemB, K, I[p], J[p], &C[p], &ABS[p],
                 SMAX ? &SMAX[p] : NULL);
    return 0;
}

/* ----------------------------------------------------------- fp16 GEMM */

/* fp16 comparison product, C = A B with A M x K row-major and B either
 * K x N row-major (b_is_nk = 0) or N x K row-major (b_is_nk = 1).
 * Products of two binary16 values are exact in float64; the K-term sum
 * rounds with relative error below K * 2^-53.  This is the half-precision
 * rung of "Treinar LLM em Swift", section "Passo 6" (FP16 in place of FP32),
 * computed with the plain loop of its section "Passo 1". */
static void f16_point(const uint16_t *A, const uint16_t *B, int64_t N, int64_t K,
                      int b_is_nk, int64_t i, int64_t j, double *out, double *abs_out)
{
    double acc = 0.0, acc_abs = 0.0;
    for (int64_t k = 0; k < K; k++) {
        uint16_t bb = b_is_nk ? B[j * K + k] : B[k * N + j];
        double p = mxref_fp16_value(A[i * K + k]) * mxref_fp16_value(bb);
        acc += p;
        acc_abs += fabs(p);
    }
    *out = acc;
    *abs_out = acc_abs;
}

int mxref_fp16_gemm(const uint16_t *A, const uint16_t *B, int64_t M, int64_t N,
                    int64_t K, int b_is_nk, double *C, double *ABS)
{
    if (K <= 0 || M < 0 || N < 0)
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; i++)
        for (int64_t j = 0; j < N; j++)
            f16_point(A, B, N, K, b_is_nk, i, j, &C[i * N + j], &ABS[i * N + j]);
    return 0;
}

int mxref_fp16_gemm_points(const uint16_t *A, const uint16_t *B, int64_t M,
                           int64_t N, int64_t K, int b_is_nk,
                           const int64_t *I, const int64_t *J, int64_t npts,
                           double *C, double *ABS)
{
    if (K <= 0)
        return -1;
    for (int64_t p = 0; p < npts; p++)
        if (I[p] < 0 || I[p] >= M || J[p] < 0 || J[p] >= N)
            return -1;
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t p = 0; p < npts; p++)
        f16_point(A, B, N, K, b_is_nk, I[p], J[p], &C[p], &ABS[p]);
    return 0;
}

/* Set the number of threads of the parallel loops (n >= 1); returns the
 * number now in effect. */
int mxref_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* Number of threads the parallel loops above use. */
int mxref_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------- epilogue */

/* The output step of the fused GEMM (bias, GELU, output type), as the plain
 * definitions.  Source of the operation: "Resumo Técnico: RIGEL", section
 * "4. Oportunidades de Otimização" (a GEMM fused with bias and GELU).
 * Reading: GELU is the Gaussian error linear unit y * Phi(y), Phi the
 * standard normal distribution function; bias is one value per output
 * column.  Phi(y) = erfc(-y / sqrt 2) / 2 (the same as (1 + erf(y / sqrt 2))
 * / 2, without its cancellation for negative y), with the C library's erfc. */
double mxref_gelu(double y)
{
    return 0.5 * y * erfc(-y / sqrt(2.0));
}

/* Round a double to the nearest value of a binary format with P significant
 * bits, smallest normal exponent EMIN and largest finite value
 * (2 - 2^(1-P)) * 2^EMAX, ties to even; beyond the largest finite value
 * (after rounding) the result is +-infinity, NaN stays NaN. */
static double round_binary(double v, int P, int EMIN, int EMAX)
{
    double a, q, r, fl;
    int e;
    if (isnan(v) || isinf(v) || v == 0.0) return v;
    a = fabs(v);
    e = ilogb(a);                      /* floor(log2 a), exact */
    if (e < EMIN) e = EMIN;            /* subnormal range: fixed quantum */
    q = ldexp(1.0, e - (P - 1));       /* spacing of the format around a */
    r = a / q;                         /* exact: power-of-two scaling */
    fl = floor(r);
    if (r - fl > 0.5 || (r - fl == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    a = fl * q;
    if (a > ldexp(2.0 - ldexp(1.0, 1 - P), EMAX)) a = INFINITY;
    return v < 0 ? -a : a;
}

/* bfloat16: 8 significant bits, exponent range of binary32. */
double mxref_round_bf16(double v) { return round_binary(v, 8, -126, 127); }
/* IEEE binary16: 11 significant bits, exponents -14 .. 15. */
double mxref_round_f16(double v) { return round_binary(v, 11, -14, 15); }

/* y[p] = act(c[p] + bias[col[p]]) for n points (bias may be NULL; act 0 =
 * none, 1 = GELU), in float64. */
int mxref_epilogue(const double *c, const int64_t *col, int64_t n, const float *bias, int act, double *y)
{
    int64_t p;
    if (!c || !y || n < 0 || (bias && !col) || (act != 0 && act != 1)) return 1;
    for (p = 0; p < n; p++) {
        double v = c[p];
        if (bias) v += (double)bias[col[p]];
        y[p] = act ? mxref_gelu(v) : v;
    }
    return 0;
}
