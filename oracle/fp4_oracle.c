/*
 * fp4_oracle.c -- plain, slow CPU reference for the block-quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this code.  It shares no source with
 * the HIP library and never calls it.
 *
 * Pages cited (title, then the section or figure the fact comes from):
 *   [AMD-MXFP4]  "Pretraining large language models with MXFP4 on Native FP4
 *                Hardware" (htx.com news item on the AMD / Penn State paper)
 *   [QUARTET-II] "Quartet II -- обучение в NVFP4 с точными несмещёнными
 *                градиентами" (Telegram channel post)
 *   [NV-NVFP4]   "NVIDIA создала метод обучения нейросетей в 4-bit точности"
 *                (news.hamidun.com)
 * Where the pages leave a step open, the reading taken is stated at the step.
 *
 * Build rules: plain C99, IEEE binary32/binary64 with round-to-nearest-even,
 * subnormals kept (no flush-to-zero), no contraction of a*b+c into an FMA
 * unless fmaf() is written out (gcc -O2 -ffp-contract=off -fno-fast-math).
 * OpenMP only splits independent rows or blocks; it never changes the order
 * of any floating-point operation.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Scalar formats                                                           */
/* ------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bfloat16 is the top half of a binary32: widening is exact. */
float oracle_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* E2M1 (FP4) magnitudes, code 0..7; bit 3 of a code is the sign.
 * [AMD-MXFP4, "Что такое MXFP4"]: each element of a block is a 4-bit float.
 * Reading: the E2M1 element of the OCP MX standard the same section names,
 * whose magnitudes are {0, 0.5, 1, 1.5, 2, 3, 4, 6}. */
static const double E2M1_VALUE[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double oracle_e2m1_decode(uint8_t code) {
    double m = E2M1_VALUE[code & 7];
    return (code & 8) ? -m : m;
}

/* Round-to-nearest onto the E2M1 grid, ties to the even code, |v| beyond the
 * largest value saturates to 6.  [AMD-MXFP4, "Что такое MXFP4"]: the element
 * is "rounded to the nearest representable FP4 value".  The midpoints between
 * neighbours are 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5; at a midpoint the even
 * code wins, so the comparison is strict (>) where the lower neighbour has an
 * even code and non-strict (>=) where the upper one has. */
uint8_t oracle_e2m1_rtn(float v) {
    float a = fabsf(v);
    uint8_t m = 0;
    m += a > 0.25f;   /* 0 (code 0, even) | 0.5 (code 1)   */
    m += a >= 0.75f;  /* 0.5 (code 1)     | 1   (code 2, even) */
    m += a > 1.25f;   /* 1   (code 2)     | 1.5 (code 3)   */
    m += a >= 1.75f;  /* 1.5 (code 3)     | 2   (code 4)   */
    m += a > 2.5f;    /* 2   (code 4)     | 3   (code 5)   */
    m += a >= 3.5f;   /* 3   (code 5)     | 4   (code 6)   */
    m += a > 5.0f;    /* 4   (code 6)     | 6   (code 7)   */
    return (uint8_t)((signbit(v) ? 8 : 0) | m);
}

/* Stochastic rounding onto the E2M1 grid.  [AMD-MXFP4, "Поисковая
 * экспериментальная работа: корень нестабильности"]: stochastic rounding makes
 * the expected rounding error zero.  With lo <= |v| < hi adjacent grid points,
 * the probability of rounding up is p = (|v| - lo) / (hi - lo); it rounds up
 * iff r < p where r = (u >> 8) * 2^-24 is uniform on [0, 1) in steps of
 * 2^-24.  |v| >= 6 saturates to 6.  Every step is exact in binary32: |v| - lo
 * is exact (lo = 0 or lo >= |v| / 2) and hi - lo is a power of two. */
uint8_t oracle_e2m1_sr(float v, uint32_t u) {
    float a = fabsf(v);
    uint8_t m;
    if (a >= 6.0f) {
        m = 7;
    } else {
        uint8_t lo = 0;
        while (lo < 7 && (float)E2M1_VALUE[lo + 1] <= a) lo++;
        float flo = (float)E2M1_VALUE[lo], fhi = (float)E2M1_VALUE[lo + 1];
        float p = (a - flo) / (fhi - flo);
        float r = (float)(u >> 8) * 0x1p-24f;
        m = (uint8_t)(r < p ? lo + 1 : lo);
    }
    return (uint8_t)((signbit(v) ? 8 : 0) | m);
}

/* E4M3 (OCP FP8, "fn" variant: no infinities, 0x7F/0xFF are NaN, largest
 * finite 448).  [QUARTET-II]: NVFP4 carries finer FP8 scales.  Decode is the
 * definition: bias 7, subnormals m/8 * 2^-6. */
double oracle_e4m3_decode(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Largest E4M3 magnitude byte whose value is <= a (a >= 0, finite).  A linear
 * search over the 127 finite non-negative codes, slow and obvious. */
static uint8_t e4m3_floor_code(double a) {
    uint8_t best = 0;
    for (int b = 0; b <= 0x7E; ++b)
        if (oracle_e4m3_decode((uint8_t)b) <= a) best = (uint8_t)b;
    return best;
}

/* Round to nearest E4M3, ties to even mantissa, saturating at 448 (values
 * above 448 become 448 rather than NaN).  Non-negative inputs only are used
 * here (block scales). */
uint8_t oracle_e4m3_rne(float x) {
    double a = fabs((double)x);
    uint8_t lo = e4m3_floor_code(a);
    if (lo == 0x7E) return lo;                 /* >= 448 saturates */
    double vlo = oracle_e4m3_decode(lo), vhi = oracle_e4m3_decode((uint8_t)(lo + 1));
    double mid = 0.5 * (vlo + vhi);
    uint8_t r;
    if (a < mid) r = lo;
    else if (a > mid) r = (uint8_t)(lo + 1);
    else r = (lo & 1) ? (uint8_t)(lo + 1) : lo;
    return (uint8_t)(r | (signbit(x) ? 0x80 : 0));
}

/* Stochastic rounding to E4M3 with the same comparator as oracle_e2m1_sr,
 * saturating at 448.  Non-negative inputs (block scales).  The probability
 * (x - lo) / (hi - lo) is formed in binary32: x - lo is exact because lo is
 * within a factor 9/8 of x (or lo = 0), and hi - lo is a power of two. */
uint8_t oracle_e4m3_sr(float x, uint32_t u) {
    float a = fabsf(x);
    uint8_t lo = e4m3_floor_code((double)a);
    if (lo == 0x7E) return lo;
    float flo = (float)oracle_e4m3_decode(lo);
    float fhi = (float)oracle_e4m3_decode((uint8_t)(lo + 1));
    float p = (a - flo) / (fhi - flo);
    float r = (float)(u >> 8) * 0x1p-24f;
    return r < p ? (uint8_t)(lo + 1) : lo;
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as  */
/* easy as 1, 2, 3", SC'11): ten rounds of the Philox S-box on a 128-bit     */
/* counter under a 64-bit key, with a Weyl-sequence key schedule.            */
/* ------------------------------------------------------------------------ */

void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;   /* round multipliers */
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;   /* key increments    */
    uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += W0; k1 += W1; }
        uint64_t p0 = (uint64_t)M0 * c[0];
        uint64_t p1 = (uint64_t)M1 * c[2];
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
    }
    memcpy(out, c, sizeof c);
}

/* The random streams of the layer.  Reading: key = the 64-bit seed (low word
 * first); counter = (index >> 2 low, index >> 2 high, purpose, 0); the word
 * used is index & 3.  Purpose 0 = element stochastic rounding (index = the
 * element's position in the quantized row-major layout), 1 = Hadamard signs
 * (index 0), 2 = NVFP4 scale stochastic rounding (index = block number). */
uint32_t oracle_stream_word(uint64_t seed, uint32_t purpose, uint64_t index) {
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint64_t g = index >> 2;
    uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), purpose, 0};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return out[index & 3];
}

/* ------------------------------------------------------------------------ */
/* Hadamard transform                                                       */
/* ------------------------------------------------------------------------ */

enum { HAD_NONE = 0, HAD_DET = 1, HAD_SIGNED = 2 };
enum { AXIS_COLS = 0, AXIS_ROWS = 1 };
enum { RND_RTN = 0, RND_SR = 1 };

/* Sign vector D of the randomized transform.  [AMD-MXFP4, "Поисковая
 * экспериментальная работа: корень нестабильности"]: the randomized variant
 * is a Hadamard transform preceded by random sign flips; the deterministic
 * one applies the same transform every step.  Reading: one vector of n signs
 * per seed, shared by every block, s_j = -1 iff bit j of word 0 of the
 * purpose-1 stream is set.  The deterministic transform uses s_j = +1. */
void oracle_hadamard_signs(int had, int n, uint64_t seed, float* s) {
    uint32_t w = (had == HAD_SIGNED) ? oracle_stream_word(seed, 1, 0) : 0u;
    for (int j = 0; j < n; ++j) s[j] = ((w >> j) & 1u) ? -1.0f : 1.0f;
}

/* 1/sqrt(n) rounded to binary32: n = 16 gives 0.25 exactly, n = 32 gives
 * 0x3E3504F3. */
float oracle_hadamard_norm(int n) { return (float)(1.0 / sqrt((double)n)); }

/* In-place normalized Walsh-Hadamard transform of one block of n = 16 or 32
 * values, in binary32: y = fl(fl(H_n D x) * fl(1/sqrt(n))), with H_n the
 * Sylvester-ordered Hadamard matrix.  [AMD-MXFP4, "Поисковая экспериментальная
 * работа: корень нестабильности"] and the figure caption of the same page (the
 * deterministic transform "H16"); [NV-NVFP4, "Как это работает"]: 16x16
 * random Hadamard transforms on the gradient inputs.  Reading: the butterfly
 * runs strides 1, 2, 4, ..., n/2 in that order, each pair (a, b) becoming
 * (a + b, a - b), and the normalization is one binary32 multiply at the end. */
void oracle_fwht(float* a, int n, const float* s) {
    for (int i = 0; i < n; ++i) a[i] = s[i] * a[i];         /* exact: s = +-1 */
    for (int h = 1; h < n; h <<= 1) {
        for (int i = 0; i < n; ++i) {
            if (i & h) continue;
            float x = a[i], y = a[i + h];
            a[i] = x + y;
            a[i + h] = x - y;
        }
    }
    float c = oracle_hadamard_norm(n);
    for (int i = 0; i < n; ++i) a[i] = a[i] * c;
}

/* ------------------------------------------------------------------------ */
/* MXFP4 quantization                                                       */
/* ------------------------------------------------------------------------ */

/* E8M0 shared exponent of one 32-element block, from its largest magnitude m
 * (m finite, >= 0).  [AMD-MXFP4, "Что такое MXFP4"]: each block shares one
 * E8M0 exponent taken from the largest exponent in the block.  Reading (the
 * OCP MX convention; the page's own formula did not survive): the scale is
 * 2^e with e = floor(log2 m) - 2, 2 being the exponent of E2M1's largest
 * value, so the block maximum lands in [4, 8); e is clamped to [-127, 127]
 * and m = 0 gives e = -127.  floor(log2 m) is read exactly with frexp. */
int oracle_mx_exponent(float m) {
    if (m == 0.0f) return -127;
    int ex;
    (void)frexp((double)m, &ex);           /* m = f * 2^ex, f in [0.5, 1) */
    int e = (ex - 1) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

static int mx_args_ok(int64_t C, int had_n, int had, int rnd) {
    if (C <= 0 || C % 32) return 0;
    if (had != HAD_NONE && had != HAD_DET && had != HAD_SIGNED) return 0;
    if (had != HAD_NONE && had_n != 16 && had_n != 32) return 0;
    if (rnd != RND_RTN && rnd != RND_SR) return 0;
    return 1;
}

/* Quantize one logical row (length C, contraction axis) of A.
 * codes_row: C/2 bytes; scales_row: C/32 bytes. */
static void mx_quantize_row(const float* arow, int64_t r, int64_t C, int had_n, int had,
                            const float* signs, int rnd, uint64_t sr_seed,
                            uint8_t* codes_row, uint8_t* scales_row) {
    float y[32];
    uint8_t q[32];
    for (int64_t b = 0; b < C / 32; ++b) {
        memcpy(y, arow + b * 32, sizeof y);
        /* 1. rotation of each had_n-block along the contraction axis */
        if (had != HAD_NONE)
            for (int o = 0; o < 32; o += had_n) oracle_fwht(y + o, had_n, signs);
        /* 2. block maximum; a non-finite value poisons the block */
        int finite = 1;
        float m = 0.0f;
        for (int i = 0; i < 32; ++i) {
            if (!isfinite(y[i])) finite = 0;
            float a = fabsf(y[i]);
            if (a > m) m = a;
        }
        if (!finite) {
            /* Reading: E8M0 0xFF is the standard's NaN scale; the codes of
             * such a block carry no information and are written as 0. */
            scales_row[b] = 0xFF;
            memset(codes_row + b * 16, 0, 16);
            continue;
        }
        /* 3. shared exponent and its E8M0 byte */
        int e = oracle_mx_exponent(m);
        scales_row[b] = (uint8_t)(e + 127);
        /* 4. element quantization of v = y * 2^-e (one binary32 multiply;
         *    2^-e is a normal binary32 since -125 <= -e <= 127) */
        float inv = (float)ldexp(1.0, -e);
        for (int i = 0; i < 32; ++i) {
            float v = y[i] * inv;
            if (rnd == RND_RTN) {
                q[i] = oracle_e2m1_rtn(v);
            } else {
                uint64_t idx = (uint64_t)r * (uint64_t)C + (uint64_t)(b * 32 + i);
                q[i] = oracle_e2m1_sr(v, oracle_stream_word(sr_seed, 0, idx));
            }
        }
        /* 5. two codes per byte, the even element in the low nibble */
        for (int j = 0; j < 16; ++j)
            codes_row[b * 16 + j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
    }
}

/* MXFP4 quantization of a bf16 matrix x[rows, cols] (row-major).
 * axis = AXIS_COLS: blocks run along cols; logical A = x, R = rows, C = cols.
 * axis = AXIS_ROWS: blocks run along rows; logical A = x^T, R = cols, C = rows.
 * Outputs codes[R, C/2] and scales[R, C/32], row-major, for the logical rows
 * r0 <= r < r1 only (the caller's buffers are the full-size ones).
 * Returns 0 on success, nonzero on a bad argument. */
int oracle_quant_mx(const uint16_t* x, int64_t rows, int64_t cols, int axis, int had_n,
                    int had, uint64_t sign_seed, int rnd, uint64_t sr_seed,
                    int64_t r0, int64_t r1, uint8_t* codes, uint8_t* scales) {
    if (axis != AXIS_COLS && axis != AXIS_ROWS) return 1;
    int64_t R = axis == AXIS_COLS ? rows : cols;
    int64_t C = axis == AXIS_COLS ? cols : rows;
    if (rows <= 0 || cols <= 0 || !mx_args_ok(C, had_n, had, rnd)) return 1;
    if (r0 < 0 || r1 > R || r0 > r1) return 1;
    float signs[32];
    if (had != HAD_NONE) oracle_hadamard_signs(had, had_n, sign_seed, signs);
    int64_t r;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = r0; r < r1; ++r) {
        float* arow = (float*)malloc((size_t)C * sizeof(float));
        for (int64_t c = 0; c < C; ++c) {
            uint16_t h = axis == AXIS_COLS ? x[r * cols + c] : x[c * cols + r];
            arow[c] = oracle_bf16_to_f32(h);
        }
        mx_quantize_row(arow, r, C, had_n, had, signs, rnd, sr_seed,
                        codes + r * (C / 2), scales + r * (C / 32));
        free(arow);
    }
    return 0;
}

/* Value of element (r, c) of a quantized MXFP4 matrix: e2m1(code) * 2^(s-127)
 * (exact in binary64; a 0xFF scale decodes to NaN). */
double oracle_mx_value(const uint8_t* codes, const uint8_t* scales, int64_t C, int64_t r, int64_t c) {
    uint8_t byte = codes[r * (C / 2) + c / 2];
    uint8_t code = (c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
    uint8_t s = scales[r * (C / 32) + c / 32];
    if (s == 0xFF) return NAN;
    return oracle_e2m1_decode(code) * ldexp(1.0, (int)s - 127);
}

/* Dequantize rows r0 <= r < r1 of an MXFP4 matrix [R, C] into out[(r-r0)*C + c]. */
void oracle_dequant_mx(const uint8_t* codes, const uint8_t* scales, int64_t C,
                       int64_t r0, int64_t r1, double* out) {
    int64_t r;
#pragma omp parallel for
    for (r = r0; r < r1; ++r)
        for (int64_t c = 0; c < C; ++c)
            out[(r - r0) * C + c] = oracle_mx_value(codes, scales, C, r, c);
}

/* ------------------------------------------------------------------------ */
/* The scaled FP4 GEMM                                                      */
/* ------------------------------------------------------------------------ */

/* C[m, n] = sum_k A[m, k] * B[n, k] over dequantized MXFP4 operands, both
 * stored along their contraction axis (A: [M, K], B: [N, K]), accumulated in
 * binary64; S[m, n] = sum_k |A[m, k] * B[n, k]| bounds the rounding error of
 * any summation order.  [AMD-MXFP4, "Поисковая экспериментальная работа:
 * корень нестабильности"]: the three GEMMs of a linear layer, Fprop
 * Y = X W^T, Dgrad dX = dY W, Wgrad dW = dY^T X, are each this product with
 * (A, B, K) = (X, W, in-features), (dY, W^T, out-features), (dY^T, X^T, tokens).
 * Computes only the entries listed in (mi[t], ni[t]), t < count, into
 * c_out[t], s_out[t]; rows of A and B are dequantized once per entry, which
 * is slow and plain. */
void oracle_gemm_mx_entries(const uint8_t* aq, const uint8_t* as, const uint8_t* bq,
                            const uint8_t* bs, int64_t K, const int64_t* mi,
                            const int64_t* ni, int64_t count, double* c_out, double* s_out) {
    int64_t t;
#pragma omp parallel for schedule(dynamic, 16)
    for (t = 0; t < count; ++t) {
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = oracle_mx_value(aq, as, K, mi[t], k) * oracle_mx_value(bq, bs, K, ni[t], k);
            acc += p;
            mag += fabs(p);
        }
        c_out[t] = acc;
        s_out[t] = mag;
    }
}

/* Rows m0 <= m < m1 of the full product: C and S are [(m1-m0), N] row-major.
 * Operands are dequantized first (A rows m0..m1, all of B), then multiplied
 * with the plain triple loop in binary64. */
void oracle_gemm_mx_rows(const uint8_t* aq, const uint8_t* as, const uint8_t* bq,
                         const uint8_t* bs, int64_t M, int64_t N, int64_t K,
                         int64_t m0, int64_t m1, double* c_out, double* s_out) {
    (void)M;
    double* a = (double*)malloc((size_t)(m1 - m0) * (size_t)K * sizeof(double));
    double* b = (double*)malloc((size_t)N * (size_t)K * sizeof(double));
    oracle_dequant_mx(aq, as, K, m0, m1, a);
    oracle_dequant_mx(bq, bs, K, 0, N, b);
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < m1 - m0; ++i) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = a[i * K + k] * b[n * K + k];
                acc += p;
                mag += fabs(p);
            }
            c_out[i * N + n] = acc;
            s_out[i * N + n] = mag;
        }
    }
    free(a);
    free(b);
}

/* ------------------------------------------------------------------------ */
/* NVFP4 quantization with the renormalization folded into the scales       */
/* ------------------------------------------------------------------------ */

/* Tensor amax of the rotated tensor, max |y| over every element, where y is
 * the row-wise 16-block transform of x (identity for HAD_NONE).  A NaN
 * element makes the result NaN. */
float oracle_nvfp4_amax(const uint16_t* x, int64_t rows, int64_t cols, int had,
                        uint64_t sign_seed) {
    float signs[16];
    if (had != HAD_NONE) oracle_hadamard_signs(had, 16, sign_seed, signs);
    float amax = 0.0f;
    int nan_seen = 0;
    int64_t r;
#pragma omp parallel for reduction(max : amax) reduction(| : nan_seen)
    for (r = 0; r < rows; ++r) {
        float y[16];
        for (int64_t b = 0; b < cols / 16; ++b) {
            for (int i = 0; i < 16; ++i) y[i] = oracle_bf16_to_f32(x[r * cols + b * 16 + i]);
            if (had != HAD_NONE) oracle_fwht(y, 16, signs);
            for (int i = 0; i < 16; ++i) {
                if (isnan(y[i])) nan_seen = 1;
                float a = fabsf(y[i]);
                if (a > amax) amax = a;
            }
        }
    }
    return nan_seen ? NAN : amax;
}

/* NVFP4 quantization of x[rows, cols] (bf16, row-major) along rows in blocks
 * of 16.  [QUARTET-II]: NVFP4 holds FP4 elements with finer FP8 block scales;
 * a randomly rotated tensor, once quantized, is collinear with the original
 * in expectation, so renormalizing makes it unbiased, but the factor
 * (about 0.94..1.06) is too fine for FP8 scales, so it is folded into the FP8
 * scales by stochastic rounding, on the scales only.  [NV-NVFP4, "Как это
 * работает"]: 16x16 random Hadamard transforms on gradient inputs.
 * Readings:
 *   - two-level scale: fp32 tensor scale s_t = amax / (6 * 448) (s_t = 1 when
 *     amax = 0), E4M3 block scale s_b = RNE(m_b / (6 s_t)), saturating at 448;
 *   - elements: v = y * fl(1 / fl(s_b s_t)), then E2M1 round-to-nearest-even;
 *   - the renormalization factor is per block, rho = |y|^2 / <y, y_hat>, and
 *     the stored scale is SR(s_b * rho) = SR(|y|^2 / (s_t * sum y_i q_i)) onto
 *     E4M3 with the purpose-2 stream at the block index; sums are binary32
 *     fmaf chains in element order.  A block with sum y_i q_i <= 0, or whose
 *     target is NaN, keeps s_b;
 *   - non-finite values (the pages are silent): the tensor amax is NaN if any
 *     rotated element is NaN, else infinite if any is; an amax without a
 *     finite positive tensor scale makes every block scale 0x7F (E4M3 NaN),
 *     every code zero and the tensor scale NaN; a block holding a NaN or an
 *     infinity gets scale 0x7F and zero codes; a block whose reciprocal
 *     scale 1 / (s_b s_t) overflows gets zero codes and scale s_b.
 * mode: 0 = elements to nearest, scale s_b; 1 = elements to nearest, scale
 * renormalized as above; 2 = every element rounded stochastically instead
 * ([QUARTET-II]: the recipe it compares against rounds each FP4 element
 * stochastically; [NV-NVFP4, "Как это работает"]: stochastic rounding in the
 * computations), scale s_b.  Reading for mode 2: the E2M1 stochastic
 * rounding of oracle_e2m1_sr with the purpose-0 stream at the element's
 * row-major index r * cols + c, the same stream as MXFP4's SR.
 * amax_in (nullable) replaces the computed tensor amax.
 * codes[rows, cols/2], scales[rows, cols/16] (E4M3 bytes), *tensor_scale. */
int oracle_nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, int had,
                          uint64_t sign_seed, int mode, uint64_t sr_seed,
                          const float* amax_in, uint8_t* codes, uint8_t* scales,
                          float* tensor_scale) {
    if (rows <= 0 || cols <= 0 || cols % 16) return 1;
    if (had != HAD_NONE && had != HAD_DET && had != HAD_SIGNED) return 1;
    if (mode != 0 && mode != 1 && mode != 2) return 1;
    float signs[16];
    if (had != HAD_NONE) oracle_hadamard_signs(had, 16, sign_seed, signs);
    float amax = amax_in ? *amax_in : oracle_nvfp4_amax(x, rows, cols, had, sign_seed);
    float s_t = (amax == 0.0f) ? 1.0f : amax / 2688.0f;   /* 2688 = 6 * 448 */
    int64_t nb = cols / 16;
    int64_t r;
    /* Reading for non-finite inputs (the pages are silent): an amax that
     * gives no finite positive tensor scale (NaN, infinite, negative, or so
     * small that A / 2688 is zero) makes the whole tensor NaN: tensor scale
     * NaN, every block scale the E4M3 NaN byte 0x7F, all codes zero. */
    if (!(isfinite(s_t) && s_t > 0.0f)) {
        uint32_t qnan = 0x7FC00000u;
        memcpy(tensor_scale, &qnan, sizeof qnan);
        memset(codes, 0, (size_t)(rows * (cols / 2)));
        memset(scales, 0x7F, (size_t)(rows * nb));
        return 0;
    }
    *tensor_scale = s_t;
    float six_st = 6.0f * s_t;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < rows; ++r) {
        float y[16];
        uint8_t q[16];
        for (int64_t b = 0; b < nb; ++b) {
            for (int i = 0; i < 16; ++i) y[i] = oracle_bf16_to_f32(x[r * cols + b * 16 + i]);
            if (had != HAD_NONE) oracle_fwht(y, 16, signs);
            uint8_t* crow = codes + r * (cols / 2) + b * 8;
            /* a block holding a NaN or an infinity (also one the rotation
             * produced): scale 0x7F (E4M3 NaN), codes zero */
            int finite = 1;
            for (int i = 0; i < 16; ++i) finite &= isfinite(y[i]) != 0;
            if (!finite) {
                memset(crow, 0, 8);
                scales[r * nb + b] = 0x7F;
                continue;
            }
            float m = 0.0f;
            for (int i = 0; i < 16; ++i) { float a = fabsf(y[i]); if (a > m) m = a; }
            uint8_t sb = oracle_e4m3_rne(m / six_st);
            if (sb == 0) {
                memset(crow, 0, 8);
                scales[r * nb + b] = 0;
                continue;
            }
            float sbf = (float)oracle_e4m3_decode(sb);
            float inv = 1.0f / (sbf * s_t);
            /* the reciprocal of the block's scale overflows (a tensor amax
             * below about 2^-125 puts s_b s_t under 2^-128): the codes are
             * zero and the scale stays s_b -- every value such a block
             * dequantizes to is below the binary32 normal range */
            if (isinf(inv)) {
                memset(crow, 0, 8);
                scales[r * nb + b] = sb;
                continue;
            }
            for (int i = 0; i < 16; ++i) {
                float v = y[i] * inv;
                if (mode == 2) {
                    uint64_t idx = (uint64_t)r * (uint64_t)cols + (uint64_t)(b * 16 + i);
                    q[i] = oracle_e2m1_sr(v, oracle_stream_word(sr_seed, 0, idx));
                } else {
                    q[i] = oracle_e2m1_rtn(v);
                }
            }
            for (int j = 0; j < 8; ++j) crow[j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
            uint8_t stored = sb;
            if (mode == 1) {
                float num = 0.0f, den = 0.0f;
                for (int i = 0; i < 16; ++i) {
                    num = fmaf(y[i], y[i], num);
                    den = fmaf(y[i], (float)oracle_e2m1_decode(q[i]), den);
                }
                /* the renormalized scale needs den > 0 and a target that is
                 * a number (sums of squares of values near the binary32 limit
                 * overflow; Inf / Inf keeps s_b, an infinite target saturates
                 * at 448) */
                if (den > 0.0f) {
                    float target = num / (s_t * den);
                    uint64_t blk = (uint64_t)r * (uint64_t)nb + (uint64_t)b;
                    if (!isnan(target))
                        stored = oracle_e4m3_sr(target, oracle_stream_word(sr_seed, 2, blk));
                }
            }
            scales[r * nb + b] = stored;
        }
    }
    return 0;
}

/* Number of OpenMP threads the oracle's parallel loops use. */
int oracle_num_threads(void) {
    int n = 1;
#ifdef _OPENMP
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
#endif
    return n;
}
