/* Drives every entry point of oracle/fp4_oracle.c on small inputs with the
 * cases the method has (zeros, -0, subnormals, huge values, NaN, +-Inf,
 * every rotation and rounding, both axes, bad arguments), for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py).
 * It checks no values: the sanitizers check the memory accesses and the
 * arithmetic; the oracle's values are pinned by the other CPU tests. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_quant_mx(const uint16_t* x, int64_t rows, int64_t cols, int axis, int had_n, int had,
                    uint64_t sign_seed, int rnd, uint64_t sr_seed, int64_t r0, int64_t r1,
                    uint8_t* codes, uint8_t* scales);
void oracle_dequant_mx(const uint8_t* codes, const uint8_t* scales, int64_t C, int64_t r0, int64_t r1,
                       double* out);
void oracle_gemm_mx_entries(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                            int64_t K, const int64_t* mi, const int64_t* ni, int64_t n, double* c,
                            double* s);
void oracle_gemm_mx_rows(const uint8_t* aq, const uint8_t* as, const uint8_t* bq, const uint8_t* bs,
                         int64_t M, int64_t N, int64_t K, int64_t m0, int64_t m1, double* c, double* s);
float oracle_nvfp4_amax(const uint16_t* x, int64_t rows, int64_t cols, int had, uint64_t sign_seed);
int oracle_nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, int had, uint64_t sign_seed,
                          int mode, uint64_t sr_seed, const float* amax_in, uint8_t* codes,
                          uint8_t* scales, float* tensor_scale);
uint32_t oracle_stream_word(uint64_t seed, uint32_t purpose, uint64_t index);

static uint16_t bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* x[rows, cols] of bf16 patterns: random values of many magnitudes with the
 * special values planted at fixed positions */
static uint16_t* make_input(int64_t rows, int64_t cols, uint64_t seed) {
    uint16_t* x = (uint16_t*)malloc((size_t)(rows * cols) * 2);
    for (int64_t i = 0; i < rows * cols; ++i) {
        uint32_t w = oracle_stream_word(seed, 7u, (uint64_t)i);
        float v = ldexpf((float)(w & 0xFFFF) / 65536.0f - 0.5f, (int)((w >> 16) % 60) - 30);
        x[i] = bf16(v);
    }
    const uint16_t specials[] = {0x0000, 0x8000, 0x0001, 0x8001, 0x7F7F, 0xFF7F, 0x7F80,
                                 0xFF80, 0x7FC0, 0x3F80, 0x40C0, 0x4100};
    for (size_t k = 0; k < sizeof(specials) / sizeof(specials[0]); ++k)
        x[(int64_t)(k * 37) % (rows * cols)] = specials[k];
    return x;
}

int main(void) {
    const int64_t rows = 96, cols = 64;
    uint16_t* x = make_input(rows, cols, 11);
    const int hads[][2] = {{0, 32}, {1, 32}, {2, 32}, {1, 16}, {2, 16}};
    for (int axis = 0; axis < 2; ++axis) {
        const int64_t R = axis == 0 ? rows : cols, C = axis == 0 ? cols : rows;
        uint8_t* codes = (uint8_t*)malloc((size_t)(R * C / 2));
        uint8_t* scales = (uint8_t*)malloc((size_t)(R * C / 32));
        double* deq = (double*)malloc((size_t)(R * C) * sizeof(double));
        for (size_t h = 0; h < sizeof(hads) / sizeof(hads[0]); ++h)
            for (int rnd = 0; rnd < 2; ++rnd) {
                if (oracle_quant_mx(x, rows, cols, axis, hads[h][1], hads[h][0], 5, rnd, 9, 0, R, codes,
                                    scales))
                    return 2;
                /* a range of logical rows only */
                if (oracle_quant_mx(x, rows, cols, axis, hads[h][1], hads[h][0], 5, rnd, 9, 3, R - 2,
                                    codes, scales))
                    return 3;
                oracle_dequant_mx(codes, scales, C, 0, R, deq);
            }
        /* the GEMM of the operand with itself: all rows, then sampled entries */
        double* c = (double*)malloc((size_t)(R * R) * sizeof(double));
        double* s = (double*)malloc((size_t)(R * R) * sizeof(double));
        oracle_gemm_mx_rows(codes, scales, codes, scales, R, R, C, 0, R, c, s);
        oracle_gemm_mx_rows(codes, scales, codes, scales, R, R, C, R - 1, R, c, s);
        int64_t mi[4] = {0, R - 1, 1, R - 1}, ni[4] = {0, 0, R - 1, R - 1};
        oracle_gemm_mx_entries(codes, scales, codes, scales, C, mi, ni, 4, c, s);
        free(c);
        free(s);
        free(deq);
        free(codes);
        free(scales);
    }
    /* bad arguments are refused without touching the buffers */
    uint8_t dummy[16];
    if (!oracle_quant_mx(x, rows, cols, 2, 32, 0, 0, 0, 0, 0, 1, dummy, dummy)) return 4;
    if (!oracle_quant_mx(x, rows, 33, 0, 32, 0, 0, 0, 0, 0, 1, dummy, dummy)) return 5;
    if (!oracle_quant_mx(x, rows, cols, 0, 8, 1, 0, 0, 0, 0, 1, dummy, dummy)) return 6;
    if (!oracle_quant_mx(x, rows, cols, 0, 32, 0, 0, 0, 0, 5, 2, dummy, dummy)) return 7;
    if (!oracle_quant_mx(x, rows, cols, 0, 32, 0, 0, 0, 0, 0, rows + 1, dummy, dummy)) return 8;

    /* NVFP4: every mode, computed and supplied amax, NaN / infinite / tiny amax */
    const int64_t nr = 48, nc = 80;
    uint16_t* y = make_input(nr, nc, 23);
    uint8_t* q = (uint8_t*)malloc((size_t)(nr * nc / 2));
    uint8_t* sc = (uint8_t*)malloc((size_t)(nr * nc / 16));
    float ts;
    const float amaxes[] = {1.0f, 0.0f, NAN, INFINITY, -1.0f, 1e-40f, 3.0e38f};
    for (int had = 0; had < 3; ++had)
        for (int mode = 0; mode < 3; ++mode) {
            (void)oracle_nvfp4_amax(y, nr, nc, had, 3);
            if (oracle_nvfp4_quantize(y, nr, nc, had, 3, mode, 4, NULL, q, sc, &ts)) return 9;
            for (size_t k = 0; k < sizeof(amaxes) / sizeof(amaxes[0]); ++k)
                if (oracle_nvfp4_quantize(y, nr, nc, had, 3, mode, 4, &amaxes[k], q, sc, &ts)) return 10;
        }
    if (!oracle_nvfp4_quantize(y, nr, 24, 1, 0, 0, 0, NULL, q, sc, &ts)) return 11;
    if (!oracle_nvfp4_quantize(y, nr, nc, 1, 0, 3, 0, NULL, q, sc, &ts)) return 12;
    free(q);
    free(sc);
    free(y);
    free(x);
    printf("ok\n");
    return 0;
}
