/*
 * sanitize_check.c -- drives every entry point of the oracle once on small seeded inputs,
 * for a build with AddressSanitizer and UndefinedBehaviorSanitizer:
 *
 *   gcc -O1 -g -std=c11 -fsanitize=address,undefined -fno-sanitize-recover=all \
 *       -ffp-contract=off -o sanitize_check oracle.c sanitize_check.c -lm
 *
 * TEST INFRASTRUCTURE ONLY (run by the CPU tests).  Every buffer is allocated at exactly the
 * size the oracle's layout rules give, so a read or write past one ends the run with a report;
 * any undefined behaviour does too.  Exit status 0 means the whole drive ran clean.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float or_bf16_to_f32(uint16_t b);
float or_fp16_decode(uint16_t h);
uint16_t or_fp16_encode(float x);
float or_e4m3_decode(uint8_t b);
uint8_t or_e4m3_encode(float x);
float or_e2m1_decode(uint8_t c);
uint8_t or_e2m1_encode(float y);
void or_nf4_codebook(float* c, double* mid);
int or_packed_size(int fmt, int dq, int64_t n, int64_t k, int64_t* codes_bytes, int64_t* scales_bytes);
int or_quantize_packed(int fmt, int dq, int64_t n, int64_t k, const float* w, uint8_t* codes_packed,
                       uint8_t* scales_packed, uint8_t* codes_logical, float* w_hat);
void or_unpack_codes4(int64_t n, int64_t k, const uint8_t* packed, uint8_t* codes);
void or_matmul_rows(int64_t nrows, const int64_t* rows, int64_t n, int64_t k, const uint16_t* x, const float* w_hat,
                    const uint16_t* bias, float* y);
int64_t or_act_scales_bytes(int64_t m, int64_t k);
void or_quantize_act_nvfp4(int64_t m, int64_t k, const uint16_t* x, uint8_t* codes_packed, uint8_t* scales_packed,
                           uint8_t* codes_logical, float* x_hat);
void or_matmul_rows_f32x(int64_t nrows, const int64_t* rows, int64_t n, int64_t k, const float* x,
                         const float* w_hat, const uint16_t* bias, float* y);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {            /* xorshift64*, for input data only */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float uniform_pm1(void) { return (float)((double)next_u32() / 4294967296.0 * 2.0 - 1.0); }

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

/* weights: mostly small uniform values, a zero block-sized run, a few large outliers */
static void fill_weights(float* w, int64_t n, int64_t k, int zero_all) {
    for (int64_t i = 0; i < n * k; i++) w[i] = zero_all ? 0.0f : 0.02f * uniform_pm1();
    if (zero_all) return;
    for (int64_t i = 0; i < 64 && i < n * k; i++) w[i] = 0.0f;
    w[n * k / 2] = 1.5f;
    w[n * k - 1] = -3.0f;
}

static void drive_format(int fmt, int dq, int64_t n, int64_t k, int zero_all) {
    int64_t cb, sb;
    if (or_packed_size(fmt, dq, n, k, &cb, &sb)) return;     /* shape not offered for this format */
    float* w = xmalloc(sizeof(float) * (size_t)(n * k));
    uint8_t* codes = xmalloc((size_t)cb);
    uint8_t* scales = xmalloc((size_t)sb);
    uint8_t* logical = xmalloc((size_t)(n * k));
    float* w_hat = xmalloc(sizeof(float) * (size_t)(n * k));
    fill_weights(w, n, k, zero_all);
    if (or_quantize_packed(fmt, dq, n, k, w, codes, scales, logical, w_hat)) {
        fprintf(stderr, "quantize failed fmt=%d dq=%d n=%lld k=%lld\n", fmt, dq, (long long)n, (long long)k);
        exit(1);
    }
    if (fmt != 4 && fmt != 8) {                               /* 4-bit packed codes */
        uint8_t* back = xmalloc((size_t)(n * k));
        or_unpack_codes4(n, k, codes, back);
        free(back);
    }
    const int64_t m = 5;
    uint16_t* x = xmalloc(sizeof(uint16_t) * (size_t)(m * k));
    for (int64_t i = 0; i < m * k; i++) x[i] = (uint16_t)(0x3F80u ^ (next_u32() & 0x80FFu));
    uint16_t* bias = xmalloc(sizeof(uint16_t) * (size_t)n);
    for (int64_t i = 0; i < n; i++) bias[i] = 0x3C00u;
    int64_t rows[3] = {4, 0, 2};
    float* y = xmalloc(sizeof(float) * (size_t)(3 * n));
    or_matmul_rows(3, rows, n, k, x, w_hat, bias, y);
    or_matmul_rows(m > 3 ? 3 : m, NULL, n, k, x, w_hat, NULL, y);
    free(w); free(codes); free(scales); free(logical); free(w_hat); free(x); free(bias); free(y);
}

static void drive_activations(int64_t m, int64_t k, int zero_all) {
    uint16_t* x = xmalloc(sizeof(uint16_t) * (size_t)(m * k));
    for (int64_t i = 0; i < m * k; i++) x[i] = zero_all ? 0 : (uint16_t)(0x3F80u ^ (next_u32() & 0x83FFu));
    uint8_t* codes = xmalloc((size_t)(m * k / 2));
    uint8_t* scales = xmalloc((size_t)or_act_scales_bytes(m, k));
    uint8_t* logical = xmalloc((size_t)(m * k));
    float* x_hat = xmalloc(sizeof(float) * (size_t)(m * k));
    or_quantize_act_nvfp4(m, k, x, codes, scales, logical, x_hat);
    const int64_t n = 32;
    float* w_hat = xmalloc(sizeof(float) * (size_t)(n * k));
    for (int64_t i = 0; i < n * k; i++) w_hat[i] = 0.02f * uniform_pm1();
    float* y = xmalloc(sizeof(float) * (size_t)(m * n));
    or_matmul_rows_f32x(m, NULL, n, k, x_hat, w_hat, NULL, y);
    free(x); free(codes); free(scales); free(logical); free(x_hat); free(w_hat); free(y);
}

int main(void) {
    /* scalar codecs over their whole input sets, and the codebook */
    volatile float acc = 0.0f;
    for (uint32_t b = 0; b < 65536; b++) acc += or_fp16_decode((uint16_t)b) * 0.0f + or_bf16_to_f32((uint16_t)b) * 0.0f;
    for (uint32_t b = 0; b < 256; b++) acc += or_e4m3_decode((uint8_t)b) * 0.0f;
    for (uint32_t c = 0; c < 16; c++) acc += or_e2m1_decode((uint8_t)c);
    const float probes[] = {0.0f, -0.0f, 1e-30f, 0.3f, 2.5f, 5.0f, 6.5f, 448.0f, 500.0f, 65504.0f, 1e30f, -1e30f};
    for (size_t i = 0; i < sizeof(probes) / sizeof(probes[0]); i++)
        acc += (float)or_fp16_encode(probes[i]) + (float)or_e4m3_encode(probes[i]) + (float)or_e2m1_encode(probes[i]);
    float c[16];
    double mid[15];
    or_nf4_codebook(c, mid);
    /* every format (NF4 with and without double quantization), two shapes, random and zero weights */
    const int64_t shapes[3][2] = {{16, 256}, {48, 512}, {16, 128}};
    for (int fmt = 1; fmt <= 8; fmt++)
        for (int dq = 0; dq <= (fmt == 1); dq++)
            for (int s = 0; s < 3; s++)
                for (int z = 0; z <= 1; z++) drive_format(fmt, dq, shapes[s][0], shapes[s][1], z);
    drive_activations(3, 48, 0);
    drive_activations(7, 160, 0);
    drive_activations(2, 16, 1);
    (void)acc;
    printf("sanitize_check: clean\n");
    return 0;
}
