/*
 * oracle.c -- plain, slow CPU reference for the weight-only 4-bit matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the CPU-baseline
 * leg of the bench may load this library.  The HIP library shares no code,
 * header, table or generator with it.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math -fopenmp
 * (-ffp-contract=off keeps every multiply and add a separately rounded binary32
 * operation; OpenMP is used only across output rows of the matmul).
 *
 * Notation: fl() is binary32 round-to-nearest-even of the exact result.  Every
 * step below is one C float operation, so it is exactly one fl().
 *
 * What the pages fix, and where:
 *   - NF4 with double-quantized absmax and bf16 compute: "asr: add a 4-bit nf4
 *     option for the Whisper engine", intro and section "What's here".
 *   - NVFP4 = E2M1 codes in 16-value blocks, an FP8 E4M3 scale per block and
 *     one FP32 global scale per module: "asr: add a 4-bit nvfp4 option for cards
 *     short of VRAM", intro; "mbehr90/whisper-large-v3-turbo-nvfp4", section
 *     "What is quantized".
 *   - q8_0 / q4_0 block formats: "Run quantized Whisper on the fused Metal
 *     decode path", sections "Summary" and "Why the policy"; q4_1, q5_0 and
 *     q4_k are named there too (section "Why the policy") as formats that
 *     decode correctly but lack fast kernels, and q6_k as one the encoder may
 *     use (same section).
 *   - NVFP4 activations quantized per 16-value group at run time (W4A4):
 *     "mbehr90/whisper-large-v3-turbo-nvfp4", section "What is quantized".
 *   - Host reference path for quantized linears used to rule out kernel bugs:
 *     same page, section "Why the policy".
 * Everything the pages leave open (codebook values, rounding, tie-breaks,
 * double-quant details, packed layout) follows the readings listed in the
 * design notes; each function states the reading it implements.
 *
 * Parity status: every function here is pinned by tests under tests/ (library
 * cross-checks, brute force on tiny inputs, closed forms, byte accounting
 * against sizes the pages print).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_NF4 1
#define OR_NVFP4 2
#define OR_Q4_0 3
#define OR_Q8_0 4
#define OR_Q4_1 5
#define OR_Q5_0 6
#define OR_Q4_K 7
#define OR_Q6_K 8

/* ------------------------------------------------------------------------ */
/* Scalar codecs                                                              */
/* ------------------------------------------------------------------------ */

/* bfloat16 bit pattern -> float (exact widening). */
float or_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* IEEE binary16 decode: sign, 5-bit exponent (bias 15), 10-bit fraction. */
float or_fp16_decode(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);               /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp(1024.0 + m, e - 25);           /* (1 + m/1024) * 2^(e-15) */
    return (float)(s ? -v : v);
}

/* binary16 encode, round-to-nearest-even, saturating to +-65504 (no infinity
 * is ever produced; the q4_0/q8_0 scale is a finite fp16 by construction).
 * The value is scaled by a power of two (exact in double) so that one quantum
 * of its binade is 1, then rint() (ties-to-even in the default rounding mode)
 * picks the integer significand; a carry into the next binade falls out of
 * the encoding naturally. */
uint16_t or_fp16_encode(float x) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (a >= 65504.0) return sign | 0x7BFF;
    if (a < ldexp(1.0, -14)) {                   /* subnormal binade, quantum 2^-24 */
        double q = rint(ldexp(a, 24));           /* 0 .. 1024 */
        return sign | (uint16_t)q;
    }
    int e2;
    frexp(a, &e2);                               /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;                              /* a in [2^E, 2^(E+1)) */
    double q = rint(ldexp(a, 10 - E));           /* 1024 .. 2048 */
    uint32_t bits = ((uint32_t)(E + 15) << 10) + ((uint32_t)q - 1024u);
    if (bits > 0x7BFF) bits = 0x7BFF;            /* rounding up past 65504 saturates */
    return sign | (uint16_t)bits;
}

/* OCP FP8 E4M3FN decode: bias 7, no infinities, S.1111.111 is NaN. */
float or_e4m3_decode(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);                /* subnormal: m/8 * 2^-6 */
    else
        v = ldexp(8.0 + m, e - 10);              /* (1 + m/8) * 2^(e-7) */
    return (float)(s ? -v : v);
}

/* E4M3 encode of a non-negative value: nearest finite E4M3 value, ties to the
 * even code, values above the largest finite (448) saturate to it.  Done by
 * brute force over the 127 non-negative finite codes. */
uint8_t or_e4m3_encode(float x) {
    if (!(x <= 448.0f)) return 0x7E;             /* > 448 or +inf: saturate */
    if (x < 0.0f) x = 0.0f;                      /* only non-negative scales occur */
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c <= 0x7E; c++) {
        double d = fabs((double)or_e4m3_decode((uint8_t)c) - (double)x);
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)best;
}

/* E2M1 magnitudes by 3-bit code: 2 exponent bits (bias 1), 1 mantissa bit. */
static const float E2M1_MAG[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

/* E2M1 decode of a 4-bit code (bit 3 = sign). */
float or_e2m1_decode(uint8_t c) {
    float v = E2M1_MAG[c & 7];
    return (c & 8) ? -v : v;
}

/* E2M1 encode: magnitude code = nearest of the 8 magnitudes to |y|, ties to
 * the even code, anything above 6 saturates to 6; sign bit = signbit(y). */
uint8_t or_e2m1_encode(float y) {
    double a = fabs((double)y);
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c < 8; c++) {
        double d = fabs((double)E2M1_MAG[c] - a);
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)(best | (signbit(y) ? 8 : 0));
}

/* ------------------------------------------------------------------------ */
/* NF4 codebook (NormalFloat, Dettmers et al. 2023 "QLoRA"; the pages only     */
/* name NF4).  Construction read from that definition:                         */
/*   delta = ((1 - 1/30) + (1 - 1/32)) / 2                                      */
/*   positive part: Phi^-1 at 9 points spaced linearly from delta to 1/2,     */
/*                  dropping the 1/2 point (8 values)                          */
/*   negative part: -Phi^-1 at 8 points spaced linearly from delta to 1/2,    */
/*                  dropping the 1/2 point (7 values)                          */
/*   add 0, sort, divide by the largest, round each to binary32.              */
/* ------------------------------------------------------------------------ */

/* Standard normal CDF from the complementary error function. */
static double norm_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

/* Phi^-1 by bisection on the monotone CDF, to the last binary64 bit. */
static double norm_ppf(double p) {
    double lo = -40.0, hi = 40.0;
    for (int it = 0; it < 400; it++) {
        double mid = 0.5 * (lo + hi);
        if (mid == lo || mid == hi) break;
        if (norm_cdf(mid) < p) lo = mid; else hi = mid;
    }
    /* pick whichever end is closer in CDF terms */
    return (fabs(norm_cdf(lo) - p) <= fabs(norm_cdf(hi) - p)) ? lo : hi;
}

static int cmp_double(const void* a, const void* b) {
    double x = *(const double*)a, y = *(const double*)b;
    return (x > y) - (x < y);
}

/* Fills c[16] (binary32 levels, ascending) and mid[15] (exact binary64
 * midpoints between neighbouring levels). */
void or_nf4_codebook(float* c, double* mid) {
    const double delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0));
    double v[16];
    int n = 0;
    for (int i = 0; i < 8; i++) {                /* 9 points, last one (1/2) dropped */
        double p = delta + (0.5 - delta) * (double)i / 8.0;
        v[n++] = norm_ppf(p);
    }
    for (int i = 0; i < 7; i++) {                /* 8 points, last one (1/2) dropped */
        double p = delta + (0.5 - delta) * (double)i / 7.0;
        v[n++] = -norm_ppf(p);
    }
    v[n++] = 0.0;
    qsort(v, 16, sizeof(double), cmp_double);
    double mx = v[15];
    for (int i = 0; i < 16; i++) c[i] = (float)(v[i] / mx);
    if (mid)
        for (int i = 0; i < 15; i++) mid[i] = ((double)c[i] + (double)c[i + 1]) / 2.0;
}

/* ------------------------------------------------------------------------ */
/* NF4 quantization, blocks of 64 along K within a row.                        */
/*   a = max |w| over the block (exact).                                        */
/*   a == 0: every code is 7 (the level 0) and the stored absmax is 0.          */
/*   else  : x = fl(w / a); code = number of midpoints strictly below x, i.e.   */
/*           the nearest level with ties going to the lower index.             */
/*   dequant: w^ = fl(c[code] * a).                                            */
/* codes: one code per byte, logical [n][k]; absmax: logical [n][k/64].        */
/* ------------------------------------------------------------------------ */
void or_nf4_quantize(int64_t n, int64_t k, const float* w, uint8_t* codes, float* absmax) {
    float c[16];
    double mid[15];
    or_nf4_codebook(c, mid);
    const int64_t nbk = k / 64;
    for (int64_t r = 0; r < n; r++) {
        for (int64_t b = 0; b < nbk; b++) {
            const float* src = w + r * k + b * 64;
            uint8_t* dst = codes + r * k + b * 64;
            float a = 0.0f;
            for (int i = 0; i < 64; i++) {
                float t = fabsf(src[i]);
                if (t > a) a = t;
            }
            absmax[r * nbk + b] = a;
            for (int i = 0; i < 64; i++) {
                if (a == 0.0f) { dst[i] = 7; continue; }
                float x = src[i] / a;
                int code = 0;
                for (int j = 0; j < 15; j++)
                    if ((double)x > mid[j]) code++;
                dst[i] = (uint8_t)code;
            }
        }
    }
}

/* Double quantization of the nb first-level absmax values a[] (logical block
 * order = row-major over [n][k/64]):
 *   mu  = fl32( (sum of a[i] in binary64, ascending i) / nb )   (division in binary64)
 *   a'  = fl(a[i] - mu)
 *   groups of 256 consecutive blocks (last may be partial):
 *   s_g = max |a'| over the group, d_g = fl(s_g / 127)
 *   q_i = 0 if d_g == 0 else clamp(rint(fl(a'_i / d_g)), -127, 127)   (int8)
 *   dequantized absmax  a^_i = fl( fl(q_i * d_g) + mu ).
 */
void or_nf4_double_quant(int64_t nb, const float* a, int8_t* q, float* d, float* mu_out) {
    double s = 0.0;
    for (int64_t i = 0; i < nb; i++) s += (double)a[i];
    float mu = (float)(s / (double)nb);
    *mu_out = mu;
    int64_t ng = (nb + 255) / 256;
    for (int64_t g = 0; g < ng; g++) {
        int64_t i0 = g * 256, i1 = i0 + 256 < nb ? i0 + 256 : nb;
        float sg = 0.0f;
        for (int64_t i = i0; i < i1; i++) {
            float t = fabsf(a[i] - mu);
            if (t > sg) sg = t;
        }
        float dg = sg / 127.0f;
        d[g] = dg;
        for (int64_t i = i0; i < i1; i++) {
            if (dg == 0.0f) { q[i] = 0; continue; }
            float r = rintf((a[i] - mu) / dg);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q[i] = (int8_t)r;
        }
    }
}

/* a^_i = fl(fl(q_i * d_g) + mu) for every block. */
void or_nf4_dq_absmax(int64_t nb, const int8_t* q, const float* d, float mu, float* ahat) {
    for (int64_t i = 0; i < nb; i++) {
        float t = (float)q[i] * d[i / 256];
        ahat[i] = t + mu;
    }
}

/* w^ = fl(c[code] * absmax_of_block); absmax is the exact absmax (plain NF4)
 * or the double-quant reconstruction a^ (NF4 with double-quant). */
void or_nf4_dequantize(int64_t n, int64_t k, const uint8_t* codes, const float* absmax, float* out) {
    float c[16];
    or_nf4_codebook(c, NULL);
    const int64_t nbk = k / 64;
    for (int64_t r = 0; r < n; r++)
        for (int64_t i = 0; i < k; i++)
            out[r * k + i] = c[codes[r * k + i] & 15] * absmax[r * nbk + i / 64];
}

/* ------------------------------------------------------------------------ */
/* NVFP4: E2M1 codes, blocks of 16 along K, one E4M3 scale per block and one    */
/* FP32 global scale g per matrix (decode direction: w^ = e2m1 * e4m3 * g).     */
/*   A = max |W| over the matrix; g = fl(A / 2688) (2688 = 6 * 448).             */
/*   g == 0: every scale byte is 0 and every code carries only the sign.       */
/*   else: t = fl(6 * g); per block a_b = max|w|, s_b = e4m3(fl(a_b / t)),      */
/*         sigma = fl(val(s_b) * g); magnitude code = 0 if sigma == 0 else      */
/*         e2m1(fl(w / sigma)); sign bit = signbit(w).                           */
/*   dequant: w^ = fl( fl(e2m1(code) * val(s_b)) * g ).                         */
/* codes logical [n][k] (4-bit per byte), scales logical [n][k/16] bytes.       */
/* ------------------------------------------------------------------------ */
void or_nvfp4_quantize(int64_t n, int64_t k, const float* w, uint8_t* codes, uint8_t* scales, float* g_out) {
    float A = 0.0f;
    for (int64_t i = 0; i < n * k; i++) {
        float t = fabsf(w[i]);
        if (t > A) A = t;
    }
    float g = A / 2688.0f;
    *g_out = g;
    const int64_t nbk = k / 16;
    if (g == 0.0f) {
        for (int64_t i = 0; i < n * k; i++) codes[i] = signbit(w[i]) ? 8 : 0;
        memset(scales, 0, (size_t)(n * nbk));
        return;
    }
    float t = 6.0f * g;
    for (int64_t r = 0; r < n; r++) {
        for (int64_t b = 0; b < nbk; b++) {
            const float* src = w + r * k + b * 16;
            float ab = 0.0f;
            for (int i = 0; i < 16; i++) {
                float u = fabsf(src[i]);
                if (u > ab) ab = u;
            }
            uint8_t sb = or_e4m3_encode(ab / t);
            scales[r * nbk + b] = sb;
            float sigma = or_e4m3_decode(sb) * g;
            for (int i = 0; i < 16; i++) {
                uint8_t code;
                if (sigma == 0.0f)
                    code = signbit(src[i]) ? 8 : 0;
                else
                    code = or_e2m1_encode(src[i] / sigma);
                codes[r * k + b * 16 + i] = code;
            }
        }
    }
}

void or_nvfp4_dequantize(int64_t n, int64_t k, const uint8_t* codes, const uint8_t* scales, float g, float* out) {
    const int64_t nbk = k / 16;
    for (int64_t r = 0; r < n; r++)
        for (int64_t i = 0; i < k; i++) {
            float v = or_e2m1_decode(codes[r * k + i]);
            float s = or_e4m3_decode(scales[r * nbk + i / 16]);
            float p = v * s;
            out[r * k + i] = p * g;
        }
}

/* ------------------------------------------------------------------------ */
/* q8_0: blocks of 32, a = max|w|, d = fp16(fl(a / 127)), delta = float(d),      */
/*   q = 0 if delta == 0 else clamp(rint(fl(w / delta)), -127, 127)  (int8),     */
/*   w^ = fl(q * delta) (exact).                                                 */
/* ------------------------------------------------------------------------ */
void or_q8_0_quantize(int64_t n, int64_t k, const float* w, int8_t* codes, uint16_t* scales) {
    const int64_t nbk = k / 32;
    for (int64_t r = 0; r < n; r++)
        for (int64_t b = 0; b < nbk; b++) {
            const float* src = w + r * k + b * 32;
            float a = 0.0f;
            for (int i = 0; i < 32; i++) {
                float t = fabsf(src[i]);
                if (t > a) a = t;
            }
            uint16_t d = or_fp16_encode(a / 127.0f);
            scales[r * nbk + b] = d;
            float delta = or_fp16_decode(d);
            for (int i = 0; i < 32; i++) {
                int8_t q = 0;
                if (delta != 0.0f) {
                    float v = rintf(src[i] / delta);
                    if (v > 127.0f) v = 127.0f;
                    if (v < -127.0f) v = -127.0f;
                    q = (int8_t)v;
                }
                codes[r * k + b * 32 + i] = q;
            }
        }
}

void or_q8_0_dequantize(int64_t n, int64_t k, const int8_t* codes, const uint16_t* scales, float* out) {
    const int64_t nbk = k / 32;
    for (int64_t r = 0; r < n; r++)
        for (int64_t i = 0; i < k; i++)
            out[r * k + i] = (float)codes[r * k + i] * or_fp16_decode(scales[r * nbk + i / 32]);
}

/* ------------------------------------------------------------------------ */
/* q4_0: blocks of 32.  m = the signed element of largest magnitude (first one  */
/* in ascending k on a tie); d = fp16(fl(m / -8)); delta = float(d);            */
/*   q = 8 if delta == 0 else clamp(rint(fl(w / delta)), -8, 7) + 8   (nibble),  */
/*   w^ = fl((q - 8) * delta) (exact; -0.0 when q == 8 and delta < 0).           */
/* ------------------------------------------------------------------------ */
void or_q4_0_quantize(int64_t n, int64_t k, const float* w, uint8_t* codes, uint16_t* scales) {
    const int64_t nbk = k / 32;
    for (int64_t r = 0; r < n; r++)
        for (int64_t b = 0; b < nbk; b++) {
            const float* src = w + r * k + b * 32;
            float amax = 0.0f, m = src[0];
            for (int i = 0; i < 32; i++) {
                float t = fabsf(src[i]);
                if (t > amax) { amax = t; m = src[i]; }
            }
            uint16_t d = or_fp16_encode(m / -8.0f);
            scales[r * nbk + b] = d;
            float delta = or_fp16_decode(d);
            for (int i = 0; i < 32; i++) {
                uint8_t q = 8;
                if (delta != 0.0f) {
                    float v = rintf(src[i] / delta);
                    if (v > 7.0f) v = 7.0f;
                    if (v < -8.0f) v = -8.0f;
                    q = (uint8_t)((int)v + 8);
                }
                codes[r * k + b * 32 + i] = q;
            }
        }
}

void or_q4_0_dequantize(int64_t n, int64_t k, const uint8_t* codes, const uint16_t* scales, float* out) {
    const int64_t nbk = k / 32;
    for (int64_t r = 0; r < n; r++)
        for (int64_t i = 0; i < k; i++)
            out[r * k + i] = (float)((int)codes[r * k + i] - 8) * or_fp16_decode(scales[r * nbk + i / 32]);
}

/* ------------------------------------------------------------------------ */
/* q4_1: blocks of 32 with an fp16 scale d and an fp16 minimum m, unsigned      */
/* codes.  The page only names the format; reading (as for q4_0): the codes are  */
/* chosen against the stored fp16 values, rounding to nearest even.             */
/*   lo = min(w), hi = max(w) over the block (exact);                            */
/*   d = fp16(fl(fl(hi - lo) / 15)), m = fp16(lo); delta = float(d), mu = float(m) */
/*   q = 0 if delta == 0 else clamp(rint(fl(fl(w - mu) / delta)), 0, 15);        */
/*   w^ = fl(q * delta + mu), one rounding (q * delta has <= 15 significant bits */
/*   and is exact).                                                               */
/* scales: [n][k/32][2] fp16, d first.                                           */
/* ------------------------------------------------------------------------ */
void or_q4_1_quantize(int64_t n, int64_t k, const float* w, uint8_t* codes, uint16_t* scales) {
    const int64_t nbk = k / 32;
    for (int64_t r = 0; r < n; r++)
        for (int64_t b = 0; b < nbk; b++) {
            const float* src = w + r * k + b * 32;
            float lo = src[0], hi = src[0];
            for (int i = 1; i < 32; i++) {
                if (src[i] < lo) lo = src[i];
                if (src[i] > hi) hi = src[i];
            }
            const float range = hi - lo;
            const uint16_t d = or_fp16_encode(range / 15.0f);
            const uint16_t m = or_fp16_encode(lo);
            scales[(r * nbk + b) * 2] = d;
            scales[(r * nbk + b) * 2 + 1] = m;
            const float delta = or_fp16_decode(d), mu = or_fp16_decode(m);
            for (int i = 0; i < 32; i++) {
                uint8_t q = 0;
                if (delta != 0.0f) {
                    const float t = src[i] - mu;
                    float v = rintf(t / delta);
                    if (v > 15.0f) v = 15.0f;
                    if (v < 0.0f) v = 0.0f;
                    q = (uint8_t)v;
                }
                codes[r * k + b * 32 + i] = q;
            }
        }
}

void or_q4_1_dequantize(int64_t n, int64_t k, const uint8_t* codes, const uint16_t* scales, float* out) {
    const int64_t nbk = k / 32;
    for (int64_t r = 0; r < n; r++)
        for (int64_t i = 0; i < k; i++) {
            const int64_t b = r * nbk + i / 32;
            const float delta = or_fp16_decode(scales[2 * b]), mu = or_fp16_decode(scales[2 * b + 1]);
            const float qd = (float)codes[r * k + i] * delta;      /* exact */
            out[r * k + i] = qd + mu;
        }
}

/* ------------------------------------------------------------------------ */
/* q5_0: blocks of 32, one fp16 scale, signed 5-bit codes.  The page only names */
/* the format; reading, as for q4_0 with one more bit:                          */
/*   m = the signed element of largest magnitude (first in ascending k on a    */
/*   tie); d = fp16(fl(m / -16)); delta = float(d);                             */
/*   q = 16 if delta == 0 else clamp(rint(fl(w / delta)), -16, 15) + 16 (0..31), */
/*   w^ = fl((q - 16) * delta) (exact: 5 + 11 significant bits).                 */
/* codes: [n][k] one 5-bit code per byte; scales: [n][k/32] fp16.              */
/* ------------------------------------------------------------------------ */
void or_q5_0_quantize(int64_t n, int64_t k, const float* w, uint8_t* codes, uint16_t* scales) {
    const int64_t nbk = k / 32;
    for (int64_t r = 0; r < n; r++)
        for (int64_t b = 0; b < nbk; b++) {
            const float* src = w + r * k + b * 32;
            float amax = 0.0f, m = src[0];
            for (int i = 0; i < 32; i++) {
                float t = fabsf(src[i]);
                if (t > amax) { amax = t; m = src[i]; }
            }
            uint16_t d = or_fp16_encode(m / -16.0f);
            scales[r * nbk + b] = d;
            float delta = or_fp16_decode(d);
            for (int i = 0; i < 32; i++) {
                uint8_t q = 16;
                if (delta != 0.0f) {
                    float v = rintf(src[i] / delta);
                    if (v > 15.0f) v = 15.0f;
                    if (v < -16.0f) v = -16.0f;
                    q = (uint8_t)((int)v + 16);
                }
                codes[r * k + b * 32 + i] = q;
            }
        }
}

void or_q5_0_dequantize(int64_t n, int64_t k, const uint8_t* codes, const uint16_t* scales, float* out) {
    const int64_t nbk = k / 32;
    for (int64_t r = 0; r < n; r++)
        for (int64_t i = 0; i < k; i++)
            out[r * k + i] = (float)((int)codes[r * k + i] - 16) * or_fp16_decode(scales[r * nbk + i / 32]);
}

/* ------------------------------------------------------------------------ */
/* q4_k: super-blocks of 256 along K, each 8 sub-blocks of 32; unsigned 4-bit   */
/* codes, per sub-block a 6-bit scale and a 6-bit minimum, per super-block an    */
/* fp16 d and an fp16 dmin.  The page only names the format; reading (one pass,  */
/* no search over scales):                                                       */
/*   per sub-block j: lo = min w, hi = max w; mn = lo if lo < 0 else 0;         */
/*     r = fl(hi - mn), canonicalised to +0 unless r > 0; s_j = fl(r / 15);     */
/*     o_j = fl(0 - mn)   (>= +0);                                               */
/*   d = fp16(fl(max_j s_j / 63)), dmin = fp16(fl(max_j o_j / 63));              */
/*   sc_j = 0 if float(d) == 0 else clamp(rint(fl(s_j / d)), 0, 63);             */
/*   m_j  = 0 if float(dmin) == 0 else clamp(rint(fl(o_j / dmin)), 0, 63);       */
/*   S_j = fl(d * sc_j), O_j = fl(dmin * m_j)  (both exact: 11 + 6 bits);         */
/*   q = 0 if S_j == 0 else clamp(rint(fl(fl(w + O_j) / S_j)), 0, 15);           */
/*   w^ = fl(S_j * q - O_j): S_j * q is exact (21 bits), so one rounding.         */
/* sub: [n][k/32][2] bytes (sc, m); dd: [n][k/256][2] fp16 (d, dmin).            */
/* ------------------------------------------------------------------------ */
void or_q4_k_quantize(int64_t n, int64_t k, const float* w, uint8_t* codes, uint8_t* sub, uint16_t* dd) {
    const int64_t nsb = k / 256;
    for (int64_t r = 0; r < n; r++)
        for (int64_t b = 0; b < nsb; b++) {
            const float* src = w + r * k + b * 256;
            float s[8], o[8], smax = 0.0f, omax = 0.0f;
            for (int j = 0; j < 8; j++) {
                float lo = src[32 * j], hi = src[32 * j];
                for (int i = 1; i < 32; i++) {
                    if (src[32 * j + i] < lo) lo = src[32 * j + i];
                    if (src[32 * j + i] > hi) hi = src[32 * j + i];
                }
                const float mn = lo < 0.0f ? lo : 0.0f;
                float range = hi - mn;
                if (!(range > 0.0f)) range = 0.0f;
                s[j] = range / 15.0f;
                o[j] = 0.0f - mn;
                if (s[j] > smax) smax = s[j];
                if (o[j] > omax) omax = o[j];
            }
            const uint16_t db = or_fp16_encode(smax / 63.0f), mb = or_fp16_encode(omax / 63.0f);
            dd[(r * nsb + b) * 2] = db;
            dd[(r * nsb + b) * 2 + 1] = mb;
            const float d = or_fp16_decode(db), dmin = or_fp16_decode(mb);
            for (int j = 0; j < 8; j++) {
                float sc = 0.0f, m = 0.0f;
                if (d != 0.0f) {
                    sc = rintf(s[j] / d);
                    if (sc > 63.0f) sc = 63.0f;
                    if (sc < 0.0f) sc = 0.0f;
                }
                if (dmin != 0.0f) {
                    m = rintf(o[j] / dmin);
                    if (m > 63.0f) m = 63.0f;
                    if (m < 0.0f) m = 0.0f;
                }
                sub[((r * (k / 32)) + b * 8 + j) * 2] = (uint8_t)sc;
                sub[((r * (k / 32)) + b * 8 + j) * 2 + 1] = (uint8_t)m;
                const float S = d * sc, O = dmin * m;
                for (int i = 0; i < 32; i++) {
                    uint8_t q = 0;
                    if (S != 0.0f) {
                        const float t = src[32 * j + i] + O;
                        float v = rintf(t / S);
                        if (v > 15.0f) v = 15.0f;
                        if (v < 0.0f) v = 0.0f;
                        q = (uint8_t)v;
                    }
                    codes[r * k + b * 256 + 32 * j + i] = q;
                }
            }
        }
}

void or_q4_k_dequantize(int64_t n, int64_t k, const uint8_t* codes, const uint8_t* sub, const uint16_t* dd, float* out) {
    const int64_t nsb = k / 256;
    for (int64_t r = 0; r < n; r++)
        for (int64_t i = 0; i < k; i++) {
            const int64_t b = i / 256, j = i / 32;
            const float d = or_fp16_decode(dd[(r * nsb + b) * 2]), dmin = or_fp16_decode(dd[(r * nsb + b) * 2 + 1]);
            const float S = d * (float)sub[(r * (k / 32) + j) * 2], O = dmin * (float)sub[(r * (k / 32) + j) * 2 + 1];
            const float sq = S * (float)codes[r * k + i];      /* exact */
            out[r * k + i] = sq - O;
        }
}

/* ------------------------------------------------------------------------ */
/* q6_k: super-blocks of 256 along K, each 16 sub-blocks of 16; signed 6-bit     */
/* codes, an int8 scale per sub-block, an fp16 d per super-block.  The page only */
/* names the format; reading (one pass, as q4_0 per sub-block):                  */
/*   per sub-block j: m = signed element of largest magnitude (first in          */
/*     ascending k on a tie); s_j = fl(m / -32);                                  */
/*   d = fp16(fl(max_j |s_j| / 127));                                            */
/*   sc_j = 0 if float(d) == 0 else clamp(rint(fl(s_j / d)), -127, 127);         */
/*   S_j = fl(d * sc_j)  (exact: 11 + 7 bits);                                    */
/*   q = 32 if S_j == 0 else clamp(rint(fl(w / S_j)), -32, 31) + 32  (0..63);    */
/*   w^ = fl(S_j * (q - 32)), exact (at most 24 significant bits).                */
/* sc: [n][k/16] int8; d: [n][k/256] fp16.                                        */
/* ------------------------------------------------------------------------ */
void or_q6_k_quantize(int64_t n, int64_t k, const float* w, uint8_t* codes, int8_t* sc, uint16_t* dsb) {
    const int64_t nsb = k / 256;
    for (int64_t r = 0; r < n; r++)
        for (int64_t b = 0; b < nsb; b++) {
            const float* src = w + r * k + b * 256;
            float s[16], amax = 0.0f;
            for (int j = 0; j < 16; j++) {
                float a = 0.0f, m = src[16 * j];
                for (int i = 0; i < 16; i++) {
                    const float t = fabsf(src[16 * j + i]);
                    if (t > a) { a = t; m = src[16 * j + i]; }
                }
                s[j] = m / -32.0f;
                if (fabsf(s[j]) > amax) amax = fabsf(s[j]);
            }
            const uint16_t db = or_fp16_encode(amax / 127.0f);
            dsb[r * nsb + b] = db;
            const float d = or_fp16_decode(db);
            for (int j = 0; j < 16; j++) {
                float c = 0.0f;
                if (d != 0.0f) {
                    c = rintf(s[j] / d);
                    if (c > 127.0f) c = 127.0f;
                    if (c < -127.0f) c = -127.0f;
                }
                sc[r * (k / 16) + b * 16 + j] = (int8_t)c;
                const float S = d * c;
                for (int i = 0; i < 16; i++) {
                    uint8_t q = 32;
                    if (S != 0.0f) {
                        float v = rintf(src[16 * j + i] / S);
                        if (v > 31.0f) v = 31.0f;
                        if (v < -32.0f) v = -32.0f;
                        q = (uint8_t)((int)v + 32);
                    }
                    codes[r * k + b * 256 + 16 * j + i] = q;
                }
            }
        }
}

void or_q6_k_dequantize(int64_t n, int64_t k, const uint8_t* codes, const int8_t* sc, const uint16_t* dsb, float* out) {
    for (int64_t r = 0; r < n; r++)
        for (int64_t i = 0; i < k; i++) {
            const float d = or_fp16_decode(dsb[r * (k / 256) + i / 256]);
            const float S = d * (float)sc[r * (k / 16) + i / 16];
            out[r * k + i] = S * (float)((int)codes[r * k + i] - 32);
        }
}

/* ------------------------------------------------------------------------ */
/* Packed layout (the library's storage format; the pages give none).          */
/*                                                                              */
/* 4-bit codes (NF4, NVFP4, q4_0, q4_1): the matrix is cut into tiles of 16     */
/* rows x                                                                        */
/* 128 K = 1024 bytes, ordered band-major (band = 16 rows), K-fastest.  Inside  */
/* a tile, 64 slots of 16 bytes; slot s holds row (s mod 16) and K-chunk        */
/* h = s div 16; byte 4j + i/2 of the slot (j = 0..3, i = 0..7) holds          */
/* k = 32j + 8h + i, even i in the low nibble, odd i in the high nibble.        */
/*                                                                              */
/* q8_0 codes: tiles of 16 rows x 64 K = 1024 bytes, same slot rule, byte      */
/* 8j + i of the slot (j = 0..1, i = 0..7) holds k = 32j + 8h + i.              */
/*                                                                              */
/* Scales, per tile, row-major over (row in band, block in tile):               */
/*   NF4     fp32 absmax, 2 per row  (32 per tile)                              */
/*   NF4+DQ  int8 q,      2 per row, then at align16(nb): fp32 d[ng], then mu  */
/*   NVFP4   E4M3 byte,   8 per row  (128 per tile), then at align16(nb): g    */
/*   q4_0    fp16,        4 per row  (64 per tile)                              */
/*   q4_1    fp16 pair (d, m), 4 per row  (64 pairs = 256 bytes per tile)       */
/*   q4_k    per tile and row 8 bytes: the 4 sub-blocks' 6-bit scales, then    */
/*           their 6-bit minimums (one byte each); then at align16(2 nb) the     */
/*           fp16 pairs (d, dmin) of the super-blocks, row-major [n][k/256].     */
/*   q6_k    codes: the low 4 bits in the 4-bit tiles, then (after n k / 2      */
/*           bytes) a plane of 512 bytes per tile: slot s gets 8 bytes, two per   */
/*           K slice j (2j: bit 4 of element i of the slot's 8 k at bit i; 2j+1:  */
/*           bit 5).  scales: per tile and row 8 int8 sub-block scales (one per   */
/*           16 k), then at align16(n k / 16) the fp16 d per super-block,        */
/*           row-major [n][k/256].                                               */
/*   q5_0    fp16 d, 4 per row (like q4_0); then at align16(2 nb) a second     */
/*           plane of one 32-bit word per block, same order (16 bytes per row   */
/*           and tile): bit i holds bit 4 of the code of element i of the block; */
/*           the codes' low 4 bits are the 4-bit codes above.                    */
/*   q8_0    fp16,        2 per row  (32 per 16x64 tile)                        */
/* ------------------------------------------------------------------------ */
static int64_t align16(int64_t v) { return (v + 15) & ~(int64_t)15; }

int or_packed_size(int fmt, int dq, int64_t n, int64_t k, int64_t* codes_bytes, int64_t* scales_bytes) {
    if (n <= 0 || k <= 0 || n % 16) return -1;
    switch (fmt) {
    case OR_NF4: {
        if (k % 128) return -1;
        int64_t nb = n * k / 64;
        *codes_bytes = n * k / 2;
        if (dq) *scales_bytes = align16(nb) + 4 * ((nb + 255) / 256) + 4;
        else *scales_bytes = 4 * nb;
        return 0;
    }
    case OR_NVFP4:
        if (k % 128) return -1;
        *codes_bytes = n * k / 2;
        *scales_bytes = align16(n * k / 16) + 4;
        return 0;
    case OR_Q4_0:
        if (k % 128) return -1;
        *codes_bytes = n * k / 2;
        *scales_bytes = 2 * (n * k / 32);
        return 0;
    case OR_Q4_1:
        if (k % 128) return -1;
        *codes_bytes = n * k / 2;
        *scales_bytes = 4 * (n * k / 32);
        return 0;
    case OR_Q5_0:
        if (k % 128) return -1;
        *codes_bytes = n * k / 2;
        *scales_bytes = align16(2 * (n * k / 32)) + 4 * (n * k / 32);
        return 0;
    case OR_Q4_K:
        if (k % 256) return -1;
        *codes_bytes = n * k / 2;
        *scales_bytes = align16(2 * (n * k / 32)) + 4 * (n * k / 256);
        return 0;
    case OR_Q6_K:
        if (k % 256) return -1;
        *codes_bytes = n * k / 2 + n * k / 4;
        *scales_bytes = align16(n * k / 16) + 2 * (n * k / 256);
        return 0;
    case OR_Q8_0:
        if (k % 64) return -1;
        *codes_bytes = n * k;
        *scales_bytes = 2 * (n * k / 32);
        return 0;
    }
    return -1;
}

/* Byte offset of code (r, kk) in a 4-bit packed matrix and its nibble (0 = low). */
static int64_t pos4(int64_t r, int64_t kk, int64_t k, int* hi) {
    int64_t band = r / 16, row = r % 16;
    int64_t kt = kk / 128, kin = kk % 128;
    int64_t j = kin / 32, h = (kin % 32) / 8, i = kin % 8;
    int64_t tile = band * (k / 128) + kt;
    int64_t slot = h * 16 + row;
    *hi = (int)(i & 1);
    return tile * 1024 + slot * 16 + j * 4 + i / 2;
}

static int64_t pos8(int64_t r, int64_t kk, int64_t k) {
    int64_t band = r / 16, row = r % 16;
    int64_t kt = kk / 64, kin = kk % 64;
    int64_t j = kin / 32, h = (kin % 32) / 8, i = kin % 8;
    int64_t tile = band * (k / 64) + kt;
    int64_t slot = h * 16 + row;
    return tile * 1024 + slot * 16 + j * 8 + i;
}

/* Scale slot of block b (block index along K, block size bs) of row r, for a
 * layout with `per_tile_k` K-values per tile (128 for 4-bit, 64 for q8_0). */
static int64_t scale_slot(int64_t r, int64_t b, int64_t k, int64_t bs, int64_t per_tile_k) {
    int64_t bpt = per_tile_k / bs;                 /* blocks per row per tile */
    int64_t band = r / 16, row = r % 16;
    int64_t kt = b / bpt, bin = b % bpt;
    int64_t tile = band * (k / per_tile_k) + kt;
    return tile * 16 * bpt + row * bpt + bin;
}

/* Pack logical 4-bit codes [n][k] (one per byte) into the tile layout. */
void or_pack_codes4(int64_t n, int64_t k, const uint8_t* codes, uint8_t* out) {
    memset(out, 0, (size_t)(n * k / 2));
    for (int64_t r = 0; r < n; r++)
        for (int64_t kk = 0; kk < k; kk++) {
            int hi;
            int64_t p = pos4(r, kk, k, &hi);
            uint8_t v = codes[r * k + kk] & 15;
            out[p] |= hi ? (uint8_t)(v << 4) : v;
        }
}

void or_pack_codes8(int64_t n, int64_t k, const int8_t* codes, int8_t* out) {
    for (int64_t r = 0; r < n; r++)
        for (int64_t kk = 0; kk < k; kk++) out[pos8(r, kk, k)] = codes[r * k + kk];
}

/* Inverse maps, used by the layout tests. */
void or_unpack_codes4(int64_t n, int64_t k, const uint8_t* packed, uint8_t* codes) {
    for (int64_t r = 0; r < n; r++)
        for (int64_t kk = 0; kk < k; kk++) {
            int hi;
            int64_t p = pos4(r, kk, k, &hi);
            codes[r * k + kk] = hi ? (packed[p] >> 4) : (packed[p] & 15);
        }
}

/* Pack per-block scales of element size esz (bytes) given logically [n][k/bs]. */
void or_pack_scales(int64_t n, int64_t k, int64_t bs, int64_t per_tile_k, int esz, const void* logical, void* out) {
    const int64_t nbk = k / bs;
    const uint8_t* src = (const uint8_t*)logical;
    uint8_t* dst = (uint8_t*)out;
    for (int64_t r = 0; r < n; r++)
        for (int64_t b = 0; b < nbk; b++)
            memcpy(dst + scale_slot(r, b, k, bs, per_tile_k) * esz, src + (r * nbk + b) * esz, (size_t)esz);
}

/* Full quantize to the packed form.  Also returns the logical codes and the
 * dequantized weights so the tests can compare every stage. */
int or_quantize_packed(int fmt, int dq, int64_t n, int64_t k, const float* w,
                       uint8_t* codes_packed, uint8_t* scales_packed,
                       uint8_t* codes_logical, float* w_hat) {
    int64_t cb, sb;
    if (or_packed_size(fmt, dq, n, k, &cb, &sb)) return -1;
    memset(scales_packed, 0, (size_t)sb);
    if (fmt == OR_NF4) {
        int64_t nb = n * k / 64;
        float* a = (float*)malloc(sizeof(float) * nb);
        or_nf4_quantize(n, k, w, codes_logical, a);
        or_pack_codes4(n, k, codes_logical, codes_packed);
        if (dq) {
            int64_t ng = (nb + 255) / 256;
            int8_t* q = (int8_t*)malloc(nb);
            float* d = (float*)malloc(sizeof(float) * ng);
            float* ahat = (float*)malloc(sizeof(float) * nb);
            float mu;
            or_nf4_double_quant(nb, a, q, d, &mu);
            or_pack_scales(n, k, 64, 128, 1, q, scales_packed);
            memcpy(scales_packed + align16(nb), d, sizeof(float) * ng);
            memcpy(scales_packed + align16(nb) + 4 * ng, &mu, 4);
            or_nf4_dq_absmax(nb, q, d, mu, ahat);
            or_nf4_dequantize(n, k, codes_logical, ahat, w_hat);
            free(q); free(d); free(ahat);
        } else {
            or_pack_scales(n, k, 64, 128, 4, a, scales_packed);
            or_nf4_dequantize(n, k, codes_logical, a, w_hat);
        }
        free(a);
        return 0;
    }
    if (fmt == OR_NVFP4) {
        int64_t nb = n * k / 16;
        uint8_t* s = (uint8_t*)malloc(nb);
        float g;
        or_nvfp4_quantize(n, k, w, codes_logical, s, &g);
        or_pack_codes4(n, k, codes_logical, codes_packed);
        or_pack_scales(n, k, 16, 128, 1, s, scales_packed);
        memcpy(scales_packed + align16(nb), &g, 4);
        or_nvfp4_dequantize(n, k, codes_logical, s, g, w_hat);
        free(s);
        return 0;
    }
    if (fmt == OR_Q4_0) {
        uint16_t* s = (uint16_t*)malloc(2 * (n * k / 32));
        or_q4_0_quantize(n, k, w, codes_logical, s);
        or_pack_codes4(n, k, codes_logical, codes_packed);
        or_pack_scales(n, k, 32, 128, 2, s, scales_packed);
        or_q4_0_dequantize(n, k, codes_logical, s, w_hat);
        free(s);
        return 0;
    }
    if (fmt == OR_Q4_1) {
        uint16_t* s = (uint16_t*)malloc(4 * (n * k / 32));
        or_q4_1_quantize(n, k, w, codes_logical, s);
        or_pack_codes4(n, k, codes_logical, codes_packed);
        or_pack_scales(n, k, 32, 128, 4, s, scales_packed);
        or_q4_1_dequantize(n, k, codes_logical, s, w_hat);
        free(s);
        return 0;
    }
    if (fmt == OR_Q5_0) {
        const int64_t nb = n * k / 32;
        uint16_t* s = (uint16_t*)malloc(2 * nb);
        uint32_t* hb = (uint32_t*)calloc((size_t)nb, 4);
        uint8_t* lo = (uint8_t*)malloc((size_t)(n * k));
        or_q5_0_quantize(n, k, w, codes_logical, s);
        for (int64_t r = 0; r < n; r++)
            for (int64_t i = 0; i < k; i++) {
                const uint8_t q = codes_logical[r * k + i];
                lo[r * k + i] = q & 15;
                if (q & 16) hb[r * (k / 32) + i / 32] |= 1u << (i % 32);
            }
        or_pack_codes4(n, k, lo, codes_packed);
        or_pack_scales(n, k, 32, 128, 2, s, scales_packed);
        or_pack_scales(n, k, 32, 128, 4, hb, scales_packed + align16(2 * nb));
        or_q5_0_dequantize(n, k, codes_logical, s, w_hat);
        free(s); free(hb); free(lo);
        return 0;
    }
    if (fmt == OR_Q4_K) {
        const int64_t nb = n * k / 32;
        uint8_t* sub = (uint8_t*)malloc((size_t)(2 * nb));
        uint16_t* dd = (uint16_t*)malloc((size_t)(4 * (n * k / 256)));
        or_q4_k_quantize(n, k, w, codes_logical, sub, dd);
        or_pack_codes4(n, k, codes_logical, codes_packed);
        /* per tile and row: sc of its 4 sub-blocks, then m of them */
        for (int64_t r = 0; r < n; r++)
            for (int64_t b = 0; b < k / 32; b++) {
                const int64_t kt = b / 4, bin = b % 4;
                const int64_t tile = (r / 16) * (k / 128) + kt;
                uint8_t* rec = scales_packed + tile * 128 + (r % 16) * 8;
                rec[bin] = sub[(r * (k / 32) + b) * 2];
                rec[4 + bin] = sub[(r * (k / 32) + b) * 2 + 1];
            }
        memcpy(scales_packed + align16(2 * nb), dd, (size_t)(4 * (n * k / 256)));
        or_q4_k_dequantize(n, k, codes_logical, sub, dd, w_hat);
        free(sub); free(dd);
        return 0;
    }
    if (fmt == OR_Q6_K) {
        int8_t* sc = (int8_t*)malloc((size_t)(n * k / 16));
        uint16_t* dsb = (uint16_t*)malloc((size_t)(2 * (n * k / 256)));
        uint8_t* lo = (uint8_t*)malloc((size_t)(n * k));
        or_q6_k_quantize(n, k, w, codes_logical, sc, dsb);
        for (int64_t i = 0; i < n * k; i++) lo[i] = codes_logical[i] & 15;
        or_pack_codes4(n, k, lo, codes_packed);
        uint8_t* high = codes_packed + n * k / 2;
        memset(high, 0, (size_t)(n * k / 4));
        for (int64_t r = 0; r < n; r++)
            for (int64_t kk = 0; kk < k; kk++) {
                const int64_t kin = kk % 128, j = kin / 32, h = (kin % 32) / 8, i = kin % 8;
                const int64_t tile = (r / 16) * (k / 128) + kk / 128, slot = h * 16 + r % 16;
                const uint8_t q = codes_logical[r * k + kk];
                high[tile * 512 + slot * 8 + 2 * j] |= (uint8_t)(((q >> 4) & 1) << i);
                high[tile * 512 + slot * 8 + 2 * j + 1] |= (uint8_t)(((q >> 5) & 1) << i);
            }
        for (int64_t r = 0; r < n; r++)
            for (int64_t t = 0; t < k / 16; t++) {
                const int64_t tile = (r / 16) * (k / 128) + t / 8;
                scales_packed[tile * 128 + (r % 16) * 8 + t % 8] = (uint8_t)sc[r * (k / 16) + t];
            }
        memcpy(scales_packed + align16(n * k / 16), dsb, (size_t)(2 * (n * k / 256)));
        or_q6_k_dequantize(n, k, codes_logical, sc, dsb, w_hat);
        free(sc); free(dsb); free(lo);
        return 0;
    }
    if (fmt == OR_Q8_0) {
        uint16_t* s = (uint16_t*)malloc(2 * (n * k / 32));
        or_q8_0_quantize(n, k, w, (int8_t*)codes_logical, s);
        or_pack_codes8(n, k, (const int8_t*)codes_logical, (int8_t*)codes_packed);
        or_pack_scales(n, k, 32, 64, 2, s, scales_packed);
        or_q8_0_dequantize(n, k, (const int8_t*)codes_logical, s, w_hat);
        free(s);
        return 0;
    }
    return -1;
}

/* ------------------------------------------------------------------------ */
/* NVFP4 activations (W4A4): "mbehr90/whisper-large-v3-turbo-nvfp4", section    */
/* "What is quantized": activations are quantized per 16-value group at run    */
/* time, the weights keep their NVFP4 form, and the product is W4A4.            */
/* Reading: X[m][k] (bf16, widened exactly) is quantized exactly as an NVFP4     */
/* weight matrix is (or_nvfp4_quantize: one FP32 global scale from the absmax   */
/* of the whole X of the call, an E4M3 scale per 16 values along k, E2M1 codes).*/
/* The calibrated static activation scale of a checkpoint is not available, so  */
/* the global scale is the call's own.  Packed layout (row-major, no tiles):    */
/*   codes : byte r*k/2 + i/2 holds element i of row r, even i in the low       */
/*           nibble;                                                             */
/*   scales: byte r*(k/16) + b holds block b of row r (E4M3); the FP32 global    */
/*           scale follows at byte offset align16(m*k/16).                       */
/* x_hat[r][i] = fl(fl(e2m1 * e4m3) * g) as for weights.                         */
/* ------------------------------------------------------------------------ */
int64_t or_act_scales_bytes(int64_t m, int64_t k) { return align16(m * (k / 16)) + 4; }

void or_quantize_act_nvfp4(int64_t m, int64_t k, const uint16_t* x, uint8_t* codes_packed, uint8_t* scales_packed,
                           uint8_t* codes_logical, float* x_hat) {
    float* xf = (float*)malloc(sizeof(float) * (size_t)(m * k));
    for (int64_t i = 0; i < m * k; i++) xf[i] = or_bf16_to_f32(x[i]);
    float g;
    or_nvfp4_quantize(m, k, xf, codes_logical, scales_packed, &g);      /* scales: [m][k/16] bytes */
    memcpy(scales_packed + align16(m * (k / 16)), &g, 4);
    memset(scales_packed + m * (k / 16), 0, (size_t)(align16(m * (k / 16)) - m * (k / 16)));
    for (int64_t i = 0; i < m * k; i += 2)
        codes_packed[i / 2] = (uint8_t)((codes_logical[i] & 15) | ((codes_logical[i + 1] & 15) << 4));
    or_nvfp4_dequantize(m, k, codes_logical, scales_packed, g, x_hat);
    free(xf);
}

/* ------------------------------------------------------------------------ */
/* Matmul reference with fp32 activations (the W4A4 product of dequantized     */
/* activations and weights): y[r][n] = fl(s + b[n]), s accumulating            */
/* fl(s + fl(x[r][k] * w^[n][k])) over k ascending, as or_matmul_rows.          */
/* ------------------------------------------------------------------------ */
void or_matmul_rows_f32x(int64_t nrows, const int64_t* rows, int64_t n, int64_t k,
                         const float* x, const float* w_hat, const uint16_t* bias, float* y) {
    #pragma omp parallel for schedule(static)
    for (int64_t rr = 0; rr < nrows; rr++) {
        int64_t m = rows ? rows[rr] : rr;
        const float* xr = x + m * k;
        for (int64_t c = 0; c < n; c++) {
            const float* wr = w_hat + c * k;
            float s = 0.0f;
            for (int64_t kk = 0; kk < k; kk++) {
                float p = xr[kk] * wr[kk];
                s = s + p;
            }
            float b = bias ? or_bf16_to_f32(bias[c]) : 0.0f;
            y[rr * n + c] = s + b;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Matmul reference: y[m][n] = fl(s + b[n]) where s accumulates                 */
/* fl(s + fl(x[m][k] * w^[n][k])) over k ascending in binary32; x and b are    */
/* bf16 widened exactly (b = 0 when no bias).  `rows` selects which rows of X  */
/* to evaluate (NULL = all m rows); y is [nrows][n].                            */
/* ------------------------------------------------------------------------ */
void or_matmul_rows(int64_t nrows, const int64_t* rows, int64_t n, int64_t k,
                    const uint16_t* x, const float* w_hat, const uint16_t* bias, float* y) {
    #pragma omp parallel for schedule(static)
    for (int64_t rr = 0; rr < nrows; rr++) {
        int64_t m = rows ? rows[rr] : rr;
        float* xr = (float*)malloc(sizeof(float) * k);
        for (int64_t kk = 0; kk < k; kk++) xr[kk] = or_bf16_to_f32(x[m * k + kk]);
        for (int64_t c = 0; c < n; c++) {
            const float* wr = w_hat + c * k;
            float s = 0.0f;
            for (int64_t kk = 0; kk < k; kk++) {
                float p = xr[kk] * wr[kk];
                s = s + p;
            }
            float b = bias ? or_bf16_to_f32(bias[c]) : 0.0f;
            y[rr * n + c] = s + b;
        }
        free(xr);
    }
}
