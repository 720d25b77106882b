// quant.hip -- blockwise absmax quantizers and the fp32 dequantizer (bit-exact
// with the format definitions).  Every arithmetic step is one IEEE binary32
// operation; this file is compiled with -ffp-contract=off and uses __fmul_rn /
// __fadd_rn where a product feeds a sum, so no step is fused.
//
// Formats: NF4 with optional double-quantized absmax ("asr: add a 4-bit nf4 option
// for the Whisper engine", "What's here"); NVFP4 ("asr: add a 4-bit nvfp4 option
// for cards short of VRAM", intro; "mbehr90/whisper-large-v3-turbo-nvfp4", "What
// is quantized"); q4_0 / q8_0 ("Run quantized Whisper on the fused Metal decode
// path", "Summary"); q4_1, q5_0, q4_k and q6_k (same page, "Why the policy").  One matrix at a time, as the checkpoint streams in ("asr:
// add a 4-bit nf4 option for the Whisper engine", "Why NF4 and not the NVFP4
// snapshot Parakeet ships"); the only temporary storage is the codes buffer.
#include "wq_device.h"
#include <climits>
#include "wq_launch.h"

namespace wq {

ScaleLayout scale_layout(int fmt, bool dq, int64_t n, int64_t k) {
    ScaleLayout L{};
    L.nb = n * k / block_k(fmt);
    switch (fmt) {
    case kNF4:
        if (dq) {
            L.ng = (L.nb + 255) / 256;
            L.d_off = align16(L.nb);
            L.mu_off = L.d_off + 4 * L.ng;
            L.bytes = L.mu_off + 4;
        } else {
            L.bytes = 4 * L.nb;
        }
        break;
    case kNVFP4:
        L.g_off = align16(L.nb);
        L.bytes = L.g_off + 4;
        break;
    case kQ4_1:
        L.bytes = 4 * L.nb;      // fp16 pair (d, m) per block
        break;
    case kQ5_0:
        L.hb_off = align16(2 * L.nb);    // fp16 d per block, then one 32-bit fifth-bit word per block
        L.bytes = L.hb_off + 4 * L.nb;
        break;
    case kQ4_K:
        // (sc, m) bytes per 32-value sub-block (per tile and row: 4 sc, then 4 m), then the
        // fp16 (d, dmin) pair of each 256-value super-block, row-major
        L.kd_off = align16(2 * L.nb);
        L.bytes = L.kd_off + 4 * (n * k / 256);
        break;
    case kQ6_K:
        // an int8 scale per 16-value sub-block (per tile and row: 8), then the fp16 d of each
        // 256-value super-block, row-major
        L.kd_off = align16(L.nb);
        L.bytes = L.kd_off + 2 * (n * k / 256);
        break;
    default:
        L.bytes = 2 * L.nb;
    }
    return L;
}

// Byte offset of the 32-bit word holding k0..k0+7 (k0 % 8 == 0) of row n (4-bit).
__device__ inline int64_t word_off4(int64_t n, int64_t k0, int64_t K) {
    int64_t band = n >> 4;
    int r = (int)(n & 15);
    int64_t kt = k0 >> 7;
    int kin = (int)(k0 & 127);
    int j = kin >> 5, h = (kin & 31) >> 3;
    return (band * (K >> 7) + kt) * kTileBytes + (h * 16 + r) * 16 + j * 4;
}

// Byte offset of the 8 bytes holding k0..k0+7 of row n (q8_0).
__device__ inline int64_t word_off8(int64_t n, int64_t k0, int64_t K) {
    int64_t band = n >> 4;
    int r = (int)(n & 15);
    int64_t kt = k0 >> 6;
    int kin = (int)(k0 & 63);
    int j = kin >> 5, h = (kin & 31) >> 3;
    return (band * (K >> 6) + kt) * kTileBytes + (h * 16 + r) * 16 + j * 8;
}

// Index of the scale entry of block b (block index along K) of row n.
template <int FMT>
__device__ inline int64_t scale_slot(int64_t n, int64_t b, int64_t K) {
    constexpr int bpt = blocks_per_tile_row(FMT);
    constexpr int tk = tile_k(FMT);
    int64_t band = n >> 4;
    int r = (int)(n & 15);
    int64_t kt = b / bpt;
    int bin = (int)(b % bpt);
    return (band * (K / tk) + kt) * (16 * bpt) + r * bpt + bin;
}

// ---------------------------------------------------------------------------
// One thread per 8 consecutive K of one row ("chunk").  Blocks of 16/32/64 are
// 2/4/8 neighbouring threads, reduced with cross-lane shuffles.
// NF4 modes: 0 = codes + fp32 absmax, 1 = absmax only (logical order, to
// `scratch`), 2 = codes only (double-quant path).
// ---------------------------------------------------------------------------
template <int FMT, int MODE>
__global__ __launch_bounds__(256) void k_quant_chunks(const float* __restrict__ w, int64_t N, int64_t K,
                                                      uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                      float* __restrict__ scratch, ScaleLayout L) {
    const int64_t nchunks = N * K / 8;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool valid = c < nchunks;
    const int64_t kc8 = K / 8;
    const int64_t n = valid ? c / kc8 : 0;
    const int64_t k0 = valid ? (c % kc8) * 8 : 0;
    float v[8];
    if (valid) {
        const float4 a = *reinterpret_cast<const float4*>(w + n * K + k0);
        const float4 b = *reinterpret_cast<const float4*>(w + n * K + k0 + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = 0.0f;
    }

    if constexpr (FMT == kNF4) {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i++) a = fmaxf(a, fabsf(v[i]));
        a = fmaxf(a, __shfl_xor(a, 1, 8));
        a = fmaxf(a, __shfl_xor(a, 2, 8));
        a = fmaxf(a, __shfl_xor(a, 4, 8));
        if (!valid) return;
        const bool lead = (k0 & 63) == 0;
        if constexpr (MODE == 1) {
            if (lead) scratch[n * (K / 64) + (k0 >> 6)] = a;
            return;
        }
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            uint32_t code = 7;
            if (a != 0.0f) {
                const float x = v[i] / a;
                code = 0;
#pragma unroll
                for (int t = 0; t < 15; t++) code += (x > __uint_as_float(kNf4ThresholdBits[t])) ? 1u : 0u;
            }
            word |= code << (4 * i);
        }
        *reinterpret_cast<uint32_t*>(codes + word_off4(n, k0, K)) = word;
        if constexpr (MODE == 0) {
            if (lead) reinterpret_cast<float*>(scales)[scale_slot<kNF4>(n, k0 >> 6, K)] = a;
        }
    } else if constexpr (FMT == kNVFP4) {
        const float g = *reinterpret_cast<const float*>(scales + L.g_off);
        float ab = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i++) ab = fmaxf(ab, fabsf(v[i]));
        ab = fmaxf(ab, __shfl_xor(ab, 1, 2));
        if (!valid) return;
        uint32_t sb = 0;
        float sigma = 0.0f;
        if (g != 0.0f) {
            const float t = 6.0f * g;
            sb = e4m3_round(ab / t);
            sigma = e4m3_value(sb) * g;
        }
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            uint32_t code = signbit(v[i]) ? 8u : 0u;
            if (sigma != 0.0f) code |= e2m1_mag_code(v[i] / sigma);
            word |= code << (4 * i);
        }
        *reinterpret_cast<uint32_t*>(codes + word_off4(n, k0, K)) = word;
        if ((k0 & 15) == 0) scales[scale_slot<kNVFP4>(n, k0 >> 4, K)] = (uint8_t)sb;
    } else if constexpr (FMT == kQ8_0) {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i++) a = fmaxf(a, fabsf(v[i]));
        a = fmaxf(a, __shfl_xor(a, 1, 4));
        a = fmaxf(a, __shfl_xor(a, 2, 4));
        if (!valid) return;
        const uint16_t d = f16_sat_bits(a / 127.0f);
        const float delta = f16_value(d);
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            int q = 0;
            if (delta != 0.0f) q = (int)fminf(fmaxf(rintf(v[i] / delta), -127.0f), 127.0f);
            const uint32_t b = (uint32_t)(q & 255);
            if (i < 4) lo |= b << (8 * i); else hi |= b << (8 * (i - 4));
        }
        *reinterpret_cast<uint2*>(codes + word_off8(n, k0, K)) = make_uint2(lo, hi);
        if ((k0 & 31) == 0) reinterpret_cast<uint16_t*>(scales)[scale_slot<kQ8_0>(n, k0 >> 5, K)] = d;
    } else if constexpr (FMT == kQ4_1) {
        // block minimum and maximum, each the first such element in ascending k (so the
        // sign of a zero minimum is that of its first occurrence)
        float lo = v[0], hi = v[0];
        int lo_k = (int)(k0 & 31), hi_k = lo_k;
#pragma unroll
        for (int i = 1; i < 8; i++) {
            if (v[i] < lo) { lo = v[i]; lo_k = (int)(k0 & 31) + i; }
            if (v[i] > hi) { hi = v[i]; hi_k = (int)(k0 & 31) + i; }
        }
#pragma unroll
        for (int s = 1; s <= 2; s <<= 1) {
            const float pl = __shfl_xor(lo, s, 4), ph = __shfl_xor(hi, s, 4);
            const int plk = __shfl_xor(lo_k, s, 4), phk = __shfl_xor(hi_k, s, 4);
            if (pl < lo || (pl == lo && plk < lo_k)) { lo = pl; lo_k = plk; }
            if (ph > hi || (ph == hi && phk < hi_k)) { hi = ph; hi_k = phk; }
        }
        if (!valid) return;
        const uint16_t d = f16_sat_bits((hi - lo) / 15.0f);
        const uint16_t m = f16_sat_bits(lo);
        const float delta = f16_value(d), mu = f16_value(m);
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            uint32_t q = 0;
            if (delta != 0.0f) q = (uint32_t)fminf(fmaxf(rintf((v[i] - mu) / delta), 0.0f), 15.0f);
            word |= q << (4 * i);
        }
        *reinterpret_cast<uint32_t*>(codes + word_off4(n, k0, K)) = word;
        if ((k0 & 31) == 0)
            reinterpret_cast<uint32_t*>(scales)[scale_slot<kQ4_1>(n, k0 >> 5, K)] = (uint32_t)d | ((uint32_t)m << 16);
    } else if constexpr (FMT == kQ4_K) {
        // sub-block (4 threads) minimum and maximum, then the super-block (32 threads)
        // maxima of the sub-block scales and offsets; every lane takes part in the shuffles
        float lo = v[0], hi = v[0];
#pragma unroll
        for (int i = 1; i < 8; i++) {
            lo = fminf(lo, v[i]);
            hi = fmaxf(hi, v[i]);
        }
#pragma unroll
        for (int s = 1; s <= 2; s <<= 1) {
            lo = fminf(lo, __shfl_xor(lo, s, 4));
            hi = fmaxf(hi, __shfl_xor(hi, s, 4));
        }
        // the sign of a zero minimum or maximum cannot matter: mn is +0 unless negative and
        // the range is canonicalised to +0
        const float mn = lo < 0.0f ? lo : 0.0f;
        float range = hi - mn;
        if (!(range > 0.0f)) range = 0.0f;
        const float s_sub = range / 15.0f;
        const float o_sub = 0.0f - mn;
        float smax = s_sub, omax = o_sub;        // all >= +0, so fmaxf is exact and order-free
#pragma unroll
        for (int s = 4; s <= 16; s <<= 1) {
            smax = fmaxf(smax, __shfl_xor(smax, s, 32));
            omax = fmaxf(omax, __shfl_xor(omax, s, 32));
        }
        if (!valid) return;
        const uint16_t db = f16_sat_bits(smax / 63.0f), mb = f16_sat_bits(omax / 63.0f);
        const float d = f16_value(db), dmin = f16_value(mb);
        const float sc = d != 0.0f ? fminf(fmaxf(rintf(s_sub / d), 0.0f), 63.0f) : 0.0f;
        const float m = dmin != 0.0f ? fminf(fmaxf(rintf(o_sub / dmin), 0.0f), 63.0f) : 0.0f;
        const float S = __fmul_rn(d, sc), O = __fmul_rn(dmin, m);     // exact
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            uint32_t q = 0;
            if (S != 0.0f) q = (uint32_t)fminf(fmaxf(rintf((v[i] + O) / S), 0.0f), 15.0f);
            word |= q << (4 * i);
        }
        *reinterpret_cast<uint32_t*>(codes + word_off4(n, k0, K)) = word;
        if ((k0 & 31) == 0) {
            uint8_t* rec = scales + ((n >> 4) * (K >> 7) + (k0 >> 7)) * 128 + (n & 15) * 8;
            const int bin = (int)((k0 >> 5) & 3);
            rec[bin] = (uint8_t)sc;
            rec[4 + bin] = (uint8_t)m;
        }
        if ((k0 & 255) == 0)
            *reinterpret_cast<uint32_t*>(scales + L.kd_off + (n * (K >> 8) + (k0 >> 8)) * 4) = (uint32_t)db | ((uint32_t)mb << 16);
    } else if constexpr (FMT == kQ6_K) {
        // sub-block (2 threads): signed element of largest magnitude, first index on ties
        float best_a = -1.0f, best_v = 0.0f;
        int best_k = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const float t = fabsf(v[i]);
            if (t > best_a) { best_a = t; best_v = v[i]; best_k = (int)(k0 & 15) + i; }
        }
        {
            const float pa = __shfl_xor(best_a, 1, 2);
            const float pv = __shfl_xor(best_v, 1, 2);
            const int pk = __shfl_xor(best_k, 1, 2);
            if (pa > best_a || (pa == best_a && pk < best_k)) { best_a = pa; best_v = pv; best_k = pk; }
        }
        const float s_sub = best_v / -32.0f;
        float amax = fabsf(s_sub);               // >= +0: fmaxf is exact and order-free
#pragma unroll
        for (int s = 2; s <= 16; s <<= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 32));
        if (!valid) return;
        const uint16_t db = f16_sat_bits(amax / 127.0f);
        const float d = f16_value(db);
        const float sc = d != 0.0f ? fminf(fmaxf(rintf(s_sub / d), -127.0f), 127.0f) : 0.0f;
        const float S = __fmul_rn(d, sc);        // exact
        uint32_t word = 0, b4 = 0, b5 = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            uint32_t q = 32;
            if (S != 0.0f) q = (uint32_t)((int)fminf(fmaxf(rintf(v[i] / S), -32.0f), 31.0f) + 32);
            word |= (q & 15u) << (4 * i);
            b4 |= ((q >> 4) & 1u) << i;
            b5 |= ((q >> 5) & 1u) << i;
        }
        *reinterpret_cast<uint32_t*>(codes + word_off4(n, k0, K)) = word;
        // bits 4 and 5: plane after the n*k/2 code bytes, 8 bytes per tile slot, two per K slice
        {
            const int64_t tile = (n >> 4) * (K >> 7) + (k0 >> 7);
            const int kin = (int)(k0 & 127), j = kin >> 5, h = (kin & 31) >> 3;
            uint8_t* hp = codes + N * K / 2 + tile * 512 + (h * 16 + (n & 15)) * 8 + 2 * j;
            hp[0] = (uint8_t)b4;
            hp[1] = (uint8_t)b5;
        }
        if ((k0 & 15) == 0)
            scales[((n >> 4) * (K >> 7) + (k0 >> 7)) * 128 + (n & 15) * 8 + ((k0 & 127) >> 4)] = (uint8_t)(int8_t)sc;
        if ((k0 & 255) == 0)
            *reinterpret_cast<uint16_t*>(scales + L.kd_off + (n * (K >> 8) + (k0 >> 8)) * 2) = db;
    } else if constexpr (FMT == kQ5_0) {
        // signed element of largest magnitude; first index (ascending k) on ties
        float best_a = -1.0f, best_v = 0.0f;
        int best_k = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const float t = fabsf(v[i]);
            if (t > best_a) { best_a = t; best_v = v[i]; best_k = (int)(k0 & 31) + i; }
        }
#pragma unroll
        for (int s = 1; s <= 2; s <<= 1) {
            const float pa = __shfl_xor(best_a, s, 4);
            const float pv = __shfl_xor(best_v, s, 4);
            const int pk = __shfl_xor(best_k, s, 4);
            if (pa > best_a || (pa == best_a && pk < best_k)) { best_a = pa; best_v = pv; best_k = pk; }
        }
        if (!valid) return;
        const uint16_t d = f16_sat_bits(best_v / -16.0f);
        const float delta = f16_value(d);
        uint32_t word = 0, high = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            uint32_t q = 16;
            if (delta != 0.0f) q = (uint32_t)((int)fminf(fmaxf(rintf(v[i] / delta), -16.0f), 15.0f) + 16);
            word |= (q & 15u) << (4 * i);
            high |= (q >> 4) << i;
        }
        *reinterpret_cast<uint32_t*>(codes + word_off4(n, k0, K)) = word;
        const int64_t slot = scale_slot<kQ5_0>(n, k0 >> 5, K);
        // this thread's 8 fifth bits are byte (k0 % 32) / 8 of the block's word
        scales[L.hb_off + 4 * slot + ((k0 & 31) >> 3)] = (uint8_t)high;
        if ((k0 & 31) == 0) reinterpret_cast<uint16_t*>(scales)[slot] = d;
    } else {  // kQ4_0
        // signed element of largest magnitude; first index (ascending k) on ties
        float best_a = -1.0f, best_v = 0.0f;
        int best_k = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const float t = fabsf(v[i]);
            if (t > best_a) { best_a = t; best_v = v[i]; best_k = (int)(k0 & 31) + i; }
        }
#pragma unroll
        for (int s = 1; s <= 2; s <<= 1) {
            const float pa = __shfl_xor(best_a, s, 4);
            const float pv = __shfl_xor(best_v, s, 4);
            const int pk = __shfl_xor(best_k, s, 4);
            if (pa > best_a || (pa == best_a && pk < best_k)) { best_a = pa; best_v = pv; best_k = pk; }
        }
        if (!valid) return;
        const uint16_t d = f16_sat_bits(best_v / -8.0f);
        const float delta = f16_value(d);
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            uint32_t q = 8;
            if (delta != 0.0f) q = (uint32_t)((int)fminf(fmaxf(rintf(v[i] / delta), -8.0f), 7.0f) + 8);
            word |= q << (4 * i);
        }
        *reinterpret_cast<uint32_t*>(codes + word_off4(n, k0, K)) = word;
        if ((k0 & 31) == 0) reinterpret_cast<uint16_t*>(scales)[scale_slot<kQ4_0>(n, k0 >> 5, K)] = d;
    }
}

// Double-quant mean: the nb absmax values summed in binary64 in ascending block
// order, divided in binary64 and rounded to binary32.
//
// Fast path, exact: write every nonzero value as odd * 2^e (odd < 2^24).  With
// L = 2^min(e), every partial sum of the sequence is a multiple of L; if the whole
// sum is below 2^53 L, each partial sum is representable in binary64, so every
// ascending addition is exact and the sequential sum is the exact sum.  The
// workgroup then adds the values as integers in units of L, in any order.
// Otherwise (values spanning a very wide range), thread 0 runs the ascending chain
// of additions, with the workgroup staging the values through two LDS buffers.
constexpr int kMeanThreads = 1024;
constexpr int kMeanChunk = 4096;   // floats per LDS buffer

__device__ inline void odd_exp(float v, uint32_t& odd, int& e) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t be = u >> 23, mant = u & 0x7FFFFFu;
    const uint32_t m = be == 0 ? mant : (mant | 0x800000u);
    const int tz = __builtin_ctz(m);
    odd = m >> tz;
    e = (be == 0 ? -149 : (int)be - 150) + tz;
}

__global__ __launch_bounds__(kMeanThreads) void k_dq_mean(const float* __restrict__ a, int64_t nb,
                                                          uint8_t* __restrict__ scales, int64_t mu_off) {
    __shared__ __attribute__((aligned(16))) float buf[2][kMeanChunk];
    __shared__ int emin_s[kMeanThreads / 64];
    __shared__ unsigned long long sum_s[kMeanThreads / 64];
    __shared__ int bad_s[kMeanThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int kWaves = kMeanThreads / 64;

    // smallest exponent of a lowest set bit
    int emin = INT_MAX;
    for (int64_t i = tid; i < nb; i += kMeanThreads) {
        const float v = a[i];
        if (v != 0.0f) {
            uint32_t odd;
            int e;
            odd_exp(v, odd, e);
            emin = min(emin, e);
        }
    }
    for (int o = 32; o > 0; o >>= 1) emin = min(emin, __shfl_xor(emin, o));
    if (lane == 0) emin_s[wave] = emin;
    __syncthreads();
    emin = emin_s[0];
    for (int w = 1; w < kWaves; w++) emin = min(emin, emin_s[w]);

    // integer sum in units of 2^emin; any term or partial sum reaching 2^53 ends the fast path
    constexpr unsigned long long kLimit = 1ull << 53;
    unsigned long long acc = 0;
    int bad = 0;
    if (emin != INT_MAX) {
        for (int64_t i = tid; i < nb; i += kMeanThreads) {
            const float v = a[i];
            if (v == 0.0f) continue;
            uint32_t odd;
            int e;
            odd_exp(v, odd, e);
            const int sh = e - emin;
            if (sh >= 40) { bad = 1; break; }                 // odd << sh would pass 2^63
            acc += (unsigned long long)odd << sh;              // each term < 2^63, acc < 2^53 before
            if (acc >= kLimit) { bad = 1; break; }
        }
    }
    for (int o = 32; o > 0; o >>= 1) {
        acc += __shfl_xor(acc, o);   // < 64 * 2^53: no wrap
        bad |= __shfl_xor(bad, o);
    }
    if (lane == 0) {
        sum_s[wave] = acc;
        bad_s[wave] = bad;
    }
    __syncthreads();
    unsigned long long total = 0;
    for (int w = 0; w < kWaves; w++) {
        total += sum_s[w];
        bad |= bad_s[w];
    }
    if (!bad && total < kLimit) {
        if (tid == 0) {
            const double s = emin == INT_MAX ? 0.0 : ldexp((double)total, emin);
            *reinterpret_cast<float*>(scales + mu_off) = (float)(s / (double)nb);
        }
        return;
    }

    // ascending chain
    const int64_t nchunks = (nb + kMeanChunk - 1) / kMeanChunk;
    auto stage = [&](int64_t c) {
        float* dst = buf[c & 1];
        for (int i = tid; i < kMeanChunk; i += kMeanThreads) {
            const int64_t idx = c * kMeanChunk + i;
            dst[i] = idx < nb ? a[idx] : 0.0f;
        }
    };
    double s = 0.0;
    stage(0);
    __syncthreads();
    for (int64_t c = 0; c < nchunks; c++) {
        if (c + 1 < nchunks) stage(c + 1);
        if (tid == 0) {
            const float* src = buf[c & 1];
            const int cnt = (int)std::min<int64_t>(kMeanChunk, nb - c * kMeanChunk);
            int i = 0;
            for (; i + 4 <= cnt; i += 4) {
                const float4 t = *reinterpret_cast<const float4*>(src + i);
                s += (double)t.x;
                s += (double)t.y;
                s += (double)t.z;
                s += (double)t.w;
            }
            for (; i < cnt; i++) s += (double)src[i];
        }
        __syncthreads();   // chunk c + 1 is staged; buffer c & 1 is free for chunk c + 2
    }
    if (tid == 0) *reinterpret_cast<float*>(scales + mu_off) = (float)(s / (double)nb);
}

// Double-quant groups: one wave per 256 consecutive blocks (logical order).
__global__ __launch_bounds__(64) void k_dq_groups(const float* __restrict__ a, int64_t nb, int64_t K,
                                                  uint8_t* __restrict__ scales, ScaleLayout L) {
    const int lane = threadIdx.x;
    const int64_t g = blockIdx.x;
    const float mu = *reinterpret_cast<const float*>(scales + L.mu_off);
    float ap[4];
    float m = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const int64_t i = g * 256 + r * 64 + lane;
        ap[r] = (i < nb) ? a[i] - mu : 0.0f;
        m = fmaxf(m, fabsf(ap[r]));
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
    const float d = m / 127.0f;
    const int64_t nbk = K / 64;
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const int64_t i = g * 256 + r * 64 + lane;
        if (i >= nb) continue;
        int q = 0;
        if (d != 0.0f) q = (int)fminf(fmaxf(rintf(ap[r] / d), -127.0f), 127.0f);
        scales[scale_slot<kNF4>(i / nbk, i % nbk, K)] = (uint8_t)(int8_t)q;
    }
    if (lane == 0) reinterpret_cast<float*>(scales + L.d_off)[g] = d;
}

// Matrix absmax for NVFP4: per-workgroup partial maxima, then one workgroup
// combines them and writes the global scale g = A / 2688.
__global__ __launch_bounds__(256) void k_absmax_partial(const float* __restrict__ w, int64_t count, float* __restrict__ partial) {
    __shared__ float red[4];
    float m = 0.0f;
    const int64_t n4 = count / 4;
    const float4* w4 = reinterpret_cast<const float4*>(w);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        const float4 t = w4[i];
        m = fmaxf(m, fmaxf(fmaxf(fabsf(t.x), fabsf(t.y)), fmaxf(fabsf(t.z), fabsf(t.w))));
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__global__ __launch_bounds__(64) void k_absmax_final(const float* __restrict__ partial, int np, uint8_t* __restrict__ scales, int64_t g_off) {
    float m = 0.0f;
    for (int i = threadIdx.x; i < np; i += 64) m = fmaxf(m, partial[i]);
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
    if (threadIdx.x == 0) *reinterpret_cast<float*>(scales + g_off) = m / 2688.0f;
}

// ---------------------------------------------------------------------------
// Dequantize: one thread per chunk of 8, fp32 out in logical row-major order.
// ---------------------------------------------------------------------------
template <int FMT, bool DQ>
__global__ __launch_bounds__(256) void k_dequant_chunks(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                        int64_t N, int64_t K, float* __restrict__ out, ScaleLayout L) {
    const int64_t nchunks = N * K / 8;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= nchunks) return;
    const int64_t kc8 = K / 8;
    const int64_t n = c / kc8;
    const int64_t k0 = (c % kc8) * 8;
    float o[8];
    if constexpr (FMT == kQ8_0) {
        const uint2 u = *reinterpret_cast<const uint2*>(codes + word_off8(n, k0, K));
        const float delta = f16_value(reinterpret_cast<const uint16_t*>(scales)[scale_slot<kQ8_0>(n, k0 >> 5, K)]);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t wv = i < 4 ? u.x : u.y;
            const int q = (int)(int8_t)(uint8_t)(wv >> (8 * (i & 3)));
            o[i] = __fmul_rn((float)q, delta);
        }
    } else {
        const uint32_t word = *reinterpret_cast<const uint32_t*>(codes + word_off4(n, k0, K));
        if constexpr (FMT == kNF4) {
            float a;
            const int64_t b = k0 >> 6;
            if constexpr (DQ) {
                const int q = (int)(int8_t)scales[scale_slot<kNF4>(n, b, K)];
                const int64_t g = (n * (K / 64) + b) / 256;
                const float d = reinterpret_cast<const float*>(scales + L.d_off)[g];
                const float mu = *reinterpret_cast<const float*>(scales + L.mu_off);
                a = __fadd_rn(__fmul_rn((float)q, d), mu);
            } else {
                a = reinterpret_cast<const float*>(scales)[scale_slot<kNF4>(n, b, K)];
            }
#pragma unroll
            for (int i = 0; i < 8; i++) o[i] = __fmul_rn(nf4_level(word >> (4 * i)), a);
        } else if constexpr (FMT == kNVFP4) {
            const float s = e4m3_value(scales[scale_slot<kNVFP4>(n, k0 >> 4, K)]);
            const float g = *reinterpret_cast<const float*>(scales + L.g_off);
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const uint32_t cd = (word >> (4 * i)) & 15u;
                float v = e2m1_mag_value(cd & 7u);
                if (cd & 8u) v = -v;
                o[i] = __fmul_rn(__fmul_rn(v, s), g);
            }
        } else if constexpr (FMT == kQ4_1) {
            const uint32_t dm = reinterpret_cast<const uint32_t*>(scales)[scale_slot<kQ4_1>(n, k0 >> 5, K)];
            const float delta = f16_value((uint16_t)(dm & 0xFFFFu)), mu = f16_value((uint16_t)(dm >> 16));
            // q * delta is exact (4 + 11 significant bits): one rounding, in the add
#pragma unroll
            for (int i = 0; i < 8; i++) o[i] = __fadd_rn(__fmul_rn((float)((word >> (4 * i)) & 15u), delta), mu);
        } else if constexpr (FMT == kQ6_K) {
            const int64_t tile = (n >> 4) * (K >> 7) + (k0 >> 7);
            const int kin = (int)(k0 & 127), j = kin >> 5, h = (kin & 31) >> 3;
            const uint8_t* hp = codes + N * K / 2 + tile * 512 + (h * 16 + (n & 15)) * 8 + 2 * j;
            const uint32_t b4 = hp[0], b5 = hp[1];
            const float d = f16_value(*reinterpret_cast<const uint16_t*>(scales + L.kd_off + (n * (K >> 8) + (k0 >> 8)) * 2));
            const float S = __fmul_rn(d, (float)(int8_t)scales[tile * 128 + (n & 15) * 8 + (kin >> 4)]);
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int q = (int)(((word >> (4 * i)) & 15u) | (((b4 >> i) & 1u) << 4) | (((b5 >> i) & 1u) << 5));
                o[i] = __fmul_rn(S, (float)(q - 32));
            }
        } else if constexpr (FMT == kQ4_K) {
            const uint8_t* rec = scales + ((n >> 4) * (K >> 7) + (k0 >> 7)) * 128 + (n & 15) * 8;
            const int bin = (int)((k0 >> 5) & 3);
            const uint32_t dm = *reinterpret_cast<const uint32_t*>(scales + L.kd_off + (n * (K >> 8) + (k0 >> 8)) * 4);
            const float S = __fmul_rn(f16_value((uint16_t)(dm & 0xFFFFu)), (float)rec[bin]);
            const float O = __fmul_rn(f16_value((uint16_t)(dm >> 16)), (float)rec[4 + bin]);
            // S * q is exact (21 significant bits): one rounding, in the subtraction
#pragma unroll
            for (int i = 0; i < 8; i++) o[i] = __fsub_rn(__fmul_rn(S, (float)((word >> (4 * i)) & 15u)), O);
        } else if constexpr (FMT == kQ5_0) {
            const int64_t slot = scale_slot<kQ5_0>(n, k0 >> 5, K);
            const float delta = f16_value(reinterpret_cast<const uint16_t*>(scales)[slot]);
            const uint32_t high = scales[L.hb_off + 4 * slot + ((k0 & 31) >> 3)];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int q = (int)(((word >> (4 * i)) & 15u) | (((high >> i) & 1u) << 4));
                o[i] = __fmul_rn((float)(q - 16), delta);
            }
        } else {  // kQ4_0
            const float delta = f16_value(reinterpret_cast<const uint16_t*>(scales)[scale_slot<kQ4_0>(n, k0 >> 5, K)]);
#pragma unroll
            for (int i = 0; i < 8; i++) o[i] = __fmul_rn((float)((int)((word >> (4 * i)) & 15u) - 8), delta);
        }
    }
    float4* dst = reinterpret_cast<float4*>(out + n * K + k0);
    dst[0] = make_float4(o[0], o[1], o[2], o[3]);
    dst[1] = make_float4(o[4], o[5], o[6], o[7]);
}

static inline unsigned grid_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

hipError_t launch_quantize(int fmt, bool dq, int64_t n, int64_t k, const float* w, uint8_t* codes,
                           uint8_t* scales, hipStream_t s) {
    const ScaleLayout L = scale_layout(fmt, dq, n, k);
    const int64_t chunks = n * k / 8;
    const unsigned grid = grid_for(chunks);
    switch (fmt) {
    case kNF4:
        if (!dq) {
            hipLaunchKernelGGL((k_quant_chunks<kNF4, 0>), dim3(grid), dim3(256), 0, s, w, n, k, codes, scales, nullptr, L);
        } else {
            float* scratch = reinterpret_cast<float*>(codes);   // nb floats <= n*k/2 bytes
            hipLaunchKernelGGL((k_quant_chunks<kNF4, 1>), dim3(grid), dim3(256), 0, s, w, n, k, codes, scales, scratch, L);
            hipLaunchKernelGGL(k_dq_mean, dim3(1), dim3(kMeanThreads), 0, s, scratch, L.nb, scales, L.mu_off);
            hipLaunchKernelGGL(k_dq_groups, dim3((unsigned)L.ng), dim3(64), 0, s, scratch, L.nb, k, scales, L);
            hipLaunchKernelGGL((k_quant_chunks<kNF4, 2>), dim3(grid), dim3(256), 0, s, w, n, k, codes, scales, nullptr, L);
        }
        break;
    case kNVFP4: {
        float* partial = reinterpret_cast<float*>(codes);      // <= 256 floats <= n*k/2 bytes
        const int np = (int)std::min<int64_t>(256, std::max<int64_t>(1, (n * k / 4 + 255) / 256));
        hipLaunchKernelGGL(k_absmax_partial, dim3(np), dim3(256), 0, s, w, n * k, partial);
        hipLaunchKernelGGL(k_absmax_final, dim3(1), dim3(64), 0, s, partial, np, scales, L.g_off);
        hipLaunchKernelGGL((k_quant_chunks<kNVFP4, 0>), dim3(grid), dim3(256), 0, s, w, n, k, codes, scales, nullptr, L);
        break;
    }
    case kQ4_0:
        hipLaunchKernelGGL((k_quant_chunks<kQ4_0, 0>), dim3(grid), dim3(256), 0, s, w, n, k, codes, scales, nullptr, L);
        break;
    case kQ4_1:
        hipLaunchKernelGGL((k_quant_chunks<kQ4_1, 0>), dim3(grid), dim3(256), 0, s, w, n, k, codes, scales, nullptr, L);
        break;
    case kQ5_0:
        hipLaunchKernelGGL((k_quant_chunks<kQ5_0, 0>), dim3(grid), dim3(256), 0, s, w, n, k, codes, scales, nullptr, L);
        break;
    case kQ4_K:
        hipLaunchKernelGGL((k_quant_chunks<kQ4_K, 0>), dim3(grid), dim3(256), 0, s, w, n, k, codes, scales, nullptr, L);
        break;
    case kQ6_K:
        hipLaunchKernelGGL((k_quant_chunks<kQ6_K, 0>), dim3(grid), dim3(256), 0, s, w, n, k, codes, scales, nullptr, L);
        break;
    case kQ8_0:
        hipLaunchKernelGGL((k_quant_chunks<kQ8_0, 0>), dim3(grid), dim3(256), 0, s, w, n, k, codes, scales, nullptr, L);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_dequantize(int fmt, bool dq, int64_t n, int64_t k, const uint8_t* codes, const uint8_t* scales,
                             float* out, hipStream_t s) {
    const ScaleLayout L = scale_layout(fmt, dq, n, k);
    const unsigned grid = grid_for(n * k / 8);
    switch (fmt) {
    case kNF4:
        if (dq) hipLaunchKernelGGL((k_dequant_chunks<kNF4, true>), dim3(grid), dim3(256), 0, s, codes, scales, n, k, out, L);
        else hipLaunchKernelGGL((k_dequant_chunks<kNF4, false>), dim3(grid), dim3(256), 0, s, codes, scales, n, k, out, L);
        break;
    case kNVFP4:
        hipLaunchKernelGGL((k_dequant_chunks<kNVFP4, false>), dim3(grid), dim3(256), 0, s, codes, scales, n, k, out, L);
        break;
    case kQ4_0:
        hipLaunchKernelGGL((k_dequant_chunks<kQ4_0, false>), dim3(grid), dim3(256), 0, s, codes, scales, n, k, out, L);
        break;
    case kQ4_1:
        hipLaunchKernelGGL((k_dequant_chunks<kQ4_1, false>), dim3(grid), dim3(256), 0, s, codes, scales, n, k, out, L);
        break;
    case kQ5_0:
        hipLaunchKernelGGL((k_dequant_chunks<kQ5_0, false>), dim3(grid), dim3(256), 0, s, codes, scales, n, k, out, L);
        break;
    case kQ4_K:
        hipLaunchKernelGGL((k_dequant_chunks<kQ4_K, false>), dim3(grid), dim3(256), 0, s, codes, scales, n, k, out, L);
        break;
    case kQ6_K:
        hipLaunchKernelGGL((k_dequant_chunks<kQ6_K, false>), dim3(grid), dim3(256), 0, s, codes, scales, n, k, out, L);
        break;
    case kQ8_0:
        hipLaunchKernelGGL((k_dequant_chunks<kQ8_0, false>), dim3(grid), dim3(256), 0, s, codes, scales, n, k, out, L);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace wq
