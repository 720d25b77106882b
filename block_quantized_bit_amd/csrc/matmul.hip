// matmul.hip -- Y = X * W^T + b with W kept packed and dequantized inside the
// kernel (the fused dequant-matmul: "asr: add a 4-bit nf4 option for the Whisper
// engine", "Why NF4 and not the NVFP4 snapshot Parakeet ships"; W4A16 GEMM:
// "mbehr90/whisper-large-v3-turbo-nvfp4", "What is quantized").
//
// Both kernels use the gfx950 16x16x32 bf16 MFMA.  The packed layout puts, in
// each 16-byte slot of a 16x128 weight tile, exactly the 8 consecutive-k values a
// lane supplies as its B operand for each of the tile's four 32-wide K slices,
// so a wave turns one 1 KiB tile load (64 lanes x 16 B, fully coalesced) into
// four MFMA B operands without any data exchange.
//
// 4-bit codes are decoded through byte-indexed tables in LDS (one entry per code
// byte, i.e. two values per lookup), replicated per lane so that concurrent
// lookups of different bytes hit different banks; the LDS address is built with
// one v_perm_b32.  The GEMV table holds bf16 values (fed straight to the MFMA),
// the GEMM table fp32 values (scaled exactly, then rounded once to bf16).
//
// GEMV (m <= 16, decode): B = raw code values (NF4 level, q4_0 q-8, q8_0 q),
//   the per-block scale is applied to the MFMA partial sum of each block; for
//   NVFP4 (16-value blocks, two per 32-K slice) B = e2m1*scale (exact in bf16).
//   Split-K over the waves of a workgroup (reduced in LDS) and, with a
//   workspace, across workgroups (last-arriving workgroup reduces).
// GEMM (m >= 17, encoder): each wave dequantizes 64 columns x 128 K of W per
//   step to bf16(w^) -- w^ computed exactly as the format defines it, then one
//   round-to-nearest-even -- straight into MFMA B registers; the X tile
//   (128 x 128 bf16) is shared through LDS.
#include "wq_device.h"
#include "wq_launch.h"

#include <algorithm>

namespace wq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLutWords = 256 * 64;   // 256 byte values x 64 lane slots

struct KArgs {
    const uint16_t* x;
    int64_t ldx;
    int m;
    int64_t n, k;
    const uint8_t* codes;
    const uint8_t* scales;
    const uint16_t* bias;
    OutSplit out;
    ScaleLayout L;
    int ksplit;          // K pieces per output tile
    int64_t kt_per;      // K tiles (of tile_k) per piece
    float* partial;      // [ksplit][m][n] when ksplit > 1
    uint32_t* counters;  // one per output tile when ksplit > 1
    int64_t tiles_m, tiles_n;
};

// bf16 image of a 4-bit code's value (before any block scale).
template <int FMT>
__device__ inline uint32_t code_bf16(uint32_t c) {
    if constexpr (FMT == kNF4) {
        return kNf4LevelBf16[c & 15u];
    } else if constexpr (FMT == kQ4_0) {
        return __float_as_uint((float)((int)(c & 15u) - 8)) >> 16;          // exact
    } else {  // NVFP4
        float v = e2m1_mag_value(c & 7u);
        if (c & 8u) v = -v;
        return __float_as_uint(v) >> 16;                                       // exact
    }
}

// Fill the replicated byte table: word (e * 64 + slot) = bf16(lo nibble) | bf16(hi nibble) << 16.
template <int FMT>
__device__ inline void build_lut(uint32_t* lut) {
    const int t = threadIdx.x;             // 256 threads
    const int slot4 = (t & 15) * 4;
#pragma unroll 4
    for (int e0 = 0; e0 < 256; e0 += 16) {
        const int e = e0 + (t >> 4);
        const uint32_t v = code_bf16<FMT>(e & 15) | (code_bf16<FMT>(e >> 4) << 16);
        *reinterpret_cast<uint4*>(lut + e * 64 + slot4) = make_uint4(v, v, v, v);
    }
}

// Two bf16 code values for byte p of `word`, from lane `lane4/4`'s copy of the table.
__device__ inline uint32_t lut_pair(const uint32_t* lut, uint32_t lane4, uint32_t word, int p) {
    // address = (byte_p << 8) | (lane << 2): byte 0 from lane4, byte 1 from word's byte p
    const uint32_t addr = __builtin_amdgcn_perm(lane4, word, 0x0C0C0004u | ((uint32_t)p << 8));
    return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(lut) + addr);
}

// fp32 value of a 4-bit code (before any block scale); exact for every format.
template <int FMT>
__device__ inline float code_f32(uint32_t c) {
    if constexpr (FMT == kNF4) {
        return nf4_level(c);
    } else if constexpr (FMT == kQ4_0) {
        return (float)((int)(c & 15u) - 8);
    } else {  // NVFP4
        const float v = e2m1_mag_value(c & 7u);
        return (c & 8u) ? -v : v;
    }
}

// Replicated byte -> (fp32 lo-nibble value, fp32 hi-nibble value) table with 32
// lane copies: pair (e, slot) at byte offset e * 256 + slot * 8.
template <int FMT>
__device__ inline void build_lut_f32(uint32_t* lut) {
    const int t = threadIdx.x;             // 256 threads
    const int slot = (t & 15) * 2;
#pragma unroll 4
    for (int e0 = 0; e0 < 256; e0 += 16) {
        const int e = e0 + (t >> 4);
        const uint32_t lo = __float_as_uint(code_f32<FMT>(e & 15)), hi = __float_as_uint(code_f32<FMT>(e >> 4));
        *reinterpret_cast<uint4*>(lut + e * 64 + slot * 2) = make_uint4(lo, hi, lo, hi);
    }
}

// The two fp32 code values for byte p of `word`, from copy (lane & 31) of the table.
__device__ inline float2 lut_pair_f32(const uint32_t* lut, uint32_t lane8, uint32_t word, int p) {
    const uint32_t addr = __builtin_amdgcn_perm(lane8, word, 0x0C0C0004u | ((uint32_t)p << 8));
    return *reinterpret_cast<const float2*>(reinterpret_cast<const char*>(lut) + addr);
}

__device__ inline float lo_f(uint32_t pr) { return __uint_as_float(pr << 16); }
__device__ inline float hi_f(uint32_t pr) { return __uint_as_float(pr & 0xFFFF0000u); }

__device__ inline uint32_t pack_bf16_rne(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ inline f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Output: scatter one value to its split, add bias, convert.
// ---------------------------------------------------------------------------
__device__ inline void store_out(const OutSplit& o, int64_t m, int64_t n, float v) {
    int s = 0;
    int64_t c0 = 0;
    if (n >= o.end[0]) {
        s = 1;
        c0 = o.end[0];
        if (n >= o.end[1]) { s = 2; c0 = o.end[1]; }
    }
    const int64_t off = m * o.ldy[s] + (n - c0);
    if (o.f32) reinterpret_cast<float*>(o.y[s])[off] = v;
    else reinterpret_cast<uint16_t*>(o.y[s])[off] = bf16_rne(v);
}

__device__ inline float finish(const KArgs& a, int64_t n, float v, float g) {
    float r = v * g;
    if (a.bias) r = r + bf16_value(a.bias[n]);
    return r;
}

// ===========================================================================
// GEMV, m <= 16.  Workgroup = 4 waves on one 16-row band and one K piece; wave w
// takes tiles w, w+4, ... of the piece.  Lane l owns row (l & 15) of the band as
// B operand and row (l & 15) of X as A operand; the 16x16 result tile has
// D[4*(l>>4)+i][l&15] in lane l.
// ===========================================================================
template <int FMT, bool DQ, int NI>
__global__ __launch_bounds__(256, 2) void k_gemv(KArgs a) {
    __shared__ uint32_t lut[(FMT == kQ8_0) ? 1 : kLutWords];
    __shared__ f32x4 red[4][64];
    __shared__ int s_last;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15;
    const int h = lane >> 4;
    const uint32_t lane4 = (uint32_t)lane << 2;
    const int M = a.m;
    const int64_t K = a.k;
    constexpr int TK = tile_k(FMT);
    const int64_t KT = K / TK;
    const int64_t nbands = a.n / 16;
    const int64_t items = nbands * a.ksplit;

    if constexpr (FMT != kQ8_0) build_lut<FMT>(lut);
    __syncthreads();

    float g = 1.0f, mu = 0.0f;
    if constexpr (FMT == kNVFP4) g = *reinterpret_cast<const float*>(a.scales + a.L.g_off);
    if constexpr (FMT == kNF4 && DQ) mu = *reinterpret_cast<const float*>(a.scales + a.L.mu_off);

    const bool mrow = r < M;
    const uint16_t* xrow = a.x + (int64_t)(mrow ? r : 0) * a.ldx + h * 8;

    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const int64_t band = item / a.ksplit;
        const int ks = (int)(item % a.ksplit);
        const int64_t kt0 = ks * a.kt_per;
        const int64_t kt1 = std::min<int64_t>(KT, kt0 + a.kt_per);
        const int64_t row = band * 16 + r;

        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int64_t kt = kt0 + wave; kt < kt1; kt += 4) {
            const int64_t tile = band * KT + kt;
            const uint4 u = *reinterpret_cast<const uint4*>(a.codes + tile * kTileBytes + lane * 16);
            const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
            // A operands: 8 consecutive bf16 of X row r at k = kt*TK + 32j + 8h
            u32x4 A[TK / 32];
#pragma unroll
            for (int j = 0; j < TK / 32; j++) {
                if (mrow) {
                    const uint4 t = *reinterpret_cast<const uint4*>(xrow + kt * TK + 32 * j);
                    A[j] = u32x4{t.x, t.y, t.z, t.w};
                } else {
                    A[j] = u32x4{0u, 0u, 0u, 0u};
                }
            }
            if constexpr (FMT == kNF4) {
                float s0, s1;
                if constexpr (DQ) {
                    const uint16_t qq = *reinterpret_cast<const uint16_t*>(a.scales + tile * 32 + r * 2);
                    const int64_t b0 = row * (K / 64) + kt * 2;
                    const float* dt = reinterpret_cast<const float*>(a.scales + a.L.d_off);
                    s0 = __fadd_rn(__fmul_rn((float)(int8_t)(qq & 255), dt[b0 >> 8]), mu);
                    s1 = __fadd_rn(__fmul_rn((float)(int8_t)(qq >> 8), dt[(b0 + 1) >> 8]), mu);
                } else {
                    const float2 sc = *reinterpret_cast<const float2*>(a.scales + (tile * 32 + r * 2) * 4);
                    s0 = sc.x;
                    s1 = sc.y;
                }
#pragma unroll
                for (int kb = 0; kb < 2; kb++) {
                    f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int jj = 0; jj < 2; jj++) {
                        const int j = kb * 2 + jj;
                        u32x4 B;
#pragma unroll
                        for (int p = 0; p < 4; p++) B[p] = lut_pair(lut, lane4, uw[j], p);
                        t = mfma(A[j], B, t);
                    }
                    const float s = kb ? s1 : s0;
#pragma unroll
                    for (int i = 0; i < NI; i++) acc[i] += t[i] * s;
                }
            } else if constexpr (FMT == kQ4_0) {
                const uint2 sc = *reinterpret_cast<const uint2*>(a.scales + (tile * 64 + r * 4) * 2);
                const uint32_t sw[2] = {sc.x, sc.y};
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    u32x4 B;
#pragma unroll
                    for (int p = 0; p < 4; p++) B[p] = lut_pair(lut, lane4, uw[j], p);
                    const f32x4 t = mfma(A[j], B, f32x4{0.f, 0.f, 0.f, 0.f});
                    const float s = f16_value((uint16_t)(sw[j >> 1] >> (16 * (j & 1))));
#pragma unroll
                    for (int i = 0; i < NI; i++) acc[i] += t[i] * s;
                }
            } else if constexpr (FMT == kNVFP4) {
                const uint2 sc = *reinterpret_cast<const uint2*>(a.scales + tile * 128 + r * 8);
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int blk = 2 * j + (h >> 1);
                    const uint32_t sb = ((blk < 4 ? sc.x : sc.y) >> (8 * (blk & 3))) & 255u;
                    const float s = e4m3_value(sb);
                    u32x4 B;
#pragma unroll
                    for (int p = 0; p < 4; p++) {
                        const uint32_t pr = lut_pair(lut, lane4, uw[j], p);
                        const float lo = lo_f(pr) * s, hi = hi_f(pr) * s;                 // exact
                        B[p] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
                    }
                    acc = mfma(A[j], B, acc);
                }
            } else {  // kQ8_0: 16 x 64 tile, slices j = 0, 1
                const uint32_t sc = *reinterpret_cast<const uint32_t*>(a.scales + (tile * 32 + r * 2) * 2);
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    u32x4 B;
#pragma unroll
                    for (int p = 0; p < 4; p++) {
                        const uint32_t wv = uw[2 * j + (p >> 1)];
                        const int sh = 16 * (p & 1);
                        const float f0 = (float)(int)(int8_t)(wv >> sh);
                        const float f1 = (float)(int)(int8_t)(wv >> (sh + 8));
                        B[p] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
                    }
                    const f32x4 t = mfma(A[j], B, f32x4{0.f, 0.f, 0.f, 0.f});
                    const float s = f16_value((uint16_t)(sc >> (16 * j)));
#pragma unroll
                    for (int i = 0; i < NI; i++) acc[i] += t[i] * s;
                }
            }
        }

        // cross-wave reduction in a fixed order
        red[wave][lane] = acc;
        __syncthreads();
        f32x4 sum = {0.f, 0.f, 0.f, 0.f};
        if (wave == 0) {
            sum = red[0][lane];
#pragma unroll
            for (int w = 1; w < 4; w++) sum += red[w][lane];
        }
        const int64_t col = band * 16 + r;
        if (a.ksplit == 1) {
            if (wave == 0) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int mm = 4 * h + i;
                    if (mm < M) store_out(a.out, mm, col, finish(a, col, sum[i], g));
                }
            }
        } else {
            if (wave == 0) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int mm = 4 * h + i;
                    if (mm < M) a.partial[((int64_t)ks * M + mm) * a.n + col] = sum[i];
                }
                __threadfence();
                if (lane == 0) {
                    const uint32_t old = atomicAdd(&a.counters[band], 1u);
                    s_last = (old == (uint32_t)(a.ksplit - 1));
                }
            }
            __syncthreads();
            if (s_last && wave == 0) {
                __threadfence();
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int mm = 4 * h + i;
                    if (mm < M) {
                        float v = 0.0f;
                        for (int s2 = 0; s2 < a.ksplit; s2++)
                            v += __builtin_nontemporal_load(&a.partial[((int64_t)s2 * M + mm) * a.n + col]);
                        store_out(a.out, mm, col, finish(a, col, v, g));
                    }
                }
                if (lane == 0) atomicExch(&a.counters[band], 0u);
            }
        }
        __syncthreads();   // red[] and s_last are reused by the next item
    }
}

// ===========================================================================
// GEMM, m >= 17.  Workgroup tile 128 (M) x 256 (N), K step 128; wave w owns
// columns [64w, 64w+64) (4 bands) for all 128 rows: 8 x 4 MFMA tiles of 16x16.
// ===========================================================================
constexpr int BM = 128, BN = 256, BK = 128;
constexpr int XS_STRIDE = BK + 8;          // bf16 elements per LDS row (272 B: conflict-free A reads)

template <int FMT, bool DQ>
__global__ __launch_bounds__(256, 1) void k_gemm(KArgs a) {
    __shared__ uint32_t lut[(FMT == kQ8_0) ? 1 : kLutWords];
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * XS_STRIDE];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r = lane & 15;
    const int h = lane >> 4;
    const uint32_t lane4 = (uint32_t)lane << 2;
    const int64_t M = a.m, N = a.n, K = a.k;
    constexpr int TK = tile_k(FMT);
    const int64_t KT = K / TK;
    const int64_t nsteps_total = K / BK;

    // XCD-aware item order: consecutive items (same N tile, neighbouring M tiles
    // and K pieces) run on the same XCD and share its L2.
    const int64_t items = a.tiles_m * a.tiles_n * a.ksplit;
    const int64_t grid = gridDim.x;
    const int64_t per_xcd = grid / 8;
    const int64_t item = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (item >= items) return;
    const int ks = (int)(item % a.ksplit);
    const int64_t tmn = item / a.ksplit;
    const int64_t tm = tmn % a.tiles_m;
    const int64_t tn = tmn / a.tiles_m;
    const int64_t m0 = tm * BM, n0 = tn * BN;
    const int64_t s0 = ks * a.kt_per, s1 = std::min<int64_t>(nsteps_total, s0 + a.kt_per);  // in BK steps

    if constexpr (FMT != kQ8_0) build_lut_f32<FMT>(lut);
    const uint32_t lane8 = (uint32_t)(lane & 31) << 3;

    float g = 1.0f, mu = 0.0f;
    if constexpr (FMT == kNVFP4) g = *reinterpret_cast<const float*>(a.scales + a.L.g_off);
    if constexpr (FMT == kNF4 && DQ) mu = *reinterpret_cast<const float*>(a.scales + a.L.mu_off);

    // X tile loader: thread t copies rows (t>>4) + 16*i, 8 columns at (t & 15) * 8
    const int xr0 = tid >> 4, xc = (tid & 15) * 8;
    uint4 xreg[8];
    auto load_x = [&](int64_t step) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int64_t mm = m0 + xr0 + 16 * i;
            if (mm < M) xreg[i] = *reinterpret_cast<const uint4*>(a.x + mm * a.ldx + step * BK + xc);
            else xreg[i] = make_uint4(0, 0, 0, 0);
        }
    };
    auto store_x = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 8; i++)
            *reinterpret_cast<uint4*>(&xs[buf][(xr0 + 16 * i) * XS_STRIDE + xc]) = xreg[i];
    };

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t band0 = n0 / 16 + wave * 4;
    const int64_t nbands = N / 16;

    if (s0 < s1) {
        load_x(s0);
        store_x(0);
    }
    __syncthreads();

    for (int64_t st = s0; st < s1; st++) {
        const int buf = (int)((st - s0) & 1);
        const bool more = st + 1 < s1;
        if (more) load_x(st + 1);

        // ---- dequantize this wave's 4 bands x 128 K into B operands, then MFMA ----
#pragma unroll
        for (int nf = 0; nf < 4; nf++) {
            const int64_t band = band0 + nf;
            const bool bval = band < nbands;
            const int64_t rowW = band * 16 + r;
            u32x4 Bq[4];   // 4 K-slices of 32
            if (!bval) {
#pragma unroll
                for (int j = 0; j < 4; j++) Bq[j] = u32x4{0u, 0u, 0u, 0u};
            } else if constexpr (FMT == kQ8_0) {
#pragma unroll
                for (int half = 0; half < 2; half++) {
                    const int64_t tile = band * KT + st * 2 + half;
                    const uint4 u = *reinterpret_cast<const uint4*>(a.codes + tile * kTileBytes + lane * 16);
                    const uint32_t sc = *reinterpret_cast<const uint32_t*>(a.scales + (tile * 32 + r * 2) * 2);
                    const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int j = 0; j < 2; j++) {
                        const float d = f16_value((uint16_t)(sc >> (16 * j)));
                        const float d128 = -128.0f * d;
#pragma unroll
                        for (int p = 0; p < 4; p++) {
                            const uint32_t wv = uw[2 * j + (p >> 1)] ^ 0x80808080u;   // q + 128
                            const int sh = 16 * (p & 1);
                            const float f0 = (float)((wv >> sh) & 255u);
                            const float f1 = (float)((wv >> (sh + 8)) & 255u);
                            // (q+128)*d - 128*d == q*d exactly (fits 19 bits); one rounding to bf16
                            Bq[2 * half + j][p] = pack_bf16_rne(__builtin_fmaf(f0, d, d128), __builtin_fmaf(f1, d, d128));
                        }
                    }
                }
            } else {
                const int64_t tile = band * KT + st;
                const uint4 u = *reinterpret_cast<const uint4*>(a.codes + tile * kTileBytes + lane * 16);
                const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
                float sj[4];
                if constexpr (FMT == kNF4) {
                    float s0_, s1_;
                    if constexpr (DQ) {
                        const uint16_t qq = *reinterpret_cast<const uint16_t*>(a.scales + tile * 32 + r * 2);
                        const int64_t b0 = rowW * (K / 64) + st * 2;
                        const float* dt = reinterpret_cast<const float*>(a.scales + a.L.d_off);
                        s0_ = __fadd_rn(__fmul_rn((float)(int8_t)(qq & 255), dt[b0 >> 8]), mu);
                        s1_ = __fadd_rn(__fmul_rn((float)(int8_t)(qq >> 8), dt[(b0 + 1) >> 8]), mu);
                    } else {
                        const float2 sc = *reinterpret_cast<const float2*>(a.scales + (tile * 32 + r * 2) * 4);
                        s0_ = sc.x;
                        s1_ = sc.y;
                    }
                    sj[0] = sj[1] = s0_;
                    sj[2] = sj[3] = s1_;
                } else if constexpr (FMT == kQ4_0) {
                    const uint2 sc = *reinterpret_cast<const uint2*>(a.scales + (tile * 64 + r * 4) * 2);
                    sj[0] = f16_value((uint16_t)sc.x);
                    sj[1] = f16_value((uint16_t)(sc.x >> 16));
                    sj[2] = f16_value((uint16_t)sc.y);
                    sj[3] = f16_value((uint16_t)(sc.y >> 16));
                } else {  // NVFP4
                    const uint2 sc = *reinterpret_cast<const uint2*>(a.scales + tile * 128 + r * 8);
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const int blk = 2 * j + (h >> 1);
                        sj[j] = e4m3_value(((blk < 4 ? sc.x : sc.y) >> (8 * (blk & 3))) & 255u);
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; j++) {
#pragma unroll
                    for (int p = 0; p < 4; p++) {
                        // w^ = fl(code * scale) exactly as the format defines it, then one RNE to bf16
                        const float2 pr = lut_pair_f32(lut, lane8, uw[j], p);
                        Bq[j][p] = pack_bf16_rne(__fmul_rn(pr.x, sj[j]), __fmul_rn(pr.y, sj[j]));
                    }
                }
            }
            // MFMA over the 8 row fragments for this band
#pragma unroll
            for (int j = 0; j < 4; j++) {
#pragma unroll
                for (int mf = 0; mf < 8; mf++) {
                    const uint4 t = *reinterpret_cast<const uint4*>(&xs[buf][(16 * mf + r) * XS_STRIDE + 32 * j + 8 * h]);
                    acc[mf][nf] = mfma(u32x4{t.x, t.y, t.z, t.w}, Bq[j], acc[mf][nf]);
                }
            }
        }

        if (more) store_x(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue ----
    const int64_t tile_id = tn * a.tiles_m + tm;
    if (a.ksplit == 1) {
#pragma unroll
        for (int nf = 0; nf < 4; nf++) {
            const int64_t col = (band0 + nf) * 16 + r;
            if (col >= N) continue;
#pragma unroll
            for (int mf = 0; mf < 8; mf++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int64_t mm = m0 + 16 * mf + 4 * h + i;
                    if (mm < M) store_out(a.out, mm, col, finish(a, col, acc[mf][nf][i], g));
                }
        }
        return;
    }
#pragma unroll
    for (int nf = 0; nf < 4; nf++) {
        const int64_t col = (band0 + nf) * 16 + r;
        if (col >= N) continue;
#pragma unroll
        for (int mf = 0; mf < 8; mf++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int64_t mm = m0 + 16 * mf + 4 * h + i;
                if (mm < M) a.partial[((int64_t)ks * M + mm) * N + col] = acc[mf][nf][i];
            }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = atomicAdd(&a.counters[tile_id], 1u);
        s_last = (old == (uint32_t)(a.ksplit - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
#pragma unroll
    for (int nf = 0; nf < 4; nf++) {
        const int64_t col = (band0 + nf) * 16 + r;
        if (col >= N) continue;
#pragma unroll
        for (int mf = 0; mf < 8; mf++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int64_t mm = m0 + 16 * mf + 4 * h + i;
                if (mm < M) {
                    float v = 0.0f;
                    for (int s2 = 0; s2 < a.ksplit; s2++)
                        v += __builtin_nontemporal_load(&a.partial[((int64_t)s2 * M + mm) * N + col]);
                    store_out(a.out, mm, col, finish(a, col, v, g));
                }
            }
    }
    if (tid == 0) atomicExch(&a.counters[tile_id], 0u);
}

// ---------------------------------------------------------------------------
// Schedules and launchers.
// ---------------------------------------------------------------------------
constexpr int kNumCU = 256;

struct Sched {
    int ksplit;
    int64_t kt_per;
    int64_t counters;
    int64_t tiles_m, tiles_n;
    unsigned grid;
};

static Sched gemv_sched(int fmt, int64_t m, int64_t n, int64_t k, bool allow_split) {
    Sched s{};
    const int64_t KT = k / tile_k(fmt);
    const int64_t nbands = n / 16;
    int ks = 1;
    if (allow_split) {
        // split K until every CU has a workgroup, keeping >= one tile per wave per piece
        while (nbands * ks < kNumCU && KT / (ks * 2) >= 4) ks *= 2;
    }
    s.ksplit = ks;
    s.kt_per = (KT + ks - 1) / ks;
    s.counters = nbands;
    s.tiles_m = 1;
    s.tiles_n = nbands;
    const int64_t items = nbands * ks;
    s.grid = (unsigned)std::min<int64_t>(items, 2 * kNumCU);
    (void)m;
    return s;
}

static Sched gemm_sched(int fmt, int64_t m, int64_t n, int64_t k, bool allow_split) {
    (void)fmt;
    Sched s{};
    s.tiles_m = (m + BM - 1) / BM;
    s.tiles_n = (n + BN - 1) / BN;
    const int64_t steps = k / BK;
    const int64_t tiles = s.tiles_m * s.tiles_n;
    int ks = 1;
    if (allow_split) {
        while (tiles * ks < kNumCU && steps / (ks * 2) >= 4) ks *= 2;
    }
    s.ksplit = ks;
    s.kt_per = (steps + ks - 1) / ks;
    s.counters = tiles;
    const int64_t items = tiles * ks;
    s.grid = (unsigned)(((items + 7) / 8) * 8);
    return s;
}

static size_t ws_bytes_for(const Sched& s, int64_t m, int64_t n) {
    if (s.ksplit <= 1) return 0;
    return (size_t)align16(256 + 4 * s.counters) + (size_t)s.ksplit * (size_t)m * (size_t)n * 4u;
}

size_t gemv_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k) {
    return ws_bytes_for(gemv_sched(fmt, m, n, k, true), m, n);
}
size_t gemm_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k) {
    return ws_bytes_for(gemm_sched(fmt, m, n, k, true), m, n);
}
size_t matmul_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k) {
    return m <= 16 ? gemv_workspace_bytes(fmt, m, n, k) : gemm_workspace_bytes(fmt, m, n, k);
}

static KArgs make_args(const MatmulProblem& p, const Sched& s) {
    KArgs a{};
    a.x = p.x;
    a.ldx = p.ldx;
    a.m = (int)p.m;
    a.n = p.n;
    a.k = p.k;
    a.codes = p.codes;
    a.scales = p.scales;
    a.bias = p.bias;
    a.out = p.out;
    a.L = scale_layout(p.fmt, p.dq, p.n, p.k);
    a.ksplit = s.ksplit;
    a.kt_per = s.kt_per;
    a.tiles_m = s.tiles_m;
    a.tiles_n = s.tiles_n;
    if (s.ksplit > 1) {
        a.counters = reinterpret_cast<uint32_t*>(p.ws);
        a.partial = reinterpret_cast<float*>(reinterpret_cast<char*>(p.ws) + align16(256 + 4 * s.counters));
    }
    return a;
}

template <int FMT, bool DQ>
static void gemv_dispatch_ni(const KArgs& a, unsigned grid, hipStream_t st) {
    switch (a.m) {
    case 1: hipLaunchKernelGGL((k_gemv<FMT, DQ, 1>), dim3(grid), dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_gemv<FMT, DQ, 2>), dim3(grid), dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL((k_gemv<FMT, DQ, 3>), dim3(grid), dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((k_gemv<FMT, DQ, 4>), dim3(grid), dim3(256), 0, st, a); break;
    }
}

hipError_t launch_gemv(const MatmulProblem& p, hipStream_t st) {
    const size_t need = gemv_workspace_bytes(p.fmt, p.m, p.n, p.k);
    const bool split = p.ws != nullptr && need > 0 && p.ws_bytes >= need;
    const Sched s = gemv_sched(p.fmt, p.m, p.n, p.k, split);
    const KArgs a = make_args(p, s);
    switch (p.fmt) {
    case kNF4:
        if (p.dq) gemv_dispatch_ni<kNF4, true>(a, s.grid, st);
        else gemv_dispatch_ni<kNF4, false>(a, s.grid, st);
        break;
    case kNVFP4: gemv_dispatch_ni<kNVFP4, false>(a, s.grid, st); break;
    case kQ4_0: gemv_dispatch_ni<kQ4_0, false>(a, s.grid, st); break;
    case kQ8_0: gemv_dispatch_ni<kQ8_0, false>(a, s.grid, st); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemm(const MatmulProblem& p, hipStream_t st) {
    const size_t need = gemm_workspace_bytes(p.fmt, p.m, p.n, p.k);
    const bool split = p.ws != nullptr && need > 0 && p.ws_bytes >= need;
    const Sched s = gemm_sched(p.fmt, p.m, p.n, p.k, split);
    const KArgs a = make_args(p, s);
    const dim3 grid(s.grid), block(256);
    switch (p.fmt) {
    case kNF4:
        if (p.dq) hipLaunchKernelGGL((k_gemm<kNF4, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((k_gemm<kNF4, false>), grid, block, 0, st, a);
        break;
    case kNVFP4: hipLaunchKernelGGL((k_gemm<kNVFP4, false>), grid, block, 0, st, a); break;
    case kQ4_0: hipLaunchKernelGGL((k_gemm<kQ4_0, false>), grid, block, 0, st, a); break;
    case kQ8_0: hipLaunchKernelGGL((k_gemm<kQ8_0, false>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace wq
