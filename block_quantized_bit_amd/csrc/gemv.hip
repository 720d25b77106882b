// gemv.hip -- the decode GEMV (m <= 16): the general kernel and the streaming kernel
// for matrices far taller than the chip, with their launchers.
#include "mm_common.h"

namespace wq {

// ===========================================================================
template <int FMT>
struct GemvTile {
    uint4 code;             // this lane's 16 bytes of the tile
    uint32_t sc[6];         // raw scale words (format dependent)
    u32x4 A[tile_k(FMT) / 32];
};

constexpr int kGemvWaves = 8;   // waves per workgroup, all on one band, splitting its K range

// Vector memory instructions gemv_load issues for a tile's codes and scales (X excluded; for
// double quant with k <= 16384, plus two per band for the row's group scales -- a wait for at
// most this many per tile outstanding can only wait longer than needed).
template <int FMT, bool DQ>
__device__ constexpr int gemv_w_loads() { return FMT == kQ6_K ? 4 : (FMT == kQ5_0 || FMT == kQ4_K) ? 3 : 2; }

// Double-quant group scales of one row, when the row holds <= 256 blocks (k <= 16384) and so
// spans at most two 256-block groups: blocks j < jt of the row are in the first.
struct DqRow {
    float dA, dB;
    int32_t jt;
};

__device__ inline DqRow dq_row(const KArgs& a, int64_t row) {
    const int64_t nbr = a.k / 64, b0 = row * nbr;
    const int64_t gA = b0 >> 8, gB = (b0 + nbr - 1) >> 8;
    const float* dt = reinterpret_cast<const float*>(a.scales + a.d_off);
    return DqRow{dt[gA], dt[gB], (int32_t)((gA + 1) * 256 - b0)};
}

// dq: non-null when the double-quant group scales come from the row's pair (DqRow) instead of
// being gathered per tile.
template <int FMT, bool DQ, bool XL = false>
__device__ inline void gemv_load(GemvTile<FMT>& t, const KArgs& a, int64_t band, int64_t kt, int lane, int r,
                                 const uint16_t* xrow, int64_t KT, const DqRow* dq = nullptr) {
    constexpr int TK = tile_k(FMT);
    const int64_t tile = band * KT + kt;
    {
        // weights are read exactly once: non-temporal
        const u32x4 c = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.codes + tile * kTileBytes + lane * 16));
        t.code = make_uint4(c[0], c[1], c[2], c[3]);
    }
    if constexpr (FMT == kNF4) {
        if constexpr (DQ) {
            t.sc[0] = *reinterpret_cast<const uint16_t*>(a.scales + tile * 32 + r * 2);
            if (dq) {
                // group scales: taken from the row's pair at use time (gemv_dq_scales)
            } else {
                const int64_t b0 = (band * 16 + r) * (a.k / 64) + kt * 2;
                const float* dt = reinterpret_cast<const float*>(a.scales + a.d_off);
                t.sc[1] = __float_as_uint(dt[b0 >> 8]);
                t.sc[2] = __float_as_uint(dt[(b0 + 1) >> 8]);
            }
        } else {
            const uint2 v = *reinterpret_cast<const uint2*>(a.scales + (tile * 32 + r * 2) * 4);
            t.sc[0] = v.x;
            t.sc[1] = v.y;
        }
    } else if constexpr (FMT == kQ4_0) {
        const uint2 v = *reinterpret_cast<const uint2*>(a.scales + (tile * 64 + r * 4) * 2);
        t.sc[0] = v.x;
        t.sc[1] = v.y;
    } else if constexpr (FMT == kQ6_K) {
        // the row's 8 sub-block scales, this lane's 8 bytes of bits 4-5 (after the n k / 2
        // code bytes) and the super-block's d
        const uint2 v = *reinterpret_cast<const uint2*>(a.scales + tile * 128 + r * 8);
        t.sc[0] = v.x;
        t.sc[1] = v.y;
        const uint2 hb = *reinterpret_cast<const uint2*>(a.codes + a.n * a.k / 2 + tile * 512 + lane * 8);
        t.sc[2] = hb.x;
        t.sc[3] = hb.y;
        t.sc[4] = *reinterpret_cast<const uint16_t*>(a.scales + a.kd_off + ((band * 16 + r) * (a.k >> 8) + (kt >> 1)) * 2);
    } else if constexpr (FMT == kQ4_K) {
        // the row's sub-block record (4 scale bytes, 4 offset bytes) and its super-block's
        // (d, dmin); a 128-K tile is half a 256-K super-block
        const uint2 v = *reinterpret_cast<const uint2*>(a.scales + tile * 128 + r * 8);
        t.sc[0] = v.x;
        t.sc[1] = v.y;
        t.sc[2] = *reinterpret_cast<const uint32_t*>(a.scales + a.kd_off + ((band * 16 + r) * (a.k >> 8) + (kt >> 1)) * 4);
    } else if constexpr (FMT == kQ5_0) {
        // the row's four fp16 scales (8 bytes), then its four fifth-bit words (16 bytes)
        const uint2 v = *reinterpret_cast<const uint2*>(a.scales + (tile * 64 + r * 4) * 2);
        t.sc[0] = v.x;
        t.sc[1] = v.y;
        const uint4 hb = *reinterpret_cast<const uint4*>(a.scales + a.hb_off + tile * 256 + r * 16);
        t.sc[2] = hb.x;
        t.sc[3] = hb.y;
        t.sc[4] = hb.z;
        t.sc[5] = hb.w;
    } else if constexpr (FMT == kQ4_1) {
        // the row's four (d, m) pairs of the tile: 16 bytes
        const uint4 v = *reinterpret_cast<const uint4*>(a.scales + tile * 256 + r * 16);
        t.sc[0] = v.x;
        t.sc[1] = v.y;
        t.sc[2] = v.z;
        t.sc[3] = v.w;
    } else if constexpr (FMT == kNVFP4) {
        const uint2 v = *reinterpret_cast<const uint2*>(a.scales + tile * 128 + r * 8);
        t.sc[0] = v.x;
        t.sc[1] = v.y;
    } else {
        t.sc[0] = *reinterpret_cast<const uint32_t*>(a.scales + (tile * 32 + r * 2) * 2);
    }
    // rows r >= m read row 0 (always valid); their products only reach output rows that are never stored
    if constexpr (!XL) {
#pragma unroll
        for (int j = 0; j < TK / 32; j++) {
            const uint4 v = *reinterpret_cast<const uint4*>(xrow + kt * TK + 32 * j);
            t.A[j] = u32x4{v.x, v.y, v.z, v.w};
        }
    }
}

// X (m rows of k bf16) copied once into LDS by LDS-direct loads of 16 bytes per lane,
// chunk-major: chunk c (elements 8c .. 8c+7) of row r lands at byte 16 (c m + r).  The
// 16 lanes that read one K chunk for 16 different rows (an A-operand read at m = 16)
// then touch 256 contiguous bytes; row-major rows k * 2 bytes apart would all fall on
// the same banks.  An LDS-direct load writes its lanes' chunks contiguously, and here
// lane i of the copy fetches destination chunk i, so only the source addresses move.
__device__ __forceinline__ void gemv_stage_x(uint16_t* xs, const KArgs& a, int wave, int lane) {
    // the copy is used for m * k <= 32768 elements, so chunk indices fit 32 bits
    const uint32_t m = (uint32_t)a.m;
    const uint32_t nchunks = m * (uint32_t)(a.k / 8);
    for (uint32_t c0 = (uint32_t)wave * 64; c0 < nchunks; c0 += 64 * kGemvWaves) {
        const uint32_t i = c0 + (uint32_t)lane;
        if (i < nchunks) {
            const uint32_t c = m == 1 ? i : i / m, row = i - c * m;
            __builtin_amdgcn_global_load_lds(a.x + (int64_t)row * a.ldx + (int64_t)c * 8, xs + c0 * 8, 16, 0, 0);
        }
    }
}

// NF4 and Q4_0 codes become bf16 pairs through the LDS table; NVFP4 and Q8_0
// convert in registers.
template <int FMT>
__host__ __device__ constexpr bool gemv_uses_lut() { return FMT == kNF4 || FMT == kQ4_0; }

template <int FMT, bool DQ, int NI>
__device__ inline void gemv_consume(const GemvTile<FMT>& t, f32x4& acc, const uint32_t* lut, uint32_t lane4,
                                    int h, float mu) {
    const uint32_t uw[4] = {t.code.x, t.code.y, t.code.z, t.code.w};
    if constexpr (FMT == kNF4) {
        float s0, s1;
        if constexpr (DQ) {
            s0 = __fadd_rn(__fmul_rn((float)(int8_t)(t.sc[0] & 255u), __uint_as_float(t.sc[1])), mu);
            s1 = __fadd_rn(__fmul_rn((float)(int8_t)((t.sc[0] >> 8) & 255u), __uint_as_float(t.sc[2])), mu);
        } else {
            s0 = __uint_as_float(t.sc[0]);
            s1 = __uint_as_float(t.sc[1]);
        }
        // the tile's 16 table reads first, then its MFMAs: one LDS round trip per tile
        u32x4 B[4];
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int q = 0; q < 4; q++) B[j][q] = lut_pair(lut, lane4, uw[j], q);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jj = 0; jj < 2; jj++) p = mfma(t.A[kb * 2 + jj], B[kb * 2 + jj], p);
            const float s = kb ? s1 : s0;
#pragma unroll
            for (int i = 0; i < NI; i++) acc[i] += p[i] * s;
        }
    } else if constexpr (FMT == kQ4_0) {
        u32x4 B[4];
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int q = 0; q < 4; q++) B[j][q] = lut_pair(lut, lane4, uw[j], q);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const f32x4 p = mfma(t.A[j], B[j], f32x4{0.f, 0.f, 0.f, 0.f});
            const float s = f16_value((uint16_t)(t.sc[j >> 1] >> (16 * (j & 1))));
#pragma unroll
            for (int i = 0; i < NI; i++) acc[i] += p[i] * s;
        }
    } else if constexpr (FMT == kQ4_1) {
        // B = bf16(w^), block j of the row for K slice j
#pragma unroll
        for (int j = 0; j < 4; j++) acc = mfma(t.A[j], q4_1_operand(uw[j], t.sc[j]), acc);
    } else if constexpr (FMT == kQ6_K) {
        // B = bf16(w^); K slice j spans sub-blocks 2j (h = 0, 1) and 2j + 1 (h = 2, 3)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float S = q6_k_scale(t.sc[0], t.sc[1], t.sc[4], 2 * j + (h >> 1));
            const uint32_t hw = t.sc[2 + (j >> 1)] >> (16 * (j & 1));
            acc = mfma(t.A[j], q6_k_operand(uw[j], hw & 255u, (hw >> 8) & 255u, S), acc);
        }
    } else if constexpr (FMT == kQ4_K) {
        // B = bf16(w^), sub-block j of the row for K slice j
#pragma unroll
        for (int j = 0; j < 4; j++) {
            float S, O;
            q4_k_sub(t.sc[0], t.sc[1], t.sc[2], j, S, O);
            acc = mfma(t.A[j], q4_k_operand(uw[j], S, O), acc);
        }
    } else if constexpr (FMT == kQ5_0) {
        // B = bf16(w^), block j of the row for K slice j; this lane's k are bits 8h .. 8h+7
        // of the block's fifth-bit word
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint16_t db = (uint16_t)(t.sc[j >> 1] >> (16 * (j & 1)));
            acc = mfma(t.A[j], q5_0_operand(uw[j], (t.sc[2 + j] >> (8 * h)) & 255u, db), acc);
        }
    } else if constexpr (FMT == kNVFP4 && NI == 1) {
        // One token leaves 15 of the 16 A rows free, so the E4M3 block scales are applied after
        // the MFMA, to per-block partial sums.  In K slice j the 16-value block 2j + (h >> 1)
        // (lanes h = 0, 1: the slice's first 16 k; h = 2, 3: its last 16) puts its x in A row
        // (2j + (h >> 1)) & 3 and zeros in every other row.  Chained over slices 0-1 (and 2-3),
        // output row i of column n is then the sum of x * e2m1 over block i (4 + i) of the tile
        // row alone: exact products, no offset term.  B holds the bare E2M1 values (exact in
        // bf16: one conversion per code pair).  Lane (0, n) holds rows 0-3 of column n and the
        // row's 8 scale bytes (block b: byte b & 3 of word b >> 2); lanes h >= 1 hold zero rows.
        const int r = __lane_id() & 15;
        f32x4 P[2];
#pragma unroll
        for (int c = 0; c < 2; c++) {
            f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jj = 0; jj < 2; jj++) {
                const int j = 2 * c + jj;
                u32x4 B;
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    bf16x2 v;
                    if (q == 0) v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(uw[j], 1.0f, 0);
                    else if (q == 1) v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(uw[j], 1.0f, 1);
                    else if (q == 2) v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(uw[j], 1.0f, 2);
                    else v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(uw[j], 1.0f, 3);
                    B[q] = __builtin_bit_cast(uint32_t, v);
                }
                const bool live = r == 2 * jj + (h >> 1);
                const u32x4 A = live ? t.A[j] : u32x4{0u, 0u, 0u, 0u};
                p = mfma(A, B, p);
            }
            P[c] = p;
        }
#pragma unroll
        for (int c = 0; c < 2; c++) {
            const int sw = (int)t.sc[c];
            acc[0] += P[c][0] * __builtin_amdgcn_cvt_f32_fp8(sw, 0);
            acc[0] += P[c][1] * __builtin_amdgcn_cvt_f32_fp8(sw, 1);
            acc[0] += P[c][2] * __builtin_amdgcn_cvt_f32_fp8(sw, 2);
            acc[0] += P[c][3] * __builtin_amdgcn_cvt_f32_fp8(sw, 3);
        }
    } else if constexpr (FMT == kNVFP4) {
        // block 2j + (h >> 1) of the row: byte 2 (j & 1) + (h >> 1) of scale word j >> 1
        const uint32_t hs = 8u * (uint32_t)(h >> 1);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t sw = t.sc[j >> 1] >> hs;
            const float s = (j & 1) ? __builtin_amdgcn_cvt_f32_fp8((int)sw, 2) : __builtin_amdgcn_cvt_f32_fp8((int)sw, 0);
            u32x4 B;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                // e2m1 pair of byte q (low nibble first) times the E4M3 scale: exact, so keeping
                // the upper halves of the fp32 products is the exact bf16 value
                f32x2 v;
                if (q == 0) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(uw[j], 1.0f, 0);
                else if (q == 1) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(uw[j], 1.0f, 1);
                else if (q == 2) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(uw[j], 1.0f, 2);
                else v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(uw[j], 1.0f, 3);
                B[q] = __builtin_amdgcn_perm(__float_as_uint(v[1] * s), __float_as_uint(v[0] * s), 0x07060302u);
            }
            acc = mfma(t.A[j], B, acc);
            // one K slice at a time: converting every slice of the tile ahead of its MFMAs
            // holds more registers and measured 0.15-0.25 us slower per decode launch
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {  // kQ8_0: 16 x 64 tile, K slices j = 0, 1
#pragma unroll
        for (int j = 0; j < 2; j++) {
            u32x4 B;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const uint32_t wv = uw[2 * j + (q >> 1)];
                const int sh = 16 * (q & 1);
                const float f0 = (float)(int)(int8_t)(wv >> sh);
                const float f1 = (float)(int)(int8_t)(wv >> (sh + 8));
                B[q] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
            }
            const f32x4 p = mfma(t.A[j], B, f32x4{0.f, 0.f, 0.f, 0.f});
            const float s = f16_value((uint16_t)(t.sc[0] >> (16 * j)));
#pragma unroll
            for (int i = 0; i < NI; i++) acc[i] += p[i] * s;
        }
    }
}

// Wave w of a workgroup owns tiles w, w + 8, w + 16, ... of its band's K range:
// C of them, all requested before any is used.  A band is finished by summing
// the 8 waves' 16x16 partial tiles in LDS in wave order.
// Double quant with fewer than 8 tiles per wave (k <= 5120 here) takes the row's two group
// scales once per band (DqRow) instead of two gathers per tile.
template <int FMT, bool DQ, int C>
__device__ constexpr bool gemv_dq_rows() { return FMT == kNF4 && DQ && C < 8; }

// The row's double-quant group scales (and, when mu is non-null, the matrix mean) are
// requested right after the first tile: the first tile's use needs them, and a wait for
// everything older than the band's requests (the X copy) does not wait for them.
template <int FMT, bool DQ, int C, bool XL>
__device__ __forceinline__ void gemv_load_band(GemvTile<FMT> (&R)[C], DqRow& dq, const KArgs& a, int64_t band,
                                               int64_t c0, int wave, int lane, int r, const uint16_t* xrow,
                                               int64_t KT, float* mu = nullptr) {
    constexpr bool DR = gemv_dq_rows<FMT, DQ, C>();
#pragma unroll
    for (int s = 0; s < C; s++) {
        const int64_t kt = std::min<int64_t>(wave + (c0 + s) * kGemvWaves, KT - 1);
        gemv_load<FMT, DQ, XL>(R[s], a, band, kt, lane, r, xrow, KT, DR ? &dq : nullptr);
        if (s == 0) {
            if constexpr (DR) dq = dq_row(a, band * 16 + r);
            if constexpr (FMT == kNF4 && DQ) {
                if (mu) *mu = load_f32_vmem(a.scales + a.mu_off);
            }
        }
    }
}

// Register loads a band request issues: C tiles, plus the row's two group scales.
template <int FMT, bool DQ, int C>
__device__ constexpr int gemv_band_loads() { return C * gemv_w_loads<FMT, DQ>() + (gemv_dq_rows<FMT, DQ, C>() ? 2 : 0); }

// XL: the A operands come from the LDS copy of X (xl = this lane's row, chunk h), read here.
template <int FMT, bool DQ, int NI, int C, bool XL>
__device__ __forceinline__ void gemv_consume_band(GemvTile<FMT> (&R)[C], const DqRow& dq, f32x4& acc, int64_t c0,
                                                  int wave, int64_t KT, const uint32_t* lut, uint32_t lane4, int h,
                                                  float mu, const uint16_t* xl, int64_t xm8) {
    constexpr int TK = tile_k(FMT);
#pragma unroll
    for (int s = 0; s < C; s++) {
        const int64_t kt = wave + (c0 + s) * kGemvWaves;
        if (kt < KT) {
            if constexpr (gemv_dq_rows<FMT, DQ, C>()) {
                R[s].sc[1] = __float_as_uint(2 * kt < dq.jt ? dq.dA : dq.dB);
                R[s].sc[2] = __float_as_uint(2 * kt + 1 < dq.jt ? dq.dA : dq.dB);
            }
            if constexpr (XL) {
#pragma unroll
                for (int j = 0; j < TK / 32; j++) {
                    // chunk kt TK / 8 + 4 j + h of this lane's row, chunk-major (gemv_stage_x)
                    const uint4 v = *reinterpret_cast<const uint4*>(xl + (kt * (TK / 8) + 4 * j) * xm8);
                    R[s].A[j] = u32x4{v.x, v.y, v.z, v.w};
                }
            }
            gemv_consume<FMT, DQ, NI>(R[s], acc, lut, lane4, h, mu);
        }
    }
}

// Output address of column col (< n <= 2^31 - 1) for the GEMV: as col_out_nobias<true>, with
// the split choice made in 32-bit arithmetic (columns, split ends and row strides are all
// 32-bit), which keeps the instructions after the band's last barrier few.
__device__ __forceinline__ ColOut gemv_col_out(const KArgs& a, int64_t col64) {
    const int col = (int)col64;
    const int e0 = __builtin_amdgcn_readfirstlane(a.end0), e1 = __builtin_amdgcn_readfirstlane(a.end1);
    const bool s1 = col >= e0, s2 = col >= e1;
    char* const y0 = out_p<true>(a.y0);
    char* const y1 = out_p<true>(a.y1);
    char* const y2 = out_p<true>(a.y2);
    char* const base = s2 ? y2 : (s1 ? y1 : y0);
    const int ld = s2 ? __builtin_amdgcn_readfirstlane(a.ldy2)
                      : (s1 ? __builtin_amdgcn_readfirstlane(a.ldy1) : __builtin_amdgcn_readfirstlane(a.ldy0));
    const int c0 = s2 ? e1 : (s1 ? e0 : 0);
    const int es = a.f32 ? 4 : 2;
    ColOut c;
    c.p = base + (int64_t)(uint32_t)(col - c0) * es;
    c.ld = (int64_t)ld * es;
    c.bias = 0.0f;
    return c;
}

// NPRE: requests of the next band already in flight (band pipelining).  The barriers only need the
// LDS writes complete; the compiler waits for the bias and for the prefetched tiles where they are
// used, so the barriers let those requests (and the last store) stay in flight.
template <int NI, int NPRE = 0>
__device__ __forceinline__ void gemv_finish_band(const KArgs& a, f32x4 (&red)[kGemvWaves][64], const f32x4& acc,
                                                 int64_t band, int wave, int lane, float g) {
    const int r = lane & 15, h = lane >> 4;
    if constexpr (NI == 1) {
        // one token: only accumulator 0 of lanes 0-15 (row 0, column r) is ever stored.  Those
        // lanes request their column's bias before the barrier, and the barrier waits for every
        // request of the wave but that last one (the counter counts in order), so its latency
        // overlaps the wait for the other waves and the sum.
        // lane-major: the 8 waves' values for lane r sit side by side, so the storing lane
        // reads them with two 16-byte reads
        float* red1 = reinterpret_cast<float*>(&red[0][0]);
        if (h == 0) red1[lane * kGemvWaves + wave] = acc[0];
        // (unconditional, without a branch around it: without a bias it reads X's first row,
        // always at least 16 elements, and the value is dropped)
        const uint16_t* const bsrc = a.bias ? a.bias + band * 16 : a.x;
        const uint16_t braw = bsrc[r];
        lds_barrier_vm<NPRE + 1>();
        if (wave == 0 && h == 0) {
            static_assert(kGemvWaves == 8, "two 16-byte reads per lane");
            const f32x4 p0 = *reinterpret_cast<const f32x4*>(red1 + lane * kGemvWaves);
            const f32x4 p1 = *reinterpret_cast<const f32x4*>(red1 + lane * kGemvWaves + 4);
            float v = p0[0];   // in wave order, as before
            v += p0[1]; v += p0[2]; v += p0[3];
            v += p1[0]; v += p1[1]; v += p1[2]; v += p1[3];
            ColOut c = gemv_col_out(a, band * 16 + r);
            c.bias = a.bias ? bf16_value(braw) : 0.0f;
            put_out(a, c, 0, v, g);
        }
        lds_barrier_vm<NPRE + 1>();
        return;
    }
    // the bias is requested before the barrier, as for one token
    red[wave][lane] = acc;
    const uint16_t* const bsrc = a.bias ? a.bias + band * 16 : a.x;
    const uint16_t braw = bsrc[r];
    lds_barrier_vm<NPRE + 1>();
    if (wave == 0) {
        f32x4 v = red[0][lane];
#pragma unroll
        for (int w = 1; w < kGemvWaves; w++) v += red[w][lane];
        ColOut c = gemv_col_out(a, band * 16 + r);
        c.bias = a.bias ? bf16_value(braw) : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int mm = 4 * h + i;
            if (mm < a.m) put_out(a, c, mm, v[i], g);
        }
    }
    lds_barrier_vm<NPRE + 1>();
}

// PIPE = false: every workgroup owns one band (grid == number of bands), its
//   tiles come in rounds of C per wave (one round when K <= 8 * C tiles).
// PIPE = true : workgroups loop over bands; each wave holds all its tiles of a
//   band in one round (K <= 8 * C tiles) and requests the next band's tiles
//   before using the current ones.  The prefetch index is clamped to the last
//   band, so the requests are unconditional.
// XL: X is copied once into (dynamic) LDS at the start -- a few LDS-direct loads
//   per workgroup instead of four 64-lane loads per tile and wave -- and the A
//   operands are read from there; used when m * k is small (decode).  The copy
//   is requested before the weights, so waiting for it (vmcnt = the weight loads
//   issued after it) never waits for a weight load.
template <int FMT, bool DQ, int NI, int C, bool PIPE, bool XL>
__global__ __launch_bounds__(64 * kGemvWaves, (C <= 2 ? 2 : 1)) void k_gemv(KArgs a) {
    __shared__ uint32_t lut[gemv_uses_lut<FMT>() ? kLutWords : 1];
    __shared__ f32x4 red[kGemvWaves][64];
    extern __shared__ __attribute__((aligned(16))) uint16_t xs_dyn[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15;
    const int h = lane >> 4;
    const uint32_t lane4 = (uint32_t)lane << 2;
    const int64_t KT = a.k / tile_k(FMT);
    const int64_t nbands = a.n / 16;

    // The double-quant mean sits with the scales, in memory as cold as the weights.  With X
    // copied to LDS it is requested with the first band's tiles (after the copy), so that
    // the wait for the copy does not wait for it; without the copy, up front.
    float g = 1.0f, mu = 0.0f;
    if constexpr (FMT == kNVFP4) g = load_f32_vmem(a.gs);
    if constexpr (FMT == kNF4 && DQ && !XL) mu = load_f32_vmem(a.scales + a.mu_off);
    constexpr int kMuLoads = (FMT == kNF4 && DQ && XL) ? 1 : 0;
    float* const mu_first = kMuLoads ? &mu : nullptr;
    const uint16_t* xrow = a.x + (int64_t)(r < a.m ? r : 0) * a.ldx + h * 8;
    // the LDS copy of X is chunk-major: chunk c of row r at element 8 (c m + r); the
    // one-token instantiation (NI = 1 is only launched for m = 1) gets a constant stride,
    // so its reads keep immediate offsets
    const int64_t xm8 = NI == 1 ? 8 : (int64_t)a.m * 8;
    const uint16_t* xl = xs_dyn + (int64_t)h * xm8 + (int64_t)(r < a.m ? r : 0) * 8;
    const int64_t per_wave = (KT + kGemvWaves - 1) / kGemvWaves;

    if constexpr (!PIPE) {
        const int64_t band = blockIdx.x;
        // With XL the code table is filled first: LDS writes issued while the LDS-direct X copy
        // is in flight would have to wait for every load.  Otherwise it is filled while the first
        // tiles are in flight.
        if constexpr (XL) {
            if constexpr (gemv_uses_lut<FMT>()) build_lut<FMT, 64 * kGemvWaves>(lut);
            gemv_stage_x(xs_dyn, a, wave, lane);
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int64_t c0 = 0; c0 < per_wave; c0 += C) {
            GemvTile<FMT> R[C];
            DqRow dq;
            gemv_load_band<FMT, DQ, C, XL>(R, dq, a, band, c0, wave, lane, r, xrow, KT, c0 == 0 ? mu_first : nullptr);
            if (c0 == 0) {
                if constexpr (XL) {
                    lds_barrier_vm<gemv_band_loads<FMT, DQ, C>() + kMuLoads>();
                } else {
                    if constexpr (gemv_uses_lut<FMT>()) build_lut<FMT, 64 * kGemvWaves>(lut);
                    __syncthreads();
                }
            }
            gemv_consume_band<FMT, DQ, NI, C, XL>(R, dq, acc, c0, wave, KT, lut, lane4, h, mu, xl, xm8);
        }
        gemv_finish_band<NI>(a, red, acc, band, wave, lane, g);
    } else {
        const int64_t stride = (int64_t)a.wg_per_cu * kNumCU;   // the grid (gemv_launch_cx)
        GemvTile<FMT> R0[C], R1[C];
        DqRow dq0, dq1;
        int64_t band = blockIdx.x;
        if constexpr (XL) {
            if constexpr (gemv_uses_lut<FMT>()) build_lut<FMT, 64 * kGemvWaves>(lut);
            gemv_stage_x(xs_dyn, a, wave, lane);
        }
        gemv_load_band<FMT, DQ, C, XL>(R0, dq0, a, band, 0, wave, lane, r, xrow, KT, mu_first);
        if constexpr (XL) {
            lds_barrier_vm<gemv_band_loads<FMT, DQ, C>() + kMuLoads>();
        } else {
            if constexpr (gemv_uses_lut<FMT>()) build_lut<FMT, 64 * kGemvWaves>(lut);
            __syncthreads();
        }
        for (; band < nbands; band += 2 * stride) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            gemv_load_band<FMT, DQ, C, XL>(R1, dq1, a, std::min<int64_t>(band + stride, nbands - 1), 0, wave, lane,
                                          r, xrow, KT);
            gemv_consume_band<FMT, DQ, NI, C, XL>(R0, dq0, acc, 0, wave, KT, lut, lane4, h, mu, xl, xm8);
            gemv_finish_band<NI, gemv_band_loads<FMT, DQ, C>()>(a, red, acc, band, wave, lane, g);
            if (band + stride >= nbands) break;
            acc = f32x4{0.f, 0.f, 0.f, 0.f};
            gemv_load_band<FMT, DQ, C, XL>(R0, dq0, a, std::min<int64_t>(band + 2 * stride, nbands - 1), 0, wave,
                                          lane, r, xrow, KT);
            gemv_consume_band<FMT, DQ, NI, C, XL>(R1, dq1, acc, 0, wave, KT, lut, lane4, h, mu, xl, xm8);
            gemv_finish_band<NI, gemv_band_loads<FMT, DQ, C>()>(a, red, acc, band + stride, wave, lane, g);
        }
    }
}

// ===========================================================================
// Streaming GEMV (many more bands than workgroups, short K, small X): each wave
// owns whole bands, so there is no cross-wave reduction and no barrier in the
// loop.  A band's T tiles are requested one band ahead into the other of two
// register sets.  Loads are buffer loads whose base is the band's first tile
// (wave-uniform, scalar arithmetic) with a per-lane offset fixed for the whole
// kernel, so addressing costs no vector instructions; the descriptor covers
// exactly the band's K tiles, so slots s >= K/tile_k read zeros (the buffer
// range check) and take their A operand from a zero row.  X is staged once per
// workgroup in LDS and read there as the MFMA A operand; the double-quant
// group scales of a lane's row are fetched once per band (a row of <= 10 tiles
// spans at most two 256-block groups).
// ===========================================================================
constexpr int kStreamXMax = 8192 - 128;   // bf16 elements of X staged in LDS (m * k), then 128 zeros
constexpr int kStreamGrid = 2 * kNumCU;     // two workgroups of 4 waves per CU

// Scale bytes per tile and per lane (one row of the tile) in the packed layout.
template <int FMT, bool DQ>
__device__ constexpr int tile_scale_bytes() {
    return FMT == kQ8_0 ? 64 : (FMT == kNF4 && DQ) ? 32 : FMT == kQ4_1 ? 256 : 128;
}

struct StreamTile {
    u32x4 code;
    uint32_t sc[2];
};

struct StreamBand {
    uint32_t braw;     // bias (bf16 bits) of this lane's column
    float dA, dB;      // double quant: group scales of the first / last block of the lane's row
    int32_t jt;        // double quant: blocks of the row that belong to group A
};

// Request tile s of a band (codes and this lane's scale record) into R.
template <int FMT, bool DQ>
__device__ __forceinline__ void stream_load_tile(StreamTile& R, BufRes rc, BufRes rs, int s, int lane, int r) {
    constexpr int SB = tile_scale_bytes<FMT, DQ>();
    R.code = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, lane * 16 + s * kTileBytes, 0, kNT));
    if constexpr (FMT == kNF4 && DQ) {
        R.sc[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, r * 2 + s * SB, 0, kNT);
    } else if constexpr (FMT == kQ8_0) {
        R.sc[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, r * 4 + s * SB, 0, kNT);
    } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, r * 8 + s * SB, 0, kNT);
        R.sc[0] = v[0];
        R.sc[1] = v[1];
    }
}

template <int FMT, bool DQ>
__device__ __forceinline__ void stream_band_res(const KArgs& a, int64_t band, int64_t KT, BufRes& rc, BufRes& rs) {
    constexpr int SB = tile_scale_bytes<FMT, DQ>();
    rc = buf_res(a.codes + band * KT * kTileBytes, (uint32_t)(KT * kTileBytes));
    rs = buf_res(a.scales + band * KT * SB, (uint32_t)(KT * SB));
}

// The per-band values of this lane's column: bias and the double-quant group scales.
template <int FMT, bool DQ>
__device__ __forceinline__ void stream_load_band_consts(StreamBand& B, const KArgs& a, int64_t band, int r) {
    const int64_t col = band * 16 + r;
    B.braw = a.bias ? (uint32_t)a.bias[col] : 0u;
    if constexpr (FMT == kNF4 && DQ) {
        const int64_t nbr = a.k / 64;                 // blocks per row
        const int64_t b0 = col * nbr;                 // first block of the row
        const int64_t gA = b0 >> 8, gB = (b0 + nbr - 1) >> 8;
        const float* dt = reinterpret_cast<const float*>(a.scales + a.d_off);
        B.dA = dt[gA];
        B.dB = dt[gB];
        B.jt = (int32_t)((gA + 1) * 256 - b0);
    }
}

template <int FMT, bool DQ, int T>
__device__ __forceinline__ void stream_load_band(StreamTile (&R)[T], StreamBand& B, const KArgs& a, int64_t band,
                                                 int lane, int r, int64_t KT) {
    BufRes rc, rs;
    stream_band_res<FMT, DQ>(a, band, KT, rc, rs);
#pragma unroll
    for (int s = 0; s < T; s++) stream_load_tile<FMT, DQ>(R[s], rc, rs, s, lane, r);
    stream_load_band_consts<FMT, DQ>(B, a, band, r);
}

// Consume band `band` from R and B.  REFILL: as soon as tile s has been used, its
// registers request tile s of band `next`, and B is reloaded for `next` after the
// outputs (otherwise the caller requests whole bands).
template <int FMT, bool DQ, int NI, int T, bool REFILL>
__device__ __forceinline__ void stream_band(StreamTile (&R)[T], StreamBand& B, const KArgs& a, int64_t band,
                                            int64_t next, const uint16_t* xrow, const uint16_t* xzero, int h,
                                            int lane, int r, uint32_t lane4, const uint32_t* lut, float mu, float g,
                                            int64_t KT) {
    constexpr int TK = tile_k(FMT);
    BufRes rc, rs;
    if constexpr (REFILL) stream_band_res<FMT, DQ>(a, next, KT, rc, rs);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < T; s++) {
        {
            GemvTile<FMT> t;
            t.code = make_uint4(R[s].code[0], R[s].code[1], R[s].code[2], R[s].code[3]);
            t.sc[0] = R[s].sc[0];
            t.sc[1] = R[s].sc[1];
            if constexpr (FMT == kNF4 && DQ) {
                t.sc[1] = __float_as_uint(2 * s < B.jt ? B.dA : B.dB);
                t.sc[2] = __float_as_uint(2 * s + 1 < B.jt ? B.dA : B.dB);
            }
            // rows r >= m read row 0: their products only reach output rows that are never stored
            const uint16_t* xp = s < KT ? xrow + s * TK : xzero;
#pragma unroll
            for (int j = 0; j < TK / 32; j++) {
                const uint4 v = *reinterpret_cast<const uint4*>(xp + 32 * j);
                t.A[j] = u32x4{v.x, v.y, v.z, v.w};
            }
            gemv_consume<FMT, DQ, NI>(t, acc, lut, lane4, h, mu);
        }
        if constexpr (REFILL) stream_load_tile<FMT, DQ>(R[s], rc, rs, s, lane, r);
        __builtin_amdgcn_sched_barrier(0);   // keep tiles in order: bounded register use
    }
    // lane (h, r) holds rows 4h .. 4h+3 of column band * 16 + r
    ColOut c = gemv_col_out(a, band * 16 + (__lane_id() & 15));
    c.bias = bf16_value((uint16_t)B.braw);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int mm = 4 * h + i;
        if (mm < a.m) put_out(a, c, mm, acc[i], g);
    }
    if constexpr (REFILL) stream_load_band_consts<FMT, DQ>(B, a, next, r);
}

// Tile-by-tile refill for the one-token NF4 double-quant kernel, where it keeps more
// requests in flight within the same registers; the other variants request whole
// bands (the refill order costs them registers: spills for q4_0 and four-row tiles).
template <int FMT, bool DQ, int NI>
constexpr bool stream_refill() { return FMT == kNF4 && DQ && NI == 1; }

// Each wave keeps two bands in two register sets.  With the refill order a set is
// refilled tile by tile while it is consumed (between one and two bands of requests in
// flight per wave); otherwise the next band's set is requested before the current one
// is consumed.  Prefetch indices past the end are clamped to the last band (in-bounds
// re-reads).
template <int FMT, bool DQ, int NI, int T>
__global__ __launch_bounds__(256, 2) void k_gemv_stream(KArgs a) {
    __shared__ uint32_t lut[gemv_uses_lut<FMT>() ? kLutWords : 1];
    __shared__ __attribute__((aligned(16))) uint16_t xs[kStreamXMax + 128];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int h = lane >> 4;
    const uint32_t lane4 = (uint32_t)lane << 2;
    const int64_t KT = a.k / tile_k(FMT);
    const int64_t nbands = a.n / 16;
    const int64_t stride = (int64_t)kStreamGrid * 4;   // waves of the grid (gemv_launch_ni)
    const int64_t last = nbands - 1;

    float g = 1.0f, mu = 0.0f;
    if constexpr (FMT == kNVFP4) g = load_f32_vmem(a.gs);
    if constexpr (FMT == kNF4 && DQ) mu = load_f32_vmem(a.scales + a.mu_off);

    int64_t band = (int64_t)blockIdx.x * 4 + wave;
    constexpr bool RF = stream_refill<FMT, DQ, NI>();
    StreamTile R0[T], R1[T];
    StreamBand B0, B1;
    stream_load_band<FMT, DQ, T>(R0, B0, a, std::min<int64_t>(band, last), lane, r, KT);
    // stage X (m rows of k bf16, rows contiguous in LDS) and the zero row
    if (tid < 16) *reinterpret_cast<uint4*>(xs + kStreamXMax + tid * 8) = make_uint4(0u, 0u, 0u, 0u);
    const int64_t nx = (int64_t)a.m * a.k;
    for (int64_t i = (int64_t)tid * 8; i < nx; i += 256 * 8) {
        const int64_t row = i / a.k, col = i - row * a.k;
        *reinterpret_cast<uint4*>(xs + i) = *reinterpret_cast<const uint4*>(a.x + row * a.ldx + col);
    }
    if constexpr (RF) stream_load_band<FMT, DQ, T>(R1, B1, a, std::min<int64_t>(band + stride, last), lane, r, KT);
    if constexpr (gemv_uses_lut<FMT>()) build_lut<FMT, 256>(lut);
    __syncthreads();
    const uint16_t* xrow = xs + (r < a.m ? r : 0) * a.k + h * 8;
    const uint16_t* xzero = xs + kStreamXMax + h * 8;

    for (; band < nbands; band += 2 * stride) {
        const int64_t b1 = std::min<int64_t>(band + stride, last), b2 = std::min<int64_t>(band + 2 * stride, last);
        if constexpr (!RF) stream_load_band<FMT, DQ, T>(R1, B1, a, b1, lane, r, KT);
        stream_band<FMT, DQ, NI, T, RF>(R0, B0, a, band, b2, xrow, xzero, h, lane, r, lane4, lut, mu, g, KT);
        if (band + stride >= nbands) break;
        if constexpr (!RF) stream_load_band<FMT, DQ, T>(R0, B0, a, b2, lane, r, KT);
        stream_band<FMT, DQ, NI, T, RF>(R1, B1, a, band + stride, std::min<int64_t>(band + 3 * stride, last), xrow,
                                        xzero, h, lane, r, lane4, lut, mu, g, KT);
    }
}

// ---------------------------------------------------------------------------
// Chunked streaming GEMV: the same scheme for every format whose band does not fit one
// register set (q8_0's 64-wide tiles, K beyond 10 tiles) or whose scale records are wider
// (q4_1, q5_0, q4_k, q6_k).  A wave walks items (band, chunk): a chunk is T consecutive
// K tiles of a band, the accumulator runs across a band's chunks and the band's outputs
// are stored after its last one.  The next item's tiles are requested into the other
// register set before the current item is consumed.  Each chunk's requests go through
// buffer descriptors that cover exactly its tiles (slots past the band's K read zeros
// and take the zero row of X).
// ---------------------------------------------------------------------------
struct StreamChunkTile {
    u32x4 code;
    uint32_t sc[6];
};

struct StreamChunk {
    uint32_t braw;     // bias (bf16 bits) of this lane's column
};

template <int FMT, bool DQ, int T>
__device__ __forceinline__ void stream_load_chunk(StreamChunkTile (&R)[T], StreamChunk& B, const KArgs& a,
                                                  int64_t band, int64_t t0, int64_t KT, int lane, int r) {
    constexpr int SB = tile_scale_bytes<FMT, DQ>();
    const int64_t tile0 = band * KT + t0;
    const uint32_t nt = (uint32_t)std::min<int64_t>(T, KT - t0);
    const BufRes rc = buf_res(a.codes + tile0 * kTileBytes, nt * (uint32_t)kTileBytes);
    const BufRes rs = buf_res(a.scales + tile0 * SB, nt * (uint32_t)SB);
    BufRes rh = rs, rk = rs;                      // (replaced below for the formats that use them)
    if constexpr (FMT == kQ5_0) rh = buf_res(a.scales + a.hb_off + tile0 * 256, nt * 256u);
    if constexpr (FMT == kQ6_K) rh = buf_res(a.codes + a.n * a.k / 2 + tile0 * 512, nt * 512u);
    // the band's rows of super-block scales: (d, dmin) fp16 pairs (q4_k) or fp16 d (q6_k)
    constexpr int KS = FMT == kQ4_K ? 4 : 2;
    const int64_t spr = a.k >> 8;                 // super-blocks per row
    if constexpr (FMT == kQ4_K || FMT == kQ6_K) rk = buf_res(a.scales + a.kd_off + band * 16 * spr * KS, (uint32_t)(16 * spr * KS));
#pragma unroll
    for (int s = 0; s < T; s++) {
        R[s].code = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, lane * 16 + s * kTileBytes, 0, kNT));
        if constexpr (FMT == kQ8_0) {
            R[s].sc[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, r * 4 + s * SB, 0, kNT);
        } else if constexpr (FMT == kQ4_1) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, r * 16 + s * SB, 0, kNT);
#pragma unroll
            for (int i = 0; i < 4; i++) R[s].sc[i] = v[i];
        } else {
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, r * 8 + s * SB, 0, kNT);
            R[s].sc[0] = v[0];
            R[s].sc[1] = v[1];
        }
        if constexpr (FMT == kQ5_0) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rh, r * 16 + s * 256, 0, kNT);
#pragma unroll
            for (int i = 0; i < 4; i++) R[s].sc[2 + i] = v[i];
        }
        if constexpr (FMT == kQ6_K) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(rh, lane * 8 + s * 512, 0, kNT);
            R[s].sc[2] = v[0];
            R[s].sc[3] = v[1];
            // the tile's super-block (slots past the band's K read a valid neighbour: their A is zero)
            const uint32_t sb = (uint32_t)std::min<int64_t>((t0 + s) >> 1, spr - 1);
            R[s].sc[4] = __builtin_amdgcn_raw_buffer_load_b16(rk, (uint32_t)((r * spr + sb) * 2), 0, 0);
        }
        if constexpr (FMT == kQ4_K) {
            const uint32_t sb = (uint32_t)std::min<int64_t>((t0 + s) >> 1, spr - 1);
            R[s].sc[2] = __builtin_amdgcn_raw_buffer_load_b32(rk, (uint32_t)((r * spr + sb) * 4), 0, 0);
        }
    }
    B.braw = a.bias ? (uint32_t)a.bias[band * 16 + r] : 0u;
}

template <int FMT, bool DQ, int NI, int T>
__device__ __forceinline__ void stream_consume_chunk(const StreamChunkTile (&R)[T], f32x4& acc, int64_t t0,
                                                     int64_t KT, const uint16_t* xrow, const uint16_t* xzero,
                                                     int h, uint32_t lane4, const uint32_t* lut, float mu) {
    constexpr int TK = tile_k(FMT);
#pragma unroll
    for (int s = 0; s < T; s++) {
        {
            GemvTile<FMT> t;
            t.code = make_uint4(R[s].code[0], R[s].code[1], R[s].code[2], R[s].code[3]);
#pragma unroll
            for (int i = 0; i < 6; i++) t.sc[i] = R[s].sc[i];
            // rows r >= m read row 0: their products only reach output rows that are never stored
            const uint16_t* xp = t0 + s < KT ? xrow + (t0 + s) * TK : xzero;
#pragma unroll
            for (int j = 0; j < TK / 32; j++) {
                const uint4 v = *reinterpret_cast<const uint4*>(xp + 32 * j);
                t.A[j] = u32x4{v.x, v.y, v.z, v.w};
            }
            gemv_consume<FMT, DQ, NI>(t, acc, lut, lane4, h, mu);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep tiles in order: bounded register use
    }
}

template <int FMT, bool DQ, int NI, int T>
__global__ __launch_bounds__(256, 2) void k_gemv_stream_chunked(KArgs a) {
    static_assert(!(FMT == kNF4 && DQ), "double quant streams through k_gemv_stream");
    __shared__ uint32_t lut[gemv_uses_lut<FMT>() ? kLutWords : 1];
    __shared__ __attribute__((aligned(16))) uint16_t xs[kStreamXMax + 128];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int h = lane >> 4;
    const uint32_t lane4 = (uint32_t)lane << 2;
    const int64_t KT = a.k / tile_k(FMT);
    const int64_t nch = (KT + T - 1) / T;          // chunks per band
    const int64_t nbands = a.n / 16;
    const int64_t stride = (int64_t)kStreamGrid * 4;   // waves of the grid (gemv_launch_ni)
    const int64_t band0 = (int64_t)blockIdx.x * 4 + wave;
    // this wave's items: bands band0, band0 + stride, ..., each of nch chunks; requests for
    // items past the last one re-read the wave's last item (in bounds, never consumed)
    const int64_t nitems = band0 < nbands ? ((nbands - 1 - band0) / stride + 1) * nch : 0;
    const int64_t ilast = nitems > 0 ? nitems - 1 : 0;
    auto item_band = [&](int64_t i) { return std::min<int64_t>(band0 + (std::min(i, ilast) / nch) * stride, nbands - 1); };
    auto item_t0 = [&](int64_t i) { return (std::min(i, ilast) % nch) * T; };

    float g = 1.0f, mu = 0.0f;
    if constexpr (FMT == kNVFP4) g = load_f32_vmem(a.gs);

    StreamChunkTile R0[T], R1[T];
    StreamChunk B0, B1;
    stream_load_chunk<FMT, DQ, T>(R0, B0, a, item_band(0), item_t0(0), KT, lane, r);
    // stage X (m rows of k bf16, rows contiguous in LDS) and the zero row
    if (tid < 16) *reinterpret_cast<uint4*>(xs + kStreamXMax + tid * 8) = make_uint4(0u, 0u, 0u, 0u);
    const int64_t nx = (int64_t)a.m * a.k;
    for (int64_t i = (int64_t)tid * 8; i < nx; i += 256 * 8) {
        const int64_t row = i / a.k, col = i - row * a.k;
        *reinterpret_cast<uint4*>(xs + i) = *reinterpret_cast<const uint4*>(a.x + row * a.ldx + col);
    }
    if constexpr (gemv_uses_lut<FMT>()) build_lut<FMT, 256>(lut);
    __syncthreads();
    const uint16_t* xrow = xs + (r < a.m ? r : 0) * a.k + h * 8;
    const uint16_t* xzero = xs + kStreamXMax + h * 8;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // the band's outputs, after its last chunk: lane (h, r) holds rows 4h .. 4h+3 of column band * 16 + r
    auto finish = [&](int64_t i, uint32_t braw) {
        if (i % nch != nch - 1) return;
        ColOut c = gemv_col_out(a, item_band(i) * 16 + r);
        c.bias = bf16_value((uint16_t)braw);
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int mm = 4 * h + q;
            if (mm < a.m) put_out(a, c, mm, acc[q], g);
        }
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    for (int64_t i = 0; i < nitems; i += 2) {
        stream_load_chunk<FMT, DQ, T>(R1, B1, a, item_band(i + 1), item_t0(i + 1), KT, lane, r);
        stream_consume_chunk<FMT, DQ, NI, T>(R0, acc, item_t0(i), KT, xrow, xzero, h, lane4, lut, mu);
        finish(i, B0.braw);
        if (i + 1 >= nitems) break;
        stream_load_chunk<FMT, DQ, T>(R0, B0, a, item_band(i + 2), item_t0(i + 2), KT, lane, r);
        stream_consume_chunk<FMT, DQ, NI, T>(R1, acc, item_t0(i + 1), KT, xrow, xzero, h, lane4, lut, mu);
        finish(i + 1, B1.braw);
    }
}

// Tiles per chunk of the chunked streaming kernel.  Measured on the 433 MB streaming
// shape (K = 1280): 10-tile chunks for q8_0 and q4_1 (q4_1 4.2 -> 4.7 TB/s against 5);
// q5_0, q4_k and q6_k, whose per-value decode is longest, gain nothing from 10 and keep 5
// (8 leaves a 2-tile second chunk and loses a quarter).  q4_0 with four-row accumulators
// would spill at 10.
template <int FMT, int NI>
constexpr int stream_chunk_tiles() {
    return (FMT == kQ5_0 || FMT == kQ4_K || FMT == kQ6_K || (FMT == kQ4_0 && NI == 4)) ? 5 : 10;
}

constexpr int64_t kStreamMinBands = 4 * 2 * 4 * kNumCU;   // bands per wave x waves

size_t gemv_workspace_bytes(int, int64_t, int64_t, int64_t) { return 0; }

size_t matmul_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k) {
    return m <= 16 ? gemv_workspace_bytes(fmt, m, n, k) : gemm_workspace_bytes(fmt, m, n, k);
}

// Tiles per wave per round: the smallest offered count covering the band's K
// range in one round (K <= 64 tiles), else rounds of 8.
static int gemv_chunk(int64_t KT) {
    const int64_t pw = (KT + kGemvWaves - 1) / kGemvWaves;
    return pw <= 1 ? 1 : pw <= 2 ? 2 : pw <= 4 ? 4 : pw <= 5 ? 5 : 8;
}

constexpr int64_t kGemvXlMax = 32768;   // bf16 elements of X (m * k) copied to LDS by the decode GEMV

// Two workgroups per CU for the small-C kernels (<= 128 VGPRs) when their LDS fits twice:
// with a code table, an X copy of at most 8 KiB; without one, the reduction buffer and the
// X copy twice in the CU's 160 KiB.
template <int FMT, int C>
static bool gemv_two_per_cu(size_t xbytes) {
    constexpr size_t kLdsPerCu = 160 * 1024;
    const size_t red = sizeof(f32x4) * kGemvWaves * 64;
    if (C > 2) return false;
    return gemv_uses_lut<FMT>() ? xbytes <= 8192 : 2 * (red + 16 + xbytes) <= kLdsPerCu;
}

template <int FMT, bool DQ, int NI, int C, bool XL>
static void gemv_launch_cx(const KArgs& a, int64_t nbands, int64_t KT, hipStream_t st) {
    const dim3 block(64 * kGemvWaves);
    const size_t xbytes = XL ? (size_t)a.m * (size_t)a.k * 2 : 0;
    const int64_t per_cu = gemv_two_per_cu<FMT, C>(xbytes) ? 2 : 1;
    // band pipelining only where its two register sets fit without spilling (C <= 2), and only
    // when the bands outnumber the workgroups that fit at once
    if constexpr (C <= 2) {
        const int64_t resident = per_cu * (int64_t)kNumCU;
        if (nbands > resident && (KT + kGemvWaves - 1) / kGemvWaves <= C) {
            KArgs b = a;
            b.wg_per_cu = (uint8_t)per_cu;
            hipLaunchKernelGGL((k_gemv<FMT, DQ, NI, C, true, XL>), dim3((unsigned)resident), block, xbytes, st, b);
            return;
        }
    }
    hipLaunchKernelGGL((k_gemv<FMT, DQ, NI, C, false, XL>), dim3((unsigned)nbands), block, xbytes, st, a);
}

// The LDS copy of X is used when it is small enough, when every band gets its own workgroup
// (no band pipelining: its per-band barriers would wait for the prefetched band's loads), and
// when it either keeps two workgroups per CU (<= 8 KiB) or the bands fit one per CU anyway.
template <int FMT, bool DQ, int NI, int C>
static void gemv_launch_c(const KArgs& a, int64_t nbands, int64_t KT, hipStream_t st) {
    const int64_t mk = (int64_t)a.m * a.k;
    // The X copy when all bands run in one round of resident workgroups.  The table formats
    // fit one workgroup per CU with a larger copy; from 12 tokens on, the copy with two bands
    // pipelined per workgroup beats reading 12-16 rows of X from L2 per tile (measured at the
    // fc1 shape, 320 bands: 8 tokens 5.3 vs 5.4 us, 12 tokens 6.1 vs 5.7, 16 tokens 6.7 vs 6.1).
    const bool xl = mk <= kGemvXlMax && nbands <= 2 * kNumCU &&
                    (mk * 2 <= 8192 || nbands <= kNumCU || (!gemv_uses_lut<FMT>() && gemv_two_per_cu<FMT, C>((size_t)mk * 2)) ||
                     (gemv_uses_lut<FMT>() && C <= 2 && a.m >= 12));
    if (xl) gemv_launch_cx<FMT, DQ, NI, C, true>(a, nbands, KT, st);
    else gemv_launch_cx<FMT, DQ, NI, C, false>(a, nbands, KT, st);
}

template <int FMT, bool DQ, int NI>
static void gemv_launch_ni(const KArgs& a, hipStream_t st) {
    const int64_t KT = a.k / tile_k(FMT);
    const int64_t nbands = a.n / 16;
    // Many more bands than resident waves and X fits in LDS: the streaming kernels (two
    // workgroups of 4 waves per CU, each wave >= 4 bands); the chunked one for wider scale
    // records and for K beyond 10 tiles (double quant with K beyond 10 tiles takes the
    // general kernel).
    if (nbands >= kStreamMinBands && (int64_t)a.m * a.k <= kStreamXMax) {
        const unsigned grid = kStreamGrid;
        constexpr bool wide = FMT == kQ4_1 || FMT == kQ5_0 || FMT == kQ4_K || FMT == kQ6_K;
        if constexpr (!wide) {
            if (KT <= 4) {
                hipLaunchKernelGGL((k_gemv_stream<FMT, DQ, NI, 4>), dim3(grid), dim3(256), 0, st, a);
                return;
            }
            if (KT <= 10) {
                hipLaunchKernelGGL((k_gemv_stream<FMT, DQ, NI, 10>), dim3(grid), dim3(256), 0, st, a);
                return;
            }
        }
        // wider scale records, or K beyond one register set: chunks of T tiles
        if constexpr (!(FMT == kNF4 && DQ)) {
            hipLaunchKernelGGL((k_gemv_stream_chunked<FMT, DQ, NI, stream_chunk_tiles<FMT, NI>()>), dim3(grid), dim3(256), 0, st, a);
            return;
        }
    }
    switch (gemv_chunk(KT)) {
    case 1: gemv_launch_c<FMT, DQ, NI, 1>(a, nbands, KT, st); break;
    case 2: gemv_launch_c<FMT, DQ, NI, 2>(a, nbands, KT, st); break;
    case 4: gemv_launch_c<FMT, DQ, NI, 4>(a, nbands, KT, st); break;
    case 5: gemv_launch_c<FMT, DQ, NI, 5>(a, nbands, KT, st); break;
    default: gemv_launch_c<FMT, DQ, NI, 8>(a, nbands, KT, st); break;
    }
}

template <int FMT, bool DQ>
static void gemv_dispatch_ni(const KArgs& a, hipStream_t st) {
    // one token updates one accumulator row per lane; more tokens update all four
    if (a.m == 1) gemv_launch_ni<FMT, DQ, 1>(a, st);
    else gemv_launch_ni<FMT, DQ, 4>(a, st);
}

hipError_t launch_gemv(const MatmulProblem& p, hipStream_t st) {
    const KArgs a = make_args(p);
    switch (p.fmt) {
    case kNF4:
        if (p.dq) gemv_dispatch_ni<kNF4, true>(a, st);
        else gemv_dispatch_ni<kNF4, false>(a, st);
        break;
    case kNVFP4: gemv_dispatch_ni<kNVFP4, false>(a, st); break;
    case kQ4_0: gemv_dispatch_ni<kQ4_0, false>(a, st); break;
    case kQ4_1: gemv_dispatch_ni<kQ4_1, false>(a, st); break;
    case kQ5_0: gemv_dispatch_ni<kQ5_0, false>(a, st); break;
    case kQ4_K: gemv_dispatch_ni<kQ4_K, false>(a, st); break;
    case kQ6_K: gemv_dispatch_ni<kQ6_K, false>(a, st); break;
    case kQ8_0: gemv_dispatch_ni<kQ8_0, false>(a, st); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace wq
