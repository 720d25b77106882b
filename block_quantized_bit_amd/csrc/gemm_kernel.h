// gemm_kernel.h -- the encoder GEMM kernels (m >= 17) on bf16 MFMA and the K-split
// reduction, shared by the translation units that instantiate and launch them
// (gemm.hip, gemm_nvfp4_wide.hip).
#pragma once

#include "mm_common.h"

namespace wq {

// ===========================================================================
// GEMM, m >= 17.  Workgroup tile 128 (M) x 256 (N), K step 128; wave w owns
// columns [64w, 64w+64) (4 bands) for all 128 rows: 8 x 4 MFMA tiles of 16x16.
// Two-stage pipeline: the X tile (LDS, filled by LDS-direct loads) and W codes/
// scales (registers) of step s+1 are requested at the start of step s and are
// waited for at the one workgroup synchronization of step s, after three of its
// four 32-wide K slices.  Requests are unconditional (rows past m and bands past
// n re-read valid rows, steps past the end re-read the last step; none of those
// results is stored).  The K slices are software-pipelined across steps: the A
// fragments and dequantized B fragments of the next slice (in the last slice,
// the next step's first) are produced while the MFMAs of the current slice run,
// and the schedule interleaves MFMA, VALU and LDS instructions explicitly.
// LDS: the fp32 code table (NF4), then two X tiles.
// ===========================================================================
// A tile is BM rows by 64 * NB columns: wave w owns bands NB w .. NB w + NB - 1 (NB = 4: 128 x 256
// tiles; NB = 2: 128 x 128 tiles for shapes whose wide tiles cannot fill the chip).
constexpr int BM = 128, BK = 128;
constexpr int kLutBytes = kLutWords * 4;
constexpr int kXsBytes = BM * BK * 2;      // one X tile: 128 rows x 256 B, 16-byte chunks XOR-swizzled by row

template <int FMT>
__device__ constexpr bool gemm_uses_lut() { return FMT == kNF4; }

template <int FMT>
struct GemmW {
    uint4 code[tile_k(FMT) == 64 ? 2 : 1];
    uint32_t sc[6];
};

// Buffer descriptors of one workgroup's loads: per band of the wave (its
// tiles, its scales), the double-quant group scales, and X from row m0 on.
// All wave-uniform, so every offset that changes with the K step is scalar.
struct GemmSrc {
    const uint8_t* code[4];     // first tile of each band
    const uint8_t* scale[4];    // scales of that tile
    uint32_t wbytes, sbytes;    // one band's codes / scales
    const uint8_t* dt;          // double-quant group scales
    uint32_t dtbytes;
    const uint8_t* hb[4];       // q5_0: fifth-bit words of the band's first tile; q4_k: the
    uint32_t hbbytes;           //   (d, dmin) pairs of the band's rows, row-major; q6_k: the
                                //   band's bit 4-5 records
    const uint8_t* kd[4];       // q6_k: the fp16 d of the band's rows, row-major
    uint32_t kdbytes;
    const uint8_t* x;           // X row m0
    uint32_t xbytes;
};

// Vector memory instructions gemm_load_w issues per band (the pipeline waits count them).
template <int FMT, bool DQ>
__device__ constexpr int gemm_w_loads() {
    return (FMT == kQ8_0 || FMT == kQ6_K) ? 4 : (FMT == kNF4 && DQ) ? 4 : (FMT == kQ5_0 || FMT == kQ4_K) ? 3 : 2;
}

// Codes and scales of K step st (one 16 x 128 tile, two 16 x 64 tiles for Q8_0) of band nf.
// rowblk: index of the first 64-value block of the lane's row (double quant only).
template <int FMT, bool DQ>
__device__ __forceinline__ void gemm_load_w(GemmW<FMT>& w, const GemmSrc& S, int nf, int64_t rowblk, int st,
                                            int lane, int r) {
    if constexpr (FMT == kQ8_0) {
#pragma unroll
        for (int half = 0; half < 2; half++) {
            const int t = 2 * st + half;
            w.code[half] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(buf_res_uni(S.code[nf], S.wbytes), lane * 16, uni(t * kTileBytes), 0));
            w.sc[half] = __builtin_amdgcn_raw_buffer_load_b32(buf_res_uni(S.scale[nf], S.sbytes), r * 4, uni(t * 64), 0);
        }
    } else {
        w.code[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(buf_res_uni(S.code[nf], S.wbytes), lane * 16, uni(st * kTileBytes), 0));
        if constexpr (FMT == kNF4 && DQ) {
            w.sc[0] = __builtin_amdgcn_raw_buffer_load_b16(buf_res_uni(S.scale[nf], S.sbytes), r * 2, uni(st * 32), 0);
            const int64_t b0 = rowblk + 2 * st;
            w.sc[1] = __builtin_amdgcn_raw_buffer_load_b32(buf_res_uni(S.dt, S.dtbytes), (uint32_t)(b0 >> 8) * 4u, 0, 0);
            w.sc[2] = __builtin_amdgcn_raw_buffer_load_b32(buf_res_uni(S.dt, S.dtbytes), (uint32_t)((b0 + 1) >> 8) * 4u, 0, 0);
        } else if constexpr (FMT == kQ6_K) {   // 8 int8 scales, the lane's bit 4-5 record, then d
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(buf_res_uni(S.scale[nf], S.sbytes), r * 8, uni(st * 128), 0);
            w.sc[0] = v[0];
            w.sc[1] = v[1];
            const auto hv = __builtin_amdgcn_raw_buffer_load_b64(buf_res_uni(S.hb[nf], S.hbbytes), lane * 8, uni(st * 512), 0);
            w.sc[2] = hv[0];
            w.sc[3] = hv[1];
            // row r's d values are S.kdbytes / 16 apart; step st is in super-block st / 2
            w.sc[4] = __builtin_amdgcn_raw_buffer_load_b16(buf_res_uni(S.kd[nf], S.kdbytes), r * (S.kdbytes >> 4),
                                                           uni((st >> 1) * 2), 0);
        } else if constexpr (FMT == kQ4_K) {   // record (4 sc, 4 m bytes), then the super-block's (d, dmin)
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(buf_res_uni(S.scale[nf], S.sbytes), r * 8, uni(st * 128), 0);
            w.sc[0] = v[0];
            w.sc[1] = v[1];
            // row r's pairs are S.hbbytes / 16 apart; step st is in super-block st / 2
            w.sc[2] = __builtin_amdgcn_raw_buffer_load_b32(buf_res_uni(S.hb[nf], S.hbbytes), r * (S.hbbytes >> 4),
                                                           uni((st >> 1) * 4), 0);
        } else if constexpr (FMT == kQ5_0) {   // 4 x fp16 d (8 bytes), 4 fifth-bit words (16 bytes)
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(buf_res_uni(S.scale[nf], S.sbytes), r * 8, uni(st * 128), 0);
            w.sc[0] = v[0];
            w.sc[1] = v[1];
            const uint4 hb = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(buf_res_uni(S.hb[nf], S.hbbytes), r * 16, uni(st * 256), 0));
            w.sc[2] = hb.x;
            w.sc[3] = hb.y;
            w.sc[4] = hb.z;
            w.sc[5] = hb.w;
        } else if constexpr (FMT == kQ4_1) {   // 4 x (fp16 d, fp16 m): 16 bytes per row and tile
            const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(buf_res_uni(S.scale[nf], S.sbytes), r * 16, uni(st * 256), 0));
            w.sc[0] = v.x;
            w.sc[1] = v.y;
            w.sc[2] = v.z;
            w.sc[3] = v.w;
        } else {   // NF4 (fp32 pair), Q4_0 (4 x fp16), NVFP4 (8 x E4M3): 8 bytes per row and tile
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(buf_res_uni(S.scale[nf], S.sbytes), r * 8, uni(st * 128), 0);
            w.sc[0] = v[0];
            w.sc[1] = v[1];
        }
    }
}

// B operand (bf16 of w^, one rounding) for K slice j of one band.  `hs` is
// 8 * (h >> 1): NVFP4 lanes of the upper half of a 32-wide slice use the
// second 16-value block's scale.
template <int FMT, bool DQ>
__device__ __forceinline__ u32x4 gemm_dequant(const GemmW<FMT>& w, int j, const uint32_t* lut, uint32_t lane8,
                                              uint32_t hs, float mu) {
    u32x4 B;
    if constexpr (FMT == kQ8_0) {
        const uint4 c = w.code[j >> 1];
        const uint32_t uw[4] = {c.x, c.y, c.z, c.w};
        const float d = f16_value((uint16_t)(w.sc[j >> 1] >> (16 * (j & 1))));
        const float d128 = -128.0f * d;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const uint32_t wv = uw[2 * (j & 1) + (q >> 1)] ^ 0x80808080u;   // q + 128 as unsigned bytes
            const int sh = 16 * (q & 1);
            const float f0 = (float)((wv >> sh) & 255u);
            const float f1 = (float)((wv >> (sh + 8)) & 255u);
            // (q+128)*d - 128*d == q*d exactly (19 significant bits); one rounding to bf16
            B[q] = pack_bf16_rne(__builtin_fmaf(f0, d, d128), __builtin_fmaf(f1, d, d128));
        }
    } else if constexpr (FMT == kNVFP4) {
        // block 2j + (h >> 1) of the tile row: byte (2j & 3) of the scale word shifted by hs
        const uint32_t sw = (j < 2 ? w.sc[0] : w.sc[1]) >> hs;
        const float s = (j & 1) ? __builtin_amdgcn_cvt_f32_fp8((int)sw, 2) : __builtin_amdgcn_cvt_f32_fp8((int)sw, 0);
        const uint32_t word = j == 0 ? w.code[0].x : j == 1 ? w.code[0].y : j == 2 ? w.code[0].z : w.code[0].w;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            // e2m1 pair of byte q (low nibble first), times the E4M3 scale: exact, so the bf16 rounding is exact too
            f32x2 v;
            if (q == 0) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0);
            else if (q == 1) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1);
            else if (q == 2) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2);
            else v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3);
            B[q] = pack_bf16_rne(__fmul_rn(v[0], s), __fmul_rn(v[1], s));
        }
    } else if constexpr (FMT == kQ4_1) {
        const uint32_t word = j == 0 ? w.code[0].x : j == 1 ? w.code[0].y : j == 2 ? w.code[0].z : w.code[0].w;
        B = q4_1_operand(word, w.sc[j]);
    } else if constexpr (FMT == kQ6_K) {
        // hs = 8 (h >> 1): K slice j spans sub-blocks 2j (h = 0, 1) and 2j + 1 (h = 2, 3)
        const uint32_t word = j == 0 ? w.code[0].x : j == 1 ? w.code[0].y : j == 2 ? w.code[0].z : w.code[0].w;
        const float Sj = q6_k_scale(w.sc[0], w.sc[1], w.sc[4], 2 * j + (int)(hs >> 3));
        const uint32_t hw = w.sc[2 + (j >> 1)] >> (16 * (j & 1));
        B = q6_k_operand(word, hw & 255u, (hw >> 8) & 255u, Sj);
    } else if constexpr (FMT == kQ4_K) {
        const uint32_t word = j == 0 ? w.code[0].x : j == 1 ? w.code[0].y : j == 2 ? w.code[0].z : w.code[0].w;
        float Sj, Oj;
        q4_k_sub(w.sc[0], w.sc[1], w.sc[2], j, Sj, Oj);
        B = q4_k_operand(word, Sj, Oj);
    } else if constexpr (FMT == kQ5_0) {
        // hs = 8 h for q5_0: this lane's k are bits 8h .. 8h+7 of block j's fifth-bit word
        const uint32_t word = j == 0 ? w.code[0].x : j == 1 ? w.code[0].y : j == 2 ? w.code[0].z : w.code[0].w;
        B = q5_0_operand(word, (w.sc[2 + j] >> hs) & 255u, (uint16_t)(w.sc[j >> 1] >> (16 * (j & 1))));
    } else if constexpr (FMT == kQ4_0) {
        // nibble c as a float, then c*d - 8d: both products are exact in fp32 (c has 4
        // significant bits, d 11), so this is (c - 8)*d exactly; one RNE to bf16
        const uint32_t word = j == 0 ? w.code[0].x : j == 1 ? w.code[0].y : j == 2 ? w.code[0].z : w.code[0].w;
        const float d = f16_value((uint16_t)(w.sc[j >> 1] >> (16 * (j & 1))));
        const float d8 = -8.0f * d;
        uint32_t lo = word & 0x0F0F0F0Fu, hi = (word >> 4) & 0x0F0F0F0Fu;
        // opaque to the optimizer, so that each byte converts with one v_cvt_f32_ubyteN
        // instead of a bit-field extract followed by a conversion
        asm("" : "+v"(lo), "+v"(hi));
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const float c0 = (float)((lo >> (8 * q)) & 255u);
            const float c1 = (float)((hi >> (8 * q)) & 255u);
            B[q] = pack_bf16_rne(__builtin_fmaf(c0, d, d8), __builtin_fmaf(c1, d, d8));
        }
    } else {   // NF4: code values from the LDS table
        const uint32_t word = j == 0 ? w.code[0].x : j == 1 ? w.code[0].y : j == 2 ? w.code[0].z : w.code[0].w;
        const int kb = j >> 1;
        float s;
        if constexpr (DQ) {
            s = __fadd_rn(__fmul_rn((float)(int8_t)((w.sc[0] >> (8 * kb)) & 255u), __uint_as_float(w.sc[1 + kb])), mu);
        } else {
            s = __uint_as_float(w.sc[kb]);
        }
#pragma unroll
        for (int q = 0; q < 4; q++) {
            // w^ = fl(code * scale) exactly as the format defines it, then one RNE to bf16
            const float2 pr = lut_pair_f32(lut, lane8, word, q);
            B[q] = pack_bf16_rne(__fmul_rn(pr.x, s), __fmul_rn(pr.y, s));
        }
    }
    return B;
}

template <int FMT, bool DQ, int NB>
__device__ __forceinline__ void gemm_load_w4(GemmW<FMT> (&w)[NB], const GemmSrc& S, const int64_t (&rowblk)[NB], int st,
                                             int lane, int r) {
#pragma unroll
    for (int nf = 0; nf < NB; nf++) gemm_load_w<FMT, DQ>(w[nf], S, nf, rowblk[nf], st, lane, r);
}

// X tile (128 x 128 bf16) global -> LDS without passing through registers.  In
// LDS, chunk c (16 bytes = 8 k) of tile row t sits at position c ^ (t & 15) of
// the row, so the 16 lanes of an A-fragment read (16 rows, one chunk) hit 16
// different bank groups.  Wave w fills rows 32w .. 32w+31, four rows per
// 64-lane instruction (8 instructions); xoff[i] is the lane's byte offset of
// its (row, chunk) at K step 0 -- rows past the matrix re-read its last row,
// whose results are never stored.
constexpr int kXLoads = 8;
__device__ __forceinline__ void gemm_load_x_lds(uint8_t* xs_buf, const GemmSrc& S, const uint32_t (&xoff)[kXLoads],
                                                int wave, int st) {
#pragma unroll
    for (int i = 0; i < kXLoads; i++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(buf_res_uni(S.x, S.xbytes), (__attribute__((address_space(3))) void*)(xs_buf + (wave * 32 + 4 * i) * 256),
                                                 16, xoff[i], uni(st * (BK * 2)), 0, 0);
}

// Bias of the lane's column in each of its NB bands (0 without a bias).  The loads are
// issued together and waited for once; bands past the matrix re-read band 0's value,
// which is never stored.
template <int NB>
__device__ __forceinline__ void gemm_bias(const KArgs& a, int64_t band0, int64_t nbands, int r, float (&bias)[NB]) {
    uint16_t raw[NB];
#pragma unroll
    for (int nf = 0; nf < NB; nf++) raw[nf] = 0;
    if (a.bias) {
#pragma unroll
        for (int nf = 0; nf < NB; nf++) raw[nf] = a.bias[(band0 + nf < nbands ? band0 + nf : 0) * 16 + r];
    }
#pragma unroll
    for (int nf = 0; nf < NB; nf++) bias[nf] = bf16_value(raw[nf]);
}

template <int FMT, bool DQ, int NB>
__device__ constexpr int gemm_step_loads() { return kXLoads + NB * gemm_w_loads<FMT, DQ>(); }

// A fragment of K slice j for rows 16 * mf + r: chunk 4j + h, stored at position (4j + h) ^ r.
__device__ __forceinline__ u32x4 gemm_load_a(const uint8_t* xcur, uint32_t arow, int mf, int j, int h, int r) {
    const uint4 t = *reinterpret_cast<const uint4*>(xcur + mf * 4096 + arow + ((uint32_t)((4 * j + h) ^ r) << 4));
    return u32x4{t.x, t.y, t.z, t.w};
}

template <int FMT, bool DQ, int NB>
__device__ __forceinline__ void gemm_dequant4(u32x4 (&B)[NB], const GemmW<FMT> (&w)[NB], int j, const uint32_t* lut,
                                              uint32_t lane8, uint32_t hs, float mu) {
#pragma unroll
    for (int nf = 0; nf < NB; nf++) B[nf] = gemm_dequant<FMT, DQ>(w[nf], j, lut, lane8, hs, mu);
}

// One K step: request step nx into (wn, xnext), compute the step held in
// (wc, xcur).  On entry A holds the A fragments of K slice 0 and B slice 0 of wc
// dequantized.  Slice j's 32 MFMAs run in row-fragment order; as soon as the four
// MFMAs of row fragment mf have issued, its register set is refilled with the
// next slice's fragment mf (8 A fragments live, not 16), and the next slice's B
// fragments are dequantized in between.
// The workgroup synchronizes once per step, after slice 2: by then every wave has
// read all of xcur (slice 3's fragments are read during slice 2), and waiting for
// all but the newest requests makes the following step's X tile (xfol) and W set
// (wf) complete.  Slice 3 then reads the following step's slice-0 A fragments and
// dequantizes its slice-0 B fragments (when `more`), so the next step starts
// with its operands in registers.  The next step's requests overwrite xcur's
// buffer only after this synchronization.
// half (q8_0 only; wave-uniform): the step holds only 64 K values (k an odd multiple of 64),
// and the MFMAs of K slices 2 and 3 are skipped.  Their loads past k read zeros (W, through the
// buffer range) or values of other columns (X), and never reach an MFMA.
template <int FMT, bool DQ, int NB, int NWAIT, bool MORE>
__device__ __forceinline__ void gemm_kstep(f32x4 (&acc)[8][NB], u32x4 (&A)[8], u32x4 (&B)[NB],
                                           const GemmW<FMT> (&wc)[NB], GemmW<FMT> (&wn)[NB], const GemmW<FMT> (&wf)[NB],
                                           const GemmSrc& S, const int64_t (&rowblk)[NB], const uint32_t (&xoff)[kXLoads],
                                           const uint8_t* xcur, uint8_t* xnext, const uint8_t* xfol, const uint32_t* lut,
                                           int nx, int wave, int lane, int r, int h, uint32_t lane8,
                                           uint32_t hs, float mu, bool half = false) {
    gemm_load_w4<FMT, DQ, NB>(wn, S, rowblk, nx, lane, r);
    gemm_load_x_lds(xnext, S, xoff, wave, nx);
    const uint32_t arow = (uint32_t)r * 256u;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        constexpr bool more = MORE;
        const bool refill = j < 3 || more;
        const uint8_t* asrc = j < 3 ? xcur : xfol;
        const int aslice = j < 3 ? j + 1 : 0;
        u32x4 Bn[NB];
        if (j < 3) gemm_dequant4<FMT, DQ, NB>(Bn, wc, j + 1, lut, lane8, hs, mu);
        else if (more) gemm_dequant4<FMT, DQ, NB>(Bn, wf, 0, lut, lane8, hs, mu);
#pragma unroll
        for (int mf = 0; mf < 8; mf++) {
#pragma unroll
            for (int nf = 0; nf < NB; nf++)
                if (FMT != kQ8_0 || j < 2 || !half) acc[mf][nf] = mfma(A[mf], B[nf], acc[mf][nf]);
            if (refill) A[mf] = gemm_load_a(asrc, arow, mf, aslice, h, r);
        }
        // 8 NB MFMAs, each followed by a share of the next slice's dequant; the A
        // refills follow the last MFMA of each row fragment, and in the first
        // slice the next step's loads are spread over the MFMAs too
        static_assert(gemm_step_loads<FMT, DQ, NB>() <= 8 * NB, "step loads spread one per MFMA");
#pragma unroll
        for (int i = 0; i < 8 * NB; i++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            // VALU share per MFMA: 2 for the byte-converting formats, 3 for NVFP4 / NF4 (measured)
            __builtin_amdgcn_sched_group_barrier(0x002, (FMT == kQ8_0 || FMT == kQ4_0 || FMT == kQ4_1) ? 2 : 3, 0);
            if (refill && (i % NB) == NB - 1) __builtin_amdgcn_sched_group_barrier(0x100, gemm_uses_lut<FMT>() ? 3 : 1, 0);
            if (j == 0 && i < gemm_step_loads<FMT, DQ, NB>()) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nf = 0; nf < NB; nf++) B[nf] = Bn[nf];
        if (j == 2) lds_barrier_vm<NWAIT>();
    }
}

template <int FMT, bool DQ, int NB>
__global__ __launch_bounds__(256, 1) void k_gemm(KArgs a) {
    constexpr int BN = 64 * NB;
    // separate LDS objects for the code table and the X buffers, so the
    // LDS-direct loads into one X buffer are never mistaken for writes to the others
    __shared__ __attribute__((aligned(16))) uint32_t lut_s[gemm_uses_lut<FMT>() ? kLutWords : 4];
    __shared__ __attribute__((aligned(16))) uint8_t xs0[kXsBytes];
    __shared__ __attribute__((aligned(16))) uint8_t xs1[kXsBytes];
    const uint32_t* lut = lut_s;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15;
    const int h = lane >> 4;
    const uint32_t lane8 = (uint32_t)(lane & 31) << 3;
    // NVFP4: byte of the scale word for this lane's 16-value block; q5_0: byte of the
    // fifth-bit word for this lane's 8 k
    const uint32_t hs = FMT == kQ5_0 ? 8u * (uint32_t)h : 8u * (uint32_t)(h >> 1);
    const int64_t M = a.m, N = a.n, K = a.k;
    constexpr int TK = tile_k(FMT);
    const int64_t KT = K / TK;
    // q8_0 k may be an odd multiple of 64: its last step is then half a step
    const int64_t nsteps_total = FMT == kQ8_0 ? (K + BK - 1) / BK : K / BK;

    // XCD-aware item order.  Workgroups are dealt to the 8 XCDs in turn, so XCD x
    // gets the consecutive items [x * per_xcd, (x + 1) * per_xcd).  Items run K piece
    // by K piece, and within a piece in groups of kGroupM row tiles by all column
    // tiles, column-major inside the group: the items an XCD runs at one time cover
    // a compact block of row and column tiles, whose X rows and W bands its L2 holds.
    // (the schedule of gemm_sched, derived here from the shape and the K-piece count)
    constexpr int64_t kGroupM = 6;
    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int64_t tiles = tiles_m * tiles_n;
    const int64_t items = tiles * a.ksplit;
    const int lks = __builtin_ctz((unsigned)a.ksplit);   // ksplit is a power of two (gemm_sched)
    const int64_t kt_per = ((K + BK - 1) / BK + a.ksplit - 1) >> lks;
    const int64_t per_xcd = (items + 7) / 8;     // the grid is per_xcd workgroups per XCD
    const int64_t item = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (item >= items) return;
    const int ks = (int)(item / tiles);
    const int64_t ti = item - (int64_t)ks * tiles;
    const int64_t grp = ti / (kGroupM * tiles_n);
    const int64_t gm = std::min<int64_t>(kGroupM, tiles_m - grp * kGroupM);
    const int64_t within = ti - grp * kGroupM * tiles_n;
    const int64_t tm = grp * kGroupM + within % gm;
    const int64_t tn = within / gm;
    const int64_t m0 = tm * BM, n0 = tn * BN;
    const int64_t s0 = ks * kt_per, s1 = std::min<int64_t>(nsteps_total, s0 + kt_per);  // in BK steps

    const int64_t band0 = n0 / 16 + wave * NB;
    const int64_t nbands = N / 16;

    float g = 1.0f, mu = 0.0f;
    if constexpr (FMT == kNVFP4) g = load_f32_vmem(a.gs);
    if constexpr (FMT == kNF4 && DQ) mu = load_f32_vmem(a.scales + a.mu_off);

    // descriptors: band tiles of this wave (bands past n re-read the last band), X rows m0 ..
    GemmSrc S;
    int64_t rowblk[NB];
    constexpr int SB = (FMT == kNF4 && DQ) ? 32 : (FMT == kQ8_0) ? 64 : (FMT == kQ4_1) ? 256 : 128;   // scale bytes per tile
#pragma unroll
    for (int nf = 0; nf < NB; nf++) {
        const int64_t band = std::min<int64_t>(band0 + nf, nbands - 1);
        S.code[nf] = a.codes + band * KT * kTileBytes;
        S.scale[nf] = a.scales + band * KT * SB;
        rowblk[nf] = (band * 16 + r) * (K / 64);
        if constexpr (FMT == kQ5_0) S.hb[nf] = a.scales + a.hb_off + band * KT * 256;
        if constexpr (FMT == kQ4_K) S.hb[nf] = a.scales + a.kd_off + band * 16 * (K / 256) * 4;
        if constexpr (FMT == kQ6_K) {
            S.hb[nf] = a.codes + N * K / 2 + band * KT * 512;
            S.kd[nf] = a.scales + a.kd_off + band * 16 * (K / 256) * 2;
        }
    }
    S.hbbytes = FMT == kQ4_K ? (uint32_t)(16 * (K / 256) * 4) : FMT == kQ6_K ? (uint32_t)(KT * 512) : (uint32_t)(KT * 256);
    S.kdbytes = (uint32_t)(16 * (K / 256) * 2);
    S.wbytes = (uint32_t)(KT * kTileBytes);
    S.sbytes = (uint32_t)(KT * SB);
    if constexpr (FMT == kNF4 && DQ) S.dt = a.scales + a.d_off;
    S.dtbytes = (uint32_t)(((N * (K / 64) + 255) / 256) * 4);   // double quant: one fp32 d per 256 blocks
    {
        const int64_t xbytes = (M - m0) * a.ldx * 2;
        S.x = reinterpret_cast<const uint8_t*>(a.x + m0 * a.ldx);
        S.xbytes = xbytes > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)xbytes;
    }
    uint32_t xoff[kXLoads];
#pragma unroll
    for (int i = 0; i < kXLoads; i++) {
        const int t = wave * 32 + 4 * i + (lane >> 4);                  // tile row of this lane
        const int c = (lane & 15) ^ (t & 15);                           // chunk it fetches
        const int64_t row = std::min<int64_t>(t, M - 1 - m0);
        xoff[i] = (uint32_t)(row * a.ldx * 2 + c * 16);
    }

    f32x4 acc[8][NB];
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
        for (int j = 0; j < NB; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // every K piece is non-empty (the schedule guarantees s0 < s1)
    const int first = (int)s0, last = (int)s1 - 1, end = (int)s1;
    const bool half_last = FMT == kQ8_0 && (K % BK) != 0 && end == nsteps_total;
    GemmW<FMT> w0[NB], w1[NB];
    gemm_load_w4<FMT, DQ, NB>(w0, S, rowblk, first, lane, r);
    gemm_load_x_lds(xs0, S, xoff, wave, first);
    if constexpr (gemm_uses_lut<FMT>()) build_lut_f32<FMT>(lut_s);
    wait_vm<0>();
    __syncthreads();
    u32x4 A[8], B[NB];
#pragma unroll
    for (int mf = 0; mf < 8; mf++) A[mf] = gemm_load_a(xs0, (uint32_t)r * 256u, mf, 0, h, r);
    gemm_dequant4<FMT, DQ, NB>(B, w0, 0, lut, lane8, hs, mu);

    // two buffer sets: step s reads (w[s%2], xs[s%2]) and requests step s + 1 into
    // the other set, whose previous contents were last read before the previous
    // step's synchronization.  Pairs of steps that both have a successor run in a
    // loop with a single exit; the last one or two steps follow it (whether a
    // step prefetches its successor is a compile-time property of each copy).
    int st = first;
    if constexpr (FMT == kQ8_0) {
        // q8_0 runs faster with four steps per iteration (measured); the others spill
        for (; st + 5 <= end; st += 4) {
            gemm_kstep<FMT, DQ, NB, 0, true>(acc, A, B, w0, w1, w1, S, rowblk, xoff, xs0, xs1, xs1, lut, st + 1,
                                         wave, lane, r, h, lane8, hs, mu);
            gemm_kstep<FMT, DQ, NB, 0, true>(acc, A, B, w1, w0, w0, S, rowblk, xoff, xs1, xs0, xs0, lut, st + 2,
                                         wave, lane, r, h, lane8, hs, mu);
            gemm_kstep<FMT, DQ, NB, 0, true>(acc, A, B, w0, w1, w1, S, rowblk, xoff, xs0, xs1, xs1, lut, st + 3,
                                         wave, lane, r, h, lane8, hs, mu);
            gemm_kstep<FMT, DQ, NB, 0, true>(acc, A, B, w1, w0, w0, S, rowblk, xoff, xs1, xs0, xs0, lut, st + 4,
                                         wave, lane, r, h, lane8, hs, mu);
        }
    }
    for (; st + 3 <= end; st += 2) {
        gemm_kstep<FMT, DQ, NB, 0, true>(acc, A, B, w0, w1, w1, S, rowblk, xoff, xs0, xs1, xs1, lut, st + 1,
                                     wave, lane, r, h, lane8, hs, mu);
        gemm_kstep<FMT, DQ, NB, 0, true>(acc, A, B, w1, w0, w0, S, rowblk, xoff, xs1, xs0, xs0, lut, st + 2,
                                     wave, lane, r, h, lane8, hs, mu);
    }
    if (st + 2 == end) {
        gemm_kstep<FMT, DQ, NB, 0, true>(acc, A, B, w0, w1, w1, S, rowblk, xoff, xs0, xs1, xs1, lut, last,
                                     wave, lane, r, h, lane8, hs, mu);
        gemm_kstep<FMT, DQ, NB, 0, false>(acc, A, B, w1, w0, w0, S, rowblk, xoff, xs1, xs0, xs0, lut, last,
                                      wave, lane, r, h, lane8, hs, mu, half_last);
    } else {
        gemm_kstep<FMT, DQ, NB, 0, false>(acc, A, B, w0, w1, w1, S, rowblk, xoff, xs0, xs1, xs1, lut, last,
                                      wave, lane, r, h, lane8, hs, mu, half_last);
    }
    wait_vm<0>();   // the last requests (re-reads of the last step) land before the workgroup ends

    // ---- epilogue ----
    // the bias of each of this lane's NB columns, all requested before the first wait
    float bias[NB];
    if (a.ksplit == 1) gemm_bias<NB>(a, band0, nbands, r, bias);
    if (a.ksplit == 1 && a.out_v16) {
        // The tile's bf16 results go through LDS (the X buffers are free once every
        // wave's loads have landed), so that each output row is written in whole
        // 128-byte pieces by 16-byte stores rather than in 32-byte fragments.
        // Wave w stages its 128 x 16 NB block (rows of RB bytes whose 16-byte chunks
        // are XOR-swizzled by row) and writes it back itself.
        constexpr int RB = 32 * NB, CH = 2 * NB;      // row bytes, 16-byte chunks per row
        __syncthreads();
        uint8_t* stg = (wave < 2 ? xs0 : xs1) + (wave & 1) * 16384;
        const int t = r & 3, q = r >> 2;
#pragma unroll
        for (int nf = 0; nf < NB; nf++) {
            if (band0 + nf >= nbands) continue;     // same for the whole wave
#pragma unroll
            for (int mf = 0; mf < 8; mf++) {
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; i++) v[i] = acc[mf][nf][i] * g + bias[nf];
                quad_transpose(v, t);   // now row 16 mf + 4h + t, columns 16 nf + 4q .. 4q + 3
                const int row = 16 * mf + 4 * h + t;
                const int ch = (2 * nf + (q >> 1)) ^ (row & (CH - 1));
                *reinterpret_cast<uint2*>(stg + row * RB + ch * 16 + (q & 1) * 8) =
                    make_uint2(pack_bf16_rne(v[0], v[1]), pack_bf16_rne(v[2], v[3]));
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
        const int c = lane & (CH - 1);
        const int64_t col = band0 * 16 + 8 * c;
        if (col < N) {
            const ColOut o = col_out_nobias<true>(a, col);
#pragma unroll
            for (int it = 0; it < 2 * CH; it++) {
                const int row = (64 / CH) * it + lane / CH;
                const uint4 v = *reinterpret_cast<const uint4*>(stg + row * RB + ((c ^ (row & (CH - 1))) << 4));
                // written once and not read again here: non-temporal
                if (m0 + row < M) __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(o.p + (m0 + row) * o.ld));
            }
        }
        return;
    }
    if (a.ksplit == 1) {
        const bool full = m0 + BM <= M;     // every row of the tile exists (all but the last row tile)
#pragma unroll
        for (int nf = 0; nf < NB; nf++) {
            if (band0 + nf >= nbands) continue;     // same for the whole wave
            ColOut c = col_out_nobias<true>(a, (band0 + nf) * 16 + r);
            c.bias = bias[nf];
            if (full) {
                // lane (h, r) owns rows 16 mf + 4h + i of its column: step through them by the row stride
                char* p = c.p + (m0 + 4 * h) * c.ld;
#pragma unroll
                for (int mf = 0; mf < 8; mf++) {
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; i++) v[i] = acc[mf][nf][i] * g + c.bias;
                    if (a.f32) {
#pragma unroll
                        for (int i = 0; i < 4; i++) *reinterpret_cast<float*>(p + i * c.ld) = v[i];
                    } else {
                        const uint32_t b01 = pack_bf16_rne(v[0], v[1]), b23 = pack_bf16_rne(v[2], v[3]);
                        *reinterpret_cast<uint16_t*>(p) = (uint16_t)b01;
                        *reinterpret_cast<uint16_t*>(p + c.ld) = (uint16_t)(b01 >> 16);
                        *reinterpret_cast<uint16_t*>(p + 2 * c.ld) = (uint16_t)b23;
                        *reinterpret_cast<uint16_t*>(p + 3 * c.ld) = (uint16_t)(b23 >> 16);
                    }
                    p += 16 * c.ld;
                }
            } else {
#pragma unroll
                for (int mf = 0; mf < 8; mf++)
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const int64_t mm = m0 + 16 * mf + 4 * h + i;
                        if (mm < M) put_out(a, c, mm, acc[mf][nf][i], g);
                    }
            }
        }
        return;
    }
    // K split: deposit this piece's partial tile; k_splitk_reduce_n finishes the outputs.
    // Staged through LDS like the bf16 output: wave w writes its 128 x 16 NB fp32 block in
    // two halves of 64 rows (rows of RB bytes with 16-byte chunks XOR-swizzled by row),
    // each row then leaving as one RB-byte piece.  The workspace is 16-byte aligned and
    // N % 16 == 0.
    constexpr int RB = 64 * NB, CH = 4 * NB;      // row bytes, 16-byte chunks per row
    __syncthreads();
    uint8_t* stg = (wave < 2 ? xs0 : xs1) + (wave & 1) * 16384;
    const int t = r & 3, q = r >> 2;
    const int c = lane & (CH - 1);
    const bool colok = band0 + (c >> 2) < nbands;
    float* const pbase = a.partial + ((int64_t)ks * M + m0) * N + band0 * 16 + 4 * c;
#pragma unroll
    for (int half = 0; half < 2; half++) {
#pragma unroll
        for (int nf = 0; nf < NB; nf++) {
#pragma unroll
            for (int mh = 0; mh < 4; mh++) {
                const int mf = 4 * half + mh;
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; i++) v[i] = acc[mf][nf][i];
                quad_transpose(v, t);   // now row 16 mf + 4h + t, columns 16 nf + 4q .. 4q + 3
                const int row = 16 * mh + 4 * h + t;
                *reinterpret_cast<f32x4*>(stg + row * RB + (((4 * nf + q) ^ (row & (CH - 1))) << 4)) =
                    f32x4{v[0], v[1], v[2], v[3]};
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int it = 0; it < CH; it++) {
            const int row = (64 / CH) * it + lane / CH;
            const f32x4 v = *reinterpret_cast<const f32x4*>(stg + row * RB + ((c ^ (row & (CH - 1))) << 4));
            const int64_t mrow = 64 * half + row;
            if (colok && m0 + mrow < M) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(pbase + mrow * N));
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
}

// Split-K reduce.  Its launch carries everything in the one argument line: the pieces'
// fp32 partials [ksplit][m][n] in the codes slot (rpartial) and the address of the
// epilogue factor in the scales slot (rfactor: the NVFP4 global scale, W4A4's g_w * g_x,
// or null for 1).  Thread t of workgroup b owns the Q quads (4 consecutive columns of
// one row) b * 256 Q + t + 256 i.  Every memory request of a thread -- its partials, the
// factor and its bias values -- is issued before its first wait.
constexpr int kRedQ = 2;   // quads per thread (four measured 0.7-1 us slower on the M = 1500 fc2 shape)

struct RedQuad {
    int64_t row, col0;
    bool live;
};

// Row and first column of quad q; 32-bit arithmetic when every quad index fits.
__device__ inline RedQuad red_quad(int64_t q, int64_t total, int64_t nq, bool small) {
    RedQuad r;
    r.live = q < total;
    if (!r.live) q = 0;
    if (small) {
        const uint32_t m32 = (uint32_t)q / (uint32_t)nq;
        r.row = m32;
        r.col0 = (int64_t)((uint32_t)q - m32 * (uint32_t)nq) * 4;
    } else {
        r.row = q / nq;
        r.col0 = (q - r.row * nq) * 4;
    }
    return r;
}

// The 4 bias values of the quad at column col0 as fp32 (one 8-byte load when aligned).
struct RedBias {
    uint32_t lo, hi;
};
__device__ inline RedBias red_bias_load(const uint16_t* bias, int64_t col0, bool al8) {
    RedBias b{0u, 0u};
    if (al8) {
        const uint2 v = *reinterpret_cast<const uint2*>(bias + col0);
        b.lo = v.x;
        b.hi = v.y;
    } else {
        b.lo = (uint32_t)bias[col0] | ((uint32_t)bias[col0 + 1] << 16);
        b.hi = (uint32_t)bias[col0 + 2] | ((uint32_t)bias[col0 + 3] << 16);
    }
    return b;
}

// y = v * g + bias for one quad, converted and stored (global stores, as in put_out).
typedef __attribute__((address_space(1))) f32x4 gf32x4_t;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) u32x2 gu32x2_t;
__device__ inline void red_store(const KArgs& a, const RedQuad& q, const f32x4& v, float g, const RedBias& b) {
    const float bv[4] = {lo_f(b.lo), hi_f(b.lo), lo_f(b.hi), hi_f(b.hi)};
    if (a.out_vec) {
        // the 4 columns lie in one output split and can be written with one store
        const ColOut c = col_out_nobias<true>(a, q.col0);
        float o[4];
#pragma unroll
        for (int u = 0; u < 4; u++) o[u] = v[u] * g + bv[u];
        char* const p = c.p + q.row * c.ld;
        if (a.f32)
            *(gf32x4_t*)p = f32x4{o[0], o[1], o[2], o[3]};
        else
            *(gu32x2_t*)p = u32x2{(uint32_t)bf16_rne(o[0]) | ((uint32_t)bf16_rne(o[1]) << 16),
                                  (uint32_t)bf16_rne(o[2]) | ((uint32_t)bf16_rne(o[3]) << 16)};
        return;
    }
#pragma unroll
    for (int u = 0; u < 4; u++) {
        ColOut c = col_out_nobias<true>(a, q.col0 + u);
        c.bias = bv[u];
        put_out(a, c, q.row, v[u], g);
    }
}

// KS pieces (2 or 4), or a.ksplit of them (KS = 0), summed in order 0, 1, ...
template <int KS>
__global__ __launch_bounds__(256) void k_splitk_reduce_n(KArgs a) {
    constexpr int Q = kRedQ;
    const int64_t nq = a.n / 4;
    const int64_t total = (int64_t)a.m * nq;
    const int64_t q0 = (int64_t)blockIdx.x * (256 * Q) + threadIdx.x;
    if (q0 >= total) return;
    const bool small = total <= 0x7FFFFFFF;
    const int64_t pstride = (int64_t)a.m * a.n;
    const float* const partial = a.rpartial;
    RedQuad qd[Q];
#pragma unroll
    for (int i = 0; i < Q; i++) qd[i] = red_quad(q0 + 256 * i, total, nq, small);   // quads past the end re-read quad 0
    f32x4 v[Q];
    if constexpr (KS > 0) {
        f32x4 t[KS][Q];
#pragma unroll
        for (int i = 0; i < Q; i++) {
#pragma unroll
            for (int s = 0; s < KS; s++)
                t[s][i] = __builtin_nontemporal_load(
                    reinterpret_cast<const f32x4*>(partial + s * pstride + (qd[i].row * a.n + qd[i].col0)));
        }
#pragma unroll
        for (int i = 0; i < Q; i++) {
            v[i] = t[0][i];
#pragma unroll
            for (int s = 1; s < KS; s++) v[i] += t[s][i];
        }
    } else {
        // loads issued four pieces at a time (indices past the last piece re-read it and are dropped)
#pragma unroll
        for (int i = 0; i < Q; i++) v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < a.ksplit; s0 += 4) {
            f32x4 t[4][Q];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const int64_t off = std::min(s0 + u, a.ksplit - 1) * pstride;
#pragma unroll
                for (int i = 0; i < Q; i++)
                    t[u][i] = __builtin_nontemporal_load(
                        reinterpret_cast<const f32x4*>(partial + off + (qd[i].row * a.n + qd[i].col0)));
            }
#pragma unroll
            for (int u = 0; u < 4; u++)
                if (s0 + u < a.ksplit) {
#pragma unroll
                    for (int i = 0; i < Q; i++) v[i] += t[u][i];
                }
        }
    }
    const float g = a.rfactor ? load_f32_vmem(reinterpret_cast<const uint8_t*>(a.rfactor)) : 1.0f;
    RedBias b[Q];
    if (a.bias) {
        const bool al8 = (reinterpret_cast<uintptr_t>(a.bias) & 7) == 0;
#pragma unroll
        for (int i = 0; i < Q; i++) b[i] = red_bias_load(a.bias, qd[i].col0, al8);
    } else {
#pragma unroll
        for (int i = 0; i < Q; i++) b[i] = RedBias{0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < Q; i++)
        if (qd[i].live) red_store(a, qd[i], v[i], g, b[i]);
}

}  // namespace wq
