// mm_common.h -- shared by the matmul kernels (gemv.hip, gemm_kernel.h): Y = X * W^T + b with W kept packed and dequantized inside the
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
// NF4 codes (and q4_0 codes in the GEMV) are decoded through byte-indexed tables
// in LDS (one entry per code byte, i.e. two values per lookup), replicated per
// lane so that concurrent lookups of different bytes hit different banks; the LDS
// address is built with one v_perm_b32.  The GEMV table holds bf16 values (fed
// straight to the MFMA), the GEMM table fp32 values (scaled exactly, then rounded
// once to bf16).  NVFP4 codes and scales are decoded with the gfx950 fp4 / fp8
// conversion instructions; q8_0 bytes, q4_1, q5_0, q4_k and q6_k codes (and
// q4_0 nibbles in the GEMM) are converted to floats in registers.
//
// GEMV (m <= 16, decode): B = raw code values (NF4 level, q4_0 q-8, q8_0 q),
//   the per-block scale is applied to the MFMA partial sum of each block; for
//   NVFP4 (16-value blocks, two per 32-K slice) B = e2m1*scale (exact in bf16),
//   except for one token, where each block's x fills its own A row, B = e2m1, and
//   the block scales are applied to the per-block sums;
//   for q4_1 (scale and minimum), q5_0 (fifth bits), q4_k and q6_k (two-level
//   scales) B = bf16(w^) as in the GEMM: with an offset, a sum of x c scaled after the
//   MFMA minus an offset times the sum of x would cancel, and its rounding error would
//   no longer be bounded by the sum of |x w^|.
//   K is split over the waves of a workgroup and reduced in LDS.
// GEMM (m >= 17, encoder): each wave dequantizes 64 columns x 128 K of W per
//   step to bf16(w^) -- w^ computed exactly as the format defines it, then one
//   round-to-nearest-even -- straight into MFMA B registers; the X tile
//   (128 x 128 bf16) is shared through LDS.  Few output tiles split K across
//   workgroups into an fp32 workspace, summed in order by a second kernel.
#pragma once

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

// Kernel arguments.  A launch reads its argument block from memory, cold, one 128-byte
// line per round trip, and a second line on a kernel's path costs a GEMV launch up to
// three quarters of a microsecond: every field a GEMV launch reads sits in the first
// line (the 32-bit fields rest on the boundary's limits: n, ldy < 2^31), and the whole
// block is that line: the kernels derive their schedules (tile counts, K pieces, grid)
// from it rather than read the hidden arguments that follow it.
struct KArgs {
    const uint16_t* x;       // 0x00
    union {                  // 0x08
        const uint8_t* codes;
        const float* rpartial;   // split-K reduce launch: the pieces' fp32 partials [ksplit][m][n]
    };
    union {                  // 0x10
        const uint8_t* scales;
        const float* rfactor;    // split-K reduce launch: address of the epilogue factor, or null (1)
    };
    union {                  // 0x18 one per format:
        const uint8_t* gs;   //   NVFP4: address of the fp32 factor applied in the epilogue (the global scale)
        int64_t d_off;       //   NF4+DQ: fp32 group scales    } offsets into scales,
        int64_t hb_off;      //   q5_0: fifth-bit words        } as in ScaleLayout
        int64_t kd_off;      //   q4_k / q6_k: super-block scales
    };
    const uint16_t* bias;    // 0x20
    union {                  // 0x28 output splits: columns [0, end0) -> y0, [end0, end1) -> y1,
        char* y0;            //   [end1, n) -> y2 (one split: end0 = end1 = n).  A K-split GEMM
        float* partial;      //   launch (the reduce kernel writes the outputs) carries here its
    };                       //   fp32 partials [ksplit][m][n]
    char* y1;                // 0x30
    char* y2;                // 0x38
    int64_t n, k;            // 0x40, 0x48
    int64_t ldx;             // 0x50
    int64_t mu_off;          // 0x58 NF4+DQ: fp32 mean (offset into scales)
    int m;                   // 0x60
    int ldy0, ldy1, ldy2;    // 0x64 row strides of the splits (elements)
    int end0, end1;          // 0x70
    uint8_t f32;             // 0x78 1: fp32 output, 0: bf16
    uint8_t out_vec;         // 0x79 every output split allows 4-column vector stores (alignment, split ends % 4)
    uint8_t out_v16;         // 0x7A bf16 output whose splits allow 8-column (16-byte) stores
    uint8_t wg_per_cu;       // 0x7B band-pipelined GEMV: workgroups per CU (its grid is that many per CU)
    int ksplit;              // 0x7C GEMM: K pieces per output tile
};
static_assert(sizeof(KArgs) == 128, "the kernel arguments are one 128-byte line");

// One fp32 value at a uniform address (the NVFP4 global scale, the double-quant mean),
// read with a vector buffer load.  A plain read of a uniform address becomes a scalar
// load, and scalar loads share one wait counter with the kernel-argument loads: the
// kernel's first wait for an argument would then also wait for this value's trip to
// memory, before any weight load is issued.
__device__ inline float load_f32_vmem(const uint8_t* p) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, 4, 0x00020000);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, 0, 0, 0));
}

// NF4 level of code c as a 16-way select over literals.  Table fills use these
// rather than indexing the level arrays: a per-lane index would turn into a
// vector memory load, and waiting for it would also wait for every weight load
// already in flight.
__device__ inline uint32_t nf4_level_bf16_sel(uint32_t c) {
    uint32_t v = kNf4LevelBf16[0];
#pragma unroll
    for (uint32_t i = 1; i < 16; i++) v = ((c & 15u) == i) ? (uint32_t)kNf4LevelBf16[i] : v;
    return v;
}

__device__ inline float nf4_level_sel(uint32_t c) {
    uint32_t v = kNf4LevelBits[0];
#pragma unroll
    for (uint32_t i = 1; i < 16; i++) v = ((c & 15u) == i) ? kNf4LevelBits[i] : v;
    return __uint_as_float(v);
}

// bf16 image of a 4-bit code's value (before any block scale).
template <int FMT>
__device__ inline uint32_t code_bf16(uint32_t c) {
    if constexpr (FMT == kNF4) {
        return nf4_level_bf16_sel(c);
    } else if constexpr (FMT == kQ4_0) {
        return __float_as_uint((float)((int)(c & 15u) - 8)) >> 16;          // exact
    } else {  // NVFP4
        float v = e2m1_mag_value(c & 7u);
        if (c & 8u) v = -v;
        return __float_as_uint(v) >> 16;                                       // exact
    }
}

// Fill the replicated byte table: word (e * 64 + slot) = bf16(lo nibble) | bf16(hi nibble) << 16,
// e = 16 * hi + lo.  Thread t (of NT = 256 or 512) owns 4 slots of entries with
// lo = (t >> 4) & 15 and hi = t >> 8 (mod NT / 256): the lo value is looked up
// once, the hi value is the same for a whole wave.
template <int FMT, int NT>
__device__ inline void build_lut(uint32_t* lut) {
    static_assert(NT == 256 || NT == 512, "table fill for blocks of 256 or 512 threads");
    const int t = threadIdx.x;
    const int slot4 = (t & 15) * 4;
    const uint32_t lo = (t >> 4) & 15;
    const uint32_t vlo = code_bf16<FMT>(lo);
    const uint32_t hsub = __builtin_amdgcn_readfirstlane(t >> 8);
#pragma unroll
    for (uint32_t h0 = 0; h0 < 16; h0 += NT / 256) {
        const uint32_t hi = h0 + hsub;
        uint32_t vhi = code_bf16<FMT>(h0);
        if constexpr (NT == 512) vhi = hsub ? code_bf16<FMT>(h0 + 1) : vhi;
        const uint32_t v = vlo | (vhi << 16);
        *reinterpret_cast<uint4*>(lut + (hi * 16 + lo) * 64 + slot4) = make_uint4(v, v, v, v);
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
        return nf4_level_sel(c);
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
    const int t = threadIdx.x;             // 256 threads: entry 16 * hi + lo with lo = t >> 4
    const int slot = (t & 15) * 2;
    const uint32_t lo = __float_as_uint(code_f32<FMT>((uint32_t)t >> 4));
#pragma unroll
    for (uint32_t e0 = 0; e0 < 256; e0 += 16) {
        const uint32_t hi = __float_as_uint(code_f32<FMT>(e0 >> 4));
        *reinterpret_cast<uint4*>(lut + (e0 + (t >> 4)) * 64 + slot * 2) = make_uint4(lo, hi, lo, hi);
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

// q4_1 B operand for one 32-wide K slice: the slice's code word (nibble i = k 8h + i)
// and its block's fp16 pair dm = d | m << 16.  w^ = fl(c * d + m) with c * d exact (4 + 11
// significant bits), so one fma is the format's w^; then one RNE to bf16.
__device__ __forceinline__ u32x4 q4_1_operand(uint32_t word, uint32_t dm) {
    const float d = f16_value((uint16_t)(dm & 0xFFFFu)), m = f16_value((uint16_t)(dm >> 16));
    uint32_t lo = word & 0x0F0F0F0Fu, hi = (word >> 4) & 0x0F0F0F0Fu;
    // opaque to the optimizer, so that each byte converts with one v_cvt_f32_ubyteN
    asm("" : "+v"(lo), "+v"(hi));
    u32x4 B;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const float c0 = (float)((lo >> (8 * q)) & 255u);
        const float c1 = (float)((hi >> (8 * q)) & 255u);
        B[q] = pack_bf16_rne(__builtin_fmaf(c0, d, m), __builtin_fmaf(c1, d, m));
    }
    return B;
}

// q5_0 B operand for one 32-wide K slice: the slice's code word (low 4 bits, nibble i =
// k 8h + i), the 8 fifth bits of those k (bit i) and the block's fp16 scale.  The fifth
// bits move to bit 4 of the byte their nibble lands in with one 24-bit multiply per
// parity: in e = bits & 0x55 (bits 2p), e * 0x410410 puts bit 2p at 8p + 4 (the shifts
// 4, 10, 16, 22 add 6p + 4 for term p; every other term lands on a different even bit and
// any carry stops at the odd bit above it), then & 0x10101010 keeps bits 8p + 4.
// c = q + 16 (0..31) as a float; w^ = (c - 16) * d = fl(c * d - 16 d) exactly (both products
// fit 16 significant bits), one fma; then one RNE to bf16.
__device__ __forceinline__ u32x4 q5_0_operand(uint32_t word, uint32_t high8, uint16_t dbits) {
    const float d = f16_value(dbits);
    const float d16 = -16.0f * d;
    uint32_t lo = word & 0x0F0F0F0Fu, hi = (word >> 4) & 0x0F0F0F0Fu;
    lo |= __umul24(high8 & 0x55u, 0x410410u) & 0x10101010u;
    hi |= __umul24((high8 >> 1) & 0x55u, 0x410410u) & 0x10101010u;
    // opaque to the optimizer, so that each byte converts with one v_cvt_f32_ubyteN
    asm("" : "+v"(lo), "+v"(hi));
    u32x4 B;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const float c0 = (float)((lo >> (8 * q)) & 255u);
        const float c1 = (float)((hi >> (8 * q)) & 255u);
        B[q] = pack_bf16_rne(__builtin_fmaf(c0, d, d16), __builtin_fmaf(c1, d, d16));
    }
    return B;
}

// q4_k B operand for one 32-wide K slice (one sub-block): the slice's code word, the
// sub-block's S = d * sc and O = dmin * m (both exact).  w^ = fl(c * S - O) with c * S exact
// (4 + 17 significant bits), one fma; then one RNE to bf16.
__device__ __forceinline__ u32x4 q4_k_operand(uint32_t word, float S, float O) {
    uint32_t lo = word & 0x0F0F0F0Fu, hi = (word >> 4) & 0x0F0F0F0Fu;
    // opaque to the optimizer, so that each byte converts with one v_cvt_f32_ubyteN
    asm("" : "+v"(lo), "+v"(hi));
    u32x4 B;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const float c0 = (float)((lo >> (8 * q)) & 255u);
        const float c1 = (float)((hi >> (8 * q)) & 255u);
        B[q] = pack_bf16_rne(__builtin_fmaf(c0, S, -O), __builtin_fmaf(c1, S, -O));
    }
    return B;
}

// S and O of sub-block j of a q4_k tile row: rec_sc / rec_m hold the 4 sub-blocks' 6-bit
// scales / offsets (byte j), dm the super-block's fp16 d | dmin << 16.
__device__ __forceinline__ void q4_k_sub(uint32_t rec_sc, uint32_t rec_m, uint32_t dm, int j, float& S, float& O) {
    S = f16_value((uint16_t)(dm & 0xFFFFu)) * (float)((rec_sc >> (8 * j)) & 255u);
    O = f16_value((uint16_t)(dm >> 16)) * (float)((rec_m >> (8 * j)) & 255u);
}

// q6_k B operand for one 32-wide K slice: the slice's code word (low 4 bits, nibble i =
// k 8h + i), bits 4 (b4) and 5 (b5) of those 8 codes (bit i), and the lane's sub-block S
// = d * sc (exact).  Each bit set moves to its byte as in q5_0_operand (bit 2p of a parity
// -> bit 8p + 4, one 24-bit multiply), bit 5 one place higher.  c = q (0..63);
// w^ = (c - 32) * S = fl(c * S - 32 S) exactly (at most 24 significant bits), one fma.
__device__ __forceinline__ u32x4 q6_k_operand(uint32_t word, uint32_t b4, uint32_t b5, float S) {
    uint32_t lo = word & 0x0F0F0F0Fu, hi = (word >> 4) & 0x0F0F0F0Fu;
    lo |= __umul24(b4 & 0x55u, 0x410410u) & 0x10101010u;
    lo |= (__umul24(b5 & 0x55u, 0x410410u) & 0x10101010u) << 1;
    hi |= __umul24((b4 >> 1) & 0x55u, 0x410410u) & 0x10101010u;
    hi |= (__umul24((b5 >> 1) & 0x55u, 0x410410u) & 0x10101010u) << 1;
    // opaque to the optimizer, so that each byte converts with one v_cvt_f32_ubyteN
    asm("" : "+v"(lo), "+v"(hi));
    const float s32 = -32.0f * S;
    u32x4 B;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const float c0 = (float)((lo >> (8 * q)) & 255u);
        const float c1 = (float)((hi >> (8 * q)) & 255u);
        B[q] = pack_bf16_rne(__builtin_fmaf(c0, S, s32), __builtin_fmaf(c1, S, s32));
    }
    return B;
}

// q6_k: S of sub-block t (0..7) of a tile row from its int8 scale record (r0: sub-blocks
// 0..3, r1: 4..7) and the super-block's fp16 d; bits 4 / 5 of K slice j from the lane's
// 8-byte high record (h0: slices 0, 1; h1: slices 2, 3).
__device__ __forceinline__ float q6_k_scale(uint32_t r0, uint32_t r1, uint32_t dbits, int t) {
    const uint32_t w = t < 4 ? r0 : r1;
    return f16_value((uint16_t)(dbits & 0xFFFFu)) * (float)(int8_t)(uint8_t)(w >> (8 * (t & 3)));
}

__device__ inline f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Output.  A lane's output column is fixed for a whole tile, so the split it
// falls in, its base pointer and leading dimension are selected once per
// column (constant-index kernel-argument reads, then selects) and the bias is
// read once per column.
// ---------------------------------------------------------------------------
struct ColOut {
    char* p;       // address of element (row 0, this column)
    int64_t ld;    // row stride in bytes
    float bias;
};

// Output fields read through readfirstlane (UNI = true).  They are the same in every
// lane; selecting between plain reads of them lets the compiler fold the per-lane
// choice of split into one per-lane load from the argument block, a vector memory
// request whose wait (in-order counting) also waits for every weight request the wave
// has in flight: the GEMV band loops, the GEMM epilogue and the split-K reduce read them
// this way (in the GEMM only after its main loop, so the copies do not live through it).
template <bool UNI>
__device__ inline uint64_t out_u64(uint64_t v) {
    if constexpr (!UNI) return v;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return (uint64_t)lo | ((uint64_t)hi << 32);
}
template <bool UNI>
__device__ inline char* out_p(char* p) { return reinterpret_cast<char*>(out_u64<UNI>(reinterpret_cast<uint64_t>(p))); }
template <bool UNI>
__device__ inline int64_t out_i(int64_t v) { return (int64_t)out_u64<UNI>((uint64_t)v); }

template <bool UNI = false>
__device__ inline ColOut col_out_nobias(const KArgs& a, int64_t col) {
    const int64_t e0 = out_i<UNI>(a.end0), e1 = out_i<UNI>(a.end1);
    const bool s1 = col >= e0, s2 = col >= e1;
    char* const y0 = out_p<UNI>(a.y0);
    char* const y1 = out_p<UNI>(a.y1);
    char* const y2 = out_p<UNI>(a.y2);
    char* const base = s2 ? y2 : (s1 ? y1 : y0);
    const int64_t ld = s2 ? out_i<UNI>(a.ldy2) : (s1 ? out_i<UNI>(a.ldy1) : out_i<UNI>(a.ldy0));
    const int64_t c0 = s2 ? e1 : (s1 ? e0 : 0);
    const int64_t es = a.f32 ? 4 : 2;
    ColOut c;
    c.p = base + (col - c0) * es;
    c.ld = ld * es;
    c.bias = 0.0f;
    return c;
}

template <bool UNI = false>
__device__ inline ColOut col_out(const KArgs& a, int64_t col) {
    ColOut c = col_out_nobias<UNI>(a, col);
    c.bias = a.bias ? bf16_value(a.bias[col]) : 0.0f;
    return c;
}

// y = acc * g + bias, converted and stored at row m.  The store names the global
// address space: a generic (flat) store would make the compiler's wait insertion treat
// the vector-memory counter as out of order for as long as the store is in flight,
// and turn every later wait of a band loop into a wait for all requests.
typedef __attribute__((address_space(1))) float gfloat_t;
typedef __attribute__((address_space(1))) uint16_t gu16_t;
__device__ inline void put_out(const KArgs& a, const ColOut& c, int64_t m, float v, float g) {
    const float r = v * g + c.bias;
    char* const p = c.p + m * c.ld;
    if (a.f32) *(gfloat_t*)p = r;
    else *(gu16_t*)p = bf16_rne(r);
}

// 4 x 4 transpose inside each quad of lanes (t = lane & 3): on entry v[i] is
// element (row i, column t) of the quad's block, on exit v[j] is (row t, column j).
// Two exchange stages, with lane t ^ 1 and then lane t ^ 2.
__device__ __forceinline__ float dpp_xor1(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
}
__device__ __forceinline__ float dpp_xor2(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
}
__device__ __forceinline__ void quad_transpose(float (&v)[4], int t) {
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; i++) p[i] = dpp_xor1(v[i ^ 1]);
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = ((i ^ t) & 1) ? p[i] : v[i];
#pragma unroll
    for (int i = 0; i < 4; i++) p[i] = dpp_xor2(v[i ^ 2]);
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = ((i ^ t) & 2) ? p[i] : v[i];
}

// Workgroup barrier for data written to LDS by this workgroup's LDS-direct loads
// and LDS stores, when the N most recent vector-memory requests (register
// loads) may stay in flight: s_waitcnt vmcnt(N) lgkmcnt(0), then s_barrier.
// __syncthreads() would wait for every outstanding load here, because its fence
// cannot tell the LDS-direct loads from the later register loads.  The compiler
// is kept from moving memory accesses across the barrier.
template <int N>
__device__ __forceinline__ void lds_barrier_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// s_waitcnt vmcnt(N) with lgkmcnt and expcnt left alone (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// ===========================================================================
// GEMV, m <= 16.  Work item = (16-row band, K piece).  Each wave owns whole
// items (no cross-wave reduction); an item's tiles are fetched C at a time --
// codes, scales and X operands of all C tiles are requested before any is
// used -- so every wave keeps up to C KiB of weights in flight.  Lane l owns row
// (l & 15) of the band as B operand and row (l & 15) of X as A operand; the
// 16x16 result tile has D[4*(l>>4)+i][l&15] in lane l.
constexpr int kBufWord3 = 0x00020000;   // buffer descriptor word 3: raw, untyped access

typedef __amdgpu_buffer_rsrc_t BufRes;

__device__ inline BufRes buf_res(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufWord3);
}

// The same for a base and size that are equal in every lane but that the
// compiler cannot prove so (results of 64-bit division, values held in
// arrays): read them from the first active lane.
__device__ inline uint32_t uni(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
__device__ inline int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline BufRes buf_res_uni(const void* base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint64_t u = (uint64_t)uni((uint32_t)b) | ((uint64_t)uni((uint32_t)(b >> 32)) << 32);
    return buf_res(reinterpret_cast<const void*>(u), uni(bytes));
}

// Buffer-load cache policy for data read exactly once (GEMV weights): non-temporal.
// On this chip a read-only stream with this hint runs about 12% faster than with
// the default policy.
constexpr int kNT = 2;


constexpr int kNumCU = 256;

inline KArgs make_args(const MatmulProblem& p) {
    KArgs a{};
    a.x = p.x;
    a.ldx = p.ldx;
    a.m = (int)p.m;
    a.n = p.n;
    a.k = p.k;
    a.codes = p.codes;
    a.scales = p.scales;
    a.bias = p.bias;
    const ScaleLayout L = scale_layout(p.fmt, p.dq, p.n, p.k);
    a.mu_off = L.mu_off;
    if (p.fmt == kNVFP4) a.gs = p.gscale ? reinterpret_cast<const uint8_t*>(p.gscale) : p.scales + L.g_off;
    else if (p.fmt == kQ5_0) a.hb_off = L.hb_off;
    else if (p.fmt == kQ4_K || p.fmt == kQ6_K) a.kd_off = L.kd_off;
    else a.d_off = L.d_off;
    a.f32 = (uint8_t)p.out.f32;
    // unused splits repeat the last one (their column ranges are empty)
    const int ns = p.out.nsplit;
    a.y0 = reinterpret_cast<char*>(p.out.y[0]);
    a.y1 = reinterpret_cast<char*>(p.out.y[ns > 1 ? 1 : 0]);
    a.y2 = reinterpret_cast<char*>(p.out.y[ns > 2 ? 2 : ns - 1]);
    a.ldy0 = (int)p.out.ldy[0];
    a.ldy1 = (int)p.out.ldy[ns > 1 ? 1 : 0];
    a.ldy2 = (int)p.out.ldy[ns > 2 ? 2 : ns - 1];
    a.end0 = (int)(ns > 1 ? p.out.end[0] : p.n);
    a.end1 = (int)(ns > 2 ? p.out.end[1] : p.n);
    a.ksplit = 1;
    const uintptr_t align = p.out.f32 ? 16 : 8;
    a.out_vec = 1;
    a.out_v16 = p.out.f32 ? 0 : 1;
    for (int i = 0; i < p.out.nsplit; i++) {
        const uintptr_t y = reinterpret_cast<uintptr_t>(p.out.y[i]);
        if (y % align != 0 || p.out.ldy[i] % 4 != 0 || p.out.end[i] % 4 != 0) a.out_vec = 0;
        if (y % 16 != 0 || p.out.ldy[i] % 8 != 0 || p.out.end[i] % 8 != 0) a.out_v16 = 0;
    }
    return a;
}

}  // namespace wq
