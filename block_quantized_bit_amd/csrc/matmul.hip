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
//   NVFP4 (16-value blocks, two per 32-K slice) B = e2m1*scale (exact in bf16);
//   for q4_1 (scale and minimum), q5_0 (fifth bits), q4_k and q6_k (two-level
//   scales) B = bf16(w^) as in the GEMM.
//   K is split over the waves of a workgroup and reduced in LDS.
// GEMM (m >= 17, encoder): each wave dequantizes 64 columns x 128 K of W per
//   step to bf16(w^) -- w^ computed exactly as the format defines it, then one
//   round-to-nearest-even -- straight into MFMA B registers; the X tile
//   (128 x 128 bf16) is shared through LDS.  Few output tiles split K across
//   workgroups into an fp32 workspace, summed in order by a second kernel.
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
    int64_t tiles_m, tiles_n;
    int out_vec;         // every output split allows 4-column vector stores (alignment, split ends % 4)
    int out_v16;         // bf16 output whose splits allow 8-column (16-byte) stores
};

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

__device__ inline ColOut col_out(const KArgs& a, int64_t col) {
    const OutSplit& o = a.out;
    const bool s1 = col >= o.end[0], s2 = col >= o.end[1];
    char* const y0 = reinterpret_cast<char*>(o.y[0]);
    char* const y1 = reinterpret_cast<char*>(o.y[1]);
    char* const y2 = reinterpret_cast<char*>(o.y[2]);
    char* const base = s2 ? y2 : (s1 ? y1 : y0);
    const int64_t ld = s2 ? o.ldy[2] : (s1 ? o.ldy[1] : o.ldy[0]);
    const int64_t c0 = s2 ? o.end[1] : (s1 ? o.end[0] : 0);
    const int64_t es = o.f32 ? 4 : 2;
    ColOut c;
    c.p = base + (col - c0) * es;
    c.ld = ld * es;
    c.bias = a.bias ? bf16_value(a.bias[col]) : 0.0f;
    return c;
}

__device__ inline ColOut col_out_nobias(const KArgs& a, int64_t col) {
    const OutSplit& o = a.out;
    const bool s1 = col >= o.end[0], s2 = col >= o.end[1];
    char* const y0 = reinterpret_cast<char*>(o.y[0]);
    char* const y1 = reinterpret_cast<char*>(o.y[1]);
    char* const y2 = reinterpret_cast<char*>(o.y[2]);
    char* const base = s2 ? y2 : (s1 ? y1 : y0);
    const int64_t ld = s2 ? o.ldy[2] : (s1 ? o.ldy[1] : o.ldy[0]);
    const int64_t c0 = s2 ? o.end[1] : (s1 ? o.end[0] : 0);
    const int64_t es = o.f32 ? 4 : 2;
    ColOut c;
    c.p = base + (col - c0) * es;
    c.ld = ld * es;
    c.bias = 0.0f;
    return c;
}

// y = acc * g + bias, converted and stored at row m.
__device__ inline void put_out(const KArgs& a, const ColOut& c, int64_t m, float v, float g) {
    const float r = v * g + c.bias;
    char* const p = c.p + m * c.ld;
    if (a.out.f32) *reinterpret_cast<float*>(p) = r;
    else *reinterpret_cast<uint16_t*>(p) = bf16_rne(r);
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
    const float* dt = reinterpret_cast<const float*>(a.scales + a.L.d_off);
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
                const float* dt = reinterpret_cast<const float*>(a.scales + a.L.d_off);
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
        t.sc[4] = *reinterpret_cast<const uint16_t*>(a.scales + a.L.kd_off + ((band * 16 + r) * (a.k >> 8) + (kt >> 1)) * 2);
    } else if constexpr (FMT == kQ4_K) {
        // the row's sub-block record (4 scale bytes, 4 offset bytes) and its super-block's
        // (d, dmin); a 128-K tile is half a 256-K super-block
        const uint2 v = *reinterpret_cast<const uint2*>(a.scales + tile * 128 + r * 8);
        t.sc[0] = v.x;
        t.sc[1] = v.y;
        t.sc[2] = *reinterpret_cast<const uint32_t*>(a.scales + a.L.kd_off + ((band * 16 + r) * (a.k >> 8) + (kt >> 1)) * 4);
    } else if constexpr (FMT == kQ5_0) {
        // the row's four fp16 scales (8 bytes), then its four fifth-bit words (16 bytes)
        const uint2 v = *reinterpret_cast<const uint2*>(a.scales + (tile * 64 + r * 4) * 2);
        t.sc[0] = v.x;
        t.sc[1] = v.y;
        const uint4 hb = *reinterpret_cast<const uint4*>(a.scales + a.L.hb_off + tile * 256 + r * 16);
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
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jj = 0; jj < 2; jj++) {
                const int j = kb * 2 + jj;
                u32x4 B;
#pragma unroll
                for (int q = 0; q < 4; q++) B[q] = lut_pair(lut, lane4, uw[j], q);
                p = mfma(t.A[j], B, p);
            }
            const float s = kb ? s1 : s0;
#pragma unroll
            for (int i = 0; i < NI; i++) acc[i] += p[i] * s;
        }
    } else if constexpr (FMT == kQ4_0) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            u32x4 B;
#pragma unroll
            for (int q = 0; q < 4; q++) B[q] = lut_pair(lut, lane4, uw[j], q);
            const f32x4 p = mfma(t.A[j], B, f32x4{0.f, 0.f, 0.f, 0.f});
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
                if (mu) *mu = load_f32_vmem(a.scales + a.L.mu_off);
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

__device__ __forceinline__ void gemv_finish_band(const KArgs& a, f32x4 (&red)[kGemvWaves][64], const f32x4& acc,
                                                 int64_t band, int wave, int lane, float g) {
    const int r = lane & 15, h = lane >> 4;
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        f32x4 v = red[0][lane];
#pragma unroll
        for (int w = 1; w < kGemvWaves; w++) v += red[w][lane];
        const ColOut c = col_out(a, band * 16 + r);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int mm = 4 * h + i;
            if (mm < a.m) put_out(a, c, mm, v[i], g);
        }
    }
    __syncthreads();
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
    if constexpr (FMT == kNVFP4) g = load_f32_vmem(a.scales + a.L.g_off);
    if constexpr (FMT == kNF4 && DQ && !XL) mu = load_f32_vmem(a.scales + a.L.mu_off);
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
        gemv_finish_band(a, red, acc, band, wave, lane, g);
    } else {
        const int64_t stride = gridDim.x;
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
            gemv_finish_band(a, red, acc, band, wave, lane, g);
            if (band + stride >= nbands) break;
            acc = f32x4{0.f, 0.f, 0.f, 0.f};
            gemv_load_band<FMT, DQ, C, XL>(R0, dq0, a, std::min<int64_t>(band + 2 * stride, nbands - 1), 0, wave,
                                          lane, r, xrow, KT);
            gemv_consume_band<FMT, DQ, NI, C, XL>(R1, dq1, acc, 0, wave, KT, lut, lane4, h, mu, xl, xm8);
            gemv_finish_band(a, red, acc, band + stride, wave, lane, g);
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

// Scale bytes per tile and per lane (one row of the tile) in the packed layout.
template <int FMT, bool DQ>
__device__ constexpr int tile_scale_bytes() {
    return FMT == kQ8_0 ? 64 : (FMT == kNF4 && DQ) ? 32 : 128;
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

template <int FMT, bool DQ, int T>
__device__ __forceinline__ void stream_load_band(StreamTile (&R)[T], StreamBand& B, const KArgs& a, int64_t band,
                                                 int lane, int r, int64_t KT) {
    constexpr int SB = tile_scale_bytes<FMT, DQ>();
    const BufRes rc = buf_res(a.codes + band * KT * kTileBytes, (uint32_t)(KT * kTileBytes));
    const BufRes rs = buf_res(a.scales + band * KT * SB, (uint32_t)(KT * SB));
#pragma unroll
    for (int s = 0; s < T; s++) {
        R[s].code = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, lane * 16 + s * kTileBytes, 0, kNT));
        if constexpr (FMT == kNF4 && DQ) {
            R[s].sc[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, r * 2 + s * SB, 0, kNT);
        } else if constexpr (FMT == kQ8_0) {
            R[s].sc[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, r * 4 + s * SB, 0, kNT);
        } else {
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, r * 8 + s * SB, 0, kNT);
            R[s].sc[0] = v[0];
            R[s].sc[1] = v[1];
        }
    }
    const int64_t col = band * 16 + r;
    B.braw = a.bias ? (uint32_t)a.bias[col] : 0u;
    if constexpr (FMT == kNF4 && DQ) {
        const int64_t nbr = a.k / 64;                 // blocks per row
        const int64_t b0 = col * nbr;                 // first block of the row
        const int64_t gA = b0 >> 8, gB = (b0 + nbr - 1) >> 8;
        const float* dt = reinterpret_cast<const float*>(a.scales + a.L.d_off);
        B.dA = dt[gA];
        B.dB = dt[gB];
        B.jt = (int32_t)((gA + 1) * 256 - b0);
    }
}

template <int FMT, bool DQ, int NI, int T>
__device__ __forceinline__ void stream_band(const StreamTile (&R)[T], const StreamBand& B, const KArgs& a,
                                            int64_t band, const uint16_t* xrow, const uint16_t* xzero, int h,
                                            uint32_t lane4, const uint32_t* lut, float mu, float g, int64_t KT) {
    constexpr int TK = tile_k(FMT);
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
        __builtin_amdgcn_sched_barrier(0);   // keep tiles in order: bounded register use
    }
    // lane (h, r) holds rows 4h .. 4h+3 of column band * 16 + r
    ColOut c = col_out_nobias(a, band * 16 + (__lane_id() & 15));
    c.bias = bf16_value((uint16_t)B.braw);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int mm = 4 * h + i;
        if (mm < a.m) put_out(a, c, mm, acc[i], g);
    }
}

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
    const int64_t stride = (int64_t)gridDim.x * 4;

    float g = 1.0f, mu = 0.0f;
    if constexpr (FMT == kNVFP4) g = load_f32_vmem(a.scales + a.L.g_off);
    if constexpr (FMT == kNF4 && DQ) mu = load_f32_vmem(a.scales + a.L.mu_off);

    int64_t band = (int64_t)blockIdx.x * 4 + wave;
    StreamTile R0[T], R1[T];
    StreamBand B0, B1;
    stream_load_band<FMT, DQ, T>(R0, B0, a, std::min<int64_t>(band, nbands - 1), lane, r, KT);
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

    for (; band < nbands; band += 2 * stride) {
        stream_load_band<FMT, DQ, T>(R1, B1, a, std::min<int64_t>(band + stride, nbands - 1), lane, r, KT);
        stream_band<FMT, DQ, NI, T>(R0, B0, a, band, xrow, xzero, h, lane4, lut, mu, g, KT);
        if (band + stride >= nbands) break;
        stream_load_band<FMT, DQ, T>(R0, B0, a, std::min<int64_t>(band + 2 * stride, nbands - 1), lane, r, KT);
        stream_band<FMT, DQ, NI, T>(R1, B1, a, band + stride, xrow, xzero, h, lane4, lut, mu, g, KT);
    }
}

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
template <int FMT, bool DQ, int NB, int NWAIT, bool MORE>
__device__ __forceinline__ void gemm_kstep(f32x4 (&acc)[8][NB], u32x4 (&A)[8], u32x4 (&B)[NB],
                                           const GemmW<FMT> (&wc)[NB], GemmW<FMT> (&wn)[NB], const GemmW<FMT> (&wf)[NB],
                                           const GemmSrc& S, const int64_t (&rowblk)[NB], const uint32_t (&xoff)[kXLoads],
                                           const uint8_t* xcur, uint8_t* xnext, const uint8_t* xfol, const uint32_t* lut,
                                           int nx, int wave, int lane, int r, int h, uint32_t lane8,
                                           uint32_t hs, float mu) {
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
            for (int nf = 0; nf < NB; nf++) acc[mf][nf] = mfma(A[mf], B[nf], acc[mf][nf]);
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
    const int64_t nsteps_total = K / BK;

    // XCD-aware item order.  Workgroups are dealt to the 8 XCDs in turn, so XCD x
    // gets the consecutive items [x * per_xcd, (x + 1) * per_xcd).  Items run K piece
    // by K piece, and within a piece in groups of kGroupM row tiles by all column
    // tiles, column-major inside the group: the items an XCD runs at one time cover
    // a compact block of row and column tiles, whose X rows and W bands its L2 holds.
    constexpr int64_t kGroupM = 6;
    const int64_t tiles = a.tiles_m * a.tiles_n;
    const int64_t items = tiles * a.ksplit;
    const int64_t per_xcd = (int64_t)gridDim.x / 8;
    const int64_t item = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    if (item >= items) return;
    const int ks = (int)(item / tiles);
    const int64_t ti = item - (int64_t)ks * tiles;
    const int64_t grp = ti / (kGroupM * a.tiles_n);
    const int64_t gm = std::min<int64_t>(kGroupM, a.tiles_m - grp * kGroupM);
    const int64_t within = ti - grp * kGroupM * a.tiles_n;
    const int64_t tm = grp * kGroupM + within % gm;
    const int64_t tn = within / gm;
    const int64_t m0 = tm * BM, n0 = tn * BN;
    const int64_t s0 = ks * a.kt_per, s1 = std::min<int64_t>(nsteps_total, s0 + a.kt_per);  // in BK steps

    const int64_t band0 = n0 / 16 + wave * NB;
    const int64_t nbands = N / 16;

    float g = 1.0f, mu = 0.0f;
    if constexpr (FMT == kNVFP4) g = load_f32_vmem(a.scales + a.L.g_off);
    if constexpr (FMT == kNF4 && DQ) mu = load_f32_vmem(a.scales + a.L.mu_off);

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
        if constexpr (FMT == kQ5_0) S.hb[nf] = a.scales + a.L.hb_off + band * KT * 256;
        if constexpr (FMT == kQ4_K) S.hb[nf] = a.scales + a.L.kd_off + band * 16 * (K / 256) * 4;
        if constexpr (FMT == kQ6_K) {
            S.hb[nf] = a.codes + N * K / 2 + band * KT * 512;
            S.kd[nf] = a.scales + a.L.kd_off + band * 16 * (K / 256) * 2;
        }
    }
    S.hbbytes = FMT == kQ4_K ? (uint32_t)(16 * (K / 256) * 4) : FMT == kQ6_K ? (uint32_t)(KT * 512) : (uint32_t)(KT * 256);
    S.kdbytes = (uint32_t)(16 * (K / 256) * 2);
    S.wbytes = (uint32_t)(KT * kTileBytes);
    S.sbytes = (uint32_t)(KT * SB);
    S.dt = a.scales + a.L.d_off;
    S.dtbytes = (uint32_t)(a.L.ng * 4);
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
                                      wave, lane, r, h, lane8, hs, mu);
    } else {
        gemm_kstep<FMT, DQ, NB, 0, false>(acc, A, B, w0, w1, w1, S, rowblk, xoff, xs0, xs1, xs1, lut, last,
                                      wave, lane, r, h, lane8, hs, mu);
    }
    wait_vm<0>();   // the last requests (re-reads of the last step) land before the workgroup ends

    // ---- epilogue ----
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
            const float bias = a.bias ? bf16_value(a.bias[(band0 + nf) * 16 + r]) : 0.0f;
#pragma unroll
            for (int mf = 0; mf < 8; mf++) {
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; i++) v[i] = acc[mf][nf][i] * g + bias;
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
            const ColOut o = col_out_nobias(a, col);
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
            const ColOut c = col_out(a, (band0 + nf) * 16 + r);
            if (full) {
                // lane (h, r) owns rows 16 mf + 4h + i of its column: step through them by the row stride
                char* p = c.p + (m0 + 4 * h) * c.ld;
#pragma unroll
                for (int mf = 0; mf < 8; mf++) {
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; i++) v[i] = acc[mf][nf][i] * g + c.bias;
                    if (a.out.f32) {
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
    // K split: deposit this piece's partial tile; k_splitk_reduce finishes the outputs.
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

// y = v * g + bias for quad q (4 consecutive columns of one row), converted and stored.
__device__ inline void reduce_store(const KArgs& a, int64_t q, const f32x4& v, float g) {
    const int64_t nq = a.n / 4;
    const int64_t mm = q / nq, col0 = (q - mm * nq) * 4;
    if (a.out_vec) {
        // the 4 columns lie in one output split and can be written with one store
        const ColOut c = col_out(a, col0);
        float o[4];
#pragma unroll
        for (int u = 0; u < 4; u++) o[u] = v[u] * g + (a.bias ? bf16_value(a.bias[col0 + u]) : 0.0f);
        char* p = c.p + mm * c.ld;
        if (a.out.f32) *reinterpret_cast<f32x4*>(p) = f32x4{o[0], o[1], o[2], o[3]};
        else *reinterpret_cast<uint2*>(p) = make_uint2((uint32_t)bf16_rne(o[0]) | ((uint32_t)bf16_rne(o[1]) << 16),
                                                      (uint32_t)bf16_rne(o[2]) | ((uint32_t)bf16_rne(o[3]) << 16));
        return;
    }
#pragma unroll
    for (int u = 0; u < 4; u++) put_out(a, col_out(a, col0 + u), mm, v[u], g);
}

// Sum the K pieces' partials of each output in piece order, add the bias,
// convert and store.  A thread owns two quads (4 consecutive columns of one
// row each) 256 quads apart, so eight 16-byte loads are in flight per thread.
// Runs after k_gemm on the same stream, so every partial is complete and visible.
__global__ __launch_bounds__(256) void k_splitk_reduce(KArgs a, int global_scale) {
    const float g = global_scale ? *reinterpret_cast<const float*>(a.scales + a.L.g_off) : 1.0f;
    const int64_t total = (int64_t)a.m * (a.n / 4);
    const int64_t qa = (int64_t)blockIdx.x * 512 + threadIdx.x, qb = qa + 256;
    if (qa >= total) return;
    const bool hb = qb < total;
    const int64_t pstride = (int64_t)a.m * a.n;
    // the partials are [ksplit][m][n] row-major with n % 4 == 0: quad q starts at element 4q
    const float* pa = a.partial + qa * 4;
    const float* pb = a.partial + (hb ? qb : qa) * 4;
    // pieces are summed in order 0, 1, ...; their loads are issued four at a time (indices
    // past the last piece re-read it and are dropped)
    f32x4 va = {0.f, 0.f, 0.f, 0.f}, vb = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < a.ksplit; s0 += 4) {
        f32x4 ta[4], tb[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int64_t off = std::min(s0 + u, a.ksplit - 1) * pstride;
            ta[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(pa + off));
            tb[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(pb + off));
        }
#pragma unroll
        for (int u = 0; u < 4; u++)
            if (s0 + u < a.ksplit) {
                va += ta[u];
                vb += tb[u];
            }
    }
    reduce_store(a, qa, va, g);
    if (hb) reduce_store(a, qb, vb, g);
}

// The same for exactly KS pieces (2 or 4): each thread owns 2 quads, spaced 256 apart,
// and issues all 2 KS of its partial loads before adding any (pieces in order).  (Four
// quads per thread at KS = 2 measured 0.7-1 us slower on the M = 1500 fc2 shape.)
template <int KS>
__global__ __launch_bounds__(256) void k_splitk_reduce_n(KArgs a, int global_scale) {
    constexpr int Q = 2;
    const float g = global_scale ? *reinterpret_cast<const float*>(a.scales + a.L.g_off) : 1.0f;
    const int64_t total = (int64_t)a.m * (a.n / 4);
    const int64_t q0 = (int64_t)blockIdx.x * (256 * Q) + threadIdx.x;
    if (q0 >= total) return;
    const int64_t pstride = (int64_t)a.m * a.n;
    f32x4 t[KS][Q];
#pragma unroll
    for (int i = 0; i < Q; i++) {
        // quads past the end re-read the first one and are dropped
        const int64_t q = q0 + 256 * i < total ? q0 + 256 * i : q0;
#pragma unroll
        for (int s = 0; s < KS; s++)
            t[s][i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.partial + s * pstride + q * 4));
    }
#pragma unroll
    for (int i = 0; i < Q; i++) {
        if (q0 + 256 * i >= total) break;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; s++) v += t[s][i];
        reduce_store(a, q0 + 256 * i, v, g);
    }
}

// ---------------------------------------------------------------------------
// Schedules and launchers.
// ---------------------------------------------------------------------------
constexpr int kNumCU = 256;
constexpr int64_t kStreamMinBands = 4 * 2 * 4 * kNumCU;   // bands per wave x waves

struct Sched {
    int nb;              // bands per wave: tiles are 128 x (64 nb)
    int ksplit;
    int64_t kt_per;
    int64_t tiles_m, tiles_n;
    unsigned grid;
};

// GEMM: one workgroup per CU.  Tiles are 128 x 256, or 128 x 128 when the wide
// tiles cannot fill half the chip.  K is split only when even then the tiles
// cannot fill half the chip, and then doubled only while all pieces still run in
// one round on the CUs and every piece keeps >= kMinPieceSteps K steps: a split
// costs the fp32 partials' round trip through memory and a second launch, about
// as much as 11 K steps of a 128 x 128 tile (measured on MI355X at M = 1500).
constexpr int64_t kMinPieceSteps = 12;

static Sched gemm_sched(int64_t m, int64_t n, int64_t k, bool allow_split) {
    Sched s{};
    s.tiles_m = (m + BM - 1) / BM;
    s.nb = s.tiles_m * ((n + 255) / 256) < kNumCU / 2 ? 2 : 4;
    const int64_t bn = 64 * s.nb;
    s.tiles_n = (n + bn - 1) / bn;
    const int64_t steps = k / BK;
    const int64_t tiles = s.tiles_m * s.tiles_n;
    int ks = 1;
    if (allow_split && tiles < kNumCU / 2) {
        while (tiles * ks * 2 <= kNumCU && steps / (ks * 2) >= kMinPieceSteps) ks *= 2;
    }
    s.ksplit = ks;
    s.kt_per = (steps + ks - 1) / ks;     // every piece non-empty: (ks - 1) * kt_per < steps
    const int64_t items = tiles * ks;
    s.grid = (unsigned)(((items + 7) / 8) * 8);
    return s;
}

size_t gemv_workspace_bytes(int, int64_t, int64_t, int64_t) { return 0; }

size_t gemm_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k) {
    (void)fmt;
    const Sched s = gemm_sched(m, n, k, true);
    return s.ksplit <= 1 ? 0 : (size_t)s.ksplit * (size_t)m * (size_t)n * 4u;
}

size_t matmul_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k) {
    return m <= 16 ? gemv_workspace_bytes(fmt, m, n, k) : gemm_workspace_bytes(fmt, m, n, k);
}

static KArgs make_args(const MatmulProblem& p) {
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
            hipLaunchKernelGGL((k_gemv<FMT, DQ, NI, C, true, XL>), dim3((unsigned)resident), block, xbytes, st, a);
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
    // Many more bands than resident waves, K <= 10 tiles, X fits in LDS: the
    // streaming kernel (two workgroups of 4 waves per CU, each wave >= 4 bands).
    // (q4_1, q5_0, q4_k and q6_k have no streaming variant: their wider scale records take
    // the general kernel)
    if constexpr (FMT != kQ4_1 && FMT != kQ5_0 && FMT != kQ4_K && FMT != kQ6_K) {
        if (nbands >= kStreamMinBands && (int64_t)a.m * a.k <= kStreamXMax && KT <= 10) {
            const unsigned grid = 2 * kNumCU;
            if (KT <= 4) hipLaunchKernelGGL((k_gemv_stream<FMT, DQ, NI, 4>), dim3(grid), dim3(256), 0, st, a);
            else hipLaunchKernelGGL((k_gemv_stream<FMT, DQ, NI, 10>), dim3(grid), dim3(256), 0, st, a);
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

template <int FMT, bool DQ>
static void gemm_launch(int nb, dim3 grid, const KArgs& a, hipStream_t st) {
    if (nb == 2) hipLaunchKernelGGL((k_gemm<FMT, DQ, 2>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_gemm<FMT, DQ, 4>), grid, dim3(256), 0, st, a);
}

hipError_t launch_gemm(const MatmulProblem& p, hipStream_t st) {
    const size_t need = gemm_workspace_bytes(p.fmt, p.m, p.n, p.k);
    const bool split = p.ws != nullptr && need > 0 && p.ws_bytes >= need;
    const Sched s = gemm_sched(p.m, p.n, p.k, split);
    KArgs a = make_args(p);
    a.ksplit = s.ksplit;
    a.kt_per = s.kt_per;
    a.tiles_m = s.tiles_m;
    a.tiles_n = s.tiles_n;
    if (s.ksplit > 1) a.partial = reinterpret_cast<float*>(p.ws);
    const dim3 grid(s.grid), block(256);
    switch (p.fmt) {
    case kNF4:
        if (p.dq) gemm_launch<kNF4, true>(s.nb, grid, a, st);
        else gemm_launch<kNF4, false>(s.nb, grid, a, st);
        break;
    case kNVFP4: gemm_launch<kNVFP4, false>(s.nb, grid, a, st); break;
    case kQ4_0: gemm_launch<kQ4_0, false>(s.nb, grid, a, st); break;
    case kQ4_1: gemm_launch<kQ4_1, false>(s.nb, grid, a, st); break;
    case kQ5_0: gemm_launch<kQ5_0, false>(s.nb, grid, a, st); break;
    case kQ4_K: gemm_launch<kQ4_K, false>(s.nb, grid, a, st); break;
    case kQ6_K: gemm_launch<kQ6_K, false>(s.nb, grid, a, st); break;
    case kQ8_0: gemm_launch<kQ8_0, false>(s.nb, grid, a, st); break;
    default: return hipErrorInvalidValue;
    }
    if (s.ksplit > 1) {
        const int64_t nquads = p.m * (p.n / 4);
        const int gs = (int)(p.fmt == kNVFP4);
        if (s.ksplit == 2)
            hipLaunchKernelGGL(k_splitk_reduce_n<2>, dim3((unsigned)((nquads + 511) / 512)), dim3(256), 0, st, a, gs);
        else if (s.ksplit == 4)
            hipLaunchKernelGGL(k_splitk_reduce_n<4>, dim3((unsigned)((nquads + 511) / 512)), dim3(256), 0, st, a, gs);
        else
            hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((nquads + 511) / 512)), dim3(256), 0, st, a, gs);
    }
    return hipGetLastError();
}

}  // namespace wq
