// wq_device.h -- device-side helpers shared by the libwq HIP kernels:
// format constants, scalar codecs, packed-layout index maps, bf16 helpers.
//
// Formats: NF4 ("asr: add a 4-bit nf4 option for the Whisper engine", "What's
// here"), NVFP4 ("asr: add a 4-bit nvfp4 option for cards short of VRAM", intro;
// "mbehr90/whisper-large-v3-turbo-nvfp4", "What is quantized"), q4_0 / q8_0
// ("Run quantized Whisper on the fused Metal decode path", "Summary"); q4_1, q5_0,
// q4_k and q6_k (same page, "Why the policy").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nf4_table.h"

namespace wq {

enum Fmt : int { kNF4 = 1, kNVFP4 = 2, kQ4_0 = 3, kQ8_0 = 4, kQ4_1 = 5, kQ5_0 = 6, kQ4_K = 7, kQ6_K = 8 };

// ---------------------------------------------------------------------------
// Packed layout.
// 4-bit formats: tiles of 16 rows x 128 K (1 KiB), band-major, K-fastest.  Slot
// s (16 bytes) of a tile holds row s%16 and K-chunk h = s/16; byte 4j + i/2 of a
// slot holds k = 32j + 8h + i, even i in the low nibble.  So the 32-bit word j of
// slot s carries 8 consecutive k (nibble i at bits 4i), exactly the 8 bf16 values
// lane s feeds to a 16x16x32 MFMA as its B operand for K-slice j.
// q8_0: tiles of 16 rows x 64 K, byte 8j + i of slot s holds k = 32j + 8h + i.
// ---------------------------------------------------------------------------
constexpr int kTileRows = 16;
constexpr int kTileBytes = 1024;

__host__ __device__ constexpr int tile_k(int fmt) { return fmt == kQ8_0 ? 64 : 128; }
__host__ __device__ constexpr int block_k(int fmt) {
    return fmt == kNF4 ? 64 : (fmt == kNVFP4 || fmt == kQ6_K) ? 16 : 32;
}
// scale entries per row per tile
__host__ __device__ constexpr int blocks_per_tile_row(int fmt) { return tile_k(fmt) / block_k(fmt); }

__host__ __device__ inline int64_t align16(int64_t v) { return (v + 15) & ~int64_t(15); }

// ---------------------------------------------------------------------------
// Scalar codecs (device).
// ---------------------------------------------------------------------------

// E4M3 (OCP, FN) value of a non-negative code (sign bit not used by scales).
__device__ inline float e4m3_value(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    const float sub = (float)m * 0.001953125f;                       // m * 2^-9, exact
    const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20)); // (1+m/8) * 2^(e-7)
    return e == 0u ? sub : nrm;
}

// Round a non-negative float to E4M3 (nearest, ties to even code), saturating to
// 448 (code 0x7E).  The value is scaled by a power of two so that the binade's
// quantum is 1 and rintf (ties-to-even) picks the significand.
__device__ inline uint32_t e4m3_round(float x) {
    if (!(x < 448.0f)) return 0x7Eu;
    if (x < 0.015625f) {                                       // below 2^-6: quantum 2^-9
        return (uint32_t)rintf(x * 512.0f);                    // 0..8 (8 = smallest normal)
    }
    int E = (int)((__float_as_uint(x) >> 23) & 255u) - 127;   // x in [2^E, 2^(E+1))
    float q = rintf(ldexpf(x, 3 - E));                         // 8..16
    return (uint32_t)(((E + 7) << 3) + ((int)q - 8));
}

// E2M1 magnitude code of |y| (nearest of 0,.5,1,1.5,2,3,4,6; ties to the even code;
// above 6 saturates to code 7), written as a count of thresholds passed.
__device__ inline uint32_t e2m1_mag_code(float y) {
    float a = fabsf(y);
    return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
           (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
           (uint32_t)(a > 5.0f);
}

__device__ inline float e2m1_mag_value(uint32_t c) {
    // 0, .5, 1, 1.5, 2, 3, 4, 6
    return c < 4 ? 0.5f * (float)c : (float)(1u << ((c >> 1) - 1)) * (1.0f + 0.5f * (float)(c & 1u));
}

// binary16 with round-to-nearest-even, saturating to +-65504.
__device__ inline uint16_t f16_sat_bits(float x) {
    float c = fminf(fabsf(x), 65504.0f);
    _Float16 h = (_Float16)copysignf(c, x);
    return __builtin_bit_cast(uint16_t, h);
}

__device__ inline float f16_value(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

__device__ inline float bf16_value(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ inline uint16_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ inline float nf4_level(uint32_t c) { return __uint_as_float(kNf4LevelBits[c & 15u]); }

}  // namespace wq
