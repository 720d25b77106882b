// act.hip -- NVFP4 activations for the W4A4 product.
//
// "mbehr90/whisper-large-v3-turbo-nvfp4", section "What is quantized": besides the
// NVFP4 weights, activations are quantized per 16-value group at run time, and the
// product is then W4A4 (section "Honest summary": true W4A4 on Blackwell).
//
// Quantization applies the weights' NVFP4 rule to X[m][k] (bf16, widened exactly):
// g = absmax(X) / 2688 (one fp32 global scale per call), per 16 consecutive k an
// E4M3 scale s = E4M3(block absmax / (6g)), codes E2M1(x / (s*g)), sign kept.
// Packed activations are plain row-major: codes [m][k/2] (element 2j of a row in the
// low nibble of byte j), scales [m][k/16], the fp32 g at byte align16(m*k/16) of the
// scales buffer (pad bytes zero).
//
// The contraction: every product term is x^ * w^ = (e2m1_x * s_x)(e2m1_w * s_w) g_x g_w,
// and e2m1 * s has at most 6 significant bits, so it is exact in bf16.  The W4A4
// matmul expands the packed activations to those exact bf16 values and runs the
// NVFP4 matmul kernels with the single epilogue factor g_w * g_x.  (gfx950's FP4
// MFMA takes one power-of-two scale per 32 values, which cannot carry an E4M3
// scale per 16 values without extra passes; the bf16 MFMA carries it exactly.)
#include <hip/hip_runtime.h>

#include <algorithm>

#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

namespace {

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// The 8 bf16 values of chunk c (row c / k8, columns 8 (c % k8) ..), widened.
__device__ inline void load_chunk(const uint16_t* __restrict__ x, int64_t ldx, uint32_t k8, uint32_t c, float v[8]) {
    const uint32_t row = c / k8, col8 = c - row * k8;
    const u16x8 u = *reinterpret_cast<const u16x8*>(x + (int64_t)row * ldx + (int64_t)col8 * 8);
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = bf16_value(u[i]);
}

}  // namespace

// Each workgroup of 256 threads covers a run of kChunksPerWg chunks of 8 values; thread t
// takes chunks t, t + 256, t + 512, t + 768 of the run (each 64-lane load instruction
// reads 1 KiB of consecutive bytes) and issues all of its loads before using any.
constexpr uint32_t kUnroll = 4;
constexpr uint32_t kChunksPerWg = 256 * kUnroll;

// Per-workgroup partial absmax of X (grid-stride over runs).
__global__ __launch_bounds__(256) void k_act_absmax_partial(const uint16_t* __restrict__ x, int64_t ldx, uint32_t k8,
                                                            uint32_t chunks, float* __restrict__ partial) {
    __shared__ float red[4];
    float m = 0.0f;
    for (uint32_t c0 = blockIdx.x * kChunksPerWg + threadIdx.x; c0 < chunks; c0 += gridDim.x * kChunksPerWg) {
        // indices past the end re-read the last chunk (the maximum is unchanged), so that
        // every load is unconditional and all of them are in flight together
        float v[kUnroll][8];
#pragma unroll
        for (uint32_t u = 0; u < kUnroll; u++) load_chunk(x, ldx, k8, min(c0 + u * 256, chunks - 1), v[u]);
#pragma unroll
        for (uint32_t u = 0; u < kUnroll; u++)
#pragma unroll
            for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(v[u][i]));
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Combine the np <= 1024 partials: g = absmax / 2688 at scales + g_off; zero the pad
// bytes [nb, g_off) between the last block scale and g.
__global__ __launch_bounds__(256) void k_act_absmax_final(const float* __restrict__ partial, int np,
                                                          uint8_t* __restrict__ scales, int64_t nb, int64_t g_off) {
    __shared__ float red[4];
    float m = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const int i = threadIdx.x + 256 * u;
        if (i < np) m = fmaxf(m, partial[i]);
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (nb + threadIdx.x < g_off) scales[nb + threadIdx.x] = 0;
    if (threadIdx.x == 0)
        *reinterpret_cast<float*>(scales + g_off) = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) / 2688.0f;
}

// Codes and block scales, one chunk per thread.  Chunk c is half of a 16-value block; the
// other half is chunk c ^ 1, held by the neighbouring lane (k/8 is even).  The kernel is
// bound by VALU issue, not memory: the exact quotients x / sigma (one IEEE division per
// value, as the rule is stated) and the E2M1 threshold count take about 40 instructions
// per value, so it keeps one chunk per thread for the most waves per SIMD.
__global__ __launch_bounds__(256) void k_act_quant(const uint16_t* __restrict__ x, int64_t ldx, uint32_t k8,
                                                   uint32_t chunks, uint8_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales, int64_t g_off) {
    const uint32_t c = blockIdx.x * 256u + threadIdx.x;
    // unconditional load (a thread past the end re-reads the last chunk; both lanes of such
    // a block are past the end, and nothing is stored for them)
    float v[8];
    load_chunk(x, ldx, k8, min(c, chunks - 1), v);
    const float g = *reinterpret_cast<const float*>(scales + g_off);
    float ab = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) ab = fmaxf(ab, fabsf(v[i]));
    ab = fmaxf(ab, __shfl_xor(ab, 1, 64));
    if (c >= chunks) return;
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
    reinterpret_cast<uint32_t*>(codes)[c] = word;          // byte 4c = row * k/2 + 4 (c % k8)
    if ((c & 1u) == 0) scales[c >> 1] = (uint8_t)sb;        // byte c/2 = row * k/16 + block
}

// Expand packed activations to bf16(+-e2m1 * s) (exact), row-major [m][k], and write the
// epilogue factor fl(g_w * g_x).
__global__ __launch_bounds__(256) void k_act_expand(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                    uint32_t chunks, int64_t g_off, const uint8_t* __restrict__ gw,
                                                    uint16_t* __restrict__ xe, float* __restrict__ gprod) {
    const uint32_t c0 = blockIdx.x * kChunksPerWg + threadIdx.x;
    if (c0 == 0) *gprod = *reinterpret_cast<const float*>(gw) * *reinterpret_cast<const float*>(scales + g_off);
    uint32_t word[kUnroll], sbyte[kUnroll];
#pragma unroll
    for (uint32_t u = 0; u < kUnroll; u++) {
        const uint32_t c = min(c0 + u * 256, chunks - 1);     // unconditional loads
        word[u] = reinterpret_cast<const uint32_t*>(codes)[c];
        sbyte[u] = scales[c >> 1];
    }
#pragma unroll
    for (uint32_t u = 0; u < kUnroll; u++) {
        const uint32_t c = c0 + u * 256;
        if (c >= chunks) continue;
        const float s = e4m3_value(sbyte[u]);
        u16x8 o;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t cd = (word[u] >> (4 * i)) & 15u;
            const float mag = e2m1_mag_value(cd & 7u) * s;                         // exact, <= 6 significant bits
            o[i] = (uint16_t)((__float_as_uint(mag) >> 16) | ((cd & 8u) << 12));    // exact in bf16; sign from the code
        }
        *reinterpret_cast<u16x8*>(xe + (int64_t)c * 8) = o;
    }
}

int64_t act_scales_bytes(int64_t m, int64_t k) { return align16(m * (k / 16)) + 4; }

hipError_t launch_quantize_act(int64_t m, int64_t k, const uint16_t* x, int64_t ldx, uint8_t* codes, uint8_t* scales,
                               hipStream_t s) {
    const uint32_t chunks = (uint32_t)(m * k / 8), k8 = (uint32_t)(k / 8);
    const int64_t nb = m * (k / 16), g_off = align16(nb);
    // the partial maxima live in the codes buffer until the codes are written:
    // np <= ceil(chunks / 1024) floats, within the 4 * chunks bytes of codes
    float* partial = reinterpret_cast<float*>(codes);
    const int64_t runs = ((int64_t)chunks + kChunksPerWg - 1) / kChunksPerWg;
    const int np = (int)std::min<int64_t>(1024, std::max<int64_t>(1, runs));
    hipLaunchKernelGGL(k_act_absmax_partial, dim3(np), dim3(256), 0, s, x, ldx, k8, chunks, partial);
    hipLaunchKernelGGL(k_act_absmax_final, dim3(1), dim3(256), 0, s, partial, np, scales, nb, g_off);
    hipLaunchKernelGGL(k_act_quant, dim3((unsigned)(((int64_t)chunks + 255) / 256)), dim3(256), 0, s, x, ldx, k8, chunks,
                       codes, scales, g_off);
    return hipGetLastError();
}

hipError_t launch_expand_act(int64_t m, int64_t k, const uint8_t* codes, const uint8_t* scales, const uint8_t* gw,
                             uint16_t* xe, float* gprod, hipStream_t s) {
    const uint32_t chunks = (uint32_t)(m * k / 8);
    const int64_t g_off = align16(m * (k / 16));
    const unsigned runs = (unsigned)std::max<int64_t>(1, ((int64_t)chunks + kChunksPerWg - 1) / kChunksPerWg);
    hipLaunchKernelGGL(k_act_expand, dim3(runs), dim3(256), 0, s, codes, scales, chunks, g_off, gw, xe, gprod);
    return hipGetLastError();
}

}  // namespace wq
