// wq_launch.h -- host-side launchers implemented by the kernel translation units
// and called by the C ABI layer after it has validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

// Offsets inside the scales buffer (bytes).
struct ScaleLayout {
    int64_t nb;        // number of blocks
    int64_t ng;        // NF4+DQ: number of 256-block groups
    int64_t d_off;     // NF4+DQ: fp32 d[ng]
    int64_t mu_off;    // NF4+DQ: fp32 mean
    int64_t g_off;     // NVFP4: fp32 global scale
    int64_t hb_off;    // Q5_0: 32-bit fifth-bit words, one per block, tile order
    int64_t kd_off;    // Q4_K: fp16 (d, dmin) per super-block; Q6_K: fp16 d per super-block;
                       //   row-major [n][k/256]
    int64_t bytes;     // total scales bytes
};

ScaleLayout scale_layout(int fmt, bool dq, int64_t n, int64_t k);

hipError_t launch_quantize(int fmt, bool dq, int64_t n, int64_t k, const float* w,
                           uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_dequantize(int fmt, bool dq, int64_t n, int64_t k, const uint8_t* codes,
                             const uint8_t* scales, float* out, hipStream_t s);

// Output description shared by the matmul kernels: columns [0, end0) -> y0,
// [end0, end1) -> y1, [end1, n) -> y2.
struct OutSplit {
    void* y[3];
    int64_t ldy[3];
    int64_t end[3];   // exclusive column end of each split (end[nsplit-1] == n)
    int nsplit;
    int f32;          // 1: fp32 output, 0: bf16
};

struct MatmulProblem {
    int fmt;
    bool dq;
    int64_t m, n, k;
    const uint16_t* x;
    int64_t ldx;
    const uint8_t* codes;
    const uint8_t* scales;
    const uint16_t* bias;
    OutSplit out;
    void* ws;
    size_t ws_bytes;
    const float* gscale;   // NVFP4: epilogue factor in device memory; null = the weights' global scale
};

// Workspace bytes the schedule for (fmt, m, n, k) would like (0 = none).
size_t matmul_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k);

hipError_t launch_gemv(const MatmulProblem& p, hipStream_t s);   // m <= 16
hipError_t launch_gemm(const MatmulProblem& p, hipStream_t s);   // m >= 17

size_t gemv_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k);
size_t gemm_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k);

// NVFP4 activations (act.hip): packed row-major codes [m][k/2] and scales [m][k/16]
// followed by the fp32 global scale at align16(m*k/16).
int64_t act_scales_bytes(int64_t m, int64_t k);
hipError_t launch_quantize_act(int64_t m, int64_t k, const uint16_t* x, int64_t ldx, uint8_t* codes,
                               uint8_t* scales, hipStream_t s);
// xe[m][k] = bf16(+-e2m1 * s) (exact) and *gprod = g_w * g_x, with g_w read at gw.
hipError_t launch_expand_act(int64_t m, int64_t k, const uint8_t* codes, const uint8_t* scales,
                             const uint8_t* gw, uint16_t* xe, float* gprod, hipStream_t s);

}  // namespace wq
