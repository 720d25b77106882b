// gemm_nvfp4_wide.hip -- the 128 x 256 NVFP4 GEMM kernel in a translation unit of its
// own, built with the compiler's default instruction scheduler: that scheduler gives
// this kernel its fastest register allocation, while the iterative ILP scheduler that
// gemm.hip is built with suits every other GEMM kernel (build.py).
#include "gemm_kernel.h"

namespace wq {

void gemm_launch_nvfp4_nb4(dim3 grid, const KArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((k_gemm<kNVFP4, false, 4>), grid, dim3(256), 0, st, a);
}

}  // namespace wq
