// gemm.hip -- the encoder GEMM (m >= 17): schedule and launchers.  The kernels
// (gemm_kernel.h) are instantiated here, except the 128 x 256 NVFP4 kernel, which
// gemm_nvfp4_wide.hip builds with the compiler's default instruction scheduler
// (this file is built with the iterative ILP scheduler; see build.py).
#include "gemm_kernel.h"

namespace wq {

// k_gemm<kNVFP4, false, 4>, launched from the translation unit that instantiates it.
void gemm_launch_nvfp4_nb4(dim3 grid, const KArgs& a, hipStream_t st);

// ---------------------------------------------------------------------------
// Schedules and launchers.
// ---------------------------------------------------------------------------
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
    const int64_t steps = (k + BK - 1) / BK;
    const int64_t tiles = s.tiles_m * s.tiles_n;
    int ks = 1;
    if (allow_split && tiles < kNumCU / 2) {
        while (tiles * ks * 2 <= kNumCU && steps / (ks * 2) >= kMinPieceSteps) ks *= 2;
    }
    s.ksplit = ks;                        // a power of two: k_gemm derives its pieces with a shift
    s.kt_per = (steps + ks - 1) / ks;     // every piece non-empty: (ks - 1) * kt_per < steps
    const int64_t items = tiles * ks;
    s.grid = (unsigned)(((items + 7) / 8) * 8);
    return s;
}

size_t gemm_workspace_bytes(int fmt, int64_t m, int64_t n, int64_t k) {
    (void)fmt;
    const Sched s = gemm_sched(m, n, k, true);
    return s.ksplit <= 1 ? 0 : (size_t)s.ksplit * (size_t)m * (size_t)n * 4u;
}

template <int FMT, bool DQ>
static void gemm_launch(int nb, dim3 grid, const KArgs& a, hipStream_t st) {
    if (nb == 2) {
        hipLaunchKernelGGL((k_gemm<FMT, DQ, 2>), grid, dim3(256), 0, st, a);
    } else if constexpr (FMT == kNVFP4 && !DQ) {
        gemm_launch_nvfp4_nb4(grid, a, st);
    } else {
        hipLaunchKernelGGL((k_gemm<FMT, DQ, 4>), grid, dim3(256), 0, st, a);
    }
}

hipError_t launch_gemm(const MatmulProblem& p, hipStream_t st) {
    const size_t need = gemm_workspace_bytes(p.fmt, p.m, p.n, p.k);
    const bool split = p.ws != nullptr && need > 0 && p.ws_bytes >= need;
    const Sched s = gemm_sched(p.m, p.n, p.k, split);
    KArgs a = make_args(p);
    a.ksplit = s.ksplit;
    // the GEMM launch of a K split writes partials, not outputs: its y0 slot carries them
    KArgs ag = a;
    float* const partial = reinterpret_cast<float*>(p.ws);
    if (s.ksplit > 1) ag.partial = partial;
    const dim3 grid(s.grid), block(256);
    switch (p.fmt) {
    case kNF4:
        if (p.dq) gemm_launch<kNF4, true>(s.nb, grid, ag, st);
        else gemm_launch<kNF4, false>(s.nb, grid, ag, st);
        break;
    case kNVFP4: gemm_launch<kNVFP4, false>(s.nb, grid, ag, st); break;
    case kQ4_0: gemm_launch<kQ4_0, false>(s.nb, grid, ag, st); break;
    case kQ4_1: gemm_launch<kQ4_1, false>(s.nb, grid, ag, st); break;
    case kQ5_0: gemm_launch<kQ5_0, false>(s.nb, grid, ag, st); break;
    case kQ4_K: gemm_launch<kQ4_K, false>(s.nb, grid, ag, st); break;
    case kQ6_K: gemm_launch<kQ6_K, false>(s.nb, grid, ag, st); break;
    case kQ8_0: gemm_launch<kQ8_0, false>(s.nb, grid, ag, st); break;
    default: return hipErrorInvalidValue;
    }
    if (s.ksplit > 1) {
        const int64_t nquads = p.m * (p.n / 4);
        KArgs ar = a;
        ar.rpartial = partial;
        ar.rfactor = p.fmt == kNVFP4 ? reinterpret_cast<const float*>(a.gs) : nullptr;
        const dim3 rgrid((unsigned)((nquads + 256 * kRedQ - 1) / (256 * kRedQ)));
        if (s.ksplit == 2) hipLaunchKernelGGL(k_splitk_reduce_n<2>, rgrid, dim3(256), 0, st, ar);
        else if (s.ksplit == 4) hipLaunchKernelGGL(k_splitk_reduce_n<4>, rgrid, dim3(256), 0, st, ar);
        else hipLaunchKernelGGL(k_splitk_reduce_n<0>, rgrid, dim3(256), 0, st, ar);
    }
    return hipGetLastError();
}
}  // namespace wq
