// wq_api.cpp -- the C ABI of libwq (declared in include/wq.h).
//
// Every argument is checked on the host before anything is enqueued; a failed
// check returns a status and launches nothing ("fails loudly" rather than running
// unquantized: "asr: add a 4-bit nf4 option for the Whisper engine", "What's
// here"; an actionable error before any work: same page, "Verified").  There is
// no dense or unfused fallback.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "wq.h"
#include "wq_launch.h"

namespace {

struct Desc {
    int fmt;
    bool dq;
    int64_t n, k;
};

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

wq_status check_desc(const wq_desc* d, Desc* out) {
    if (!d) return WQ_ERR_INVALID_ARG;
    if (d->reserved != 0) return WQ_ERR_INVALID_ARG;
    int bk;
    switch (d->format) {
    case WQ_NF4: bk = 64; break;
    case WQ_NVFP4: bk = 16; break;
    case WQ_Q4_0:
    case WQ_Q4_1:
    case WQ_Q5_0:
    case WQ_Q8_0: bk = 32; break;
    case WQ_Q4_K:
    case WQ_Q6_K: bk = 256; break;
    default: return WQ_ERR_INVALID_ARG;
    }
    if (d->block != 0 && d->block != bk) return WQ_ERR_UNSUPPORTED;
    if (d->format == WQ_NF4) {
        if (d->dq_group != 0 && d->dq_group != 256) return WQ_ERR_UNSUPPORTED;
    } else if (d->dq_group != 0) {
        return WQ_ERR_UNSUPPORTED;
    }
    const int64_t tk = d->format == WQ_Q8_0 ? 64 : (d->format == WQ_Q4_K || d->format == WQ_Q6_K) ? 256 : 128;
    if (d->n <= 0 || d->k <= 0 || d->n % 16 != 0 || d->k % tk != 0) return WQ_ERR_SHAPE;
    if (d->n > (int64_t(1) << 40) / d->k) return WQ_ERR_SHAPE;   // keep every byte offset far from overflow
    if (d->k > (int64_t(1) << 24)) return WQ_ERR_SHAPE;           // a band's codes within one 32-bit buffer range
    out->fmt = d->format;
    out->dq = d->format == WQ_NF4 && d->dq_group == 256;
    out->n = d->n;
    out->k = d->k;
    return WQ_OK;
}

wq_status check_packed(const wq_packed& w) {
    if (!w.codes || !w.scales) return WQ_ERR_INVALID_ARG;
    if (!aligned(w.codes, 16) || !aligned(w.scales, 16)) return WQ_ERR_ALIGNMENT;
    return WQ_OK;
}

wq_status from_hip(hipError_t e) { return e == hipSuccess ? WQ_OK : WQ_ERR_HIP; }

// Output columns and row strides of a matmul call travel as 32-bit kernel arguments.
constexpr int64_t kMaxOut = 0x7FFFFFFF;

// Common checks of a matmul call; fills everything of the problem except the outputs.
wq_status check_matmul(const wq_desc* d, int64_t m, const uint16_t* x, int64_t ldx, wq_packed w,
                       const uint16_t* bias, int32_t ydt, void* ws, size_t ws_bytes, wq::MatmulProblem* p) {
    Desc dd;
    wq_status st = check_desc(d, &dd);
    if (st != WQ_OK) return st;
    if ((st = check_packed(w)) != WQ_OK) return st;
    if (m < 0 || m > 0x7FFFFFFF) return WQ_ERR_SHAPE;
    if (dd.n > kMaxOut) return WQ_ERR_SHAPE;   // output columns (and split ends) as 32-bit kernel arguments
    if (!x) return WQ_ERR_INVALID_ARG;
    if (ldx < dd.k || ldx % 8 != 0 || ldx > (int64_t(1) << 24)) return WQ_ERR_INVALID_ARG;   // 128 rows of X < 4 GiB
    if (!aligned(x, 16)) return WQ_ERR_ALIGNMENT;
    if (bias && !aligned(bias, 2)) return WQ_ERR_ALIGNMENT;
    if (ydt != WQ_BF16 && ydt != WQ_F32) return WQ_ERR_INVALID_ARG;
    if (ws) {
        if (!aligned(ws, 16)) return WQ_ERR_ALIGNMENT;
        if (m > 0 && ws_bytes < wq::matmul_workspace_bytes(dd.fmt, m, dd.n, dd.k)) return WQ_ERR_WORKSPACE;
    }
    p->fmt = dd.fmt;
    p->dq = dd.dq;
    p->m = m;
    p->n = dd.n;
    p->k = dd.k;
    p->x = x;
    p->ldx = ldx;
    p->codes = static_cast<const uint8_t*>(w.codes);
    p->scales = static_cast<const uint8_t*>(w.scales);
    p->bias = bias;
    p->ws = ws;
    p->ws_bytes = ws_bytes;
    p->out.f32 = ydt == WQ_F32;
    return WQ_OK;
}

int64_t floor_div(int64_t a, int64_t b) {   // b > 0
    const int64_t q = a / b;
    return (a % b != 0 && a < 0) ? q - 1 : q;
}

// Do two strided output windows share a byte?  Window i covers rows r = 0..m-1, each the
// byte range [base_i + r*ld_i*es, base_i + r*ld_i*es + w_i*es).  Row r1 of A meets row r2
// of B iff b + r2*lb < a_hi and b + r2*lb + wb > a_lo, an interval of r2 that is solved
// in closed form; with equal strides r2 - r1 is the only unknown, so one interval covers
// every row.
bool windows_overlap(const void* pa, int64_t lda, int64_t wa, const void* pb, int64_t ldb, int64_t wb,
                     int64_t m, int64_t es) {
    const int64_t a = (int64_t)reinterpret_cast<uintptr_t>(pa), b = (int64_t)reinterpret_cast<uintptr_t>(pb);
    const int64_t la = lda * es, lb = ldb * es, na = wa * es, nb = wb * es;
    if (la == lb) {
        // rows r1, r2 = r1 + t meet iff -nb < (b - a) + t*la < na, for some |t| <= m - 1
        const int64_t d = b - a;
        const int64_t tmin = floor_div(-nb - d, la) + 1, tmax = -floor_div(-(na - d), la) - 1;
        return std::max<int64_t>(tmin, -(m - 1)) <= std::min<int64_t>(tmax, m - 1);
    }
    for (int64_t r1 = 0; r1 < m; r1++) {
        const int64_t lo = a + r1 * la, hi = lo + na;
        const int64_t r2min = floor_div(lo - nb - b, lb) + 1, r2max = -floor_div(-(hi - b), lb) - 1;
        if (std::max<int64_t>(r2min, 0) <= std::min<int64_t>(r2max, m - 1)) return true;
    }
    return false;
}

// NVFP4 activations: k a multiple of 16 and m*k <= 2^34 (chunk indices of 8 values fit 32 bits).
bool act_shape_ok(int64_t m, int64_t k) {
    if (m < 0 || k <= 0 || k % 16 != 0 || k > (int64_t(1) << 24)) return false;
    return m <= (int64_t(1) << 34) / k;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

size_t w4a4_workspace(int64_t m, int64_t n, int64_t k) {
    return 256 + align256((size_t)m * (size_t)k * 2) + wq::matmul_workspace_bytes(WQ_NVFP4, m, n, k);
}

wq_status run_matmul(const wq::MatmulProblem& p, void* stream) {
    if (p.m == 0) return WQ_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return from_hip(p.m <= 16 ? wq::launch_gemv(p, s) : wq::launch_gemm(p, s));
}

// Device scratch of the allocation-free entry point: the fp32 partial sums of a K-split GEMM.
// The split schedule never asks for more than 16 MiB (fewer than 128 output tiles of at
// most 128 x 128, times at most 256 / tiles pieces, times 4 bytes).  Each GPU the library
// runs on holds its own copy of this array from module load until the process ends.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The device address of the current device's copy of `scratch`, looked up once per device
// with that device current.  In host code the array's name is only a host-side stand-in.
wq_status scratch_for_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return WQ_ERR_HIP;
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) return WQ_ERR_HIP;
    *out = g_scratch_ptr[dev];
    return WQ_OK;
}

}  // namespace

extern "C" {

const char* wq_status_str(wq_status s) {
    switch (s) {
    case WQ_OK: return "WQ_OK";
    case WQ_ERR_INVALID_ARG: return "WQ_ERR_INVALID_ARG";
    case WQ_ERR_UNSUPPORTED: return "WQ_ERR_UNSUPPORTED";
    case WQ_ERR_SHAPE: return "WQ_ERR_SHAPE";
    case WQ_ERR_ALIGNMENT: return "WQ_ERR_ALIGNMENT";
    case WQ_ERR_MIXED_FORMAT: return "WQ_ERR_MIXED_FORMAT";
    case WQ_ERR_WORKSPACE: return "WQ_ERR_WORKSPACE";
    case WQ_ERR_HIP: return "WQ_ERR_HIP";
    }
    return "WQ_ERR_UNKNOWN";
}

wq_status wq_packed_size(const wq_desc* d, size_t* codes_bytes, size_t* scales_bytes) {
    Desc dd;
    wq_status st = check_desc(d, &dd);
    if (st != WQ_OK) return st;
    if (!codes_bytes || !scales_bytes) return WQ_ERR_INVALID_ARG;
    *codes_bytes = (size_t)(dd.fmt == WQ_Q8_0 ? dd.n * dd.k : dd.fmt == WQ_Q6_K ? dd.n * dd.k / 4 * 3 : dd.n * dd.k / 2);
    *scales_bytes = (size_t)wq::scale_layout(dd.fmt, dd.dq, dd.n, dd.k).bytes;
    return WQ_OK;
}

wq_status wq_quantize(const wq_desc* d, const float* w, wq_packed out, void* stream) {
    Desc dd;
    wq_status st = check_desc(d, &dd);
    if (st != WQ_OK) return st;
    if ((st = check_packed(out)) != WQ_OK) return st;
    if (!w) return WQ_ERR_INVALID_ARG;
    if (!aligned(w, 16)) return WQ_ERR_ALIGNMENT;
    return from_hip(wq::launch_quantize(dd.fmt, dd.dq, dd.n, dd.k, w, static_cast<uint8_t*>(out.codes),
                                        static_cast<uint8_t*>(out.scales), static_cast<hipStream_t>(stream)));
}

wq_status wq_dequantize(const wq_desc* d, wq_packed in, float* w_out, void* stream) {
    Desc dd;
    wq_status st = check_desc(d, &dd);
    if (st != WQ_OK) return st;
    if ((st = check_packed(in)) != WQ_OK) return st;
    if (!w_out) return WQ_ERR_INVALID_ARG;
    if (!aligned(w_out, 16)) return WQ_ERR_ALIGNMENT;
    return from_hip(wq::launch_dequantize(dd.fmt, dd.dq, dd.n, dd.k, static_cast<const uint8_t*>(in.codes),
                                          static_cast<const uint8_t*>(in.scales), w_out, static_cast<hipStream_t>(stream)));
}

wq_status wq_workspace_size(const wq_desc* d, int64_t m, size_t* bytes) {
    Desc dd;
    wq_status st = check_desc(d, &dd);
    if (st != WQ_OK) return st;
    if (!bytes) return WQ_ERR_INVALID_ARG;
    if (m < 0 || m > 0x7FFFFFFF) return WQ_ERR_SHAPE;
    *bytes = m == 0 ? 0 : wq::matmul_workspace_bytes(dd.fmt, m, dd.n, dd.k);
    return WQ_OK;
}

wq_status wq_matmul(const wq_desc* d, int64_t m, const uint16_t* x, int64_t ldx, wq_packed w,
                    const uint16_t* bias, void* y, int32_t ydt, int64_t ldy, void* ws, size_t ws_bytes,
                    void* stream) {
    wq::MatmulProblem p{};
    wq_status st = check_matmul(d, m, x, ldx, w, bias, ydt, ws, ws_bytes, &p);
    if (st != WQ_OK) return st;
    if (!y) return WQ_ERR_INVALID_ARG;
    if (!aligned(y, ydt == WQ_F32 ? 4 : 2)) return WQ_ERR_ALIGNMENT;
    if (ldy < p.n || ldy > kMaxOut) return WQ_ERR_INVALID_ARG;
    p.out.nsplit = 1;
    p.out.y[0] = y;
    p.out.ldy[0] = ldy;
    p.out.end[0] = p.out.end[1] = p.out.end[2] = p.n;
    return run_matmul(p, stream);
}

wq_status wq_matmul_noalloc(const wq_desc* d, int64_t m, const uint16_t* x, int64_t ldx, wq_packed w,
                            const uint16_t* bias, void* y, int32_t ydt, int64_t ldy, void* stream) {
    wq::MatmulProblem p{};
    wq_status st = check_matmul(d, m, x, ldx, w, bias, ydt, nullptr, 0, &p);
    if (st != WQ_OK) return st;
    if (!y) return WQ_ERR_INVALID_ARG;
    if (!aligned(y, ydt == WQ_F32 ? 4 : 2)) return WQ_ERR_ALIGNMENT;
    if (ldy < p.n || ldy > kMaxOut) return WQ_ERR_INVALID_ARG;
    if (m == 0) return WQ_OK;
    const size_t need = wq::matmul_workspace_bytes(p.fmt, p.m, p.n, p.k);
    if (need > kScratchBytes) return WQ_ERR_WORKSPACE;
    if (need > 0) {
        if ((st = scratch_for_current_device(&p.ws)) != WQ_OK) return st;
        p.ws_bytes = kScratchBytes;
    }
    p.out.nsplit = 1;
    p.out.y[0] = y;
    p.out.ldy[0] = ldy;
    p.out.end[0] = p.out.end[1] = p.out.end[2] = p.n;
    return run_matmul(p, stream);
}

wq_status wq_matmul_qkv(const wq_desc* d, int64_t m, const uint16_t* x, int64_t ldx, wq_packed w,
                        const uint16_t* bias, int32_t nsplit, const int64_t* split_n, void* const* y,
                        const int64_t* ldy, int32_t ydt, void* ws, size_t ws_bytes, void* stream) {
    wq::MatmulProblem p{};
    wq_status st = check_matmul(d, m, x, ldx, w, bias, ydt, ws, ws_bytes, &p);
    if (st != WQ_OK) return st;
    if (nsplit != 2 && nsplit != 3) return WQ_ERR_INVALID_ARG;
    if (!split_n || !y || !ldy) return WQ_ERR_INVALID_ARG;
    int64_t sum = 0;
    for (int i = 0; i < nsplit; i++) {
        if (split_n[i] <= 0) return WQ_ERR_SHAPE;
        sum += split_n[i];
    }
    if (sum != p.n) return WQ_ERR_SHAPE;
    for (int i = 0; i < nsplit; i++) {
        if (!y[i]) return WQ_ERR_INVALID_ARG;
        if (!aligned(y[i], ydt == WQ_F32 ? 4 : 2)) return WQ_ERR_ALIGNMENT;
        if (ldy[i] < split_n[i] || ldy[i] > kMaxOut) return WQ_ERR_INVALID_ARG;
    }
    // the splits' destination windows must be disjoint (every output element is written once)
    const int64_t es = ydt == WQ_F32 ? 4 : 2;
    for (int i = 0; i < nsplit; i++)
        for (int j = i + 1; j < nsplit; j++)
            if (m > 0 && windows_overlap(y[i], ldy[i], split_n[i], y[j], ldy[j], split_n[j], m, es))
                return WQ_ERR_INVALID_ARG;
    p.out.nsplit = nsplit;
    int64_t e = 0;
    for (int i = 0; i < 3; i++) {
        if (i < nsplit) {
            e += split_n[i];
            p.out.y[i] = y[i];
            p.out.ldy[i] = ldy[i];
        } else {
            p.out.y[i] = y[nsplit - 1];
            p.out.ldy[i] = ldy[nsplit - 1];
        }
        p.out.end[i] = e;
    }
    return run_matmul(p, stream);
}

wq_status wq_act_packed_size(int64_t m, int64_t k, size_t* codes_bytes, size_t* scales_bytes) {
    if (!codes_bytes || !scales_bytes) return WQ_ERR_INVALID_ARG;
    if (!act_shape_ok(m, k)) return WQ_ERR_SHAPE;
    *codes_bytes = (size_t)(m * k / 2);
    *scales_bytes = (size_t)wq::act_scales_bytes(m, k);
    return WQ_OK;
}

wq_status wq_quantize_act(int64_t m, int64_t k, const uint16_t* x, int64_t ldx, void* codes, void* scales,
                          void* stream) {
    if (!act_shape_ok(m, k)) return WQ_ERR_SHAPE;
    if (!x || !codes || !scales) return WQ_ERR_INVALID_ARG;
    if (ldx < k || ldx % 8 != 0 || ldx > (int64_t(1) << 24)) return WQ_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 16)) return WQ_ERR_ALIGNMENT;
    if (m == 0) return WQ_OK;
    return from_hip(wq::launch_quantize_act(m, k, x, ldx, static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales),
                                            static_cast<hipStream_t>(stream)));
}

wq_status wq_w4a4_workspace_size(const wq_desc* d, int64_t m, size_t* bytes) {
    Desc dd;
    wq_status st = check_desc(d, &dd);
    if (st != WQ_OK) return st;
    if (dd.fmt != WQ_NVFP4) return WQ_ERR_UNSUPPORTED;
    if (!bytes) return WQ_ERR_INVALID_ARG;
    if (m < 0 || m > 0x7FFFFFFF || !act_shape_ok(m, dd.k)) return WQ_ERR_SHAPE;
    *bytes = m == 0 ? 0 : w4a4_workspace(m, dd.n, dd.k);
    return WQ_OK;
}

wq_status wq_matmul_w4a4(const wq_desc* d, int64_t m, const void* xcodes, const void* xscales, wq_packed w,
                         const uint16_t* bias, void* y, int32_t ydt, int64_t ldy, void* ws, size_t ws_bytes,
                         void* stream) {
    Desc dd;
    wq_status st = check_desc(d, &dd);
    if (st != WQ_OK) return st;
    if (dd.fmt != WQ_NVFP4) return WQ_ERR_UNSUPPORTED;
    if (m < 0 || m > 0x7FFFFFFF || !act_shape_ok(m, dd.k)) return WQ_ERR_SHAPE;
    if (!xcodes || !xscales) return WQ_ERR_INVALID_ARG;
    if (!aligned(xcodes, 16) || !aligned(xscales, 16)) return WQ_ERR_ALIGNMENT;
    if (m > 0) {
        if (!ws || ws_bytes < w4a4_workspace(m, dd.n, dd.k)) return WQ_ERR_WORKSPACE;
        if (!aligned(ws, 16)) return WQ_ERR_ALIGNMENT;
    }
    // workspace: [0, 256) the epilogue factor g_w * g_x; then the expanded activations
    // X'[m][k] (bf16); then the matmul's own workspace
    uint8_t* const base = static_cast<uint8_t*>(ws);
    const size_t xe_bytes = align256((size_t)m * (size_t)dd.k * 2);
    // (m == 0: X' is never read; the codes pointer stands in for it in the checks)
    const uint16_t* const xe = m > 0 ? reinterpret_cast<const uint16_t*>(base + 256) : static_cast<const uint16_t*>(xcodes);
    void* const mws = m > 0 ? base + 256 + xe_bytes : nullptr;
    const size_t mws_bytes = m > 0 ? ws_bytes - 256 - xe_bytes : 0;
    wq::MatmulProblem p{};
    st = check_matmul(d, m, xe, dd.k, w, bias, ydt, mws, mws_bytes, &p);
    if (st != WQ_OK) return st;
    if (!y) return WQ_ERR_INVALID_ARG;
    if (!aligned(y, ydt == WQ_F32 ? 4 : 2)) return WQ_ERR_ALIGNMENT;
    if (ldy < p.n || ldy > kMaxOut) return WQ_ERR_INVALID_ARG;
    if (m == 0) return WQ_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const wq::ScaleLayout L = wq::scale_layout(dd.fmt, false, dd.n, dd.k);
    float* const gprod = reinterpret_cast<float*>(base);
    hipError_t e = wq::launch_expand_act(m, dd.k, static_cast<const uint8_t*>(xcodes),
                                         static_cast<const uint8_t*>(xscales), p.scales + L.g_off,
                                         reinterpret_cast<uint16_t*>(base + 256), gprod, s);
    if (e != hipSuccess) return WQ_ERR_HIP;
    p.gscale = gprod;
    p.out.nsplit = 1;
    p.out.y[0] = y;
    p.out.ldy[0] = ldy;
    p.out.end[0] = p.out.end[1] = p.out.end[2] = p.n;
    return run_matmul(p, stream);
}

}  // extern "C"
