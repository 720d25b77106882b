/*
 * wq.h -- libwq: weight-only 4-bit (and 5-, 6- and 8-bit) matmul with
 * dequantization fused in, for AMD Instinct MI355X (gfx950).
 *
 * Y[M,N] = X[M,K] * W^[N,K]^T + b, where X is bf16, W^ is the dequantized form
 * of a block-quantized weight matrix, accumulation is fp32.
 *
 * Formats (what the pages fix):
 *   NF4    4-bit NormalFloat codes, one absmax per 64 values along K, optional
 *          double quantization of the absmax values ("asr: add a 4-bit nf4 option
 *          for the Whisper engine", intro and "What's here": double-quant, bf16
 *          compute; the fused dequant-matmul is the reason NF4 is 1.66x and not
 *          4.1x of bf16 -- section "Why NF4 and not the NVFP4 snapshot ...").
 *   NVFP4  E2M1 codes in 16-value blocks, one E4M3 scale per block and one FP32
 *          global scale per matrix ("asr: add a 4-bit nvfp4 option for cards short
 *          of VRAM", intro; "mbehr90/whisper-large-v3-turbo-nvfp4", section "What
 *          is quantized"; run as a W4A16 GEMM -- same section).
 *   Q4_0 / Q8_0  32-value blocks with one fp16 scale and signed 4-/8-bit codes
 *          ("Run quantized Whisper on the fused Metal decode path", "Summary" and
 *          "Why the policy").
 *   Q4_1   32-value blocks with an fp16 scale and an fp16 minimum, unsigned 4-bit
 *          codes (named on the same page, "Why the policy", among the formats
 *          that decode correctly but lacked fast kernels).
 *   Q5_0   32-value blocks with one fp16 scale and signed 5-bit codes (same
 *          passage).
 *   Q4_K   256-value super-blocks of eight 32-value sub-blocks: unsigned 4-bit
 *          codes, per sub-block a 6-bit scale and a 6-bit offset, per super-block
 *          an fp16 d and an fp16 dmin (same passage).
 *   Q6_K   256-value super-blocks of sixteen 16-value sub-blocks: signed 6-bit
 *          codes, an int8 scale per sub-block, an fp16 d per super-block (same
 *          passage, as a format the encoder may use).
 * The pages leave the exact rounding rules, the NF4 levels, the double-quant
 * scheme and the storage layout open; this library fixes them as follows.
 *   NF4     levels: QLoRA's NormalFloat quantiles (binary64 construction, rounded
 *           to binary32); code = nearest level to w/absmax (ties to the lower
 *           level); double-quant: mean of the absmax values (binary64 sum in block
 *           order), int8 symmetric codes of (absmax - mean) per 256 blocks.
 *   NVFP4   global scale g = absmax(W)/2688, block scale = E4M3(block absmax /
 *           (6g)) round-to-nearest-even saturating at 448, codes E2M1 of
 *           w/(scale*g) nearest, ties to even; w^ = e2m1 * scale * g.
 *   Q8_0    d = fp16(absmax/127), q = clamp(rint(w/d), -127, 127).
 *   Q4_0    d = fp16(m/-8) with m the signed element of largest magnitude (first
 *           on ties), q = clamp(rint(w/d), -8, 7) + 8.
 *   Q4_1    d = fp16((max - min)/15), m = fp16(min), q = clamp(rint((w - m)/d),
 *           0, 15) (q = 0 when d = 0); w^ = q*d + m.
 *   Q5_0    d = fp16(m/-16) with m as for Q4_0, q = clamp(rint(w/d), -16, 15) + 16;
 *           the low 4 bits of q are stored as a 4-bit code, bit 4 in a per-block
 *           32-bit word (bit i for element i of the block).
 *   Q4_K    per sub-block s = (max - min(min, 0))/15, o = -min(min, 0); d =
 *           fp16(max s / 63), dmin = fp16(max o / 63); sc = rint(s/d), m = rint(o/dmin)
 *           in 0..63; S = d*sc, O = dmin*m; q = clamp(rint((w + O)/S), 0, 15);
 *           w^ = S*q - O.  One pass, no search over scales.
 *   Q6_K    per sub-block s = m/-32 with m as for Q4_0; d = fp16(max |s| / 127),
 *           sc = clamp(rint(s/d), -127, 127), S = d*sc; q = clamp(rint(w/S), -32,
 *           31) + 32; w^ = S*(q - 32).  The low 4 bits of q are stored as a 4-bit
 *           code, bits 4 and 5 after all the 4-bit codes (512 bytes per tile).
 *   Layout  codes in 1 KiB tiles of 16 rows x 128 K (64 K for Q8_0), ordered by
 *           16-row band then K; 16-byte slot s of a tile holds row s%16, and its
 *           32-bit word j holds k = 32j + 8(s/16) + 0..7 (Q8_0: 8-byte word j);
 *           scales are grouped per tile in row-major (row, block) order; the
 *           per-super-block values of Q4_K and Q6_K follow in a row-major
 *           [n][k/256] plane.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  libwq never
 *     allocates, frees or synchronizes; work is enqueued on `stream` (a
 *     hipStream_t; NULL = the default stream) and the call returns.
 *   - Arguments are validated on the host before anything is enqueued.  A call
 *     that returns a status other than WQ_OK has enqueued nothing.  There is no
 *     fallback to a dense or unfused path and no silent format conversion.
 *   - A HIP launch error maps to WQ_ERR_HIP.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Shapes: n > 0 and n % 16 == 0; k > 0 and k % 128 == 0 (NF4, NVFP4, Q4_0,
 *     Q4_1, Q5_0), k % 256 == 0 (Q4_K, Q6_K) or k % 64 == 0 (Q8_0); m >= 0
 *     (m == 0 is a no-op that returns WQ_OK).  k <= 2^24 and n * k <= 2^40, so that
 *     a 16-row band of codes and a 128-row tile of X (ldx <= 2^24) each stay under
 *     the 4 GiB that one buffer descriptor of the kernels addresses.
 */
#ifndef LIBWQ_WQ_H
#define LIBWQ_WQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    WQ_OK = 0,
    WQ_ERR_INVALID_ARG = 1,   /* NULL pointer, bad enum value, bad stride */
    WQ_ERR_UNSUPPORTED = 2,   /* format/block/double-quant combination not offered */
    WQ_ERR_SHAPE = 3,         /* n, k, m or split sizes violate the shape rules */
    WQ_ERR_ALIGNMENT = 4,     /* a pointer or stride is not aligned as required */
    WQ_ERR_MIXED_FORMAT = 5,  /* reserved: one descriptor always means one format */
    WQ_ERR_WORKSPACE = 6,     /* non-NULL workspace smaller than wq_workspace_size */
    WQ_ERR_HIP = 7            /* a HIP runtime call or kernel launch failed */
} wq_status;

typedef enum { WQ_NF4 = 1, WQ_NVFP4 = 2, WQ_Q4_0 = 3, WQ_Q8_0 = 4, WQ_Q4_1 = 5, WQ_Q5_0 = 6, WQ_Q4_K = 7,
               WQ_Q6_K = 8 } wq_format;

typedef enum { WQ_BF16 = 1, WQ_F32 = 2 } wq_dtype;

/* One quantized weight matrix W[n, k] (PyTorch Linear layout: [out, in]).
 *   format   : wq_format
 *   block    : 0 (= the format's block) or exactly 64 (NF4), 16 (NVFP4), 32 (Q4_0, Q8_0, Q4_1, Q5_0),
 *              256 (Q4_K, Q6_K: the super-block)
 *   n, k     : matrix shape
 *   dq_group : NF4 only: 0 = plain fp32 absmax per block, 256 = double quantization
 *              (int8 absmax codes, one fp32 scale per 256 consecutive blocks in
 *              row-major block order, one fp32 mean per matrix).  Must be 0 for
 *              the other formats. */
typedef struct {
    int32_t format;
    int32_t block;
    int64_t n;
    int64_t k;
    int32_t dq_group;
    int32_t reserved;   /* must be 0 */
} wq_desc;

/* The two device buffers holding a packed matrix; both 16-byte aligned. */
typedef struct {
    void* codes;
    void* scales;
} wq_packed;

/* Human-readable name of a status. Never NULL. */
const char* wq_status_str(wq_status s);

/* Host-only.  Bytes of the two packed buffers for descriptor d:
 *   codes : n*k/2 (4-bit formats), n*k (Q8_0) or 3*n*k/4 (Q6_K)
 *   scales: NF4 4*n*k/64; NF4+DQ align16(n*k/64) + 4*ceil(n*k/64/256) + 4;
 *           NVFP4 align16(n*k/16) + 4; Q4_0 and Q8_0 2*n*k/32; Q4_1 4*n*k/32
 *           (an fp16 pair d, m per block); Q5_0 align16(2*n*k/32) + 4*n*k/32
 *           (fp16 d per block, then one 32-bit word of fifth bits per block);
 *           Q4_K align16(2*n*k/32) + 4*n*k/256 (a 6-bit scale and offset byte per
 *           sub-block, then an fp16 pair d, dmin per super-block); Q6_K
 *           align16(n*k/16) + 2*n*k/256 (an int8 scale per 16-value sub-block, then
 *           an fp16 d per super-block). */
wq_status wq_packed_size(const wq_desc* d, size_t* codes_bytes, size_t* scales_bytes);

/* Quantize fp32 W[n,k] (row-major, leading dimension k, 16-byte aligned) into the
 * packed buffers `out` (sizes from wq_packed_size, 16-byte aligned).  Bit-exact
 * with the format definitions: codes and scales are a pure function of W.
 * W must be finite.  Uses `out.codes` as temporary storage while it runs (no
 * other scratch).  Passages: as for the formats above; NF4 quantizes one matrix
 * at a time as the checkpoint streams in ("asr: add a 4-bit nf4 option for the
 * Whisper engine", "Why NF4 and not the NVFP4 snapshot Parakeet ships"). */
wq_status wq_quantize(const wq_desc* d, const float* w, wq_packed out, void* stream);

/* Dequantize the packed matrix to fp32 W^[n,k] (row-major, leading dimension k,
 * 16-byte aligned).  Bit-exact: W^ = the format's decode of every code/scale. */
wq_status wq_dequantize(const wq_desc* d, wq_packed in, float* w_out, void* stream);

/* Host-only.  Workspace bytes wq_matmul / wq_matmul_qkv can use for an
 * m-row call with descriptor d: fp32 partial sums when the K dimension is split
 * so that shapes with few output tiles (small n at m >= 17) still spread over
 * all compute units.  0 means the call never uses one (every m <= 16 call).
 * Without a workspace (ws == NULL) the call runs with no K split; the result
 * meets the same bound.  The workspace needs no initialization; one workspace
 * must not be used by calls that may run concurrently (different streams). */
wq_status wq_workspace_size(const wq_desc* d, int64_t m, size_t* bytes);

/* Y = X * W^T + bias.
 *   x    : bf16 [m, k], leading dimension ldx >= k, ldx % 8 == 0, 16-byte aligned
 *   w    : packed matrix for d
 *   bias : bf16 [n] or NULL (2-byte aligned)
 *   y    : [m, n] of type ydt (WQ_BF16 or WQ_F32), leading dimension ldy >= n,
 *          ldy <= 2^31 - 1, aligned to its element size.  Only the m x n window is
 *          written.  (A matmul needs n <= 2^31 - 1, else WQ_ERR_SHAPE: output
 *          columns and row strides travel as 32-bit kernel arguments.)
 *   ws   : workspace (see wq_workspace_size) or NULL; ws_bytes its size
 * Accumulation is fp32 over bf16 activations times bf16-rounded (or exact)
 * dequantized weights; per element |y - y_ref| <= 4e-3 * sum_k |x_k * w^_k| + 1e-6
 * against the fp32 reference (plus the final bf16 rounding for WQ_BF16 outputs).
 * m <= 16 runs the GEMV, K split over the waves of a workgroup (decode: token-at-a-time, "asr: add a 4-bit nf4
 * option for the Whisper engine", "Why NF4 and not the NVFP4 snapshot ..."),
 * m >= 17 the MFMA GEMM (encoder frames, "mbehr90/whisper-large-v3-turbo-nvfp4",
 * "Honest summary: on H100 this is not a win"). */
wq_status wq_matmul(const wq_desc* d, int64_t m, const uint16_t* x, int64_t ldx, wq_packed w,
                    const uint16_t* bias, void* y, int32_t ydt, int64_t ldy,
                    void* ws, size_t ws_bytes, void* stream);

/* wq_matmul without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, layouts, bound and errors as wq_matmul.  The K-split
 * partial sums go to a static device array of 16 MiB that the library holds on each
 * GPU it runs on until the process ends; no call allocates or frees anything.  A
 * shape whose split would need more than 16 MiB returns WQ_ERR_WORKSPACE (the current
 * schedules never do).  Every call on one GPU shares that GPU's array: calls that may
 * overlap on one GPU (different streams, or graphs replayed concurrently) race and
 * must be ordered by the caller.  The first call on a device looks up that device's
 * copy of the array (a HIP symbol query, no allocation); a failure returns WQ_ERR_HIP. */
wq_status wq_matmul_noalloc(const wq_desc* d, int64_t m, const uint16_t* x, int64_t ldx, wq_packed w,
                            const uint16_t* bias, void* y, int32_t ydt, int64_t ldy, void* stream);

/* Fused projection over a row-concatenated weight W[n0 + n1 (+ n2), k] in one
 * pass over W (one kernel; a K-split GEMM adds one small reduction kernel):
 * columns [0, n0) go to y[0], [n0, n0+n1) to y[1], [n0+n1, n) to y[2],
 * each with its own leading dimension split_n[i] <= ldy[i] <= 2^31 - 1, so the destinations
 * may be rows of a K/V cache slab; nothing outside each m x split_n[i] window is
 * touched.  The windows must not share a byte (WQ_ERR_INVALID_ARG otherwise; the
 * check is closed-form for equal leading dimensions and O(m) for different ones).  bias is bf16 [n] or NULL (use zeros where a split has none, e.g. the
 * key projection).  nsplit is 2 (merged cross-attention K/V) or 3 (Q/K/V);
 * split_n[i] > 0 and sum(split_n) == d->n.  Passages: "Run quantized Whisper on
 * the fused Metal decode path", "Summary" (fused Q/K/V writing into slab rows
 * with the bias applied on device) and "Test plan" (neighbouring rows
 * untouched); "mbehr90/whisper-large-v3-turbo-nvfp4", "Why the encoder/decoder
 * split matters" (two-way merged cross-attention K/V).  A projection whose
 * parts use different formats cannot be described by one descriptor: callers
 * fall back to separate wq_matmul calls. */
wq_status wq_matmul_qkv(const wq_desc* d, int64_t m, const uint16_t* x, int64_t ldx, wq_packed w,
                        const uint16_t* bias, int32_t nsplit, const int64_t* split_n,
                        void* const* y, const int64_t* ldy, int32_t ydt,
                        void* ws, size_t ws_bytes, void* stream);

/* ---- NVFP4 activations and the W4A4 product ---------------------------------
 * "mbehr90/whisper-large-v3-turbo-nvfp4", section "What is quantized": activations
 * are quantized per 16-value group at run time and multiplied with NVFP4 weights
 * (W4A4; section "Honest summary: on H100 this is not a win" names it the Blackwell
 * mode).  The activation rule is the NVFP4 weight rule applied to X: g_x =
 * absmax(X)/2688 over the whole [m, k] input of the call (fp32), per 16 consecutive
 * k an E4M3 scale E4M3(block absmax / (6 g_x)), nearest-even saturating at 448,
 * codes E2M1(x / (scale * g_x)) nearest, ties to even, sign kept (also of zeros);
 * x^ = e2m1 * scale * g_x.  Inputs must be finite.
 * Packed activations are plain row-major (no tiles):
 *   codes : m*k/2 bytes; byte r*k/2 + j holds elements 2j (low nibble) and 2j+1 of row r
 *   scales: E4M3 byte r*(k/16) + b for block b of row r, zero pad bytes, then the fp32
 *           g_x at byte align16(m*k/16); align16(m*k/16) + 4 bytes in all.
 * Shapes: k % 16 == 0, k <= 2^24, m >= 0, m*k <= 2^34 (else WQ_ERR_SHAPE). */

/* Host-only.  Bytes of the packed activation buffers for an [m, k] input. */
wq_status wq_act_packed_size(int64_t m, int64_t k, size_t* codes_bytes, size_t* scales_bytes);

/* Quantize X[m, k] (bf16, leading dimension ldx >= k, ldx % 8 == 0, ldx <= 2^24;
 * 16-byte aligned) to packed NVFP4 activations.  codes and scales (device, 16-byte
 * aligned, sizes from wq_act_packed_size) are written whole; the codes buffer also
 * holds the per-workgroup maxima between the call's kernels.  Codes, scales and g_x
 * are bit-exact with the rule above.  m == 0 is a no-op. */
wq_status wq_quantize_act(int64_t m, int64_t k, const uint16_t* x, int64_t ldx, void* codes, void* scales,
                          void* stream);

/* Workspace bytes wq_matmul_w4a4 needs for descriptor d (NVFP4 only, else
 * WQ_ERR_UNSUPPORTED) at m rows: 256 + align256(2*m*k) + the matmul's own share. */
wq_status wq_w4a4_workspace_size(const wq_desc* d, int64_t m, size_t* bytes);

/* Y = X^ * W^T + bias with X^ the packed NVFP4 activations [m, k] (xcodes, xscales as
 * written by wq_quantize_act, 16-byte aligned) and W packed NVFP4 (d->format ==
 * WQ_NVFP4, else WQ_ERR_UNSUPPORTED).  bias, y, ydt, ldy as for wq_matmul.  ws is
 * required (WQ_ERR_WORKSPACE when NULL or smaller than wq_w4a4_workspace_size): the
 * call expands the activations there to the exact bf16 values e2m1 * scale and runs
 * the NVFP4 matmul on them with the one epilogue factor g_w * g_x.  Per element
 * |y - y_ref| <= 4e-3 * sum_k |x^_k * w^_k| + 1e-6 against the fp32 reference
 * y_ref = sum_k x^_k w^_k + b (plus the final bf16 rounding for WQ_BF16). */
wq_status wq_matmul_w4a4(const wq_desc* d, int64_t m, const void* xcodes, const void* xscales, wq_packed w,
                         const uint16_t* bias, void* y, int32_t ydt, int64_t ldy, void* ws, size_t ws_bytes,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBWQ_WQ_H */
