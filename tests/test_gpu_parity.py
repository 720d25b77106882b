"""GPU parity: libwq (through its C ABI) against the CPU oracle on the same
seeded inputs.  Codes, scales and dequantized weights must match bit for bit;
matmul outputs must satisfy |y - y_ref| <= 4e-3 * sum_k |x_k w^_k| + 1e-6.
"""
import numpy as np
import pytest
import torch

from block_quantized_bit_amd import wq
from block_quantized_bit_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits, gen_x, linear_case

from gpu_helpers import (abs_dot, check_bound, dev_bf16, gpu_dequantize, gpu_matmul, gpu_quantize,
                         require_gpu, say, workspace, DEV, NAMES)

pytestmark = pytest.mark.gpu

NF4, NVFP4, Q4_0, Q8_0, Q4_1, Q5_0, Q4_K, Q6_K = 1, 2, 3, 4, 5, 6, 7, 8
FORMATS = [(NF4, False), (NF4, True), (NVFP4, False), (Q4_0, False), (Q8_0, False), (Q4_1, False), (Q5_0, False),
           (Q4_K, False), (Q6_K, False)]
FMT_IDS = ["nf4", "nf4dq", "nvfp4", "q4_0", "q8_0", "q4_1", "q5_0", "q4_k", "q6_k"]


def kfor(fmt, k):
    """q4_k's and q6_k's 256-value super-blocks need k % 256 == 0: the next such k for them."""
    return (k + 255) // 256 * 256 if fmt in (Q4_K, Q6_K) else k


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


_cache = {}


def quantized(orc, fmt, dq, seed, n, k, **kw):
    """Seeded W quantized by both sides; asserts bit-exact codes/scales/dequant."""
    key = (fmt, dq, seed, n, k, tuple(sorted(kw.items())))
    if key in _cache:
        return _cache[key]
    w, b, _ = linear_case(seed, n, k, 1, **kw)
    say("quantize", NAMES[fmt], "dq" if dq else "", seed, n, k)
    ref = orc.quantize(fmt, w, dq)
    d, codes, scales = gpu_quantize(fmt, w, dq)
    assert np.array_equal(codes.cpu().numpy(), ref["codes"]), "packed codes differ"
    assert np.array_equal(scales.cpu().numpy(), ref["scales"]), "packed scales differ"
    w_hat = gpu_dequantize(d, codes, scales)
    assert np.array_equal(w_hat.view(np.uint32), ref["w_hat"].view(np.uint32)), "dequantized weights differ"
    out = (d, codes, scales, ref, b)
    _cache[key] = out
    return out


# --------------------------------------------------------------- quantize / dequantize

@pytest.mark.parametrize("fmt,dq", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("n,k", [(16, 128), (48, 384), (272, 640)])
def test_quantize_dequantize_bit_exact(orc, fmt, dq, n, k):
    k = kfor(fmt, k)
    quantized(orc, fmt, dq, 11, n, k, outlier_frac=0.01)


def test_whisper_tiny_fc1_config(orc):
    """whisper-tiny fc1: X[4,384], W[1536,384] ~N(0,0.02), bias ~N(0,0.01), NF4 block 64, no double-quant."""
    w, b, x = linear_case(1, 1536, 384, 4)
    ref = orc.quantize(NF4, w, False)
    d, codes, scales = gpu_quantize(NF4, w, False)
    assert np.array_equal(codes.cpu().numpy(), ref["codes"])
    assert np.array_equal(scales.cpu().numpy(), ref["scales"])
    assert np.array_equal(gpu_dequantize(d, codes, scales).view(np.uint32), ref["w_hat"].view(np.uint32))
    y_ref = orc.matmul(x, ref["w_hat"], b)
    ad = abs_dot(x, ref["w_hat"])
    for ydt in (wq.WQ_F32, wq.WQ_BF16):
        y = gpu_matmul(d, codes, scales, x, b, ydt=ydt)
        check_bound(y, y_ref, ad, bf16_out=ydt == wq.WQ_BF16, what="whisper-tiny fc1")


@pytest.mark.parametrize("fmt,dq", FORMATS, ids=FMT_IDS)
def test_quantize_special_values(orc, fmt, dq):
    """Zero blocks, signed zeros, exact ties, huge and tiny magnitudes (fp16 scale
    saturation and underflow, E4M3 saturation)."""
    rng = np.random.default_rng(5)
    n, k = 64, 256
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[0] = 0.0
    w[1, :] = -0.0
    w[2, :64] = np.float32(0.5)
    w[2, 64:128] = -np.float32(0.5)
    w[3] = rng.standard_normal(k).astype(np.float32) * np.float32(1e5)      # fp16 scale saturates
    w[4] = rng.standard_normal(k).astype(np.float32) * np.float32(1e-9)     # tiny
    w[5, ::7] = np.float32(3e4)
    w[6] = np.where(rng.integers(0, 2, k) == 1, 1.0, -1.0).astype(np.float32)
    w[7, :32] = np.linspace(-1, 1, 32, dtype=np.float32)
    w[7, 32:64] = np.float32(0.25) * np.arange(32, dtype=np.float32)
    say("special", NAMES[fmt], dq)
    ref = orc.quantize(fmt, w, dq)
    d, codes, scales = gpu_quantize(fmt, w, dq)
    assert np.array_equal(codes.cpu().numpy(), ref["codes"])
    assert np.array_equal(scales.cpu().numpy(), ref["scales"])
    assert np.array_equal(gpu_dequantize(d, codes, scales).view(np.uint32), ref["w_hat"].view(np.uint32))


@pytest.mark.parametrize("wide", [False, True], ids=["integer-sum", "ascending-chain"])
def test_double_quant_mean_both_paths(orc, wide):
    """The double-quant mean (ascending binary64 sum of the absmax values) on its two
    GPU paths, bit-exact against the oracle: absmax values of one magnitude make every
    ascending addition exact, so the integer sum of the workgroup is taken; one row
    scaled by 1e-12 spreads their lowest set bits over more than 2^40, which sends the
    sum down the sequential chain (20 800 blocks: five 4096-value chunks and a ragged one)."""
    rng = np.random.default_rng(17)
    n, k = 1040, 1280
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    if wide:
        w[7] *= np.float32(1e-12)
    say("dq mean", "wide" if wide else "narrow")
    ref = orc.quantize(NF4, w, True)
    d, codes, scales = gpu_quantize(NF4, w, True)
    assert np.array_equal(scales.cpu().numpy(), ref["scales"]), "scales (mean, group scales, int8 absmax) differ"
    assert np.array_equal(codes.cpu().numpy(), ref["codes"])


@pytest.mark.parametrize("fmt,dq,shapes", [
    (NF4, True, [(3840, 1280), (1280, 1280), (5120, 1280), (1280, 5120)]),
    (NVFP4, False, [(5120, 1280), (1280, 5120)]),
    (Q8_0, False, [(1280, 1280), (5120, 1280), (1280, 5120)]),
    (Q4_0, False, [(1280, 1280), (5120, 1280), (1280, 5120)]),
    (Q4_1, False, [(1280, 1280), (5120, 1280), (1280, 5120)]),
    (Q5_0, False, [(1280, 1280), (5120, 1280), (1280, 5120)]),
    (Q4_K, False, [(1280, 1280), (5120, 1280), (1280, 5120)]),
    (Q6_K, False, [(1280, 1280), (5120, 1280), (1280, 5120)]),
], ids=["decoder-nf4dq", "encoder-nvfp4", "encoder-q8_0", "encoder-q4_0", "encoder-q4_1", "encoder-q5_0",
        "encoder-q4_k", "encoder-q6_k"])
def test_quantize_full_whisper_shapes(orc, fmt, dq, shapes):
    for i, (n, k) in enumerate(shapes):
        kw = dict(outlier_frac=0.001) if fmt == NF4 else (dict(row_lognormal_sigma=0.3) if fmt == NVFP4 else {})
        quantized(orc, fmt, dq, 2000 + i, n, k, **kw)


# --------------------------------------------------------------- matmul

@pytest.mark.parametrize("fmt,dq", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 16, 17, 64, 129, 300])
def test_matmul_ragged(orc, fmt, dq, m):
    n, k = 272, kfor(fmt, 640)
    d, codes, scales, ref, b = quantized(orc, fmt, dq, 11, n, k, outlier_frac=0.01)
    rng = np.random.default_rng(100 + m)
    x = f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    y_ref = orc.matmul(x, ref["w_hat"], b)
    ad = abs_dot(x, ref["w_hat"])
    say("matmul", NAMES[fmt], dq, m, n, k)
    for use_ws in (True, False):
        y = gpu_matmul(d, codes, scales, x, b, use_ws=use_ws, ldx_pad=8, ldy_pad=16)
        check_bound(y, y_ref, ad, what=f"{NAMES[fmt]} m={m} ws={use_ws}")
    y = gpu_matmul(d, codes, scales, x, None, ydt=wq.WQ_BF16)
    check_bound(y, orc.matmul(x, ref["w_hat"], None), ad, bf16_out=True, what="bf16 out, no bias")
    # an odd output stride rules out the 4-column vector stores: the per-element store path
    y = gpu_matmul(d, codes, scales, x, b, ydt=wq.WQ_BF16, ldy_pad=3)
    check_bound(y, y_ref, ad, bf16_out=True, what="bf16 out, odd ldy")


@pytest.mark.parametrize("fmt,dq", [(NVFP4, False), (Q8_0, False), (Q4_0, False), (NF4, True), (Q6_K, False)],
                         ids=["nvfp4", "q8_0", "q4_0", "nf4dq", "q6_k"])
@pytest.mark.parametrize("k", [64, 128, 192, 256, 320, 384, 512, 640, 768, 896, 1664])
def test_gemm_k_steps_and_pipeline_tails(orc, fmt, dq, k):
    """GEMM (M = 100 and 300, 128 x 128 tiles) over every count of 128-wide K steps up to 7
    and 13: the pipeline's prologue, its three-step loop and each of its tails; q8_0 also at
    k = 64 mod 128 (its tiles are 64 wide)."""
    if fmt != Q8_0 and k % 128:
        pytest.skip("k must be a multiple of 128 for this format")
    if fmt == Q6_K and k % 256:
        pytest.skip("q6_k needs k % 256 == 0")
    n = 272
    d, codes, scales, ref, b = quantized(orc, fmt, dq, 4300, n, k)
    for m in (100, 300):
        x = linear_case(4300 + m, n, k, m)[2]
        say("gemm k steps", NAMES[fmt], m, n, k)
        y = gpu_matmul(d, codes, scales, x, b)
        check_bound(y, orc.matmul(x, ref["w_hat"], b), abs_dot(x, ref["w_hat"]), what=f"{NAMES[fmt]} m={m} k={k}")


@pytest.mark.parametrize("fmt,dq", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("ydt,ldy_pad", [(wq.WQ_F32, 0), (wq.WQ_BF16, 0), (wq.WQ_BF16, 1), (wq.WQ_F32, 3)],
                         ids=["f32", "bf16", "bf16-odd-ldy", "f32-odd-ldy"])
@pytest.mark.parametrize("k", [5120, 6144, 12288], ids=["2pieces", "4pieces", "8pieces"])
def test_gemm_split_k_full_tiles(orc, fmt, dq, ydt, ldy_pad, k):
    """Few output tiles (N = 512) with several full 128-row tiles (M = 300) and long K:
    the GEMM splits K (in 2 pieces at K = 5120, 4 at K = 6144, 8 at K = 12288), deposits full-tile
    partials with vector stores and reduces them in a second kernel (vector or
    per-element stores, by output alignment).  The workspace starts as random bytes."""
    n, m = 512, 300
    d, codes, scales, ref, b = quantized(orc, fmt, dq, 4200, n, k)
    x = linear_case(4200, n, k, m)[2]
    assert wq.wq_workspace_size(d, m) > 0
    say("split-K gemm", NAMES[fmt], m, n, k, ydt, ldy_pad)
    y = gpu_matmul(d, codes, scales, x, b, ydt=ydt, ldy_pad=ldy_pad)
    rows = _sample_rows(m, 5)
    check_bound(y[rows], orc.matmul(x, ref["w_hat"], b, rows=rows), abs_dot(x, ref["w_hat"], rows=rows),
                bf16_out=ydt == wq.WQ_BF16, what=f"split-K {NAMES[fmt]} ydt={ydt} pad={ldy_pad}")


@pytest.mark.parametrize("ydt", [wq.WQ_F32, wq.WQ_BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("m", [1, 4, 16])
def test_decoder_gemv_set_full(orc, m, ydt):
    """Decoder GEMV set, NF4 + double-quant: QKV 1280->3840, out 1280->1280,
    fc1 1280->5120, fc2 5120->1280; W ~N(0,0.02) with 0.1% outliers x8; X ~N(0,1).
    bf16 output is the configuration the decode step is timed in."""
    for i, (n, k) in enumerate([(3840, 1280), (1280, 1280), (5120, 1280), (1280, 5120)]):
        d, codes, scales, ref, b = quantized(orc, NF4, True, 2000 + i, n, k, outlier_frac=0.001)
        x = linear_case(2000 + i, n, k, 16, outlier_frac=0.001)[2][:m]
        say("decoder gemv", n, k, m, "bf16" if ydt == wq.WQ_BF16 else "f32")
        y = gpu_matmul(d, codes, scales, x, b, ydt=ydt)
        check_bound(y, orc.matmul(x, ref["w_hat"], b), abs_dot(x, ref["w_hat"]), bf16_out=ydt == wq.WQ_BF16,
                    what=f"dec {n}x{k} m={m}")


@pytest.mark.parametrize("fmt,dq", [(NVFP4, False), (Q4_1, False), (Q5_0, False), (Q4_K, False), (Q6_K, False),
                                    (NF4, True), (Q4_0, False), (Q8_0, False)],
                         ids=["nvfp4", "q4_1", "q5_0", "q4_k", "q6_k", "nf4dq", "q4_0", "q8_0"])
@pytest.mark.parametrize("m", [1, 5, 11, 12, 16])
def test_decode_fc1_shape_many_tokens(orc, fmt, dq, m):
    """fc1 geometry (5120 x 1280, 320 bands) at one and several tokens: at several tokens the
    formats without a code table copy X to LDS with two workgroups per CU (one round for all
    bands), the table formats read X from L2 below 12 tokens and copy it, two bands pipelined
    per workgroup, from 12 on; q8_0 takes 4-tile rounds.  Every output is checked."""
    n, k = 5120, kfor(fmt, 1280)
    d, codes, scales, ref, b = quantized(orc, fmt, dq, 2002, n, k, outlier_frac=0.001)
    x = linear_case(2002, n, k, 16, outlier_frac=0.001)[2][:m]
    say("decode fc1 shape", NAMES[fmt], m)
    y = gpu_matmul(d, codes, scales, x, b, ydt=wq.WQ_BF16)
    check_bound(y, orc.matmul(x, ref["w_hat"], b), abs_dot(x, ref["w_hat"]), bf16_out=True,
                what=f"fc1 shape {NAMES[fmt]} m={m}")


# N = 131072 is 8192 16-row bands: enough that each of the 2048 resident waves
# owns >= 4 bands, which selects the many-band streaming GEMV (same kernel and
# grid as the 655360-row streaming measurement).  Every output is checked.
STREAM_N = 131072


@pytest.mark.parametrize("fmt,dq,k,m,use_bias,ydt", [
    (NF4, True, 1280, 1, True, wq.WQ_F32),       # fc1 geometry, K = 10 tiles
    (NVFP4, False, 384, 3, True, wq.WQ_BF16),    # K = 3 tiles (the 4-tile variant: slot 3 reads zeros)
    (Q8_0, False, 256, 2, False, wq.WQ_F32),     # K = 4 tiles of 64
    (Q4_0, False, 640, 5, True, wq.WQ_F32),      # K = 5 tiles (the 10-tile variant)
    (NF4, False, 512, 15, True, wq.WQ_F32),      # m * k = 7680, near the most X the kernel stages
    (NF4, False, 384, 16, True, wq.WQ_BF16),     # all 16 rows, K = 3 tiles
    # the chunked streaming kernel: chunks of 5 tiles for the wide-record formats, of 10 for K
    # beyond 10 tiles; ragged last chunks, super-blocks split across chunks, four-row calls
    (Q4_1, False, 1280, 1, True, wq.WQ_BF16),    # 1 chunk of 10
    (Q5_0, False, 640, 3, True, wq.WQ_F32),      # 1 chunk
    (Q4_K, False, 768, 2, True, wq.WQ_BF16),     # 5 + 1 tiles (three super-blocks per row)
    (Q6_K, False, 512, 4, False, wq.WQ_F32),     # 1 chunk of 4
    (Q6_K, False, 1280, 1, True, wq.WQ_BF16),    # super-block 2 spans chunks 0 and 1
    (Q5_0, False, 1280, 6, True, wq.WQ_BF16),    # m * k = 7680
    (Q4_K, False, 1536, 1, False, wq.WQ_F32),    # 5 + 1 + ... tiles, K = 12 tiles
    (Q8_0, False, 1280, 1, True, wq.WQ_BF16),    # 20 tiles of 64: 2 chunks of 10
    (NF4, False, 1536, 1, True, wq.WQ_F32),      # 10 + 2 tiles, code table
    (NVFP4, False, 2048, 3, True, wq.WQ_BF16),   # 10 + 6 tiles, four-row accumulators
    (Q4_0, False, 1536, 4, True, wq.WQ_F32),     # four-row q4_0: chunks of 5 (5 + 5 + 2 tiles)
    (Q4_1, False, 1280, 3, True, wq.WQ_F32),     # four-row accumulators, 1 chunk of 10
    # one-token NVFP4 (block scales applied after the MFMA) in each streaming kernel
    (NVFP4, False, 384, 1, False, wq.WQ_F32),    # the 4-tile variant
    (NVFP4, False, 1280, 1, True, wq.WQ_BF16),   # the 10-tile variant
    (NVFP4, False, 2048, 1, True, wq.WQ_F32),    # chunked, 10 + 6 tiles
], ids=["nf4dq-k1280-m1", "nvfp4-k384-m3", "q8_0-k256-m2", "q4_0-k640-m5", "nf4-k512-m15", "nf4-k384-m16",
        "q4_1-k1280-m1", "q5_0-k640-m3", "q4_k-k768-m2", "q6_k-k512-m4", "q6_k-k1280-m1", "q5_0-k1280-m6",
        "q4_k-k1536-m1", "q8_0-k1280-m1", "nf4-k1536-m1", "nvfp4-k2048-m3", "q4_0-k1536-m4", "q4_1-k1280-m3",
        "nvfp4-k384-m1", "nvfp4-k1280-m1", "nvfp4-k2048-m1"])
def test_streaming_gemv_many_bands(orc, fmt, dq, k, m, use_bias, ydt):
    d, codes, scales, ref, b = quantized(orc, fmt, dq, 6000 + k, STREAM_N, k, outlier_frac=0.001)
    x = gen_x(np.random.default_rng(6100 + k), m, k)
    b = b if use_bias else None
    say("streaming gemv", NAMES[fmt], "dq" if dq else "", STREAM_N, k, m)
    y = gpu_matmul(d, codes, scales, x, b, ydt=ydt, ldy_pad=16)
    check_bound(y, orc.matmul(x, ref["w_hat"], b), abs_dot(x, ref["w_hat"]), bf16_out=ydt == wq.WQ_BF16,
                what=f"stream {NAMES[fmt]} k={k} m={m}")


@pytest.mark.parametrize("n,k", [(272, 640), (1280, 5120), (256, 16384), (10240, 1280), (9600, 3072)],
                         ids=["lds-x-1tile", "lds-x-5tiles", "lds-x-2rounds-of-8", "band-pipelined", "x-from-l2-4tiles"])
def test_one_token_nvfp4_general_kernel(orc, n, k):
    """One NVFP4 token puts each 16-value block's x in its own A row and applies the E4M3 block
    scales to the per-block MFMA sums.  Every variant of the general GEMV kernel that one token
    reaches: X copied to LDS with 1, 5 or 2 x 8 tiles per wave, band-pipelined workgroups (more
    bands than resident workgroups), and X read from L2 (more than 512 bands, 4 tiles per wave).
    Weights with log-normal row scales spread the block scales over E4M3's range."""
    d, codes, scales, ref, b = quantized(orc, NVFP4, False, 6500 + n + k, n, k, row_lognormal_sigma=0.5)
    x = gen_x(np.random.default_rng(6600 + k), 1, k)
    say("one-token nvfp4", n, k)
    y = gpu_matmul(d, codes, scales, x, b, ydt=wq.WQ_F32)
    check_bound(y, orc.matmul(x, ref["w_hat"], b), abs_dot(x, ref["w_hat"]), what=f"nvfp4 m=1 n={n} k={k}")


def test_streaming_gemv_qkv_split(orc):
    """The streaming kernel's per-column split selection: three strided windows,
    each equal to the single-output call's columns, nothing else written."""
    k, m = 1280, 1
    d, codes, scales, ref, b = quantized(orc, NF4, True, 6000 + k, STREAM_N, k, outlier_frac=0.001)
    x = gen_x(np.random.default_rng(6100 + k), m, k)
    splits = [65536, 32768, 32768]
    X, B = dev_bf16(x), dev_bf16(b)
    canary = 0x7BAD
    slabs, ys, ldys = [], [], []
    for i, s in enumerate(splits):
        ld = s + 64
        slab = torch.full((m + 2, ld), canary, dtype=torch.int16, device=DEV)
        slabs.append(slab)
        ys.append(slab[1:].data_ptr() + 2 * 16)
        ldys.append(ld)
    say("streaming qkv", splits)
    wq.wq_matmul_qkv(d, m, X, k, codes, scales, B, splits, ys, ldys, wq.WQ_BF16, None, 0)
    Y = torch.empty((m, STREAM_N), dtype=torch.int16, device=DEV)
    wq.wq_matmul(d, m, X, k, codes, scales, B, Y, wq.WQ_BF16, STREAM_N, None, 0)
    torch.cuda.synchronize()
    yfull = Y.cpu().numpy()
    c0 = 0
    for i, s in enumerate(splits):
        sl = slabs[i].cpu().numpy()
        assert np.array_equal(sl[1:1 + m, 16:16 + s], yfull[:, c0:c0 + s]), f"split {i} differs"
        mask = np.ones_like(sl, bool)
        mask[1:1 + m, 16:16 + s] = False
        assert np.all(sl[mask] == canary), f"split {i}: writes outside its window"
        c0 += s


def _sample_rows(m, seed):
    rng = np.random.default_rng(seed)
    rows = set([0, m - 1]) | set(rng.choice(m, size=min(m, 62), replace=False).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("fmt,m,shapes,kw", [
    (NVFP4, 1500, [(5120, 1280), (1280, 5120)], dict(row_lognormal_sigma=0.3)),
    (Q8_0, 6000, [(1280, 1280), (5120, 1280), (1280, 5120)], {}),
    (Q4_0, 6000, [(1280, 1280), (5120, 1280), (1280, 5120)], {}),
    # the linear sweep's encoder layers: q8_0 at 1500 frames (the 1280-wide outputs take the K split)
    (Q8_0, 1500, [(1280, 1280), (5120, 1280), (1280, 5120)], {}),
    (Q4_1, 1500, [(1280, 1280), (5120, 1280), (1280, 5120)], {}),
    (Q5_0, 1500, [(1280, 1280), (5120, 1280), (1280, 5120)], {}),
    (Q4_K, 1500, [(1280, 1280), (5120, 1280), (1280, 5120)], {}),
    (Q6_K, 1500, [(1280, 1280), (5120, 1280), (1280, 5120)], {}),
], ids=["encoder-nvfp4-1500", "layer-q8_0-6000", "layer-q4_0-6000", "sweep-q8_0-1500", "encoder-q4_1-1500",
        "encoder-q5_0-1500", "encoder-q4_k-1500", "encoder-q6_k-1500"])
@pytest.mark.parametrize("ydt", [wq.WQ_F32, wq.WQ_BF16], ids=["f32", "bf16"])
def test_encoder_gemm_sampled_rows(orc, fmt, m, shapes, kw, ydt):
    """Full-size encoder GEMMs (bf16 output is the timed configuration); 64 sampled
    rows, first and last included, are checked against the oracle."""
    for i, (n, k) in enumerate(shapes):
        d, codes, scales, ref, b = quantized(orc, fmt, False, 3000 + i, n, k, **kw)
        x = linear_case(3000 + i, n, k, m, **kw)[2]
        say("encoder gemm", NAMES[fmt], m, n, k, "bf16" if ydt == wq.WQ_BF16 else "f32")
        y = gpu_matmul(d, codes, scales, x, b, ydt=ydt)
        rows = _sample_rows(m, i)
        y_ref = orc.matmul(x, ref["w_hat"], b, rows=rows)
        check_bound(y[rows], y_ref, abs_dot(x, ref["w_hat"], rows=rows), bf16_out=ydt == wq.WQ_BF16,
                    what=f"{NAMES[fmt]} {n}x{k} m={m}")
        assert np.all(np.isfinite(y))


@pytest.mark.parametrize("fmt,dq", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("n,ydt", [(3840, wq.WQ_BF16), (3600, wq.WQ_F32)], ids=["n3840-bf16", "n3600-f32"])
def test_gemm_qkv_width_and_ragged_columns(orc, fmt, dq, n, ydt):
    """M = 1500 with N = 3840 (the fused Q/K/V projection) or 3600 (a last column tile of
    which only 1 of the 4 waves' band groups exists).  64 sampled rows."""
    m, k = 1500, 512
    d, codes, scales, ref, b = quantized(orc, fmt, dq, 4400, n, k)
    x = linear_case(4400, n, k, m)[2]
    say("gemm qkv width", NAMES[fmt], m, n, k)
    y = gpu_matmul(d, codes, scales, x, b, ydt=ydt)
    rows = _sample_rows(m, 3)
    check_bound(y[rows], orc.matmul(x, ref["w_hat"], b, rows=rows), abs_dot(x, ref["w_hat"], rows=rows),
                bf16_out=ydt == wq.WQ_BF16, what=f"{NAMES[fmt]} qkv width n={n}")
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("fmt,dq", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("m", [1, 16, 100])
def test_special_cases(orc, fmt, dq, m):
    n, k = 64, 256
    # W = 0: Y is exactly the bias
    w = np.zeros((n, k), np.float32)
    rng = np.random.default_rng(9)
    b = f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32) * 0.01)
    x = f32_to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    d, codes, scales = gpu_quantize(fmt, w, dq)
    y = gpu_matmul(d, codes, scales, x, b)
    assert np.array_equal(y, np.tile(bf16_bits_to_f32(b), (m, 1)))
    # one-hot X picks rows of W^ (+ bias), within the bound
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    ref = orc.quantize(fmt, w, dq)
    d, codes, scales = gpu_quantize(fmt, w, dq)
    x = np.zeros((m, k), np.uint16)
    for i in range(m):
        x[i, (37 * i) % k] = f32_to_bf16_bits(np.float32([1.0]))[0]
    y = gpu_matmul(d, codes, scales, x, b)
    check_bound(y, orc.matmul(x, ref["w_hat"], b), abs_dot(x, ref["w_hat"]), what="one-hot")


@pytest.mark.parametrize("fmt,dq", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("m", [1, 16, 300])
def test_repeatable_and_workspace_reusable(orc, fmt, dq, m):
    """Same inputs -> bit-identical outputs, call after call, reusing one workspace."""
    n, k = 1280, 5120
    d, codes, scales, ref, b = quantized(orc, fmt, dq, 4100, n, k)
    x = linear_case(4100, n, k, m)[2]
    X = dev_bf16(x)
    B = dev_bf16(b)
    ws, wsb = workspace(d, m)
    outs = []
    for _ in range(3):
        Y = torch.empty((m, n), dtype=torch.float32, device=DEV)
        wq.wq_matmul(d, m, X, k, codes, scales, B, Y, wq.WQ_F32, n, ws, wsb)
        outs.append(Y)
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    rows = _sample_rows(m, 1)
    check_bound(outs[0].cpu().numpy()[rows], orc.matmul(x, ref["w_hat"], b, rows=rows),
                abs_dot(x, ref["w_hat"], rows=rows), what="repeat")


@pytest.mark.parametrize("fmt,dq", [(NVFP4, False), (NF4, True), (Q8_0, False)], ids=["nvfp4", "nf4dq", "q8_0"])
@pytest.mark.parametrize("m", [1500, 200], ids=["2pieces", "4pieces"])
def test_split_k_graph_replays(orc, fmt, dq, m):
    """A K-split GEMM (fc2 shape, 1280 x 5120) captured in a HIP graph: every replay,
    with eager calls on the same workspace in between, gives the eager result bit for
    bit, and that result meets the bound."""
    n, k = 1280, 5120
    d, codes, scales, ref, b = quantized(orc, fmt, dq, 4300, n, k)
    x = linear_case(4300, n, k, m)[2]
    X = dev_bf16(x)
    B = dev_bf16(b)
    ws, wsb = workspace(d, m, seed=5)
    assert ws is not None
    say("graph replays", NAMES[fmt], m, n, k)
    st = torch.cuda.Stream()
    Y0 = torch.empty((m, n), dtype=torch.float32, device=DEV)
    Y = torch.empty((m, n), dtype=torch.float32, device=DEV)
    with torch.cuda.stream(st):
        wq.wq_matmul(d, m, X, k, codes, scales, B, Y0, wq.WQ_F32, n, ws, wsb, stream=st)
    st.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            wq.wq_matmul(d, m, X, k, codes, scales, B, Y, wq.WQ_F32, n, ws, wsb, stream=st)
    torch.cuda.synchronize()
    for rep in range(4):
        Y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, Y0), f"replay {rep} differs from the eager result"
        if rep % 2 == 1:
            # an eager call with its own token on the same workspace between replays
            Y2 = torch.empty((m, n), dtype=torch.float32, device=DEV)
            wq.wq_matmul(d, m, X, k, codes, scales, B, Y2, wq.WQ_F32, n, ws, wsb)
            torch.cuda.synchronize()
            assert torch.equal(Y2, Y0), "eager call between replays differs"
    rows = _sample_rows(m, 6)
    check_bound(Y0.cpu().numpy()[rows], orc.matmul(x, ref["w_hat"], b, rows=rows),
                abs_dot(x, ref["w_hat"], rows=rows), what=f"graph split-K {NAMES[fmt]} m={m}")


# --------------------------------------------------------------- fused QKV / merged K/V

@pytest.mark.parametrize("fmt,dq", [(NF4, True), (Q8_0, False), (NVFP4, False)], ids=["nf4dq", "q8_0", "nvfp4"])
@pytest.mark.parametrize("m,splits", [(1, [1280, 1280, 1280]), (16, [1280, 1280, 1280]),
                                      (1500, [1280, 1280]), (40, [512, 256, 512])])
def test_matmul_qkv_into_slab_rows(orc, fmt, dq, m, splits):
    """One launch writes each split into its own strided destination; bias
    applied on device; canary-filled rows and columns around every window
    stay untouched; equals the single-output call column for column."""
    n = sum(splits)
    k = 1280
    d, codes, scales, ref, b = quantized(orc, fmt, dq, 5000 + len(splits), n, k)
    b = b.copy()
    if len(splits) == 3:
        b[splits[0]:splits[0] + splits[1]] = 0          # key projection has no bias
    x = linear_case(5000 + len(splits), n, k, m)[2]
    X = dev_bf16(x)
    B = dev_bf16(b)
    canary = -777.0
    slabs, ys, ldys = [], [], []
    for i, s in enumerate(splits):
        ld = s + 48 + 16 * i
        slab = torch.full((m + 3, ld), canary, dtype=torch.float32, device=DEV)
        slabs.append(slab)
        ys.append(slab[1:].data_ptr() + 4 * 8)           # window starts at row 1, column 8
        ldys.append(ld)
    ws, wsb = workspace(d, m)
    say("qkv", NAMES[fmt], m, splits)
    wq.wq_matmul_qkv(d, m, X, k, codes, scales, B, splits, ys, ldys, wq.WQ_F32, ws, wsb)
    Y = torch.empty((m, n), dtype=torch.float32, device=DEV)
    ws2, wsb2 = workspace(d, m)
    wq.wq_matmul(d, m, X, k, codes, scales, B, Y, wq.WQ_F32, n, ws2, wsb2)
    torch.cuda.synchronize()
    yfull = Y.cpu().numpy()
    c0 = 0
    for i, s in enumerate(splits):
        sl = slabs[i].cpu().numpy()
        win = sl[1:1 + m, 8:8 + s]
        assert np.array_equal(win, yfull[:, c0:c0 + s]), f"split {i} differs from the single-output call"
        mask = np.ones_like(sl, bool)
        mask[1:1 + m, 8:8 + s] = False
        assert np.all(sl[mask] == canary), f"split {i}: writes outside its window"
        c0 += s
    rows = _sample_rows(m, 3)
    check_bound(yfull[rows], orc.matmul(x, ref["w_hat"], b, rows=rows), abs_dot(x, ref["w_hat"], rows=rows),
                what="qkv")


@pytest.mark.parametrize("m", [1500, 6000])
def test_encoder_qkv_q8_0_as_timed(orc, m):
    """The encoder's fused Q/K/V in q8_0 exactly as the encoder sweep and the batch-4 layer
    run it: one wq_matmul_qkv over the concatenated 3840 x 1280 weights, bf16 output, the
    three 1280-column windows side by side in one [m, 3840] buffer (row stride 3840, key
    bias zero).  Equal to the single-output call bit for bit, within the bound of the
    oracle on sampled rows."""
    n, k = 3 * 1280, 1280
    d, codes, scales, ref, b = quantized(orc, Q8_0, False, 5100, n, k)
    b = b.copy()
    b[1280:2560] = 0
    x = linear_case(5100, n, k, m)[2]
    X, B = dev_bf16(x), dev_bf16(b)
    say("encoder qkv q8_0", m)
    Yq = torch.full((m, n), 0x7BAD, dtype=torch.int16, device=DEV)
    p0 = Yq.data_ptr()
    ws, wsb = workspace(d, m)
    wq.wq_matmul_qkv(d, m, X, k, codes, scales, B, [1280] * 3, [p0, p0 + 2 * 1280, p0 + 4 * 1280], [n] * 3,
                     wq.WQ_BF16, ws, wsb)
    Y = torch.full((m, n), 0x7BAD, dtype=torch.int16, device=DEV)
    ws2, wsb2 = workspace(d, m)
    wq.wq_matmul(d, m, X, k, codes, scales, B, Y, wq.WQ_BF16, n, ws2, wsb2)
    torch.cuda.synchronize()
    yq = Yq.cpu().numpy()
    assert np.array_equal(yq, Y.cpu().numpy())
    rows = _sample_rows(m, 8)
    y = bf16_bits_to_f32(yq.view(np.uint16))
    check_bound(y[rows], orc.matmul(x, ref["w_hat"], b, rows=rows), abs_dot(x, ref["w_hat"], rows=rows),
                bf16_out=True, what=f"encoder qkv q8_0 m={m}")


def test_zero_rows_and_errors_touch_nothing(orc):
    d, codes, scales, ref, b = quantized(orc, NF4, False, 11, 272, 640, outlier_frac=0.01)
    Y = torch.full((4, 272), 3.0, dtype=torch.float32, device=DEV)
    X = torch.zeros((4, 640), dtype=torch.int16, device=DEV)
    assert wq.wq_matmul(d, 0, X, 640, codes, scales, None, Y, wq.WQ_F32, 272) == 0
    # a too-small workspace is rejected and nothing runs (m = 20 rows, few tiles: the GEMM wants a K split)
    dd, c2, s2, _, _ = quantized(orc, NF4, False, 4100, 1280, 5120)
    need = wq.wq_workspace_size(dd, 20)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    X2 = torch.zeros((20, 5120), dtype=torch.int16, device=DEV)
    Y2 = torch.full((20, 1280), 3.0, dtype=torch.float32, device=DEV)
    st = wq.wq_matmul(dd, 20, X2, 5120, c2, s2, None, Y2, wq.WQ_F32, 1280, ws, need - 16, check=False)
    assert st == 6
    torch.cuda.synchronize()
    assert bool((Y == 3.0).all()) and bool((Y2 == 3.0).all())
