"""GPU parity of the NVFP4 W4A4 path ("mbehr90/whisper-large-v3-turbo-nvfp4", section "What
is quantized": activations quantized per 16-value group at run time) against the oracle.

  * wq_quantize_act: codes, scales (pad bytes included) and the global scale bit-exact;
  * wq_matmul_w4a4: |y - y_ref| <= 4e-3 * sum_k |x^_k w^_k| + 1e-6 with y_ref the oracle's
    fp32 product of its own dequantized activations and weights;
  * the encoder GEMM shape X[1500, 1280] with fc1 1280->5120 and fc2 5120->1280 (row std of
    W drawn from LogNormal(0, 0.3)), on sampled rows;
  * edge cases: m = 0, a zero input (g = 0), one huge element, decode-sized m, ragged m,
    strided X.
"""
import numpy as np
import pytest
import torch

from block_quantized_bit_amd import wq
from block_quantized_bit_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits, gen_x, linear_case

from gpu_helpers import dev_bf16, gpu_quantize, require_gpu, say, DEV

pytestmark = pytest.mark.gpu

NVFP4 = 2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def gpu_quantize_act(x_bits: np.ndarray, ldx_pad: int = 0):
    m, k = x_bits.shape
    ldx = k + ldx_pad
    xb = np.full((m, ldx), 0x7FC0, np.uint16)          # padding columns hold NaN
    xb[:, :k] = x_bits
    cb, sb = wq.wq_act_packed_size(m, k)
    codes = torch.full((max(cb, 16),), 0xA5, dtype=torch.uint8, device=DEV)
    scales = torch.full((sb,), 0x5A, dtype=torch.uint8, device=DEV)
    wq.wq_quantize_act(m, k, dev_bf16(xb), ldx, codes, scales)
    torch.cuda.synchronize()
    return codes, scales


def check_act(orc, x_bits, ldx_pad=0, what=""):
    codes, scales = gpu_quantize_act(x_bits, ldx_pad)
    ref = orc.quantize_act_nvfp4(x_bits)
    c = codes.cpu().numpy()[:ref["codes"].size]
    s = scales.cpu().numpy()
    assert np.array_equal(c, ref["codes"]), f"{what}: codes differ at {np.flatnonzero(c != ref['codes'])[:8]}"
    assert np.array_equal(s, ref["scales"]), f"{what}: scales differ at {np.flatnonzero(s != ref['scales'])[:8]}"
    return codes, scales, ref


def w4a4(d, xcodes, xscales, wcodes, wscales, bias_bits, m, ydt=wq.WQ_F32, seed=91):
    ws_bytes = wq.wq_w4a4_workspace_size(d, m)
    ws = torch.from_numpy(np.random.default_rng(seed).integers(0, 256, max(ws_bytes, 16), dtype=np.uint8)).to(DEV)
    B = None if bias_bits is None else dev_bf16(bias_bits)
    if ydt == wq.WQ_F32:
        Y = torch.full((m, d.n), -12345.0, dtype=torch.float32, device=DEV)
    else:
        Y = torch.full((m, d.n), 0x7BAD, dtype=torch.int16, device=DEV)
    wq.wq_matmul_w4a4(d, m, xcodes, xscales, wcodes, wscales, B, Y, ydt, d.n, ws, ws_bytes)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    if ydt == wq.WQ_BF16:
        y = bf16_bits_to_f32(y.view(np.uint16))
    return y


def check(y, y_ref, x_hat, w_hat, bf16_out=False, what=""):
    absdot = np.abs(x_hat.astype(np.float64)) @ np.abs(w_hat.astype(np.float64)).T
    tol = 4e-3 * absdot + 1e-6
    if bf16_out:
        tol = tol + np.abs(y_ref.astype(np.float64)) * 2.0 ** -8
    err = np.abs(y.astype(np.float64) - y_ref.astype(np.float64))
    bad = ~(err <= tol)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {bad.sum()} outside the bound; first {i} y={y[i]} ref={y_ref[i]} tol={tol[i]}")


@pytest.mark.parametrize("m,k,pad", [(1, 128, 0), (3, 48, 8), (16, 1280, 0), (37, 384, 24), (1500, 1280, 0),
                                     (1500, 5120, 0), (6000, 1280, 0)])
def test_quantize_act_bit_exact(orc, m, k, pad):
    say("quantize_act", m, k, pad)
    x = gen_x(np.random.default_rng(5000 + m + k), m, k)
    check_act(orc, x, pad, what=f"{m}x{k}")


def test_quantize_act_special_inputs(orc):
    m, k = 9, 256
    say("quantize_act special")
    z = np.zeros((m, k), np.uint16)
    z[2, 7] = 0x8000                                       # -0 keeps its sign bit
    _, s, ref = check_act(orc, z, what="zero")
    assert ref["g"] == 0
    x = gen_x(np.random.default_rng(5100), m, k)
    x[4, 100] = f32_to_bf16_bits(np.float32([-3.0e4]))[0]  # one element far above the rest
    check_act(orc, x, what="spike")
    x[:, :16] = 0                                          # a zero block in every row
    check_act(orc, x, what="zero blocks")


def test_zero_rows_is_a_noop():
    d = wq.desc("nvfp4", 256, 128)
    buf = torch.full((64,), 7, dtype=torch.uint8, device=DEV)
    x = torch.zeros((1, 128), dtype=torch.int16, device=DEV)
    wq.wq_quantize_act(0, 128, x, 128, buf, buf)
    y = torch.full((1, 256), 3.0, device=DEV)
    wq.wq_matmul_w4a4(d, 0, buf, buf, buf, buf, None, y, wq.WQ_F32, 256, None, 0)
    torch.cuda.synchronize()
    assert torch.all(buf == 7) and torch.all(y == 3.0)


@pytest.mark.parametrize("m", [1, 4, 16, 17, 200])
@pytest.mark.parametrize("ydt", [wq.WQ_F32, wq.WQ_BF16], ids=["f32", "bf16"])
def test_w4a4_matmul_small(orc, m, ydt):
    n, k = 384, 640
    w, b, x = linear_case(5200 + m, n, k, m)
    say("w4a4", m, n, k, ydt)
    d, wc, wsc = gpu_quantize(NVFP4, w)
    wref = orc.quantize(NVFP4, w)
    assert np.array_equal(wc.cpu().numpy(), wref["codes"]) and np.array_equal(wsc.cpu().numpy(), wref["scales"])
    xc, xs, aref = check_act(orc, x)
    y = w4a4(d, xc, xs, wc, wsc, b, m, ydt)
    y_ref = orc.matmul_f32x(aref["x_hat"], wref["w_hat"], b)
    check(y, y_ref, aref["x_hat"], wref["w_hat"], bf16_out=ydt == wq.WQ_BF16, what=f"m={m}")
    assert np.all(np.isfinite(y))


def _sample_rows(m, seed):
    rng = np.random.default_rng(seed)
    rows = set([0, m - 1]) | set(rng.choice(m, size=min(m, 62), replace=False).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("ydt", [wq.WQ_F32, wq.WQ_BF16], ids=["f32", "bf16"])
def test_w4a4_encoder_shape_sampled_rows(orc, ydt):
    """X[1500, 1280] through fc1 (1280 -> 5120), its output's shape through fc2 (5120 -> 1280)."""
    m = 1500
    for i, (n, k) in enumerate([(5120, 1280), (1280, 5120)]):
        w, b, x = linear_case(5300 + i, n, k, m, row_lognormal_sigma=0.3)
        say("w4a4 encoder", m, n, k, ydt)
        d, wc, wsc = gpu_quantize(NVFP4, w)
        wref = orc.quantize(NVFP4, w)
        assert np.array_equal(wc.cpu().numpy(), wref["codes"]) and np.array_equal(wsc.cpu().numpy(), wref["scales"])
        xc, xs, aref = check_act(orc, x, what=f"encoder {n}x{k}")
        y = w4a4(d, xc, xs, wc, wsc, b, m, ydt)
        rows = _sample_rows(m, 5300 + i)
        y_ref = orc.matmul_f32x(aref["x_hat"], wref["w_hat"], b, rows=rows)
        check(y[rows], y_ref, aref["x_hat"][rows], wref["w_hat"], bf16_out=ydt == wq.WQ_BF16,
              what=f"encoder {n}x{k}")
        assert np.all(np.isfinite(y))


def test_w4a4_repeatable_and_zero_activations(orc):
    """Same inputs give bit-identical outputs; a zero input gives exactly the bias."""
    m, n, k = 300, 1280, 5120
    w, b, x = linear_case(5400, n, k, m)
    say("w4a4 repeat", m, n, k)
    d, wc, wsc = gpu_quantize(NVFP4, w)
    xc, xs = gpu_quantize_act(x)
    y1 = w4a4(d, xc, xs, wc, wsc, b, m, seed=1)
    y2 = w4a4(d, xc, xs, wc, wsc, b, m, seed=2)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    zc, zs = gpu_quantize_act(np.zeros((m, k), np.uint16))
    y0 = w4a4(d, zc, zs, wc, wsc, b, m)
    assert np.array_equal(y0, np.tile(bf16_bits_to_f32(b), (m, 1)))
