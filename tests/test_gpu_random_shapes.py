"""Seeded random-shape sweep of wq_matmul and wq_matmul_qkv against the oracle: every
format, the decode GEMV (m <= 16) and the MFMA GEMM (m >= 17), bf16 and fp32 outputs, odd
row strides of X and Y, with and without bias, and two- and three-way output splits with
split ends off the 4-column grid.  Shapes are drawn from one generator with a fixed seed,
so the sweep is the same on every run; each case prints its parameters before it runs.
Packed codes, scales and dequantized weights are checked bit for bit, outputs within
|y - y_ref| <= 4e-3 sum_k |x_k w^_k| + 1e-6 (plus the bf16 output rounding)."""
import numpy as np
import pytest
import torch

from block_quantized_bit_amd import wq
from block_quantized_bit_amd.inputs import bf16_bits_to_f32, linear_case

from gpu_helpers import DEV, NAMES, abs_dot, check_bound, dev_bf16, gpu_dequantize, gpu_quantize, require_gpu, say, workspace

pytestmark = pytest.mark.gpu

FORMATS = [(1, False), (1, True), (2, False), (3, False), (4, False), (5, False), (6, False), (7, False), (8, False)]
NCASES = 36


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _case(i):
    rng = np.random.default_rng(9000 + i)
    fmt, dq = FORMATS[i % len(FORMATS)]
    kq = 256 if fmt in (7, 8) else 64 if fmt == 4 else 128
    k = kq * int(rng.integers(1, max(2, 2304 // kq) + 1))
    n = 16 * int(rng.integers(1, 97))
    m = int(rng.integers(1, 17)) if i % 2 == 0 else int(rng.integers(17, 400))
    ydt = wq.WQ_BF16 if rng.random() < 0.5 else wq.WQ_F32
    ldx_pad = 8 * int(rng.integers(0, 3))
    ldy_pad = int(rng.integers(0, 6))
    use_bias = rng.random() < 0.7
    nsplit = 1 if n < 48 or rng.random() < 0.6 else int(rng.integers(2, 4))
    return fmt, dq, m, n, k, ydt, ldx_pad, ldy_pad, use_bias, nsplit, rng


@pytest.mark.parametrize("i", range(NCASES))
def test_random_shape(orc, i):
    fmt, dq, m, n, k, ydt, ldx_pad, ldy_pad, use_bias, nsplit, rng = _case(i)
    say("random", i, NAMES[fmt], "dq" if dq else "", "m", m, "n", n, "k", k, "bf16" if ydt == wq.WQ_BF16 else "f32",
        "ldx+", ldx_pad, "ldy+", ldy_pad, "bias" if use_bias else "no bias", "splits", nsplit)
    w, b, x = linear_case(9100 + i, n, k, m, outlier_frac=0.002)
    b = b if use_bias else None
    ref = orc.quantize(fmt, w, dq)
    d, codes, scales = gpu_quantize(fmt, w, dq)
    assert np.array_equal(codes.cpu().numpy(), ref["codes"]) and np.array_equal(scales.cpu().numpy(), ref["scales"])
    assert np.array_equal(gpu_dequantize(d, codes, scales).view(np.uint32), ref["w_hat"].view(np.uint32))

    ldx = k + ldx_pad
    xb = np.full((m, ldx), 0x7FC0, np.uint16)          # padding columns hold NaN
    xb[:, :k] = x
    X = dev_bf16(xb)
    B = None if b is None else dev_bf16(b)
    es = 4 if ydt == wq.WQ_F32 else 2
    ws, wsb = workspace(d, m, seed=i)
    if nsplit == 1:
        ldy = n + ldy_pad
        Y = (torch.full((m, ldy), -12345.0, dtype=torch.float32, device=DEV) if es == 4
             else torch.full((m, ldy), 0x7BAD, dtype=torch.int16, device=DEV))
        wq.wq_matmul(d, m, X, ldx, codes, scales, B, Y, ydt, ldy, ws, wsb)
        torch.cuda.synchronize()
        yall = Y.cpu().numpy()
        if ldy_pad:
            pad = yall[:, n:]
            assert np.all(pad == (-12345.0 if es == 4 else 0x7BAD)), "columns past n were written"
        y = yall[:, :n]
    else:
        # split ends at any column: inside a 16-column band, off the 4- and 8-column store grids
        cuts = np.sort(rng.choice(np.arange(1, n), size=nsplit - 1, replace=False))
        split_n = np.diff(np.concatenate([[0], cuts, [n]])).astype(np.int64).tolist()
        # each split into its own buffer with its own row stride
        ldys = [s_ + int(rng.integers(0, 4)) for s_ in split_n]
        bufs = [(torch.full((m, l), -12345.0, dtype=torch.float32, device=DEV) if es == 4
                 else torch.full((m, l), 0x7BAD, dtype=torch.int16, device=DEV)) for l in ldys]
        wq.wq_matmul_qkv(d, m, X, ldx, codes, scales, B, split_n, [t.data_ptr() for t in bufs], ldys, ydt, ws, wsb)
        torch.cuda.synchronize()
        parts = []
        for t, s_, l in zip(bufs, split_n, ldys):
            a = t.cpu().numpy()
            if l > s_:
                assert np.all(a[:, s_:] == (-12345.0 if es == 4 else 0x7BAD)), "columns past a split were written"
            parts.append(a[:, :s_])
        y = np.concatenate(parts, axis=1)
    if es == 2:
        y = bf16_bits_to_f32(np.ascontiguousarray(y).view(np.uint16))
    rows = None if m * n * k <= 64 * 1024 * 1024 else np.unique(np.concatenate([[0, m - 1], rng.choice(m, 48)]))
    y_ref = orc.matmul(x, ref["w_hat"], b, rows=rows)
    yy = y if rows is None else y[rows]
    check_bound(yy, y_ref, abs_dot(x, ref["w_hat"], rows=rows), bf16_out=es == 2,
                what=f"random {i} {NAMES[fmt]} m={m} n={n} k={k} splits={nsplit}")
    assert np.all(np.isfinite(y))
