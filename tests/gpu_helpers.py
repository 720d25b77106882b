"""Helpers for the GPU parity tests: move seeded inputs to the device, call
libwq through its C ABI, and compare with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from block_quantized_bit_amd import wq
from block_quantized_bit_amd.inputs import bf16_bits_to_f32

DEV = "cuda:0"
NAMES = {1: "nf4", 2: "nvfp4", 3: "q4_0", 4: "q8_0", 5: "q4_1", 6: "q5_0", 7: "q4_k", 8: "q6_k"}


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X; refusing to pass vacuously"
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), f"expected gfx950, found {name}"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns -> int16 device tensor (same bytes)."""
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).to(DEV)


def gpu_quantize(fmt: int, w: np.ndarray, dq: bool = False):
    n, k = w.shape
    d = wq.desc(fmt, n, k, dq)
    cb, sb = wq.wq_packed_size(d)
    W = torch.from_numpy(np.ascontiguousarray(w, np.float32)).to(DEV)
    codes = torch.full((cb,), 0xA5, dtype=torch.uint8, device=DEV)
    scales = torch.full((sb,), 0x5A, dtype=torch.uint8, device=DEV)
    wq.wq_quantize(d, W, codes, scales)
    torch.cuda.synchronize()
    return d, codes, scales


def gpu_dequantize(d, codes, scales):
    out = torch.full((d.n, d.k), float("nan"), dtype=torch.float32, device=DEV)
    wq.wq_dequantize(d, codes, scales, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def workspace(d, m, seed=77):
    """The workspace a call asks for, filled with seeded random bytes: the library
    must not rely on its contents."""
    b = wq.wq_workspace_size(d, m)
    if b == 0:
        return None, 0
    junk = np.random.default_rng(seed).integers(0, 256, size=b, dtype=np.uint8)
    return torch.from_numpy(junk).to(DEV), b


def gpu_matmul(d, codes, scales, x_bits: np.ndarray, bias_bits, ydt=wq.WQ_F32, use_ws=True,
               ldx_pad: int = 0, ldy_pad: int = 0):
    m, k = x_bits.shape
    ldx = k + ldx_pad
    xb = np.full((m, ldx), 0x7FC0, np.uint16)                  # padding columns hold NaN
    xb[:, :k] = x_bits
    X = dev_bf16(xb)
    B = None if bias_bits is None else dev_bf16(bias_bits)
    ldy = d.n + ldy_pad
    if ydt == wq.WQ_F32:
        Y = torch.full((m, ldy), -12345.0, dtype=torch.float32, device=DEV)
    else:
        Y = torch.full((m, ldy), 0x7BAD, dtype=torch.int16, device=DEV)
    ws, wsb = workspace(d, m) if use_ws else (None, 0)
    wq.wq_matmul(d, m, X, ldx, codes, scales, B, Y, ydt, ldy, ws, wsb)
    torch.cuda.synchronize()
    y = Y.cpu().numpy()
    if ldy_pad:
        pad = y[:, d.n:]
        if ydt == wq.WQ_F32:
            assert np.all(pad == -12345.0), "columns beyond n were written"
        else:
            assert np.all(pad == 0x7BAD), "columns beyond n were written"
    y = y[:, :d.n]
    if ydt == wq.WQ_BF16:
        y = bf16_bits_to_f32(y.view(np.uint16))
    return y


def abs_dot(x_bits: np.ndarray, w_hat: np.ndarray, rows=None) -> np.ndarray:
    xf = bf16_bits_to_f32(x_bits).astype(np.float64)
    if rows is not None:
        xf = xf[rows]
    return np.abs(xf) @ np.abs(w_hat.astype(np.float64)).T


def check_bound(y, y_ref, absdot, bf16_out=False, what=""):
    """|y - y_ref| <= 4e-3 * sum_k |x_k w^_k| + 1e-6 (+ the final bf16 rounding for bf16 output)."""
    tol = 4e-3 * absdot + 1e-6
    if bf16_out:
        tol = tol + np.abs(y_ref.astype(np.float64)) * 2.0 ** -8
    err = np.abs(y.astype(np.float64) - y_ref.astype(np.float64))
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements outside the bound; first {tuple(i)} "
                             f"y={y[tuple(i)]} ref={y_ref[tuple(i)]} tol={tol[tuple(i)]}")
    return float((err / np.maximum(absdot, 1e-30)).max())
