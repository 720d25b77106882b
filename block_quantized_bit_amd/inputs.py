"""Seeded synthetic inputs for the weight-only 4-bit matmul (shared by tests and bench).

This module draws random tensors and nothing else: it holds none of the
quantization or matmul arithmetic.  Both the CPU oracle and the HIP path
receive exactly the arrays produced here.

Shapes follow the Whisper Linear layers the pages talk about: d_model 1280,
FFN 5120, 1500 encoder frames, token-at-a-time decode with up to 16 concurrent
requests ("mbehr90/whisper-large-v3-turbo-nvfp4", sections "Measured on H100"
and "Why the encoder/decoder split matters"); whisper-tiny fc1 is 384 -> 1536.

Recipe (numpy Generator(PCG64(seed))), generation order W -> outliers -> bias -> X:
  * W[N, K]  float32 = standard_normal(float32) * std (per-row std optional)
  * outliers: rng.choice(N*K, round(frac*N*K), replace=False) entries multiplied by `mult`
  * bias[N]  bf16    = RNE(standard_normal(float32) * 0.01)
  * X[M, K]  bf16    = RNE(standard_normal(float32))
All bf16 tensors are returned as uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "gen_weight", "gen_bias", "gen_x",
    "linear_case", "WHISPER_D", "WHISPER_FFN", "ENC_FRAMES",
]

WHISPER_D = 1280
WHISPER_FFN = 5120
ENC_FRAMES = 1500


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even), returned as uint16 bits.

    Inputs are finite by construction; this is plumbing for the activations, not
    part of the method.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def gen_weight(rng: np.random.Generator, n: int, k: int, std: float = 0.02,
               row_lognormal_sigma: float | None = None,
               outlier_frac: float = 0.0, outlier_mult: float = 8.0) -> np.ndarray:
    """W[n, k] float32.  With `row_lognormal_sigma`, row n is scaled by r_n ~ LogNormal(0, sigma)."""
    if row_lognormal_sigma is not None:
        r = rng.lognormal(0.0, row_lognormal_sigma, size=n).astype(np.float32)
        z = rng.standard_normal((n, k), dtype=np.float32)
        w = (np.float32(std) * r[:, None]) * z
    else:
        w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(std)
    w = np.ascontiguousarray(w, dtype=np.float32)
    if outlier_frac > 0:
        cnt = int(round(outlier_frac * n * k))
        idx = rng.choice(n * k, size=cnt, replace=False)
        flat = w.reshape(-1)
        flat[idx] *= np.float32(outlier_mult)
    return w


def gen_bias(rng: np.random.Generator, n: int, std: float = 0.01) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(n, dtype=np.float32) * np.float32(std))


def gen_x(rng: np.random.Generator, m: int, k: int) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))


def linear_case(seed: int, n: int, k: int, m: int, *, std: float = 0.02,
                row_lognormal_sigma: float | None = None, outlier_frac: float = 0.0,
                bias: bool = True):
    """One seeded Linear: returns (W f32 [n,k], bias bf16 bits [n] or None, X bf16 bits [m,k])."""
    rng = np.random.Generator(np.random.PCG64(seed))
    w = gen_weight(rng, n, k, std=std, row_lognormal_sigma=row_lognormal_sigma,
                   outlier_frac=outlier_frac)
    b = gen_bias(rng, n) if bias else None
    x = gen_x(rng, m, k)
    return w, b, x
