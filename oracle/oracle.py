"""ctypes wrapper over the plain C oracle (oracle/oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
CPU-baseline leg of the bench, never by the library.  It shares no code with
the HIP path; it only receives the same seeded inputs.

Format numbers match the library's public enum values so a test can pass one
number to both sides: NF4 = 1, NVFP4 = 2, Q4_0 = 3, Q8_0 = 4, Q4_1 = 5, Q5_0 = 6, Q4_K = 7,
Q6_K = 8.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

NF4, NVFP4, Q4_0, Q8_0, Q4_1, Q5_0, Q4_K, Q6_K = 1, 2, 3, 4, 5, 6, 7, 8

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_CMD = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-fopenmp", "-o", _LIB, _SRC, "-lm"]


def build() -> str:
    """Compile the oracle with gcc (always; cheap)."""
    subprocess.run(GCC_CMD, check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.or_bf16_to_f32.restype = ctypes.c_float
        L.or_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.or_fp16_decode.restype = ctypes.c_float
        L.or_fp16_decode.argtypes = [ctypes.c_uint16]
        L.or_fp16_encode.restype = ctypes.c_uint16
        L.or_fp16_encode.argtypes = [ctypes.c_float]
        L.or_e4m3_decode.restype = ctypes.c_float
        L.or_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.or_e4m3_encode.restype = ctypes.c_uint8
        L.or_e4m3_encode.argtypes = [ctypes.c_float]
        L.or_e2m1_decode.restype = ctypes.c_float
        L.or_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.or_e2m1_encode.restype = ctypes.c_uint8
        L.or_e2m1_encode.argtypes = [ctypes.c_float]
        L.or_nf4_codebook.restype = None
        L.or_nf4_codebook.argtypes = [P, P]
        for name in ("or_nf4_quantize",):
            getattr(L, name).argtypes = [i64, i64, P, P, P]
        L.or_nf4_double_quant.argtypes = [i64, P, P, P, P]
        L.or_nf4_dq_absmax.argtypes = [i64, P, P, ctypes.c_float, P]
        L.or_nf4_dequantize.argtypes = [i64, i64, P, P, P]
        L.or_nvfp4_quantize.argtypes = [i64, i64, P, P, P, P]
        L.or_nvfp4_dequantize.argtypes = [i64, i64, P, P, ctypes.c_float, P]
        L.or_q8_0_quantize.argtypes = [i64, i64, P, P, P]
        L.or_q8_0_dequantize.argtypes = [i64, i64, P, P, P]
        L.or_q4_0_quantize.argtypes = [i64, i64, P, P, P]
        L.or_q4_0_dequantize.argtypes = [i64, i64, P, P, P]
        L.or_q4_1_quantize.argtypes = [i64, i64, P, P, P]
        L.or_q4_1_dequantize.argtypes = [i64, i64, P, P, P]
        L.or_q5_0_quantize.argtypes = [i64, i64, P, P, P]
        L.or_q5_0_dequantize.argtypes = [i64, i64, P, P, P]
        L.or_q4_k_quantize.argtypes = [i64, i64, P, P, P, P]
        L.or_q4_k_dequantize.argtypes = [i64, i64, P, P, P, P]
        L.or_q6_k_quantize.argtypes = [i64, i64, P, P, P, P]
        L.or_q6_k_dequantize.argtypes = [i64, i64, P, P, P, P]
        L.or_packed_size.restype = ctypes.c_int
        L.or_packed_size.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64,
                                     ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.or_pack_codes4.argtypes = [i64, i64, P, P]
        L.or_pack_codes8.argtypes = [i64, i64, P, P]
        L.or_unpack_codes4.argtypes = [i64, i64, P, P]
        L.or_pack_scales.argtypes = [i64, i64, i64, i64, ctypes.c_int, P, P]
        L.or_quantize_packed.restype = ctypes.c_int
        L.or_quantize_packed.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, P, P, P, P, P]
        L.or_matmul_rows.argtypes = [i64, P, i64, i64, P, P, P, P]
        L.or_act_scales_bytes.restype = i64
        L.or_act_scales_bytes.argtypes = [i64, i64]
        L.or_quantize_act_nvfp4.argtypes = [i64, i64, P, P, P, P, P]
        L.or_matmul_rows_f32x.argtypes = [i64, P, i64, i64, P, P, P, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---- scalar codecs -------------------------------------------------------------

def fp16_encode(x: float) -> int:
    return int(lib().or_fp16_encode(float(x)))


def fp16_decode(h: int) -> float:
    return float(lib().or_fp16_decode(int(h)))


def e4m3_encode(x: float) -> int:
    return int(lib().or_e4m3_encode(float(x)))


def e4m3_decode(b: int) -> float:
    return float(lib().or_e4m3_decode(int(b)))


def e2m1_encode(x: float) -> int:
    return int(lib().or_e2m1_encode(float(x)))


def e2m1_decode(c: int) -> float:
    return float(lib().or_e2m1_decode(int(c)))


def nf4_codebook():
    c = np.zeros(16, np.float32)
    mid = np.zeros(15, np.float64)
    lib().or_nf4_codebook(_p(c), _p(mid))
    return c, mid


# ---- per-format logical quantizers ----------------------------------------------

def nf4_quantize(w: np.ndarray):
    w = np.ascontiguousarray(w, np.float32)
    n, k = w.shape
    codes = np.zeros((n, k), np.uint8)
    a = np.zeros(n * k // 64, np.float32)
    lib().or_nf4_quantize(n, k, _p(w), _p(codes), _p(a))
    return codes, a


def nf4_double_quant(a: np.ndarray):
    a = np.ascontiguousarray(a, np.float32)
    nb = a.size
    q = np.zeros(nb, np.int8)
    d = np.zeros((nb + 255) // 256, np.float32)
    mu = np.zeros(1, np.float32)
    lib().or_nf4_double_quant(nb, _p(a), _p(q), _p(d), _p(mu))
    return q, d, np.float32(mu[0])


def nf4_dq_absmax(q, d, mu):
    q = np.ascontiguousarray(q, np.int8)
    d = np.ascontiguousarray(d, np.float32)
    out = np.zeros(q.size, np.float32)
    lib().or_nf4_dq_absmax(q.size, _p(q), _p(d), float(mu), _p(out))
    return out


def nf4_dequantize(codes, absmax):
    codes = np.ascontiguousarray(codes, np.uint8)
    absmax = np.ascontiguousarray(absmax, np.float32)
    n, k = codes.shape
    out = np.zeros((n, k), np.float32)
    lib().or_nf4_dequantize(n, k, _p(codes), _p(absmax), _p(out))
    return out


def nvfp4_quantize(w: np.ndarray):
    w = np.ascontiguousarray(w, np.float32)
    n, k = w.shape
    codes = np.zeros((n, k), np.uint8)
    s = np.zeros(n * k // 16, np.uint8)
    g = np.zeros(1, np.float32)
    lib().or_nvfp4_quantize(n, k, _p(w), _p(codes), _p(s), _p(g))
    return codes, s, np.float32(g[0])


def nvfp4_dequantize(codes, scales, g):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    n, k = codes.shape
    out = np.zeros((n, k), np.float32)
    lib().or_nvfp4_dequantize(n, k, _p(codes), _p(scales), float(g), _p(out))
    return out


def q8_0_quantize(w: np.ndarray):
    w = np.ascontiguousarray(w, np.float32)
    n, k = w.shape
    codes = np.zeros((n, k), np.int8)
    s = np.zeros(n * k // 32, np.uint16)
    lib().or_q8_0_quantize(n, k, _p(w), _p(codes), _p(s))
    return codes, s


def q8_0_dequantize(codes, scales):
    codes = np.ascontiguousarray(codes, np.int8)
    scales = np.ascontiguousarray(scales, np.uint16)
    n, k = codes.shape
    out = np.zeros((n, k), np.float32)
    lib().or_q8_0_dequantize(n, k, _p(codes), _p(scales), _p(out))
    return out


def q4_0_quantize(w: np.ndarray):
    w = np.ascontiguousarray(w, np.float32)
    n, k = w.shape
    codes = np.zeros((n, k), np.uint8)
    s = np.zeros(n * k // 32, np.uint16)
    lib().or_q4_0_quantize(n, k, _p(w), _p(codes), _p(s))
    return codes, s


def q4_0_dequantize(codes, scales):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint16)
    n, k = codes.shape
    out = np.zeros((n, k), np.float32)
    lib().or_q4_0_dequantize(n, k, _p(codes), _p(scales), _p(out))
    return out


def q4_1_quantize(w: np.ndarray):
    """Logical codes [n,k] and scales [n*k/32, 2] (fp16 bits: d, m)."""
    w = np.ascontiguousarray(w, np.float32)
    n, k = w.shape
    codes = np.zeros((n, k), np.uint8)
    s = np.zeros((n * k // 32, 2), np.uint16)
    lib().or_q4_1_quantize(n, k, _p(w), _p(codes), _p(s))
    return codes, s


def q4_1_dequantize(codes, scales):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint16)
    n, k = codes.shape
    out = np.zeros((n, k), np.float32)
    lib().or_q4_1_dequantize(n, k, _p(codes), _p(scales), _p(out))
    return out


def q5_0_quantize(w: np.ndarray):
    """Logical 5-bit codes [n,k] (0..31) and fp16 scales [n*k/32]."""
    w = np.ascontiguousarray(w, np.float32)
    n, k = w.shape
    codes = np.zeros((n, k), np.uint8)
    s = np.zeros(n * k // 32, np.uint16)
    lib().or_q5_0_quantize(n, k, _p(w), _p(codes), _p(s))
    return codes, s


def q5_0_dequantize(codes, scales):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint16)
    n, k = codes.shape
    out = np.zeros((n, k), np.float32)
    lib().or_q5_0_dequantize(n, k, _p(codes), _p(scales), _p(out))
    return out


def q4_k_quantize(w: np.ndarray):
    """Logical codes [n,k], sub-block (sc, m) bytes [n*k/32, 2], super-block fp16
    (d, dmin) [n*k/256, 2]."""
    w = np.ascontiguousarray(w, np.float32)
    n, k = w.shape
    codes = np.zeros((n, k), np.uint8)
    sub = np.zeros((n * k // 32, 2), np.uint8)
    dd = np.zeros((n * k // 256, 2), np.uint16)
    lib().or_q4_k_quantize(n, k, _p(w), _p(codes), _p(sub), _p(dd))
    return codes, sub, dd


def q4_k_dequantize(codes, sub, dd):
    codes = np.ascontiguousarray(codes, np.uint8)
    sub = np.ascontiguousarray(sub, np.uint8)
    dd = np.ascontiguousarray(dd, np.uint16)
    n, k = codes.shape
    out = np.zeros((n, k), np.float32)
    lib().or_q4_k_dequantize(n, k, _p(codes), _p(sub), _p(dd), _p(out))
    return out


def q6_k_quantize(w: np.ndarray):
    """Logical 6-bit codes [n,k] (0..63), int8 sub-block scales [n*k/16], fp16 d [n*k/256]."""
    w = np.ascontiguousarray(w, np.float32)
    n, k = w.shape
    codes = np.zeros((n, k), np.uint8)
    sc = np.zeros(n * k // 16, np.int8)
    d = np.zeros(n * k // 256, np.uint16)
    lib().or_q6_k_quantize(n, k, _p(w), _p(codes), _p(sc), _p(d))
    return codes, sc, d


def q6_k_dequantize(codes, sc, d):
    codes = np.ascontiguousarray(codes, np.uint8)
    sc = np.ascontiguousarray(sc, np.int8)
    d = np.ascontiguousarray(d, np.uint16)
    n, k = codes.shape
    out = np.zeros((n, k), np.float32)
    lib().or_q6_k_dequantize(n, k, _p(codes), _p(sc), _p(d), _p(out))
    return out


# ---- packed form ---------------------------------------------------------------

def packed_size(fmt: int, dq: bool, n: int, k: int):
    cb = ctypes.c_int64()
    sb = ctypes.c_int64()
    rc = lib().or_packed_size(fmt, int(bool(dq)), n, k, ctypes.byref(cb), ctypes.byref(sb))
    if rc:
        raise ValueError(f"unsupported shape/format for oracle: fmt={fmt} n={n} k={k}")
    return cb.value, sb.value


def pack_codes4(codes):
    codes = np.ascontiguousarray(codes, np.uint8)
    n, k = codes.shape
    out = np.zeros(n * k // 2, np.uint8)
    lib().or_pack_codes4(n, k, _p(codes), _p(out))
    return out


def unpack_codes4(packed, n, k):
    packed = np.ascontiguousarray(packed, np.uint8)
    out = np.zeros((n, k), np.uint8)
    lib().or_unpack_codes4(n, k, _p(packed), _p(out))
    return out


def pack_codes8(codes):
    codes = np.ascontiguousarray(codes, np.int8)
    n, k = codes.shape
    out = np.zeros(n * k, np.int8)
    lib().or_pack_codes8(n, k, _p(codes), _p(out))
    return out


def quantize(fmt: int, w: np.ndarray, dq: bool = False):
    """Quantize W[n,k] -> dict(codes=packed uint8, scales=packed uint8,
    logical=logical codes [n,k], w_hat=dequantized fp32 [n,k])."""
    w = np.ascontiguousarray(w, np.float32)
    n, k = w.shape
    cb, sb = packed_size(fmt, dq, n, k)
    codes = np.zeros(cb, np.uint8)
    scales = np.zeros(sb, np.uint8)
    logical = np.zeros((n, k), np.uint8)
    w_hat = np.zeros((n, k), np.float32)
    rc = lib().or_quantize_packed(fmt, int(bool(dq)), n, k, _p(w), _p(codes), _p(scales),
                                  _p(logical), _p(w_hat))
    if rc:
        raise ValueError("oracle quantize failed")
    return dict(codes=codes, scales=scales, logical=logical, w_hat=w_hat)


def matmul(x_bf16: np.ndarray, w_hat: np.ndarray, bias_bf16=None, rows=None):
    """y = X * W^T + b as the oracle defines it (fp32, k ascending).  `rows`
    selects rows of X; returns [len(rows) or m, n] float32."""
    x = np.ascontiguousarray(x_bf16, np.uint16)
    w_hat = np.ascontiguousarray(w_hat, np.float32)
    m, k = x.shape
    n = w_hat.shape[0]
    assert w_hat.shape[1] == k
    if rows is None:
        nr = m
        rp = None
    else:
        rows = np.ascontiguousarray(rows, np.int64)
        nr = rows.size
        rp = _p(rows)
    y = np.zeros((nr, n), np.float32)
    b = None if bias_bf16 is None else np.ascontiguousarray(bias_bf16, np.uint16)
    lib().or_matmul_rows(nr, rp, n, k, _p(x), _p(w_hat), None if b is None else _p(b), _p(y))
    return y


def quantize_act_nvfp4(x_bf16: np.ndarray):
    """NVFP4 activations (W4A4): X[m,k] bf16 bits -> dict(codes=[m*k/2] packed row-major,
    scales=E4M3 [m][k/16] then the fp32 global scale at align16(m*k/16), logical=[m,k] codes,
    x_hat=[m,k] fp32, g=global scale)."""
    x = np.ascontiguousarray(x_bf16, np.uint16)
    m, k = x.shape
    if k % 16:
        raise ValueError("k must be a multiple of 16")
    codes = np.zeros(m * k // 2, np.uint8)
    scales = np.zeros(int(lib().or_act_scales_bytes(m, k)), np.uint8)
    logical = np.zeros((m, k), np.uint8)
    x_hat = np.zeros((m, k), np.float32)
    lib().or_quantize_act_nvfp4(m, k, _p(x), _p(codes), _p(scales), _p(logical), _p(x_hat))
    g = np.frombuffer(scales[-4:].tobytes(), np.float32)[0]
    return dict(codes=codes, scales=scales, logical=logical, x_hat=x_hat, g=np.float32(g))


def matmul_f32x(x: np.ndarray, w_hat: np.ndarray, bias_bf16=None, rows=None):
    """y = X * W^T + b with fp32 X (the dequantized activations of a W4A4 product), fp32 sums
    in k-ascending order as matmul()."""
    x = np.ascontiguousarray(x, np.float32)
    w_hat = np.ascontiguousarray(w_hat, np.float32)
    m, k = x.shape
    n = w_hat.shape[0]
    assert w_hat.shape[1] == k
    rp = None
    nr = m
    if rows is not None:
        rows = np.ascontiguousarray(rows, np.int64)
        nr = rows.size
        rp = _p(rows)
    y = np.zeros((nr, n), np.float32)
    b = None if bias_bf16 is None else np.ascontiguousarray(bias_bf16, np.uint16)
    lib().or_matmul_rows_f32x(nr, rp, n, k, _p(x), _p(w_hat), None if b is None else _p(b), _p(y))
    return y


def pack_scales(n: int, k: int, bs: int, per_tile_k: int, logical: np.ndarray) -> np.ndarray:
    """Place logical per-block scales [n][k/bs] (any element size) into the tile order."""
    logical = np.ascontiguousarray(logical)
    esz = logical.dtype.itemsize
    out = np.zeros(logical.size, logical.dtype)
    lib().or_pack_scales(n, k, bs, per_tile_k, esz, _p(logical), _p(out))
    return out
