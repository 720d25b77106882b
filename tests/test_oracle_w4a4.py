"""Pins for the oracle's NVFP4 activation quantizer and its fp32-activation matmul (W4A4).

"mbehr90/whisper-large-v3-turbo-nvfp4", section "What is quantized": activations are quantized
per 16-value group at run time, with the same element (E2M1) and block-scale (E4M3) formats as
the weights.  Each check compares the oracle with something other than itself:

  * brute force over the 8 E2M1 magnitudes and the 127 finite positive E4M3 values (decoded
    here from the bit fields, not by the oracle);
  * blocks built from representable values, which must come back exactly;
  * the amax block's scale saturating at 448, the largest E4M3 value;
  * zero inputs;
  * the weight quantizer (pinned elsewhere) on the same fp32 values;
  * the packed bytes decoded by hand;
  * fp64 sums within the fp32 summation bound for the matmul.
"""
import numpy as np
import pytest
import torch

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e4m3_value(b: int) -> float:
    """E4M3 (OCP FP8, bias 7, no infinities) from its bit fields."""
    s = -1.0 if b & 0x80 else 1.0
    e, m = (b >> 3) & 15, b & 7
    if e == 0:
        return s * m / 8.0 * 2.0 ** -6
    if e == 15 and m == 7:
        return float("nan")
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_POS = np.array([e4m3_value(b) for b in range(127)])        # bytes 0x00..0x7E, all finite


def bf16_bits(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def nearest_even(grid: np.ndarray, q: float) -> int:
    """Index of the grid value nearest q; on a tie the even index (mantissa bit 0)."""
    d = np.abs(grid - q)
    best = np.flatnonzero(d == d.min())
    ev = [i for i in best if i % 2 == 0]
    return int(ev[0] if ev else best[0])


def unpack_codes(packed: np.ndarray, m: int, k: int) -> np.ndarray:
    """Row-major packed nibbles -> [m, k] codes; element 2j in the low nibble of byte j."""
    out = np.zeros(m * k, np.uint8)
    out[0::2] = packed & 15
    out[1::2] = packed >> 4
    return out.reshape(m, k)


def decode_act(q: dict, m: int, k: int) -> np.ndarray:
    """Values the packed activation encodes, from the bytes alone (in float64)."""
    codes = unpack_codes(q["codes"], m, k)
    nb = m * (k // 16)
    sc = np.array([e4m3_value(int(b)) for b in q["scales"][:nb]]).reshape(m, k // 16)
    off = (nb + 15) // 16 * 16
    g = float(np.frombuffer(q["scales"][off:off + 4].tobytes(), np.float32)[0])
    sign = np.where(codes & 8, -1.0, 1.0)
    return sign * E2M1[codes & 7] * np.repeat(sc, 16, axis=1) * g, g


def test_brute_force_scales_and_codes(orc):
    """Every block scale is the E4M3 value nearest a_b / (6 g) and every code the E2M1
    magnitude nearest |x| / sigma, by enumeration, with g = amax / (6 * 448)."""
    rng = np.random.default_rng(11)
    m, k = 3, 64
    x = rng.standard_normal((m, k)).astype(np.float32) * np.exp2(rng.integers(-6, 6, (m, 1)))
    xb = bf16_bits(x)
    xf = bf16_value(xb)
    q = orc.quantize_act_nvfp4(xb)
    amax = np.float32(np.abs(xf).max())
    g = np.float32(amax / np.float32(2688.0))
    assert q["g"] == g
    t = np.float32(np.float32(6.0) * g)
    sbytes = q["scales"][:m * k // 16].reshape(m, k // 16)
    for r in range(m):
        for b in range(k // 16):
            blk = xf[r, 16 * b:16 * b + 16]
            ratio = np.float32(np.float32(np.abs(blk).max()) / t)
            assert sbytes[r, b] == nearest_even(E4M3_POS, float(ratio))
            sigma = np.float32(np.float32(E4M3_POS[sbytes[r, b]]) * g)
            for i, v in enumerate(blk):
                c = q["logical"][r, 16 * b + i]
                assert c & 7 == nearest_even(E2M1, float(np.float32(abs(v) / sigma)))
                assert (c >> 3) == (1 if np.signbit(v) else 0)


def test_packed_bytes_decode_to_x_hat(orc):
    """The packed codes and scales, decoded by hand, give x_hat; logical codes agree with the
    nibbles (even k in the low nibble)."""
    rng = np.random.default_rng(12)
    m, k = 5, 48
    xb = bf16_bits(rng.standard_normal((m, k)))
    q = orc.quantize_act_nvfp4(xb)
    assert np.array_equal(unpack_codes(q["codes"], m, k), q["logical"])
    dec, g = decode_act(q, m, k)
    assert g == q["g"]
    # x_hat = fl(fl(e2m1 * s) * g): the e2m1*s product is exact, one rounding for * g
    ref = (dec / g).astype(np.float32) * np.float32(g)
    assert np.array_equal(q["x_hat"].view(np.uint32), ref.astype(np.float32).view(np.uint32))


def test_representable_blocks_round_trip_exactly(orc):
    """With amax = 2688 * 2^-4 the global scale is 2^-4; blocks whose max is 6 * s * g and
    whose elements are E2M1 multiples of s * g come back bit-exactly."""
    rng = np.random.default_rng(13)
    m, k = 4, 64
    g = 2.0 ** -4
    scales = [448.0, 1.0, 1.875, 0.5, 3.25, 0.015625, 104.0, 2.0 ** -9 * 5]
    x = np.zeros((m, k))
    si = 0
    for r in range(m):
        for b in range(k // 16):
            s = scales[si % len(scales)]
            si += 1
            mags = E2M1[rng.integers(0, 8, 16)]
            mags[rng.integers(0, 16)] = 6.0
            signs = np.where(rng.random(16) < 0.5, -1.0, 1.0)
            x[r, 16 * b:16 * b + 16] = signs * mags * s * g
    x[0, 0] = 6.0 * 448.0 * g      # the global amax
    xb = bf16_bits(x)
    assert np.array_equal(bf16_value(xb).astype(np.float64), x)
    q = orc.quantize_act_nvfp4(xb)
    assert q["g"] == np.float32(g)
    assert np.array_equal(q["x_hat"].astype(np.float64), x)


def test_amax_block_saturates_scale_and_code(orc):
    """The block that holds the global amax gets the largest E4M3 scale (448, byte 0x7E) and
    the amax element the largest E2M1 code."""
    rng = np.random.default_rng(14)
    m, k = 6, 96
    x = rng.standard_normal((m, k)).astype(np.float32)
    r0, c0 = 4, 37
    x[r0, c0] = -9.5
    xb = bf16_bits(x)
    q = orc.quantize_act_nvfp4(xb)
    assert q["scales"][r0 * (k // 16) + c0 // 16] == 0x7E
    assert q["logical"][r0, c0] == 0xF                      # sign + code 7 (magnitude 6)
    # every block that is not tiny against the amax keeps a max element coded as 6
    xf = bf16_value(xb)
    for r in range(m):
        for b in range(k // 16):
            blk = np.abs(xf[r, 16 * b:16 * b + 16])
            if blk.max() > np.abs(xf).max() / 64:
                assert (q["logical"][r, 16 * b + int(blk.argmax())] & 7) == 7


def test_zero_input_and_zero_rows(orc):
    m, k = 3, 32
    z = np.zeros((m, k), np.uint16)
    z[1, 5] = 0x8000                                         # -0
    q = orc.quantize_act_nvfp4(z)
    assert q["g"] == 0 and not q["x_hat"].any()
    assert not q["scales"].any()
    assert q["logical"][1, 5] == 8 and np.count_nonzero(q["logical"]) == 1
    # a zero row inside a nonzero matrix: scale bytes 0 and x_hat 0 for that row
    rng = np.random.default_rng(15)
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[2] = 0
    q = orc.quantize_act_nvfp4(bf16_bits(x))
    assert not q["scales"][2 * (k // 16):3 * (k // 16)].any()
    assert not q["x_hat"][2].any()


def test_agrees_with_the_weight_quantizer(orc):
    """Activation quantization is the weight rule applied to X: same codes, scales and g as the
    NVFP4 weight quantizer on the same fp32 values."""
    rng = np.random.default_rng(16)
    m, k = 7, 160
    xb = bf16_bits(rng.standard_normal((m, k)) * 3)
    q = orc.quantize_act_nvfp4(xb)
    codes, s, g = orc.nvfp4_quantize(bf16_value(xb).reshape(m, k))
    assert np.array_equal(q["logical"], codes)
    assert np.array_equal(q["scales"][:m * k // 16], s)
    assert q["g"] == g


def test_rejects_k_not_multiple_of_16(orc):
    with pytest.raises(ValueError):
        orc.quantize_act_nvfp4(np.zeros((2, 24), np.uint16))


def test_f32x_matmul_equals_bf16_matmul_on_bf16_inputs(orc):
    """With X exactly bf16 the fp32-activation product is the bf16 one bit for bit."""
    rng = np.random.default_rng(17)
    m, n, k = 5, 19, 96
    xb = bf16_bits(rng.standard_normal((m, k)))
    w = rng.standard_normal((n, k)).astype(np.float32) * 0.02
    bias = bf16_bits(rng.standard_normal(n) * 0.01)
    a = orc.matmul(xb, w, bias)
    b = orc.matmul_f32x(bf16_value(xb), w, bias)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    rows = np.array([4, 0, 2])
    assert np.array_equal(orc.matmul_f32x(bf16_value(xb), w, bias, rows=rows), b[rows])


def test_w4a4_product_within_fp32_bound_of_exact(orc):
    """y = x_hat . w_hat^T + b from the quantized operands, within the fp32 summation bound
    of the fp64 sum of the same operands."""
    rng = np.random.default_rng(18)
    m, n, k = 6, 33, 320
    xb = bf16_bits(rng.standard_normal((m, k)))
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    qa = orc.quantize_act_nvfp4(xb)
    w_hat = orc.nvfp4_dequantize(*orc.nvfp4_quantize(w))
    y = orc.matmul_f32x(qa["x_hat"], w_hat)
    exact = qa["x_hat"].astype(np.float64) @ w_hat.astype(np.float64).T
    mag = np.abs(qa["x_hat"].astype(np.float64)) @ np.abs(w_hat.astype(np.float64)).T
    assert np.all(np.abs(y - exact) <= (k + 1) * 2.0 ** -24 * mag + 1e-30)
    # x_hat is the exact decoded value after one fp32 rounding
    dec, _ = decode_act(qa, m, k)
    assert np.allclose(dec, qa["x_hat"], rtol=2 ** -23, atol=0)
