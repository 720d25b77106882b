"""Pins for the oracle's block quantizers: brute force on tiny blocks, exact
reproduction of the block-absmax element, round trips on representable values,
exact-rational bounds for the double-quant mean, and special cases.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

NF4, NVFP4, Q4_0, Q8_0 = 1, 2, 3, 4


def _f32(x):
    return np.float32(x)


# ------------------------------------------------------------------ NF4 ----

def _nf4_brute(x, c):
    """Nearest level to x by exhaustive search in exact arithmetic; ties go to
    the lower index."""
    d = [abs(Fraction(float(x)) - Fraction(float(ci))) for ci in c]
    best = min(d)
    return d.index(best)


def test_nf4_codes_brute_force_random(orc):
    c, _ = orc.nf4_codebook()
    rng = np.random.default_rng(101)
    w = (rng.standard_normal((16, 128)) * 0.02).astype(np.float32)
    codes, a = orc.nf4_quantize(w)
    for r in range(16):
        for b in range(2):
            blk = w[r, 64 * b:64 * b + 64]
            amax = np.abs(blk).max()
            assert a[r * 2 + b] == amax
            for i in range(64):
                x = _f32(blk[i]) / _f32(amax)          # the block-normalised value
                assert codes[r, 64 * b + i] == _nf4_brute(x, c)


def test_nf4_codes_at_midpoints(orc):
    """Elements placed exactly on, and one ulp either side of, every midpoint."""
    c, mid = orc.nf4_codebook()
    vals = [1.0]
    for m in mid:
        f = np.float32(m)
        vals += [f, np.nextafter(f, np.float32(-2)), np.nextafter(f, np.float32(2))]
    vals = np.array(vals, np.float32)
    pad = (-len(vals)) % 64
    vals = np.concatenate([vals, np.zeros(pad, np.float32)])
    w = np.tile(vals.reshape(1, -1), (16, 1))
    k = w.shape[1]
    k2 = ((k + 127) // 128) * 128
    w = np.concatenate([w, np.zeros((16, k2 - k), np.float32)], axis=1)
    w[:, 64:128][:, 0] = 1.0                            # every block has absmax 1
    codes, a = orc.nf4_quantize(w)
    for i in range(k2):
        blk = i // 64
        amax = np.abs(w[0, 64 * blk:64 * blk + 64]).max()
        x = _f32(w[0, i]) / _f32(amax) if amax else None
        want = 7 if amax == 0 else _nf4_brute(x, c)
        assert codes[0, i] == want, (i, w[0, i])


def test_nf4_absmax_element_exact_and_round_trip(orc):
    c, _ = orc.nf4_codebook()
    rng = np.random.default_rng(5)
    a = np.float32(0.37)
    idx = rng.integers(0, 16, size=(16, 128))
    w = (c[idx] * a).astype(np.float32)                # fl(c_i * a)
    w[:, 0] = a
    w[:, 64] = -a
    codes, am = orc.nf4_quantize(w)
    assert np.all(am == a)
    want = idx.copy()
    want[:, 0] = 15
    want[:, 64] = 0
    assert np.array_equal(codes, want)
    w_hat = orc.nf4_dequantize(codes, am)
    assert np.array_equal(w_hat.view(np.uint32), w.view(np.uint32))


def test_nf4_zero_block(orc):
    w = np.zeros((16, 128), np.float32)
    w[3, 70] = 0.5                                     # one nonzero block
    codes, a = orc.nf4_quantize(w)
    assert a[3 * 2 + 1] == 0.5 and (a != 0).sum() == 1
    mask = np.ones_like(codes, bool)
    mask[3, 64:128] = False
    assert np.all(codes[mask] == 7)
    assert codes[3, 70] == 15
    w_hat = orc.nf4_dequantize(codes, a)
    assert np.array_equal(w_hat, w)


# ------------------------------------------------------ NF4 double-quant ----

def test_double_quant_mean_within_rounding_of_exact(orc):
    rng = np.random.default_rng(3)
    a = np.abs(rng.standard_normal(1000)).astype(np.float32) * np.float32(0.05)
    q, d, mu = orc.nf4_double_quant(a)
    exact = sum(Fraction(float(v)) for v in a) / len(a)
    # binary64 running sum (n roundings of <= 2^-53 relative) + division + cast to binary32
    err = abs(Fraction(float(mu)) - exact)
    bound = Fraction(len(a)) * Fraction(1, 2 ** 53) * exact * 2 + Fraction(float(mu)) * Fraction(1, 2 ** 24)
    assert err <= bound


def test_double_quant_codes_brute_force(orc):
    rng = np.random.default_rng(4)
    a = np.abs(rng.standard_normal(700)).astype(np.float32) * np.float32(0.03)
    q, d, mu = orc.nf4_double_quant(a)
    assert d.size == 3                                  # groups of 256, last partial
    for g in range(3):
        seg = a[256 * g:256 * (g + 1)]
        ap = [Fraction(float(_f32(v) - mu)) for v in seg]   # a' = fl(a - mu)
        sg = max(abs(v) for v in ap)
        # d_g is the binary32 value nearest to s_g / 127
        dg = Fraction(float(d[g]))
        assert abs(dg - sg / 127) <= abs(Fraction(float(np.nextafter(d[g], np.float32(1)))) - dg) / 2
        for i, v in enumerate(ap):
            # nearest integer in [-127, 127] to a'/d_g (ties to even) -- exact search
            t = v / dg
            cands = range(-127, 128)
            best = min(cands, key=lambda z: (abs(t - z), z % 2))
            qi = int(q[256 * g + i])
            if qi != best:
                # allowed only where binary32 rounding of a'/d_g moved it across .5
                assert abs(abs(t - qi) - Fraction(1, 2)) < Fraction(1, 2 ** 18)


def test_double_quant_reconstruction_and_group_counts(orc):
    rng = np.random.default_rng(6)
    a = np.abs(rng.standard_normal(513)).astype(np.float32)
    q, d, mu = orc.nf4_double_quant(a)
    ahat = orc.nf4_dq_absmax(q, d, mu)
    for i in range(a.size):
        qd = Fraction(int(q[i])) * Fraction(float(d[i // 256]))
        exact = qd + Fraction(float(mu))
        # two binary32 roundings: fl(q*d) then fl(. + mu), each <= 2^-24 relative
        u = Fraction(1, 2 ** 24)
        assert abs(Fraction(float(ahat[i])) - exact) <= u * abs(qd) * (1 + u) + u * (abs(exact) + u * abs(qd))
        assert abs(float(ahat[i]) - float(a[i])) <= float(d[i // 256]) * 0.5 * (1 + 1e-5) + 1e-7
    # group counts of the decoder GEMV set (64-blocks, 256-block groups)
    for (n, k), groups in {(3840, 1280): 300, (1280, 1280): 100, (5120, 1280): 400, (1280, 5120): 400}.items():
        cb, sb = orc.packed_size(NF4, True, n, k)
        nb = n * k // 64
        assert (sb - ((nb + 15) // 16) * 16 - 4) // 4 == groups


# ---------------------------------------------------------------- NVFP4 ----

def test_nvfp4_exact_on_representable_blocks(orc):
    """Power-of-two global scale and E4M3-valued block scales: every stage is
    exact, so codes and values must reproduce."""
    rng = np.random.default_rng(8)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    e4 = torch.arange(1, 0x7F, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    n, k = 16, 128
    g = np.float32(2.0 ** -12)
    s = e4[rng.integers(40, e4.size - 1, size=(n, k // 16))]        # block scales
    code = rng.integers(0, 8, size=(n, k))
    sign = rng.integers(0, 2, size=(n, k))
    code[:, ::16] = 7                                                   # every block reaches 6*s
    sign[0, 0] = 0
    s[0, 0] = 448                                                       # A = 6*448*g = 2688*g exactly
    w = (np.where(sign == 1, -1, 1) * mags[code]) * np.repeat(s, 16, axis=1) * g
    w = w.astype(np.float32)
    codes, sc, gg = orc.nvfp4_quantize(w)
    assert gg == g
    want_s = torch.from_numpy(s.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(sc.reshape(n, k // 16), want_s)
    assert np.array_equal(codes & 7, code)
    assert np.array_equal((codes >> 3) & 1, sign)
    w_hat = orc.nvfp4_dequantize(codes, sc, gg)
    assert np.array_equal(w_hat.view(np.uint32), w.view(np.uint32))


def test_nvfp4_codes_follow_independent_codecs(orc):
    """Random weights: scale bytes equal torch's E4M3 cast of fl(a_b/t) (or 448
    when above range), codes equal binade round-to-nearest-even of fl(w/sigma)."""
    rng = np.random.default_rng(9)
    n, k = 32, 256
    r = rng.lognormal(0, 0.3, n).astype(np.float32)
    w = (np.float32(0.02) * r[:, None] * rng.standard_normal((n, k), dtype=np.float32)).astype(np.float32)
    codes, sc, g = orc.nvfp4_quantize(w)
    A = np.abs(w).max()
    assert g == _f32(A) / _f32(2688)
    t = _f32(6) * g
    ab = np.abs(w).reshape(n, k // 16, 16).max(axis=2).astype(np.float32)
    ratio = (ab / t).astype(np.float32)
    want = torch.from_numpy(np.minimum(ratio, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(sc.reshape(n, k // 16), want)
    sval = torch.from_numpy(sc.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy().reshape(n, k // 16)
    sigma = (sval * g).astype(np.float32)
    y = (w / np.repeat(sigma, 16, axis=1)).astype(np.float32)
    a = np.abs(y).astype(np.float64)
    rne = np.where(a < 2, np.round(a / 0.5) * 0.5, np.where(a < 4, np.round(a), np.round(a / 2) * 2))
    rne = np.minimum(rne, 6)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    assert np.array_equal(mags[codes & 7], rne)
    assert np.array_equal((codes >> 3) & 1, np.signbit(w).astype(np.uint8))
    # the block holding the tensor absmax saturates to 448 or sits just below; never NaN
    assert sc.max() <= 0x7E
    w_hat = orc.nvfp4_dequantize(codes, sc, g)
    assert np.all(np.abs(w_hat - w) <= np.repeat(sigma, 16, axis=1) * 1.0 + 1e-12)


def test_nvfp4_zero_matrix_keeps_signs(orc):
    w = np.zeros((16, 128), np.float32)
    w[2, 5] = -0.0
    codes, sc, g = orc.nvfp4_quantize(w)
    assert g == 0 and np.all(sc == 0)
    assert codes[2, 5] == 8 and (codes == 8).sum() == 1
    w_hat = orc.nvfp4_dequantize(codes, sc, g)
    assert np.all(w_hat == 0) and np.signbit(w_hat[2, 5])


# ----------------------------------------------------------------- q8_0 ----

def _q_brute(w, delta, lo, hi):
    t = Fraction(float(w)) / Fraction(float(delta))
    return min(range(lo, hi + 1), key=lambda z: (abs(t - z), z % 2))


def test_q8_0_brute_force_and_scale(orc):
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((16, 64)) * 0.02).astype(np.float32)
    codes, sc = orc.q8_0_quantize(w)
    for r in range(16):
        for b in range(2):
            blk = w[r, 32 * b:32 * b + 32]
            a = np.abs(blk).max()
            want_d = np.array([_f32(a) / _f32(127)], np.float32).astype(np.float16).view(np.uint16)[0]
            assert sc[r * 2 + b] == want_d
            delta = np.uint16(want_d).view(np.float16).astype(np.float32)
            for i in range(32):
                qb = _q_brute(blk[i], delta, -127, 127)
                qi = int(codes[r, 32 * b + i])
                if qi != qb:
                    t = Fraction(float(blk[i])) / Fraction(float(delta))
                    assert abs(abs(t - qi) - Fraction(1, 2)) < Fraction(1, 2 ** 18)


def test_q8_0_absmax_exact_and_round_trip(orc):
    rng = np.random.default_rng(13)
    delta = np.float32(2.0 ** -9)
    q = rng.integers(-127, 128, size=(16, 64))
    q[:, 0] = 127
    q[:, 32] = -127
    w = (q * delta).astype(np.float32)
    codes, sc = orc.q8_0_quantize(w)
    assert np.array_equal(codes.astype(np.int64), q)
    w_hat = orc.q8_0_dequantize(codes, sc)
    assert np.array_equal(w_hat, w)
    # general absmax element: within 2^-11 relative
    w = (rng.standard_normal((16, 64)) * 0.02).astype(np.float32)
    codes, sc = orc.q8_0_quantize(w)
    w_hat = orc.q8_0_dequantize(codes, sc)
    for r in range(16):
        for b in range(2):
            blk = w[r, 32 * b:32 * b + 32]
            j = np.argmax(np.abs(blk))
            assert abs(w_hat[r, 32 * b + j] - blk[j]) <= 2.0 ** -11 * abs(blk[j]) * 1.0001


# ----------------------------------------------------------------- q4_0 ----

def test_q4_0_brute_force(orc):
    rng = np.random.default_rng(14)
    w = (rng.standard_normal((16, 128)) * 0.02).astype(np.float32)
    codes, sc = orc.q4_0_quantize(w)
    for r in range(16):
        for b in range(4):
            blk = w[r, 32 * b:32 * b + 32]
            j = int(np.argmax(np.abs(blk)))                   # first index on ties
            m = blk[j]
            want_d = np.array([_f32(m) / _f32(-8)], np.float32).astype(np.float16).view(np.uint16)[0]
            assert sc[r * 4 + b] == want_d
            delta = np.uint16(want_d).view(np.float16).astype(np.float32)
            assert codes[r, 32 * b + j] == 0                   # the extreme maps to -8
            for i in range(32):
                qb = _q_brute(blk[i], delta, -8, 7) + 8
                qi = int(codes[r, 32 * b + i])
                if qi != qb:
                    t = Fraction(float(blk[i])) / Fraction(float(delta))
                    assert abs(abs(t - (qi - 8)) - Fraction(1, 2)) < Fraction(1, 2 ** 18)


def test_q4_0_extreme_exact_negative_zero_and_ties(orc):
    w = np.zeros((16, 128), np.float32)
    w[0, :32] = np.linspace(-0.5, 0.5, 32, dtype=np.float32)
    w[0, 3] = 0.75                     # m = 0.75 -> d = -0.09375 (fp16 exact)
    w[0, 4] = 0.0
    w[1, 32:64] = 0.25
    w[1, 40] = -0.5
    w[1, 41] = 0.5                     # tie in |w|: the first (negative) one wins
    codes, sc = orc.q4_0_quantize(w)
    w_hat = orc.q4_0_dequantize(codes, sc)
    assert w_hat[0, 3] == np.float32(0.75) and codes[0, 3] == 0
    assert w_hat[0, 4] == 0 and np.signbit(w_hat[0, 4])       # (8-8) * negative delta = -0.0
    d1 = np.uint16(sc[1 * 4 + 1]).view(np.float16).astype(np.float32)
    assert d1 == np.float32(0.0625)                            # -0.5 / -8
    assert codes[1, 40] == 0 and w_hat[1, 40] == -0.5
    assert codes[1, 41] == 15 and w_hat[1, 41] == np.float32(7 * 0.0625)
    # an all-zero block: delta = 0, every code 8
    assert np.all(codes[2] == 8) and np.all(w_hat[2] == 0)


# ----------------------------------------------------------------- q4_1 ----
# q4_1 is only named ("Run quantized Whisper on the fused Metal decode path",
# "Why the policy"); the reading: d = fp16((max - min) / 15), m = fp16(min),
# codes = the nearest of the 16 levels q*d + m, chosen against the stored fp16
# values, w^ = q*d + m.

def _f16(x):
    return np.array([x], np.float32).astype(np.float16)


def test_q4_1_brute_force(orc):
    """Scales follow from the block's extremes; every code is the nearest level
    found by exhaustive search in exact arithmetic (near-ties excepted)."""
    rng = np.random.default_rng(15)
    w = (rng.standard_normal((16, 128)) * 0.02).astype(np.float32)
    w[3, 40] = 0.1                                         # an outlier in one block
    codes, sc = orc.q4_1_quantize(w)
    assert codes.max() <= 15
    for r in range(16):
        for b in range(4):
            blk = w[r, 32 * b:32 * b + 32]
            lo, hi = blk.min(), blk.max()
            want_d = _f16(_f32(_f32(hi - lo) / _f32(15))).view(np.uint16)[0]
            want_m = _f16(lo).view(np.uint16)[0]
            assert sc[r * 4 + b, 0] == want_d and sc[r * 4 + b, 1] == want_m
            delta = Fraction(float(np.uint16(want_d).view(np.float16)))
            mu = Fraction(float(np.uint16(want_m).view(np.float16)))
            for i in range(32):
                t = Fraction(float(blk[i]))
                dist = [abs(t - (q * delta + mu)) for q in range(16)]
                qb = dist.index(min(dist))
                qi = int(codes[r, 32 * b + i])
                if qi != qb:                                   # only a near-tie may differ
                    assert abs(dist[qi] - dist[qb]) <= delta / 2 ** 16


def test_q4_1_round_trip_constant_blocks_and_positions(orc):
    w = np.zeros((16, 128), np.float32)
    # block of exactly representable levels: m = -0.25, d = 0.03125 (both fp16-exact, (hi - lo) / 15 exact)
    q = np.arange(32) % 16
    w[0, :32] = (np.float32(-0.25) + q.astype(np.float32) * np.float32(0.03125)).astype(np.float32)
    w[1, 32:64] = np.float32(0.375)                        # constant block: d = 0, codes 0, w^ = m
    w[2, 64:96] = np.float32(-1.5)
    codes, sc = orc.q4_1_quantize(w)
    w_hat = orc.q4_1_dequantize(codes, sc)
    assert np.array_equal(codes[0, :32], q) and np.array_equal(w_hat[0, :32], w[0, :32])
    assert sc[1 * 4 + 1, 0] == 0 and np.all(codes[1, 32:64] == 0) and np.all(w_hat[1, 32:64] == np.float32(0.375))
    assert np.all(w_hat[2, 64:96] == np.float32(-1.5))
    # an all-zero block: d = 0, m = +0, w^ = 0
    assert np.all(codes[3] == 0) and np.all(w_hat[3] == 0)
    # packed scales: block b of row r at byte 256 * tile + 16 * (r % 16) + 4 * (b % 4), d first
    res = orc.quantize(5, w)
    sp = res["scales"].view(np.uint16)
    for r, b in [(0, 0), (1, 1), (2, 2), (15, 3)]:
        off = (256 * (b // 4) + 16 * r + 4 * (b % 4)) // 2
        assert sp[off] == sc[r * 4 + b, 0] and sp[off + 1] == sc[r * 4 + b, 1]
    assert np.array_equal(res["w_hat"], w_hat)
    # 0.625 bytes per weight: 4-bit codes plus two fp16 per 32 values
    assert orc.packed_size(5, False, 16, 128) == (1024, 256)


def test_q4_1_error_bound(orc):
    """Every w^ lies within half a level (plus the fp16 rounding of the minimum)
    of w, and the block minimum decodes to m exactly."""
    rng = np.random.default_rng(16)
    w = (rng.standard_normal((32, 256)) * 0.02).astype(np.float32)
    codes, sc = orc.q4_1_quantize(w)
    w_hat = orc.q4_1_dequantize(codes, sc)
    for r in range(32):
        for b in range(8):
            blk = w[r, 32 * b:32 * b + 32]
            d = float(np.uint16(sc[r * 8 + b, 0]).view(np.float16))
            m = float(np.uint16(sc[r * 8 + b, 1]).view(np.float16))
            err = np.abs(w_hat[r, 32 * b:32 * b + 32].astype(np.float64) - blk)
            assert err.max() <= d / 2 + abs(m - float(blk.min())) + 1e-9
            j = int(np.argmin(blk))
            assert codes[r, 32 * b + j] == 0 and w_hat[r, 32 * b + j] == np.float32(m)


# ----------------------------------------------------------------- q5_0 ----
# q5_0 is only named ("Run quantized Whisper on the fused Metal decode path",
# "Why the policy"); the reading: as q4_0 with 5-bit codes, d = fp16(m / -16),
# q = clamp(rint(w / d), -16, 15) + 16, w^ = (q - 16) d.

def test_q5_0_brute_force(orc):
    rng = np.random.default_rng(17)
    w = (rng.standard_normal((16, 128)) * 0.02).astype(np.float32)
    codes, sc = orc.q5_0_quantize(w)
    assert codes.max() <= 31
    for r in range(16):
        for b in range(4):
            blk = w[r, 32 * b:32 * b + 32]
            j = int(np.argmax(np.abs(blk)))                   # first index on ties
            want_d = _f16(_f32(blk[j]) / _f32(-16)).view(np.uint16)[0]
            assert sc[r * 4 + b] == want_d
            delta = np.uint16(want_d).view(np.float16).astype(np.float32)
            assert codes[r, 32 * b + j] == 0                   # the extreme maps to -16
            for i in range(32):
                qb = _q_brute(blk[i], delta, -16, 15) + 16
                qi = int(codes[r, 32 * b + i])
                if qi != qb:
                    t = Fraction(float(blk[i])) / Fraction(float(delta))
                    assert abs(abs(t - (qi - 16)) - Fraction(1, 2)) < Fraction(1, 2 ** 18)


def test_q5_0_extreme_exact_zero_block_and_packing(orc):
    w = np.zeros((16, 128), np.float32)
    w[0, :32] = np.linspace(-0.5, 0.5, 32, dtype=np.float32)
    w[0, 5] = 0.75                     # m = 0.75 -> d = -0.046875 (fp16 exact)
    w[0, 6] = 0.0
    w[1, 32:64] = (np.arange(32, dtype=np.float32) - 16) * np.float32(0.125)   # -2 .. 1.875: exact levels
    codes, sc = orc.q5_0_quantize(w)
    w_hat = orc.q5_0_dequantize(codes, sc)
    assert w_hat[0, 5] == np.float32(0.75) and codes[0, 5] == 0
    assert w_hat[0, 6] == 0 and np.signbit(w_hat[0, 6])       # (16-16) * negative delta = -0.0
    assert np.array_equal(w_hat[1, 32:64], w[1, 32:64])         # m = -2 -> d = 0.125, every level exact
    assert np.array_equal(codes[1, 32:64], np.arange(32))
    assert np.all(codes[2] == 16) and np.all(w_hat[2] == 0)     # all-zero block
    # packed: low nibbles in the 4-bit tiles, bit 4 of each code in the block's 32-bit word
    res = orc.quantize(6, w)
    assert orc.packed_size(6, False, 16, 128) == (1024, 128 + 256)
    assert np.array_equal(orc.unpack_codes4(res["codes"], 16, 128), codes & 15)
    hb = res["scales"][128:].view(np.uint32)
    for r in range(16):
        for b in range(4):
            word = int(hb[r * 4 + b])                           # one tile: slot = 4 r + b
            want = sum(1 << i for i in range(32) if codes[r, 32 * b + i] & 16)
            assert word == want
    assert np.array_equal(res["scales"][:128].view(np.uint16), sc.reshape(16, 4).reshape(-1))


# ----------------------------------------------------------------- q4_k ----
# q4_k is only named ("Run quantized Whisper on the fused Metal decode path",
# "Why the policy"); the reading: per 32-value sub-block a scale (range / 15) and
# an offset (-min when the minimum is negative), both as 6-bit multiples of the
# 256-value super-block's fp16 d = max scale / 63 and dmin = max offset / 63;
# codes = nearest of the 16 levels q*S - O.

def _q4_k_scales(blk256):
    """The scale derivation written out with numpy float32 operations."""
    s, o = [], []
    for j in range(8):
        sb = blk256[32 * j:32 * j + 32]
        lo, hi = sb.min(), sb.max()
        mn = lo if lo < 0 else np.float32(0)
        r = _f32(hi - mn)
        r = r if r > 0 else np.float32(0)
        s.append(_f32(r / _f32(15)))
        o.append(_f32(np.float32(0) - mn))
    d = _f16(_f32(max(s) / _f32(63)))
    dm = _f16(_f32(max(o) / _f32(63)))
    df, dmf = np.float32(d[0]), np.float32(dm[0])
    sc = [0 if df == 0 else int(min(max(np.rint(_f32(sj / df)), 0), 63)) for sj in s]
    m = [0 if dmf == 0 else int(min(max(np.rint(_f32(oj / dmf)), 0), 63)) for oj in o]
    return d.view(np.uint16)[0], dm.view(np.uint16)[0], sc, m


def test_q4_k_scales_and_brute_force(orc):
    rng = np.random.default_rng(18)
    w = (rng.standard_normal((16, 512)) * 0.02).astype(np.float32)
    w[2, 256:288] = np.abs(w[2, 256:288])                 # a non-negative sub-block: offset 0
    w[5, 300] = 0.2                                       # an outlier sets d for its super-block
    codes, sub, dd = orc.q4_k_quantize(w)
    assert codes.max() <= 15 and sub.max() <= 63
    for r in range(16):
        for b in range(2):
            d, dm, sc, m = _q4_k_scales(w[r, 256 * b:256 * b + 256])
            assert dd[r * 2 + b, 0] == d and dd[r * 2 + b, 1] == dm
            df = Fraction(float(np.uint16(d).view(np.float16)))
            dmf = Fraction(float(np.uint16(dm).view(np.float16)))
            for j in range(8):
                assert sub[(r * 16 + b * 8 + j), 0] == sc[j] and sub[(r * 16 + b * 8 + j), 1] == m[j]
                S, O = df * sc[j], dmf * m[j]
                if S == 0:
                    assert np.all(codes[r, 256 * b + 32 * j:256 * b + 32 * j + 32] == 0)
                    continue
                for i in range(32):
                    t = Fraction(float(w[r, 256 * b + 32 * j + i]))
                    dist = [abs(t - (q * S - O)) for q in range(16)]
                    qb = dist.index(min(dist))
                    qi = int(codes[r, 256 * b + 32 * j + i])
                    if qi != qb:                                # only a near-tie may differ
                        assert abs(dist[qi] - dist[qb]) <= S / 2 ** 16
    assert np.all(sub[(2 * 16 + 8), 1] == 0)                     # the non-negative sub-block has no offset


def test_q4_k_zero_superblock_dequant_and_packing(orc):
    rng = np.random.default_rng(19)
    w = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    w[3] = 0.0
    w[4] = -0.0
    codes, sub, dd = orc.q4_k_quantize(w)
    w_hat = orc.q4_k_dequantize(codes, sub, dd)
    for r in (3, 4):
        assert dd[r, 0] == 0 and dd[r, 1] == 0 and np.all(codes[r] == 0) and np.all(w_hat[r] == 0)
    # w^ = S q - O with S = d sc and O = dmin m, one rounding (S q is exact)
    r, j = 0, 5
    S = np.float32(np.uint16(dd[r, 0]).view(np.float16)) * np.float32(sub[r * 8 + j, 0])
    O = np.float32(np.uint16(dd[r, 1]).view(np.float16)) * np.float32(sub[r * 8 + j, 1])
    want = (S * codes[r, 32 * j:32 * j + 32].astype(np.float32)).astype(np.float32) - O
    assert np.array_equal(w_hat[r, 32 * j:32 * j + 32], want.astype(np.float32))
    # packed: per tile and row 8 bytes (the 4 sub-blocks' sc, then m), then the (d, dmin) plane
    res = orc.quantize(7, w)
    assert orc.packed_size(7, False, 16, 256) == (2048, 256 + 64)
    sp = res["scales"]
    for r, b in [(0, 0), (1, 5), (15, 7)]:
        off = 128 * (b // 4) + 8 * r + (b % 4)
        assert sp[off] == sub[r * 8 + b, 0] and sp[off + 4] == sub[r * 8 + b, 1]
    ddp = sp[256:].view(np.uint16).reshape(16, 2)
    assert np.array_equal(ddp, dd)
    assert np.array_equal(res["w_hat"], w_hat)


# ----------------------------------------------------------------- q6_k ----
# q6_k is only named ("Run quantized Whisper on the fused Metal decode path",
# "Why the policy"); the reading: per 16-value sub-block s = (signed extreme) / -32,
# d = fp16(max |s| / 127), int8 sc = rint(s / d), S = d*sc, 6-bit codes
# q = clamp(rint(w / S), -32, 31) + 32, w^ = S*(q - 32).

def test_q6_k_scales_and_brute_force(orc):
    rng = np.random.default_rng(20)
    w = (rng.standard_normal((16, 512)) * 0.02).astype(np.float32)
    w[4, 100] = -0.3                                      # an outlier sets d for its super-block
    codes, sc, d = orc.q6_k_quantize(w)
    assert codes.max() <= 63
    for r in range(16):
        for b in range(2):
            blk = w[r, 256 * b:256 * b + 256]
            s = []
            for j in range(16):
                sb = blk[16 * j:16 * j + 16]
                jj = int(np.argmax(np.abs(sb)))            # first index on ties
                s.append(_f32(sb[jj] / _f32(-32)))
            want_d = _f16(_f32(max(abs(x) for x in s) / _f32(127))).view(np.uint16)[0]
            assert d[r * 2 + b] == want_d
            df = np.float32(np.uint16(want_d).view(np.float16))
            for j in range(16):
                want_sc = 0 if df == 0 else int(min(max(np.rint(_f32(s[j] / df)), -127), 127))
                assert sc[r * 32 + b * 16 + j] == want_sc
                S = Fraction(float(df)) * want_sc
                seg = slice(256 * b + 16 * j, 256 * b + 16 * j + 16)
                if S == 0:
                    assert np.all(codes[r, seg] == 32)
                    continue
                for i in range(16):
                    t = Fraction(float(w[r, 256 * b + 16 * j + i]))
                    dist = [abs(t - (q - 32) * S) for q in range(64)]
                    qb = dist.index(min(dist))
                    qi = int(codes[r, 256 * b + 16 * j + i])
                    if qi != qb:                                      # only a near-tie may differ
                        assert abs(dist[qi] - dist[qb]) <= abs(S) / 2 ** 16


def test_q6_k_zero_superblock_exact_levels_and_packing(orc):
    w = np.zeros((16, 256), np.float32)
    rng = np.random.default_rng(21)
    w[1] = (rng.standard_normal(256) * 0.02).astype(np.float32)
    codes, sc, d = orc.q6_k_quantize(w)
    w_hat = orc.q6_k_dequantize(codes, sc, d)
    assert d[0] == 0 and np.all(codes[0] == 32) and np.all(w_hat[0] == 0)       # all-zero super-block
    S = np.float32(np.uint16(d[1]).view(np.float16)) * np.float32(sc[16 + 3])
    want = (S * (codes[1, 48:64].astype(np.float32) - np.float32(32))).astype(np.float32)
    assert np.array_equal(w_hat[1, 48:64], want)
    res = orc.quantize(8, w)
    assert orc.packed_size(8, False, 16, 256) == (2048 + 1024, 256 + 32)
    cp = res["codes"]
    assert np.array_equal(orc.unpack_codes4(cp[:2048], 16, 256), codes & 15)
    high = cp[2048:]
    for r, kk in [(1, 0), (1, 77), (1, 255), (5, 130)]:
        kin, tile = kk % 128, kk // 128
        j, h, i = kin // 32, (kin % 32) // 8, kin % 8
        base = tile * 512 + (h * 16 + r) * 8 + 2 * j
        assert (high[base] >> i) & 1 == (codes[r, kk] >> 4) & 1
        assert (high[base + 1] >> i) & 1 == (codes[r, kk] >> 5) & 1
    sp = res["scales"]
    for r, t in [(1, 0), (1, 9), (15, 15)]:
        assert sp[(t // 8) * 128 + r * 8 + t % 8].astype(np.int8) == sc[r * 16 + t]
    assert np.array_equal(sp[256:].view(np.uint16), d)
    assert np.array_equal(res["w_hat"], w_hat)
