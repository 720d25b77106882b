"""Pins for the oracle's scalar codecs and the NF4 codebook.

Each check compares the oracle with something other than itself: numpy's
binary16, torch's float8_e4m3fn, an independent binade-rounding formula for
E2M1, scipy / stdlib inverse normal CDFs for NF4, and the E2M1 value list.
"""
import os
import statistics

import numpy as np
import pytest
import torch
from scipy.stats import norm

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------- fp16 ----

def test_fp16_decode_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([orc.fp16_decode(int(b)) for b in bits], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_fp16_encode_representable_and_midpoints(orc):
    bits = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)   # +0 .. 65504
    vals = bits.view(np.float16).astype(np.float32)
    for b, v in zip(bits, vals):
        assert orc.fp16_encode(float(v)) == int(b)
        assert orc.fp16_encode(float(-v)) == int(b) | 0x8000
    # midpoints between neighbours are exact in float32; numpy rounds half to even
    mids = ((vals[:-1].astype(np.float64) + vals[1:].astype(np.float64)) / 2).astype(np.float32)
    ref = mids.astype(np.float16).view(np.uint16)
    got = np.array([orc.fp16_encode(float(m)) for m in mids], np.uint16)
    assert np.array_equal(got, ref)


def test_fp16_encode_random_and_saturation(orc):
    rng = np.random.default_rng(7)
    x = (rng.uniform(-1, 1, 20000) * np.exp2(rng.uniform(-30, 18, 20000))).astype(np.float32)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16)
    refb = ref.view(np.uint16).copy()
    inf = np.isinf(ref)
    refb[inf] = np.where(x[inf] > 0, 0x7BFF, 0xFBFF)          # saturating reading
    got = np.array([orc.fp16_encode(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, refb)
    assert orc.fp16_encode(1e30) == 0x7BFF and orc.fp16_encode(-1e30) == 0xFBFF


# ---------------------------------------------------------------- E4M3 ----

def _torch_e4m3_decode_all():
    a = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return a.view(torch.float8_e4m3fn).to(torch.float32).numpy()


def test_e4m3_decode_all_patterns_match_torch(orc):
    ref = _torch_e4m3_decode_all()
    got = np.array([orc.e4m3_decode(b) for b in range(256)], np.float32)
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_e4m3_encode_matches_torch_in_range(orc):
    ref_vals = _torch_e4m3_decode_all()[:0x7F]                 # non-negative finite
    rng = np.random.default_rng(11)
    mids = ((ref_vals[:-1].astype(np.float64) + ref_vals[1:]) / 2).astype(np.float32)
    rnd = (np.exp2(rng.uniform(-12, 8.8, 5000))).astype(np.float32)
    xs = np.concatenate([ref_vals, mids, rnd[rnd <= 448]])
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(v)) for v in xs], np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates_never_nan(orc):
    for v in (448.0, 449.0, 463.9, 464.0, 500.0, 1e6, float("inf")):
        assert orc.e4m3_encode(v) == 0x7E


# ---------------------------------------------------------------- E2M1 ----

def _golden_e2m1():
    vals = []
    with open(os.path.join(HERE, "golden", "e2m1_magnitudes.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                vals.append(float(v))
    return np.array(vals)


def test_e2m1_decode_all_codes(orc):
    mags = _golden_e2m1()
    for c in range(16):
        v = orc.e2m1_decode(c)
        assert abs(v) == mags[c & 7]
        assert np.signbit(v) == bool(c & 8)


def _e2m1_rne_by_binade(a):
    """Independent statement of round-to-nearest-even on the E2M1 grid:
    spacing 0.5 below 2, 1 in [2, 4), 2 in [4, 6]; saturate at 6."""
    a = np.asarray(a, np.float64)
    out = np.where(a < 2, np.round(a / 0.5) * 0.5,
                   np.where(a < 4, np.round(a), np.round(a / 2) * 2))
    return np.minimum(out, 6.0)


def test_e2m1_encode_ties_and_grid(orc):
    mags = _golden_e2m1()
    grid = np.unique(np.concatenate([
        mags, (mags[:-1] + mags[1:]) / 2, np.linspace(0, 7, 561),
        np.nextafter((mags[:-1] + mags[1:]) / 2, 0), np.nextafter((mags[:-1] + mags[1:]) / 2, 10)]))
    grid = grid.astype(np.float32)
    want = _e2m1_rne_by_binade(grid)
    for x, w in zip(grid, want):
        for s in (1.0, -1.0):
            c = orc.e2m1_encode(float(s * x))
            assert mags[c & 7] == w, (x, c)
            assert bool(c & 8) == (s < 0)
    # the ties listed as the reading: 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4
    for x, w in ((0.25, 0), (0.75, 1), (1.25, 1), (1.75, 2), (2.5, 2), (3.5, 4), (5, 4), (9, 6)):
        assert mags[orc.e2m1_encode(x) & 7] == w


# ---------------------------------------------------------------- NF4 -----

def _nf4_from(ppf):
    delta = 0.5 * ((1 - 1 / 30) + (1 - 1 / 32))
    pos = [ppf(p) for p in np.linspace(delta, 0.5, 9)[:-1]]
    neg = [-ppf(p) for p in np.linspace(delta, 0.5, 8)[:-1]]
    v = np.sort(np.array(pos + neg + [0.0]))
    return (v / v.max()).astype(np.float32)


def test_nf4_codebook_matches_two_library_routines(orc):
    c, mid = orc.nf4_codebook()
    by_scipy = _nf4_from(norm.ppf)
    by_stdlib = _nf4_from(statistics.NormalDist().inv_cdf)
    assert np.array_equal(c.view(np.uint32), by_scipy.view(np.uint32))
    assert np.array_equal(c.view(np.uint32), by_stdlib.view(np.uint32))


def test_nf4_codebook_invariants(orc):
    c, mid = orc.nf4_codebook()
    assert c.shape == (16,)
    assert np.all(np.diff(c.astype(np.float64)) > 0)
    assert c[0] == -1.0 and c[15] == 1.0 and c[7] == 0.0
    assert (c < 0).sum() == 7 and (c > 0).sum() == 8
    # midpoints are exact binary64 averages of neighbouring binary32 levels
    assert np.array_equal(mid, (c[:-1].astype(np.float64) + c[1:]) / 2)
    # shape of the NormalFloat levels (QLoRA): quantiles of N(0,1), so spacing
    # grows toward the tails on both sides
    gaps = np.diff(c.astype(np.float64))
    assert np.all(np.diff(gaps[7:]) > 0) and np.all(np.diff(gaps[:7]) < 0)
