"""Pins for the packed layout (hand-derived positions, permutation) and for the
packed-size formulas (against model sizes the pages print)."""
import json
import os

import numpy as np

NF4, NVFP4, Q4_0, Q8_0 = 1, 2, 3, 4
HERE = os.path.dirname(os.path.abspath(__file__))


def _golden_layout():
    rows = []
    with open(os.path.join(HERE, "golden", "layout_positions.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_layout_positions_match_hand_derivation(orc):
    for row in _golden_layout():
        kind = row[0]
        if kind == "codes4":
            n, k, r, kk, byte, nib = map(int, row[1:7])
            codes = np.zeros((n, k), np.uint8)
            codes[r, kk] = 0xA
            packed = orc.pack_codes4(codes)
            nz = np.flatnonzero(packed)
            assert list(nz) == [byte], row
            assert packed[byte] == (0xA0 if nib else 0x0A), row
        elif kind == "codes8":
            n, k, r, kk, byte = map(int, row[1:6])
            codes = np.zeros((n, k), np.int8)
            codes[r, kk] = -5
            packed = orc.pack_codes8(codes)
            assert list(np.flatnonzero(packed)) == [byte], row
            assert packed[byte] == -5
        else:
            n, k, bs, ptk, r, b, idx = map(int, row[1:8])
            logical = np.zeros((n, k // bs), np.float32)
            logical[r, b] = 1.0
            packed = orc.pack_scales(n, k, bs, ptk, logical)
            assert list(np.flatnonzero(packed)) == [idx], row


def test_layout_is_a_permutation(orc):
    rng = np.random.default_rng(0)
    for n, k in ((16, 128), (48, 384), (32, 1280)):
        codes = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
        packed = orc.pack_codes4(codes)
        assert packed.size == n * k // 2
        assert np.array_equal(orc.unpack_codes4(packed, n, k), codes)
        full = orc.pack_codes4(np.full((n, k), 15, np.uint8))
        assert np.all(full == 0xFF)                      # every nibble written exactly once
        ids = (np.arange(n * k) % 251).astype(np.int8).reshape(n, k)
        p8 = orc.pack_codes8(ids)
        assert np.array_equal(np.sort(p8.view(np.uint8)), np.sort(ids.reshape(-1).view(np.uint8)))
    # scales: a permutation of the logical order
    logical = np.arange(48 * 384 // 16, dtype=np.float32).reshape(48, -1)
    p = orc.pack_scales(48, 384, 16, 128, logical)
    assert np.array_equal(np.sort(p), np.sort(logical.reshape(-1)))


def test_bytes_per_weight(orc):
    n, k = 5120, 1280
    want = {(NF4, False): 0.5625, (NVFP4, False): 0.5625, (Q4_0, False): 0.5625, (Q8_0, False): 1.0625}
    for (fmt, dq), bpw in want.items():
        cb, sb = orc.packed_size(fmt, dq, n, k)
        assert abs((cb + sb) / (n * k) - bpw) < 1e-5
    cb, sb = orc.packed_size(NF4, True, n, k)
    assert abs((cb + sb) / (n * k) - (0.5 + 1 / 64 + 4 / (64 * 256))) < 1e-5


# ----------------------------------------------- sizes printed on the pages ----

def _whisper_linears(d, ffn, n_enc, n_dec):
    enc = [(d, d)] * 4 + [(ffn, d), (d, ffn)]
    dec = [(d, d)] * 8 + [(ffn, d), (d, ffn)]
    return enc * n_enc, dec * n_dec


def _packed_total(orc, fmt, dq, shapes):
    tot = 0
    for n, k in shapes:
        cb, sb = orc.packed_size(fmt, dq, n, k)
        tot += cb + sb
    return tot


def test_whisper_sizes_printed_on_pages(orc):
    g = json.load(open(os.path.join(HERE, "golden", "page_sizes.json")))
    d = g["d_model"]["value"]
    enc, dec = _whisper_linears(d, 4 * d, 32, 4)
    assert len(enc) == g["encoder_linears"]["value"] and len(dec) == g["decoder_linears"]["value"]
    lin = sum(n * k for n, k in enc + dec)
    # whole-model parameter count from the fp16 (2 bytes/param) sizes on two pages
    p_gib = g["fp16_disk_GiB"]["value"] * 2 ** 30 / 2
    p_gb = g["bf16_weights_GB"]["value"] * 1e9 / 2
    assert abs(p_gib - p_gb) / p_gb < 0.01
    rest = p_gb - lin                              # embeddings, convs, norms, biases: bf16

    nf4dq = (_packed_total(orc, NF4, True, enc + dec) + 2 * rest) / 1e9
    nf4 = (_packed_total(orc, NF4, False, enc + dec) + 2 * rest) / 1e9
    want = g["nf4_weights_GB"]["value"]
    assert abs(nf4dq - want) / want < 0.015               # double-quant fits the page ...
    assert abs(nf4 - want) / want > 0.05                  # ... single-level absmax does not

    nvfp4 = (_packed_total(orc, NVFP4, False, enc + dec) + 2 * rest) / 2 ** 30
    assert round(nvfp4, 2) == g["nvfp4_disk_GiB"]["value"]

    # GGUF bundles: encoder stays q8_0, decoder layers take the requested format, so the
    # q8_0 - q4_0 size difference is the decoder Linears' byte difference.
    for name, dm, n_layers in (("large_v3_turbo", 1280, (32, 4)), ("small", 768, (12, 12))):
        e, dl = _whisper_linears(dm, 4 * dm, *n_layers)
        diff = (_packed_total(orc, Q8_0, False, dl) - _packed_total(orc, Q4_0, False, dl)) / 2 ** 20
        page = g[f"gguf_{name}_q8_0_MB"]["value"] - g[f"gguf_{name}_q4_0_MB"]["value"]
        assert abs(diff - page) <= 1.0, (name, diff, page)
