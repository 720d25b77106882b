"""The NF4 constants compiled into the HIP library (csrc/nf4_table.h) against the oracle's own
construction of the codebook ("asr: add a 4-bit nf4 option for the Whisper engine", intro and
section "What's here": NF4 levels).

  * the 16 fp32 levels are the oracle's levels, bit for bit;
  * each of the 15 fp32 thresholds decides "above the midpoint" exactly as the oracle's binary64
    midpoint does for every fp32 input: it is the largest float32 not above the midpoint;
  * the 16 bf16 images are the levels rounded to nearest even.
"""
import os
import re

import numpy as np

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "block_quantized_bit_amd", "csrc", "nf4_table.h")


def _array(name):
    txt = open(HEADER).read()
    body = re.search(name + r"\[\d+\]\s*=\s*\{(.*?)\};", txt, re.S).group(1)
    return [int(v, 16) for v in re.findall(r"0x([0-9a-fA-F]+)u?", body)]


def test_levels_equal_the_oracle_codebook(orc):
    c, _ = orc.nf4_codebook()
    lv = np.array(_array("kNf4LevelBits"), np.uint32)
    assert lv.size == 16
    assert np.array_equal(lv, c.view(np.uint32))


def test_thresholds_decide_like_the_binary64_midpoints(orc):
    _, mid = orc.nf4_codebook()
    th = np.array(_array("kNf4ThresholdBits"), np.uint32).view(np.float32)
    assert th.size == 15
    for t, m in zip(th, mid):
        up = np.nextafter(t, np.float32(np.inf), dtype=np.float32)
        assert float(t) <= m < float(up), (t, m)


def test_bf16_images_round_the_levels_to_nearest_even(orc):
    c, _ = orc.nf4_codebook()
    u = c.view(np.uint32).astype(np.uint64)
    rne = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(np.array(_array("kNf4LevelBf16"), np.uint16), rne)
