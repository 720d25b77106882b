"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, agrees with the oracle on packed sizes, and rejects bad
arguments on the host before anything is enqueued."""
import os
import re

import pytest

from block_quantized_bit_amd import wq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wq.h")
NF4, NVFP4, Q4_0, Q8_0, Q4_1, Q5_0, Q4_K, Q6_K = 1, 2, 3, 4, 5, 6, 7, 8


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(wq_[a-z0-9_]+)\s*\(", txt)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(wq.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = wq.lib()
    for name in _declared():
        assert hasattr(L, name), name
    out = os.popen(f"nm -D --defined-only {wq.LIB_PATH}").read()
    exported = set(re.findall(r" T (wq_[a-z0-9_]+)", out))
    assert set(_declared()) <= exported


def test_status_strings():
    for s, name in wq.STATUS_NAMES.items():
        assert wq.wq_status_str(s) == name


SHAPES = [(16, 128), (48, 384), (272, 640), (1536, 384), (3840, 1280), (1280, 5120)]


@pytest.mark.parametrize("fmt,dq", [(NF4, False), (NF4, True), (NVFP4, False), (Q4_0, False), (Q8_0, False),
                                    (Q4_1, False), (Q5_0, False), (Q4_K, False), (Q6_K, False)])
def test_packed_size_matches_oracle(orc, fmt, dq):
    for n, k in SHAPES:
        if fmt in (Q4_K, Q6_K) and k % 256:
            continue                                   # q4_k and q6_k need whole 256-value super-blocks
        assert wq.wq_packed_size(wq.desc(fmt, n, k, dq)) == orc.packed_size(fmt, dq, n, k)
    # q8_0 also accepts K % 64 == 0
    if fmt == Q8_0:
        assert wq.wq_packed_size(wq.desc(fmt, 32, 192)) == orc.packed_size(fmt, False, 32, 192)


def _status(fn, *a):
    try:
        fn(*a)
    except wq.WqError as e:
        return e.status
    return 0


def test_descriptor_validation():
    bad = [
        (wq.wq_desc(9, 0, 16, 128, 0, 0), 1),           # unknown format
        (wq.wq_desc(NF4, 32, 16, 128, 0, 0), 2),        # NF4 block must be 64
        (wq.wq_desc(NVFP4, 0, 16, 128, 256, 0), 2),     # double-quant only for NF4
        (wq.wq_desc(NF4, 0, 16, 128, 128, 0), 2),       # group must be 256
        (wq.wq_desc(NF4, 0, 24, 128, 0, 0), 3),         # n % 16
        (wq.wq_desc(Q4_0, 0, 16, 64, 0, 0), 3),         # k % 128 for 4-bit
        (wq.wq_desc(Q4_1, 0, 16, 64, 0, 0), 3),         # k % 128 for q4_1 too
        (wq.wq_desc(Q4_1, 16, 16, 128, 0, 0), 2),       # q4_1 blocks are 32
        (wq.wq_desc(Q4_1, 0, 16, 128, 256, 0), 2),      # double-quant only for NF4
        (wq.wq_desc(Q5_0, 0, 16, 64, 0, 0), 3),         # k % 128 for q5_0
        (wq.wq_desc(Q5_0, 0, 16, 128, 256, 0), 2),      # double-quant only for NF4
        (wq.wq_desc(Q4_K, 0, 16, 384, 0, 0), 3),        # k % 256 for q4_k (super-blocks)
        (wq.wq_desc(Q4_K, 32, 16, 256, 0, 0), 2),       # its block is the 256-value super-block
        (wq.wq_desc(Q6_K, 0, 16, 640, 0, 0), 3),        # k % 256 for q6_k
        (wq.wq_desc(9, 0, 16, 128, 0, 0), 1),           # past the last format
        (wq.wq_desc(Q8_0, 0, 16, 96, 0, 0), 3),         # k % 64 for q8_0
        (wq.wq_desc(Q8_0, 0, 0, 64, 0, 0), 3),          # n > 0
        (wq.wq_desc(NF4, 0, 16, 128, 0, 7), 1),         # reserved
        (wq.wq_desc(NF4, 0, 16, (1 << 24) + 128, 0, 0), 3),   # k beyond one band's 32-bit buffer range
        (wq.wq_desc(NF4, 0, 1 << 20, 1 << 21, 0, 0), 3),      # n * k beyond 2^40
    ]
    for d, want in bad:
        assert _status(wq.wq_packed_size, d) == want
        assert _status(wq.wq_workspace_size, d, 4) == want


FAKE = 1 << 20   # a 16-aligned non-NULL address; every call below must fail before use


def test_matmul_argument_validation_returns_before_launch():
    d = wq.desc(NF4, 64, 256)
    mm = lambda **kw: _status(wq.wq_matmul, kw.get("d", d), kw.get("m", 4), kw.get("x", FAKE),
                              kw.get("ldx", 256), kw.get("codes", FAKE), kw.get("scales", FAKE),
                              kw.get("bias", None), kw.get("y", FAKE), kw.get("ydt", wq.WQ_F32),
                              kw.get("ldy", 64), kw.get("ws", None), kw.get("ws_bytes", 0), 0)
    assert mm(m=-1) == 3
    assert mm(x=None) == 1
    assert mm(x=FAKE + 8) == 4
    assert mm(ldx=200) == 1
    assert mm(ldx=260) == 1             # ldx % 8
    assert mm(ldx=(1 << 24) + 8) == 1   # 128 rows of X must stay within one 32-bit buffer range
    assert mm(codes=None) == 1
    assert mm(scales=FAKE + 4) == 4
    assert mm(bias=FAKE + 1) == 4
    assert mm(y=None) == 1
    assert mm(y=FAKE + 2) == 4          # fp32 output needs 4-byte alignment
    assert mm(ydt=3) == 1
    assert mm(ldy=32) == 1
    assert mm(ldy=1 << 31) == 1         # output strides and columns travel as 32-bit kernel arguments
    big = wq.desc(NF4, (1 << 31) + 16, 128)
    assert _status(wq.wq_packed_size, big) == 0                   # a valid weight ...
    assert mm(d=big, ldx=128, ldy=(1 << 31) + 16) == 3             # ... too wide for a matmul
    assert mm(ws=FAKE + 8) == 4
    assert mm(d=wq.desc(NF4, 24, 256)) == 3
    # a workspace smaller than asked for is an error (only checked when a split is wanted)
    dd = wq.desc(NF4, 1280, 5120)
    assert wq.wq_workspace_size(dd, 1) == 0          # decode GEMV never splits across workgroups
    need = wq.wq_workspace_size(dd, 20)              # 10 output tiles, 40 K steps: the GEMM splits K
    assert need > 0
    assert mm(d=dd, m=20, ldx=5120, ldy=1280, ws=FAKE, ws_bytes=need - 1) == 6
    # m == 0 is a no-op: validated, nothing enqueued
    assert mm(m=0) == 0


def test_qkv_argument_validation():
    d = wq.desc(NF4, 96, 256)
    def q(split, ys=None, ldys=None, **kw):
        ys = ys if ys is not None else [FAKE] * len(split)
        ldys = ldys if ldys is not None else [max(s, 1) for s in split]
        return _status(wq.wq_matmul_qkv, kw.get("d", d), 2, FAKE, 256, FAKE, FAKE, None, split, ys, ldys,
                       wq.WQ_BF16, None, 0, 0)
    assert q([96]) == 1                         # nsplit must be 2 or 3
    assert q([32, 32, 16, 16]) == 1
    assert q([32, 32, 16]) == 3                 # does not sum to n
    assert q([64, 0, 32]) == 3
    assert q([32, 32, 32], ys=[FAKE, None, FAKE]) == 1
    assert q([32, 32, 32], ys=[FAKE, FAKE + 1, FAKE]) == 4
    assert q([32, 32, 32], ldys=[32, 16, 32]) == 1
    assert q([32, 32, 32], ldys=[32, 1 << 31, 32]) == 1
    # destination windows that share a byte are refused before anything is enqueued
    assert q([32, 32, 32], ys=[FAKE, FAKE, FAKE + 1024]) == 1            # same base
    assert q([32, 32, 32], ys=[FAKE, FAKE + 62, FAKE + 1024]) == 1       # 1 bf16 column of row 0 shared
    # slab rows: three windows interleaved in rows of 96 (row r of split i at 96r + 32i); a
    # one-element shift makes row 0 of split 1 end inside row 0 of split 2
    assert q([32, 32, 32], ys=[FAKE, FAKE + 66, FAKE + 128], ldys=[96, 96, 96]) == 1
    # different strides: row 1 of the first window (stride 64) meets row 0 of the second
    assert q([32, 32, 32], ys=[FAKE, FAKE + 2 * 64 + 8, FAKE + 4096], ldys=[64, 32, 32]) == 1
    with pytest.raises(ValueError):
        wq.wq_matmul_qkv(d, 2, FAKE, 256, FAKE, FAKE, None, [32, 32, 32], [FAKE, FAKE], [32, 32, 32], wq.WQ_BF16)


def test_quantize_argument_validation():
    d = wq.desc(NVFP4, 32, 256)
    assert _status(wq.wq_quantize, d, None, FAKE, FAKE, 0) == 1
    assert _status(wq.wq_quantize, d, FAKE + 4, FAKE, FAKE, 0) == 4
    assert _status(wq.wq_quantize, d, FAKE, None, FAKE, 0) == 1
    assert _status(wq.wq_dequantize, d, FAKE, FAKE, FAKE + 8, 0) == 4
    assert _status(wq.wq_dequantize, wq.desc(NVFP4, 32, 200), FAKE, FAKE, FAKE, 0) == 3


def test_w4a4_argument_validation():
    """NVFP4 activations and the W4A4 product: every check returns before anything is enqueued."""
    assert wq.wq_act_packed_size(1500, 1280) == (1500 * 640, 1500 * 80 + 4)
    assert wq.wq_act_packed_size(3, 48) == (72, 16 + 4)            # 9 scale bytes, padded to 16, then g
    with pytest.raises(wq.WqError):
        wq.wq_act_packed_size(4, 24)                               # k % 16
    qa = lambda **kw: _status(wq.wq_quantize_act, kw.get("m", 4), kw.get("k", 256), kw.get("x", FAKE),
                              kw.get("ldx", 256), kw.get("codes", FAKE), kw.get("scales", FAKE), 0)
    assert qa(k=200) == 3
    assert qa(m=-1) == 3
    assert qa(m=1 << 27, k=1 << 10) == 3                           # m*k above 2^34
    assert qa(x=None) == 1 and qa(codes=None) == 1 and qa(scales=None) == 1
    assert qa(ldx=128) == 1 and qa(ldx=260) == 1
    assert qa(x=FAKE + 2) == 4 and qa(codes=FAKE + 4) == 4 and qa(scales=FAKE + 8) == 4
    assert qa(m=0) == 0
    d = wq.desc(NVFP4, 256, 512)
    need = wq.wq_w4a4_workspace_size(d, 20)
    assert need >= 256 + 20 * 512 * 2
    assert wq.wq_w4a4_workspace_size(d, 0) == 0
    with pytest.raises(wq.WqError):
        wq.wq_w4a4_workspace_size(wq.desc(NF4, 256, 512), 20)   # NVFP4 weights only
    mm = lambda **kw: _status(wq.wq_matmul_w4a4, kw.get("d", d), kw.get("m", 20), kw.get("xc", FAKE),
                              kw.get("xs", FAKE), kw.get("codes", FAKE), kw.get("scales", FAKE), kw.get("bias", None),
                              kw.get("y", FAKE), kw.get("ydt", wq.WQ_F32), kw.get("ldy", 256), kw.get("ws", FAKE),
                              kw.get("ws_bytes", need), 0)
    assert mm(d=wq.desc(Q4_0, 256, 512)) == 2
    assert mm(xc=None) == 1 and mm(xs=None) == 1
    assert mm(xc=FAKE + 8) == 4 and mm(xs=FAKE + 4) == 4
    assert mm(ws=None) == 6 and mm(ws_bytes=need - 1) == 6
    assert mm(ws=FAKE + 8) == 4
    assert mm(codes=None) == 1 and mm(y=None) == 1 and mm(ldy=128) == 1 and mm(ydt=5) == 1
    assert mm(ldy=1 << 31) == 1
    assert mm(bias=FAKE + 1) == 4
    assert mm(m=-1) == 3
    assert mm(m=0, ws=None, ws_bytes=0) == 0


def test_format_names():
    assert wq.format_from_name("nf4") == wq.format_from_name("4bit") == wq.format_from_name("INT4") == NF4
    assert wq.format_from_name("nvfp4") == NVFP4
    assert wq.format_from_name("q4_0") == Q4_0 and wq.format_from_name("q8_0") == Q8_0
    assert wq.format_from_name("q4_1") == Q4_1 and wq.format_from_name("q5_0") == Q5_0
    assert wq.format_from_name("q4_k") == Q4_K and wq.format_from_name("q6_k") == Q6_K
    with pytest.raises(ValueError):
        wq.format_from_name("fp8")


def test_binding_refuses_host_tensors():
    """The binding passes tensors' device addresses; a host tensor is refused before any
    call into the library, which would hand its address to a GPU kernel."""
    import torch
    d = wq.desc(NVFP4, 32, 256)
    w = torch.zeros((32, 256), dtype=torch.float32)
    with pytest.raises(ValueError, match="device buffers"):
        wq.wq_quantize(d, w, FAKE, FAKE, stream=0)
