"""The call plan of the per-Linear format policy, run on the GPU: a projection whose parts
share a format runs as one fused wq_matmul_qkv, and one whose parts differ falls back to
separate wq_matmul calls ("Run quantized Whisper on the fused Metal decode path", "Test plan":
mixed-format fallback, neighbouring rows untouched).  Either way each part lands in its
window of a K/V-cache-like slab, within the matmul bound against the CPU oracle, and nothing
outside the windows changes."""
import numpy as np
import pytest
import torch

from block_quantized_bit_amd import policy as P
from block_quantized_bit_amd import wq
from block_quantized_bit_amd.inputs import bf16_bits_to_f32, linear_case

from gpu_helpers import abs_dot, check_bound, dev_bf16, gpu_quantize, require_gpu, say, DEV

pytestmark = pytest.mark.gpu

SENT = 0x7BAD   # bf16 bit pattern left in every slab element no call may write


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _fmt_args(fmt):
    return (wq.WQ_NF4, True) if fmt == "nf4dq" else (wq.format_from_name(fmt), False)


def _run_group(orc, pol, members, m, seed, merge_cross_kv=False):
    calls = [c for c in P.plan(pol, merge_cross_kv) if set(c.names) <= set(members)]
    names = [n for c in calls for n in c.names]
    parts = len(names)
    k = P.D_MODEL
    _, _, x = linear_case(seed, 16, k, m)
    X = dev_bf16(x)
    pad = 64
    ld = parts * P.D_MODEL + pad                 # slab row: the parts side by side, then padding
    slab = torch.full((m, ld), SENT, dtype=torch.int16, device=DEV)
    refs = {}
    col = 0
    for c in calls:
        fmt_id, dq = _fmt_args(c.fmt)
        ws, bs, offs = [], [], []
        for i, name in enumerate(c.names):
            w, b, _ = linear_case(seed + 100 + names.index(name), P.D_MODEL, k, 1)
            if name.endswith(".k"):
                b = np.zeros_like(b)                 # the key projection has no bias
            ws.append(w)
            bs.append(b)
            offs.append(col + i * P.D_MODEL)
        W = np.concatenate(ws)
        Bb = np.concatenate(bs)
        ref = orc.quantize(fmt_id, W, dq)
        d, codes, scales = gpu_quantize(fmt_id, W, dq)
        B = dev_bf16(Bb)
        nb = wq.wq_workspace_size(d, m)
        wsb = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
        base = slab.data_ptr()
        if c.fused:
            ys = [base + 2 * o for o in offs]
            wq.wq_matmul_qkv(d, m, X, k, codes, scales, B, list(c.split_n), ys, [ld] * len(ys), wq.WQ_BF16,
                             wsb if nb else None, nb)
        else:
            wq.wq_matmul(d, m, X, k, codes, scales, B, base + 2 * offs[0], wq.WQ_BF16, ld, wsb if nb else None, nb)
        for i, name in enumerate(c.names):
            rows = slice(i * P.D_MODEL, (i + 1) * P.D_MODEL)
            refs[name] = (offs[i], ref["w_hat"][rows], Bb[rows])
        col += len(c.names) * P.D_MODEL
    torch.cuda.synchronize()
    y = slab.cpu().numpy().view(np.uint16)
    assert np.all(y[:, parts * P.D_MODEL:] == SENT), "padding columns were written"
    for name, (off, w_hat, b) in refs.items():
        got = bf16_bits_to_f32(y[:, off:off + P.D_MODEL])
        check_bound(got, orc.matmul(x, w_hat, b), abs_dot(x, w_hat), bf16_out=True, what=name)
    return calls


@pytest.mark.parametrize("m", [1, 16])
def test_self_attention_qkv_fused_and_mixed(orc, m):
    say("policy self-attn qkv", m)
    qkv = [f"decoder.0.self_attn.{s}" for s in "qkv"]
    fused = _run_group(orc, P.make_policy("nf4dq"), qkv, m, 7100)
    assert len(fused) == 1 and fused[0].fused
    mixed = _run_group(orc, P.make_policy("nf4dq", {"decoder.0.self_attn.k": "q8_0"}), qkv, m, 7100)
    assert [c.fmt for c in mixed] == ["nf4dq", "q8_0", "nf4dq"] and not any(c.fused for c in mixed)


def test_cross_attention_kv_mixed_at_encoder_frames(orc):
    kv = ["decoder.3.cross_attn.k", "decoder.3.cross_attn.v"]
    say("policy cross-attn kv", 300)
    fused = _run_group(orc, P.make_policy("q4_0"), kv, 300, 7200)
    assert len(fused) == 1 and fused[0].fused and fused[0].fmt == "q4_0"
    mixed = _run_group(orc, P.make_policy("q4_0", {"decoder.3.cross_attn.v": "nvfp4"}), kv, 300, 7200)
    assert [(c.names, c.fmt) for c in mixed] == [((kv[0],), "q4_0"), ((kv[1],), "nvfp4")]


def test_cross_attention_kv_merged_across_layers(orc):
    """All four layers' cross-attention K/V as one merged call (N = 10240) at 300 frames: each
    part lands in its 1280-column window of the slab; with one layer in another format the
    other three still merge."""
    kv = [f"decoder.{l}.cross_attn.{s}" for l in range(4) for s in "kv"]
    say("policy cross-attn kv merged", 300)
    merged = _run_group(orc, P.make_policy("nf4dq"), kv, 300, 7300, merge_cross_kv=True)
    assert len(merged) == 1 and merged[0].merged and merged[0].n == 10240
    pol = P.make_policy("nf4dq", {"decoder.2.cross_attn.k": "q4_0", "decoder.2.cross_attn.v": "q4_0"})
    calls = _run_group(orc, pol, kv, 300, 7300, merge_cross_kv=True)
    assert [(len(c.names), c.fmt, c.merged) for c in calls] == [(6, "nf4dq", True), (2, "q4_0", False)]
