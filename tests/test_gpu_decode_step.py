"""The whole per-token decoder step of whisper-large-v3-turbo as a decoder calls it: the 24
calls of the policy's call plan (4 layers x {self-attention Q/K/V as one wq_matmul_qkv, self O,
cross Q, cross O, fc1, fc2}, NF4 with double quant) captured in one HIP graph ("Run quantized
Whisper on the fused Metal decode path", "Summary": the per-token work as one submission).
Every replay, with eager work between replays, must give the eager outputs bit for bit, and
every eager output meets the matmul bound against the CPU oracle.  (A single launch over
these calls is not possible: attention, norms and the activation sit between them.)"""
import numpy as np
import pytest
import torch

from block_quantized_bit_amd import policy as P
from block_quantized_bit_amd import wq
from block_quantized_bit_amd.inputs import bf16_bits_to_f32, linear_case

from gpu_helpers import abs_dot, check_bound, dev_bf16, gpu_quantize, require_gpu, say, DEV

pytestmark = pytest.mark.gpu

NF4 = 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.fixture(scope="module")
def step(orc):
    calls = [c for c in P.plan(P.make_policy("nf4dq")) if c.rows == "tokens"]
    assert len(calls) == 24
    mats = []
    for i, c in enumerate(calls):
        w, b, _ = linear_case(7300 + i, c.n, c.k, 1, outlier_frac=0.001)
        if c.fused:
            b = b.copy()
            b[1280:2560] = 0                      # the key projection has no bias
        say("decode step quantize", i, c.names[0], c.n, c.k)
        ref = orc.quantize(NF4, w, True)
        d, codes, scales = gpu_quantize(NF4, w, True)
        assert np.array_equal(codes.cpu().numpy(), ref["codes"]) and np.array_equal(scales.cpu().numpy(), ref["scales"])
        mats.append(dict(call=c, d=d, codes=codes, scales=scales, w_hat=ref["w_hat"], b=b, B=dev_bf16(b)))
    return mats


@pytest.mark.parametrize("m", [1, 16])
def test_graph_replayed_decoder_step(orc, step, m):
    xs = {k: linear_case(7400 + k, 16, k, m)[2] for k in (1280, 5120)}
    X = {k: dev_bf16(v) for k, v in xs.items()}
    outs = [torch.empty((m, e["call"].n), dtype=torch.float32, device=DEV) for e in step]
    st = torch.cuda.Stream()

    def enqueue(stream):
        for e, y in zip(step, outs):
            c = e["call"]
            if c.fused:
                p0 = y.data_ptr()
                wq.wq_matmul_qkv(e["d"], m, X[c.k], c.k, e["codes"], e["scales"], e["B"], list(c.split_n),
                                 [p0, p0 + 4 * 1280, p0 + 4 * 2560], [c.n] * 3, wq.WQ_F32, stream=stream)
            else:
                wq.wq_matmul(e["d"], m, X[c.k], c.k, e["codes"], e["scales"], e["B"], y, wq.WQ_F32, c.n, stream=stream)

    say("decode step eager", m)
    with torch.cuda.stream(st):
        enqueue(st)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for e, y in zip(step, eager):
        c = e["call"]
        x = xs[c.k]
        check_bound(y.cpu().numpy(), orc.matmul(x, e["w_hat"], e["b"]), abs_dot(x, e["w_hat"]),
                    what=f"{c.names[0]} m={m}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            enqueue(st)
    for rep in range(3):
        say("decode step replay", m, rep)
        for o in outs:
            o.fill_(float("nan"))                 # eager work between replays; stale outputs would show
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for y, ref in zip(outs, eager):
            assert torch.equal(y, ref), f"replay {rep} differs from the eager step"
