"""wq_matmul_noalloc: the allocation-free form of wq_matmul (its K-split partial sums go
to the library's static device array instead of a caller workspace).  Checked through
the C ABI against wq_matmul with a workspace (bit for bit: the same kernels and
schedule run) and against the CPU oracle on sampled rows (the matmul bound), on two
calls in a row, the second with a smaller input that leaves the first call's partials
behind in the array."""
import numpy as np
import pytest
import torch

from block_quantized_bit_amd import wq
from block_quantized_bit_amd.inputs import linear_case

from gpu_helpers import abs_dot, check_bound, dev_bf16, gpu_quantize, require_gpu, say, workspace, DEV

pytestmark = pytest.mark.gpu

NF4, NVFP4, Q8_0 = 1, 2, 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _rows(m):
    r = np.random.default_rng(m).choice(m, size=min(m, 30), replace=False)
    return np.unique(np.concatenate([[0, m - 1], r]))


@pytest.mark.parametrize("fmt,dq", [(NVFP4, False), (NF4, True), (Q8_0, False)], ids=["nvfp4", "nf4dq", "q8_0"])
def test_noalloc_matches_workspace_call(orc, fmt, dq):
    n, k = 1280, 5120                                     # encoder fc2: few output tiles, K is split
    w, b, x_all = linear_case(4300, n, k, 1500)
    ref = orc.quantize(fmt, w, dq)
    d, codes, scales = gpu_quantize(fmt, w, dq)
    B = dev_bf16(b)
    for m in (1500, 300, 4):                              # second and third calls smaller
        x = x_all[:m]
        say("noalloc", fmt, "dq" if dq else "", m, n, k)
        X = dev_bf16(x)
        need = wq.wq_workspace_size(d, m)
        assert m <= 16 or need > 0, "this shape should use the K split"
        ws, wsb = workspace(d, m)
        y_ws = torch.full((m, n), -1.0, dtype=torch.float32, device=DEV)
        wq.wq_matmul(d, m, X, k, codes, scales, B, y_ws, wq.WQ_F32, n, ws, wsb)
        y_na = torch.full((m, n), -2.0, dtype=torch.float32, device=DEV)
        wq.wq_matmul_noalloc(d, m, X, k, codes, scales, B, y_na, wq.WQ_F32, n)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws), f"m={m}: allocation-free result differs from the workspace call"
        rows = _rows(m)
        check_bound(y_na.cpu().numpy()[rows], orc.matmul(x, ref["w_hat"], b, rows=rows),
                    abs_dot(x, ref["w_hat"], rows=rows), what=f"noalloc m={m}")
        # bf16 output too, same bits as the workspace call
        z_ws = torch.empty((m, n), dtype=torch.int16, device=DEV)
        z_na = torch.empty((m, n), dtype=torch.int16, device=DEV)
        wq.wq_matmul(d, m, X, k, codes, scales, B, z_ws, wq.WQ_BF16, n, ws, wsb)
        wq.wq_matmul_noalloc(d, m, X, k, codes, scales, B, z_na, wq.WQ_BF16, n)
        torch.cuda.synchronize()
        assert torch.equal(z_na, z_ws)
