"""libwq for MI355X: weight-only 4-bit (NF4, NVFP4, q4_0, q4_1, q4_k), 5-bit (q5_0), 6-bit (q6_k) and 8-bit
(q8_0) matmul
with dequantization fused into hand-written gfx950 HIP kernels.

The C ABI is include/wq.h; `block_quantized_bit_amd.wq` is its Python binding.
"""
from . import wq  # noqa: F401
from .wq import (WQ_BF16, WQ_F32, WQ_NF4, WQ_NVFP4, WQ_Q4_0, WQ_Q4_1, WQ_Q4_K, WQ_Q5_0, WQ_Q6_K, WQ_Q8_0,  # noqa: F401
                 WqError,
                 desc,
                 format_from_name, wq_dequantize, wq_matmul, wq_matmul_qkv, wq_packed_size,
                 wq_quantize, wq_status_str, wq_workspace_size)

__all__ = ["wq", "desc", "format_from_name", "WqError", "wq_packed_size", "wq_quantize",
           "wq_dequantize", "wq_workspace_size", "wq_matmul", "wq_matmul_qkv", "wq_status_str",
           "WQ_NF4", "WQ_NVFP4", "WQ_Q4_0", "WQ_Q4_1", "WQ_Q4_K", "WQ_Q5_0", "WQ_Q6_K", "WQ_Q8_0", "WQ_BF16",
           "WQ_F32"]
