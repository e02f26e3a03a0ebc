"""MI355X-native (gfx950) W4A8 quantized linear layer.

The kernels live in libw4a8.so (HIP, built in-tree by
``python -m w4a8_quantized_linear_amd.build``); this package is its ctypes
binding.  The library is loaded on first use, so importing the package (or its
``workloads`` / ``accounting`` helpers) does not need a GPU.
"""
from ._lib import (  # noqa: F401
    W4A8Error,
    attention_kv4_decode,
    gemm_w4a8,
    gemm_w4a8_noalloc,
    gemm_w4a8_decode_candidates,
    gemm_w4a8_plan,
    gemm_w4a8_plan_detail,
    gemm_w4a8_selector_score,
    gemm_w4a16,
    gemm_w4a8_workspace_bytes,
    kv4_attention_workspace_bytes,
    kv4_cache_alloc,
    kv4_cache_bytes,
    kv4_unpack,
    linear,
    norm_quantize_act_i8,
    quantize_act_per_token_i8,
    quantize_kv4,
    quantize_weights_w4g128,
    status_string,
    version,
    w4a8_packed_weight_bytes,
    w4a8_unpack_weights,
)

__all__ = [
    "W4A8Error", "attention_kv4_decode", "gemm_w4a8", "gemm_w4a8_noalloc", "gemm_w4a8_decode_candidates", "gemm_w4a8_plan", "gemm_w4a8_plan_detail",
    "gemm_w4a8_selector_score", "gemm_w4a16", "gemm_w4a8_workspace_bytes",
    "kv4_attention_workspace_bytes", "kv4_cache_alloc", "kv4_cache_bytes", "kv4_unpack", "linear",
    "norm_quantize_act_i8", "quantize_act_per_token_i8", "quantize_kv4",
    "quantize_weights_w4g128", "status_string", "version", "w4a8_packed_weight_bytes",
    "w4a8_unpack_weights",
]
