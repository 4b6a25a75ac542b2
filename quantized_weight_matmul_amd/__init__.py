"""MI355X-native accelerator linear layer.

A batch of matmuls sharing one f32 input, y[t][n_out] = x[t][n_in] * W^T, with
each weight stored as bf16, Q8 or Q4, behind the C ABI of ``include/il.h``
(libil.so, hand-written HIP kernels for gfx950).  ``il`` is the ctypes
binding with the C names; ``workloads`` draws seeded synthetic inputs.
"""
from .il import (  # noqa: F401
    IL_BF16, IL_Q4, IL_Q8, IL_SRC_BF16, IL_SRC_F32, LIB_PATH, Weight, il_centroid_argmax,
    il_centroid_argmax_workspace, il_download, il_free,
    il_last_error, il_matmul, il_matmul_gelu_mul, il_name, il_stats, il_upload, il_upload_quantize, il_wants,
    il_weight_bytes,
)

__all__ = [
    "IL_BF16", "IL_Q8", "IL_Q4", "IL_SRC_F32", "IL_SRC_BF16", "LIB_PATH", "Weight", "il_upload",
    "il_upload_quantize", "il_download", "il_free", "il_matmul", "il_matmul_gelu_mul", "il_centroid_argmax",
    "il_centroid_argmax_workspace",
    "il_wants", "il_name",
    "il_stats",
    "il_weight_bytes", "il_last_error",
]
