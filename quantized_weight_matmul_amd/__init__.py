"""MI355X-native accelerator linear layer.

A batch of matmuls sharing one f32 input, y[t][n_out] = x[t][n_in] * W^T, with
each weight stored as bf16, Q8 or Q4, behind the C ABI of ``include/il.h``
(libil.so, hand-written HIP kernels for gfx950).  ``il`` is the ctypes
binding with the C names; ``workloads`` draws seeded synthetic inputs.

One decode step over three projections that share x::

    import torch
    import quantized_weight_matmul_amd as il
    # host weights: bf16 bits as uint16 [n_out, n_in], or the packed Q8 / Q4
    # block bytes (il_upload_quantize builds Q8 / Q4 from f32 or bf16)
    hq = il.il_upload(wq, il.IL_BF16, 4096, 4096)
    hk = il.il_upload(wk, il.IL_BF16, 1024, 4096)
    hv = il.il_upload(wv, il.IL_BF16, 1024, 4096)
    x = torch.randn(1, 4096, device="cuda")
    yq, yk, yv = (torch.empty(1, n, device="cuda") for n in (4096, 1024, 1024))
    if il.il_matmul(x, 1, 4096, [(hq, 4096, yq), (hk, 1024, yk), (hv, 1024, yv)]) != 1:
        raise RuntimeError(il.il_last_error())   # nothing was computed
    # results are ready once torch's current stream reaches this point
"""
from .il import (  # noqa: F401
    IL_BF16, IL_Q4, IL_Q8, IL_SRC_BF16, IL_SRC_F32, LIB_PATH, Weight, il_centroid_argmax,
    il_centroid_argmax_workspace, il_download, il_free,
    il_last_error, il_matmul, il_matmul_gelu_mul, il_matmul_noalloc, il_name, il_read_probe, il_stats, il_upload, il_upload_quantize, il_wants,
    il_weight_bytes,
)

__all__ = [
    "IL_BF16", "IL_Q8", "IL_Q4", "IL_SRC_F32", "IL_SRC_BF16", "LIB_PATH", "Weight", "il_upload",
    "il_upload_quantize", "il_download", "il_free", "il_matmul", "il_matmul_noalloc", "il_matmul_gelu_mul", "il_centroid_argmax",
    "il_centroid_argmax_workspace",
    "il_wants", "il_name", "il_read_probe",
    "il_stats",
    "il_weight_bytes", "il_last_error",
]
