"""ctypes binding of the C ABI in include/il.h, with the same names.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libil.so.  PyTorch supplies device memory and streams.  If the
library is missing, the first call raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

IL_BF16, IL_Q8, IL_Q4 = 0, 1, 2
IL_SRC_F32, IL_SRC_BF16 = 0, 1
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libil.so")

_lock = threading.Lock()
_lib = None
_i64 = ctypes.c_int64


class il_job(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("n_out", ctypes.c_int64), ("y", ctypes.c_void_p)]


def lib() -> ctypes.CDLL:
    """The loaded libil.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with __graft_entry__.build() or "
                    "python -m quantized_weight_matmul_amd._build (there is no CPU fallback)")
            L = ctypes.CDLL(LIB_PATH)
            L.il_upload.restype = ctypes.c_void_p
            L.il_upload.argtypes = [ctypes.c_void_p, ctypes.c_int, _i64, _i64]
            L.il_upload_quantize.restype = ctypes.c_void_p
            L.il_upload_quantize.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, _i64, _i64]
            L.il_download.restype = _i64
            L.il_download.argtypes = [ctypes.c_void_p, ctypes.c_void_p, _i64]
            L.il_free.restype = None
            L.il_free.argtypes = [ctypes.c_void_p]
            L.il_matmul.restype = ctypes.c_int
            L.il_matmul.argtypes = [ctypes.c_void_p, _i64, _i64, ctypes.POINTER(il_job), _i64,
                                    ctypes.c_void_p]
            L.il_matmul_noalloc.restype = ctypes.c_int
            L.il_matmul_noalloc.argtypes = [ctypes.c_void_p, _i64, _i64, ctypes.POINTER(il_job), _i64,
                                            ctypes.c_void_p]
            L.il_matmul_gelu_mul.restype = ctypes.c_int
            L.il_matmul_gelu_mul.argtypes = [ctypes.c_void_p, _i64, _i64, ctypes.c_void_p, ctypes.c_void_p, _i64,
                                             ctypes.c_void_p, ctypes.c_void_p]
            L.il_centroid_argmax.restype = ctypes.c_int
            L.il_centroid_argmax.argtypes = [ctypes.c_void_p, _i64, _i64, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, _i64, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, _i64, ctypes.c_void_p]
            L.il_centroid_argmax_workspace.restype = _i64
            L.il_centroid_argmax_workspace.argtypes = [_i64, _i64, _i64]
            L.il_read_probe.restype = ctypes.c_int
            L.il_read_probe.argtypes = [ctypes.c_void_p, _i64, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        _i64, ctypes.c_void_p]
            L.il_wants.restype = ctypes.c_int
            L.il_wants.argtypes = [_i64, _i64, _i64]
            L.il_name.restype = ctypes.c_char_p
            L.il_name.argtypes = []
            L.il_stats.restype = _i64
            L.il_stats.argtypes = [ctypes.c_char_p, _i64]
            L.il_weight_bytes.restype = _i64
            L.il_weight_bytes.argtypes = [ctypes.c_void_p]
            L.il_last_error.restype = ctypes.c_char_p
            L.il_last_error.argtypes = []
            _lib = L
    return _lib


class Weight:
    """An il_weight handle; il_free runs when the object is collected."""

    __slots__ = ("handle", "fmt", "n_out", "n_in", "__weakref__")

    def __init__(self, handle: int, fmt: int, n_out: int, n_in: int):
        self.handle = handle
        self.fmt = fmt
        self.n_out = n_out
        self.n_in = n_in

    def free(self) -> None:
        if self.handle:
            lib().il_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass

    @property
    def bytes(self) -> int:
        return int(lib().il_weight_bytes(self.handle))


def _ptr(a) -> int:
    """Address of a torch tensor, numpy array, int address or None."""
    if a is None:
        return 0
    if isinstance(a, int):
        return a
    if hasattr(a, "data_ptr"):
        return int(a.data_ptr())
    if isinstance(a, np.ndarray):
        return int(a.ctypes.data)
    raise TypeError(f"cannot take the address of {type(a).__name__}")


def il_upload(weight, fmt: int, n_out: int, n_in: int):
    """Copy a HOST weight (numpy array / bytes) to the device; None if declined."""
    if isinstance(weight, (bytes, bytearray)):
        weight = np.frombuffer(weight, dtype=np.uint8)
    w = np.ascontiguousarray(weight)
    h = lib().il_upload(ctypes.c_void_p(w.ctypes.data), int(fmt), int(n_out), int(n_in))
    if not h:
        return None
    return Weight(h, int(fmt), int(n_out), int(n_in))


def il_upload_quantize(weight, src: int, fmt: int, n_out: int, n_in: int):
    """Quantise full-precision weights to Q8 / Q4 on the device; None if
    declined.  `weight` is a numpy array (float32, or bfloat16 bits as
    uint16) or a contiguous torch tensor (float32 or bfloat16) on the host or
    on the current device; a device tensor must be ready (synchronized)."""
    if hasattr(weight, "data_ptr"):
        import torch
        want = torch.float32 if src == IL_SRC_F32 else torch.bfloat16
        if weight.dtype != want or not weight.is_contiguous():
            raise TypeError(f"src {src} expects a contiguous {want} tensor, got {weight.dtype}")
        n = weight.numel()
        ptr = weight.data_ptr()
    else:
        weight = np.ascontiguousarray(weight)
        want = np.float32 if src == IL_SRC_F32 else np.uint16
        if weight.dtype != want:
            raise TypeError(f"src {src} expects {np.dtype(want).name} weights, got {weight.dtype}")
        n = weight.size
        ptr = weight.ctypes.data
    if n != n_out * n_in:
        raise ValueError(f"weight has {n} elements, shape needs {n_out * n_in}")
    h = lib().il_upload_quantize(ctypes.c_void_p(ptr), int(src), int(fmt), int(n_out), int(n_in))
    if not h:
        return None
    return Weight(h, int(fmt), int(n_out), int(n_in))


def il_download(w: Weight) -> np.ndarray:
    """The handle's weight in its host format, as uint8 bytes."""
    n = int(lib().il_download(w.handle, None, 0))
    if n < 0:
        raise RuntimeError(il_last_error())
    out = np.empty(n, dtype=np.uint8)
    if int(lib().il_download(w.handle, ctypes.c_void_p(out.ctypes.data), n)) != n:
        raise RuntimeError(il_last_error())
    return out


def il_free(w: Weight) -> None:
    w.free()


def _job_array(jobs):
    arr = (il_job * max(1, len(jobs)))()
    keep = []
    for i, (w, n_out, y) in enumerate(jobs):
        if w is None or not isinstance(w, Weight):
            arr[i].w = None
        else:
            arr[i].w = w.handle
        arr[i].n_out = int(n_out)
        arr[i].y = _ptr(y)
    return arr


def il_matmul(x, t: int, n_in: int, jobs, stream=None) -> int:
    """Run every job over x in one submission.

    x      : device tensor (or address) holding float32 [t, n_in]
    jobs   : sequence of (Weight, n_out, y) with y a device tensor (or address)
             holding float32 [t, n_out]
    stream : torch.cuda.Stream, raw hipStream_t address, or None for torch's
             current stream
    Returns 1 on success, 0 if nothing was computed (see il_last_error()).
    """
    return int(lib().il_matmul(ctypes.c_void_p(_ptr(x)), int(t), int(n_in), _job_array(jobs), len(jobs),
                               ctypes.c_void_p(int(_stream_handle(stream)))))


def il_matmul_noalloc(x, t: int, n_in: int, jobs, stream=None) -> int:
    """il_matmul that allocates nothing: the prefill path's bf16 copy of x
    lives in the library's static 32 MiB buffer per device (t * n_in <= 2^24
    where a copy is needed), shared by every call on the device."""
    return int(lib().il_matmul_noalloc(ctypes.c_void_p(_ptr(x)), int(t), int(n_in), _job_array(jobs), len(jobs),
                                       ctypes.c_void_p(int(_stream_handle(stream)))))


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def il_matmul_gelu_mul(x, t: int, n_in: int, gate: Weight, up: Weight, n_out: int, y, stream=None) -> int:
    """y = GELU(x G^T) * (x U^T) in one submission; 1 on success, 0 if
    nothing was computed (see il_last_error())."""
    return int(lib().il_matmul_gelu_mul(ctypes.c_void_p(_ptr(x)), int(t), int(n_in),
                                        gate.handle if gate else None, up.handle if up else None,
                                        int(n_out), ctypes.c_void_p(_ptr(y)),
                                        ctypes.c_void_p(int(_stream_handle(stream)))))


def il_centroid_argmax(x, t: int, h: int, centroids: Weight, embed: Weight, ordering, top_k: int, token,
                       clusters=None, score=None, workspace=None, workspace_bytes: int = 0, stream=None) -> int:
    """Centroid-masked LM head: token[t] (device int32) per row of x; the
    chosen clusters [t, top_k] and scores [t] when those buffers are given.
    ordering is a device uint32 [V] tensor; workspace an optional device
    buffer of il_centroid_argmax_workspace(t, C, top_k) bytes.  1 on
    success, 0 otherwise."""
    if workspace is not None and not workspace_bytes and hasattr(workspace, "numel"):
        workspace_bytes = workspace.numel() * workspace.element_size()
    return int(lib().il_centroid_argmax(ctypes.c_void_p(_ptr(x)), int(t), int(h),
                                        centroids.handle if centroids else None, embed.handle if embed else None,
                                        ctypes.c_void_p(_ptr(ordering)), int(top_k), ctypes.c_void_p(_ptr(token)),
                                        ctypes.c_void_p(_ptr(clusters)), ctypes.c_void_p(_ptr(score)),
                                        ctypes.c_void_p(_ptr(workspace)), int(workspace_bytes),
                                        ctypes.c_void_p(int(_stream_handle(stream)))))


def il_centroid_argmax_workspace(t: int, n_centroids: int, top_k: int) -> int:
    return int(lib().il_centroid_argmax_workspace(int(t), int(n_centroids), int(top_k)))


def il_read_probe(buf, nbytes: int, chunk: int, waves: int, depth: int, sink, sink_bytes: int, stream=None) -> int:
    """Plain streaming read of nbytes of device memory (a measurement aid);
    1 after enqueueing, 0 on bad arguments."""
    return int(lib().il_read_probe(ctypes.c_void_p(_ptr(buf)), int(nbytes), int(chunk), int(waves), int(depth),
                                   ctypes.c_void_p(_ptr(sink)), int(sink_bytes),
                                   ctypes.c_void_p(int(_stream_handle(stream)))))


def il_wants(n_out: int, n_in: int, t: int) -> int:
    return int(lib().il_wants(int(n_out), int(n_in), int(t)))


def il_name() -> str:
    return lib().il_name().decode()


def il_stats() -> str:
    n = lib().il_stats(None, 0)
    buf = ctypes.create_string_buffer(int(n) + 1)
    lib().il_stats(buf, n + 1)
    return buf.value.decode()


def il_weight_bytes(w: Weight) -> int:
    return int(lib().il_weight_bytes(w.handle if w else None))


def il_last_error() -> str:
    return lib().il_last_error().decode()
