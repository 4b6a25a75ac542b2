"""C ABI contract on the CPU (no GPU needed): the library loads, exports every
symbol the header declares, and rejects bad arguments before touching a device."""
import ctypes
import os
import re

import numpy as np
import pytest

import quantized_weight_matmul_amd as il
from quantized_weight_matmul_amd import il as binding
from quantized_weight_matmul_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "il.h")


def header_symbols():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"IL_API\s+[\w\s\*]*?\b(il_\w+)\s*\(", src)))


def test_header_declares_the_abi():
    assert header_symbols() == sorted([
        "il_upload", "il_upload_quantize", "il_download", "il_free", "il_matmul", "il_matmul_noalloc",
        "il_matmul_gelu_mul",
        "il_centroid_argmax", "il_centroid_argmax_workspace", "il_read_probe", "il_wants", "il_name", "il_stats",
        "il_weight_bytes", "il_last_error"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    for name in header_symbols():
        assert hasattr(lib, name), name


def test_library_exports_nothing_else():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines() if " T " in l})
    assert exported == header_symbols()


def test_name_and_stats():
    assert il.il_name() == "il-hip-gfx950"
    s = il.il_stats()
    assert "decode_gemv:" in s and "prefill_gemm:" in s and "uploads:" in s
    need = binding.lib().il_stats(None, 0)
    assert need == len(s)
    small = ctypes.create_string_buffer(8)
    assert binding.lib().il_stats(small, 8) == need
    assert small.value == s[:7].encode()


def test_weight_bytes_null():
    assert binding.lib().il_weight_bytes(None) == -1


def test_wants_policy():
    # a pure, monotone function of the sizes; true for every workload shape
    for sub in wl.SUBMISSIONS.values():
        for j in sub.jobs:
            assert il.il_wants(j.n_out, sub.n_in, sub.t) == 1
    assert il.il_wants(0, 4096, 1) == 0
    assert il.il_wants(4096, 0, 1) == 0
    assert il.il_wants(4096, 4096, 0) == 0
    assert il.il_wants(1, 32, 1) == 0  # 64 flops: below the default 2^18
    prev = 0
    for n in [1, 2, 8, 64, 256, 1024, 4096]:
        cur = il.il_wants(n, 256, 1)
        assert cur >= prev
        prev = cur


def test_wants_env_threshold(monkeypatch):
    monkeypatch.setenv("IL_WANTS_MIN_FLOP", "1e12")
    assert il.il_wants(4096, 4096, 1) == 0
    monkeypatch.setenv("IL_WANTS_MIN_FLOP", "0")
    assert il.il_wants(1, 32, 1) == 1


@pytest.mark.parametrize("args,msg", [
    ((None, 0, 4, 64), "NULL"),
    ((b"\0" * 512, 7, 4, 64), "unknown format"),
    ((b"\0" * 512, 0, 0, 64), "n_out"),
    ((b"\0" * 512, 0, -3, 64), "n_out"),
    ((b"\0" * 512, 0, 4, 48), "multiple of 32"),
    ((b"\0" * 512, 1, 4, 0), "multiple of 32"),
    ((b"\0" * 512, 2, 4, 16), "multiple of 32"),
])
def test_upload_rejects_bad_arguments(args, msg):
    weight, fmt, n_out, n_in = args
    lib = binding.lib()
    buf = ctypes.create_string_buffer(weight) if weight is not None else None
    h = lib.il_upload(buf, fmt, n_out, n_in)
    assert not h
    assert msg in il.il_last_error()


def test_upload_injected_failure(monkeypatch):
    monkeypatch.setenv("IL_FORCE_FAIL", "upload")
    assert il.il_upload(np.zeros((4, 64), np.uint16), il.IL_BF16, 4, 64) is None
    assert "IL_FORCE_FAIL" in il.il_last_error()


def test_upload_without_a_device_declines():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert il.il_upload(np.zeros((4, 64), np.uint16), il.IL_BF16, 4, 64) is None
    assert il.il_last_error()  # the reason is reported


def _matmul_raw(x, t, n_in, jobs, n_jobs=None):
    lib = binding.lib()
    arr = (binding.il_job * max(1, len(jobs)))()
    for i, (w, n_out, y) in enumerate(jobs):
        arr[i].w, arr[i].n_out, arr[i].y = w, n_out, y
    return lib.il_matmul(x, t, n_in, arr, len(jobs) if n_jobs is None else n_jobs, None)


def test_matmul_trivial_calls_succeed():
    assert _matmul_raw(None, 0, 64, []) == 1  # t == 0
    assert _matmul_raw(0x1000, 4, 64, [], n_jobs=0) == 1  # no jobs


@pytest.mark.parametrize("x,t,n_in,jobs,msg", [
    (0x1000, -1, 64, [(0x10, 4, 0x2000)], "negative"),
    (None, 1, 64, [(0x10, 4, 0x2000)], "x is NULL"),
    (0x1000, 1, 48, [(0x10, 4, 0x2000)], "bad sizes"),
    (0x1004, 1, 64, [(0x10, 4, 0x2000)], "aligned"),
])
def test_matmul_rejects_bad_arguments(x, t, n_in, jobs, msg):
    assert _matmul_raw(x, t, n_in, jobs) == 0
    assert msg in il.il_last_error()


def test_matmul_rejects_negative_job_count():
    assert _matmul_raw(0x1000, 1, 64, [(0x10, 4, 0x2000)], n_jobs=-1) == 0


def test_matmul_injected_failure(monkeypatch):
    monkeypatch.setenv("IL_FORCE_FAIL", "upload,matmul")
    assert _matmul_raw(0x1000, 1, 64, [(0x10, 4, 0x2000)]) == 0
    assert "IL_FORCE_FAIL" in il.il_last_error()


@pytest.mark.parametrize("args,msg", [
    ((None, 0, 1, 4, 64), "NULL"),
    ((b"\0" * 1024, 5, 1, 4, 64), "source type"),
    ((b"\0" * 1024, 0, 0, 4, 64), "not a quantised format"),
    ((b"\0" * 1024, 0, 9, 4, 64), "not a quantised format"),
    ((b"\0" * 1024, 0, 1, 0, 64), "n_out"),
    ((b"\0" * 1024, 1, 2, 4, 40), "multiple of 32"),
])
def test_upload_quantize_rejects_bad_arguments(args, msg):
    weight, src, fmt, n_out, n_in = args
    buf = ctypes.create_string_buffer(weight) if weight is not None else None
    assert not binding.lib().il_upload_quantize(buf, src, fmt, n_out, n_in)
    assert msg in il.il_last_error()


def test_upload_quantize_injected_failure(monkeypatch):
    monkeypatch.setenv("IL_FORCE_FAIL", "upload")
    w = np.zeros((4, 64), np.float32)
    assert il.il_upload_quantize(w, il.IL_SRC_F32, il.IL_Q8, 4, 64) is None
    assert "IL_FORCE_FAIL" in il.il_last_error()


def test_upload_quantize_binding_checks_dtype_and_size():
    with pytest.raises(TypeError):
        il.il_upload_quantize(np.zeros((4, 64), np.float64), il.IL_SRC_F32, il.IL_Q8, 4, 64)
    with pytest.raises(TypeError):
        il.il_upload_quantize(np.zeros((4, 64), np.float32), il.IL_SRC_BF16, il.IL_Q4, 4, 64)
    with pytest.raises(ValueError):
        il.il_upload_quantize(np.zeros((4, 32), np.float32), il.IL_SRC_F32, il.IL_Q8, 4, 64)


def test_upload_quantize_without_a_device_declines():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert il.il_upload_quantize(np.zeros((4, 64), np.float32), il.IL_SRC_F32, il.IL_Q4, 4, 64) is None
    assert il.il_last_error()


def test_download_null_handle():
    assert binding.lib().il_download(None, None, 0) == -1
    assert "NULL" in il.il_last_error()


def test_centroid_argmax_workspace_size():
    assert il.il_centroid_argmax_workspace(1, 2048, 32) == (2048 + 64) * 4
    assert il.il_centroid_argmax_workspace(8, 100, 3) == 8 * (100 + 6) * 4
    assert il.il_centroid_argmax_workspace(9, 2048, 32) == -1  # at most 8 rows
    assert il.il_centroid_argmax_workspace(1, 0, 1) == -1
