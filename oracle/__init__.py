"""CPU oracle for the accelerator linear layer -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the C-ABI library and
its Python binding in ``quantized_weight_matmul_amd``) never imports, links or
calls it, and the two share no code.

What it computes: y[t][n_out] = x[t][n_in] * W^T (oxinfer 0.0.0 ``src/gpu.rs``
page, doc comment of ``struct Job``) for W in one of the storage formats of
``enum WeightRef`` on that page: each weight element is decoded to the f32
value it denotes, products are formed exactly in f64 and summed in f64 in
increasing k, and the sum is rounded once to f32.  ``bound`` is
sum_k |x*w| in f64; the acceptance test is |y - y_ref| <= 4e-3 * bound per
output element.  The arithmetic lives in ``il_oracle.c`` (plain C, gcc -O2);
this module only marshals numpy arrays.

Also here: ``centroid_argmax`` (the centroid-masked LM head: centroid
logits, top-k clusters, exact scores of their tokens, first-max argmax) with
``token_score``; ``gelu_mul`` (the fused gate/up feed-forward step, GELU(x G^T) *
(x U^T), with its propagated error bound; ``gelu`` alone), and, for the
upload-quantiser row, ``quantize`` (f32 weights -> Q8 / Q4
host blocks by per-block absmax scaling, rule stated in ``il_oracle.c``) and
``f16_bits`` (f32 -> binary16, round to nearest even, from the format
definition).

Pins live in ``tests/oracle_pins.py`` (run by ``tests/test_oracle_pins.py``):
exhaustive bf16 / f16 decode against library casts; exact-rational brute
force on tiny shapes; closed forms (one-hot / identity W selects x columns,
x = 1 gives row sums, all-zero codes give 0); Q8/Q4 round trips on
representable values; hand-derived fixtures under ``tests/golden/``; numpy
float64 matmul at full shapes; for the quantiser, numpy's float16 cast,
hand-derived blocks, exact round trips and the nearest-grid-point property.
``tests/test_oracle_mutants.py`` plants
mistakes in copies of ``il_oracle.c`` and checks that the pins catch each.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

BF16, Q8, Q4 = 0, 1, 2
BLOCK = 32
TOL = 4e-3

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "il_oracle.c")
SO = os.path.join(_HERE, "liboracle.so")

_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p


def compile_oracle(src: str, out: str, verbose: bool = False) -> str:
    """gcc -O2 (no fast-math, no intrinsics) -fopenmp -> shared library."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = False, verbose: bool = False) -> str:
    if force or not os.path.exists(SO) or os.path.getmtime(SO) < os.path.getmtime(SRC):
        compile_oracle(SRC, SO, verbose)
    return SO


def _p(a: np.ndarray):
    return a.ctypes.data_as(_ptr)


def weight_bytes(fmt: int, n_out: int, n_in: int) -> int:
    """Host-format size; -1 for a bad format or shape (mirrors the C rule)."""
    if n_out <= 0 or n_in <= 0:
        return -1
    if fmt == BF16:
        return 2 * n_out * n_in
    if n_in % BLOCK:
        return -1
    if fmt == Q8:
        return 36 * n_out * (n_in // BLOCK)
    if fmt == Q4:
        return 18 * n_out * (n_in // BLOCK)
    return -1


class Oracle:
    """ctypes view of one compiled oracle library (the real one, or a planted
    mutant in the mutation tests)."""

    def __init__(self, so_path: str):
        lib = ctypes.CDLL(so_path)
        lib.orc_bf16_value.restype = ctypes.c_double
        lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
        lib.orc_f16_value.restype = ctypes.c_double
        lib.orc_f16_value.argtypes = [ctypes.c_uint16]
        lib.orc_weight_bytes.restype = _i64
        lib.orc_weight_bytes.argtypes = [ctypes.c_int, _i64, _i64]
        lib.orc_dequant_row.restype = ctypes.c_int
        lib.orc_dequant_row.argtypes = [_ptr, ctypes.c_int, _i64, _i64, _ptr]
        lib.orc_matmul_rows.restype = ctypes.c_int
        lib.orc_matmul_rows.argtypes = [_ptr, _i64, _i64, _ptr, ctypes.c_int, _i64, _i64, _i64,
                                        _ptr, _ptr, ctypes.c_int]
        lib.orc_matmul_points.restype = ctypes.c_int
        lib.orc_matmul_points.argtypes = [_ptr, _i64, _i64, _ptr, ctypes.c_int, _i64, _i64,
                                          _ptr, _ptr, _ptr, _ptr, ctypes.c_int]
        lib.orc_f16_bits.restype = ctypes.c_uint16
        lib.orc_f16_bits.argtypes = [ctypes.c_float]
        lib.orc_f16_bits_array.restype = None
        lib.orc_f16_bits_array.argtypes = [_ptr, _i64, _ptr]
        lib.orc_quantize.restype = ctypes.c_int
        lib.orc_quantize.argtypes = [_ptr, ctypes.c_int, _i64, _i64, _ptr]
        lib.orc_gelu.restype = ctypes.c_double
        lib.orc_gelu.argtypes = [ctypes.c_double]
        lib.orc_gelu_mul_rows.restype = ctypes.c_int
        lib.orc_gelu_mul_rows.argtypes = [_ptr, _i64, _i64, _ptr, _ptr, ctypes.c_int, _i64, _i64, _i64,
                                          _ptr, _ptr, ctypes.c_int]
        lib.orc_centroid_argmax.restype = ctypes.c_int
        lib.orc_centroid_argmax.argtypes = [_ptr, _i64, _i64, _ptr, _i64, _ptr, _i64, _ptr, _i64,
                                            _ptr, _ptr, _ptr, _ptr, _ptr]
        lib.orc_token_score.restype = ctypes.c_double
        lib.orc_token_score.argtypes = [_ptr, _i64, _ptr, _i64, ctypes.POINTER(ctypes.c_double)]
        lib.orc_check.restype = _i64
        lib.orc_check.argtypes = [_ptr, _ptr, _ptr, _i64, ctypes.c_double,
                                  ctypes.POINTER(_i64), ctypes.POINTER(ctypes.c_double)]
        self.lib = lib
        self.path = so_path

    # -- helpers ---------------------------------------------------------
    def _host_weight(self, weight, fmt: int, n_out: int, n_in: int) -> np.ndarray:
        w = np.ascontiguousarray(weight)
        need = int(self.lib.orc_weight_bytes(fmt, n_out, n_in))
        if need < 0:
            raise ValueError("bad format or shape")
        if w.nbytes != need:
            raise ValueError(f"weight holds {w.nbytes} bytes, format needs {need}")
        return w

    # -- API -------------------------------------------------------------
    def bf16_value(self, bits) -> np.ndarray:
        """bfloat16 bit patterns -> float64, decoded from the format definition."""
        b = np.asarray(bits, dtype=np.uint16)
        f = self.lib.orc_bf16_value
        return np.array([f(int(v)) for v in b.ravel()], dtype=np.float64).reshape(b.shape)

    def f16_value(self, bits) -> np.ndarray:
        """IEEE binary16 bit patterns -> float64, decoded from the format definition."""
        b = np.asarray(bits, dtype=np.uint16)
        f = self.lib.orc_f16_value
        return np.array([f(int(v)) for v in b.ravel()], dtype=np.float64).reshape(b.shape)

    def dequant(self, weight, fmt: int, n_out: int, n_in: int, rows=None) -> np.ndarray:
        """Decoded f32 weight rows, [len(rows), n_in] (all rows by default)."""
        w = self._host_weight(weight, fmt, n_out, n_in)
        rows = range(n_out) if rows is None else rows
        out = np.empty((len(rows), n_in), dtype=np.float32)
        for j, r in enumerate(rows):
            if not 0 <= r < n_out:
                raise IndexError(r)
            if self.lib.orc_dequant_row(_p(w), fmt, n_in, int(r), _p(out[j])) != 0:
                raise ValueError("dequant failed")
        return out

    def matmul(self, x: np.ndarray, weight, fmt: int, n_out: int, r0: int = 0,
               r1: int | None = None, threads: int = 0):
        """(y_ref [t, r1-r0] f32, bound [t, r1-r0] f64) for output rows [r0, r1)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        if x.ndim != 2:
            raise ValueError("x must be [t, n_in]")
        t, n_in = x.shape
        w = self._host_weight(weight, fmt, n_out, n_in)
        r1 = n_out if r1 is None else r1
        y = np.empty((t, r1 - r0), dtype=np.float32)
        bound = np.empty((t, r1 - r0), dtype=np.float64)
        if self.lib.orc_matmul_rows(_p(x), t, n_in, _p(w), fmt, n_out, r0, r1, _p(y), _p(bound),
                                    int(threads)) != 0:
            raise ValueError("oracle matmul failed")
        return y, bound

    def matmul_points(self, x: np.ndarray, weight, fmt: int, n_out: int, ii, rr,
                      threads: int = 0):
        """(y_ref[p], bound[p]) for the outputs (ii[p], rr[p])."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        t, n_in = x.shape
        w = self._host_weight(weight, fmt, n_out, n_in)
        ii = np.ascontiguousarray(ii, dtype=np.int64)
        rr = np.ascontiguousarray(rr, dtype=np.int64)
        if ii.shape != rr.shape:
            raise ValueError("ii and rr differ in shape")
        y = np.empty(ii.shape, dtype=np.float32)
        bound = np.empty(ii.shape, dtype=np.float64)
        if self.lib.orc_matmul_points(_p(x), t, n_in, _p(w), fmt, n_out, ii.size, _p(ii),
                                      _p(rr), _p(y), _p(bound), int(threads)) != 0:
            raise ValueError("oracle matmul_points failed")
        return y, bound

    def f16_bits(self, values) -> np.ndarray:
        """f32 values -> binary16 bit patterns (round to nearest even),
        converted from the format definition."""
        v = np.ascontiguousarray(values, dtype=np.float32)
        out = np.empty(v.shape, dtype=np.uint16)
        self.lib.orc_f16_bits_array(_p(v), v.size, _p(out))
        return out

    def quantize(self, w, fmt: int) -> np.ndarray:
        """f32 weights [n_out, n_in] -> host-format Q8 / Q4 blocks (uint8),
        by the absmax rule of ``orc_quantize``."""
        w = np.ascontiguousarray(w, dtype=np.float32)
        if w.ndim != 2:
            raise ValueError("w must be [n_out, n_in]")
        n_out, n_in = w.shape
        need = int(self.lib.orc_weight_bytes(fmt, n_out, n_in))
        if need < 0 or fmt == BF16:
            raise ValueError("bad format or shape")
        out = np.empty(need, dtype=np.uint8)
        if self.lib.orc_quantize(_p(w), fmt, n_out, n_in, _p(out)) != 0:
            raise ValueError("oracle quantize failed")
        return out

    def gelu(self, v) -> np.ndarray:
        """GELU(v) = v * Phi(v) in double (erf from the C library)."""
        a = np.asarray(v, dtype=np.float64)
        f = self.lib.orc_gelu
        return np.array([f(float(e)) for e in a.ravel()], dtype=np.float64).reshape(a.shape)

    def gelu_mul(self, x: np.ndarray, gate, up, fmt: int, n_out: int, r0: int = 0,
                 r1: int | None = None, threads: int = 0):
        """(y_ref [t, r1-r0] f32, bound [t, r1-r0] f64) of GELU(x G^T) * (x U^T);
        check with the usual 4e-3 * bound rule (the bound carries the
        propagation of both matmuls' tolerance through GELU)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        t, n_in = x.shape
        g = self._host_weight(gate, fmt, n_out, n_in)
        u = self._host_weight(up, fmt, n_out, n_in)
        r1 = n_out if r1 is None else r1
        y = np.empty((t, r1 - r0), dtype=np.float32)
        bound = np.empty((t, r1 - r0), dtype=np.float64)
        if self.lib.orc_gelu_mul_rows(_p(x), t, n_in, _p(g), _p(u), fmt, n_out, r0, r1, _p(y), _p(bound),
                                      int(threads)) != 0:
            raise ValueError("oracle gelu_mul failed")
        return y, bound

    def centroid_argmax(self, x, centroids, embed, ordering, k: int) -> dict:
        """Centroid-masked LM head per row of x [t, h]: centroids bf16 bits
        [C, h], embed bf16 bits [V, h], ordering uint32 [V], k clusters.
        Returns token [t], clusters [t, min(k, C)] (visiting order), score [t]
        (f32), cl and cl_bound [t, C] (exact f64 logits and sum |x*w|).  A k
        above C takes every cluster (`top_k_centroids.min(num_centroids)` in
        Drafter::step, oxinfer 0.0.1 src/drafter.rs page)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        t, h = x.shape
        cen = np.ascontiguousarray(centroids, dtype=np.uint16)
        emb = np.ascontiguousarray(embed, dtype=np.uint16)
        order = np.ascontiguousarray(ordering, dtype=np.uint32)
        n_c, vocab = cen.shape[0], emb.shape[0]
        if cen.shape[1] != h or emb.shape[1] != h or order.shape != (vocab,):
            raise ValueError("shape mismatch")
        out = {"token": np.empty(t, np.int32), "clusters": np.empty((t, min(int(k), n_c)), np.int32),
               "score": np.empty(t, np.float32), "cl": np.empty((t, n_c), np.float64),
               "cl_bound": np.empty((t, n_c), np.float64)}
        if self.lib.orc_centroid_argmax(_p(x), t, h, _p(cen), n_c, _p(emb), vocab, _p(order), k,
                                        _p(out["token"]), _p(out["clusters"]), _p(out["score"]),
                                        _p(out["cl"]), _p(out["cl_bound"])) != 0:
            raise ValueError("oracle centroid_argmax failed")
        return out

    def token_score(self, x_row, embed, tok: int):
        """(exact f64 score, bound) of one token against one row of x."""
        x_row = np.ascontiguousarray(x_row, dtype=np.float32)
        emb = np.ascontiguousarray(embed, dtype=np.uint16)
        b = ctypes.c_double(0.0)
        v = self.lib.orc_token_score(_p(x_row), x_row.size, _p(emb), int(tok), ctypes.byref(b))
        return float(v), float(b.value)

    def check(self, y, y_ref, bound, tol: float = TOL) -> dict:
        """Element-wise |y - y_ref| <= tol * bound (NaN/Inf in y fail)."""
        y = np.ascontiguousarray(y, dtype=np.float32)
        y_ref = np.ascontiguousarray(y_ref, dtype=np.float32)
        bound = np.ascontiguousarray(bound, dtype=np.float64)
        if not (y.shape == y_ref.shape == bound.shape):
            raise ValueError(f"shape mismatch {y.shape} {y_ref.shape} {bound.shape}")
        first = _i64(-1)
        worst = ctypes.c_double(0.0)
        bad = self.lib.orc_check(_p(y), _p(y_ref), _p(bound), y.size, tol, ctypes.byref(first),
                                 ctypes.byref(worst))
        return {"n": int(y.size), "bad": int(bad), "first_bad": int(first.value),
                "worst": float(worst.value), "ok": bad == 0}


_default = None
_lock = threading.Lock()


def default() -> Oracle:
    global _default
    with _lock:
        if _default is None:
            build()
            _default = Oracle(SO)
    return _default


def bf16_value(bits):
    return default().bf16_value(bits)


def f16_value(bits):
    return default().f16_value(bits)


def dequant(weight, fmt, n_out, n_in, rows=None):
    return default().dequant(weight, fmt, n_out, n_in, rows)


def matmul(x, weight, fmt, n_out, r0=0, r1=None, threads=0):
    return default().matmul(x, weight, fmt, n_out, r0, r1, threads)


def matmul_points(x, weight, fmt, n_out, ii, rr, threads=0):
    return default().matmul_points(x, weight, fmt, n_out, ii, rr, threads)


def check(y, y_ref, bound, tol=TOL):
    return default().check(y, y_ref, bound, tol)


def gelu(v):
    return default().gelu(v)


def gelu_mul(x, gate, up, fmt, n_out, r0=0, r1=None, threads=0):
    return default().gelu_mul(x, gate, up, fmt, n_out, r0, r1, threads)


def centroid_argmax(x, centroids, embed, ordering, k):
    return default().centroid_argmax(x, centroids, embed, ordering, k)


def token_score(x_row, embed, tok):
    return default().token_score(x_row, embed, tok)


def f16_bits(values):
    return default().f16_bits(values)


def quantize(w, fmt):
    return default().quantize(w, fmt)
