"""GPU parity at the edges of the block-scale range, on every kernel family.

The Q8 / Q4 formats of `enum WeightRef` (oxinfer 0.0.0 src/gpu.rs page) carry
one scale per 32-element block: an f32 for Q8, an IEEE binary16 for Q4.  The
workloads draw scales well inside the normal range; these cases drive the
extremes through il_matmul and compare every output with the oracle at
|y - y_ref| <= 4e-3 * sum_k |x_k w_k|:

* Q4 blocks whose f16 scales are subnormal (0x0001 .. 0x03FF) or the smallest
  normals, mixed with ordinary blocks in the same rows;
* Q8 blocks whose f32 scales sit near the bottom of the f32 range (normal
  and subnormal, around 1e-38), mixed with ordinary blocks;
* one-hot rows whose value code * scale is not a bf16 number, against x at a
  bf16 rounding midpoint (x = 1 + 2^-8): a path that rounds both operands to
  bf16 misses by ~6.8e-3 of the bound;
* whole rows of tiny scales, so that every term of an output is tiny.

Each runs at t in {1, 2, 8, 20, 300} under every kernel pin that t has
(IL_DECODE = valu | mfma for t <= 8, IL_PREFILL = verify | gemm above).
"""
import numpy as np
import pytest

import quantized_weight_matmul_amd as il
from quantized_weight_matmul_amd import workloads as wl
from conftest import gpu_available
from gpu_util import check_full, run, say, upload_all

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

BF16, Q8, Q4 = il.IL_BF16, il.IL_Q8, il.IL_Q4
FMT_NAME = {BF16: "bf16", Q8: "q8", Q4: "q4"}


def _cases():
    out = []
    for t in (1, 2, 8, 20, 300):
        if t <= 8:
            paths = ("valu", "mfma")
        elif t <= 128:
            paths = ("verify", "gemm")
        else:
            paths = ("gemm",)
        out += [(t, p) for p in paths]
    return out


def _pin(monkeypatch, path):
    if path in ("valu", "mfma"):
        monkeypatch.setenv("IL_DECODE", path)
    else:
        monkeypatch.setenv("IL_PREFILL", path)


def _q4_edge_scales(g, n_out, nb):
    """f16 scale bits: a third subnormal (0x0001..0x03FF), a third among the
    smallest normals (0x0400..0x07FF), the rest ordinary (~1e-3..1e-1), in
    random positions of every row."""
    kind = g.integers(0, 3, (n_out, nb))
    sub = g.integers(1, 0x400, (n_out, nb))
    small = g.integers(0x400, 0x800, (n_out, nb))
    normal = g.uniform(1e-3, 1e-1, (n_out, nb)).astype(np.float16).view(np.uint16)
    s = np.where(kind == 0, sub, np.where(kind == 1, small, normal)).astype(np.uint16)
    s[0, :] = 0x0001  # one row of the smallest subnormal only
    return s


def _q8_edge_scales(g, n_out, nb):
    """f32 scales: a third around 1e-38 (normal and subnormal f32), a third
    at 1e-36..1e-34, the rest ordinary (1e-4..1e-3)."""
    kind = g.integers(0, 3, (n_out, nb))
    tiny = g.uniform(5e-40, 5e-38, (n_out, nb))
    low = 10.0 ** g.uniform(-36, -34, (n_out, nb))
    normal = g.uniform(1e-4, 1e-3, (n_out, nb))
    s = np.where(kind == 0, tiny, np.where(kind == 1, low, normal)).astype(np.float32)
    s[0, :] = np.float32(1.2e-38)  # one row of near-minimum normal scales only
    s[1, :] = np.float32(3e-39)    # and one of subnormal scales only
    return s


@pytest.mark.parametrize("t,path", _cases())
def test_q4_subnormal_scales(t, path, monkeypatch):
    _pin(monkeypatch, path)
    g = np.random.default_rng(3100 + t)
    n_in = 1056  # 33 blocks: several K steps of every kernel and a ragged one
    n_outs = [300, 37]
    nb = n_in // 32
    say(f"[edge q4 subnormal] t={t} path={path} n_in={n_in} n_outs={n_outs}")
    x = g.standard_normal((t, n_in)).astype(np.float32)
    ws = [wl.encode_q4(g.integers(0, 16, (n, n_in)).astype(np.uint8), _q4_edge_scales(g, n, nb)) for n in n_outs]
    hs = upload_all(ws, [Q4] * len(n_outs), n_outs, n_in)
    ys = run(x, hs, n_outs)
    for w, n, y in zip(ws, n_outs, ys):
        r = check_full(y, x, w, Q4, n, what=f"q4 subnormal scales t {t} {path} n_out {n}")
        say(f"  n_out {n}: worst |err|/bound = {r['worst']:.2e}")


@pytest.mark.parametrize("t,path", _cases())
def test_q8_tiny_scales(t, path, monkeypatch):
    _pin(monkeypatch, path)
    g = np.random.default_rng(3200 + t)
    n_in = 1056
    n_outs = [300, 37]
    nb = n_in // 32
    say(f"[edge q8 tiny] t={t} path={path} n_in={n_in} n_outs={n_outs}")
    x = g.standard_normal((t, n_in)).astype(np.float32)
    ws = [wl.encode_q8(g.integers(-127, 128, (n, n_in)).astype(np.int8), _q8_edge_scales(g, n, nb))
          for n in n_outs]
    hs = upload_all(ws, [Q8] * len(n_outs), n_outs, n_in)
    ys = run(x, hs, n_outs)
    for w, n, y in zip(ws, n_outs, ys):
        r = check_full(y, x, w, Q8, n, what=f"q8 tiny scales t {t} {path} n_out {n}")
        say(f"  n_out {n}: worst |err|/bound = {r['worst']:.2e}")


@pytest.mark.parametrize("fmt", [Q8, Q4], ids=lambda f: FMT_NAME[f])
@pytest.mark.parametrize("t,path", _cases())
def test_onehot_off_grid_values(fmt, t, path, monkeypatch):
    """One-hot rows whose single value code * scale is not a bf16 number,
    against x at bf16 rounding midpoints (1 + 2^-8 times a power of two): the
    only term of each output must stay within 4e-3 of itself."""
    _pin(monkeypatch, path)
    g = np.random.default_rng(3300 + 7 * t + fmt)
    n_in, n_out = 320, 272
    nb = n_in // 32
    cols = g.integers(0, n_in, n_out)
    say(f"[edge one-hot off grid] fmt={FMT_NAME[fmt]} t={t} path={path}")
    x = (np.float32(1 + 2 ** -8) * np.float32(2.0) ** g.integers(-3, 4, (t, n_in))).astype(np.float32)
    x *= np.where(g.integers(0, 2, (t, n_in)) == 0, 1, -1).astype(np.float32)
    if fmt == Q4:
        codes = np.full((n_out, n_in), 8, np.uint8)
        codes[np.arange(n_out), cols] = g.integers(9, 16, n_out)  # values 1..7
        # f16 scales 1 + k 2^-10 with k odd: code * scale needs more than 8 bits
        sbits = np.full((n_out, nb), 0x3C00, np.uint16) + (2 * g.integers(0, 512, (n_out, nb)) + 1).astype(np.uint16)
        sbits[0, :] = 0x3C03  # the advisor's case: code 9, scale 1 + 3 * 2^-10
        codes[0, cols[0]] = 9
        w = wl.encode_q4(codes, sbits)
    else:
        codes = np.zeros((n_out, n_in), np.int8)
        codes[np.arange(n_out), cols] = g.integers(1, 128, n_out)
        sc = (1.0 + g.integers(1, 1 << 15, (n_out, nb)) * 2.0 ** -16).astype(np.float32)
        w = wl.encode_q8(codes, sc)
    (h,) = upload_all([w], [fmt], [n_out], n_in)
    (y,) = run(x, [h], [n_out])
    r = check_full(y, x, w, fmt, n_out, what=f"one-hot off grid fmt {fmt} t {t} {path}")
    say(f"  worst |err|/bound = {r['worst']:.2e}")


@pytest.mark.parametrize("fmt", [BF16, Q8, Q4], ids=lambda f: FMT_NAME[f])
@pytest.mark.parametrize("t,path", _cases())
def test_dense_midpoint_bias(fmt, t, path, monkeypatch):
    """Every x at a bf16 rounding midpoint ((1 + 2^-8) * 2^k, which rounds to
    2^k: each term loses 2^-8 / (1 + 2^-8) of itself) and every weight of
    the same sign, over 5120 inputs: on the paths that round x to bf16 the
    error of each output is that whole bias, ~0.973 of the 4e-3 tolerance,
    plus the f32 sums of every kernel -- the margin the bound leaves."""
    _pin(monkeypatch, path)
    g = np.random.default_rng(3400 + 11 * t + fmt)
    n_in, n_out = 5120, 272
    nb = n_in // 32
    say(f"[edge dense midpoint] fmt={FMT_NAME[fmt]} t={t} path={path}")
    x = (np.float32(1 + 2 ** -8) * np.float32(2.0) ** g.integers(-3, 4, (t, n_in))).astype(np.float32)
    x *= np.where(np.arange(t) % 2 == 0, 1, -1).astype(np.float32)[:, None]  # one sign per token
    if fmt == BF16:
        w = wl.f32_to_bf16_bits(g.uniform(0.5, 2.0, (n_out, n_in)).astype(np.float32))
    elif fmt == Q8:
        w = wl.encode_q8(g.integers(1, 128, (n_out, n_in)).astype(np.int8),
                         g.uniform(1e-3, 1e-2, (n_out, nb)).astype(np.float32))
    else:
        w = wl.encode_q4(g.integers(9, 16, (n_out, n_in)).astype(np.uint8),
                         g.uniform(1e-3, 1e-2, (n_out, nb)).astype(np.float16).view(np.uint16))
    (h,) = upload_all([w], [fmt], [n_out], n_in)
    (y,) = run(x, [h], [n_out])
    r = check_full(y, x, w, fmt, n_out, what=f"dense midpoint fmt {fmt} t {t} {path}")
    say(f"  worst |err|/bound = {r['worst']:.6f} ({r['worst'] / 4e-3:.4f} of the tolerance)")
