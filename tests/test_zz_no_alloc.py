"""il_matmul_noalloc against il_matmul, through the C ABI.

il_matmul_noalloc is il_matmul for callers that cannot allocate: the prefill
path's bf16 copy of x lives in a static 32 MiB buffer per device instead of a
buffer the library allocates.  Its results must equal il_matmul's (the same
kernels run), bit for bit, and be within the tolerance of the oracle
(|y - y_ref| <= 4e-3 * sum |x w|); two prefill calls in a row, the second
smaller, must both be right although they share the buffer; a call that
would need more than the buffer holds must fail before anything runs.
"""
import numpy as np
import pytest

import quantized_weight_matmul_amd as il
from quantized_weight_matmul_amd import workloads as wl
from conftest import gpu_available
from gpu_util import check_full, check_sampled, say, upload_all

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

BF16, Q8, Q4 = il.IL_BF16, il.IL_Q8, il.IL_Q4
FMT_NAME = {BF16: "bf16", Q8: "q8", Q4: "q4"}
LIMIT = 32 << 20  # bytes of the static buffer


def _weight(fmt, g, n_out, n_in):
    nb = n_in // 32
    if fmt == BF16:
        return wl.f32_to_bf16_bits((g.standard_normal((n_out, n_in)) * 0.05).astype(np.float32))
    if fmt == Q8:
        return wl.encode_q8(g.integers(-127, 128, (n_out, n_in)).astype(np.int8),
                            g.uniform(1e-3, 1e-2, (n_out, nb)).astype(np.float32))
    return wl.encode_q4(g.integers(0, 16, (n_out, n_in)).astype(np.uint8),
                        g.uniform(1e-3, 1e-1, (n_out, nb)).astype(np.float16).view(np.uint16))


def _call(fn, x_np, handles, n_outs):
    import torch
    t, n_in = x_np.shape
    x = torch.from_numpy(np.ascontiguousarray(x_np)).cuda()
    ys = [torch.full((t, n), float("nan"), dtype=torch.float32, device="cuda") for n in n_outs]
    rc = fn(x, t, n_in, [(h, n, y) for h, n, y in zip(handles, n_outs, ys)])
    assert rc == 1, il.il_last_error()
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys]


@pytest.mark.parametrize("fmt", [BF16, Q8, Q4], ids=lambda f: FMT_NAME[f])
def test_noalloc_equals_il_matmul(fmt):
    g = np.random.default_rng(4100 + fmt)
    n_in = 1056
    n_outs = [300, 17]
    ws = [_weight(fmt, g, n, n_in) for n in n_outs]
    hs = upload_all(ws, [fmt] * len(n_outs), n_outs, n_in)
    # two prefill calls in a row, the second smaller; then the paths that use
    # no scratch (decode, mid-size rounding x itself) and a mid-size call that
    # reads the bf16 copy of x
    for t in (300, 100, 2, 12, 24):
        say(f"[noalloc] fmt={FMT_NAME[fmt]} t={t} n_in={n_in} n_outs={n_outs}")
        x = g.standard_normal((t, n_in)).astype(np.float32)
        got = _call(il.il_matmul_noalloc, x, hs, n_outs)
        ref = _call(il.il_matmul, x, hs, n_outs)
        for w, n, a, b in zip(ws, n_outs, got, ref):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"t {t} n_out {n}: differs from il_matmul"
            check_full(a, x, w, fmt, n, what=f"noalloc fmt {fmt} t {t} n_out {n}")


@pytest.mark.parametrize("fmt", [Q8, Q4], ids=lambda f: FMT_NAME[f])
def test_noalloc_mid_split(fmt):
    """The mid-size plan whose last round is split over K keeps its chunk
    sums in the static scratch too: two calls in a row (the second smaller),
    each bitwise equal to il_matmul."""
    g = np.random.default_rng(4300 + fmt)
    n_in, n_outs = 256, [17408, 17408]
    ws = [_weight(fmt, g, n, n_in) for n in n_outs]
    hs = upload_all(ws, [fmt] * len(n_outs), n_outs, n_in)
    for t in (100, 40):
        say(f"[noalloc mid] fmt={FMT_NAME[fmt]} t={t} n_in={n_in} n_outs={n_outs}")
        x = g.standard_normal((t, n_in)).astype(np.float32)
        got = _call(il.il_matmul_noalloc, x, hs, n_outs)
        ref = _call(il.il_matmul, x, hs, n_outs)
        for w, n, a, b in zip(ws, n_outs, got, ref):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"t {t} n_out {n}: differs from il_matmul"
            check_sampled(a, x, w, fmt, n, what=f"noalloc mid fmt {fmt} t {t} n_out {n}")


def test_noalloc_size_limit():
    """t * n_in * 2 bytes of scratch: at the limit the call runs and equals
    il_matmul; one row more and it fails before anything runs, y untouched."""
    import torch
    g = np.random.default_rng(4200)
    n_in, n_out = 4096, 64
    w = _weight(BF16, g, n_out, n_in)
    (h,) = upload_all([w], [BF16], [n_out], n_in)
    t = LIMIT // (2 * n_in)  # 4096 tokens: exactly the buffer
    say(f"[noalloc limit] t={t} n_in={n_in}")
    x = g.standard_normal((t, n_in)).astype(np.float32)
    (a,) = _call(il.il_matmul_noalloc, x, [h], [n_out])
    (b,) = _call(il.il_matmul, x, [h], [n_out])
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    xd = torch.from_numpy(g.standard_normal((t + 1, n_in)).astype(np.float32)).cuda()
    y = torch.full((t + 1, n_out), 7.0, device="cuda")
    assert il.il_matmul_noalloc(xd, t + 1, n_in, [(h, n_out, y)]) == 0
    err = il.il_last_error()
    assert "static" in err and "scratch" in err, err
    torch.cuda.synchronize()
    assert torch.all(y == 7.0), "y was written by a rejected call"
    # decode needs no scratch whatever the size of x
    yd = torch.empty((1, n_out), device="cuda")
    assert il.il_matmul_noalloc(xd[:1], 1, n_in, [(h, n_out, yd)]) == 1, il.il_last_error()
