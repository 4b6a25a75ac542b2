"""GPU parity of the fused gate/up step, y = GELU(x G^T) * (x U^T)
(il_matmul_gelu_mul), against the oracle's gelu_mul, whose bound carries the
4e-3 matmul tolerance of g and u through GELU.  Every kernel family that can
run it is pinned in turn: decode t <= 8 on the streaming ("valu") and
matrix-core ("mfma") kernels, t = 9..32 on the wide matrix-core mode
("verify") and the GEMM, larger t on the GEMM.  Beside the oracle, the fused
result must agree with GELU applied (on the host, in double) to the g and u
that il_matmul computes with the same kernels, to within the rounding of
GELU itself: the fusion changes where g and u go, not how they are summed.
"""
import numpy as np
import pytest

import oracle
import quantized_weight_matmul_amd as il
from quantized_weight_matmul_amd import workloads as wl
from conftest import gpu_available
from gpu_util import run, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

BF16, Q8, Q4 = il.IL_BF16, il.IL_Q8, il.IL_Q4
NAME = {BF16: "bf16", Q8: "q8", Q4: "q4"}


def _paths(t):
    if t <= 8:
        return ("valu", "mfma")
    # the matrix-core wide mode takes up to 128 tokens (in slices of <= 32)
    return ("verify", "gemm") if t <= 128 else ("gemm",)


def _pin(monkeypatch, path):
    if path in ("valu", "mfma"):
        monkeypatch.setenv("IL_DECODE", path)
    else:
        monkeypatch.setenv("IL_PREFILL", path)


def _fused(x_np, gate, up, n_out, fill=np.nan):
    import torch
    t, n_in = x_np.shape
    x = torch.from_numpy(np.ascontiguousarray(x_np)).cuda()
    y = torch.full((t, n_out), float(fill), dtype=torch.float32, device="cuda")
    assert il.il_matmul_gelu_mul(x, t, n_in, gate, up, n_out, y) == 1, il.il_last_error()
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _gelu64(v):
    return oracle.gelu(np.asarray(v, np.float64))


CASES = [(t, p) for t in (1, 2, 3, 5, 8, 9, 16, 17, 32, 33, 64, 130, 257) for p in _paths(t)]


@pytest.mark.parametrize("fmt", [BF16, Q8, Q4], ids=lambda f: NAME[f])
@pytest.mark.parametrize("t,path", CASES, ids=[f"t{t}-{p}" for t, p in CASES])
def test_gelu_mul_matches_oracle(fmt, t, path, monkeypatch):
    _pin(monkeypatch, path)
    n_out, n_in = 200, 96 if t > 64 else 1024  # n_out: not a multiple of 16 or 128
    say(f"[gelu_mul] {NAME[fmt]} t={t} path={path} [{n_out}, {n_in}]")
    G = wl.gen_weight(fmt, 9, 1, n_out, n_in)
    U = wl.gen_weight(fmt, 9, 2, n_out, n_in)
    x = np.random.default_rng(t).standard_normal((t, n_in)).astype(np.float32)
    hg, hu = il.il_upload(G, fmt, n_out, n_in), il.il_upload(U, fmt, n_out, n_in)
    y = _fused(x, hg, hu, n_out)
    y_ref, bound = oracle.gelu_mul(x, G, U, fmt, n_out)
    r = oracle.check(y, y_ref, bound)
    assert r["ok"], f"{r['bad']}/{r['n']} outside the propagated tolerance, worst {r['worst']:.3g}"
    g, u = run(x, [hg, hu], [n_out, n_out])
    want = _gelu64(g) * u.astype(np.float64)
    err = np.abs(y.astype(np.float64) - want)
    # f32 GELU: a few ulp relative, plus erff's absolute error (~2^-22) times
    # |g| / 2 where 1 + erf cancels for negative g
    allow = 2.0 ** -18 * np.abs(want) + 2.0 ** -21 * np.abs(g.astype(np.float64) * u)
    assert np.all(err <= allow), \
        f"fused differs from GELU(g) * u of the unfused kernels: worst {np.max(err / (allow + 1e-300)):.3g} x allowed"


@pytest.mark.parametrize("name", ["f3_q8_t1", "f3_q4_t1", "f3_bf16_t1", "f3_q8_t512", "f3_q4_t512"])
def test_gelu_mul_workload_sampled(name):
    """The measured workloads at full size: a band of rows at the start, the
    middle and the end checked against the oracle."""
    fmt, n_out, n_in, t, cfg = wl.GELU_MUL[name]
    say(f"[gelu_mul] {name}: {NAME[fmt]} t={t} 2 x [{n_out}, {n_in}]")
    x, G, U = wl.make_gelu_mul_inputs(name)
    hg, hu = il.il_upload(G, fmt, n_out, n_in), il.il_upload(U, fmt, n_out, n_in)
    y = _fused(x, hg, hu, n_out)
    assert np.all(np.isfinite(y))
    for r0 in (0, n_out // 2, n_out - 256):
        y_ref, bound = oracle.gelu_mul(x, G, U, fmt, n_out, r0, r0 + 256)
        r = oracle.check(y[:, r0:r0 + 256], y_ref, bound)
        assert r["ok"], f"rows {r0}..: {r['bad']} outside, worst {r['worst']:.3g}"


def test_gelu_mul_rejects_mismatched_weights_and_leaves_y():
    import torch
    n_in = 64
    a = il.il_upload(wl.gen_weight(Q8, 9, 3, 32, n_in), Q8, 32, n_in)
    b = il.il_upload(wl.gen_weight(Q4, 9, 4, 32, n_in), Q4, 32, n_in)
    c = il.il_upload(wl.gen_weight(Q8, 9, 5, 48, n_in), Q8, 48, n_in)
    x = torch.ones((2, n_in), device="cuda")
    y = torch.full((2, 32), 7.0, device="cuda")
    assert il.il_matmul_gelu_mul(x, 2, n_in, a, b, 32, y) == 0 and "share the format" in il.il_last_error()
    assert il.il_matmul_gelu_mul(x, 2, n_in, a, c, 32, y) == 0
    assert il.il_matmul_gelu_mul(x, 2, 32, a, a, 32, y) == 0
    torch.cuda.synchronize()
    assert torch.all(y == 7.0).item(), "y must be untouched after a rejected call"
    assert il.il_matmul_gelu_mul(x, 0, n_in, a, a, 32, y) == 1  # t == 0: no-op
