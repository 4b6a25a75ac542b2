"""GPU parity on weights whose device planes pass 2 GiB.

The kernels address weights through 64-bit bases (one buffer descriptor per
row, per 16-row tile or per GEMM tile), so rows past the first 2^31 bytes of
a plane must come out right.  The matrix-core decode and mid-size kernels
take 32-bit offsets over a whole plane and decline such weights; the call
then runs on the f32 decode kernel or the GEMM, which these cases pin down
by t and IL_DECODE / IL_PREFILL.  Weights are a seeded random block of 997
rows repeated down the matrix (997 is prime, so the sampled rows differ);
the outputs checked against the oracle include the rows on either side of
the 2 GiB boundary of the code plane and the last row.
"""
import numpy as np
import pytest

import oracle
import quantized_weight_matmul_amd as il
from quantized_weight_matmul_amd import workloads as wl
from conftest import gpu_available
from gpu_util import TOL, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

BF16, Q8, Q4 = il.IL_BF16, il.IL_Q8, il.IL_Q4
N_IN = 4096
BLOCK_ROWS = 997
# rows per format so that the device code plane passes 2^31 bytes
N_OUT = {BF16: 270_000, Q8: 540_000, Q4: 1_100_000}
CODE_BYTES_PER_ROW = {BF16: 2 * N_IN, Q8: N_IN, Q4: N_IN // 2}
# (t, env): the f32 decode kernel, the matrix-core decode declining to it,
# and the GEMM (the mid-size kernel declining to it)
CASES = {
    BF16: [(1, {}), (2, {"IL_DECODE": "mfma"}), (24, {"IL_PREFILL": "verify"}), (300, {})],
    Q8: [(1, {}), (5, {}), (300, {})],
    Q4: [(1, {}), (20, {})],
}


def _big_weight(fmt, g):
    n_out, nb = N_OUT[fmt], N_IN // 32
    if fmt == BF16:
        block = wl.f32_to_bf16_bits((g.standard_normal((BLOCK_ROWS, N_IN)) * 0.02).astype(np.float32))
    elif fmt == Q8:
        block = wl.encode_q8(g.integers(-127, 128, (BLOCK_ROWS, N_IN)).astype(np.int8),
                             g.uniform(1e-4, 1e-3, (BLOCK_ROWS, nb)).astype(np.float32)).reshape(BLOCK_ROWS, -1)
    else:
        block = wl.encode_q4(g.integers(0, 16, (BLOCK_ROWS, N_IN)).astype(np.uint8),
                             g.uniform(1e-3, 1e-2, (BLOCK_ROWS, nb)).astype(np.float16).view(np.uint16)
                             ).reshape(BLOCK_ROWS, -1)
    reps = -(-n_out // BLOCK_ROWS)
    return np.ascontiguousarray(np.tile(block, (reps, 1))[:n_out])


@pytest.mark.parametrize("fmt", [BF16, Q8, Q4], ids=["bf16", "q8", "q4"])
def test_planes_past_2_gib(fmt, monkeypatch):
    import torch
    n_out = N_OUT[fmt]
    assert n_out * CODE_BYTES_PER_ROW[fmt] > 2 ** 31
    g = np.random.default_rng(31 + fmt)
    say(f"[large] fmt={fmt} n_out={n_out} n_in={N_IN}: building the host weight")
    w = _big_weight(fmt, g)
    h = il.il_upload(w, fmt, n_out, N_IN)
    assert h is not None, il.il_last_error()
    edge = 2 ** 31 // CODE_BYTES_PER_ROW[fmt]  # first row whose codes start past 2 GiB
    rows = np.r_[0, edge - 2, edge - 1, edge, edge + 1, n_out - 1, g.integers(0, n_out, 200)]
    for t, env in CASES[fmt]:
        monkeypatch.delenv("IL_DECODE", raising=False)
        monkeypatch.delenv("IL_PREFILL", raising=False)
        for k, v in env.items():
            monkeypatch.setenv(k, v)
        say(f"[large] fmt={fmt} t={t} env={env}")
        x_np = g.standard_normal((t, N_IN)).astype(np.float32)
        x = torch.from_numpy(x_np).cuda()
        y = torch.full((t, n_out), float("nan"), device="cuda")
        assert il.il_matmul(x, t, N_IN, [(h, n_out, y)]) == 1, il.il_last_error()
        torch.cuda.synchronize()
        ii = np.repeat(np.arange(t), rows.size) if t <= 8 else np.repeat([0, t // 2, t - 1], rows.size)
        rr = np.tile(rows, ii.size // rows.size)
        got = y[torch.from_numpy(ii).cuda(), torch.from_numpy(rr).cuda()].cpu().numpy()
        y_ref, bound = oracle.matmul_points(x_np, w, fmt, n_out, ii, rr)
        r = oracle.check(got, y_ref, bound, TOL)
        assert r["ok"], f"fmt {fmt} t {t}: {r['bad']}/{r['n']} outside tolerance, worst {r['worst']:.3g}"
        assert bool(torch.isfinite(y).all()), f"fmt {fmt} t {t}: an output was not written"
        del y, x
    h.free()
