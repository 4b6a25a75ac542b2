"""GPU parity on seeded random shapes: format, t, n_in, the number of jobs
and their n_out drawn at random (ragged row counts, K that is not a whole
number of 128-element steps, several jobs per launch), under the library's
own kernel choice or a random pin of the family (IL_DECODE for t <= 8,
IL_PREFILL above).  Every output is compared with the oracle at
|y - y_ref| <= 4e-3 * sum_k |x_k w_k| (the matmul of `struct Job` on the
oxinfer 0.0.0 src/gpu.rs page, all jobs in one submission as Backend::matmul
on that page submits them)."""
import numpy as np
import pytest

import quantized_weight_matmul_amd as il
from quantized_weight_matmul_amd import workloads as wl
from conftest import gpu_available
from gpu_util import check_full, run, say, upload_all

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

FMTS = (il.IL_BF16, il.IL_Q8, il.IL_Q4)
TS = (1, 2, 3, 4, 5, 6, 7, 8, 9, 13, 16, 17, 24, 32, 33, 47, 64, 65, 100, 128, 129, 200, 300)


def _case(i):
    g = np.random.default_rng(5000 + i)
    fmt = int(g.choice(FMTS))
    t = int(g.choice(TS))
    n_in = 32 * int(g.integers(1, 161))
    n_jobs = int(g.integers(1, 4))
    cap = 3000 if t <= 64 else 900
    n_outs = [int(g.integers(1, cap + 1)) for _ in range(n_jobs)]
    pins = ["valu", "mfma"] if t <= 8 else ["verify", "gemm", "tiles"]
    pin = None if g.random() < 0.5 else str(g.choice(pins))
    return fmt, t, n_in, n_outs, pin


CASES = [_case(i) for i in range(48)]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_random_shape(i, monkeypatch):
    fmt, t, n_in, n_outs, pin = CASES[i]
    if pin in ("valu", "mfma"):
        monkeypatch.setenv("IL_DECODE", pin)
    elif pin is not None:
        monkeypatch.setenv("IL_PREFILL", pin)
    say(f"[random {i}] fmt={wl.FMT_NAMES[fmt]} t={t} n_in={n_in} n_outs={n_outs} pin={pin}")
    x = np.random.default_rng(6000 + i).standard_normal((t, n_in)).astype(np.float32)
    ws = [wl.gen_weight(fmt, 70 + i, j, n, n_in) for j, n in enumerate(n_outs)]
    hs = upload_all(ws, [fmt] * len(n_outs), n_outs, n_in)
    ys = run(x, hs, n_outs)
    for j, (y, w, n) in enumerate(zip(ys, ws, n_outs)):
        r = check_full(y, x, w, fmt, n, what=f"random case {i} job {j}")
        say(f"  job {j}: {r['n']} outputs, worst |err|/bound {r['worst']:.2e}")
    for h in hs:
        il.il_free(h)
