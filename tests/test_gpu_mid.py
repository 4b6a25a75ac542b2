"""GPU parity of the mid-size plan: Q8/Q4 weights at 32 < t <= 128 on GEMM
units that hold all t tokens (64 or 128 rows of x) by 128 weight rows, each
summed over K in fixed chunks (Q4 at t <= 64 on the 4-wave units, the rest
on the 8-wave units).  When the units are whole rounds of the compute units
plus a few (the Q4 verify shape, 2 x [17408, 5120], has 272 units for 256
CUs), those few are split over K, one workgroup per chunk, and a second
launch adds each split unit's chunk sums in chunk order.  Checked here, on
shapes with that unit count:
  * every output against the oracle (ragged K, and a job whose last unit
    holds fewer than 128 rows, included);
  * the bits of a job do not depend on whether its units ran whole or split
    (the job alone against the job in a batch that splits it), and repeat
    run to run whatever order the chunks finish in;
  * the fused gate/up + GELU step on the same plan.
The full-size verify workloads at t = 64 and 128 are checked (sampled) in
test_gpu_parity.py.
"""
import numpy as np
import pytest

import oracle
import quantized_weight_matmul_amd as il
from quantized_weight_matmul_amd import workloads as wl
from conftest import gpu_available
from gpu_util import check_full, run, say, upload_all

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

Q8, Q4 = il.IL_Q8, il.IL_Q4
NAME = {Q8: "q8", Q4: "q4"}
N_OUT = 17408  # 136 units of 128 rows per job: two jobs make 272


def _weights(fmt, n_in, ids):
    return [wl.gen_weight(fmt, 11, i, N_OUT, n_in) for i in ids]


CASES = [(Q4, 33, 1024), (Q4, 64, 1024), (Q4, 40, 288), (Q4, 128, 1024), (Q4, 100, 288), (Q8, 64, 1024),
         (Q8, 128, 1024), (Q8, 65, 288)]


@pytest.mark.parametrize("fmt,t,n_in", CASES, ids=[f"{NAME[f]}-t{t}-k{k}" for f, t, k in CASES])
def test_mid_split_matches_oracle(fmt, t, n_in):
    say(f"[mid] {NAME[fmt]} t={t} 2 x [{N_OUT}, {n_in}]")
    ws = _weights(fmt, n_in, (1, 2))
    x = np.random.default_rng(t + n_in).standard_normal((t, n_in)).astype(np.float32)
    hs = upload_all(ws, [fmt, fmt], [N_OUT, N_OUT], n_in)
    ys = run(x, hs, [N_OUT, N_OUT])
    for j, (y, w) in enumerate(zip(ys, ws)):
        r = check_full(y, x, w, fmt, N_OUT, what=f"job {j}")
        say(f"  job {j}: {r['n']} outputs ok, worst {r['worst']:.2e}")


@pytest.mark.parametrize("fmt,t", [(Q8, 100), (Q4, 100), (Q4, 64)], ids=["q8-t100", "q4-t100", "q4-t64"])
def test_mid_split_bits_do_not_depend_on_the_split(fmt, t):
    """Job B's last 16 units are split in the batch [A, B] (272 units) and
    run whole when B is alone (136 units): the same bits either way."""
    n_in = 1024
    say(f"[mid] invariance {NAME[fmt]} t={t}")
    ws = _weights(fmt, n_in, (3, 4))
    x = np.random.default_rng(7).standard_normal((t, n_in)).astype(np.float32)
    hs = upload_all(ws, [fmt, fmt], [N_OUT, N_OUT], n_in)
    a = run(x, hs, [N_OUT, N_OUT])
    b = run(x, hs, [N_OUT, N_OUT])
    alone_b = run(x, hs[1:], [N_OUT])[0]
    alone_a = run(x, hs[:1], [N_OUT])[0]
    for ya, yb in zip(a, b):
        assert np.array_equal(ya, yb), "not bitwise reproducible"
    assert np.array_equal(a[1], alone_b), "a split unit differs from the same unit run whole"
    assert np.array_equal(a[0], alone_a)
    check_full(a[1], x, ws[1], fmt, N_OUT, what="job B")


@pytest.mark.parametrize("fmt", [Q8, Q4], ids=lambda f: NAME[f])
def test_mid_glu_split(fmt):
    """Gate/up + GELU on the mid plan: 17408 outputs are 272 units of 64
    (each unit's B tile holds 64 gate and 64 up rows)."""
    import torch
    t, n_in = 80, 256
    say(f"[mid] gelu_mul {NAME[fmt]} t={t} 2 x [{N_OUT}, {n_in}]")
    G, U = _weights(fmt, n_in, (5, 6))
    x_np = np.random.default_rng(9).standard_normal((t, n_in)).astype(np.float32)
    hg, hu = il.il_upload(G, fmt, N_OUT, n_in), il.il_upload(U, fmt, N_OUT, n_in)
    x = torch.from_numpy(x_np).cuda()
    y = torch.full((t, N_OUT), float("nan"), dtype=torch.float32, device="cuda")
    assert il.il_matmul_gelu_mul(x, t, n_in, hg, hu, N_OUT, y) == 1, il.il_last_error()
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    y_ref, bound = oracle.gelu_mul(x_np, G, U, fmt, N_OUT)
    r = oracle.check(y, y_ref, bound)
    assert r["ok"], f"{r['bad']}/{r['n']} outside the propagated tolerance, worst {r['worst']:.3g}"
    say(f"  {r['n']} outputs ok, worst {r['worst']:.2e}")


def test_mid_q4_ragged_rows_split():
    """The 4-wave units with a job whose last unit holds 28 rows, ragged K
    (9 blocks: the last K step has one), and that unit among the split ones
    (136 + 136 units): every output against the oracle, and job B's bits
    the same alone (136 units, none split)."""
    t, n_in, n_b = 57, 288, N_OUT - 100
    say(f"[mid] q4 ragged t={t} [{N_OUT}, {n_in}] + [{n_b}, {n_in}]")
    wa = wl.gen_weight(Q4, 12, 1, N_OUT, n_in)
    wb = wl.gen_weight(Q4, 12, 2, n_b, n_in)
    x = np.random.default_rng(57).standard_normal((t, n_in)).astype(np.float32)
    hs = upload_all([wa, wb], [Q4, Q4], [N_OUT, n_b], n_in)
    ya, yb = run(x, hs, [N_OUT, n_b])
    check_full(ya, x, wa, Q4, N_OUT, what="job A")
    r = check_full(yb, x, wb, Q4, n_b, what="job B")
    say(f"  job B: {r['n']} outputs ok, worst {r['worst']:.2e}")
    alone_b = run(x, hs[1:], [n_b])[0]
    assert np.array_equal(yb, alone_b), "a split unit differs from the same unit run whole"
