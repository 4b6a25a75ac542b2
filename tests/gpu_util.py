"""Helpers for the GPU parity tests: run a submission through the C ABI and
compare it with the oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import quantized_weight_matmul_amd as il
from quantized_weight_matmul_amd import workloads as wl

TOL = 4e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def upload_all(weights, fmts, n_outs, n_in):
    hs = []
    for w, fmt, n_out in zip(weights, fmts, n_outs):
        h = il.il_upload(w, fmt, n_out, n_in)
        assert h is not None, il.il_last_error()
        hs.append(h)
    return hs


def run(x_np: np.ndarray, handles, n_outs, fill=float("nan"), stream=None):
    """il_matmul on device copies; returns the y arrays on the host."""
    import torch
    t, n_in = x_np.shape
    x = torch.from_numpy(np.ascontiguousarray(x_np)).cuda()
    ys = [torch.full((t, n), fill, dtype=torch.float32, device="cuda") for n in n_outs]
    rc = il.il_matmul(x, t, n_in, [(h, n, y) for h, n, y in zip(handles, n_outs, ys)], stream)
    assert rc == 1, il.il_last_error()
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys]


def check_full(y, x, weight, fmt, n_out, what=""):
    y_ref, bound = oracle.matmul(x, weight, fmt, n_out)
    r = oracle.check(y, y_ref, bound, TOL)
    assert r["ok"], f"{what}: {r['bad']}/{r['n']} outside tolerance, first {r['first_bad']}, worst {r['worst']:.3g}"
    return r


def check_sampled(y, x, weight, fmt, n_out, n_pts=2048, seed=0, what=""):
    t = x.shape[0]
    g = np.random.default_rng(seed)
    ii = np.r_[0, t - 1, g.integers(0, t, n_pts)]
    rr = np.r_[0, n_out - 1, g.integers(0, n_out, n_pts)]
    y_ref, bound = oracle.matmul_points(x, weight, fmt, n_out, ii, rr)
    r = oracle.check(y[ii, rr], y_ref, bound, TOL)
    assert r["ok"], f"{what}: {r['bad']}/{r['n']} sampled outputs outside tolerance, worst {r['worst']:.3g}"
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    return r


def submission_inputs(sub: wl.Submission):
    return wl.make_x(sub), wl.make_weights(sub)
