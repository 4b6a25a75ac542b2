"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: |y - y_ref| <= 4e-3 * sum_k |x_k w_k| for every output checked (the
oracle computes y_ref and the bound), and the workload shapes checked at the
launch configuration the benchmark times.  Plus device-side closed forms and
invariants: one-hot / identity W, zero codes, determinism, batch-composition
invariance, power-of-two scaling, full coverage of y, no writes outside y,
and the validation paths that must leave y untouched.

Decode (t <= 8) has two kernel families, the f32 streaming kernel ("valu")
and the matrix-core kernel ("mfma"); the library picks one per format and t,
and IL_DECODE pins it, so decode cases run under both.  Mid-size t (9..32)
runs either the matrix-core kernel's wide mode ("verify") or the tiled GEMM
("gemm"), pinned by IL_PREFILL, and is tested under both.
"""
import numpy as np
import pytest

import oracle
import quantized_weight_matmul_amd as il
from quantized_weight_matmul_amd import workloads as wl
from conftest import gpu_available
from gpu_util import check_full, check_sampled, run, say, submission_inputs, upload_all

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

BF16, Q8, Q4 = il.IL_BF16, il.IL_Q8, il.IL_Q4
FMT_NAME = {BF16: "bf16", Q8: "q8", Q4: "q4"}


def _bf16_rne(a):
    """f32 -> nearest bf16 value (ties to even), as f32."""
    bits = wl.f32_to_bf16_bits(a).astype(np.uint32) << 16
    return bits.view(np.float32)


def _paths(t):
    if t <= 8:
        return ("valu", "mfma")
    # the matrix-core wide mode takes up to 128 tokens (in slices of <= 32)
    return ("verify", "gemm") if t <= 128 else ("gemm",)


def _decode_cases(ts):
    """(t, path) pairs: both kernel families wherever t has two."""
    return [(t, p) for t in ts for p in _paths(t)]


def _pin(monkeypatch, path):
    if path in ("valu", "mfma"):
        monkeypatch.setenv("IL_DECODE", path)
    if path in ("verify", "gemm"):
        monkeypatch.setenv("IL_PREFILL", path)


def _selected(x, path):
    """What a one-hot weight row returns for x on each path."""
    if path == "valu":
        return x
    return _bf16_rne(x)  # matrix-core decode, verify and gemm: bf16(x)


# ------------------------------------------------------------- workloads
@pytest.mark.parametrize("name", ["c1", "c2", "c3a", "c3b", "c4_t1", "c4_t2", "c4_t4", "c4_t8", "c4_t16", "c4_t32"])
def test_workload_full(name):
    sub = wl.SUBMISSIONS[name]
    say(f"[parity] {name}: t={sub.t} n_in={sub.n_in} jobs={[(FMT_NAME[j.fmt], j.n_out) for j in sub.jobs]}")
    x, ws = submission_inputs(sub)
    hs = upload_all(ws, [j.fmt for j in sub.jobs], [j.n_out for j in sub.jobs], sub.n_in)
    ys = run(x, hs, [j.n_out for j in sub.jobs])
    for j, w, y in zip(sub.jobs, ws, ys):
        r = check_full(y, x, w, j.fmt, j.n_out, what=f"{name} job {j.tensor_id}")
        say(f"  job {j.tensor_id}: {r['n']} outputs ok, worst |err|/bound = {r['worst']:.2e}")


@pytest.mark.parametrize("name", ["c4_t64", "c4_t128", "c5a", "c5b"])
def test_workload_sampled(name):
    sub = wl.SUBMISSIONS[name]
    say(f"[parity] {name}: t={sub.t} n_in={sub.n_in} jobs={[(FMT_NAME[j.fmt], j.n_out) for j in sub.jobs]}")
    x, ws = submission_inputs(sub)
    hs = upload_all(ws, [j.fmt for j in sub.jobs], [j.n_out for j in sub.jobs], sub.n_in)
    ys = run(x, hs, [j.n_out for j in sub.jobs])
    for j, w, y in zip(sub.jobs, ws, ys):
        r = check_sampled(y, x, w, j.fmt, j.n_out, n_pts=4096, what=f"{name} job {j.tensor_id}")
        say(f"  job {j.tensor_id}: {r['n']} sampled outputs ok, worst {r['worst']:.2e}")


# ---------------------------------------------------- odd shapes, all paths
def _rand_weight(fmt, g, n_out, n_in):
    nb = n_in // 32
    if fmt == BF16:
        return wl.f32_to_bf16_bits((g.standard_normal((n_out, n_in)) * 0.05).astype(np.float32))
    if fmt == Q8:
        return wl.encode_q8(g.integers(-128, 128, (n_out, n_in)).astype(np.int8),
                            g.uniform(1e-3, 1e-2, (n_out, nb)).astype(np.float32))
    return wl.encode_q4(g.integers(0, 16, (n_out, n_in)).astype(np.uint8),
                        g.uniform(1e-3, 1e-1, (n_out, nb)).astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("fmt", [BF16, Q8, Q4], ids=lambda f: FMT_NAME[f])
@pytest.mark.parametrize("t,path", _decode_cases([1, 2, 3, 5, 8, 9, 16, 17, 32, 33, 130, 257]))
def test_odd_shapes(fmt, t, path, monkeypatch):
    """Several tiles plus ragged tails in every dimension, three jobs per call."""
    _pin(monkeypatch, path)
    g = np.random.default_rng(1000 + 10 * t + fmt)
    for n_in in (32, 288, 4160):
        n_outs = [1, 17, 1000] if n_in < 4160 else [200, 129]
        say(f"[odd] fmt={FMT_NAME[fmt]} t={t} path={path} n_in={n_in} n_outs={n_outs}")
        x = g.standard_normal((t, n_in)).astype(np.float32)
        ws = [_rand_weight(fmt, g, n, n_in) for n in n_outs]
        hs = upload_all(ws, [fmt] * len(n_outs), n_outs, n_in)
        ys = run(x, hs, n_outs)
        for w, n, y in zip(ws, n_outs, ys):
            check_full(y, x, w, fmt, n, what=f"fmt {fmt} t {t} n_in {n_in} n_out {n}")


@pytest.mark.parametrize("fmt", [BF16, Q8, Q4], ids=lambda f: FMT_NAME[f])
@pytest.mark.parametrize("path", ["valu", "mfma"])
@pytest.mark.parametrize("t,n_in", [(1, 41024), (3, 13664), (8, 5152)])
def test_x_past_the_lds_limit(fmt, path, t, n_in, monkeypatch):
    """t * n_in * 4 bytes of x just past one workgroup's 160 KiB of LDS: the
    streaming kernel declines, and the decode runs on the kernel that stages
    x in K chunks (or on the matrix-core kernel, which keeps x in registers)."""
    _pin(monkeypatch, path)
    g = np.random.default_rng(1900 + 7 * t + fmt)
    n_outs = [65, 300]
    say(f"[lds limit] fmt={FMT_NAME[fmt]} path={path} t={t} n_in={n_in} n_outs={n_outs}")
    assert t * n_in * 4 > 160 * 1024
    x = g.standard_normal((t, n_in)).astype(np.float32)
    ws = [_rand_weight(fmt, g, n, n_in) for n in n_outs]
    hs = upload_all(ws, [fmt] * len(n_outs), n_outs, n_in)
    ys = run(x, hs, n_outs)
    for w, n, y in zip(ws, n_outs, ys):
        check_full(y, x, w, fmt, n, what=f"fmt {fmt} t {t} n_in {n_in} n_out {n}")


@pytest.mark.parametrize("fmt", [BF16, Q8], ids=lambda f: FMT_NAME[f])
@pytest.mark.parametrize("t", [1, 2, 4])
@pytest.mark.parametrize("n_in", [8160, 8192, 8224, 14336])
def test_long_rows_two_per_wave(fmt, t, n_in, monkeypatch):
    """Rows of 8192 inputs or more stream two per wave on the f32 kernel:
    either side of that threshold, row counts that leave the last
    workgroup's waves partly or wholly without a row."""
    _pin(monkeypatch, "valu")
    g = np.random.default_rng(2300 + 11 * t + fmt + n_in)
    n_outs = [1, 17, 263]
    say(f"[long rows] fmt={FMT_NAME[fmt]} t={t} n_in={n_in} n_outs={n_outs}")
    x = g.standard_normal((t, n_in)).astype(np.float32)
    ws = [_rand_weight(fmt, g, n, n_in) for n in n_outs]
    hs = upload_all(ws, [fmt] * len(n_outs), n_outs, n_in)
    ys = run(x, hs, n_outs)
    for w, n, y in zip(ws, n_outs, ys):
        check_full(y, x, w, fmt, n, what=f"fmt {fmt} t {t} n_in {n_in} n_out {n}")


@pytest.mark.parametrize("fmt", [BF16, Q8, Q4], ids=lambda f: FMT_NAME[f])
@pytest.mark.parametrize("t,path", [(2, "valu"), (2, "mfma"), (20, "verify"), (300, "gemm")])
def test_jobs_split_across_launches(fmt, t, path, monkeypatch):
    """il_matmul starts a new launch before one launch's rows would pass a
    limit (2^31 - 1: the kernels count rows in 32-bit ints; IL_LAUNCH_ROWS
    lowers it for tests).  Splitting the jobs over several launches leaves
    every result bitwise unchanged."""
    _pin(monkeypatch, path)
    g = np.random.default_rng(2400 + 10 * t + fmt)
    n_in = 512
    n_outs = [300, 17, 129, 256, 64, 200]
    say(f"[split] fmt={FMT_NAME[fmt]} t={t} path={path} n_outs={n_outs}")
    x = g.standard_normal((t, n_in)).astype(np.float32)
    ws = [_rand_weight(fmt, g, n, n_in) for n in n_outs]
    hs = upload_all(ws, [fmt] * len(n_outs), n_outs, n_in)
    whole = run(x, hs, n_outs)
    monkeypatch.setenv("IL_LAUNCH_ROWS", "320")  # launches of 300 + 17 | 129 | 256 + 64 | 200 rows
    split = run(x, hs, n_outs)
    for k, (a, b) in enumerate(zip(whole, split)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"job {k} differs when split"
    for w, n, y in zip(ws, n_outs, split):
        check_full(y, x, w, fmt, n, what=f"split fmt {fmt} t {t} n_out {n}")


def test_mixed_formats_one_call():
    g = np.random.default_rng(5)
    n_in = 256
    fmts = [Q4, BF16, Q8, BF16, Q4]
    n_outs = [64, 33, 100, 7, 512]
    for t in (1, 4, 40):
        say(f"[mixed] t={t}")
        x = g.standard_normal((t, n_in)).astype(np.float32)
        ws = [_rand_weight(f, g, n, n_in) for f, n in zip(fmts, n_outs)]
        hs = upload_all(ws, fmts, n_outs, n_in)
        ys = run(x, hs, n_outs)
        for f, w, n, y in zip(fmts, ws, n_outs, ys):
            check_full(y, x, w, f, n, what=f"mixed t {t} fmt {f}")


@pytest.mark.parametrize("t,path", [(2, "valu"), (2, "mfma"), (20, "verify"), (40, "gemm")])
def test_many_jobs_one_call(t, path, monkeypatch):
    """More jobs than one launch's job table holds, on every path."""
    _pin(monkeypatch, path)
    g = np.random.default_rng(6)
    n_in = 64
    n_outs = [3 + 5 * i for i in range(19)]
    x = g.standard_normal((t, n_in)).astype(np.float32)
    ws = [_rand_weight(BF16, g, n, n_in) for n in n_outs]
    hs = upload_all(ws, [BF16] * len(ws), n_outs, n_in)
    ys = run(x, hs, n_outs)
    for w, n, y in zip(ws, n_outs, ys):
        check_full(y, x, w, BF16, n, what=f"many jobs n_out {n}")


@pytest.mark.parametrize("fmt", [BF16, Q8, Q4], ids=lambda f: FMT_NAME[f])
@pytest.mark.parametrize("t", [2, 5, 8])
def test_mfma_decode_many_tiles(fmt, t, monkeypatch):
    """More 16-row tiles than workgroups (several tile groups per workgroup),
    a workgroup's tile range crossing from one job into the next, a ragged
    last tile, and a K range (33 blocks) that splits unevenly over the waves."""
    _pin(monkeypatch, "mfma")
    g = np.random.default_rng(1500 + 10 * t + fmt)
    n_in = 1056
    n_outs = [20000, 777, 31]
    say(f"[mfma tiles] fmt={FMT_NAME[fmt]} t={t} n_in={n_in} n_outs={n_outs}")
    x = g.standard_normal((t, n_in)).astype(np.float32)
    ws = [_rand_weight(fmt, g, n, n_in) for n in n_outs]
    hs = upload_all(ws, [fmt] * len(n_outs), n_outs, n_in)
    ys = run(x, hs, n_outs)
    for w, n, y in zip(ws, n_outs, ys):
        check_full(y, x, w, fmt, n, what=f"fmt {fmt} t {t} n_out {n}")


@pytest.mark.parametrize("fmt", [BF16, Q8, Q4], ids=lambda f: FMT_NAME[f])
@pytest.mark.parametrize("t", [9, 16, 17, 32, 33, 64, 100])
def test_verify_wide_many_tiles(fmt, t, monkeypatch):
    """Mid-size t on the matrix-core kernel's wide mode: one or two groups of
    16 tokens per weight operand (t > 32: slices of at most 32 tokens, one
    launch each), several chunks per workgroup, a job boundary inside a
    workgroup's range and ragged tiles and K."""
    _pin(monkeypatch, "verify")
    g = np.random.default_rng(1800 + 10 * t + fmt)
    n_in = 1056
    n_outs = [20000, 777, 31]
    say(f"[verify tiles] fmt={FMT_NAME[fmt]} t={t} n_in={n_in} n_outs={n_outs}")
    x = g.standard_normal((t, n_in)).astype(np.float32)
    ws = [_rand_weight(fmt, g, n, n_in) for n in n_outs]
    hs = upload_all(ws, [fmt] * len(n_outs), n_outs, n_in)
    ys = run(x, hs, n_outs)
    for w, n, y in zip(ws, n_outs, ys):
        check_full(y, x, w, fmt, n, what=f"fmt {fmt} t {t} n_out {n}")


@pytest.mark.parametrize("fmt", [BF16, Q8, Q4], ids=lambda f: FMT_NAME[f])
def test_gemm_full_rounds_and_tail(fmt):
    """Prefill with more 256 x 256 tiles than compute units: whole rounds of
    big tiles plus a tail run as 128 x 128 quarters, with ragged edges in t,
    in every job's n_out and in K (n_in = 96 is one and a half K steps)."""
    g = np.random.default_rng(1700 + fmt)
    t, n_in = 600, 96
    n_outs = [20000, 2000]
    say(f"[gemm rounds] fmt={FMT_NAME[fmt]} t={t} n_in={n_in} n_outs={n_outs}")
    x = g.standard_normal((t, n_in)).astype(np.float32)
    ws = [_rand_weight(fmt, g, n, n_in) for n in n_outs]
    hs = upload_all(ws, [fmt] * len(n_outs), n_outs, n_in)
    ys = run(x, hs, n_outs)
    for w, n, y in zip(ws, n_outs, ys):
        check_full(y, x, w, fmt, n, what=f"fmt {fmt} t {t} n_out {n}")


@pytest.mark.parametrize("fmt", [Q8, Q4], ids=lambda f: FMT_NAME[f])
def test_gemm_halves_and_quarters(fmt):
    """Quantised prefill with fewer 256 x 256 tiles than compute units:
    2 x 70 = 140 tiles run as a round of 256 x 128 halves (128 tiles) and the
    other 12 as 128 x 128 quarters; ragged edges in t and n_out."""
    g = np.random.default_rng(1760 + fmt)
    t, n_in = 300, 64
    n_outs = [17000, 700]
    say(f"[gemm halves] fmt={FMT_NAME[fmt]} t={t} n_in={n_in} n_outs={n_outs}")
    x = g.standard_normal((t, n_in)).astype(np.float32)
    ws = [_rand_weight(fmt, g, n, n_in) for n in n_outs]
    hs = upload_all(ws, [fmt] * len(n_outs), n_outs, n_in)
    ys = run(x, hs, n_outs)
    for w, n, y in zip(ws, n_outs, ys):
        check_full(y, x, w, fmt, n, what=f"fmt {fmt} t {t} n_out {n}")


@pytest.mark.parametrize("fmt", [BF16, Q8, Q4], ids=lambda f: FMT_NAME[f])
def test_gemm_unaligned_outputs(fmt):
    """Prefill epilogue: 16-byte stores only where a job's y rows are 16-byte
    aligned.  Job 0's y starts one float into its allocation, job 1 has
    n_out % 4 == 2, job 2 is aligned; the floats around job 0's y stay
    untouched."""
    import torch
    g = np.random.default_rng(1750 + fmt)
    t, n_in = 600, 64  # 3 x 89 tiles: a round of 256 x 256 tiles and quarters
    n_outs = [22001, 258, 64]
    say(f"[gemm unaligned] fmt={FMT_NAME[fmt]} t={t} n_in={n_in} n_outs={n_outs}")
    x = g.standard_normal((t, n_in)).astype(np.float32)
    ws = [_rand_weight(fmt, g, n, n_in) for n in n_outs]
    hs = upload_all(ws, [fmt] * len(n_outs), n_outs, n_in)
    buf = torch.full((t * n_outs[0] + 2,), 7.0, dtype=torch.float32, device="cuda")
    ys = [buf[1:1 + t * n_outs[0]].view(t, n_outs[0])]
    ys += [torch.full((t, n), float("nan"), dtype=torch.float32, device="cuda") for n in n_outs[1:]]
    xd = torch.from_numpy(x).cuda()
    assert il.il_matmul(xd, t, n_in, [(h, n, y) for h, n, y in zip(hs, n_outs, ys)]) == 1, il.il_last_error()
    torch.cuda.synchronize()
    edge = buf[[0, -1]].cpu().numpy()
    assert np.all(edge == 7.0), f"wrote outside y: {edge}"
    for w, n, y in zip(ws, n_outs, ys):
        check_full(y.cpu().numpy(), x, w, fmt, n, what=f"fmt {fmt} n_out {n}")


def test_concurrent_calls_from_threads():
    """Host threads share the weight handles and the library's context: each
    uploads and frees a weight of its own and runs repeated submissions (decode
    and prefill, all formats) on its own stream; every result equals the
    single-threaded one bit for bit (the kernels are deterministic)."""
    import threading
    import torch
    g = np.random.default_rng(77)
    n_in = 512
    fmts, n_outs = [BF16, Q8, Q4], [3000, 1500, 2200]
    ws = [_rand_weight(f, g, n, n_in) for f, n in zip(fmts, n_outs)]
    hs = upload_all(ws, fmts, n_outs, n_in)
    xs = {t: torch.from_numpy(g.standard_normal((t, n_in)).astype(np.float32)).cuda() for t in (1, 5, 40)}
    ref = {}
    for t, x in xs.items():
        ys = [torch.empty(t, n, device="cuda") for n in n_outs]
        assert il.il_matmul(x, t, n_in, list(zip(hs, n_outs, ys))) == 1, il.il_last_error()
        torch.cuda.synchronize()
        ref[t] = [y.cpu().numpy() for y in ys]
    n_threads, reps = 8, 10
    streams = [torch.cuda.Stream() for _ in range(n_threads)]
    errors = []

    def worker(k):
        try:
            extra = il.il_upload(_rand_weight(Q8, np.random.default_rng(k), 64, n_in), Q8, 64, n_in)
            assert extra is not None, il.il_last_error()
            out = {}
            with torch.cuda.stream(streams[k]):
                for r in range(reps):
                    for t, x in xs.items():
                        ys = [torch.empty(t, n, device="cuda") for n in n_outs]
                        if il.il_matmul(x, t, n_in, list(zip(hs, n_outs, ys)), streams[k]) != 1:
                            errors.append(f"thread {k}: {il.il_last_error()}")
                            return
                        out[(r, t)] = ys
            streams[k].synchronize()
            il.il_free(extra)
            for (r, t), ys in out.items():
                for j, y in enumerate(ys):
                    if not np.array_equal(y.cpu().numpy(), ref[t][j]):
                        errors.append(f"thread {k} rep {r} t {t} job {j} differs")
        except Exception as e:  # reported below
            errors.append(f"thread {k}: {e!r}")

    say(f"[threads] {n_threads} threads x {reps} reps x t in {sorted(xs)}")
    threads = [threading.Thread(target=worker, args=(k,)) for k in range(n_threads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=90)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors[:5]


# ----------------------------------------------------- closed forms on GPU
def _onehot(fmt, n_out, n_in, cols):
    if fmt == BF16:
        w = np.zeros((n_out, n_in), np.uint16)
        w[np.arange(n_out), cols] = 0x3F80
        return w
    nb = n_in // 32
    if fmt == Q8:
        c = np.zeros((n_out, n_in), np.int8)
        c[np.arange(n_out), cols] = 1
        return wl.encode_q8(c, np.ones((n_out, nb), np.float32))
    c = np.full((n_out, n_in), 8, np.uint8)
    c[np.arange(n_out), cols] = 9
    return wl.encode_q4(c, np.full((n_out, nb), 0x3C00, np.uint16))


@pytest.mark.parametrize("fmt", [BF16, Q8, Q4], ids=lambda f: FMT_NAME[f])
@pytest.mark.parametrize("t,path", _decode_cases([1, 3, 8, 9, 20, 200]))
def test_onehot_selects_columns(fmt, t, path, monkeypatch):
    """One-hot W: y[:, r] = x[:, c_r] exactly on the f32 decode path and
    bf16(x) (round to nearest even) on the matrix-core paths (decode, verify
    and GEMM)."""
    _pin(monkeypatch, path)
    g = np.random.default_rng(20 + t)
    n_in, n_out = 320, 300
    cols = g.integers(0, n_in, n_out)
    x = g.standard_normal((t, n_in)).astype(np.float32)
    (h,) = upload_all([_onehot(fmt, n_out, n_in, cols)], [fmt], [n_out], n_in)
    (y,) = run(x, [h], [n_out])
    assert np.array_equal(y, _selected(x, path)[:, cols])


@pytest.mark.parametrize("t,path", _decode_cases([2, 64]))
def test_identity(t, path, monkeypatch):
    _pin(monkeypatch, path)
    g = np.random.default_rng(30)
    n = 256
    x = g.standard_normal((t, n)).astype(np.float32)
    for fmt in (BF16, Q8, Q4):
        (h,) = upload_all([_onehot(fmt, n, n, np.arange(n))], [fmt], [n], n)
        (y,) = run(x, [h], [n])
        assert np.array_equal(y, _selected(x, path)), f"identity fmt {fmt}"


@pytest.mark.parametrize("t,path", _decode_cases([1, 5, 70]))
def test_zero_codes_give_exact_zeros(t, path, monkeypatch):
    _pin(monkeypatch, path)
    g = np.random.default_rng(40)
    n_out, n_in = 96, 512
    nb = n_in // 32
    x = g.standard_normal((t, n_in)).astype(np.float32)
    z4 = wl.encode_q4(np.full((n_out, n_in), 8, np.uint8),
                      g.integers(0x1000, 0x5000, (n_out, nb)).astype(np.uint16))
    z8 = wl.encode_q8(np.zeros((n_out, n_in), np.int8), g.uniform(0.1, 10, (n_out, nb)).astype(np.float32))
    hs = upload_all([z4, z8], [Q4, Q8], [n_out, n_out], n_in)
    for y in run(x, hs, [n_out, n_out]):
        assert np.all(y == 0)


@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_row_sums_with_x_one(path, monkeypatch):
    """x = 1: y[r] = sum_k w[r][k]; Q4 codes k % 16 give -16 per block."""
    _pin(monkeypatch, path)
    n_out, n_in = 40, 1024
    nb = n_in // 32
    k = np.arange(n_in)
    codes = np.tile((k % 16).astype(np.uint8), (n_out, 1))
    sbits = np.array([[(15 - (r % 10)) << 10] * nb for r in range(n_out)], np.uint16)
    (h,) = upload_all([wl.encode_q4(codes, sbits)], [Q4], [n_out], n_in)
    for t in (1, 16):
        (y,) = run(np.ones((t, n_in), np.float32), [h], [n_out])
        want = np.array([-16.0 * nb * 2.0 ** -(r % 10) for r in range(n_out)], np.float32)
        assert np.array_equal(y, np.tile(want, (t, 1)))


# ------------------------------------------------------------- invariants
@pytest.mark.parametrize("t,path", _decode_cases([1, 4, 8, 24, 300]))
def test_deterministic_and_batch_invariant(t, path, monkeypatch):
    _pin(monkeypatch, path)
    g = np.random.default_rng(50 + t)
    n_in = 1024
    n_outs = [512, 130, 96]
    fmts = [Q4, Q4, Q8]
    x = g.standard_normal((t, n_in)).astype(np.float32)
    ws = [_rand_weight(f, g, n, n_in) for f, n in zip(fmts, n_outs)]
    hs = upload_all(ws, fmts, n_outs, n_in)
    a = run(x, hs, n_outs)
    b = run(x, hs, n_outs)
    alone = run(x, hs[:1], n_outs[:1])
    for ya, yb in zip(a, b):
        assert np.array_equal(ya, yb), "not bitwise reproducible"
    assert np.array_equal(a[0], alone[0]), "result depends on the other jobs in the batch"


@pytest.mark.parametrize("t,path", _decode_cases([2, 96]))
def test_power_of_two_scaling(t, path, monkeypatch):
    _pin(monkeypatch, path)
    g = np.random.default_rng(60)
    n_in, n_out = 512, 256
    x = g.standard_normal((t, n_in)).astype(np.float32)
    for fmt in (BF16, Q8, Q4):
        (h,) = upload_all([_rand_weight(fmt, g, n_out, n_in)], [fmt], [n_out], n_in)
        (y1,) = run(x, [h], [n_out])
        (y2,) = run(x * np.float32(8.0), [h], [n_out])
        assert np.array_equal(y2, y1 * np.float32(8.0)), f"fmt {fmt}"


@pytest.mark.parametrize("t,path", _decode_cases([3, 20]))
def test_writes_exactly_y(t, path, monkeypatch):
    """Every y element is written (NaN sentinel gone) and nothing around y is
    (guard bands of a larger buffer keep their canary value)."""
    import torch
    _pin(monkeypatch, path)
    g = np.random.default_rng(70)
    n_in, n_out = 256, 333
    x_np = g.standard_normal((t, n_in)).astype(np.float32)
    (h,) = upload_all([_rand_weight(Q4, g, n_out, n_in)], [Q4], [n_out], n_in)
    pad = 4096
    buf = torch.full((pad + t * n_out + pad,), 12345.0, dtype=torch.float32, device="cuda")
    y = buf[pad:pad + t * n_out]
    y.fill_(float("nan"))
    x = torch.from_numpy(x_np).cuda()
    assert il.il_matmul(x, t, n_in, [(h, n_out, y)]) == 1, il.il_last_error()
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.all(b[:pad] == 12345.0) and np.all(b[pad + t * n_out:] == 12345.0)
    assert np.all(np.isfinite(b[pad:pad + t * n_out]))


# -------------------------------------------------------- validation on GPU
def test_validation_leaves_y_untouched():
    import torch
    g = np.random.default_rng(80)
    n_in, n_out, t = 64, 32, 2
    (h,) = upload_all([_rand_weight(BF16, g, n_out, n_in)], [BF16], [n_out], n_in)
    (h2,) = upload_all([_rand_weight(BF16, g, n_out, 96)], [BF16], [n_out], 96)
    x_host = g.standard_normal((t, n_in)).astype(np.float32)
    x = torch.from_numpy(x_host).cuda()
    y = torch.full((t, n_out), 7.0, device="cuda")
    y2 = torch.full((t, n_out), 7.0, device="cuda")
    cases = {
        "host x": (x_host.ctypes.data, [(h, n_out, y)]),
        "wrong n_in": (x, [(h2, n_out, y)]),
        "wrong n_out": (x, [(h, n_out + 1, y)]),
        "null weight": (x, [(None, n_out, y)]),
        "overlapping y": (x, [(h, n_out, y), (h, n_out, y)]),
        "y is x": (x, [(h, n_out, x)]),
        "bad second job": (x, [(h, n_out, y), (h2, n_out, y2)]),
    }
    for what, (xx, jobs) in cases.items():
        say(f"[validation] {what}")
        assert il.il_matmul(xx, t, n_in, jobs) == 0, what
        assert il.il_last_error(), what
        torch.cuda.synchronize()
        assert torch.all(y == 7.0) and torch.all(y2 == 7.0), f"{what}: y was written"


def test_upload_roundtrip_is_handle_metadata():
    g = np.random.default_rng(90)
    for fmt, n_out, n_in in ((BF16, 10, 64), (Q8, 7, 96), (Q4, 5, 128)):
        w = _rand_weight(fmt, g, n_out, n_in)
        (h,) = upload_all([w], [fmt], [n_out], n_in)
        assert h.bytes == wl.weight_bytes(fmt, n_out, n_in) == w.nbytes
