"""HIP-graph capture of every path through the C ABI.

Each case runs once eagerly (checked against the oracle), then the same
calls are captured into a graph (torch.cuda.CUDAGraph) and the graph is
replayed several times.  Between the replays the outputs are refilled with
NaN and the program does its own eager work (more library calls into other
buffers, torch kernels) and synchronises.  Every path is deterministic, so
every replay must reproduce the eager outputs bit for bit.  The paths that
take stream-ordered scratch inside a call (the x pre-pass of the mid-size
and prefill paths, the LM head without a caller workspace) record
allocation nodes in the graph; none records a memset.
"""
import numpy as np
import pytest

import oracle
import quantized_weight_matmul_amd as il
from quantized_weight_matmul_amd import workloads as wl
from conftest import gpu_available
from gpu_util import check_full, check_sampled, say, upload_all

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

BF16, Q8, Q4 = il.IL_BF16, il.IL_Q8, il.IL_Q4
REPLAYS = 3


def _rand_weight(fmt, g, n_out, n_in):
    nb = n_in // 32
    if fmt == BF16:
        return wl.f32_to_bf16_bits((g.standard_normal((n_out, n_in)) * 0.02).astype(np.float32))
    if fmt == Q8:
        return wl.encode_q8(g.integers(-127, 128, (n_out, n_in)).astype(np.int8),
                            g.uniform(1e-4, 1e-3, (n_out, nb)).astype(np.float32))
    return wl.encode_q4(g.integers(0, 16, (n_out, n_in)).astype(np.uint8),
                        g.uniform(1e-3, 1e-2, (n_out, nb)).astype(np.float16).view(np.uint16))


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def _replay_and_compare(graph, outs, eager, between):
    """Replay `graph` REPLAYS times; before each, refill `outs` with NaN and
    run `between()` (eager work); after each, compare with `eager` bitwise."""
    import torch
    for rep in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan")) if o.dtype == torch.float32 else o.fill_(-7)
        between()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert np.array_equal(_bits(o.cpu().numpy()), _bits(e)), f"replay {rep}: output {i} differs from eager"


# (id, fmt, t, n_in, n_outs, env pins): both decode families, the two-rows-
# per-wave long rows, the matrix-core mid-size kernel without and with the
# x pre-pass and in slices, GEMM halves, whole rounds of big tiles plus
# quarters, and the mid-size plan with its last round split over K (272
# units: three launches, chunk sums in the stream's scratch)
CASES = [
    ("bf16-valu-t1", BF16, 1, 1024, [512, 300], {"IL_DECODE": "valu"}),
    ("q8-valu-t3-long-rows", Q8, 3, 8192, [40, 17], {"IL_DECODE": "valu"}),
    ("q4-mfma-t2", Q4, 2, 1024, [700, 33], {"IL_DECODE": "mfma"}),
    ("q8-mfma-t8", Q8, 8, 512, [300], {"IL_DECODE": "mfma"}),
    ("q4-verify-t16", Q4, 16, 1024, [500], {"IL_PREFILL": "verify"}),
    ("bf16-verify-t24", BF16, 24, 512, [300, 65], {"IL_PREFILL": "verify"}),
    ("q4-verify-slices-t70", Q4, 70, 512, [300], {"IL_PREFILL": "verify"}),
    ("q8-gemm-halves-t40", Q8, 40, 512, [700], {"IL_PREFILL": "tiles"}),
    ("q4-mid-split-t100", Q4, 100, 256, [17408, 17408], {}),
    ("q8-mid-split-t64", Q8, 64, 288, [17408, 17408], {}),
    ("q4-gemm-t300", Q4, 300, 256, [1000, 129], {}),
    ("bf16-gemm-rounds-t600", BF16, 600, 256, [22016], {}),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_matmul_graph_replays(case, monkeypatch):
    import torch
    name, fmt, t, n_in, n_outs, env = case
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    say(f"[graph] {name} t={t} n_in={n_in} n_outs={n_outs}")
    g = np.random.default_rng(sum(map(ord, name)))
    x_np = g.standard_normal((t, n_in)).astype(np.float32)
    ws = [_rand_weight(fmt, g, n, n_in) for n in n_outs]
    hs = upload_all(ws, [fmt] * len(n_outs), n_outs, n_in)
    x = torch.from_numpy(x_np).cuda()
    ys = [torch.full((t, n), float("nan"), device="cuda") for n in n_outs]
    assert il.il_matmul(x, t, n_in, list(zip(hs, n_outs, ys))) == 1, il.il_last_error()
    torch.cuda.synchronize()
    eager = [y.cpu().numpy() for y in ys]
    for w, n, y in zip(ws, n_outs, eager):
        if t * n <= 1 << 20:
            check_full(y, x_np, w, fmt, n, what=f"{name} eager n_out {n}")
        else:
            check_sampled(y, x_np, w, fmt, n, what=f"{name} eager n_out {n}")

    # two calls per graph, into two sets of outputs
    ys2 = [torch.full((t, n), float("nan"), device="cuda") for n in n_outs]
    others = [torch.empty((t, n), device="cuda") for n in n_outs]
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        assert il.il_matmul(x, t, n_in, list(zip(hs, n_outs, ys))) == 1, il.il_last_error()
        assert il.il_matmul(x, t, n_in, list(zip(hs, n_outs, ys2))) == 1, il.il_last_error()

    def between():
        assert il.il_matmul(x, t, n_in, list(zip(hs, n_outs, others))) == 1, il.il_last_error()
        (x * 3.0).sum()

    _replay_and_compare(graph, ys + ys2, eager + eager, between)
    for o, e in zip(others, eager):  # the eager calls between replays are right too
        assert np.array_equal(_bits(o.cpu().numpy()), _bits(e))


@pytest.mark.parametrize("fmt,t,env", [(BF16, 1, {}), (Q4, 2, {}), (Q8, 5, {"IL_DECODE": "mfma"}),
                                       (Q4, 20, {}), (BF16, 64, {"IL_PREFILL": "gemm"})],
                         ids=["bf16-t1", "q4-t2", "q8-t5-mfma", "q4-t20", "bf16-t64-gemm"])
def test_gelu_mul_graph_replays(fmt, t, env, monkeypatch):
    import torch
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    n_in, n_out = 512, 333
    say(f"[graph] gelu_mul fmt={fmt} t={t}")
    g = np.random.default_rng(77 + 10 * t + fmt)
    x_np = g.standard_normal((t, n_in)).astype(np.float32)
    G, U = _rand_weight(fmt, g, n_out, n_in), _rand_weight(fmt, g, n_out, n_in)
    hg, hu = upload_all([G, U], [fmt, fmt], [n_out, n_out], n_in)
    x = torch.from_numpy(x_np).cuda()
    y = torch.full((t, n_out), float("nan"), device="cuda")
    assert il.il_matmul_gelu_mul(x, t, n_in, hg, hu, n_out, y) == 1, il.il_last_error()
    torch.cuda.synchronize()
    eager = y.cpu().numpy()
    y_ref, bound = oracle.gelu_mul(x_np, G, U, fmt, n_out)
    r = oracle.check(eager, y_ref, bound)
    assert r["ok"], f"gelu_mul eager: {r['bad']}/{r['n']} outside tolerance"

    other = torch.empty_like(y)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        assert il.il_matmul_gelu_mul(x, t, n_in, hg, hu, n_out, y) == 1, il.il_last_error()

    def between():
        assert il.il_matmul_gelu_mul(x, t, n_in, hg, hu, n_out, other) == 1, il.il_last_error()
        (x - 1.0).abs().max()

    _replay_and_compare(graph, [y], [eager], between)


@pytest.mark.parametrize("workspace", [False, True], ids=["stream-ordered-scratch", "caller-workspace"])
def test_lm_head_graph_replays(workspace):
    """Integer inputs: the eager call equals the oracle exactly; replays
    equal the eager call bitwise."""
    import torch
    t, h, n_c, per, k = 2, 64, 100, 3, 10
    say(f"[graph] lm_head workspace={workspace}")
    rng = np.random.default_rng(4242)
    vocab = n_c * per
    to_bf = lambda a: wl.f32_to_bf16_bits(a.astype(np.float32))
    x_np = rng.integers(-3, 4, (t, h)).astype(np.float32)
    cen = to_bf(rng.integers(-2, 3, (n_c, h)))
    emb = to_bf(rng.integers(-2, 3, (vocab, h)))
    order = rng.permutation(vocab).astype(np.uint32)
    ref = oracle.centroid_argmax(x_np, cen, emb, order, k)
    hc = il.il_upload(cen, il.IL_BF16, n_c, h)
    he = il.il_upload(emb, il.IL_BF16, vocab, h)
    assert hc is not None and he is not None, il.il_last_error()
    x = torch.from_numpy(x_np).cuda()
    od = torch.from_numpy(order.view(np.int32)).cuda()
    tok = torch.full((t,), -7, dtype=torch.int32, device="cuda")
    clu = torch.full((t, k), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((t,), float("nan"), device="cuda")
    ws = None
    if workspace:
        ws = torch.full((il.il_centroid_argmax_workspace(t, n_c, k) // 4,), float("nan"), device="cuda")
    call = lambda a, b, c: il.il_centroid_argmax(x, t, h, hc, he, od, k, a, b, c, workspace=ws)
    assert call(tok, clu, sc) == 1, il.il_last_error()
    torch.cuda.synchronize()
    eager = [tok.cpu().numpy(), clu.cpu().numpy(), sc.cpu().numpy()]
    assert np.array_equal(eager[0], ref["token"]) and np.array_equal(eager[1], ref["clusters"])
    assert np.array_equal(eager[2], ref["score"])

    o_tok, o_clu, o_sc = torch.empty_like(tok), torch.empty_like(clu), torch.empty_like(sc)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        assert call(tok, clu, sc) == 1, il.il_last_error()

    def between():
        # with a caller workspace this eager call reuses the graph's scratch;
        # it runs to completion before the next replay starts
        assert call(o_tok, o_clu, o_sc) == 1, il.il_last_error()

    _replay_and_compare(graph, [tok, clu, sc], eager, between)
    assert np.array_equal(o_tok.cpu().numpy(), eager[0])
