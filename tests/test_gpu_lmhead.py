"""GPU parity of the centroid-masked LM head (il_centroid_argmax).

Integer-valued inputs make every logit and score exact in f32 whatever the
summation order, so there the GPU must reproduce the oracle's clusters,
token and score exactly, ties included (equal logits by increasing index,
first maximum in visiting order).  On real-valued inputs several answers can
be correct where logits or scores are closer than their rounding; the test
then checks that the GPU's answer is one of them: its clusters are a top-k
and its token the first maximum under some perturbation of every logit and
score within 4e-3 of its sum |x*w| (and equal to the oracle's wherever the
oracle's margins exceed that).
"""
import numpy as np
import pytest

import oracle
import quantized_weight_matmul_amd as il
from quantized_weight_matmul_amd import workloads as wl
from conftest import gpu_available
from gpu_util import say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

TOL = 4e-3


def _run(x, cen, emb, order, k, workspace=False, k_out=None):
    """k_out: columns of the clusters output (min(k, C), the clusters visited)."""
    import torch
    t, h = x.shape
    n_c, vocab = cen.shape[0], emb.shape[0]
    k_out = k if k_out is None else k_out
    hc = il.il_upload(cen, il.IL_BF16, n_c, h)
    he = il.il_upload(emb, il.IL_BF16, vocab, h)
    assert hc is not None and he is not None, il.il_last_error()
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    od = torch.from_numpy(order.view(np.int32)).cuda()
    tok = torch.full((t,), -7, dtype=torch.int32, device="cuda")
    clu = torch.full((t, k_out), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((t,), np.nan, dtype=torch.float32, device="cuda")
    ws = None
    if workspace:  # caller-owned scratch, filled with junk first
        nb = il.il_centroid_argmax_workspace(t, n_c, k)
        ws = torch.full((nb // 4,), float("nan"), dtype=torch.float32, device="cuda")
    assert il.il_centroid_argmax(xd, t, h, hc, he, od, k, tok, clu, sc, workspace=ws) == 1, il.il_last_error()
    torch.cuda.synchronize()
    return tok.cpu().numpy(), clu.cpu().numpy(), sc.cpu().numpy()


def _ints(rng, shape, lo, hi):
    return rng.integers(lo, hi + 1, shape)


@pytest.mark.parametrize("t,h,n_c,per,k", [(1, 32, 8, 4, 1), (1, 64, 16, 8, 4), (3, 96, 12, 5, 12),
                                           (8, 256, 64, 16, 8), (2, 128, 100, 3, 33), (1, 256, 2048, 4, 32),
                                           (1, 64, 64, 2, 64), (2, 64, 300, 2, 100), (1, 32, 129, 1, 129),
                                           (1, 64, 30000, 1, 3)])
def test_lm_head_exact_on_integer_inputs(t, h, n_c, per, k):
    say(f"[lm_head] integers t={t} h={h} C={n_c} per={per} k={k}")
    rng = np.random.default_rng(h + n_c + k)
    vocab = n_c * per
    x = _ints(rng, (t, h), -3, 3)
    cen = _ints(rng, (n_c, h), -2, 2)
    emb = _ints(rng, (vocab, h), -2, 2)
    cen[1] = cen[0]
    cen[n_c - 1] = cen[0]  # equal logits
    emb[:: max(1, vocab // 7)] = emb[3]  # many equal scores
    order = rng.permutation(vocab).astype(np.uint32)
    to_bf = lambda a: wl.f32_to_bf16_bits(a.astype(np.float32))
    ref = oracle.centroid_argmax(x.astype(np.float32), to_bf(cen), to_bf(emb), order, k)
    for ws in (False, True):
        tok, clu, sc = _run(x.astype(np.float32), to_bf(cen), to_bf(emb), order, k, workspace=ws)
        assert np.array_equal(clu, ref["clusters"]), f"clusters (workspace={ws})"
        assert np.array_equal(tok, ref["token"]), f"token (workspace={ws})"
        assert np.array_equal(sc, ref["score"]), f"score (workspace={ws})"


def _check_valid(x, cen, emb, order, k, tok, clu, sc):
    """The GPU's answer is a correct one within the tolerance of every sum."""
    ref = oracle.centroid_argmax(x, cen, emb, order, k)
    t = x.shape[0]
    n_c, vocab = cen.shape[0], emb.shape[0]
    per = vocab // n_c
    for i in range(t):
        cl, eps = ref["cl"][i], TOL * ref["cl_bound"][i]
        sel = clu[i]
        assert len(set(sel.tolist())) == k and sel.min() >= 0 and sel.max() < n_c, "clusters malformed"
        rest = np.setdiff1d(np.arange(n_c), sel)
        if rest.size:
            assert (cl[sel] + eps[sel]).min() >= (cl[rest] - eps[rest]).max(), "not a top-k selection"
        lo, hi = cl[sel] - eps[sel], cl[sel] + eps[sel]
        assert np.all(hi[:-1] >= lo[1:]), "visiting order not by decreasing logit"
        cand = np.concatenate([order[c * per:(c + 1) * per] for c in sel])
        exact = np.array([oracle.token_score(x[i], emb, int(c)) for c in cand])
        s, b = exact[:, 0], TOL * exact[:, 1]
        assert tok[i] in cand, "token not among the chosen clusters' tokens"
        j = int(np.flatnonzero(cand == tok[i])[0])
        assert s[j] + b[j] >= (s - b).max(), "token is not a maximum within tolerance"
        assert abs(sc[i] - s[j]) <= b[j], "reported score"
        if np.array_equal(sel, ref["clusters"][i]):
            srt = np.sort(s)
            if srt[-1] - srt[-2] > 2 * b.max():
                assert tok[i] == ref["token"][i], "clear winner missed"


@pytest.mark.parametrize("t,h,n_c,per,k", [(1, 64, 32, 8, 4), (4, 256, 256, 16, 16), (8, 128, 1000, 2, 50)])
def test_lm_head_valid_on_real_inputs(t, h, n_c, per, k):
    say(f"[lm_head] real t={t} h={h} C={n_c} per={per} k={k}")
    rng = np.random.default_rng(7 * h + n_c)
    vocab = n_c * per
    x = rng.standard_normal((t, h)).astype(np.float32)
    cen = wl.f32_to_bf16_bits((rng.standard_normal((n_c, h)) * 0.02).astype(np.float32))
    emb = wl.f32_to_bf16_bits((rng.standard_normal((vocab, h)) * 0.02).astype(np.float32))
    order = rng.permutation(vocab).astype(np.uint32)
    tok, clu, sc = _run(x, cen, emb, order, k)
    _check_valid(x, cen, emb, order, k, tok, clu, sc)


def test_lm_head_workload_full():
    name = "f4_lmhead_t1"
    h, n_c, k, vocab, t, cfg = wl.LM_HEAD[name]
    say(f"[lm_head] {name}: h={h} C={n_c} k={k} V={vocab}")
    x, cen, emb, order = wl.make_lm_head_inputs(name)
    tok, clu, sc = _run(x, cen, emb, order, k, workspace=True)
    _check_valid(x, cen, emb, order, k, tok, clu, sc)


def test_lm_head_top_k_above_clusters():
    """top_k above C takes every cluster (Drafter::step: k =
    top_k_centroids.min(num_centroids)); the result equals top_k = C and the
    oracle's, exactly (integer inputs)."""
    rng = np.random.default_rng(11)
    t, h, n_c, per = 2, 64, 12, 5
    vocab = n_c * per
    to_bf = lambda a: wl.f32_to_bf16_bits(a.astype(np.float32))
    x = _ints(rng, (t, h), -3, 3).astype(np.float32)
    cen, emb = to_bf(_ints(rng, (n_c, h), -2, 2)), to_bf(_ints(rng, (vocab, h), -2, 2))
    order = rng.permutation(vocab).astype(np.uint32)
    ref = oracle.centroid_argmax(x, cen, emb, order, n_c)
    for k in (n_c, n_c + 1, 100):
        say(f"[lm_head] top_k={k} C={n_c}")
        tok, clu, sc = _run(x, cen, emb, order, k, k_out=min(k, n_c), workspace=True)
        assert np.array_equal(clu, ref["clusters"]) and np.array_equal(tok, ref["token"]), f"top_k={k}"
        assert np.array_equal(sc, ref["score"]), f"top_k={k}"


def test_lm_head_skips_out_of_range_ordering_and_rejects_bad_calls():
    import torch
    rng = np.random.default_rng(3)
    h, n_c, per, k = 64, 8, 4, 2
    vocab = n_c * per
    x = rng.standard_normal((1, h)).astype(np.float32)
    cen = wl.f32_to_bf16_bits(rng.standard_normal((n_c, h)).astype(np.float32))
    emb = wl.f32_to_bf16_bits(rng.standard_normal((vocab, h)).astype(np.float32))
    bad = np.full(vocab, vocab + 5, dtype=np.uint32)  # every entry out of range
    tok, clu, sc = _run(x, cen, emb, bad, k)
    assert tok[0] == -1, "a row with no valid candidate reports -1"
    hc = il.il_upload(cen, il.IL_BF16, n_c, h)
    he = il.il_upload(emb, il.IL_BF16, vocab, h)
    hq = il.il_upload(wl.gen_weight(il.IL_Q8, 1, 1, n_c, h), il.IL_Q8, n_c, h)
    xd = torch.from_numpy(x).cuda()
    od = torch.zeros(vocab, dtype=torch.int32, device="cuda")
    out = torch.full((1,), 9, dtype=torch.int32, device="cuda")
    assert il.il_centroid_argmax(xd, 1, h, hc, he, od, 0, out) == 0 and "top_k" in il.il_last_error()
    assert il.il_centroid_argmax(xd, 1, h, hq, he, od, 1, out) == 0 and "bf16" in il.il_last_error()
    assert il.il_centroid_argmax(xd, 1, h, he, hc, od, 1, out) == 0 and "multiple" in il.il_last_error()
    big = il.il_upload(np.zeros((40000, h), np.uint16), il.IL_BF16, 40000, h)  # (40000 + h + 2) * 4 > 152 KiB
    assert il.il_centroid_argmax(xd, 1, h, big, big, od, 1, out) == 0 and "LDS" in il.il_last_error()
    small = torch.zeros(il.il_centroid_argmax_workspace(1, n_c, 2) // 4 - 1, dtype=torch.float32, device="cuda")
    assert il.il_centroid_argmax(xd, 1, h, hc, he, od, 2, out, workspace=small) == 0
    assert "workspace" in il.il_last_error()
    torch.cuda.synchronize()
    assert out.item() == 9, "rejected calls write nothing"
