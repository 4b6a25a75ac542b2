"""Pins for the CPU oracle: checks of ``oracle`` against things other than itself.

Every function takes an ``oracle.Oracle`` (the real library, or a planted
mutant in ``test_oracle_mutants.py``) and raises AssertionError when the
oracle disagrees with:

* library casts (torch bfloat16, numpy float16/float32) on every bit pattern;
* exact rational arithmetic (``fractions.Fraction``) on tiny shapes;
* closed forms: one-hot / identity W selects columns of x, x = 1 gives row
  sums, all-zero codes give 0, Q8/Q4 codes round-trip through dequantisation;
* hand-derived fixtures in ``tests/golden`` (the storage-format readings);
* numpy float64 ``x @ W.T`` on library-decoded weights at the workloads' shapes.

The method pinned is y[t][n_out] = x[t][n_in] * W^T of the oxinfer 0.0.0
``src/gpu.rs`` page (doc comment of ``struct Job``), with W stored in one of
the formats of ``enum WeightRef`` on that page.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

import oracle as O_mod
from quantized_weight_matmul_amd import workloads as wl

BF16, Q8, Q4 = O_mod.BF16, O_mod.Q8, O_mod.Q4
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
FMTS = {"bf16": BF16, "q8": Q8, "q4": Q4}


# ------------------------------------------------------------ library decodes
def lib_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bits -> float64 via torch's bfloat16 dtype."""
    import torch
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


def lib_f16(bits: np.ndarray) -> np.ndarray:
    """binary16 bits -> float64 via numpy's float16 dtype."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def lib_q8_values(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """float32(q) * float32(scale) with numpy's IEEE f32 multiply."""
    n_out, n_in = codes.shape
    s = np.repeat(scales.astype(np.float32), wl.BLOCK, axis=1)
    return codes.astype(np.float32) * s


def lib_q4_values(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    s = np.repeat(lib_f16(scale_bits), wl.BLOCK, axis=1)
    return ((codes.astype(np.float64) - 8.0) * s).astype(np.float32)


def _nan_equal(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    both_nan = np.isnan(a) & np.isnan(b)
    same = (a == b) & (np.signbit(a) == np.signbit(b))
    return bool(np.all(both_nan | same))


# --------------------------------------------------------------- decoders
def pin_bf16_exhaustive(O):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    assert _nan_equal(O.bf16_value(bits), lib_bf16(bits)), "bf16 decode disagrees with torch"


def pin_f16_exhaustive(O):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    assert _nan_equal(O.f16_value(bits), lib_f16(bits)), "f16 decode disagrees with numpy"


# ----------------------------------------------------------------- goldens
def load_golden(path):
    fields = {}
    wb = []
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, _, val = line.partition(" ")
            if key == "weight_bytes":
                wb.append(val.replace(" ", ""))
            else:
                fields[key] = val.strip()
    fmt = FMTS[fields["fmt"]]
    n_out, n_in = int(fields["n_out"]), int(fields["n_in"])
    if fmt == BF16:
        weight = np.array([int(h, 16) for h in fields["weight_u16"].split()], dtype=np.uint16)
    else:
        weight = np.frombuffer(bytes.fromhex("".join(wb)), dtype=np.uint8).copy()
    if fields["x"] == "ones":
        x = np.ones((1, n_in), dtype=np.float32)
    else:
        x = np.array([[float(v) for v in row.split(",")] for row in fields["x"].split(";")],
                     dtype=np.float32)
    y = np.array([[float(v) for v in row.split(",")] for row in fields["y"].split(";")])
    closed = np.array(eval(fields["closed_form"], {"__builtins__": {}},
                           {"sum": sum, "range": range}), dtype=np.float64)
    return fmt, n_out, n_in, weight, x, y, closed


def golden_files():
    return sorted(f for f in os.listdir(GOLDEN) if f.endswith(".txt"))


def pin_goldens(O):
    files = golden_files()
    assert len(files) >= 7
    for name in files:
        fmt, n_out, n_in, weight, x, y, closed = load_golden(os.path.join(GOLDEN, name))
        assert np.array_equal(y.ravel(), closed), f"{name}: stored y is not its closed form"
        got, bound = O.matmul(x, weight, fmt, n_out)
        assert got.shape == y.shape, name
        assert np.array_equal(got.astype(np.float64), y), f"{name}: oracle {got} != {y}"


# ------------------------------------------------------------ closed forms
def _onehot_weight(fmt, n_out, n_in, cols):
    """W[r][cols[r]] = 1, every other element 0, in each host format; built
    from the encodings of 1 and 0 directly (no decoding involved)."""
    if fmt == BF16:
        w = np.zeros((n_out, n_in), dtype=np.uint16)
        w[np.arange(n_out), cols] = 0x3F80  # 1.0
        return w
    nb = n_in // wl.BLOCK
    if fmt == Q8:
        codes = np.zeros((n_out, n_in), dtype=np.int8)
        codes[np.arange(n_out), cols] = 64
        scales = np.full((n_out, nb), 2.0 ** -6, dtype=np.float32)  # 64 * 2^-6 = 1
        return wl.encode_q8(codes, scales)
    codes = np.full((n_out, n_in), 8, dtype=np.uint8)  # code 8 -> value 0
    codes[np.arange(n_out), cols] = 9  # (9 - 8) * 1.0
    return wl.encode_q4(codes, np.full((n_out, nb), 0x3C00, dtype=np.uint16))


def pin_onehot(O):
    rng = np.random.default_rng(7)
    n_out, n_in, t = 7, 64, 3
    x = rng.standard_normal((t, n_in)).astype(np.float32)
    for fmt in (BF16, Q8, Q4):
        cols = rng.integers(0, n_in, n_out)
        w = _onehot_weight(fmt, n_out, n_in, cols)
        y, bound = O.matmul(x, w, fmt, n_out)
        assert np.array_equal(y, x[:, cols]), f"one-hot fmt {fmt}"
        assert np.array_equal(bound, np.abs(x[:, cols]).astype(np.float64)), f"one-hot bound {fmt}"


def pin_identity(O):
    rng = np.random.default_rng(8)
    n = 64
    x = rng.standard_normal((2, n)).astype(np.float32)
    for fmt in (BF16, Q8, Q4):
        y, _ = O.matmul(x, _onehot_weight(fmt, n, n, np.arange(n)), fmt, n)
        assert np.array_equal(y, x), f"identity fmt {fmt}"


def pin_row_sums(O):
    """x = 1 gives y[r] = sum_k w[r][k]; codes chosen so the sums are closed forms."""
    n_out, n_in = 5, 96
    nb = n_in // wl.BLOCK
    x = np.ones((1, n_in), dtype=np.float32)
    k = np.arange(n_in)
    # Q4: code k % 16 in every row; per block sum(code - 8) = 2 * (-8) = -16.
    # Row r has scale 2^-r (f16 bits (15 - r) << 10), so y[r] = -16 * nb * 2^-r.
    codes = np.tile((k % 16).astype(np.uint8), (n_out, 1))
    sbits = np.array([[(15 - r) << 10] * nb for r in range(n_out)], dtype=np.uint16)
    y, _ = O.matmul(x, wl.encode_q4(codes, sbits), Q4, n_out)
    assert np.array_equal(y[0], np.array([-16.0 * nb * 2.0 ** -r for r in range(n_out)])), "q4 sums"
    # Q8: code (k % 32) - 16 -> per block sum = -16; row scale r + 1 -> y = -16 nb (r + 1).
    codes8 = np.tile(((k % 32) - 16).astype(np.int8), (n_out, 1))
    sc = np.array([[r + 1.0] * nb for r in range(n_out)], dtype=np.float32)
    y, _ = O.matmul(x, wl.encode_q8(codes8, sc), Q8, n_out)
    assert np.array_equal(y[0], np.array([-16.0 * nb * (r + 1) for r in range(n_out)])), "q8 sums"
    # bf16: w[r][k] = 2^-(k % 4) * (+1 if r even else -1); row sum = +-nb*32/4 * (1+.5+.25+.125)
    vals = np.array([0x3F80, 0x3F00, 0x3E80, 0x3E00], dtype=np.uint16)  # 1, 1/2, 1/4, 1/8
    w = np.tile(vals[k % 4], (n_out, 1))
    w[1::2] |= 0x8000
    y, _ = O.matmul(x, w, BF16, n_out)
    want = np.array([(n_in // 4) * 1.875 * (1 if r % 2 == 0 else -1) for r in range(n_out)])
    assert np.array_equal(y[0], want), "bf16 sums"


def pin_zero_codes(O):
    rng = np.random.default_rng(9)
    n_out, n_in = 4, 64
    nb = n_in // wl.BLOCK
    x = rng.standard_normal((3, n_in)).astype(np.float32)
    z4 = wl.encode_q4(np.full((n_out, n_in), 8, np.uint8),
                      rng.integers(0x1000, 0x5000, (n_out, nb)).astype(np.uint16))
    z8 = wl.encode_q8(np.zeros((n_out, n_in), np.int8),
                      rng.uniform(0.1, 10, (n_out, nb)).astype(np.float32))
    for fmt, w in ((Q4, z4), (Q8, z8)):
        y, bound = O.matmul(x, w, fmt, n_out)
        assert np.all(y == 0) and np.all(bound == 0), f"zero codes fmt {fmt}"


def pin_roundtrip_q8(O):
    """Every int8 code survives dequantisation: rint(w / s) == q, and for
    power-of-two scales w == q * s exactly."""
    codes_row = np.arange(-128, 128, dtype=np.int16).astype(np.int8)  # 256 = 8 blocks
    pow2 = [2.0 ** e for e in range(-14, 1)]
    rnd = list(np.random.default_rng(10).uniform(1e-4, 1e-3, 8))
    scales = np.array(pow2 + rnd, dtype=np.float32)
    n_out, n_in = len(scales), codes_row.size
    codes = np.tile(codes_row, (n_out, 1))
    w = O.dequant(wl.encode_q8(codes, np.repeat(scales[:, None], n_in // 32, 1)), Q8, n_out, n_in)
    q_back = np.rint(w.astype(np.float64) / scales[:, None].astype(np.float64))
    assert np.array_equal(q_back, codes.astype(np.float64)), "Q8 codes do not round-trip"
    for r, e in enumerate(range(-14, 1)):
        assert np.array_equal(w[r], np.ldexp(codes_row.astype(np.float64), e)), "Q8 pow2 scale"


def pin_roundtrip_q4(O):
    """Every 4-bit code survives: w / s + 8 == code exactly (f16 scales)."""
    codes_row = np.tile(np.arange(16, dtype=np.uint8), 2)  # one block, each code twice
    sbits = [(e + 15) << 10 for e in range(-14, 2)]  # powers of two 2^-14 .. 2^1
    sbits += list(np.random.default_rng(11).integers(0x1400, 0x2400, 8))
    sbits += [0x0001, 0x03FF]  # subnormal scales
    sbits = np.array(sbits, dtype=np.uint16)
    n_out = len(sbits)
    codes = np.tile(codes_row, (n_out, 1))
    w = O.dequant(wl.encode_q4(codes, sbits[:, None]), Q4, n_out, 32)
    s = lib_f16(sbits)[:, None]
    assert np.array_equal(w.astype(np.float64) / s + 8.0, codes.astype(np.float64)), "Q4 round trip"


# ---------------------------------------------------- gate/up with GELU
# The fused feed-forward step GELU(x G^T) * (x U^T) (gelu_mul of the drafter
# page).  Pinned by scipy's normal CDF (GELU(v) = v Phi(v)), the exact
# identity GELU(v) - GELU(-v) = v, one-hot weights that select x columns,
# the composition with a numpy float64 matmul of library-decoded weights,
# and a Monte Carlo check that the bound covers every g, u within the
# matmul tolerance of the exact sums.
def _lib_gelu(v):
    from scipy.stats import norm
    v = np.asarray(v, dtype=np.float64)
    return v * norm.cdf(v)


def _lib_values(fmt, parts):
    """Library-decoded weight values (float64) of generated parts."""
    if fmt == BF16:
        return lib_bf16(parts)
    if fmt == Q8:
        return lib_q8_values(*parts).astype(np.float64)
    return lib_q4_values(*parts).astype(np.float64)


def pin_gelu_values(O):
    v = np.concatenate([np.linspace(-12, 12, 2401), [0.0, 1e-300, -1e-300, 1e-8, 37.0, -37.0]])
    g = O.gelu(v)
    assert np.all(np.abs(g - _lib_gelu(v)) <= 1e-15 * np.maximum(1, np.abs(v))), "GELU vs v * Phi(v)"
    assert np.all(np.abs(g - O.gelu(-v) - v) <= 1e-15 * np.maximum(1, np.abs(v))), "GELU(v) - GELU(-v) = v"
    assert O.gelu(np.array([0.0]))[0] == 0.0 and O.gelu(np.array([10.0]))[0] == 10.0
    assert abs(O.gelu(np.array([-10.0]))[0]) < 1e-20
    d = np.diff(g[:2401]) / np.diff(v[:2401])
    assert 1.12 < d.max() <= 1.13, "largest GELU slope (the bound's constant)"


def pin_gelu_mul_onehot(O):
    n_out, n_in = 6, 64
    cg = np.array([0, 5, 17, 63, 31, 2])
    cu = np.array([1, 5, 40, 0, 31, 63])
    x = (np.random.default_rng(30).standard_normal((3, n_in)) * 2).astype(np.float32)
    xg, xu = x[:, cg].astype(np.float64), x[:, cu].astype(np.float64)
    want = (_lib_gelu(xg) * xu).astype(np.float32)
    for fmt in (BF16, Q8, Q4):
        y, bound = O.gelu_mul(x, _onehot_weight(fmt, n_out, n_in, cg), _onehot_weight(fmt, n_out, n_in, cu),
                              fmt, n_out)
        assert np.all(np.abs(y.astype(np.float64) - want) <= 2.0 ** -23 * np.abs(want)), f"one-hot fmt {fmt}"
        # the bound holds at least the up term |GELU(G)| Bu and the gate term 1.13 Bg |U|
        assert np.all(bound >= np.abs(_lib_gelu(xg)) * np.abs(xu) * 0.999), "bound: up term"
        assert np.all(bound >= 1.13 * np.abs(xg) * np.abs(xu) * 0.999), "bound: gate term"
    zg = _onehot_weight(Q4, n_out, n_in, cg)
    zero = wl.encode_q4(np.full((n_out, n_in), 8, np.uint8), np.full((n_out, 2), 0x3C00, np.uint16))
    for G, U in ((zero, zg), (zg, zero)):
        y, bound = O.gelu_mul(x, G, U, Q4, n_out)
        assert np.all(y == 0) and np.all(bound == 0), "an all-zero projection gives exactly 0"


def pin_gelu_mul_composition(O):
    rng = np.random.default_rng(31)
    t, n_out, n_in = 3, 20, 96
    x = rng.standard_normal((t, n_in)).astype(np.float32)
    for fmt in (BF16, Q8, Q4):
        parts = [_random_parts(fmt, rng, n_out, n_in) for _ in range(2)]
        (G, U) = [_encode(fmt, p) for p in parts]
        Wg, Wu = [_lib_values(fmt, p) for p in parts]
        g64 = x.astype(np.float64) @ Wg.T
        u64 = x.astype(np.float64) @ Wu.T
        want = _lib_gelu(g64) * u64
        y, bound = O.gelu_mul(x, G, U, fmt, n_out)
        err = np.abs(y.astype(np.float64) - want)
        assert np.all(err <= 2.0 ** -23 * np.abs(want) + 1e-12 * bound), f"composition fmt {fmt}"
        # Monte Carlo: any g, u within the matmul tolerance stays within the bound
        bg = np.abs(x.astype(np.float64)) @ np.abs(Wg).T
        bu = np.abs(x.astype(np.float64)) @ np.abs(Wu).T
        for _ in range(200):
            g = g64 + 4e-3 * bg * rng.uniform(-1, 1, g64.shape)
            u = u64 + 4e-3 * bu * rng.uniform(-1, 1, u64.shape)
            assert np.all(np.abs(_lib_gelu(g) * u - y) <= 4e-3 * bound * (1 + 1e-9)), "bound too small"


# --------------------------------------------- centroid-masked LM head
# Top-k centroids by logit, then the first token of largest score over their
# clusters.  Pinned by integer-valued inputs (every sum exact in f32, so ties
# are exact and the tie rules are tested) against a brute force in Python
# integers, and by random inputs against a numpy float64 matmul plus a
# selection written with numpy's lexsort / argmax.
def _lm_head_brute(x_int, cen_int, emb_int, ordering, k):
    t = x_int.shape[0]
    n_c, vocab = cen_int.shape[0], emb_int.shape[0]
    per = vocab // n_c
    toks, clus, scores = [], [], []
    for i in range(t):
        cl = [int(np.dot(cen_int[c].astype(np.int64), x_int[i].astype(np.int64))) for c in range(n_c)]
        sel = sorted(range(n_c), key=lambda c: (-cl[c], c))[:k]
        best = None
        for c in sel:
            for j in range(per):
                tok = int(ordering[c * per + j])
                sc = int(np.dot(emb_int[tok].astype(np.int64), x_int[i].astype(np.int64)))
                if best is None or sc > best[0]:
                    best = (sc, tok)
        toks.append(best[1]); clus.append(sel); scores.append(best[0])
    return np.array(toks), np.array(clus), np.array(scores, dtype=np.float64)


def _bf16_of_ints(a):
    return wl.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def pin_lm_head_integers(O):
    rng = np.random.default_rng(40)
    for h, n_c, per, k in ((16, 8, 4, 1), (16, 8, 4, 3), (24, 12, 8, 12), (8, 16, 2, 5)):
        vocab = n_c * per
        x = rng.integers(-3, 4, (4, h))
        cen = rng.integers(-2, 3, (n_c, h))
        emb = rng.integers(-2, 3, (vocab, h))
        cen[1] = cen[0]            # equal logits: the lower cluster index goes first
        emb[5] = emb[2]            # equal scores: the first met wins
        order = rng.permutation(vocab).astype(np.uint32)
        r = O.centroid_argmax(x.astype(np.float32), _bf16_of_ints(cen), _bf16_of_ints(emb), order, k)
        tok, clus, sc = _lm_head_brute(x, cen, emb, order, k)
        assert np.array_equal(r["clusters"], clus), f"clusters h={h} C={n_c} k={k}"
        assert np.array_equal(r["token"], tok), f"token h={h} C={n_c} k={k}"
        assert np.array_equal(r["score"].astype(np.float64), sc), "score"


def pin_lm_head_topk_clamp(O):
    """k above the number of clusters takes all of them: the page's
    `let k = self.top_k_centroids.min(self.num_centroids)` in Drafter::step
    (oxinfer 0.0.1 src/drafter.rs), checked against brute force with k = C."""
    rng = np.random.default_rng(43)
    h, n_c, per = 16, 6, 3
    vocab = n_c * per
    x = rng.integers(-3, 4, (2, h))
    cen = rng.integers(-2, 3, (n_c, h))
    emb = rng.integers(-2, 3, (vocab, h))
    order = rng.permutation(vocab).astype(np.uint32)
    tok, clus, sc = _lm_head_brute(x, cen, emb, order, n_c)
    for k in (n_c, n_c + 1, 4 * n_c):
        r = O.centroid_argmax(x.astype(np.float32), _bf16_of_ints(cen), _bf16_of_ints(emb), order, k)
        assert r["clusters"].shape == (2, n_c), f"k={k}: clusters shape {r['clusters'].shape}"
        assert np.array_equal(r["clusters"], clus) and np.array_equal(r["token"], tok), f"k={k}"


def pin_lm_head_random(O):
    rng = np.random.default_rng(41)
    t, h, n_c, per, k = 3, 64, 32, 8, 4
    vocab = n_c * per
    x = rng.standard_normal((t, h)).astype(np.float32)
    cen = wl.f32_to_bf16_bits(rng.standard_normal((n_c, h)).astype(np.float32))
    emb = wl.f32_to_bf16_bits(rng.standard_normal((vocab, h)).astype(np.float32))
    order = rng.permutation(vocab).astype(np.uint32)
    r = O.centroid_argmax(x, cen, emb, order, k)
    cenf, embf = lib_bf16(cen), lib_bf16(emb)
    cl = x.astype(np.float64) @ cenf.T
    assert np.allclose(r["cl"], cl, rtol=1e-12, atol=1e-12), "centroid logits"
    assert np.allclose(r["cl_bound"], np.abs(x.astype(np.float64)) @ np.abs(cenf).T, rtol=1e-12), "bounds"
    for i in range(t):
        cl32 = r["cl"][i].astype(np.float32)
        sel = np.lexsort((np.arange(n_c), -cl32))[:k]  # decreasing logit, then increasing index
        assert np.array_equal(r["clusters"][i], sel), "selection rule"
        cand = np.concatenate([order[c * per:(c + 1) * per] for c in sel])
        sc = (embf[cand] @ x[i].astype(np.float64)).astype(np.float32)
        j = int(np.argmax(sc))  # first occurrence of the maximum
        assert r["token"][i] == cand[j] and r["score"][i] == sc[j], "first-max argmax"


def pin_token_score(O):
    """One token's score embed[tok] . x and its bound sum |embed[tok] * x|
    (the `dot_bf16(row, xr)` of the candidate scan in `Drafter::step` on the
    oxinfer 0.0.1 src/drafter.rs page) against numpy float64 on torch-decoded
    bf16 rows: first, last and inner tokens, several rows of x, mixed signs
    so that a signed bound or a shifted row cannot agree by chance."""
    rng = np.random.default_rng(42)
    for h, vocab in ((64, 37), (256, 300), (32, 2)):
        emb = wl.f32_to_bf16_bits(rng.standard_normal((vocab, h)).astype(np.float32))
        embf = lib_bf16(emb)
        xs = rng.standard_normal((3, h)).astype(np.float32)
        for x in xs:
            for tok in sorted({0, 1, vocab // 2, vocab - 2, vocab - 1}):
                v, b = O.token_score(x, emb, tok)
                want = float(embf[tok] @ x.astype(np.float64))
                want_b = float(np.abs(embf[tok]) @ np.abs(x.astype(np.float64)))
                assert abs(v - want) <= 1e-12 * want_b, f"score h={h} tok={tok}: {v} vs {want}"
                assert abs(b - want_b) <= 1e-12 * want_b, f"bound h={h} tok={tok}: {b} vs {want_b}"
    # an exact case: integer rows, whose dot products are exact in both
    emb_i = np.array([[1, -2, 3, 0], [4, 0, -1, 2], [-3, 3, 3, -3]], np.int64)
    x_i = np.array([2.0, -1.0, 0.5, 4.0], np.float32)
    for tok, (want, want_b) in enumerate(((5.5, 5.5), (15.5, 16.5), (-19.5, 22.5))):
        v, b = O.token_score(x_i, _bf16_of_ints(emb_i), tok)
        assert (v, b) == (want, want_b), f"integer row {tok}: ({v}, {b})"


# --------------------------------------------------------------- quantiser
# The upload quantiser (absmax per 32-element block; the rule is stated in
# il_oracle.c).  Its pins: numpy's float16 cast on every binary16 value, on
# every midpoint between neighbours and on random f32 values; hand-derived
# blocks; exact round trips of codes on power-of-two scales; and, on random
# blocks, the properties the rule implies (largest code reaches the grid end,
# every code is the nearest grid point to its weight, the Q4 scale is the
# nearest binary16 to amax / 7).  The block decoders below read the host
# formats directly, without the oracle.
def _q8_parts(blocks, n_out, n_in):
    nb = n_in // 32
    blk = np.asarray(blocks, dtype=np.uint8).reshape(n_out, nb, 36)
    scales = blk[:, :, :4].copy().view("<f4").reshape(n_out, nb)
    codes = blk[:, :, 4:].copy().view(np.int8).reshape(n_out, n_in)
    return codes, scales


def _q4_parts(blocks, n_out, n_in):
    nb = n_in // 32
    blk = np.asarray(blocks, dtype=np.uint8).reshape(n_out, nb, 18)
    sbits = blk[:, :, :2].copy().view("<u2").reshape(n_out, nb)
    qs = blk[:, :, 2:]
    codes = np.empty((n_out, nb, 32), dtype=np.uint8)
    codes[:, :, 0::2] = qs & 0x0F
    codes[:, :, 1::2] = qs >> 4
    return codes.reshape(n_out, n_in), sbits


def pin_f16_rounding(O):
    """f32 -> binary16 agrees with numpy's float16 cast (round to nearest
    even) on every finite binary16 value, every midpoint between neighbours
    (the ties) and random f32 values across the whole range."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = pats.view(np.float16)
    fin = np.isfinite(vals)
    got = O.f16_bits(vals[fin].astype(np.float32))
    assert np.array_equal(got, pats[fin]), "f16 values do not map to themselves"
    pos = np.sort(vals[fin & (vals >= 0) & ~np.signbit(vals)].astype(np.float64))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)  # exact: <= 12 significant bits
    mids = np.concatenate([mids, -mids, np.float32([65520.0, -65520.0, 65519.0])])
    rng = np.random.default_rng(20)
    rnd = (rng.uniform(1, 2, 200000) * np.exp2(rng.integers(-30, 18, 200000))).astype(np.float32)
    rnd *= np.where(rng.random(200000) < 0.5, -1, 1).astype(np.float32)
    for v in (mids, rnd):
        with np.errstate(over="ignore"):
            want = v.astype(np.float16).view(np.uint16)
        assert np.array_equal(O.f16_bits(v), want), "f16 rounding differs from numpy"
    nan = int(O.f16_bits(np.float32([np.nan]))[0])
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x3FF) != 0, "NaN must stay NaN"


def pin_quantize_hand(O):
    """Hand-derived blocks.  Q8: amax = 127/8, so s = 1/8 and w / s is the
    list 127, -64, 0.5, 1.5, 2.5 -> codes 127, -64, 0, 2, 2 (ties to even).
    Q4: amax = 7/4, s = 1/4 (binary16 0x3400) and w / s = 7, -7, 3.5, -0.5,
    1.5, 2.5 -> values 7, -7, 4, 0, 2, 2 -> codes 15, 1, 12, 8, 10, 10."""
    w8 = np.zeros((1, 32), np.float32)
    w8[0, :5] = np.array([127, -64, 0.5, 1.5, 2.5]) / 8
    codes, scales = _q8_parts(O.quantize(w8, Q8), 1, 32)
    assert scales[0, 0] == np.float32(0.125), "Q8 hand scale"
    assert list(codes[0, :5]) == [127, -64, 0, 2, 2] and not codes[0, 5:].any(), "Q8 hand codes"
    w4 = np.zeros((1, 32), np.float32)
    w4[0, :6] = np.array([7, -7, 3.5, -0.5, 1.5, 2.5]) / 4
    codes, sbits = _q4_parts(O.quantize(w4, Q4), 1, 32)
    assert sbits[0, 0] == 0x3400, "Q4 hand scale"
    assert list(codes[0, :6]) == [15, 1, 12, 8, 10, 10] and np.all(codes[0, 6:] == 8), "Q4 hand codes"
    z = np.zeros((2, 64), np.float32)
    c8, s8 = _q8_parts(O.quantize(z, Q8), 2, 64)
    c4, s4 = _q4_parts(O.quantize(z, Q4), 2, 64)
    assert not c8.any() and not s8.any() and np.all(c4 == 8) and not s4.any(), "zero blocks"


def pin_quantize_roundtrip(O):
    """Codes on a power-of-two scale, each block holding the grid end (Q8
    +-127, Q4 +-7): quantising the exact values returns those codes and
    that scale bit for bit."""
    rng = np.random.default_rng(21)
    n_out, n_in = 24, 128
    for fmt, top, exps in ((Q8, 127, range(-20, 4)), (Q4, 7, range(-14, 10))):
        v = rng.integers(-top, top + 1, (n_out, n_in))
        blocks = v.reshape(n_out, -1, 32)
        pos = rng.integers(0, 32, blocks.shape[:2])
        sign = np.where(rng.random(blocks.shape[:2]) < 0.5, -1, 1)
        np.put_along_axis(blocks, pos[..., None], (top * sign)[..., None], axis=2)
        e = np.array(list(exps))[:n_out]
        w = (v.astype(np.float64) * np.exp2(e)[:, None]).astype(np.float32)
        if fmt == Q8:
            codes, scales = _q8_parts(O.quantize(w, Q8), n_out, n_in)
            assert np.array_equal(codes, v), "Q8 codes do not round-trip"
            assert np.array_equal(scales, np.repeat(np.exp2(e)[:, None], n_in // 32, 1).astype(np.float32))
        else:
            codes, sbits = _q4_parts(O.quantize(w, Q4), n_out, n_in)
            assert np.array_equal(codes.astype(np.int64) - 8, v), "Q4 codes do not round-trip"
            assert np.array_equal(sbits, np.repeat(((e + 15) << 10)[:, None], n_in // 32, 1)), "Q4 scale"


def pin_quantize_nearest(O):
    """Random blocks over 12 decades of scale: the Q8 scale is amax / 127 to
    within f32 rounding and the largest |code| is 127; the Q4 scale is the
    binary16 nearest amax / 7; every code is the grid point nearest its
    weight on the stored scale (within f32 rounding of the quotient), or the
    end of the grid it was clamped to."""
    rng = np.random.default_rng(22)
    n_out, n_in = 64, 256
    sig = np.exp2(rng.uniform(-20, 20, (n_out, 1)))
    w = (rng.standard_normal((n_out, n_in)) * sig).astype(np.float32)
    w[3, 32:64] = 0.0  # one all-zero block
    amax = np.abs(w.astype(np.float64)).reshape(n_out, -1, 32).max(axis=2)
    slack = 1 + 2.0 ** -20
    codes, scales = _q8_parts(O.quantize(w, Q8), n_out, n_in)
    s = scales.astype(np.float64)
    assert np.all(np.abs(s * 127 - amax) <= amax * 2.0 ** -22), "Q8 scale is not amax / 127"
    nz = amax > 0
    top = np.abs(codes.astype(np.int64)).reshape(n_out, -1, 32).max(axis=2)
    assert np.all(top[nz] == 127) and np.all(top[~nz] == 0), "Q8 grid end not reached"
    se = np.repeat(s, 32, axis=1)
    err = np.abs(w - codes * se)
    assert np.all(err <= 0.5 * se * slack), "Q8 code is not the nearest grid point"
    codes, sbits = _q4_parts(O.quantize(w, Q4), n_out, n_in)
    s16 = lib_f16(sbits)
    q = amax / 7
    spacing = np.spacing(s16.astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(s16 - q) <= 0.5 * spacing * slack), "Q4 scale is not the nearest binary16"
    se = np.repeat(s16, 32, axis=1)
    v = codes.astype(np.float64) - 8
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(se > 0, w / se, 0.0)
    inside = (ratio >= -8.5) & (ratio <= 7.5)
    assert np.all(np.abs(w - v * se)[inside] <= 0.5 * se[inside] * slack), "Q4 code is not the nearest"
    assert np.all(v[ratio > 7.5] == 7) and np.all(v[ratio < -8.5] == -8), "Q4 clamp"


# -------------------------------------------------------------- brute force
def _exact_values(fmt, parts):
    """Exact rationals of every weight element, from library-decoded values."""
    if fmt == BF16:
        return [[Fraction(float(v)) for v in row] for row in lib_bf16(parts)]
    if fmt == Q8:
        return [[Fraction(float(v)) for v in row] for row in lib_q8_values(*parts)]
    codes, sbits = parts
    s = lib_f16(sbits)
    return [[(int(c) - 8) * Fraction(float(s[r][k // 32])) for k, c in enumerate(row)]
            for r, row in enumerate(codes)]


def _random_parts(fmt, rng, n_out, n_in):
    nb = n_in // 32
    if fmt == BF16:
        return wl.f32_to_bf16_bits(rng.standard_normal((n_out, n_in)).astype(np.float32))
    if fmt == Q8:
        return (rng.integers(-128, 128, (n_out, n_in)).astype(np.int8),
                rng.uniform(1e-3, 1.0, (n_out, nb)).astype(np.float32))
    return (rng.integers(0, 16, (n_out, n_in)).astype(np.uint8),
            rng.uniform(1e-3, 1.0, (n_out, nb)).astype(np.float16).view(np.uint16))


def _encode(fmt, parts):
    if fmt == BF16:
        return parts
    return wl.encode_q8(*parts) if fmt == Q8 else wl.encode_q4(*parts)


def _f32_neighbours(v: float):
    f = np.float32(v)
    return {f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))}


def pin_bruteforce(O):
    """Exact rational result on tiny shapes: the oracle is within one f32 ulp
    of the correctly rounded value, and its bound matches sum |x w|."""
    rng = np.random.default_rng(12)
    for fmt in (BF16, Q8, Q4):
        for t, n_out, n_in in ((1, 1, 32), (2, 3, 32), (3, 5, 64), (3, 4, 64)):
            parts = _random_parts(fmt, rng, n_out, n_in)
            x = rng.standard_normal((t, n_in)).astype(np.float32)
            W = _exact_values(fmt, parts)
            y, bound = O.matmul(x, _encode(fmt, parts), fmt, n_out)
            for i in range(t):
                xi = [Fraction(float(v)) for v in x[i]]
                for r in range(n_out):
                    exact = sum(a * b for a, b in zip(xi, W[r]))
                    mag = sum(abs(a * b) for a, b in zip(xi, W[r]))
                    assert y[i, r] in _f32_neighbours(float(exact)), (
                        f"fmt {fmt} ({i},{r}): oracle {y[i, r]!r} vs exact {float(exact)!r}")
                    assert math.isclose(bound[i, r], float(mag), rel_tol=1e-12), "bound"


# --------------------------------------------------------- library routine
def pin_numpy_matmul(O, rows_per_job: int = 64):
    """numpy float64 x @ W.T on library-decoded weights, at the workloads'
    shapes (row subsets of the large jobs keep the CPU time low)."""
    seen = set()
    for name, sub in wl.SUBMISSIONS.items():
        x = wl.make_x(sub)
        if sub.t > 8:
            x = x[:16]
        for j in sub.jobs:
            if (sub.cfg, j.tensor_id) in seen:  # c4 repeats its weights at each t
                continue
            if sub.name.startswith("c4") and sub.t != 8:
                continue
            seen.add((sub.cfg, j.tensor_id))
            n_rows = min(j.n_out, rows_per_job if sub.name != "c1" else j.n_out)
            rows = np.unique(np.r_[0, j.n_out - 1,
                                   np.random.default_rng(13).integers(0, j.n_out, n_rows)])
            if j.fmt == BF16:
                bits = wl.gen_bf16(sub.cfg, j.tensor_id, j.n_out, sub.n_in)
                wd = lib_bf16(bits[rows])
                host = bits
            elif j.fmt == Q8:
                codes, sc = wl.gen_q8_parts(sub.cfg, j.tensor_id, j.n_out, sub.n_in)
                wd = lib_q8_values(codes[rows], sc[rows]).astype(np.float64)
                host = wl.encode_q8(codes, sc)
            else:
                codes, sb = wl.gen_q4_parts(sub.cfg, j.tensor_id, j.n_out, sub.n_in)
                wd = lib_q4_values(codes[rows], sb[rows]).astype(np.float64)
                host = wl.encode_q4(codes, sb)
            want = x.astype(np.float64) @ wd.T
            mag = np.abs(x.astype(np.float64)) @ np.abs(wd).T
            ii = np.repeat(np.arange(x.shape[0]), rows.size)
            rr = np.tile(rows, x.shape[0])
            got, bound = O.matmul_points(x, host, j.fmt, j.n_out, ii, rr)
            got = got.reshape(x.shape[0], rows.size).astype(np.float64)
            bound = bound.reshape(x.shape[0], rows.size)
            err = np.abs(got - want)
            # f32 rounding of the oracle's result plus summation-order noise
            assert np.all(err <= np.abs(want) * 2.0 ** -23 + 1e-12 * mag), (
                f"{name} job {j.tensor_id}: max err {err.max()}")
            assert np.allclose(bound, mag, rtol=1e-12, atol=0), f"{name}: bound"


# --------------------------------------------------------------- internals
def pin_points_equal_rows(O):
    rng = np.random.default_rng(14)
    for fmt in (BF16, Q8, Q4):
        parts = _random_parts(fmt, rng, 9, 96)
        x = rng.standard_normal((3, 96)).astype(np.float32)
        w = _encode(fmt, parts)
        y, b = O.matmul(x, w, fmt, 9)
        ii = np.repeat(np.arange(3), 9)
        rr = np.tile(np.arange(9), 3)
        yp, bp = O.matmul_points(x, w, fmt, 9, ii, rr)
        assert np.array_equal(yp, y.ravel()) and np.array_equal(bp, b.ravel()), f"fmt {fmt}"
        y2, b2 = O.matmul(x, w, fmt, 9, r0=3, r1=7)
        assert np.array_equal(y2, y[:, 3:7]) and np.array_equal(b2, b[:, 3:7])


def pin_thread_invariance(O):
    rng = np.random.default_rng(15)
    parts = _random_parts(Q4, rng, 64, 256)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    w = _encode(Q4, parts)
    y1, b1 = O.matmul(x, w, Q4, 64, threads=1)
    y8, b8 = O.matmul(x, w, Q4, 64, threads=8)
    assert np.array_equal(y1, y8) and np.array_equal(b1, b8)


def pin_check_rule(O):
    yr = np.array([1.0, -2.0, 0.0, 5.0], np.float32)
    bd = np.array([1.0, 2.0, 0.0, 10.0])
    assert O.check(yr, yr, bd)["ok"]
    ok_edge = yr + np.array([4e-3 * 0.999, 0, 0, 0], np.float32)
    assert O.check(ok_edge, yr, bd)["ok"]
    assert not O.check(yr + np.array([0, 0, 0, 0.05], np.float32), yr, bd)["ok"]
    assert not O.check(np.array([1.0, -2.0, 1e-30, 5.0], np.float32), yr, bd)["ok"]
    for bad in (np.nan, np.inf):
        r = O.check(np.array([bad, -2.0, 0.0, 5.0], np.float32), yr, bd)
        assert r["bad"] == 1 and r["first_bad"] == 0


ALL_PINS = [
    pin_bf16_exhaustive, pin_f16_exhaustive, pin_goldens, pin_onehot, pin_identity,
    pin_row_sums, pin_zero_codes, pin_roundtrip_q8, pin_roundtrip_q4, pin_bruteforce,
    pin_numpy_matmul, pin_points_equal_rows, pin_thread_invariance, pin_check_rule,
    pin_f16_rounding, pin_quantize_hand, pin_quantize_roundtrip, pin_quantize_nearest,
    pin_gelu_values, pin_gelu_mul_onehot, pin_gelu_mul_composition,
    pin_lm_head_integers, pin_lm_head_random, pin_token_score, pin_lm_head_topk_clamp,
]


def run_all(O, quick: bool = False) -> list:
    """Run every pin; returns the names of the pins that failed."""
    failed = []
    for pin in ALL_PINS:
        try:
            if quick and pin is pin_numpy_matmul:
                continue  # full-shape generation dominates the run time
            pin(O)
        except Exception as e:  # noqa: BLE001 -- a mutant may fail any way it likes
            failed.append(f"{pin.__name__}: {type(e).__name__}: {str(e)[:200]}")
    return failed
