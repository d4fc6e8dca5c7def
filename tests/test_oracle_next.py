"""Pins of the oracle's functions for the steps next to the path: token
packing (pack / unpack) and the gradient of the pooling (pool_backward).

Each is checked against something other than itself:
  * hand-worked examples (tests/golden/next_forms.json);
  * for packing: numpy's cumulative sum and bincount for cu_seqlens and
    doc_id, the pack/unpack round trip, and rejection of counts outside
    [0, P];
  * for the gradient: central finite differences of the pooled means
    computed in exact rational arithmetic (fractions.Fraction), in Voronoi
    and kNN mode (pulses in several lists), weighted and unweighted; the
    plain-mean special case (gradient = g / member count); pass-through
    tokens (gradient = g); tokens of zero weight (no gradient); linearity in
    the incoming gradient.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "next_forms.json")


def _golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


# ---------------------------------------------------------------- packing

def test_pack_worked_example(oracle_mod):
    g = _golden()["pack"]
    tc = np.array(g["token_count"], np.int32)
    B, P, D = tc.size, g["P"], g["D"]
    rows = np.arange(B * P * D, dtype=np.float32).reshape(B, P, D)
    packed, doc, cu = oracle_mod.pack(tc, rows)
    np.testing.assert_array_equal(packed, np.array(g["packed"], np.float32))
    np.testing.assert_array_equal(doc, g["doc_id"])
    np.testing.assert_array_equal(cu, g["cu_seqlens"])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_pack_counts_and_round_trip(oracle_mod, seed):
    rng = np.random.default_rng(seed)
    B, P, D = 37, 16, 5
    tc = rng.integers(0, P + 1, B).astype(np.int32)
    tc[::7] = 0
    tc[3] = P
    rows = rng.standard_normal((B, P, D)).astype(np.float32)
    packed, doc, cu = oracle_mod.pack(tc, rows)
    np.testing.assert_array_equal(cu, np.concatenate([[0], np.cumsum(tc)]))
    np.testing.assert_array_equal(np.bincount(doc, minlength=B), tc)
    assert packed.shape == (int(tc.sum()), D)
    back = oracle_mod.unpack(tc, cu, packed, P)
    mask = np.arange(P)[None, :] < tc[:, None]
    np.testing.assert_array_equal(back[mask], rows[mask])
    assert np.all(back[~mask] == 0)


def test_pack_rejects_bad_counts(oracle_mod):
    rows = np.zeros((2, 4, 1), np.float32)
    for bad in ([5, 0], [-1, 2]):
        with pytest.raises(RuntimeError):
            oracle_mod.pack(np.array(bad, np.int32), rows)


# --------------------------------------------------------- pooling gradient

def _members(mode, n, T, assign, knn, k):
    if mode == 0:
        return [[i for i in range(n) if assign[i] == j] for j in range(T)]
    return [[int(q) for q in knn[j * k:(j + 1) * k] if q >= 0] for j in range(T)]


def _exact_pool(f, members, wcol):
    """Pooled means of one event in exact rational arithmetic."""
    out = []
    for mem in members:
        W = sum((f[i][wcol] if wcol >= 0 else Fraction(1)) for i in mem)
        if W == 0:
            out.append([Fraction(0)] * len(f[0]))
            continue
        row = []
        for c in range(len(f[0])):
            row.append(sum((f[i][wcol] if wcol >= 0 else Fraction(1)) * f[i][c] for i in mem) / W)
        out.append(row)
    return out


def _fd_grad(fl, members, wcol, g):
    """Central differences of sum_j g_j . m_j with respect to every feature."""
    h = Fraction(1, 1 << 22)
    f = [[Fraction(float(v)) for v in row] for row in fl]
    grad = np.zeros((len(f), len(f[0])))
    for i in range(len(f)):
        for c in range(len(f[0])):
            vals = []
            for s in (1, -1):
                f2 = [row[:] for row in f]
                f2[i][c] += s * h
                m = _exact_pool(f2, members, wcol)
                vals.append(sum(Fraction(float(g[j][q])) * m[j][q]
                                for j in range(len(m)) for q in range(len(m[0]))))
            grad[i, c] = float((vals[0] - vals[1]) / (2 * h))
    return grad


def _case(seed, mode, weighted):
    rng = np.random.default_rng(seed)
    n, P, C, k = 11, 4, 3, 4
    f = rng.integers(-8, 9, (n, C)).astype(np.float32) / 4
    if weighted:
        f[:, 1] = rng.integers(1, 9, n).astype(np.float32) / 2  # positive charges
    T = P
    assign = rng.integers(0, T, n).astype(np.int32)
    assign[:T] = np.arange(T)  # no empty cell
    knn = np.full((P, k), -1, np.int32)
    for j in range(T):
        kk = int(rng.integers(1, k + 1))
        knn[j, :kk] = rng.choice(n, kk, replace=False)
    return f, P, C, k, T, assign, knn


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("seed", [0, 1])
def test_pool_backward_finite_differences(oracle_mod, mode, weighted, seed):
    f, P, C, k, T, assign, knn = _case(seed, mode, weighted)
    n = f.shape[0]
    wcol = 1 if weighted else -1
    off = np.array([0, n], np.int64)
    tc = np.array([T], np.int32)
    kw = dict(mode=mode, assign=assign if mode == 0 else None,
              knn_idx=knn[None] if mode == 1 else None, k=k, weighted=weighted, charge_col=1)
    pooled, _ = oracle_mod.pool(f, off, P, tc, **kw)
    g = np.random.default_rng(seed + 10).standard_normal((1, P, C)).astype(np.float32)
    got = oracle_mod.pool_backward(f, off, P, tc, pooled, g, **kw)
    mem = _members(mode, n, T, assign, knn.reshape(-1), k)
    want = _fd_grad(f, mem, wcol, g[0])
    scale = np.abs(want).max()
    np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-5 * scale)


def test_pool_backward_worked_example(oracle_mod):
    g = _golden()["pool_backward"]
    f = np.array(g["features"], np.float32)
    out = oracle_mod.pool_backward(
        f, np.array(g["offsets"]), g["P"], np.array(g["token_count"], np.int32),
        np.array(g["pooled"], np.float32)[None], np.array(g["grad_pooled"], np.float32)[None],
        mode=0, assign=np.array(g["assign"], np.int32), weighted=True, charge_col=g["charge_col"])
    np.testing.assert_array_equal(out, np.array(g["grad_features"], np.float32))


def test_pool_backward_plain_mean_and_passthrough(oracle_mod):
    rng = np.random.default_rng(5)
    n, P, C = 40, 8, 4
    f = rng.standard_normal((n, C)).astype(np.float32)
    f[:, 2] = rng.uniform(0.5, 3, n).astype(np.float32)
    assign = rng.integers(0, P, n).astype(np.int32)
    assign[:P] = np.arange(P)
    off = np.array([0, n], np.int64)
    tc = np.array([P], np.int32)
    g = rng.standard_normal((1, P, C)).astype(np.float32)
    pooled, cnt = oracle_mod.pool(f, off, P, tc, mode=0, assign=assign, weighted=False)
    got = oracle_mod.pool_backward(f, off, P, tc, pooled, g, mode=0, assign=assign,
                                   weighted=False, charge_col=2)
    want = (g[0][assign].astype(np.float64) / cnt[0][assign][:, None]).astype(np.float32)
    np.testing.assert_array_equal(got, want)
    # a pass-through event (n <= P, one pulse per token): the gradient is g,
    # weighted or not, except for a pulse of zero weight
    m = 6
    fp = f[:m].copy()
    fp[4, 2] = 0.0
    offp = np.array([0, m], np.int64)
    tcp = np.array([m], np.int32)
    ap = np.arange(m, dtype=np.int32)
    gp = g[:, :m].copy()
    pooled_p, _ = oracle_mod.pool(fp, offp, m, tcp, mode=0, assign=ap, weighted=True, charge_col=2)
    gotp = oracle_mod.pool_backward(fp, offp, m, tcp, pooled_p, gp, mode=0, assign=ap,
                                    weighted=True, charge_col=2)
    keep = np.arange(m) != 4
    np.testing.assert_array_equal(gotp[keep], gp[0][keep])
    assert np.all(gotp[4] == 0)


def test_pool_backward_zero_weight_token_and_linearity(oracle_mod):
    rng = np.random.default_rng(6)
    n, P, C, k = 30, 5, 3, 6
    f = rng.standard_normal((n, C)).astype(np.float32)
    f[:, 0] = rng.uniform(0.5, 2, n).astype(np.float32)
    knn = np.full((1, P, k), -1, np.int32)
    for j in range(P):
        knn[0, j] = rng.choice(n, k, replace=False)
    f[knn[0, 2], 0] = 0.0  # token 2 has zero weight
    # pulses only in token 2 get no gradient
    only2 = [i for i in knn[0, 2] if all(i not in knn[0, j] for j in range(P) if j != 2)]
    off = np.array([0, n], np.int64)
    tc = np.array([P], np.int32)
    kw = dict(mode=1, knn_idx=knn, k=k, weighted=True, charge_col=0)
    pooled, _ = oracle_mod.pool(f, off, P, tc, **kw)
    g1 = rng.standard_normal((1, P, C)).astype(np.float32)
    g2 = rng.standard_normal((1, P, C)).astype(np.float32)
    a = oracle_mod.pool_backward(f, off, P, tc, pooled, g1, **kw).astype(np.float64)
    b = oracle_mod.pool_backward(f, off, P, tc, pooled, g2, **kw).astype(np.float64)
    s = oracle_mod.pool_backward(f, off, P, tc, pooled, g1 + g2, **kw).astype(np.float64)
    np.testing.assert_allclose(s, a + b, rtol=1e-6, atol=1e-6)
    assert only2 and np.all(a[only2] == 0)
    # rows j >= T are ignored
    g3 = g1.copy()
    g3[0, P - 1] = 1e6
    tcs = np.array([P - 1], np.int32)
    knn_s = knn.copy()
    knn_s[0, P - 1] = -1
    kws = dict(kw, knn_idx=knn_s)
    p_s, _ = oracle_mod.pool(f, off, P, tcs, **kws)
    np.testing.assert_array_equal(oracle_mod.pool_backward(f, off, P, tcs, p_s, g3, **kws),
                                  oracle_mod.pool_backward(f, off, P, tcs, p_s, g1, **kws))


# ------------------------------------------------------- random FPS start

def test_philox_known_answers(oracle_mod):
    with open(os.path.join(os.path.dirname(__file__), "golden", "philox_kat.json")) as fh:
        vecs = json.load(fh)["vectors"]
    for v in vecs:
        c = np.array([int(h, 16) for h in v["counter"]], np.uint32)
        k = np.array([int(h, 16) for h in v["key"]], np.uint32)
        np.testing.assert_array_equal(oracle_mod.philox4x32_10(c, k),
                                      np.array([int(h, 16) for h in v["out"]], np.uint32))


def test_random_start_mapping_and_spread(oracle_mod):
    rng = np.random.default_rng(3)
    n = rng.integers(0, 5000, 4000)
    n[:7] = [0, 1, 2, 3, 2**31 - 1, 7, 1]
    off = np.concatenate([[0], np.cumsum(n.astype(np.int64))])
    s = oracle_mod.random_start(off, seed=12345, step=0)
    # the mapping from word 0 of the counter's block, recomputed per event
    for b in (0, 1, 2, 5, 100, 3999):
        u = int(oracle_mod.philox4x32_10(np.array([b, 0, 0, 0], np.uint32),
                                         np.array([12345, 0], np.uint32))[0])
        assert s[b] == ((u * int(n[b])) >> 32 if n[b] > 0 else 0)
    assert np.all((s >= 0) & ((s < n) | (n == 0)))
    # roughly uniform: start / n over many events fills ten equal bins
    frac = s[n > 100] / n[n > 100]
    h = np.histogram(frac, bins=10, range=(0, 1))[0]
    expect = frac.size / 10
    assert ((h - expect) ** 2 / expect).sum() < 30  # chi-square, 9 dof
    # a different step or seed gives different starts; the same ones repeat
    assert np.any(oracle_mod.random_start(off, 12345, 1) != s)
    assert np.any(oracle_mod.random_start(off, 12346, 0) != s)
    np.testing.assert_array_equal(oracle_mod.random_start(off, 12345, 0), s)


def test_random_start_from_the_known_answer_vector(oracle_mod):
    """The index mapping and the choice of word 0, worked by hand from the
    generator's first known-answer vector (tests/golden/random_start_forms.json)."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "random_start_forms.json")) as fh:
        g = json.load(fh)
    for case in g["cases"]:
        off = np.array([0, case["n"]], np.int64)
        assert oracle_mod.random_start(off, g["seed"], g["step"])[0] == case["start"], case


# Philox4x32-10 written again from its definition in Salmon, Moraes, Dror and
# Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011), with Python
# integers: each round takes the two 32x32-bit products of counter words 0
# and 2, crosses their high halves with words 1 and 3 and the round key, and
# the key advances by the two Weyl constants after every round.
_PHILOX_M = (0xD2511F53, 0xCD9E8D57)
_PHILOX_W = (0x9E3779B9, 0xBB67AE85)


def _philox_py(ctr, key):
    c = [int(v) for v in ctr]
    k = [int(v) for v in key]
    for _ in range(10):
        p0, p1 = _PHILOX_M[0] * c[0], _PHILOX_M[1] * c[2]
        c = [(p1 >> 32) ^ c[1] ^ k[0], p1 & 0xFFFFFFFF, (p0 >> 32) ^ c[3] ^ k[1], p0 & 0xFFFFFFFF]
        k = [(k[0] + _PHILOX_W[0]) & 0xFFFFFFFF, (k[1] + _PHILOX_W[1]) & 0xFFFFFFFF]
    return c


def test_random_start_counter_layout(oracle_mod):
    """Event index in counter words 0-1, step in words 2-3 (its high word
    non-zero), seed in the key (both words non-zero): the oracle against the
    independent Python generator above, which is itself checked against the
    published known-answer vectors first."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "philox_kat.json")) as fh:
        for v in json.load(fh)["vectors"]:
            assert _philox_py([int(h, 16) for h in v["counter"]],
                              [int(h, 16) for h in v["key"]]) == [int(h, 16) for h in v["out"]]
    rng = np.random.default_rng(11)
    n = rng.integers(1, 100000, 300).astype(np.int64)
    off = np.concatenate([[0], np.cumsum(n)])
    for seed, step in ((0x299F31D0A4093822, (7 << 32) + 3), (5, 2**64 - 1), (2**63 + 1, 1 << 40)):
        s = oracle_mod.random_start(off, seed, step)
        for b in (0, 1, 2, 17, 255, 299):
            w0 = _philox_py([b & 0xFFFFFFFF, b >> 32, step & 0xFFFFFFFF, step >> 32],
                            [seed & 0xFFFFFFFF, seed >> 32])[0]
            assert s[b] == (w0 * int(n[b])) >> 32, (seed, step, b)


# ------------------------------------------------ low-precision inputs

def test_upcast_binary16_exhaustive(oracle_mod):
    """Every binary16 bit pattern against numpy's IEEE conversion (an
    independent implementation; exact for every value, subnormals included)."""
    h = np.arange(65536, dtype=np.uint16)
    got = oracle_mod.upcast(h, oracle_mod.F16)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    np.testing.assert_array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.isnan(got[nan]).all()
    # hand-checked patterns: 1.0, -2.0, the smallest subnormal 2^-24, the
    # largest finite 65504, +infinity
    for bits, val in ((0x3C00, 1.0), (0xC000, -2.0), (0x0001, 2.0 ** -24), (0x7BFF, 65504.0),
                      (0x7C00, float("inf"))):
        assert oracle_mod.upcast(np.array([bits], np.uint16), oracle_mod.F16)[0] == val


def _bf16_value(h):
    """bfloat16 from its definition: sign, 8-bit exponent biased by 127,
    7-bit fraction; exponent 0 = zero and subnormals, 255 = inf / NaN."""
    s = -1.0 if h >> 15 else 1.0
    e = (h >> 7) & 0xFF
    m = h & 0x7F
    if e == 0:
        return s * math.ldexp(m, -133)          # m / 128 * 2^-126
    if e == 255:
        return s * math.inf if m == 0 else math.nan
    return s * math.ldexp(128 + m, e - 134)     # (1 + m / 128) * 2^(e - 127)


def test_upcast_bfloat16_exhaustive(oracle_mod):
    h = np.arange(65536, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # the NaN patterns
        got = oracle_mod.upcast(h, oracle_mod.BF16).astype(np.float64)
    ref = np.array([_bf16_value(int(x)) for x in h])
    nan = np.isnan(ref)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert np.isnan(got[nan]).all()
    with pytest.raises(RuntimeError):
        oracle_mod.upcast(h[:4], 3)


def test_tokenize_on_upcast_inputs_is_the_float32_path(oracle_mod):
    """Low-precision inputs are the float32 inputs of equal value: the
    tokenizer on upcast binary16 / bfloat16 coordinates and features equals
    the tokenizer on the same values written directly in float32 (numpy's
    binary16 conversion; bfloat16 by rounding float32 to its top 16 bits)."""
    from point_cloud_tokenization_amd import synth

    b = synth.icecube_events([40, 300, 900, 2], 71, C=6)
    x, f, off = b["coords"], b["features"], b["offsets"]
    x16 = x.astype(np.float16)
    f16 = f.astype(np.float16)
    xb = ((x.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)  # round half up to bfloat16
    fb = ((f.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)
    kw = dict(P=128, mode=0, L=1, weighted=True, charge_col=5)
    for (xs, fs, dt, x32, f32) in (
            (x16.view(np.uint16), f16.view(np.uint16), oracle_mod.F16,
             x16.astype(np.float32), f16.astype(np.float32)),
            (xb, fb, oracle_mod.BF16, (xb.astype(np.uint32) << 16).view(np.float32),
             (fb.astype(np.uint32) << 16).view(np.float32))):
        got = oracle_mod.tokenize(oracle_mod.upcast(xs, dt), oracle_mod.upcast(fs, dt), off, **kw)
        ref = oracle_mod.tokenize(x32, f32, off, **kw)
        for key in got:
            if got[key] is not None:
                np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
