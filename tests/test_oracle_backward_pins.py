"""Pins of the backward oracle (column-wise quantization, both gradients).

Checked against: exact rational arithmetic with IEEE rounding written from its
definition (brute_int8), inputs built so that every quantization is exact and
the result must equal a plain float64 matrix product, a closed-form error
bound, and invariants.  No GPU.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from brute_int8 import BruteBackward, brute_colwise_quant, f16, f32
from test_oracle_pins import _all_finite_f16, _fl32_of_exact, _rne_int_exact, _scales


def _near_f16_midpoint(y: Fraction) -> bool:
    r = f16(y)
    lo, hi = f16(y - abs(y) * Fraction(1, 2**30)), f16(y + abs(y) * Fraction(1, 2**30))
    return lo != r or hi != r


@pytest.mark.parametrize("seed", range(30))
def test_colwise_quant_brute_force(seed):
    rng = np.random.default_rng([7, seed])
    r, c = (int(v) for v in rng.integers(1, 8, size=2))
    a = (rng.standard_normal((r, c)) * rng.choice([0.01, 1.0, 40.0])).astype(np.float16)
    if c > 1:
        a[:, rng.integers(c)] = 0                      # an all-zero column
    zero = sorted(set(int(v) for v in rng.integers(0, c, size=rng.integers(0, 3))))
    qt, s = oracle.colwise_quant(a, zero)
    bq, bs = brute_colwise_quant(a.astype(np.float64).tolist(), zero)
    assert qt.shape == (c, r) and qt.dtype == np.int8
    assert qt.tolist() == bq
    assert [Fraction(float(v)) for v in s] == bs


def test_colwise_codes_exhaustive_all_fp16():
    # one column per scale s (an fp16 value): s itself, then every finite fp16
    # x with |x| <= s; the codes must be the exact-integer evaluation of
    # rne(fl32(x * fl32(127 / s))), clamped
    xs = _all_finite_f16()
    checked = 0
    for s in _scales():
        if float(np.float16(s)) != s:
            continue
        xv = xs[np.abs(xs.astype(np.float64)) <= s]
        col = np.concatenate([np.array([s], np.float16), xv])
        inv = float(f32(Fraction(127) / Fraction(s)))
        want = np.clip(_rne_int_exact(_fl32_of_exact(col.astype(np.float64) * inv)), -127, 127)
        qt, sc = oracle.colwise_quant(col[:, None])
        assert sc.tolist() == [s]
        assert np.array_equal(qt[0], want.astype(np.int8)), s
        checked += col.size
    assert checked > 2_000_000


def test_colwise_quant_hand_worked():
    # column 0: scale 2, codes rne(x * 63.5); column 1: scale 4, codes rne(x * 31.75)
    a = np.array([[2.0, -4.0], [1.0, 2.0], [-0.5, 1.0]], dtype=np.float16)
    qt, s = oracle.colwise_quant(a)
    assert s.tolist() == [2.0, 4.0]
    assert qt[0].tolist() == [127, 64, -32]            # 63.5 -> 64 (tie to even), -31.75 -> -32
    assert qt[1].tolist() == [-127, 64, 32]            # 63.5 -> 64, 31.75 -> 32
    qt0, _ = oracle.colwise_quant(a, [1])
    assert qt0[1].tolist() == [0, 0, 0] and qt0[0].tolist() == qt[0].tolist()


@pytest.mark.parametrize("seed", range(25))
def test_backward_brute_force_tiny(seed):
    rng = np.random.default_rng([8, seed])
    m, n, k = (int(v) for v in rng.integers(1, 6, size=3))
    g = (rng.standard_normal((m, n)) * 0.5).astype(np.float16)
    x = rng.uniform(-5, 5, size=(m, k)).astype(np.float16)
    cols = []
    if k > 1:
        j = int(rng.integers(k))
        x[:, j] = rng.uniform(6, 9, m) * rng.choice([-1, 1], m)
        cols = [j]
    w = (rng.standard_normal((n, k)) * 0.05).astype(np.float16)
    r = oracle.linear_backward(g, x, w, cols)
    b = BruteBackward(g.astype(np.float64).tolist(), x.astype(np.float64).tolist(),
                      w.astype(np.float64).tolist(), cols)
    assert r.g_q.tolist() == b.g_q
    assert r.wt_q.tolist() == b.wt_q and r.gt_q.tolist() == b.gt_q and r.xt_q.tolist() == b.xt_q
    assert r.c_x.tolist() == b.c_x and r.c_w.tolist() == b.c_w
    for i in range(m):
        for j in range(k):
            if not _near_f16_midpoint(b.gx[i][j]):
                assert Fraction(float(r.grad_x[i, j])) == f16(b.gx[i][j])
    for nn in range(n):
        for j in range(k):
            if not _near_f16_midpoint(b.gw[nn][j]):
                assert Fraction(float(r.grad_w[nn, j])) == f16(b.gw[nn][j])


def _exact_cols(rng, r, c, emin, emax):
    """fp16 matrix whose column j is an integer matrix with max |.| = 127 times 2^e_j."""
    ints = rng.integers(-127, 128, size=(r, c))
    ints[rng.integers(r, size=c), np.arange(c)] = 127 * rng.choice([-1, 1], c)
    e = rng.integers(emin, emax + 1, size=c)
    return (ints * np.exp2(e)[None, :]).astype(np.float16)


@pytest.mark.parametrize("seed", range(6))
def test_grad_input_exact_when_quantization_is_exact(seed):
    # g rows and W columns are 127-scaled integers times powers of two: every
    # code is exact, so grad_x must be exactly g . W (before its fp16 rounding)
    rng = np.random.default_rng([9, seed])
    m, n, k = 7, 13, 10
    g = _exact_cols(rng, n, m, -12, -3).T.copy()       # exact per row
    w = _exact_cols(rng, n, k, -14, -6)
    gx16, gx, *_ = oracle.grad_input(g, w)
    ref = g.astype(np.float64) @ w.astype(np.float64)
    assert np.array_equal(gx, ref)
    assert np.array_equal(gx16, ref.astype(np.float16))


@pytest.mark.parametrize("seed", range(6))
def test_grad_weight_exact_with_outlier_columns(seed):
    # g columns and x's non-outlier columns are exact under column-wise
    # quantization; the outlier columns are arbitrary short-mantissa fp16 with
    # |x| >= 6: the fp16 path must give them exactly g^T x, and the int8 path
    # must not add anything to them (CAt zeroed there)
    rng = np.random.default_rng([10, seed])
    m, n, k = 11, 6, 9
    g = _exact_cols(rng, m, n, -10, -4)
    x = _exact_cols(rng, m, k, -9, -6)                 # |x| <= 127 * 2^-6 < 6
    cols = sorted(set(int(v) for v in rng.choice(k, size=3, replace=False)))
    for j in cols:
        x[:, j] = (rng.integers(-60, 61, size=m) * 0.25).astype(np.float16)
        x[rng.integers(m), j] = 7.5
    gw16, gw, *_ = oracle.grad_weight(g, x, cols)
    ref = g.astype(np.float64).T @ x.astype(np.float64)
    assert np.array_equal(gw, ref)
    assert np.array_equal(gw16, ref.astype(np.float16))


def test_grad_weight_missing_zeroing_would_double_count():
    # the same data with the outlier columns NOT zeroed in CAt gives a wrong
    # result: the pin above separates the two
    rng = np.random.default_rng(11)
    g = _exact_cols(rng, 8, 4, -8, -4)
    x = _exact_cols(rng, 8, 5, -9, -6)
    x[:, 2] = 7.0
    _, gw, *_ = oracle.grad_weight(g, x, [2])
    _, gw_plain, *_ = oracle.grad_weight(g, x, [])
    ref = g.astype(np.float64).T @ x.astype(np.float64)
    assert np.array_equal(gw[:, 2], ref[:, 2])
    assert np.array_equal(gw_plain[:, 2], ref[:, 2])   # int8 alone is exact on a constant column
    assert np.array_equal(gw[:, [0, 1, 3, 4]], gw_plain[:, [0, 1, 3, 4]])


@pytest.mark.parametrize("seed", range(4))
def test_backward_error_bound(seed):
    # |q * s / 127 - a| <= s / 254 (plus the fp32 rounding of the code's
    # product, below 2^-17 * s): the closed-form bound of both gradients
    rng = np.random.default_rng([12, seed])
    m, n, k = 33, 21, 17
    g = (rng.standard_normal((m, n)) * 0.1).astype(np.float16)
    x = rng.uniform(-3, 3, size=(m, k)).astype(np.float16)
    x[:, 4] = 8.0
    w = (rng.standard_normal((n, k)) * 0.03).astype(np.float16)
    r = oracle.linear_backward(g, x, w, [4])
    G, X, W = (a.astype(np.float64) for a in (g, x, w))
    eg = np.abs(G).max(axis=1) / 254 * (1 + 2**-16)    # per row of g
    ew = np.abs(W).max(axis=0) / 254 * (1 + 2**-16)    # per column of W
    bound_x = (eg[:, None] * np.abs(W).sum(axis=0)[None, :]
               + np.abs(G) @ np.ones((n, k)) * ew[None, :] + eg[:, None] * n * ew[None, :])
    assert np.all(np.abs(r.gx - G @ W) <= bound_x + 1e-12)
    egt = np.abs(G).max(axis=0) / 254 * (1 + 2**-16)   # per column of g
    ext = np.abs(X).max(axis=0) / 254 * (1 + 2**-16)   # per column of x
    bound_w = (egt[:, None] * np.abs(X).sum(axis=0)[None, :]
               + np.abs(G).T @ np.ones((m, k)) * ext[None, :] + egt[:, None] * m * ext[None, :])
    err = np.abs(r.gw - G.T @ X)
    assert np.all(err <= bound_w + 1e-12)
    assert np.all(err[:, 4] <= 1e-9 * np.abs(G).T.sum(axis=1) * 8.0)


def test_backward_permutation_invariance():
    # permuting the output features n permutes grad_W's rows and leaves grad_x
    rng = np.random.default_rng(13)
    m, n, k = 12, 9, 7
    g = (rng.standard_normal((m, n))).astype(np.float16)
    x = rng.uniform(-4, 4, size=(m, k)).astype(np.float16)
    w = (rng.standard_normal((n, k)) * 0.1).astype(np.float16)
    p = rng.permutation(n)
    a = oracle.linear_backward(g, x, w, [])
    b = oracle.linear_backward(g[:, p], x, w[p], [])
    assert np.array_equal(a.grad_w[p], b.grad_w)
    assert np.allclose(a.gx, b.gx, rtol=1e-12, atol=0)
    # permuting the rows m leaves grad_W unchanged (column scales see the same sets)
    q = rng.permutation(m)
    c = oracle.linear_backward(g[q], x[q], w, [])
    assert np.allclose(a.gw, c.gw, rtol=1e-12, atol=0)
    assert np.array_equal(a.grad_x[q], c.grad_x)


def test_backward_zero_gradient():
    g = np.zeros((5, 3), np.float16)
    x = np.ones((5, 4), np.float16)
    w = np.ones((3, 4), np.float16)
    r = oracle.linear_backward(g, x, w, [1])
    assert not r.grad_x.any() and not r.grad_w.any()
    assert not r.gt_q.any() and r.gt_s.tolist() == [0, 0, 0]
