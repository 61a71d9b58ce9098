"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test checks the oracle against: exact rational arithmetic with IEEE
rounding written from its definition (brute_int8), hand-worked values,
closed forms, invariants of the method, or a different library routine.
The pages print no worked example for this path, so nothing here pins the
oracle to numbers on the pages themselves.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from brute_int8 import BruteLinear, brute_weight_quant, f16, f32, quant_code
from synth import make_inputs

# ----------------------------------------------------------------------------
# hand-worked examples
# ----------------------------------------------------------------------------


def test_hand_worked_linear():
    # X row 0 = [1, -2, 0.5, 8], row 1 = [0, 0, 0, 7]; tau = 6.
    #   O = {3}: both rows reach 6 in column 3 only.
    #   row 0: absmax over columns {0,1,2} = 2, fl32(127/2) = 63.5 exactly;
    #          1*63.5 = 63.5 -> tie -> even 64; -2*63.5 = -127; 0.5*63.5 = 31.75 -> 32.
    #   row 1: no nonzero value outside O -> absmax 0, all codes 0.
    # W_q = [[1, 2, 3, 4]], w_absmax = 127 (so W_deq = W_q).
    #   C = [64 - 254 + 96, 0] = [-94, 0];  P = [8*4, 7*4] = [32, 28].
    #   y0 = -94*2/127 + 32 = 30.5196850...; fp16 spacing in [16, 32) is 1/64,
    #   30.5196850 * 64 = 1953.26 -> 1953/64 = 30.515625.   y1 = 28.
    x = np.array([[1, -2, 0.5, 8], [0, 0, 0, 7]], dtype=np.float16)
    wq = np.array([[1, 2, 3, 4]], dtype=np.int8)
    sw = np.array([127.0], dtype=np.float32)
    r = oracle.linear_forward(x, wq, sw, None, 6.0)
    assert r.quant.cols.tolist() == [3]
    assert r.quant.absmax.tolist() == [2.0, 0.0]
    assert r.quant.q.tolist() == [[64, -127, 32, 0], [0, 0, 0, 0]]
    assert r.c.tolist() == [[-94], [0]]
    assert r.p.tolist() == [[32.0], [28.0]]
    assert r.out.astype(np.float64).tolist() == [[30.515625], [28.0]]
    assert r.quant.bitmap.tolist() == [0b1000]


def test_hand_worked_ties_round_to_even():
    # absmax 127 -> factor exactly 1 -> the code is x rounded half to even.
    x = np.array([[127, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, 126.5]], dtype=np.float16)
    r = oracle.vectorwise_quant(x, 0.0)
    assert r.q.tolist() == [[127, 2, 4, -2, 0, 2, 0, 126]]
    assert r.absmax.tolist() == [127.0]


def test_hand_worked_outlier_extract_and_bitmap():
    # columns 0, 33 and 64 are outliers in a 70-wide input
    x = np.zeros((2, 70), dtype=np.float16)
    x[0, 0] = 7
    x[1, 33] = -9
    x[0, 64] = 6  # exactly tau: counts (>=)
    x[1, 64] = 1
    x[0, 5] = 5.99  # below tau
    r = oracle.vectorwise_quant(x, 6.0)
    assert r.cols.tolist() == [0, 33, 64]
    assert r.bitmap.tolist() == [1, 2, 1]
    assert oracle.bitmap_to_columns(r.bitmap, 70).tolist() == [0, 33, 64]
    idx, count, xo = oracle.outlier_extract(x, r.cols, 4)
    assert count == 3
    assert idx.tolist() == [0, 33, 64, -1]
    assert xo.astype(np.float64).tolist() == [[7, 0, 6, 0], [0, -9, 1, 0]]
    # capacity smaller than the count keeps the first columns
    idx2, count2, xo2 = oracle.outlier_extract(x, r.cols, 2)
    assert count2 == 3 and idx2.tolist() == [0, 33]
    assert xo2.astype(np.float64).tolist() == [[7, 0], [0, -9]]


# ----------------------------------------------------------------------------
# brute force on tiny inputs (exact rationals, IEEE rounding from its definition)
# ----------------------------------------------------------------------------


def _tiny_case(rng, m, k, n, tau):
    x = rng.uniform(-5, 5, size=(m, k)).astype(np.float16)
    # plant: one column fully large, one column with a single large element,
    # one element exactly equal to tau, and a zero row when m > 2
    if k >= 2:
        x[:, rng.integers(k)] = rng.choice([-1, 1], m) * rng.uniform(6, 9, m)
    if k >= 3:
        x[rng.integers(m), rng.integers(k)] = np.float16(-7.5)
    x[rng.integers(m), rng.integers(k)] = np.float16(tau)
    if m > 2:
        x[rng.integers(m), :] = 0
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float16)
    b = (rng.standard_normal(n) * 0.01).astype(np.float16) if rng.random() < 0.5 else None
    return x.astype(np.float16), w, b


def _near_f16_midpoint(y: Fraction) -> bool:
    r = f16(y)
    # distance to the nearest rounding boundary relative to the spacing
    lo, hi = f16(y - abs(y) * Fraction(1, 2**30)), f16(y + abs(y) * Fraction(1, 2**30))
    return lo != r or hi != r


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng([99, seed])
    m, k, n = (int(v) for v in rng.integers(1, 7, size=3))
    tau = 6.0
    x, w, b = _tiny_case(rng, m, k, n, tau)
    wq, sw = oracle.quantize_weight(w)
    bq, bs = brute_weight_quant(w.astype(np.float64).tolist())
    assert wq.tolist() == bq
    assert [Fraction(float(v)) for v in sw] == bs
    br = BruteLinear(x.astype(np.float64).tolist(), wq.tolist(), sw.astype(np.float64).tolist(),
                     None if b is None else b.astype(np.float64).tolist(), tau)
    r = oracle.linear_forward(x, wq, sw, b, tau)
    assert r.quant.cols.tolist() == br.cols
    assert [Fraction(float(v)) for v in r.quant.absmax] == br.absmax
    assert r.quant.q.tolist() == br.q
    assert r.c.tolist() == br.c
    for i in range(m):
        for j in range(n):
            assert Fraction(float(r.p[i, j])) == br.p[i][j]  # few exact products: no rounding
            got = Fraction(float(r.out[i, j]))
            if not _near_f16_midpoint(br.y[i][j]):
                assert got == br.out[i][j], (i, j, float(br.y[i][j]))


# ----------------------------------------------------------------------------
# exhaustive code check over every finite fp16 value (integer-exact rounding)
# ----------------------------------------------------------------------------


def _all_finite_f16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    return v[np.isfinite(v)]


def _rne_int_exact(r: np.ndarray) -> np.ndarray:
    """Round float64 values that hold exact dyadic rationals half-to-even, using
    only exact operations (floor, subtraction of representable values)."""
    fl = np.floor(r)
    frac = r - fl
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(fl, 2) == 1))
    return fl + up


def _fl32_of_exact(p: np.ndarray) -> np.ndarray:
    """Round exact float64 products (<= 35 significant bits) to binary32, RNE,
    by scaling the significand to 24 bits and rounding it as an integer."""
    mant, e = np.frexp(p)                 # p = mant * 2**e, 0.5 <= |mant| < 1
    r = np.ldexp(mant, 24)                # exact
    r = _rne_int_exact(r)
    return np.ldexp(r, e - 24)


def _scales():
    s = [2.0 ** e for e in range(-24, 16)]
    rng = np.random.default_rng(7)
    f = _all_finite_f16()
    pos = f[f > 0]
    s += [float(v) for v in rng.choice(pos, 300, replace=False)]
    s += [65504.0, 6.0, 5.9990234375, 127.0, 100.0, 3.0, 1.0009765625]
    return sorted(set(s))


def test_exhaustive_codes_all_fp16():
    xs = _all_finite_f16()
    xs64 = xs.astype(np.float64)
    checked = 0
    for s in _scales():
        sel = np.abs(xs64) <= s
        xv = xs[sel]
        inv = float(f32(Fraction(127) / Fraction(s)))          # exact binary32 value
        prod = _fl32_of_exact(xv.astype(np.float64) * inv)     # exact product, then fl32
        want = np.clip(_rne_int_exact(prod), -127, 127).astype(np.int8)
        got = oracle.quantize_rows(xv[None, :], np.array([s], np.float32), np.zeros(0, np.int64))[0]
        assert np.array_equal(got, want), s
        # symmetry of the code
        assert np.array_equal(got, -oracle.quantize_rows(
            (-xv)[None, :], np.array([s], np.float32), np.zeros(0, np.int64))[0])
        checked += xv.size
    assert checked > 5_000_000
    # spot-check the integer route against the Fraction route on a sample
    rng = np.random.default_rng(3)
    for _ in range(300):
        s = float(rng.choice([v for v in _scales()]))
        cand = xs[np.abs(xs.astype(np.float64)) <= s]
        xv = float(rng.choice(cand))
        got = oracle.quantize_rows(np.array([[xv]], np.float16), np.array([s], np.float32),
                                   np.zeros(0, np.int64))[0, 0]
        assert int(got) == quant_code(Fraction(xv), Fraction(s))


def test_absmax_element_codes_to_127():
    xs = _all_finite_f16()
    xs = xs[xs != 0]
    s = np.abs(xs.astype(np.float32))
    # one row per value, the value is its row's absmax
    # every value as its own row's absmax (one row per value)
    q = oracle.quantize_rows(xs[:, None], s, np.zeros(0, np.int64))[:, 0]
    sign = np.sign(xs.astype(np.float64))
    assert np.array_equal(q.astype(np.float64), 127 * sign)


# ----------------------------------------------------------------------------
# closed forms and special cases
# ----------------------------------------------------------------------------


def _layer(seed, m, k, n, o, bias=True, frac=1.0):
    L = make_inputs(m, k, n, n_outlier=o, lo=6.0, hi=60.0, bias_std=0.01 if bias else None,
                    seed=(50, seed, 0), outlier_row_frac=frac)
    wq, sw = oracle.quantize_weight(L.w)
    return L, wq, sw


@pytest.mark.parametrize("seed,m,k,n,o,frac", [
    (0, 7, 64, 9, 3, 1.0), (1, 33, 257, 40, 5, 1.0), (2, 16, 1024, 64, 4, 0.3),
    (3, 1, 100, 5, 0, 1.0), (4, 64, 96, 17, 12, 0.05),
])
def test_error_bound_against_exact_product(seed, m, k, n, o, frac):
    """|y - (x . W_deq^T + b)| <= (s_x/254)(1 + 2^-13) * sum_{j not in O} |W_deq[n, j]|.

    Each code is within half a step of x*127/s (plus binary32 rounding of the
    factor and the product); the outlier term and bias are exact in y.
    """
    L, wq, sw = _layer(seed, m, k, n, o, frac=frac)
    r = oracle.linear_forward(L.x, wq, sw, L.bias, 6.0)
    wdeq = wq.astype(np.float64) * (sw.astype(np.float64)[:, None] / 127.0)
    exact = L.x.astype(np.float64) @ wdeq.T + L.bias.astype(np.float64)[None, :]
    keep = np.ones(k, bool)
    keep[r.quant.cols] = False
    bound = (r.quant.absmax.astype(np.float64)[:, None] / 254.0) * (1 + 2.0**-13) \
        * np.abs(wdeq[:, keep]).sum(axis=1)[None, :]
    err = np.abs(r.y - exact)
    assert np.all(err <= bound + 1e-12 * (1 + np.abs(exact)))
    # the planted columns are exactly the outlier set
    assert r.quant.cols.tolist() == L.planted_cols.tolist()
    # a dropped outlier term would break the bound on these inputs
    if o:
        y_bad = r.y - (sw.astype(np.float64)[None, :] / 127.0) * r.p
        assert np.any(np.abs(y_bad - exact) > bound + 1e-12)


def test_no_outliers_is_pure_int8():
    L, wq, sw = _layer(10, 24, 300, 31, 0)
    r = oracle.linear_forward(L.x, wq, sw, L.bias, 0.0)
    assert r.quant.cols.size == 0 and not r.p.any()
    c64 = r.quant.q.astype(np.int64) @ wq.astype(np.int64).T      # integer matmul, other routine
    assert np.array_equal(r.c.astype(np.int64), c64)
    y = (sw.astype(np.float64)[None, :] / 127) * (c64 * r.quant.absmax.astype(np.float64)[:, None] / 127) \
        + L.bias.astype(np.float64)[None, :]
    assert np.array_equal(r.out, y.astype(np.float16))


def test_all_columns_outliers_is_fp16_matmul():
    rng = np.random.default_rng(11)
    x = rng.uniform(0.5, 4, size=(12, 40)).astype(np.float16) * rng.choice([-1, 1], (12, 40)).astype(np.float16)
    w = (rng.standard_normal((9, 40)) * 0.02).astype(np.float16)
    b = (rng.standard_normal(9) * 0.01).astype(np.float16)
    wq, sw = oracle.quantize_weight(w)
    r = oracle.linear_forward(x, wq, sw, b, 2.0**-24)   # every nonzero column is an outlier
    assert r.quant.cols.size == 40
    assert not r.quant.q.any() and not r.quant.absmax.any() and not r.c.any()
    wdeq = wq.astype(np.float64) * (sw.astype(np.float64)[:, None] / 127.0)
    exact = x.astype(np.float64) @ wdeq.T + b.astype(np.float64)
    assert np.allclose(r.y, exact, rtol=1e-13, atol=1e-15)
    ulp = np.spacing(np.abs(exact).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(r.out.astype(np.float64) - exact) <= ulp)


def test_zero_input_gives_bias():
    L, wq, sw = _layer(12, 5, 70, 13, 0)
    x = np.zeros_like(L.x)
    r = oracle.linear_forward(x, wq, sw, L.bias, 6.0)
    assert not r.quant.q.any() and not r.quant.absmax.any()
    assert np.array_equal(r.out, L.bias[None, :].repeat(5, 0))


def test_zero_rows_inside_a_batch():
    L, wq, sw = _layer(13, 9, 128, 7, 2)
    x = L.x.copy()
    x[[1, 4], :] = 0
    r = oracle.linear_forward(x, wq, sw, None, 6.0)
    assert r.quant.absmax[1] == 0 and r.quant.absmax[4] == 0
    assert not r.quant.q[[1, 4]].any() and not r.c[[1, 4]].any()


def test_one_nonzero_per_row():
    rng = np.random.default_rng(14)
    m, k, n = 6, 50, 8
    x = np.zeros((m, k), np.float16)
    cols = rng.choice(k, m, replace=False)
    vals = rng.uniform(0.1, 5, m) * rng.choice([-1, 1], m)
    x[np.arange(m), cols] = vals
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float16)
    wq, sw = oracle.quantize_weight(w)
    r = oracle.linear_forward(x, wq, sw, None, 6.0)
    sign = np.sign(x[np.arange(m), cols].astype(np.float64)).astype(np.int64)
    assert np.array_equal(r.c.astype(np.int64), 127 * sign[:, None] * wq[:, cols].T.astype(np.int64))


def test_weight_quant_reaches_127_on_every_row():
    w = (np.random.default_rng(15).standard_normal((33, 77)) * 0.02).astype(np.float16)
    wq, sw = oracle.quantize_weight(w)
    assert np.all(np.abs(wq).max(axis=1) == 127)
    assert np.array_equal(sw, np.abs(w.astype(np.float32)).max(axis=1))
    assert wq.min() >= -127


def test_dequant_op():
    q = np.array([[127, -127, 0, 64]], np.int8)
    s = np.array([2.5], np.float32)
    d = oracle.vectorwise_dequant(q, s)
    assert d[0, 0] == 2.5 and d[0, 1] == -2.5 and d[0, 2] == 0
    assert d[0, 3] == pytest.approx(64 * 2.5 / 127, rel=1e-15)


# ----------------------------------------------------------------------------
# metamorphic invariants
# ----------------------------------------------------------------------------


def test_k_permutation_invariance():
    """Reordering K in both operands (the exllama s_col(A) s_row(B) = A B identity)."""
    L, wq, sw = _layer(20, 20, 200, 11, 5, frac=0.5)
    r = oracle.linear_forward(L.x, wq, sw, L.bias, 6.0)
    perm = np.random.default_rng(21).permutation(200)
    r2 = oracle.linear_forward(L.x[:, perm], wq[:, perm], sw, L.bias, 6.0)
    inv = np.argsort(perm)
    assert sorted(inv[r.quant.cols].tolist()) == r2.quant.cols.tolist()
    assert np.array_equal(r2.quant.absmax, r.quant.absmax)
    assert np.array_equal(r2.quant.q, r.quant.q[:, perm])
    assert np.array_equal(r2.c, r.c)
    assert np.allclose(r2.y, r.y, rtol=1e-12, atol=1e-14)


def test_row_permutation_and_negation():
    L, wq, sw = _layer(22, 17, 90, 6, 3, frac=0.4)
    r = oracle.vectorwise_quant(L.x, 6.0)
    perm = np.random.default_rng(23).permutation(17)
    rp = oracle.vectorwise_quant(L.x[perm], 6.0)
    assert np.array_equal(rp.cols, r.cols)
    assert np.array_equal(rp.q, r.q[perm]) and np.array_equal(rp.absmax, r.absmax[perm])
    rn = oracle.vectorwise_quant(-L.x, 6.0)
    assert np.array_equal(rn.cols, r.cols) and np.array_equal(rn.q, -r.q)
    assert np.array_equal(rn.absmax, r.absmax)


@pytest.mark.parametrize("e", [1, 2, 3])
def test_power_of_two_scaling(e):
    L, wq, sw = _layer(24, 13, 120, 5, 2, frac=0.6)
    x2 = (L.x.astype(np.float32) * 2.0**e).astype(np.float16)
    assert np.array_equal(x2.astype(np.float32), L.x.astype(np.float32) * 2.0**e)  # exact scaling
    r = oracle.vectorwise_quant(L.x, 6.0)
    r2 = oracle.vectorwise_quant(x2, 6.0 * 2**e)
    assert np.array_equal(r2.cols, r.cols) and np.array_equal(r2.q, r.q)
    assert np.array_equal(r2.absmax, r.absmax * np.float32(2.0**e))


# ----------------------------------------------------------------------------
# integer range and library conversions
# ----------------------------------------------------------------------------


def test_int32_bound():
    k = oracle.INT32_SAFE_K
    assert k == 133144
    a = np.full((1, k), 127, np.int8)
    c = oracle.int8_linear_matmul(a, a)
    assert int(c[0, 0]) == 2147479576
    big = np.full((1, k + 1), 127, np.int8)
    with pytest.raises(ValueError):
        oracle.int8_linear_matmul(big, big)


def test_numpy_f16_rounding_matches_definition():
    """The oracle's final fp16 rounding (numpy float64 -> float16) is RNE."""
    rng = np.random.default_rng(30)
    vals = list(rng.uniform(-100, 100, 2000)) + [1 + 2**-11, 1 + 3 * 2**-11, -(1 + 2**-11),
                                                  2**-24 * 1.5, 2**-25, 65519.0, 0.0]
    for v in vals:
        assert float(np.float64(v).astype(np.float16)) == float(f16(Fraction(v)))


def test_numpy_f32_division_is_correctly_rounded():
    rng = np.random.default_rng(31)
    f = _all_finite_f16()
    pos = f[f > 0]
    for s in rng.choice(pos, 400):
        got = np.float32(127.0) / np.float32(s)
        assert Fraction(float(got)) == f32(Fraction(127) / Fraction(float(s)))
