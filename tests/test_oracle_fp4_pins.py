"""Pins of the 4-bit (FP4 E2M1, blocks of 64, double quantization) oracle.

Checked against: the E2M1 values rebuilt from the fp16 bit layout, a
threshold-count formulation of round-to-nearest-even over every finite fp16
value, exact rational arithmetic on small cases, inputs built so that the
quantization is exact, closed-form error bounds, and properties of the double
quantization.  No GPU.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import fp4
from brute_int8 import f32
from test_oracle_pins import _all_finite_f16, _scales


def test_e2m1_values_from_the_fp16_bit_layout():
    # E2M1 with exponent bias 1 embeds in fp16: exponent e >= 1 -> fp16 exponent
    # e - 1 + 15, mantissa bit -> the top fp16 mantissa bit; e = 0 is 0 or 0.5
    want = []
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e == 0:
            bits = (s << 15) | ((14 << 10) if m else 0)       # 0.5 = 2^-1 -> exponent field 14
        else:
            bits = (s << 15) | ((e - 1 + 15) << 10) | (m << 9)
        want.append(float(np.array([bits], np.uint16).view(np.float16)[0]))
    got = fp4.e2m1_value(np.arange(16)).tolist()
    assert [abs(v) for v in got] == [abs(v) for v in want]
    assert np.array_equal(np.signbit(got), np.signbit(want))
    assert got[:8] == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _mag_by_thresholds(v: np.ndarray) -> np.ndarray:
    """Nearest E2M1 magnitude code with ties to the even code, as a count of the
    midpoints below v plus the three midpoints whose upper neighbour is even."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    v = np.minimum(v, 6.0)
    code = (v[:, None] > mids[None, :]).sum(axis=1)
    code += np.isin(v, [0.75, 1.75, 3.5])
    return code.astype(np.uint8)


def test_codes_exhaustive_all_fp16():
    xs = _all_finite_f16()
    checked = 0
    for a in _scales():
        if float(np.float16(a)) != a or a <= 0:
            continue
        blk = xs[np.abs(xs.astype(np.float64)) <= a]
        inv = float(f32(Fraction(6) / Fraction(a)))
        v = (np.abs(blk.astype(np.float64)) * inv).astype(np.float32).astype(np.float64)  # fl32 of the exact product
        want_mag = _mag_by_thresholds(v)
        # one block per 63 values plus the scale element itself
        pad = (-blk.size) % 63
        body = np.concatenate([blk, np.zeros(pad, np.float16)]).reshape(-1, 63)
        w = np.concatenate([np.full((body.shape[0], 1), a, np.float16), body], axis=1)
        codes, absmax = fp4.fp4_quantize(w)
        assert np.all(absmax == np.float32(a))
        got = codes[:, 1:].reshape(-1)[: blk.size]
        assert np.array_equal(got & 7, want_mag), a
        assert np.array_equal(got >> 3, (blk.view(np.uint16) >> 15).astype(np.uint8))
        assert np.all(codes[:, 0] == 7)                      # the absmax element maps to 6
        checked += blk.size
    assert checked > 2_000_000


def test_hand_worked_block():
    w = np.zeros((1, 64), np.float16)
    w[0, :8] = [12.0, -6.0, 1.0, 3.0, 5.0, 7.0, -0.0, 0.5]   # absmax 12: v = w / 2
    codes, absmax = fp4.fp4_quantize(w)
    assert absmax.tolist() == [[12.0]]
    # v = 6, -3, 0.5, 1.5, 2.5 (tie -> 2), 3.5 (tie -> 4), -0, 0.25 (tie -> 0)
    assert codes[0, :8].tolist() == [7, 8 | 5, 1, 3, 4, 6, 8, 0]
    d = fp4.fp4_dequantize(codes, absmax)
    assert d[0, :8].tolist() == [12.0, -6.0, 1.0, 3.0, 4.0, 8.0, -0.0, 0.0]


def test_zero_block_and_packing():
    w = np.zeros((2, 128), np.float16)
    w[1, 64:] = np.linspace(-1, 1, 64).astype(np.float16)
    codes, absmax = fp4.fp4_quantize(w)
    assert absmax[0].tolist() == [0.0, 0.0] and absmax[1, 0] == 0.0
    assert not (codes[0] & 7).any()
    p = fp4.pack_nibbles(codes)
    assert p.shape == (2, 64)
    assert np.array_equal(fp4.unpack_nibbles(p), codes)
    assert p[1, 32] == (codes[1, 64] | (codes[1, 65] << 4))


@pytest.mark.parametrize("seed", range(5))
def test_linear_exact_when_weights_are_on_the_grid(seed):
    # each block: E2M1 values times 2^e with one +-6 * 2^e: codes reproduce w
    # exactly, so the 4-bit linear must equal x . w^T exactly in float64
    rng = np.random.default_rng([20, seed])
    n, k, m = 9, 256, 3
    grid = fp4.e2m1_value(np.arange(16))
    idx = rng.integers(0, 16, size=(n, k))
    e = rng.integers(-8, 3, size=(n, k // 64))
    w = grid[idx] * np.repeat(np.exp2(e), 64, axis=1)
    w[np.arange(n)[:, None], np.arange(0, k, 64)[None, :]] = 6.0 * np.exp2(e)
    w = w.astype(np.float16)
    x = (rng.integers(-64, 65, size=(m, k)) / 8).astype(np.float16)
    codes, absmax = fp4.fp4_quantize(w)
    assert np.array_equal(fp4.fp4_dequantize(codes, absmax), w.astype(np.float32))
    _, y = fp4.fp4_linear(x, codes, absmax)
    assert np.array_equal(y, x.astype(np.float64) @ w.astype(np.float64).T)


@pytest.mark.parametrize("seed", range(4))
def test_round_trip_error_bound(seed):
    rng = np.random.default_rng([21, seed])
    w = (rng.standard_normal((16, 512)) * 0.03).astype(np.float16)
    codes, absmax = fp4.fp4_quantize(w)
    d = fp4.fp4_dequantize(codes, absmax).astype(np.float64)
    a = np.repeat(absmax.astype(np.float64), 64, axis=1)
    v = np.abs(w.astype(np.float64)) * 6 / a
    # half the local grid gap: 0.25 below 2, 0.5 in [2, 4], 1 in [4, 6]
    half_gap = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    err = np.abs(d - w.astype(np.float64))
    assert np.all(err <= half_gap * a / 6 * (1 + 2**-20) + 1e-12)
    assert np.array_equal(np.sign(d[d != 0]), np.sign(w.astype(np.float64)[d != 0]))


def test_double_quant_properties():
    rng = np.random.default_rng(22)
    a = rng.uniform(0.001, 0.2, size=(37, 20)).astype(np.float32)   # 740 scales: groups 256, 256, 228
    a[5, 3] = 0.0
    c8, s2 = fp4.double_quant(a)
    flat = a.reshape(-1)
    assert s2.shape == (3,) and c8.shape == (740,)
    for gi in range(3):
        blk = flat[gi * 256:(gi + 1) * 256]
        assert s2[gi] == blk.max()
        assert c8[gi * 256 + int(np.argmax(blk))] == 255
    assert c8[5 * 20 + 3] == 0
    r = fp4.double_dequant(c8, s2)
    step = np.repeat(s2.astype(np.float64), 256)[:740] / 255
    assert np.all(np.abs(r.astype(np.float64) - flat) <= step / 2 * (1 + 2**-20) + 1e-12)
    # codes by exact rationals on a sample
    for j in rng.choice(740, 60, replace=False):
        s = Fraction(float(s2[j // 256]))
        inv = f32(Fraction(255) / s)
        p = f32(Fraction(float(flat[j])) * inv)
        q = int(p.numerator // p.denominator)
        rem = p - q
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and q % 2 == 1):
            q += 1
        assert c8[j] == min(255, max(0, q))


@pytest.mark.parametrize("seed", range(10))
def test_linear_brute_force_tiny(seed):
    rng = np.random.default_rng([23, seed])
    n, m = int(rng.integers(1, 4)), int(rng.integers(1, 3))
    k = 64 * int(rng.integers(1, 3))
    w = (rng.standard_normal((n, k)) * rng.choice([0.01, 1.0])).astype(np.float16)
    x = rng.standard_normal((m, k)).astype(np.float16)
    b = rng.standard_normal(n).astype(np.float16)
    codes, absmax = fp4.fp4_quantize(w)
    out, y = fp4.fp4_linear(x, codes, absmax, b)
    grid = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    for r in range(n):
        for blk in range(k // 64):
            seg = [Fraction(float(v)) for v in w[r, blk * 64:(blk + 1) * 64]]
            a = max(abs(v) for v in seg)
            assert Fraction(float(absmax[r, blk])) == a
            inv = f32(Fraction(6) / a) if a else Fraction(0)
            for j, v in enumerate(seg):
                t = min(f32(abs(v) * inv), Fraction(6))
                dist = [abs(t - g) for g in grid]
                best = min(dist)
                cands = [i for i, dd in enumerate(dist) if dd == best]
                mag = [i for i in cands if i % 2 == 0][0] if len(cands) > 1 else cands[0]
                assert codes[r, blk * 64 + j] & 7 == mag
    wq = [[(-1 if codes[r, j] & 8 else 1) * f32(grid[codes[r, j] & 7] * f32(Fraction(float(absmax[r, j // 64])) / 6))
           for j in range(k)] for r in range(n)]
    for i in range(m):
        for r in range(n):
            exact = sum((Fraction(float(x[i, j])) * wq[r][j] for j in range(k)), Fraction(0)) + Fraction(float(b[r]))
            assert abs(Fraction(float(y[i, r])) - exact) <= abs(exact) * Fraction(1, 2**50) + Fraction(1, 2**60)


def test_double_dequant_exact_rationals():
    """The reconstructed scale fl32(c8 * fl32(s2 / 255)) for every code 0..255
    under a set of group maxima, against exact rationals rounded to binary32
    twice, as F4 reads.  A one-rounding (float64) evaluation of the same
    product differs on this set, so the pin tells the two apart."""
    rng = np.random.default_rng(24)
    s2 = np.concatenate([rng.uniform(1e-4, 1.0, 6), [0.1, 0.2, 1.0 / 3.0]]).astype(np.float32)
    c8 = np.tile(np.arange(256, dtype=np.uint8), s2.size)
    r = fp4.double_dequant(c8, s2)
    for j in range(c8.size):
        step = f32(Fraction(float(s2[j // 256])) / 255)
        assert Fraction(float(r[j])) == f32(Fraction(int(c8[j])) * step), j
    one_rounding = (c8.astype(np.float64) * (np.repeat(s2.astype(np.float64), 256) / 255.0)).astype(np.float32)
    assert not np.array_equal(one_rounding, r)
