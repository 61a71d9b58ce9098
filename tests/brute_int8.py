"""Independent exact-arithmetic checker for the CPU oracle (tests only).

Pure Python: every value is a ``fractions.Fraction``; IEEE binary32 and
binary16 round-to-nearest-even are implemented here from their definition
(significand width, exponent range, ties to the even significand), without
numpy's floating point.  Used on tiny inputs to pin the vectorized oracle.
"""

from __future__ import annotations

from fractions import Fraction
from typing import List, Optional, Sequence

# (significand bits including the hidden one, minimum normal exponent, maximum exponent)
BINARY32 = (24, -126, 127)
BINARY16 = (11, -14, 15)


def _floor_log2(a: Fraction) -> int:
    """Largest e with 2**e <= a, for a > 0 (exact)."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # correct by at most one step either way
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_half_even_int(a: Fraction) -> int:
    n = a.numerator // a.denominator          # floor
    rem = a - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def round_to_format(a: Fraction, fmt=BINARY32) -> Fraction:
    """Round an exact rational to the nearest value of an IEEE binary format.

    Ties go to the even significand; results beyond the largest finite value
    raise OverflowError (never produced on the method's domain).
    """
    p, emin, emax = fmt
    if a == 0:
        return Fraction(0)
    sign = -1 if a < 0 else 1
    mag = -a if a < 0 else a
    e = max(_floor_log2(mag), emin)
    ulp = Fraction(2) ** (e - (p - 1))
    r = round_half_even_int(mag / ulp) * ulp
    if r >= Fraction(2) ** (emax + 1):
        raise OverflowError("beyond the format's range")
    return sign * r


def f32(a: Fraction) -> Fraction:
    return round_to_format(a, BINARY32)


def f16(a: Fraction) -> Fraction:
    return round_to_format(a, BINARY16)


def quant_code(x: Fraction, s: Fraction) -> int:
    """Code of x under row absmax s > 0: clamp(rne(fl32(x * fl32(127 / s))))."""
    inv = f32(Fraction(127) / s)
    prod = f32(x * inv)
    q = round_half_even_int(prod)
    return max(-127, min(127, q))


class BruteLinear:
    """Nested-loop evaluation of the whole linear on lists of exact rationals."""

    def __init__(self, x: Sequence[Sequence[float]], w_q: Sequence[Sequence[int]],
                 w_absmax: Sequence[float], bias: Optional[Sequence[float]], tau: float):
        self.m = len(x)
        self.k = len(x[0]) if self.m else 0
        self.n = len(w_q)
        X = [[Fraction(float(v)) for v in row] for row in x]
        T = Fraction(float(tau))
        # outlier columns
        O: List[int] = []
        if tau > 0:
            for j in range(self.k):
                for i in range(self.m):
                    if abs(X[i][j]) >= T:
                        O.append(j)
                        break
        self.cols = O
        inO = set(O)
        # row absmax over non-outlier columns
        S = []
        for i in range(self.m):
            best = Fraction(0)
            for j in range(self.k):
                if j not in inO and abs(X[i][j]) > best:
                    best = abs(X[i][j])
            S.append(best)
        self.absmax = S
        # codes
        Q = []
        for i in range(self.m):
            row = []
            for j in range(self.k):
                if j in inO or S[i] == 0:
                    row.append(0)
                else:
                    row.append(quant_code(X[i][j], S[i]))
            Q.append(row)
        self.q = Q
        # exact integer GEMM and exact outlier term
        C = [[sum(Q[i][kk] * int(w_q[nn][kk]) for kk in range(self.k)) for nn in range(self.n)]
             for i in range(self.m)]
        self.c = C
        P = [[sum((X[i][j] * int(w_q[nn][j]) for j in O), Fraction(0)) for nn in range(self.n)]
             for i in range(self.m)]
        self.p = P
        SW = [Fraction(float(v)) for v in w_absmax]
        B = [Fraction(float(v)) for v in bias] if bias is not None else [Fraction(0)] * self.n
        Y = [[(SW[nn] / 127) * (C[i][nn] * S[i] / 127 + P[i][nn]) + B[nn] for nn in range(self.n)]
             for i in range(self.m)]
        self.y = Y
        self.out = [[f16(v) for v in row] for row in Y]


def brute_weight_quant(w: Sequence[Sequence[float]]):
    """Row-wise int8 weight codes and absmax with no outlier handling."""
    q, s = [], []
    for row in w:
        R = [Fraction(float(v)) for v in row]
        a = max((abs(v) for v in R), default=Fraction(0))
        s.append(a)
        q.append([0 if a == 0 else quant_code(v, a) for v in R])
    return q, s


def brute_colwise_quant(a: Sequence[Sequence[float]], zero_cols: Sequence[int] = ()):
    """Column-wise codes, transposed ([c][r]), and column absmax, by nested loops."""
    r = len(a)
    c = len(a[0]) if r else 0
    A = [[Fraction(float(v)) for v in row] for row in a]
    zc = set(zero_cols)
    qt, s = [], []
    for j in range(c):
        col = [A[i][j] for i in range(r)]
        sj = max((abs(v) for v in col), default=Fraction(0))
        s.append(sj)
        qt.append([0 if (sj == 0 or j in zc) else quant_code(v, sj) for v in col])
    return qt, s


class BruteBackward:
    """Nested-loop evaluation of both gradients on exact rationals (tiny inputs)."""

    def __init__(self, g, x, w, cols):
        m, n, k = len(g), len(w), len(w[0])
        G = [[Fraction(float(v)) for v in row] for row in g]
        X = [[Fraction(float(v)) for v in row] for row in x]
        # grad_x: g row-wise (threshold off), W column-wise
        gq, gs = brute_weight_quant(g)
        wtq, wts = brute_colwise_quant(w)
        self.c_x = [[sum(gq[i][nn] * wtq[j][nn] for nn in range(n)) for j in range(k)] for i in range(m)]
        self.gx = [[(wts[j] / 127) * (self.c_x[i][j] * gs[i] / 127) for j in range(k)] for i in range(m)]
        # grad_W: g column-wise, x column-wise with the outlier columns zeroed
        gtq, gts = brute_colwise_quant(g)
        xtq, xts = brute_colwise_quant(x, cols)
        self.c_w = [[sum(gtq[nn][i] * xtq[j][i] for i in range(m)) for j in range(k)] for nn in range(n)]
        oc = set(cols)
        self.gw = [[(sum((G[i][nn] * X[i][j] for i in range(m)), Fraction(0)) if j in oc else
                     (xts[j] / 127) * (self.c_w[nn][j] * gts[nn] / 127)) for j in range(k)] for nn in range(n)]
        self.g_q, self.g_s, self.wt_q, self.wt_s = gq, gs, wtq, wts
        self.gt_q, self.gt_s, self.xt_q, self.xt_s = gtq, gts, xtq, xts
