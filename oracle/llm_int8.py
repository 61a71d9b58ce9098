"""Plain, slow CPU oracle of the LLM.int8() vector-wise mixed-precision linear.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code,
tables or helpers with the HIP library.

What the pages fix, and what is a reading
-----------------------------------------
The method is stated in one sentence on the transformers PR page
("`bitsandbytes` - `Linear8bitLt` integration into `transformers` models",
section "About the mixed quantization method in few words"): operations on the
outliers run in fp16, all other operations in int8.  The bitsandbytes PR
"LLM.int8() Refactoring: Part 1" names the ops that carry it out (section
"Enhancements": a fused kernel for activation scale calibration and
quantization exposed as int8_vectorwise_quant; section "Deprecations":
int8_linear_matmul replacing igemmlt, int8_mm_dequant replacing mm_dequant,
extract_outliers; section "Next steps": sparse decomposition, an int8
dequantize op) and, in its review of bitsandbytes/autograd/_functions.py,
zeroes the outlier *columns* of the transposed int8 input, indexing them by
the saved outlier index list.
No formula, threshold or rounding rule is printed.  The readings used here are:

1. outliers are activation columns: O = { j : some row has |x[i, j]| >= tau };
   tau <= 0 switches outlier handling off (this is also weight quantization);
2. the row scale is the absolute maximum of the row over the columns not in O
   (0 if there is none or the row is zero); it is stored as that absmax (fp32);
3. code = clamp(round_half_even(fl32(x * fl32(127 / absmax))), -127, 127), every
   step an IEEE binary32 operation; codes in outlier columns and in rows with a
   zero absmax are 0;
4. C = A_q . W_q^T exactly (integers);
5. the outlier term uses the int8 weights: P[i, n] = sum_{j in O} x[i, j] * W_q[n, j];
6. y = (w_absmax[n] / 127) * (C[i, n] * x_absmax[i] / 127 + P[i, n]) + bias[n],
   evaluated in float64, then rounded once to fp16 (round half to even).

Where floating point decides an integer (a code), the decision is taken in
binary32 on both sides; everything after the integer GEMM is float64 here.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

# Largest K for which K * 127 * 127 fits a signed 32-bit accumulator.
INT32_SAFE_K = (2**31 - 1) // (127 * 127)


def _as_f32(x: np.ndarray) -> np.ndarray:
    if x.dtype != np.float16:
        raise TypeError(f"activations must be fp16, got {x.dtype}")
    x32 = x.astype(np.float32)          # exact widening
    if not np.all(np.isfinite(x32)):
        raise ValueError("non-finite input is outside the method's domain")
    return x32


def outlier_columns(x: np.ndarray, tau: float) -> np.ndarray:
    """Sorted column indices j with |x[i, j]| >= tau for some row i (reading 1).

    Detection of outlier feature dimensions, whose matmul runs in fp16
    (transformers PR page, "About the mixed quantization method in few words";
    bitsandbytes PR "LLM.int8() Refactoring: Part 1", extract_outliers and the
    column indexing by the outlier index list in the autograd review).
    """
    x32 = _as_f32(x)
    if tau <= 0 or x32.size == 0:
        return np.zeros(0, dtype=np.int64)
    hit = np.abs(x32) >= np.float32(tau)
    return np.nonzero(hit.any(axis=0))[0].astype(np.int64)


def outlier_bitmap(cols: np.ndarray, k: int) -> np.ndarray:
    """uint32 words, bit b of word w set iff column 32*w + b is an outlier."""
    words = np.zeros((k + 31) // 32, dtype=np.uint32)
    for j in np.asarray(cols, dtype=np.int64):
        words[j // 32] |= np.uint32(1) << np.uint32(j % 32)
    return words


def bitmap_to_columns(words: np.ndarray, k: int) -> np.ndarray:
    cols = []
    for w, v in enumerate(np.asarray(words, dtype=np.uint32)):
        for b in range(32):
            if (int(v) >> b) & 1:
                j = 32 * w + b
                if j < k:
                    cols.append(j)
    return np.array(cols, dtype=np.int64)


def row_absmax(x: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """Row scale = max |x[i, j]| over j not in O, as fp32 (reading 2).

    The "activation scale calibration" half of the fused op of the bitsandbytes
    PR ("Enhancements").  Exact: it is one of the (widened) inputs.
    """
    x32 = np.abs(_as_f32(x))
    if x32.shape[1] == 0:
        return np.zeros(x32.shape[0], dtype=np.float32)
    keep = np.ones(x32.shape[1], dtype=bool)
    keep[np.asarray(cols, dtype=np.int64)] = False
    if not keep.any():
        return np.zeros(x32.shape[0], dtype=np.float32)
    return x32[:, keep].max(axis=1).astype(np.float32)


def quantize_rows(x: np.ndarray, absmax: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """int8 codes per reading 3 (the "quantization" half of int8_vectorwise_quant).

    All arithmetic that decides a code is IEEE binary32: the factor 127/absmax
    is one correctly rounded division, the product one correctly rounded
    multiply, then round-half-to-even and a clamp to [-127, 127].
    """
    x32 = _as_f32(x)
    s = np.asarray(absmax, dtype=np.float32)
    pos = s > 0
    inv = np.zeros_like(s)
    inv[pos] = np.float32(127.0) / s[pos]                 # fl32(127 / s)
    prod = x32 * inv[:, None]                             # fl32(x * inv)
    q = np.clip(np.rint(prod), -127, 127)                 # half to even
    q[~pos, :] = 0
    q[:, np.asarray(cols, dtype=np.int64)] = 0            # outlier columns carry no int8 part
    return q.astype(np.int8)


@dataclass
class QuantResult:
    q: np.ndarray          # int8 [m, k]
    absmax: np.ndarray     # fp32 [m]
    cols: np.ndarray       # int64 sorted outlier columns
    bitmap: np.ndarray     # uint32 [ceil(k/32)]


def vectorwise_quant(x: np.ndarray, tau: float) -> QuantResult:
    """int8_vectorwise_quant: outlier detection, row calibration, quantization.

    bitsandbytes PR "LLM.int8() Refactoring: Part 1", section "Enhancements"
    (fused activation scale calibration and quantization) with the outlier
    columns of the same PR's sparse decomposition; readings 1-3.
    """
    cols = outlier_columns(x, tau)
    s = row_absmax(x, cols)
    q = quantize_rows(x, s, cols)
    return QuantResult(q, s, cols, outlier_bitmap(cols, x.shape[1]))


def quantize_weight(w: np.ndarray):
    """Row-wise int8 weight state (codes + per-row absmax), threshold off.

    The int8 weight plus its quantization statistics that replace the fp16
    weight (transformers PR page: has_fp16_weights, quantization statistics;
    bitsandbytes PR autograd review: ``CB``).
    """
    r = vectorwise_quant(w, 0.0)
    return r.q, r.absmax


def vectorwise_dequant(q: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """int8 dequantize op ("Next steps" of the bitsandbytes PR): q * absmax / 127.

    float64 result (the GPU rounds it to fp32 or fp16).
    """
    return q.astype(np.float64) * (np.asarray(absmax, np.float64)[:, None] / 127.0)


def outlier_extract(x: np.ndarray, cols: np.ndarray, cap: int):
    """extract_outliers: the fp16 sub-matrix X[:, O] and the index list.

    Returns (idx int32 [cap] with -1 past the count, count, x_out fp16 [m, cap]
    zero-padded).  Only the first ``cap`` outlier columns fit.
    """
    m = x.shape[0]
    cols = np.asarray(cols, dtype=np.int64)
    count = int(cols.size)
    idx = np.full(cap, -1, dtype=np.int32)
    use = cols[:cap]
    idx[: use.size] = use
    out = np.zeros((m, cap), dtype=np.float16)
    out[:, : use.size] = x[:, use]
    return idx, count, out


def int8_linear_matmul(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """int8_linear_matmul (replacement of igemmlt): C = A . B^T, exact int32.

    bitsandbytes PR "LLM.int8() Refactoring: Part 1", section "Deprecations".
    Computed as a float64 matmul of the integer-valued arrays: every partial
    sum is an integer of magnitude <= K * 127^2 < 2^31 < 2^53, so it is exact.
    """
    if a.dtype != np.int8 or b.dtype != np.int8:
        raise TypeError("int8 operands expected")
    if a.shape[1] != b.shape[1]:
        raise ValueError("inner dimensions differ")
    if a.shape[1] > INT32_SAFE_K:
        raise ValueError("K too large for an exact int32 accumulator")
    c = a.astype(np.float64) @ b.astype(np.float64).T
    assert np.all(np.abs(c) <= 2**31 - 1)
    return c.astype(np.int32)


def outlier_matmul(x: np.ndarray, cols: np.ndarray, w_q: np.ndarray) -> np.ndarray:
    """Sparse-decomposition term P = X[:, O] . W_q[:, O]^T in float64 (reading 5).

    bitsandbytes PR "LLM.int8() Refactoring: Part 1", "Next steps" (sparse
    decomposition); the outlier part of the mixed decomposition of the
    transformers PR page.
    """
    cols = np.asarray(cols, dtype=np.int64)
    m, n = x.shape[0], w_q.shape[0]
    if cols.size == 0:
        return np.zeros((m, n), dtype=np.float64)
    return x[:, cols].astype(np.float64) @ w_q[:, cols].astype(np.float64).T


def mm_dequant(c: np.ndarray, row_absmax: np.ndarray, col_absmax: np.ndarray,
               bias: Optional[np.ndarray] = None,
               outlier: Optional[np.ndarray] = None) -> np.ndarray:
    """int8_mm_dequant: fp16( (col_absmax/127) * (C * row_absmax/127 + P) + bias ).

    bitsandbytes PR "LLM.int8() Refactoring: Part 1", "Deprecations"
    (mm_dequant and vectorwise_mm_dequant replaced by int8_mm_dequant); reading 6.
    """
    y = _dequant_f64(c, row_absmax, col_absmax, bias, outlier)
    return y.astype(np.float16)


def _dequant_f64(c, row_absmax, col_absmax, bias, outlier):
    sx = np.asarray(row_absmax, dtype=np.float64)[:, None]
    sw = np.asarray(col_absmax, dtype=np.float64)[None, :]
    y = c.astype(np.float64) * sx / 127.0
    if outlier is not None:
        y = y + outlier
    y = (sw / 127.0) * y
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y


@dataclass
class ForwardResult:
    out: np.ndarray        # fp16 [m, n]
    y: np.ndarray          # float64 [m, n] before the final fp16 rounding
    quant: QuantResult
    c: np.ndarray          # int32 [m, n]
    p: np.ndarray          # float64 [m, n] outlier term


def linear_forward(x: np.ndarray, w_q: np.ndarray, w_absmax: np.ndarray,
                   bias: Optional[np.ndarray], tau: float) -> ForwardResult:
    """The whole mixed-precision linear, steps in the order the method takes them.

    int8_vectorwise_quant -> int8_linear_matmul -> sparse-decomposition term ->
    int8_mm_dequant (+ bias), per the bitsandbytes PR "LLM.int8() Refactoring:
    Part 1" and the method statement of the transformers PR page.
    """
    qr = vectorwise_quant(x, tau)
    c = int8_linear_matmul(qr.q, w_q)
    p = outlier_matmul(x, qr.cols, w_q)
    y = _dequant_f64(c, qr.absmax, w_absmax, bias, p)
    return ForwardResult(y.astype(np.float16), y, qr, c, p)
