"""Plain, slow CPU oracle of the backward pass through the int8 linear.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code,
tables or helpers with the HIP library.

What the pages fix, and what is a reading
-----------------------------------------
The bitsandbytes PR "LLM.int8() Refactoring: Part 1" reviews the autograd
function (bitsandbytes/autograd/_functions.py) that keeps a transposed int8
copy of the layer input, ``CAt``, and zeroes its outlier columns, indexed by
the forward's saved outlier list, before the backward uses it.  The
transformers PR page ("`bitsandbytes` - `Linear8bitLt` integration into
`transformers` models", its discussion of fine-tuning) says that training
through these layers works while the fp16 weights are kept.  No formula is
printed.  This module is the training step those remarks describe, in the
int8/fp16 split of the forward (outliers in fp16, the rest in int8):

7. column-wise ("transposed") quantization of a matrix A [r x c]: column j's
   scale is max_i |A[i, j]|, and codes follow reading 3 of the forward with that
   scale in place of the row scale.  The codes are handed over transposed, as
   At_q [c x r] (At_q[j, i] is the code of A[i, j]), the K-contiguous layout of
   an int8 GEMM operand.  Listed columns can be zeroed (CAt);
8. grad_x = g . W, with g = dL/dy [m x n] quantized row-wise (threshold off) and
   the fp16 weight W [n x k] quantized column-wise (CBt):
       grad_x[i, j] = fp16( (s_wt[j] / 127) * (C[i, j] * s_g[i] / 127) ),
       C = g_q . (Wt_q)^T exact in int32 (contraction over n);
   there is no outlier term: outliers are input features of x, and neither g
   nor the contraction over n carries them;
9. grad_W = g^T . x, with g quantized column-wise (one scale per output
   feature n, over the m rows) and x quantized column-wise with its outlier
   columns O (the forward's) zeroed (CAt):
       grad_W[n, j] = fp16( (s_xt[j] / 127) * (C[n, j] * s_gt[n] / 127) ),  j not in O
       grad_W[n, j] = fp16( sum_i g[i, n] * x[i, j] ),                    j in O
   with C = Gt_q . (CAt)^T exact in int32 (contraction over the m rows); the
   outlier columns take the fp16 path, their int8 part being zero.

Every code is decided in IEEE binary32 (reading 3); everything after the
integer GEMMs is float64 here, rounded once to fp16.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Sequence

import numpy as np

from .llm_int8 import INT32_SAFE_K, int8_linear_matmul, quantize_weight


def colwise_absmax(a: np.ndarray) -> np.ndarray:
    """Column scale = max_i |a[i, j]| as fp32 (reading 7), 0 for an empty or zero column."""
    a32 = np.abs(np.asarray(a, dtype=np.float16).astype(np.float32))
    if a32.shape[0] == 0:
        return np.zeros(a32.shape[1], dtype=np.float32)
    return a32.max(axis=0).astype(np.float32)


def colwise_quant(a: np.ndarray, zero_cols: Sequence[int] = ()):
    """Transposed int8 quantization (reading 7): (At_q int8 [c, r], absmax fp32 [c]).

    Codes per column j: clamp(rne(fl32(a[i, j] * fl32(127 / s_j))), -127, 127),
    every step IEEE binary32, 0 where s_j = 0.  The columns in zero_cols keep
    their scale but get all-zero codes (the CAt of the bitsandbytes PR review).
    """
    a32 = np.asarray(a, dtype=np.float16).astype(np.float32)
    s = colwise_absmax(a)
    pos = s > 0
    inv = np.zeros_like(s)
    inv[pos] = np.float32(127.0) / s[pos]                  # fl32(127 / s_j)
    prod = a32 * inv[None, :]                              # fl32(a * inv)
    q = np.clip(np.rint(prod), -127, 127)                  # half to even
    q[:, ~pos] = 0
    q[:, np.asarray(list(zero_cols), dtype=np.int64)] = 0
    return np.ascontiguousarray(q.astype(np.int8).T), s


@dataclass
class BackwardResult:
    grad_x: np.ndarray     # fp16 [m, k]
    grad_w: np.ndarray     # fp16 [n, k]
    gx: np.ndarray         # float64 [m, k] before the fp16 rounding
    gw: np.ndarray         # float64 [n, k] before the fp16 rounding
    g_q: np.ndarray        # int8 [m, n]   row-wise codes of g
    g_s: np.ndarray        # fp32 [m]
    wt_q: np.ndarray       # int8 [k, n]   column-wise codes of W (CBt)
    wt_s: np.ndarray       # fp32 [k]
    gt_q: np.ndarray       # int8 [n, m]   column-wise codes of g
    gt_s: np.ndarray       # fp32 [n]
    xt_q: np.ndarray       # int8 [k, m]   column-wise codes of x, outlier columns zeroed (CAt)
    xt_s: np.ndarray       # fp32 [k]
    c_x: np.ndarray        # int32 [m, k]
    c_w: np.ndarray        # int32 [n, k]


def grad_input(g: np.ndarray, w: np.ndarray):
    """Reading 8: (grad_x fp16 [m, k], its float64 value, g_q, s_g, Wt_q, s_wt, C)."""
    g_q, g_s = quantize_weight(g)              # row-wise codes, threshold off
    wt_q, wt_s = colwise_quant(w)
    c = int8_linear_matmul(g_q, wt_q)          # [m, k], contraction over n
    y = (wt_s.astype(np.float64)[None, :] / 127.0) * (
        c.astype(np.float64) * g_s.astype(np.float64)[:, None] / 127.0)
    return y.astype(np.float16), y, g_q, g_s, wt_q, wt_s, c


def grad_weight(g: np.ndarray, x: np.ndarray, cols: Sequence[int]):
    """Reading 9: (grad_W fp16 [n, k], its float64 value, Gt_q, s_gt, CAt, s_xt, C)."""
    cols = np.asarray(list(cols), dtype=np.int64)
    gt_q, gt_s = colwise_quant(g)
    xt_q, xt_s = colwise_quant(x, cols)
    c = int8_linear_matmul(gt_q, xt_q)         # [n, k], contraction over the m rows
    y = (xt_s.astype(np.float64)[None, :] / 127.0) * (
        c.astype(np.float64) * gt_s.astype(np.float64)[:, None] / 127.0)
    if cols.size:
        # the outlier columns in fp16 operands: exact products, float64 sums
        y[:, cols] = y[:, cols] + (np.asarray(g, np.float16).astype(np.float64).T
                                   @ np.asarray(x, np.float16)[:, cols].astype(np.float64))
    return y.astype(np.float16), y, gt_q, gt_s, xt_q, xt_s, c


def linear_backward(g: np.ndarray, x: np.ndarray, w: np.ndarray, cols: Sequence[int]) -> BackwardResult:
    """Both gradients of y = x . W^T (+ b) for dL/dy = g, readings 7-9.

    g fp16 [m, n], x fp16 [m, k], W fp16 [n, k] (the training copy of the
    weight), cols = the forward's outlier columns of x.
    """
    if g.shape[0] != x.shape[0] or g.shape[1] != w.shape[0] or x.shape[1] != w.shape[1]:
        raise ValueError("shapes of g, x and W do not match")
    if max(g.shape[1], g.shape[0]) > INT32_SAFE_K:
        raise ValueError("contraction too long for an exact int32 accumulator")
    gx16, gx, g_q, g_s, wt_q, wt_s, c_x = grad_input(g, w)
    gw16, gw, gt_q, gt_s, xt_q, xt_s, c_w = grad_weight(g, x, cols)
    return BackwardResult(gx16, gw16, gx, gw, g_q, g_s, wt_q, wt_s, gt_q, gt_s, xt_q, xt_s, c_x, c_w)
