"""Plain, slow CPU oracle of the blockwise 4-bit (FP4) weight path.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code,
tables or helpers with the HIP library.

What the pages fix, and what is a reading
-----------------------------------------
The page "Loading an LLM in 4 bits using bitsandbytes" (its "Normalized
Float" and "Double Quantization" sections, under the bnb_4bit_quant_type and
bnb_4bit_use_double_quant options) says: fp4 has a 1-bit sign, a 2-bit exponent and a 1-bit mantissa and
is the default 4-bit type; weights are quantized in blocks of 64, each block
with a 32-bit scaling factor; double quantization groups those scaling factors
in blocks of 256 and quantizes them to 8 bits.  The bitsandbytes PR
"LLM.int8() Refactoring: Part 1" (its inference benchmark overview) runs the
4-bit type on the same inference workloads as int8.  The page's nf4 type has
no value table on the pages and is not built.  The readings:

F1. the 4-bit value set is IEEE-style E2M1 (exponent bias 1, a subnormal at
    exponent 0): magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6, the magnitude code
    being the 3 low bits (e1 e0 m) and bit 3 the sign;
F2. a block is 64 consecutive weights of a row of W [n x k] (k a multiple of
    64, so this is also 64 consecutive elements of the flattened tensor); its
    scale is absmax_b = max |w| over the block (fp32, exact);
F3. code = sign bit of w (the fp16 sign, so -0 keeps it) and magnitude
    RNE_E2M1(min(fl32(|w| * fl32(6 / absmax_b)), 6)), round to nearest with
    ties to the even mantissa bit; a zero block has inv = 0 (all magnitudes 0);
F4. double quantization: the block scales in flattened order, groups of 256
    (the last group may be shorter); s2 = max over the group (fp32);
    c8 = clamp(rne(fl32(absmax_b * fl32(255 / s2))), 0, 255), 0 if s2 = 0;
    the reconstructed scale is fl32(c8 * fl32(s2 / 255));
F5. dequantized weight w' = fl32(E2M1 value * fl32(A / 6)), A the block
    scale (reconstructed when double-quantized): one binary32 rounding of the
    product (exact when A / 6 has at most 22 significant bits);
F6. the 4-bit linear: y[i, n] = fp16( sum_k x[i, k] * w'[n, k] + bias[n] ),
    float64 here (the GPU sums in fp32).

Where floating point decides an integer (a code), both sides decide in
binary32.
"""

from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

BLOCK = 64
DQ_GROUP = 256
E2M1_MAX = 6.0


def e2m1_value(code: np.ndarray) -> np.ndarray:
    """Value of 4-bit E2M1 codes from their bits (F1): sign, 2-bit exponent, 1-bit mantissa."""
    c = np.asarray(code).astype(np.int64)
    s = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return s * mag


def _rne_e2m1_magnitude(v: np.ndarray) -> np.ndarray:
    """Magnitude code (0..7) of non-negative fp32 values, nearest E2M1 value,
    ties to the even code (the mantissa bit is the code's low bit)."""
    grid = e2m1_value(np.arange(8))                      # 0, .5, 1, 1.5, 2, 3, 4, 6
    v = np.minimum(np.asarray(v, np.float64), E2M1_MAX)  # saturate
    d = np.abs(v[..., None] - grid)                      # exact in float64
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # among the (at most two) nearest, the even code
    even = cand & (np.arange(8) % 2 == 0)
    pick = np.where(even.any(axis=-1, keepdims=True), even, cand)
    return np.argmax(pick, axis=-1).astype(np.uint8)


def fp4_quantize(w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(codes uint8 [n, k] one code per element, absmax fp32 [n, k/64]) per F2-F3."""
    w = np.asarray(w, dtype=np.float16)
    n, k = w.shape
    if k % BLOCK:
        raise ValueError("k must be a multiple of 64")
    a32 = np.abs(w.astype(np.float32)).reshape(n, k // BLOCK, BLOCK)
    absmax = a32.max(axis=2).astype(np.float32) if k else np.zeros((n, 0), np.float32)
    inv = np.zeros_like(absmax)
    pos = absmax > 0
    inv[pos] = np.float32(E2M1_MAX) / absmax[pos]                      # fl32(6 / absmax)
    v = (a32 * inv[:, :, None]).astype(np.float32)                    # fl32(|w| * inv)
    mag = _rne_e2m1_magnitude(v).reshape(n, k)
    sign = (w.view(np.uint16) >> 15).astype(np.uint8)
    return (mag | (sign << 3)).astype(np.uint8), absmax


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte: element 2j in the low nibble, 2j + 1 in the high one."""
    c = np.asarray(codes, np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), np.uint8)
    out[:, 0::2] = p & 15
    out[:, 1::2] = p >> 4
    return out


def double_quant(absmax: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(c8 uint8 [nb], s2 fp32 [ceil(nb/256)]) over the flattened block scales (F4)."""
    a = np.asarray(absmax, np.float32).reshape(-1)
    nb = a.size
    groups = (nb + DQ_GROUP - 1) // DQ_GROUP
    c8 = np.zeros(nb, np.uint8)
    s2 = np.zeros(groups, np.float32)
    for gi in range(groups):
        blk = a[gi * DQ_GROUP:(gi + 1) * DQ_GROUP]
        s = np.float32(blk.max()) if blk.size else np.float32(0)
        s2[gi] = s
        if s > 0:
            inv = np.float32(255.0) / s                                # fl32(255 / s2)
            q = np.rint((blk * inv).astype(np.float32))                # fl32 product, half to even
            c8[gi * DQ_GROUP:gi * DQ_GROUP + blk.size] = np.clip(q, 0, 255).astype(np.uint8)
    return c8, s2


def double_dequant(c8: np.ndarray, s2: np.ndarray) -> np.ndarray:
    """Reconstructed block scales fl32(c8 * fl32(s2 / 255)) (F4), flattened."""
    c = np.asarray(c8, np.uint8).reshape(-1)
    step = (np.asarray(s2, np.float32) / np.float32(255.0)).astype(np.float32)
    return (c.astype(np.float32) * np.repeat(step, DQ_GROUP)[: c.size]).astype(np.float32)


def fp4_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """w' = fl32(E2M1 value * fl32(A / 6)) per F5, as fp32; codes one per element."""
    c = np.asarray(codes, np.uint8)
    n, k = c.shape
    d = (np.asarray(scales, np.float32).reshape(n, k // BLOCK) / np.float32(E2M1_MAX)).astype(np.float32)
    vals = e2m1_value(c).astype(np.float32)
    return (vals.reshape(n, k // BLOCK, BLOCK) * d[:, :, None]).astype(np.float32).reshape(n, k)


def fp4_linear(x: np.ndarray, codes: np.ndarray, scales: np.ndarray,
               bias: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """F6: (fp16 out [m, n], its float64 value) with w' from codes and block scales."""
    w = fp4_dequantize(codes, scales).astype(np.float64)
    y = np.asarray(x, np.float16).astype(np.float64) @ w.T
    if bias is not None:
        y = y + np.asarray(bias, np.float16).astype(np.float64)[None, :]
    return y.astype(np.float16), y
