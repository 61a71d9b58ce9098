"""LLM.int8() vector-wise mixed-precision linear for AMD MI355X (gfx950).

Thin Python binding of libi8mp.so.  Every step of the computation runs in the
library's HIP kernels; this module checks devices, dtypes and layouts (all
non-None tensors on one GPU, as the bitsandbytes pre-call check requires),
allocates outputs and workspaces with PyTorch, and passes the current stream.
There is no CPU fallback: calling an op without the built library, or on
tensors that are not on a GPU, raises.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from ._lib import (  # noqa: F401
    EXPORTS,
    BackwardWorkspaceLayout,
    I8MP_MAX_K,
    I8MP_NOALLOC_SCRATCH_BYTES,
    I8mpError,
    LinearWorkspaceLayout,
    check,
    lib,
    status_string,
)
from .serialize import load_int8_weights, save_int8_weights  # noqa: F401

__all__ = [
    "quantize_weight",
    "save_int8_weights",
    "load_int8_weights",
    "vectorwise_quant",
    "outlier_extract",
    "linear_matmul",
    "mm_dequant",
    "vectorwise_dequant",
    "linear",
    "linear_forward_noalloc",
    "linear_quantize",
    "linear_matmul_dequant",
    "LinearWorkspace",
    "colwise_quant",
    "linear_backward",
    "BackwardWorkspace",
    "Fp4Weight",
    "fp4_quantize",
    "fp4_double_quant",
    "fp4_dequantize",
    "fp4_linear",
    "I8mpError",
]

DEFAULT_THRESHOLD = 6.0
DEFAULT_CAP = 256


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _device_of(*tensors) -> torch.device:
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one device, got {sorted(map(str, devs))}")
    dev = devs.pop()
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a GPU (got {dev}); there is no CPU path")
    return dev


def _rowmajor(t: torch.Tensor, name: str, dtype: torch.dtype) -> int:
    """Leading dimension of a row-major 2-D tensor with unit column stride."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.numel() > 0 and t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return max(t.stride(0), t.shape[1], 1)


def _vec(t: torch.Tensor, name: str, dtype: torch.dtype, n: int) -> None:
    if t.dtype != dtype or t.dim() != 1 or t.shape[0] != n or (n > 1 and t.stride(0) != 1):
        raise ValueError(f"{name} must be a contiguous {dtype} vector of length {n}")


def vectorwise_quant(x: torch.Tensor, threshold: float = DEFAULT_THRESHOLD,
                     ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """int8_vectorwise_quant: (codes int8 [m,k], row absmax fp32 [m], outlier bitmap uint32-as-int32)."""
    dev = _device_of(x)
    ldx = _rowmajor(x, "x", torch.float16)
    m, k = x.shape
    q = torch.empty((m, k), dtype=torch.int8, device=dev)
    absmax = torch.empty(m, dtype=torch.float32, device=dev)
    bitmap = torch.empty((k + 31) // 32, dtype=torch.int32, device=dev)
    L = lib()
    wsb = L.i8mp_quant_workspace_bytes(m, k) if threshold > 0 else 0
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        check(L.i8mp_int8_vectorwise_quant(_ptr(x), m, k, ldx, threshold, _ptr(q), k, _ptr(absmax),
                                           _ptr(bitmap), _ptr(ws), wsb, _stream(dev)),
              "i8mp_int8_vectorwise_quant")
    return q, absmax, bitmap


def quantize_weight(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Row-wise int8 weight state (codes, per-row absmax) of an fp16 weight [n, k]."""
    q, absmax, _ = vectorwise_quant(w, 0.0)
    return q, absmax


def outlier_extract(x: torch.Tensor, bitmap: torch.Tensor, cap: Optional[int] = None, strict: bool = True
                    ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """extract_outliers: (idx int32 [cap], count int32 [1], x_out fp16 [m, cap]).

    ``cap`` defaults to k, which holds every outlier column.  With a smaller
    cap and more outlier columns than it, only the first cap are listed;
    ``strict`` (default) then raises instead, reading the count back (a
    synchronization), since the sparse decomposition built from such a list
    would drop columns.
    """
    dev = _device_of(x, bitmap)
    ldx = _rowmajor(x, "x", torch.float16)
    m, k = x.shape
    _vec(bitmap, "bitmap", torch.int32, (k + 31) // 32)
    if cap is None:
        cap = k
    idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    count = torch.empty(1, dtype=torch.int32, device=dev)
    xo = torch.empty((m, max(cap, 1)), dtype=torch.float16, device=dev)
    with torch.cuda.device(dev):
        check(lib().i8mp_outlier_extract(_ptr(x), m, k, ldx, _ptr(bitmap), cap, _ptr(idx), _ptr(count),
                                         _ptr(xo), max(cap, 1), _stream(dev)),
              "i8mp_outlier_extract")
    if strict and cap < k:
        found = int(count.item())
        if found > cap:
            raise ValueError(f"{found} outlier columns found, more than cap={cap}: extract with a larger cap")
    return idx[:cap], count, xo[:, :cap]


def linear_matmul(a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """int8_linear_matmul: C = A . B^T, exact int32 [m, n]."""
    dev = _device_of(a, b)
    lda = _rowmajor(a, "a", torch.int8)
    ldb = _rowmajor(b, "b", torch.int8)
    m, k = a.shape
    n, kb = b.shape
    if kb != k:
        raise ValueError("inner dimensions differ")
    c = torch.empty((m, n), dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        check(lib().i8mp_int8_linear_matmul(_ptr(a), lda, _ptr(b), ldb, m, n, k, _ptr(c), max(n, 1),
                                            _stream(dev)),
              "i8mp_int8_linear_matmul")
    return c


def mm_dequant(c: torch.Tensor, row_absmax: torch.Tensor, col_absmax: torch.Tensor,
               bias: Optional[torch.Tensor] = None,
               outliers: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]] = None,
               ) -> torch.Tensor:
    """int8_mm_dequant (+ bias, + the sparse-decomposition term).

    ``outliers`` = (x_out fp16 [m, cap], idx int32 [cap], count int32 [1], w_q int8 [n, k]).
    """
    xo = idx = count = wq = None
    if outliers is not None:
        xo, idx, count, wq = outliers
    dev = _device_of(c, row_absmax, col_absmax, bias, xo, idx, count, wq)
    ldc = _rowmajor(c, "c", torch.int32)
    m, n = c.shape
    _vec(row_absmax, "row_absmax", torch.float32, m)
    _vec(col_absmax, "col_absmax", torch.float32, n)
    if bias is not None:
        _vec(bias, "bias", torch.float16, n)
    cap, ldo, ldb, k = 0, 0, 0, 1
    if outliers is not None:
        ldo = _rowmajor(xo, "x_out", torch.float16)
        cap = xo.shape[1]
        ldb = _rowmajor(wq, "w_q", torch.int8)
        k = wq.shape[1]
    out = torch.empty((m, n), dtype=torch.float16, device=dev)
    with torch.cuda.device(dev):
        check(lib().i8mp_int8_mm_dequant(_ptr(c), ldc, _ptr(row_absmax), _ptr(col_absmax), _ptr(bias), m, n,
                                         _ptr(xo), ldo, _ptr(idx), _ptr(count), cap, _ptr(wq), ldb, k,
                                         _ptr(out), max(n, 1), _stream(dev)),
              "i8mp_int8_mm_dequant")
    return out


@dataclass
class LinearWorkspace:
    """Device workspace of i8mp_linear_forward plus views of its intermediates."""

    m: int
    n: int
    k: int
    cap: int
    layout: LinearWorkspaceLayout
    buf: torch.Tensor

    @classmethod
    def create(cls, m: int, n: int, k: int, cap: int, device) -> "LinearWorkspace":
        L = LinearWorkspaceLayout()
        check(lib().i8mp_linear_workspace_query(m, n, k, cap, ctypes.byref(L)), "i8mp_linear_workspace_query")
        buf = torch.empty(max(L.bytes, 1), dtype=torch.uint8, device=device)
        return cls(m, n, k, cap, L, buf)

    def fits(self, m: int, n: int, k: int, cap: int) -> bool:
        L = LinearWorkspaceLayout()
        check(lib().i8mp_linear_workspace_query(m, n, k, cap, ctypes.byref(L)), "i8mp_linear_workspace_query")
        return L.bytes <= self.buf.numel() and (m, k, cap) == (self.m, self.k, self.cap)

    def _view(self, off: int, count: int, dtype: torch.dtype) -> torch.Tensor:
        nbytes = count * torch.tensor([], dtype=dtype).element_size()
        return self.buf[off:off + nbytes].view(dtype)

    # intermediates left by the last forward call (for tests and inspection)
    def codes(self) -> torch.Tensor:
        return self._view(self.layout.q_offset, self.m * self.layout.ldq, torch.int8).view(
            self.m, self.layout.ldq)[:, : self.k]

    def absmax(self) -> torch.Tensor:
        return self._view(self.layout.absmax_offset, self.m, torch.float32)

    def bitmap(self) -> torch.Tensor:
        return self._view(self.layout.bitmap_offset, (self.k + 31) // 32, torch.int32)

    def idx(self) -> torch.Tensor:
        """Every outlier column, ascending, -1 past the count (idx_len entries)."""
        return self._view(self.layout.idx_offset, self.layout.idx_len, torch.int32)

    def count(self) -> torch.Tensor:
        return self._view(self.layout.count_offset, 1, torch.int32)

    def x_out(self) -> torch.Tensor:
        cp = self.layout.cap_pad
        return self._view(self.layout.xo_offset, self.m * cp, torch.float16).view(self.m, cp)[:, : self.cap]

    def outliers_past_cap(self) -> bool:
        """True if the last call found more outlier columns than cap (synchronizes).

        The output is the method's either way; the columns past cap read their
        x values through the index list, which is slower."""
        return int(self.count().item()) > self.cap


def vectorwise_dequant(q: torch.Tensor, absmax: torch.Tensor, dtype: torch.dtype = torch.float16,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int8 vectorwise dequantize: q[i, j] * (absmax[i] / 127) in fp32, as fp16 or fp32."""
    if dtype not in (torch.float16, torch.float32):
        raise ValueError("dtype must be torch.float16 or torch.float32")
    dev = _device_of(q, absmax, out)
    ldq = _rowmajor(q, "q", torch.int8)
    m, k = q.shape
    _vec(absmax, "absmax", torch.float32, m)
    if out is None:
        out = torch.empty((m, k), dtype=dtype, device=dev)
    ldout = _rowmajor(out, "out", dtype)
    if tuple(out.shape) != (m, k):
        raise ValueError("out has the wrong shape")
    code = 0 if dtype == torch.float16 else 1
    with torch.cuda.device(dev):
        check(lib().i8mp_int8_vectorwise_dequant(_ptr(q), ldq, m, k, _ptr(absmax), code, _ptr(out), ldout,
                                                 _stream(dev)),
              "i8mp_int8_vectorwise_dequant")
    return out


def linear(x: torch.Tensor, w_q: torch.Tensor, w_absmax: torch.Tensor,
           bias: Optional[torch.Tensor] = None, threshold: float = DEFAULT_THRESHOLD,
           cap: int = DEFAULT_CAP, workspace: Optional[LinearWorkspace] = None,
           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The fused mixed-precision linear: fp16 out [m, n] = x . dequant(w)^T + bias.

    Every outlier column takes the fp16 path for any count; ``cap`` sizes the
    workspace's gathered copy of the outlier columns (the fast path)."""
    dev = _device_of(x, w_q, w_absmax, bias, out)
    ldx = _rowmajor(x, "x", torch.float16)
    ldw = _rowmajor(w_q, "w_q", torch.int8)
    m, k = x.shape
    n, kw = w_q.shape
    if kw != k:
        raise ValueError("x and w_q differ in k")
    _vec(w_absmax, "w_absmax", torch.float32, n)
    if bias is not None:
        _vec(bias, "bias", torch.float16, n)
    if out is None:
        out = torch.empty((m, n), dtype=torch.float16, device=dev)
    ldout = _rowmajor(out, "out", torch.float16)
    if tuple(out.shape) != (m, n):
        raise ValueError("out has the wrong shape")
    if workspace is None:
        workspace = LinearWorkspace.create(m, n, k, cap, dev)
    elif not workspace.fits(m, n, k, cap):
        raise ValueError("workspace was created for another shape or capacity")
    with torch.cuda.device(dev):
        check(lib().i8mp_linear_forward(_ptr(x), m, k, ldx, _ptr(w_q), ldw, _ptr(w_absmax), n, _ptr(bias),
                                        threshold, cap, _ptr(out), ldout, _ptr(workspace.buf),
                                        workspace.buf.numel(), _stream(dev)),
              "i8mp_linear_forward")
    return out


def linear_forward_noalloc(x: torch.Tensor, w_q: torch.Tensor, w_absmax: torch.Tensor, out: torch.Tensor,
                           bias: Optional[torch.Tensor] = None, threshold: float = DEFAULT_THRESHOLD,
                           cap: int = DEFAULT_CAP) -> torch.Tensor:
    """``linear`` into a caller-owned ``out`` with the library's fixed scratch
    array as workspace: the call allocates nothing (for graph capture and
    serving loops).  Shapes whose workspace exceeds the array raise; calls
    that overlap on one GPU share the array and race."""
    dev = _device_of(x, w_q, w_absmax, bias, out)
    ldx = _rowmajor(x, "x", torch.float16)
    ldw = _rowmajor(w_q, "w_q", torch.int8)
    m, k = x.shape
    n, kw = w_q.shape
    if kw != k:
        raise ValueError("x and w_q differ in k")
    _vec(w_absmax, "w_absmax", torch.float32, n)
    if bias is not None:
        _vec(bias, "bias", torch.float16, n)
    ldout = _rowmajor(out, "out", torch.float16)
    if tuple(out.shape) != (m, n):
        raise ValueError("out has the wrong shape")
    with torch.cuda.device(dev):
        check(lib().i8mp_linear_forward_noalloc(_ptr(x), m, k, ldx, _ptr(w_q), ldw, _ptr(w_absmax), n, _ptr(bias),
                                                threshold, cap, _ptr(out), ldout, _stream(dev)),
              "i8mp_linear_forward_noalloc")
    return out


def linear_quantize(x: torch.Tensor, workspace: LinearWorkspace,
                    threshold: float = DEFAULT_THRESHOLD) -> None:
    """First half of ``linear``: detect, calibrate, quantize and extract into the workspace."""
    dev = _device_of(x, workspace.buf)
    ldx = _rowmajor(x, "x", torch.float16)
    m, k = x.shape
    if (m, k) != (workspace.m, workspace.k):
        raise ValueError("workspace was created for another shape")
    with torch.cuda.device(dev):
        check(lib().i8mp_linear_quantize(_ptr(x), m, k, ldx, threshold, workspace.cap, _ptr(workspace.buf),
                                         workspace.buf.numel(), _stream(dev)),
              "i8mp_linear_quantize")


def linear_matmul_dequant(x: torch.Tensor, workspace: LinearWorkspace, w_q: torch.Tensor,
                          w_absmax: torch.Tensor, bias: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Second half of ``linear``: fused int8 GEMM + dequant epilogue from the
    workspace that ``linear_quantize(x, workspace)`` filled (x is read for
    outlier columns past the workspace's cap)."""
    dev = _device_of(x, workspace.buf, w_q, w_absmax, bias, out)
    ldx = _rowmajor(x, "x", torch.float16)
    ldw = _rowmajor(w_q, "w_q", torch.int8)
    n, k = w_q.shape
    if k != workspace.k or tuple(x.shape) != (workspace.m, workspace.k):
        raise ValueError("x, w_q and the workspace differ in shape")
    _vec(w_absmax, "w_absmax", torch.float32, n)
    if bias is not None:
        _vec(bias, "bias", torch.float16, n)
    m = workspace.m
    if out is None:
        out = torch.empty((m, n), dtype=torch.float16, device=dev)
    ldout = _rowmajor(out, "out", torch.float16)
    with torch.cuda.device(dev):
        check(lib().i8mp_linear_matmul_dequant(_ptr(x), ldx, _ptr(workspace.buf), workspace.buf.numel(), m, k,
                                               workspace.cap,
                                               _ptr(w_q), ldw, _ptr(w_absmax), n, _ptr(bias), _ptr(out),
                                               ldout, _stream(dev)),
              "i8mp_linear_matmul_dequant")
    return out


def colwise_quant(a: torch.Tensor, zero_idx: Optional[torch.Tensor] = None,
                  zero_count: Optional[torch.Tensor] = None, ldqt: Optional[int] = None
                  ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Column-wise (transposed) int8 quantization: (qt int8 [cols, ldqt], col absmax fp32 [cols]).

    qt[j, i] is the code of a[i, j] under column j's absmax; columns listed in
    zero_idx[:min(zero_count, len)] get zero codes; rows >= a.shape[0] of qt are 0.
    """
    dev = _device_of(a, zero_idx, zero_count)
    lda = _rowmajor(a, "a", torch.float16)
    rows, cols = a.shape
    if (zero_idx is None) != (zero_count is None):
        raise ValueError("zero_idx and zero_count go together")
    cap = 0
    if zero_idx is not None:
        if zero_idx.dtype != torch.int32 or zero_idx.dim() != 1 or not zero_idx.is_contiguous():
            raise ValueError("zero_idx must be a contiguous int32 vector")
        _vec(zero_count, "zero_count", torch.int32, 1)
        cap = zero_idx.shape[0]
    ldqt = rows if ldqt is None else ldqt
    qt = torch.empty((cols, max(ldqt, 1)), dtype=torch.int8, device=dev)
    absmax = torch.empty(cols, dtype=torch.float32, device=dev)
    L = lib()
    wsb = L.i8mp_colwise_quant_workspace_bytes(rows, max(cols, 1))
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        check(L.i8mp_int8_colwise_quant(_ptr(a), rows, cols, lda, _ptr(zero_idx), _ptr(zero_count), cap, _ptr(qt),
                                        ldqt, _ptr(absmax), _ptr(ws), wsb, _stream(dev)),
              "i8mp_int8_colwise_quant")
    return qt[:, :ldqt], absmax


@dataclass
class BackwardWorkspace:
    """Device workspace of i8mp_linear_backward plus views of the GEMM operands it holds."""

    m: int
    n: int
    k: int
    cap: int
    layout: BackwardWorkspaceLayout
    buf: torch.Tensor

    @classmethod
    def create(cls, m: int, n: int, k: int, cap: int, device) -> "BackwardWorkspace":
        L = BackwardWorkspaceLayout()
        check(lib().i8mp_linear_backward_workspace_query(m, n, k, cap, ctypes.byref(L)),
              "i8mp_linear_backward_workspace_query")
        return cls(m, n, k, cap, L, torch.empty(max(L.bytes, 1), dtype=torch.uint8, device=device))

    def _mat(self, off: int, rows: int, ld: int, cols: int) -> torch.Tensor:
        return self.buf[off:off + rows * ld].view(rows, ld)[:, :cols]

    def _f32(self, off: int, count: int) -> torch.Tensor:
        return self.buf[off:off + 4 * count].view(torch.float32)

    # operands left by the last call (for tests and inspection)
    def g_q(self):
        return self._mat(self.layout.gq_offset, self.m, self.layout.ld_n, self.n).view(torch.int8)

    def g_s(self):
        return self._f32(self.layout.gs_offset, self.m)

    def wt_q(self):
        return self._mat(self.layout.wtq_offset, self.k, self.layout.ld_n, self.n).view(torch.int8)

    def wt_s(self):
        return self._f32(self.layout.wts_offset, self.k)

    def gt_q(self):
        return self._mat(self.layout.gtq_offset, self.n, self.layout.ld_m, self.m).view(torch.int8)

    def gt_s(self):
        return self._f32(self.layout.gts_offset, self.n)

    def xt_q(self):
        return self._mat(self.layout.xtq_offset, self.k, self.layout.ld_m, self.m).view(torch.int8)

    def xt_s(self):
        return self._f32(self.layout.xts_offset, self.k)


def linear_backward(grad_out: torch.Tensor, x: torch.Tensor, w: Optional[torch.Tensor],
                    forward_workspace: Optional[LinearWorkspace] = None,
                    need_grad_x: bool = True, need_grad_w: bool = True,
                    workspace: Optional[BackwardWorkspace] = None,
                    out_x: Optional[torch.Tensor] = None, out_w: Optional[torch.Tensor] = None,
                    ) -> Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]:
    """Both gradients of ``linear`` for dL/dout = grad_out: (grad_x fp16 [m, k], grad_w fp16 [n, k]).

    w is the fp16 weight kept for training (needed for grad_x).  The outlier
    columns are those the forward left in ``forward_workspace`` (None: none).
    """
    dev = _device_of(grad_out, x, w, None if forward_workspace is None else forward_workspace.buf)
    ldg = _rowmajor(grad_out, "grad_out", torch.float16)
    ldx = _rowmajor(x, "x", torch.float16)
    m, n = grad_out.shape
    mx, k = x.shape
    if mx != m:
        raise ValueError("grad_out and x differ in rows")
    ldw = k
    if need_grad_x:
        if w is None:
            raise ValueError("grad_x needs the fp16 weight")
        ldw = _rowmajor(w, "w", torch.float16)
        if tuple(w.shape) != (n, k):
            raise ValueError("w must be [n, k]")
    cap = 0
    if forward_workspace is not None:
        if (forward_workspace.m, forward_workspace.k) != (m, k):
            raise ValueError("forward workspace was made for another shape")
        cap = forward_workspace.cap
    if workspace is None:
        workspace = BackwardWorkspace.create(m, n, k, cap, dev)
    elif (workspace.m, workspace.n, workspace.k, workspace.cap) != (m, n, k, cap):
        raise ValueError("backward workspace was created for another shape or capacity")
    gx = gw = None
    if need_grad_x:
        gx = torch.empty((m, k), dtype=torch.float16, device=dev) if out_x is None else out_x
        if tuple(gx.shape) != (m, k) or not gx.is_contiguous() or gx.dtype != torch.float16:
            raise ValueError("out_x must be a contiguous fp16 [m, k] tensor")
    if need_grad_w:
        gw = torch.empty((n, k), dtype=torch.float16, device=dev) if out_w is None else out_w
        if tuple(gw.shape) != (n, k) or not gw.is_contiguous() or gw.dtype != torch.float16:
            raise ValueError("out_w must be a contiguous fp16 [n, k] tensor")
    fws = None if forward_workspace is None else forward_workspace.buf
    with torch.cuda.device(dev):
        check(lib().i8mp_linear_backward(_ptr(grad_out), ldg, _ptr(x), ldx, _ptr(w if need_grad_x else None), ldw,
                                         m, n, k, cap, _ptr(fws), 0 if fws is None else fws.numel(),
                                         _ptr(gx), k, _ptr(gw), k, _ptr(workspace.buf), workspace.buf.numel(),
                                         _stream(dev)),
              "i8mp_linear_backward")
    return gx, gw


@dataclass
class Fp4Weight:
    """A weight in blockwise 4-bit E2M1 form: packed codes [n, ldc] (ldc = k/2
    rounded up to 16 bytes), and either fp32 block scales [n, k/64] or their
    8-bit double quantization (c8 [n * k/64], s2 [ceil(n * k/64 / 256)])."""

    codes: torch.Tensor
    k: int
    absmax: Optional[torch.Tensor] = None
    c8: Optional[torch.Tensor] = None
    s2: Optional[torch.Tensor] = None

    @property
    def n(self) -> int:
        return self.codes.shape[0]

    def scale_ptrs(self):
        if self.absmax is not None:
            return _ptr(self.absmax), None, None
        return None, _ptr(self.c8), _ptr(self.s2)


def fp4_quantize(w: torch.Tensor, double_quant: bool = False) -> Fp4Weight:
    """Blockwise 4-bit E2M1 quantization of an fp16 weight [n, k] (k a multiple of 64)."""
    dev = _device_of(w)
    ldw = _rowmajor(w, "w", torch.float16)
    n, k = w.shape
    if k % 64 or k == 0:
        raise ValueError("k must be a positive multiple of 64")
    ldc = (k // 2 + 15) // 16 * 16
    codes = torch.zeros((n, ldc), dtype=torch.uint8, device=dev)
    absmax = torch.empty((n, k // 64), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        check(lib().i8mp_fp4_quantize(_ptr(w), n, k, ldw, _ptr(codes), ldc, _ptr(absmax), _stream(dev)),
              "i8mp_fp4_quantize")
    fw = Fp4Weight(codes, k, absmax)
    return fp4_double_quant(fw) if double_quant else fw


def fp4_double_quant(fw: Fp4Weight) -> Fp4Weight:
    """The same weight with its block scales quantized to 8 bits in groups of 256."""
    if fw.absmax is None:
        raise ValueError("already double-quantized")
    dev = _device_of(fw.codes, fw.absmax)
    nb = fw.absmax.numel()
    c8 = torch.empty(nb, dtype=torch.uint8, device=dev)
    s2 = torch.empty(max((nb + 255) // 256, 1), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        check(lib().i8mp_fp4_double_quant(_ptr(fw.absmax), nb, _ptr(c8), _ptr(s2), _stream(dev)),
              "i8mp_fp4_double_quant")
    return Fp4Weight(fw.codes, fw.k, None, c8, s2[: (nb + 255) // 256])


def fp4_dequantize(fw: Fp4Weight, dtype: torch.dtype = torch.float16) -> torch.Tensor:
    """w' [n, k] = E2M1 value * (block scale / 6), as fp16 or fp32."""
    if dtype not in (torch.float16, torch.float32):
        raise ValueError("dtype must be torch.float16 or torch.float32")
    dev = _device_of(fw.codes)
    out = torch.empty((fw.n, fw.k), dtype=dtype, device=dev)
    a, c8, s2 = fw.scale_ptrs()
    with torch.cuda.device(dev):
        check(lib().i8mp_fp4_dequantize(_ptr(fw.codes), fw.codes.stride(0), fw.n, fw.k, a, c8, s2,
                                        0 if dtype == torch.float16 else 1, _ptr(out), fw.k, _stream(dev)),
              "i8mp_fp4_dequantize")
    return out


def fp4_linear(x: torch.Tensor, fw: Fp4Weight, bias: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The 4-bit linear for decode-sized batches: fp16 out [m, n] = x . w'^T + bias."""
    dev = _device_of(x, fw.codes, bias, out)
    ldx = _rowmajor(x, "x", torch.float16)
    m, k = x.shape
    if k != fw.k:
        raise ValueError("x and the weight differ in k")
    if bias is not None:
        _vec(bias, "bias", torch.float16, fw.n)
    if out is None:
        out = torch.empty((m, fw.n), dtype=torch.float16, device=dev)
    ldout = _rowmajor(out, "out", torch.float16)
    a, c8, s2 = fw.scale_ptrs()
    with torch.cuda.device(dev):
        check(lib().i8mp_fp4_linear(_ptr(x), m, k, ldx, _ptr(fw.codes), fw.codes.stride(0), a, c8, s2, fw.n,
                                    _ptr(bias), _ptr(out), ldout, _stream(dev)),
              "i8mp_fp4_linear")
    return out

