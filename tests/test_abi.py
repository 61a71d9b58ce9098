"""The C-ABI library loads, exports what include/i8mp.h declares, and rejects
bad arguments with the documented status codes before touching a device.

No compute calls are made here: every call below fails validation (or, on a
machine without a GPU, the device check) before anything is enqueued.
"""

import ctypes
import os
import re

import pytest

import int8_mixed_precision_vectorwise_amd as i8
from int8_mixed_precision_vectorwise_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "i8mp.h")

OK, EINVAL, ERANGE, EWORKSPACE, EDEVICE = 0, -1, -2, -3, -4
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
MAX_LD = int(re.search(r"#define I8MP_MAX_LD (\d+)", open(HEADER).read()).group(1))


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(i8mp_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libi8mp.so is not built (run __graft_entry__.build())")
    return _lib.lib()


def test_exports_match_header(L):
    declared = _header_functions()
    assert declared == sorted(_lib.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings(L):
    for s in (OK, EINVAL, ERANGE, EWORKSPACE, EDEVICE, -5):
        assert len(L.i8mp_status_string(s)) > 0
    assert L.i8mp_abi_version() >> 16 == 3


def test_workspace_queries(L):
    assert L.i8mp_quant_workspace_bytes(2048, 4096) > 0
    assert L.i8mp_quant_workspace_bytes(0, 4096) == 0
    assert L.i8mp_quant_workspace_bytes(16, 133145) == 0
    lay = _lib.LinearWorkspaceLayout()
    assert L.i8mp_linear_workspace_query(2048, 4096, 4096, 20, ctypes.byref(lay)) == OK
    assert lay.ldq % 128 == 0 and lay.ldq >= 4096
    assert lay.cap_pad == 32
    assert lay.idx_len == 4096                       # every column fits the index list
    assert lay.count_offset - lay.idx_offset >= 4 * lay.idx_len
    offs = [lay.scratch_offset, lay.bitmap_offset, lay.idx_offset, lay.count_offset,
            lay.absmax_offset, lay.q_offset, lay.xo_offset]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.bytes >= lay.xo_offset + 2048 * 32 * 2
    assert lay.q_offset + 2048 * lay.ldq <= lay.xo_offset
    assert 0 < lay.scratch_bytes <= lay.bitmap_offset - lay.scratch_offset
    assert L.i8mp_linear_workspace_query(16, 16, 133145, 8, ctypes.byref(lay)) == ERANGE
    assert L.i8mp_linear_workspace_query(16, 16, 0, 8, ctypes.byref(lay)) == EINVAL
    assert L.i8mp_linear_workspace_query(16, 16, 64, -1, ctypes.byref(lay)) == EINVAL
    assert L.i8mp_linear_workspace_query(16, 16, 64, 8, None) == EINVAL


def test_quant_validation(L):
    q = L.i8mp_int8_vectorwise_quant
    assert q(None, 4, 64, 64, 6.0, FAKE, 64, FAKE, None, FAKE, 1 << 20, None) == EINVAL
    assert q(FAKE, 4, 64, 32, 6.0, FAKE, 64, FAKE, None, FAKE, 1 << 20, None) == EINVAL   # ldx < k
    assert q(FAKE, 4, 64, 64, 6.0, FAKE, 63, FAKE, None, FAKE, 1 << 20, None) == EINVAL   # ldq < k
    assert q(FAKE, -1, 64, 64, 6.0, FAKE, 64, FAKE, None, FAKE, 1 << 20, None) == EINVAL
    assert q(FAKE, 4, 0, 64, 6.0, FAKE, 64, FAKE, None, FAKE, 1 << 20, None) == EINVAL
    assert q(FAKE, 4, 133145, 133145, 6.0, FAKE, 133145, FAKE, None, FAKE, 1 << 30, None) == ERANGE
    assert q(FAKE, 4, 64, 64, 6.0, FAKE, 64, FAKE, None, None, 0, None) == EWORKSPACE
    need = L.i8mp_quant_workspace_bytes(4, 64)
    assert q(FAKE, 4, 64, 64, 6.0, FAKE, 64, FAKE, None, FAKE, need - 1, None) == EWORKSPACE
    assert q(FAKE, 0, 64, 64, 6.0, None, 64, None, None, None, 0, None) == OK  # empty


def test_extract_validation(L):
    e = L.i8mp_outlier_extract
    assert e(FAKE, 4, 64, 64, None, 8, FAKE, FAKE, FAKE, 8, None) == EINVAL     # no bitmap
    assert e(FAKE, 4, 64, 64, FAKE, -1, FAKE, FAKE, FAKE, 8, None) == EINVAL    # cap < 0
    assert e(FAKE, 4, 64, 64, FAKE, 8, FAKE, FAKE, FAKE, 7, None) == EINVAL     # ldo < cap
    assert e(FAKE, 4, 64, 64, FAKE, 8, None, FAKE, FAKE, 8, None) == EINVAL     # no idx
    assert e(FAKE, 4, 64, 64, FAKE, 8, FAKE, None, FAKE, 8, None) == EINVAL     # no count


def test_matmul_validation(L):
    mm = L.i8mp_int8_linear_matmul
    assert mm(FAKE, 63, FAKE, 64, 4, 4, 64, FAKE, 4, None) == EINVAL   # lda < k
    assert mm(FAKE, 64, FAKE, 63, 4, 4, 64, FAKE, 4, None) == EINVAL   # ldb < k
    assert mm(FAKE, 64, FAKE, 64, 4, 4, 64, FAKE, 3, None) == EINVAL   # ldc < n
    assert mm(None, 64, FAKE, 64, 4, 4, 64, FAKE, 4, None) == EINVAL
    assert mm(FAKE, 64, FAKE, 64, 4, 4, 0, FAKE, 4, None) == EINVAL
    k = 133145
    assert mm(FAKE, k, FAKE, k, 1, 1, k, FAKE, 1, None) == ERANGE
    assert mm(None, 64, None, 64, 0, 4, 64, None, 4, None) == OK      # empty m
    big = MAX_LD + 1                                                   # 32-bit tile offsets
    assert mm(FAKE, 64, FAKE, big, 4, 4, 64, FAKE, 4, None) == EINVAL
    assert mm(FAKE, big, FAKE, 64, 4, 4, 64, FAKE, 4, None) == EINVAL
    assert mm(FAKE, 64, FAKE, 64, 4, 4, 64, FAKE, big, None) == EINVAL
    assert mm(None, 64, None, 64, 0, 4, 64, None, MAX_LD, None) == OK
    assert mm(None, 64, None, 64, 4, 0, 64, None, 0, None) == OK      # empty n


def test_dequant_validation(L):
    d = L.i8mp_int8_mm_dequant
    # outlier arguments must be all NULL or all set
    assert d(FAKE, 4, FAKE, FAKE, None, 4, 4, FAKE, 8, None, FAKE, 8, FAKE, 64, 64, FAKE, 4, None) == EINVAL
    assert d(FAKE, 3, FAKE, FAKE, None, 4, 4, None, 0, None, None, 0, None, 0, 1, FAKE, 4, None) == EINVAL
    assert d(None, 4, FAKE, FAKE, None, 4, 4, None, 0, None, None, 0, None, 0, 1, FAKE, 4, None) == EINVAL
    assert d(FAKE, 4, FAKE, FAKE, None, 4, 4, FAKE, 7, FAKE, FAKE, 8, FAKE, 64, 64, FAKE, 4, None) == EINVAL


def test_vectorwise_dequant_validation(L):
    d = L.i8mp_int8_vectorwise_dequant
    F16, F32 = 0, 1
    assert d(FAKE, 3, 4, 4, FAKE, F16, FAKE, 4, None) == EINVAL        # ldq < k
    assert d(FAKE, 4, 4, 4, FAKE, F16, FAKE, 3, None) == EINVAL        # ldout < k
    assert d(FAKE, 4, 4, 4, FAKE, 2, FAKE, 4, None) == EINVAL          # unknown output type
    assert d(FAKE, 4, -1, 4, FAKE, F16, FAKE, 4, None) == EINVAL
    assert d(None, 4, 4, 4, FAKE, F32, FAKE, 4, None) == EINVAL        # NULL codes
    assert d(FAKE, 4, 4, 4, FAKE, F32, None, 4, None) == EINVAL        # NULL out
    assert d(FAKE, MAX_LD + 1, 4, 4, FAKE, F16, FAKE, 4, None) == EINVAL
    assert d(None, 4, 0, 4, None, F16, None, 4, None) == OK           # empty
    assert d(None, 4, 4, 0, None, F32, None, 0, None) == OK


def test_forward_validation(L):
    f = L.i8mp_linear_forward
    lay = _lib.LinearWorkspaceLayout()
    assert L.i8mp_linear_workspace_query(16, 32, 64, 8, ctypes.byref(lay)) == OK
    args = dict(x=FAKE, m=16, k=64, ldx=64, w=FAKE, ldw=64, sw=FAKE, n=32, b=None, t=6.0, cap=8,
                out=FAKE, ldo=32, ws=FAKE, wsb=lay.bytes)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["x"], a["m"], a["k"], a["ldx"], a["w"], a["ldw"], a["sw"], a["n"], a["b"], a["t"],
                 a["cap"], a["out"], a["ldo"], a["ws"], a["wsb"], None)

    assert call(x=None) == EINVAL
    assert call(w=None) == EINVAL
    assert call(sw=None) == EINVAL
    assert call(out=None) == EINVAL
    assert call(ldx=63) == EINVAL
    assert call(ldw=63) == EINVAL
    assert call(ldo=31) == EINVAL
    assert call(cap=-1) == EINVAL
    assert call(k=133145, ldx=133145, ldw=133145) == ERANGE
    assert call(ws=None) == EWORKSPACE
    assert call(wsb=lay.bytes - 1) == EWORKSPACE
    assert call(m=0) == OK
    assert call(n=0) == OK
    assert call(ldw=MAX_LD + 1) == EINVAL
    assert call(ldx=MAX_LD + 1) == EINVAL
    assert call(ldo=MAX_LD + 1) == EINVAL
    assert call(cap=MAX_LD + 1) == EINVAL
    assert L.i8mp_linear_workspace_query(16, 32, 64, MAX_LD + 1, ctypes.byref(lay)) == EINVAL

    qz = L.i8mp_linear_quantize
    assert qz(None, 16, 64, 64, 6.0, 8, FAKE, lay.bytes, None) == EINVAL
    assert qz(FAKE, 16, 64, 63, 6.0, 8, FAKE, lay.bytes, None) == EINVAL
    assert qz(FAKE, 16, 64, 64, 6.0, -1, FAKE, lay.bytes, None) == EINVAL
    assert qz(FAKE, 16, 64, 64, 6.0, 8, FAKE, lay.bytes - 1, None) == EWORKSPACE
    assert qz(FAKE, 16, 133145, 133145, 6.0, 8, FAKE, 1 << 40, None) == ERANGE
    assert qz(None, 0, 64, 64, 6.0, 8, None, 0, None) == OK
    md = L.i8mp_linear_matmul_dequant
    assert md(FAKE, 64, FAKE, lay.bytes, 16, 64, 8, None, 64, FAKE, 32, None, FAKE, 32, None) == EINVAL
    assert md(FAKE, 64, FAKE, lay.bytes, 16, 64, 8, FAKE, 63, FAKE, 32, None, FAKE, 32, None) == EINVAL
    assert md(FAKE, 64, FAKE, lay.bytes, 16, 64, 8, FAKE, 64, FAKE, 32, None, FAKE, 31, None) == EINVAL
    assert md(None, 64, FAKE, lay.bytes, 16, 64, 8, FAKE, 64, FAKE, 32, None, FAKE, 32, None) == EINVAL  # x
    assert md(FAKE, 63, FAKE, lay.bytes, 16, 64, 8, FAKE, 64, FAKE, 32, None, FAKE, 32, None) == EINVAL  # ldx < k
    assert md(FAKE, MAX_LD + 1, FAKE, lay.bytes, 16, 64, 8, FAKE, 64, FAKE, 32, None, FAKE, 32, None) == EINVAL
    assert md(FAKE, 64, None, lay.bytes, 16, 64, 8, FAKE, 64, FAKE, 32, None, FAKE, 32, None) == EWORKSPACE
    assert md(FAKE, 64, FAKE, lay.bytes - 1, 16, 64, 8, FAKE, 64, FAKE, 32, None, FAKE, 32, None) == EWORKSPACE
    assert md(FAKE, 64, FAKE, lay.bytes, 16, 64, 8, FAKE, 64, FAKE, 0, None, FAKE, 32, None) == OK


def test_noalloc_forward_validation(L):
    f = L.i8mp_linear_forward_noalloc
    ESCRATCH = _lib.I8MP_ESCRATCH
    assert len(L.i8mp_status_string(ESCRATCH)) > 0
    # the workspace of 4096 x 22016 (90 MB of codes) does not fit the fixed array
    assert f(FAKE, 4096, 22016, 22016, FAKE, 22016, FAKE, 64, None, 6.0, 256, FAKE, 64, None) == ESCRATCH
    lay = _lib.LinearWorkspaceLayout()
    for m, k, cap in ((2048, 11008, 256), (16, 13824, 256), (1, 133144, 256)):
        assert L.i8mp_linear_workspace_query(m, 64, k, cap, ctypes.byref(lay)) == OK
        assert lay.bytes <= _lib.I8MP_NOALLOC_SCRATCH_BYTES, (m, k)
    assert f(None, 16, 64, 64, FAKE, 64, FAKE, 32, None, 6.0, 8, FAKE, 32, None) == EINVAL
    assert f(FAKE, 16, 64, 63, FAKE, 64, FAKE, 32, None, 6.0, 8, FAKE, 32, None) == EINVAL
    assert f(FAKE, 16, 133145, 133145, FAKE, 133145, FAKE, 32, None, 6.0, 8, FAKE, 32, None) == ERANGE
    assert f(None, 0, 64, 64, None, 64, None, 32, None, 6.0, 8, None, 32, None) == OK   # empty


def test_backward_validation(L):
    lay = _lib.BackwardWorkspaceLayout()
    assert L.i8mp_linear_backward_workspace_query(2048, 4096, 11008, 20, ctypes.byref(lay)) == OK
    assert lay.ld_n == 4096 and lay.ld_m == 2048
    offs = [lay.gq_offset, lay.gs_offset, lay.wtq_offset, lay.wts_offset, lay.gtq_offset, lay.gts_offset,
            lay.xtq_offset, lay.xts_offset, lay.scratch_offset]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.wtq_offset - lay.gq_offset >= 2048 * 4096
    assert lay.bytes >= lay.scratch_offset + lay.scratch_bytes
    assert L.i8mp_linear_backward_workspace_query(133145, 16, 64, 0, ctypes.byref(lay)) == ERANGE
    assert L.i8mp_linear_backward_workspace_query(16, 133145, 64, 0, ctypes.byref(lay)) == ERANGE
    assert L.i8mp_linear_backward_workspace_query(16, 16, 0, 0, ctypes.byref(lay)) == EINVAL
    assert L.i8mp_linear_backward_workspace_query(16, 16, 64, -1, ctypes.byref(lay)) == EINVAL
    assert L.i8mp_linear_backward_workspace_query(16, 16, 64, 0, None) == EINVAL

    assert L.i8mp_linear_backward_workspace_query(16, 32, 64, 8, ctypes.byref(lay)) == OK
    fl = _lib.LinearWorkspaceLayout()
    assert L.i8mp_linear_workspace_query(16, 32, 64, 8, ctypes.byref(fl)) == OK
    args = dict(g=FAKE, ldg=32, x=FAKE, ldx=64, w=FAKE, ldw=64, m=16, n=32, k=64, cap=8, fws=FAKE,
                fwsb=fl.bytes, gx=FAKE, ldgx=64, gw=FAKE, ldgw=64, ws=FAKE, wsb=lay.bytes)

    def call(**kw):
        a = dict(args, **kw)
        return L.i8mp_linear_backward(a["g"], a["ldg"], a["x"], a["ldx"], a["w"], a["ldw"], a["m"], a["n"],
                                      a["k"], a["cap"], a["fws"], a["fwsb"], a["gx"], a["ldgx"], a["gw"],
                                      a["ldgw"], a["ws"], a["wsb"], None)

    assert call(g=None) == EINVAL
    assert call(w=None) == EINVAL
    assert call(x=None) == EINVAL
    assert call(ldg=31) == EINVAL
    assert call(ldw=63) == EINVAL
    assert call(ldx=63) == EINVAL
    assert call(ldgx=63) == EINVAL
    assert call(ldgw=63) == EINVAL
    assert call(ldgw=MAX_LD + 1, gx=None) == EINVAL
    assert call(k=0) == EINVAL
    assert call(cap=-1) == EINVAL
    assert call(m=133145) == ERANGE
    assert call(n=133145, ldg=133145) == ERANGE
    assert call(ws=None) == EWORKSPACE
    assert call(wsb=lay.bytes - 1) == EWORKSPACE
    assert call(fwsb=fl.bytes - 1) == EWORKSPACE
    assert call(gx=None, gw=None) == OK
    assert call(m=0, gw=None) == OK
    assert call(n=0, gx=None) == OK
    # w is only needed for grad_x, x only for grad_w
    if not _has_gpu():
        assert call(w=None, gx=None) == EDEVICE
        assert call(x=None, gw=None) == EDEVICE

    cq = L.i8mp_int8_colwise_quant
    wsb = L.i8mp_colwise_quant_workspace_bytes(100, 70)
    assert wsb >= 70 * 4 and L.i8mp_colwise_quant_workspace_bytes(-1, 70) == 0
    assert cq(FAKE, 100, 70, 70, None, None, 0, FAKE, 99, FAKE, FAKE, wsb, None) == EINVAL   # ldqt < rows
    assert cq(FAKE, 100, 70, 69, None, None, 0, FAKE, 100, FAKE, FAKE, wsb, None) == EINVAL  # lda < cols
    assert cq(FAKE, 100, 70, 70, FAKE, None, 4, FAKE, 100, FAKE, FAKE, wsb, None) == EINVAL  # idx without count
    assert cq(FAKE, 100, 70, 70, None, None, 0, None, 100, FAKE, FAKE, wsb, None) == EINVAL
    assert cq(FAKE, 100, 70, 70, None, None, 0, FAKE, 100, None, FAKE, wsb, None) == EINVAL
    assert cq(FAKE, 100, 70, 70, None, None, 0, FAKE, MAX_LD + 1, FAKE, FAKE, wsb, None) == EINVAL
    assert cq(FAKE, 100, 70, 70, None, None, 0, FAKE, 100, FAKE, FAKE, wsb - 1, None) == EWORKSPACE
    assert cq(FAKE, 100, 0, 70, None, None, 0, FAKE, 100, FAKE, None, 0, None) == OK
    if not _has_gpu():
        assert cq(FAKE, 100, 70, 70, None, None, 0, FAKE, 100, FAKE, FAKE, wsb, None) == EDEVICE


def test_fp4_validation(L):
    q, dqf, dq, lin = L.i8mp_fp4_quantize, L.i8mp_fp4_double_quant, L.i8mp_fp4_dequantize, L.i8mp_fp4_linear
    # quantize: k a positive multiple of 64, ld checks, n == 0 no-op
    assert q(FAKE, 4, 100, 100, FAKE, 64, FAKE, None) == EINVAL
    assert q(FAKE, 4, 0, 64, FAKE, 64, FAKE, None) == EINVAL
    assert q(FAKE, 4, 128, 127, FAKE, 64, FAKE, None) == EINVAL
    assert q(FAKE, 4, 128, 128, FAKE, 63, FAKE, None) == EINVAL
    assert q(None, 4, 128, 128, FAKE, 64, FAKE, None) == EINVAL
    assert q(FAKE, 4, 128, 128, FAKE, 64, None, None) == EINVAL
    assert q(None, 0, 128, 128, None, 64, None, None) == OK
    assert dqf(FAKE, -1, FAKE, FAKE, None) == EINVAL
    assert dqf(None, 0, None, None, None) == OK
    assert dqf(None, 10, FAKE, FAKE, None) == EINVAL
    # dequantize: exactly one kind of scales, a known dtype
    assert dq(FAKE, 64, 4, 128, FAKE, FAKE, FAKE, 0, FAKE, 128, None) == EINVAL
    assert dq(FAKE, 64, 4, 128, None, FAKE, None, 0, FAKE, 128, None) == EINVAL
    assert dq(FAKE, 64, 4, 128, None, None, None, 0, FAKE, 128, None) == EINVAL
    assert dq(FAKE, 64, 4, 128, FAKE, None, None, 7, FAKE, 128, None) == EINVAL
    assert dq(FAKE, 64, 4, 128, FAKE, None, None, 0, FAKE, 127, None) == EINVAL
    assert dq(FAKE, 64, 0, 128, FAKE, None, None, 1, FAKE, 128, None) == OK
    # linear: x and codes 16-byte aligned, ldx a multiple of 8, ldc of 16
    A16 = ctypes.c_void_p(0x1000)
    assert lin(A16, 2, 128, 132, A16, 64, FAKE, None, None, 8, None, A16, 8, None) == EINVAL   # ldx % 8
    assert lin(A16, 2, 128, 128, A16, 72, FAKE, None, None, 8, None, A16, 8, None) == EINVAL   # ldc % 16
    assert lin(ctypes.c_void_p(0x1008), 2, 128, 128, A16, 64, FAKE, None, None, 8, None, A16, 8, None) == EINVAL
    assert lin(A16, 2, 128, 128, A16, 64, FAKE, FAKE, FAKE, 8, None, A16, 8, None) == EINVAL   # both scales
    assert lin(A16, 2, 128, 128, A16, 64, FAKE, None, None, 8, None, A16, 7, None) == EINVAL   # ldout < n
    assert lin(A16, 2, 100, 128, A16, 64, FAKE, None, None, 8, None, A16, 8, None) == EINVAL   # k % 64
    assert lin(None, 0, 128, 128, None, 64, FAKE, None, None, 8, None, None, 8, None) == OK
    if not _has_gpu():
        assert lin(A16, 2, 128, 128, A16, 64, FAKE, None, None, 8, None, A16, 8, None) == EDEVICE
        assert q(FAKE, 4, 128, 128, FAKE, 64, FAKE, None) == EDEVICE


def _has_gpu():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # pragma: no cover
        return False


@pytest.mark.skipif(_has_gpu(), reason="device check only observable without a GPU")
def test_no_device_reported(L):
    lay = _lib.LinearWorkspaceLayout()
    L.i8mp_linear_workspace_query(16, 32, 64, 8, ctypes.byref(lay))
    st = L.i8mp_linear_forward(FAKE, 16, 64, 64, FAKE, 64, FAKE, 32, None, 6.0, 8, FAKE, 32, FAKE,
                               lay.bytes, None)
    assert st == EDEVICE


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        i8.vectorwise_quant(x, 6.0)
    with pytest.raises(ValueError, match="GPU"):
        i8.linear(x, torch.zeros(8, 64, dtype=torch.int8), torch.ones(8))
