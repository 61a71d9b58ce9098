"""The allocation-free forward (fixed scratch array in the library) against
the forward with a caller workspace, called through the C ABI, on two calls
in a row (the second smaller), plus the size limit."""

import ctypes

import numpy as np
import pytest
import torch

import int8_mixed_precision_vectorwise_amd as i8
import oracle
from gpu_util import assert_fp16_close, dev, say
from int8_mixed_precision_vectorwise_amd import _lib
from synth import make_inputs

pytestmark = pytest.mark.gpu

TAU = 6.0


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _both(m, k, n, o, cap, seed):
    L = make_inputs(m, k, n, n_outlier=o, bias_std=0.01, seed=(90, seed, 0), outlier_row_frac=0.5)
    wq, ws = oracle.quantize_weight(L.w)
    x, w, s, b = dev(L.x), dev(wq), dev(ws), dev(L.bias)
    lib = _lib.lib()
    out_a = torch.full((m, n), 7.0, dtype=torch.float16, device="cuda")
    out_b = torch.full((m, n), -7.0, dtype=torch.float16, device="cuda")
    lay = _lib.LinearWorkspaceLayout()
    assert lib.i8mp_linear_workspace_query(m, n, k, cap, ctypes.byref(lay)) == 0
    assert lay.bytes <= _lib.I8MP_NOALLOC_SCRATCH_BYTES
    wsp = torch.empty(lay.bytes, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    say(f"linear_forward_noalloc m={m} k={k} n={n} o={o} cap={cap}")
    st = lib.i8mp_linear_forward_noalloc(_p(x), m, k, k, _p(w), k, _p(s), n, _p(b), TAU, cap, _p(out_a), n,
                                         _stream())
    assert st == 0, _lib.status_string(st)
    say(f"linear_forward (workspace) m={m} k={k} n={n} o={o} cap={cap}")
    st = lib.i8mp_linear_forward(_p(x), m, k, k, _p(w), k, _p(s), n, _p(b), TAU, cap, _p(out_b), n, _p(wsp),
                                 lay.bytes, _stream())
    assert st == 0, _lib.status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    ref = oracle.linear_forward(L.x, wq, ws, L.bias, TAU)
    assert_fp16_close(out_a, ref.out)


def test_noalloc_forward_two_calls_second_smaller():
    _both(300, 1024, 520, 6, 32, 0)      # prefill tiles, two launches
    _both(3, 512, 200, 40, 8, 1)         # one-launch decode forward, past cap, smaller


def test_noalloc_forward_rejects_too_large():
    lib = _lib.lib()
    m, k, n = 4096, 22016, 64           # codes alone are 90 MB
    x = torch.empty((1, 1), dtype=torch.float16, device="cuda")
    say("linear_forward_noalloc too large")
    st = lib.i8mp_linear_forward_noalloc(_p(x), m, k, k, _p(x), k, _p(x), n, None, TAU, 256, _p(x), n,
                                         _stream())
    assert st == _lib.I8MP_ESCRATCH
    with pytest.raises(i8.I8mpError):
        i8.linear_forward_noalloc(torch.empty((m, k), dtype=torch.float16, device="cuda"),
                                  torch.empty((n, k), dtype=torch.int8, device="cuda"),
                                  torch.ones(n, device="cuda"), torch.empty((m, n), dtype=torch.float16,
                                                                              device="cuda"))


def test_noalloc_forward_python_binding():
    m, k, n = 16, 1024, 1024
    L = make_inputs(m, k, n, n_outlier=4, bias_std=0.01, seed=(90, 2, 0))
    wq, ws = oracle.quantize_weight(L.w)
    out = torch.empty((m, n), dtype=torch.float16, device="cuda")
    say("linear_forward_noalloc python binding")
    i8.linear_forward_noalloc(dev(L.x), dev(wq), dev(ws), out, dev(L.bias), TAU, 32)
    torch.cuda.synchronize()
    assert_fp16_close(out, oracle.linear_forward(L.x, wq, ws, L.bias, TAU).out)
