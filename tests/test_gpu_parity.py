"""GPU parity: every entry point of libi8mp.so against the CPU oracle.

Bit-exact: codes, row absmax, outlier bitmap / indices / count, gathered
outlier values, int32 accumulators, weight codes and statistics.
Tolerance (fp16 outputs, fp32 epilogue arithmetic): |gpu - oracle| <=
1e-3 + 1e-2 |oracle| per element.
"""

import numpy as np
import pytest
import torch

import int8_mixed_precision_vectorwise_amd as i8
import oracle
from gpu_util import assert_equal, assert_fp16_close, dev, host, say
from synth import make_inputs

pytestmark = pytest.mark.gpu

TAU = 6.0

QUANT_CASES = [
    # m, k, n_outlier, row_frac, tau
    (1, 1, 0, 1.0, TAU),
    (1, 7, 1, 1.0, TAU),
    (3, 33, 2, 1.0, TAU),
    (5, 257, 3, 0.5, TAU),
    (16, 1024, 4, 1.0, TAU),
    (17, 1000, 6, 0.2, TAU),
    (64, 2049, 9, 0.05, TAU),
    (130, 4096, 7, 1.0, TAU),
    (9, 20000, 20, 0.3, TAU),      # register-resident chunks, largest bucket
    (4, 40000, 5, 1.0, TAU),       # streamed rows
    (2100, 4000, 6, 0.4, TAU),     # two kernels, a wavefront per row
    (300, 20000, 9, 0.5, TAU),     # two kernels, a workgroup per row, 16-load batches
    (33, 300, 0, 1.0, 0.0),        # threshold off
    (8, 96, 96, 1.0, TAU),         # every column an outlier
]


def _quant_layer(m, k, o, frac, seed):
    return make_inputs(m, k, 1, n_outlier=o, lo=6.0, hi=60.0, seed=(70, seed, 0), outlier_row_frac=frac,
                       with_weight=False)


@pytest.mark.parametrize("case", QUANT_CASES, ids=lambda c: "m%d_k%d_o%d_f%g_t%g" % c)
def test_vectorwise_quant_bit_exact(case):
    m, k, o, frac, tau = case
    L = _quant_layer(m, k, o, frac, hash(case) % 1000)
    x = L.x.copy()
    if m > 2:
        x[1] = 0  # a zero row
    say(f"vectorwise_quant m={m} k={k} o={o} tau={tau}")
    q, s, bm = i8.vectorwise_quant(dev(x), tau)
    torch.cuda.synchronize()
    ref = oracle.vectorwise_quant(x, tau)
    assert_equal(q, ref.q, "codes")
    assert_equal(s, ref.absmax, "absmax")
    assert_equal(bm.view(torch.int32), ref.bitmap.view(np.int32), "bitmap")


def test_vectorwise_quant_unaligned_rows():
    m, k = 37, 301
    L = _quant_layer(m, k + 3, 4, 0.7, 5)
    full = dev(L.x)
    x = full[:, 1:k + 1]             # odd element offset, ld = k + 3
    say("vectorwise_quant unaligned view")
    q, s, bm = i8.vectorwise_quant(x, TAU)
    torch.cuda.synchronize()
    ref = oracle.vectorwise_quant(np.ascontiguousarray(L.x[:, 1:k + 1]), TAU)
    assert_equal(q, ref.q, "codes")
    assert_equal(s, ref.absmax, "absmax")
    assert_equal(bm.view(torch.int32), ref.bitmap.view(np.int32), "bitmap")


@pytest.mark.parametrize("n,k", [(1, 1), (7, 33), (300, 1000), (4096, 1024), (64, 13824)])
def test_weight_quant_bit_exact(n, k):
    w = (np.random.default_rng([71, n, k]).standard_normal((n, k)) * 0.02).astype(np.float16)
    say(f"quantize_weight n={n} k={k}")
    wq, ws = i8.quantize_weight(dev(w))
    torch.cuda.synchronize()
    rq, rs = oracle.quantize_weight(w)
    assert_equal(wq, rq, "weight codes")
    assert_equal(ws, rs, "weight absmax")


@pytest.mark.parametrize("m,k,o,cap", [(5, 100, 3, 8), (64, 4096, 7, 32), (16, 1024, 0, 8),
                                       (4, 200, 12, 5), (1, 70, 2, 0), (7, 300, 9, None)])
def test_outlier_extract_bit_exact(m, k, o, cap):
    L = _quant_layer(m, k, o, 0.6, 9)
    say(f"outlier_extract m={m} k={k} o={o} cap={cap}")
    xd = dev(L.x)
    _, _, bm = i8.vectorwise_quant(xd, TAU)
    idx, count, xo = i8.outlier_extract(xd, bm, cap, strict=False)
    cap = k if cap is None else cap
    torch.cuda.synchronize()
    ref = oracle.vectorwise_quant(L.x, TAU)
    ridx, rcount, rxo = oracle.outlier_extract(L.x, ref.cols, cap)
    assert int(host(count)[0]) == rcount
    assert_equal(idx, ridx, "idx")
    assert_equal(xo.view(torch.int16), rxo.view(np.int16), "x_out")


@pytest.mark.parametrize("m,k", [(512, 1024), (300, 20000), (6, 5000)], ids=["wave_rows", "block_rows", "col_slices"])
def test_quant_workspace_reuse(m, k):
    """Three calls on one workspace, each with other outlier columns: every
    result is the oracle's (nothing carries over from the previous call)."""
    ws = i8.LinearWorkspace.create(m, 8, k, 64, torch.device("cuda"))
    for call in range(3):
        L = make_inputs(m, k, 1, n_outlier=3 + call, lo=6.0, hi=60.0, seed=(72, call, m), outlier_row_frac=0.5,
                        with_weight=False)
        say(f"linear_quantize reuse m={m} k={k} call={call}")
        i8.linear_quantize(dev(L.x), ws, TAU)
        torch.cuda.synchronize()
        ref = oracle.vectorwise_quant(L.x, TAU)
        assert_equal(ws.codes(), ref.q, "codes")
        assert_equal(ws.absmax(), ref.absmax, "absmax")
        assert_equal(ws.bitmap().view(torch.int32), ref.bitmap.view(np.int32), "bitmap")
        ridx, rcount, rxo = oracle.outlier_extract(L.x, ref.cols, 64)
        assert int(host(ws.count())[0]) == rcount
        assert_equal(ws.idx()[:64], ridx, "idx")
        assert_equal(ws.x_out().view(torch.int16), rxo.view(np.int16), "x_out")


MM_SHAPES = [(1, 1, 1), (3, 5, 17), (17, 63, 65), (65, 127, 129), (255, 257, 128), (300, 600, 300),
             (512, 256, 1024), (1, 4096, 5120), (16, 13824, 640), (257, 259, 4100),
             (3, 777, 1280), (2, 513, 640), (4, 100, 13824),
             (200, 300, 2560), (130, 190, 2176),  # two K pipelines per workgroup (17 K tiles: one pipeline's last is empty)
             (2100, 5000, 512), (2100, 5000, 640), (1800, 6000, 128),  # 256 x 256 ping-pong tiles, ragged m and n
             # whole rounds of 256 x 256 tiles, the remaining columns in a second launch of smaller tiles
             (2048, 9000, 512), (2100, 9000, 512),
             # m <= 16 with 257 to 512 groups of 16 rows and long K: one workgroup per CU, two blocks
             (16, 5003, 8192), (7, 4490, 8320), (12, 8000, 8200), (2, 4500, 16512),
             # ... 513 to 1024 groups: two groups per workgroup
             (16, 9001, 4096), (9, 12000, 4200), (5, 9001, 4224), (12, 16000, 4100),
             # ... and past 1024 groups, whole 16-row groups
             (4, 17000, 4096)]


@pytest.mark.parametrize("m,n,k", MM_SHAPES)
def test_linear_matmul_bit_exact(m, n, k):
    rng = np.random.default_rng([72, m, n, k])
    a = rng.integers(-128, 128, (m, k), dtype=np.int16).astype(np.int8)
    b = rng.integers(-128, 128, (n, k), dtype=np.int16).astype(np.int8)
    say(f"linear_matmul m={m} n={n} k={k}")
    c = i8.linear_matmul(dev(a), dev(b))
    torch.cuda.synchronize()
    ref = a.astype(np.int64) @ b.astype(np.int64).T
    assert_equal(c, oracle.int8_linear_matmul(a, b), "C")
    assert np.array_equal(host(c).astype(np.int64), ref)


def test_linear_matmul_unaligned_and_strided():
    rng = np.random.default_rng(73)
    m, n, k = 70, 90, 203
    a_full = rng.integers(-127, 128, (m, k + 5), dtype=np.int16).astype(np.int8)
    b_full = rng.integers(-127, 128, (n, k + 3), dtype=np.int16).astype(np.int8)
    say("linear_matmul unaligned")
    c = i8.linear_matmul(dev(a_full)[:, 1:k + 1], dev(b_full)[:, 2:k + 2])
    torch.cuda.synchronize()
    assert_equal(c, oracle.int8_linear_matmul(np.ascontiguousarray(a_full[:, 1:k + 1]),
                                              np.ascontiguousarray(b_full[:, 2:k + 2])), "C")


def test_linear_matmul_int32_extreme():
    k = 8192
    a = np.full((3, k), 127, np.int8)
    a[1] = -127
    b = np.full((2, k), 127, np.int8)
    b[1, ::2] = -128
    say("linear_matmul extremes")
    c = i8.linear_matmul(dev(a), dev(b))
    torch.cuda.synchronize()
    assert_equal(c, oracle.int8_linear_matmul(a, b), "C")


@pytest.mark.parametrize("m,n,k,o,bias", [(16, 1024, 1024, 4, True), (70, 300, 513, 9, False),
                                          (33, 65, 200, 0, True), (5, 40, 64, 40, True)])
def test_mm_dequant_parity(m, n, k, o, bias):
    L = make_inputs(m, k, n, n_outlier=o, bias_std=0.01 if bias else None, seed=(74, m, 0))
    wq, ws = oracle.quantize_weight(L.w)
    ref = oracle.linear_forward(L.x, wq, ws, L.bias, TAU)
    cap = max(o, 1)
    ridx, rcount, rxo = oracle.outlier_extract(L.x, ref.quant.cols, cap)
    say(f"mm_dequant m={m} n={n} k={k} o={o}")
    count = torch.tensor([rcount], dtype=torch.int32, device="cuda")
    out = i8.mm_dequant(dev(ref.c), dev(ref.quant.absmax), dev(ws), dev(L.bias) if bias else None,
                        (dev(rxo), dev(ridx), count, dev(wq)))
    out_plain = i8.mm_dequant(dev(ref.c), dev(ref.quant.absmax), dev(ws), dev(L.bias) if bias else None)
    torch.cuda.synchronize()
    assert_fp16_close(out, ref.out)
    no_outl = oracle.mm_dequant(ref.c, ref.quant.absmax, ws, L.bias)
    assert_fp16_close(out_plain, no_outl, "out without outlier term")


FWD_CASES = [
    # m, k, n, o, frac, bias, tau, cap
    (16, 1024, 1024, 4, 1.0, True, TAU, 256),     # tiny workload shape
    (1, 64, 32, 1, 1.0, False, TAU, 8),
    (3, 33, 5, 2, 1.0, True, TAU, 8),
    (300, 520, 600, 11, 0.3, True, TAU, 64),
    (257, 1000, 259, 5, 1.0, False, TAU, 32),
    (40, 2100, 300, 5, 1.0, True, TAU, 32),       # two K pipelines, 17 K tiles
    (64, 256, 512, 0, 1.0, True, TAU, 32),        # no outliers present
    (40, 300, 100, 3, 1.0, True, 0.0, 32),        # threshold off
    (12, 96, 70, 96, 1.0, True, TAU, 96),         # every column an outlier
    (4, 5120, 1000, 8, 1.0, False, TAU, 256),     # decode-shaped
    (16, 2048, 512, 40, 0.5, False, TAU, 64),     # more outliers than one fp16 MFMA step
    # prefill tiles past the 16 outlier slots copied to LDS before the epilogue
    (1536, 384, 6144, 20, 0.5, True, TAU, 64),    # 256 x 256: slots 16..19 from the stash
    (1536, 256, 6144, 40, 0.5, False, TAU, 64),   # 256 x 256: slots 24..39 gathered
    (768, 256, 6144, 30, 0.5, True, TAU, 64),     # 256 x 128: slots 16..29 gathered
    (768, 256, 3072, 17, 1.0, False, TAU, 32),    # 128 x 128: one slot past 16
    (256, 256, 6144, 16, 0.5, True, TAU, 16),     # 128 x 64: exactly 16 slots, cap 16
    # weights with rows of 250 bytes (not 16-byte aligned): the register-staged kernel
    (768, 250, 6144, 20, 0.5, True, TAU, 64),     # 256 x 128: copies in the wave's staging area
    (1536, 250, 6144, 30, 0.5, False, TAU, 64),   # 256 x 256 without a stash: every slot gathered
    (2100, 1000, 5000, 9, 0.5, True, TAU, 64),    # 256 x 256 ping-pong, ragged m, n and k
    # 256 x 256 tiles over whole rounds, then the remaining columns in a second launch
    (2048, 512, 9000, 9, 0.5, True, TAU, 64),     # tail of 128 x 64 tiles: bias and outliers offset
    (2100, 512, 9000, 30, 0.5, False, TAU, 64),   # tail of 128 x 128 tiles, ragged m, slots past 16
    # m <= 2: the dot-product GEMV (outliers taken from the weight stream)
    (1, 1000, 77, 3, 1.0, True, TAU, 16),         # unaligned k and n
    (2, 4096, 264, 5, 0.5, False, TAU, 32),
    (1, 13824, 1024, 70, 0.5, True, TAU, 128),    # more outlier columns than the stream handles
    (2, 640, 2048, 0, 1.0, False, TAU, 8),        # no outliers
    (2, 512, 96, 0, 1.0, True, 0.0, 8),           # threshold off
    (1, 2048, 5000, 3, 1.0, True, TAU, 16),       # three weight rows per wave, the last wave short
    (2, 16384, 256, 10, 1.0, True, TAU, 64),      # the one-launch forward's most chunks per thread at m = 2
    (1, 32768, 128, 12, 0.5, False, TAU, 64),     # ... and at m = 1 (32 KB of activations)
    # 3 <= m <= 16, or m <= 2 past the GEMV's LDS: the MFMA decode kernel (outliers from its ring)
    (3, 2000, 130, 9, 1.0, True, TAU, 32),        # k not a multiple of 128, n of 16
    (4, 8192, 600, 8, 1.0, False, TAU, 256),
    (4, 13824, 300, 12, 0.5, True, TAU, 64),
    (2, 16512, 200, 6, 1.0, True, TAU, 32),       # m = 2 one chunk past the GEMV's 32 KB
    (9, 3000, 200, 33, 1.0, False, TAU, 64),      # past the ring's 32 columns: the rest gathered
    (3, 1024, 4500, 70, 0.5, False, TAU, 128),    # several rows per wave and the gathered outliers
    (1, 96, 70, 96, 1.0, True, TAU, 96),          # every column an outlier, past the stream's 64
    # the MFMA decode kernel on long rows: column-slice quantizer, four waves per group
    (8, 13824, 700, 40, 0.5, True, TAU, 16),      # ring + gathered outliers, past cap
    (16, 8192, 1000, 5, 1.0, False, TAU, 64),     # n not a multiple of 16
    (16, 5120, 2000, 8, 1.0, True, TAU, 256),     # two waves per group
    # 257 to 512 groups of 16 rows and long K: one workgroup per CU, one group of ceil(n / 256) rows
    (16, 8192, 5003, 8, 1.0, True, TAU, 64),      # 20-row groups, the last 3 rows
    (7, 8320, 4490, 40, 0.5, False, TAU, 16),     # half the activation rows, past the ring and cap, last group 8 rows
    (12, 8200, 8000, 9, 1.0, True, TAU, 256),     # 32-row groups, k not a multiple of 128
    (2, 16512, 4500, 6, 1.0, True, TAU, 32),      # two rows past the GEMV's LDS
    # 513 to 1024 groups: two groups of ceil(n / 512) rows per workgroup
    (16, 4096, 9001, 12, 0.5, True, TAU, 64),     # 18-row groups, the last 1 row
    (6, 5120, 13824, 40, 1.0, False, TAU, 16),    # 27-row groups, past the ring and cap
    (9, 4200, 12000, 8, 1.0, True, TAU, 32),      # k not a multiple of 128
    (5, 4224, 9001, 40, 0.5, False, TAU, 16),     # past the ring and cap
    (4, 4100, 16000, 9, 1.0, True, TAU, 256),     # 32-row groups, k not a multiple of 128
    # past 1024 groups: whole 16-row groups again
    (4, 4096, 17000, 9, 1.0, True, TAU, 64),
]


def _check_workspace(wsp, x, ref, cap):
    """Codes, absmax, bitmap, count, the whole index list and the first cap
    gathered columns of a forward workspace, bit for bit."""
    assert_equal(wsp.codes(), ref.q, "codes")
    assert_equal(wsp.absmax(), ref.absmax, "absmax")
    assert_equal(wsp.bitmap().view(torch.int32), ref.bitmap.view(np.int32), "bitmap")
    assert int(host(wsp.count())[0]) == ref.cols.size
    ridx, _, _ = oracle.outlier_extract(x, ref.cols, int(wsp.layout.idx_len))
    assert_equal(wsp.idx(), ridx, "idx (every outlier column)")
    _, _, rxo = oracle.outlier_extract(x, ref.cols, cap)
    assert_equal(wsp.x_out().contiguous().view(torch.int16), rxo.view(np.int16), "x_out")


def _check_forward(L, wq, ws, tau, cap, what):
    ref = oracle.linear_forward(L.x, wq, ws, L.bias, tau)
    m, k = L.x.shape
    n = wq.shape[0]
    say(f"linear_forward {what}")
    wsp = i8.LinearWorkspace.create(m, n, k, cap, "cuda")
    out = i8.linear(dev(L.x), dev(wq), dev(ws), dev(L.bias) if L.bias is not None else None, tau, cap, wsp)
    torch.cuda.synchronize()
    _check_workspace(wsp, L.x, ref.quant, cap)
    assert_fp16_close(out, ref.out)
    return out, ref


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "m%d_k%d_n%d_o%d_f%g_b%d_t%g_c%d" % c)
def test_linear_forward_parity(case):
    m, k, n, o, frac, bias, tau, cap = case
    L = make_inputs(m, k, n, n_outlier=o, bias_std=0.01 if bias else None, seed=(75, m, k),
                    outlier_row_frac=frac)
    wq, ws = oracle.quantize_weight(L.w)
    _check_forward(L, wq, ws, tau, cap, str(case))


def test_linear_forward_gpu_quantized_weights():
    """Weights quantized on the GPU are the oracle's, so the whole path can run
    from the fp16 weight without touching the oracle."""
    L = make_inputs(48, 700, 333, n_outlier=3, bias_std=0.01, seed=(76, 0, 0))
    say("forward from GPU-quantized weights")
    wq_g, ws_g = i8.quantize_weight(dev(L.w))
    out = i8.linear(dev(L.x), wq_g, ws_g, dev(L.bias), TAU, 32)
    torch.cuda.synchronize()
    wq, ws = oracle.quantize_weight(L.w)
    assert_equal(wq_g, wq, "weight codes")
    ref = oracle.linear_forward(L.x, wq, ws, L.bias, TAU)
    assert_fp16_close(out, ref.out)


def test_saved_int8_weights_reload_bit_exact(tmp_path):
    """Weight state quantized on the GPU, saved with its row absmax, read back
    onto the GPU: the same tensors, and the forward from them is the same."""
    L = make_inputs(40, 520, 300, n_outlier=4, bias_std=0.01, seed=(76, 1, 0))
    say("save / load int8 weights")
    wq_g, ws_g = i8.quantize_weight(dev(L.w))
    path = str(tmp_path / "w.safetensors")
    i8.save_int8_weights(path, {"layer": (wq_g, ws_g)})
    wq_l, ws_l = i8.load_int8_weights(path, device="cuda")["layer"]
    assert wq_l.device.type == "cuda" and torch.equal(wq_l, wq_g) and torch.equal(ws_l, ws_g)
    out_a = i8.linear(dev(L.x), wq_g, ws_g, dev(L.bias), TAU, 32)
    out_b = i8.linear(dev(L.x), wq_l, ws_l, dev(L.bias), TAU, 32)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    wq, ws = oracle.quantize_weight(L.w)
    assert_equal(wq_l, wq, "weight codes")
    assert_equal(ws_l, ws, "weight row absmax")


def test_linear_forward_zero_rows_and_zero_input():
    L = make_inputs(20, 256, 130, n_outlier=2, bias_std=0.01, seed=(77, 0, 0))
    L.x[[0, 7, 19]] = 0
    wq, ws = oracle.quantize_weight(L.w)
    _check_forward(L, wq, ws, TAU, 32, "zero rows")
    L.x[:] = 0
    out, ref = _check_forward(L, wq, ws, TAU, 32, "zero input")
    assert np.array_equal(host(out), np.repeat(L.bias[None, :], 20, 0))


PAST_CAP_CASES = [
    # m, k, n, o, frac, bias, cap: more outlier columns than the gathered
    # capacity; every path must still give the method's result
    (8, 512, 64, 12, 1.0, False, 4),          # prefill 64 x 64 tiles
    (300, 520, 600, 11, 0.3, True, 0),        # no gathered columns at all
    (768, 256, 6144, 30, 0.5, True, 4),       # 256 x 128: operands of the first 16 slots not copied early
    (1536, 384, 6144, 40, 0.5, False, 8),     # 256 x 256: stash for 24 slots, X_O for 8, x past them
    (1536, 256, 6144, 20, 1.0, True, 17),     # 256 x 256: a 16-slot group straddling cap
    (768, 250, 6144, 20, 0.5, True, 5),       # register-staged kernel (unaligned weight rows)
    (40, 2100, 300, 5, 1.0, True, 2),         # two K pipelines
    (1, 4096, 300, 70, 0.5, True, 8),         # one-launch GEMV forward, past the stream's 64 columns
    (2, 2000, 130, 9, 1.0, False, 4),         # one-launch GEMV forward, m = 2
    (2, 8192, 200, 70, 1.0, False, 0),        # one-launch GEMV forward, no gathered columns
    (3, 2000, 130, 9, 1.0, False, 4),         # MFMA decode kernel, m = 3
    (4, 8192, 200, 70, 1.0, False, 0),        # MFMA decode kernel, every column past the ring gathered
    (9, 3000, 200, 33, 1.0, True, 4),         # MFMA decode kernel: ring 32, then gathered
    (16, 1024, 256, 40, 0.5, False, 0),       # MFMA decode kernel, no gathered columns
    (4, 13824, 300, 12, 0.5, True, 2),        # MFMA decode kernel, four waves per group
]


@pytest.mark.parametrize("case", PAST_CAP_CASES, ids=lambda c: "m%d_k%d_n%d_o%d_f%g_b%d_c%d" % c)
def test_linear_forward_past_cap(case):
    """The fused forward gives the oracle's result for any outlier count: the
    columns past cap read x through the index list.  The index list holds
    every outlier column, X_O the first cap."""
    m, k, n, o, frac, bias, cap = case
    L = make_inputs(m, k, n, n_outlier=o, bias_std=0.01 if bias else None, seed=(78, m, k),
                    outlier_row_frac=frac)
    wq, ws = oracle.quantize_weight(L.w)
    out, ref = _check_forward(L, wq, ws, TAU, cap, f"past cap {case}")
    assert ref.quant.cols.size == o > cap


@pytest.mark.parametrize("case", [(2, 4096, 264, 40, 4), (3, 2000, 130, 70, 0), (12, 3000, 200, 45, 8),
                                  (520, 300, 1000, 30, 3)], ids=lambda c: "m%d_k%d_n%d_o%d_c%d" % c)
def test_two_launch_forward_past_cap(case):
    """linear_quantize + linear_matmul_dequant (the GEMV of m <= 2 reading the
    workspace codes, the MFMA decode kernel, a prefill tile) past cap."""
    m, k, n, o, cap = case
    L = make_inputs(m, k, n, n_outlier=o, bias_std=0.01, seed=(78, 1, m), outlier_row_frac=0.5)
    wq, ws = oracle.quantize_weight(L.w)
    ref = oracle.linear_forward(L.x, wq, ws, L.bias, TAU)
    x = dev(L.x)
    wsp = i8.LinearWorkspace.create(m, n, k, cap, "cuda")
    say(f"two-launch forward past cap {case}")
    i8.linear_quantize(x, wsp, TAU)
    out = i8.linear_matmul_dequant(x, wsp, dev(wq), dev(ws), dev(L.bias))
    torch.cuda.synchronize()
    assert wsp.outliers_past_cap()
    _check_workspace(wsp, L.x, ref.quant, cap)
    assert_fp16_close(out, ref.out)


def _workspace_state(wsp):
    return [wsp.codes().clone(), wsp.absmax().clone(), wsp.bitmap().clone(), wsp.idx().clone(),
            wsp.count().clone(), wsp.x_out().clone()]


@pytest.mark.parametrize("m,k,n,o,cap", [(1, 5120, 384, 8, 256), (2, 4096, 264, 5, 32), (3, 2000, 130, 9, 4),
                                         (4, 8192, 200, 70, 128), (4, 5120, 256, 0, 8), (1, 64, 16, 40, 16)])
def test_decode_forward_matches_two_launches(m, k, n, o, cap):
    """One or two rows: the one-launch forward (quantization inside the GEMV)
    leaves the workspace and the output of quantize + matmul_dequant, bit for
    bit.  Three and four rows take the two launches either way."""
    L = make_inputs(m, k, n, n_outlier=o, bias_std=0.01, seed=(82, m, k), outlier_row_frac=0.5)
    wq, ws = oracle.quantize_weight(L.w)
    x, w, s, b = dev(L.x), dev(wq), dev(ws), dev(L.bias)
    wa = i8.LinearWorkspace.create(m, n, k, cap, "cuda")
    wb = i8.LinearWorkspace.create(m, n, k, cap, "cuda")
    say(f"one-launch forward m={m} k={k} n={n} o={o} cap={cap}")
    one = i8.linear(x, w, s, b, TAU, cap, wa)
    torch.cuda.synchronize()
    say(f"two-launch forward m={m} k={k} n={n} o={o} cap={cap}")
    i8.linear_quantize(x, wb, TAU)
    two = i8.linear_matmul_dequant(x, wb, w, s, b)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))
    for name, a, c in zip(("codes", "absmax", "bitmap", "idx", "count", "x_out"),
                          _workspace_state(wa), _workspace_state(wb)):
        assert torch.equal(a.view(torch.uint8), c.view(torch.uint8)), name
    assert int(host(wa.count())[0]) == o
    assert wa.outliers_past_cap() == (o > cap)
    ref = oracle.linear_forward(L.x, wq, ws, L.bias, TAU)
    assert_fp16_close(one, ref.out)


@pytest.mark.parametrize("m", [1, 2])
def test_gemv_outlier_columns_sharing_a_lane(m):
    """Outlier columns 5, 6, 7, 1029 and 2053 all sit in lane 0's bytes of
    their 1 KB chunks (more than a lane keeps in registers), 100 in lane 6."""
    k, n = 4096, 300
    L = make_inputs(m, k, n, bias_std=0.01, seed=(84, m, 0))
    cols = [5, 6, 7, 100, 1029, 2053]
    L.x[:, cols] = np.float16(25.0)
    L.x[0, 6] = np.float16(-40.0)
    wq, ws = oracle.quantize_weight(L.w)
    ref = oracle.linear_forward(L.x, wq, ws, L.bias, TAU)
    assert list(ref.quant.cols) == cols
    x, w, s_, b = dev(L.x), dev(wq), dev(ws), dev(L.bias)
    say(f"gemv outliers sharing a lane m={m}")
    wa = i8.LinearWorkspace.create(m, n, k, 32, "cuda")
    one = i8.linear(x, w, s_, b, TAU, 32, wa)
    wb = i8.LinearWorkspace.create(m, n, k, 32, "cuda")
    i8.linear_quantize(x, wb, TAU)
    two = i8.linear_matmul_dequant(x, wb, w, s_, b)
    torch.cuda.synchronize()
    assert_fp16_close(one, ref.out)
    assert_fp16_close(two, ref.out)


@pytest.mark.parametrize("pad", [8, 1], ids=["ldx_aligned", "ldx_odd"])
def test_decode_forward_strided_x(pad):
    """x with a row stride: an aligned one takes the one-launch forward, an odd
    one the two-launch path; both give the oracle's result."""
    m, k, n = 2, 1536, 256
    L = make_inputs(m, k, n, n_outlier=4, bias_std=0.01, seed=(83, pad, 0))
    wq, ws = oracle.quantize_weight(L.w)
    big = torch.zeros((m, k + pad), dtype=torch.float16, device="cuda")
    big[:, :k] = dev(L.x)
    x = big[:, :k]
    say(f"strided x m={m} k={k} ldx={k + pad}")
    wsp = i8.LinearWorkspace.create(m, n, k, 32, "cuda")
    out = i8.linear(x, dev(wq), dev(ws), dev(L.bias), TAU, 32, wsp)
    torch.cuda.synchronize()
    ref = oracle.linear_forward(L.x, wq, ws, L.bias, TAU)
    assert_equal(wsp.codes(), ref.quant.q, "codes")
    assert_fp16_close(out, ref.out)


DEQ_CASES = [
    # m, k, ldq pad, dtype
    (1, 1, 0, "f16"),
    (3, 17, 0, "f32"),        # ragged: a partial 16-code chunk
    (64, 4096, 0, "f16"),
    (64, 4096, 0, "f32"),
    (300, 1000, 24, "f16"),   # strided codes: the element-wise path
    (5, 7000, 0, "f32"),
]


@pytest.mark.parametrize("case", DEQ_CASES, ids=lambda c: "m%d_k%d_pad%d_%s" % c)
def test_vectorwise_dequant(case):
    """out = q * fl32(absmax / 127) against the oracle (fp32: two fp32
    roundings, |err| <= 2^-22 |ref|; fp16: one more, half an fp16 ulp or the
    subnormal step), and bit for bit against the same two IEEE fp32 operations."""
    m, k, pad, dt = case
    rng = np.random.default_rng(m * 131 + k)
    qfull = rng.integers(-127, 128, size=(m, k + pad), dtype=np.int8)
    absmax = (rng.random(m) * 8 + 1e-3).astype(np.float32)
    q = torch.from_numpy(qfull).cuda()[:, :k]
    dtype = torch.float16 if dt == "f16" else torch.float32
    say(f"vectorwise_dequant m={m} k={k} pad={pad} {dt}")
    out = i8.vectorwise_dequant(q, dev(absmax), dtype)
    torch.cuda.synchronize()
    got = host(out).astype(np.float64)
    ref = oracle.vectorwise_dequant(qfull[:, :k], absmax)
    if dt == "f32":
        assert np.all(np.abs(got - ref) <= 2.0 ** -22 * np.abs(ref))
    else:
        assert np.all(np.abs(got - ref) <= 2.0 ** -11 * np.abs(ref) * (1 + 2.0 ** -10) + 2.0 ** -24)
    f32 = qfull[:, :k].astype(np.float32) * (absmax / np.float32(127))[:, None]
    want = f32 if dt == "f32" else f32.astype(np.float16)
    assert np.array_equal(host(out).view(np.uint32 if dt == "f32" else np.uint16),
                          want.view(np.uint32 if dt == "f32" else np.uint16))


def test_vectorwise_dequant_round_trip():
    """Quantize then dequantize: within half a code of x (s / 254 plus the fp32
    roundings) in every non-outlier column, 0 in outlier columns."""
    L = make_inputs(40, 3000, 1, n_outlier=5, seed=(85, 0, 0), with_weight=False)
    say("quant -> dequant round trip")
    q, s_, bm = i8.vectorwise_quant(dev(L.x), TAU)
    back = i8.vectorwise_dequant(q, s_, torch.float32)
    torch.cuda.synchronize()
    x = L.x.astype(np.float64)
    sx = host(s_).astype(np.float64)
    ref = oracle.vectorwise_quant(L.x, TAU)
    keep = np.ones(x.shape[1], bool)
    keep[ref.cols] = False
    err = np.abs(host(back).astype(np.float64) - x)[:, keep]
    assert np.all(err <= (sx / 254.0)[:, None] * (1 + 2.0 ** -12) + 1e-30)
    assert np.all(host(back)[:, ~keep] == 0)


def test_empty_calls_are_noops():
    say("empty calls")
    x = torch.empty((0, 64), dtype=torch.float16, device="cuda")
    q, s, bm = i8.vectorwise_quant(x, TAU)
    assert q.shape == (0, 64)
    c = i8.linear_matmul(torch.empty((0, 64), dtype=torch.int8, device="cuda"),
                         torch.zeros((5, 64), dtype=torch.int8, device="cuda"))
    assert c.shape == (0, 5)
    out = i8.linear(x, torch.zeros((5, 64), dtype=torch.int8, device="cuda"),
                    torch.ones(5, device="cuda"), None, TAU, 8)
    torch.cuda.synchronize()
    assert out.shape == (0, 5)
    assert not host(bm).any()


def test_deterministic_repeat():
    L = make_inputs(300, 1024, 700, n_outlier=6, bias_std=0.01, seed=(79, 0, 0))
    wq, ws = oracle.quantize_weight(L.w)
    x, w, s, b = dev(L.x), dev(wq), dev(ws), dev(L.bias)
    say("determinism")
    o1 = i8.linear(x, w, s, b, TAU, 32).clone()
    o2 = i8.linear(x, w, s, b, TAU, 32).clone()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_non_default_stream():
    L = make_inputs(64, 512, 256, n_outlier=3, bias_std=0.01, seed=(80, 0, 0))
    wq, ws = oracle.quantize_weight(L.w)
    x, w, s, b = dev(L.x), dev(wq), dev(ws), dev(L.bias)
    torch.cuda.synchronize()
    say("side stream")
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        out = i8.linear(x, w, s, b, TAU, 32)
    st.synchronize()
    ref = oracle.linear_forward(L.x, wq, ws, L.bias, TAU)
    assert_fp16_close(out, ref.out)


@pytest.mark.parametrize("m,k,n", [(128, 1024, 512), (2, 1024, 512), (8, 1024, 512), (1100, 1024, 512),
                                   (16, 8192, 5003)])
def test_graph_capture_replays_match_eager(m, k, n):
    """m = 2: the one-launch GEMV forward; 8: the column-slice quantizer and the
    MFMA decode kernel; 16 with 313 groups of 16 rows: the decode kernel's
    one-workgroup-per-CU groups; 128: detection + quantization launches; 1100:
    the single read of x (bitmap clearing, atomics into the partial bitmaps).
    Every replay runs on a workspace filled with garbage first."""
    L = make_inputs(m, k, n, n_outlier=5, bias_std=0.01, seed=(81, m, 0))
    wq, ws = oracle.quantize_weight(L.w)
    x, w, s, b = dev(L.x), dev(wq), dev(ws), dev(L.bias)
    wsp = i8.LinearWorkspace.create(m, n, k, 32, "cuda")
    out = torch.empty((m, n), dtype=torch.float16, device="cuda")
    say(f"graph capture m={m} k={k} n={n}")
    eager = i8.linear(x, w, s, b, TAU, 32, wsp).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            i8.linear(x, w, s, b, TAU, 32, wsp, out)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(0)
        wsp.buf.fill_(0x5a)      # the replay must not depend on workspace contents
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), rep
    ref = oracle.linear_forward(L.x, wq, ws, L.bias, TAU)
    assert_fp16_close(out, ref.out)


def test_outlier_extract_strict_raises_past_cap():
    L = _quant_layer(6, 300, 9, 1.0, 11)
    xd = dev(L.x)
    _, _, bm = i8.vectorwise_quant(xd, TAU)
    say("outlier_extract strict past cap")
    with pytest.raises(ValueError):
        i8.outlier_extract(xd, bm, 4)
    idx, count, _ = i8.outlier_extract(xd, bm)     # cap = k: every column
    torch.cuda.synchronize()
    assert int(host(count)[0]) == 9


# ---- the threshold's edge: |x| >= tau decides, in fp32 on both sides --------

BELOW6 = np.float16(5.99609375)    # largest fp16 below 6
ABOVE6 = np.float16(6.00390625)    # smallest fp16 above 6


def _edge_input(m, k, n, seed):
    """Seeded layer (bulk below 6) with columns planted at the threshold's
    edge, each large in a single row only: +6.0 (col a), -6.0 (col a2),
    the largest fp16 below 6 (col b, in two rows with both signs), the
    smallest above 6 (col c).  Columns straddle 8-column chunks and 32-column
    bitmap words.  Returns the layer and the columns."""
    L = make_inputs(m, k, n, bias_std=0.01, seed=(86, m, k))
    rng = np.random.default_rng([86, m, k, n])
    cols = np.sort(rng.choice(np.arange(1, k - 1), size=4, replace=False))
    a, a2, b, c = (int(v) for v in rng.permutation(cols))
    rows = rng.integers(0, m, size=5)
    L.x[rows[0], a] = np.float16(6.0)
    L.x[rows[1], a2] = np.float16(-6.0)
    L.x[rows[2], b] = BELOW6
    L.x[rows[3], b] = -BELOW6
    L.x[rows[4], c] = ABOVE6
    return L, (a, a2, b, c)


EDGE_CASES = [
    # m, k, n, tau: tau = 6.001 is not an fp16 value (6.0 is then below it)
    (1, 1000, 77, 6.0),        # one-launch GEMV forward (detection in its prologue)
    (1, 1000, 77, 6.001),
    (3, 2048, 130, 6.0),
    (9, 3000, 200, 6.0),       # quantizer kernels + MFMA decode kernel
    (9, 3000, 200, 6.001),
    (300, 1024, 520, 6.0),     # detect + quantize kernels + prefill tile
    (300, 1024, 520, 6.001),
    (1100, 1024, 130, 6.0),    # single-read quantizer (1024 rows or more) + prefill tile
    (1100, 1024, 130, 6.001),
    (2, 33000, 64, 6.0),       # single-workgroup quantizer (two rows), MFMA decode kernel
]


@pytest.mark.parametrize("case", EDGE_CASES, ids=lambda c: "m%d_k%d_n%d_t%g" % c)
def test_threshold_edge_forward(case):
    m, k, n, tau = case
    L, (a, a2, b, c) = _edge_input(m, k, n, seed=0)
    wq, ws = oracle.quantize_weight(L.w)
    ref = oracle.linear_forward(L.x, wq, ws, L.bias, tau)
    want = {c} | ({a, a2} if tau == 6.0 else set())
    assert set(ref.quant.cols.tolist()) == want     # the oracle's own decision at the edge
    _check_forward(L, wq, ws, tau, 32, f"threshold edge {case}")


@pytest.mark.parametrize("m,k,tau", [(2, 1000, 6.0), (2, 1000, 6.001), (40, 3000, 6.0), (300, 20000, 6.0),
                                     (300, 20000, 6.001), (1100, 3000, 6.0), (1100, 3000, 6.001)])
def test_threshold_edge_quant(m, k, tau):
    """int8_vectorwise_quant on its own: the two-row single-workgroup kernel,
    detect + quantize with a wavefront or a workgroup per row, and the
    single-read pair from 1024 rows."""
    L, _ = _edge_input(m, k, 1, seed=1)
    say(f"vectorwise_quant threshold edge m={m} k={k} tau={tau}")
    q, s, bm = i8.vectorwise_quant(dev(L.x), tau)
    torch.cuda.synchronize()
    ref = oracle.vectorwise_quant(L.x, tau)
    assert_equal(q, ref.q, "codes")
    assert_equal(s, ref.absmax, "absmax")
    assert_equal(bm.view(torch.int32), ref.bitmap.view(np.int32), "bitmap")


# ---- int32 accumulation at the largest k (k * 127^2 < 2^31) ------------------

def test_linear_matmul_int32_bound():
    k = i8.I8MP_MAX_K
    a = np.full((3, k), 127, np.int8)
    a[1] = -127
    a[2, 1::2] = -127
    b = np.full((2, k), 127, np.int8)
    b[1] = -127
    say(f"linear_matmul k={k} all +-127")
    c = i8.linear_matmul(dev(a), dev(b))
    torch.cuda.synchronize()
    ref = oracle.int8_linear_matmul(a, b)
    assert ref[0, 0] == 2147479576 and ref[1, 0] == -2147479576
    assert_equal(c, ref, "C at k = 133144")
    c1 = i8.linear_matmul(dev(a[:1]), dev(b[:1]))
    torch.cuda.synchronize()
    assert int(host(c1)[0, 0]) == 2147479576


def test_linear_matmul_int32_bound_tiles():
    """Random codes at the largest k through a prefill tile (ragged m and n)."""
    k = i8.I8MP_MAX_K
    rng = np.random.default_rng(87)
    a = rng.integers(-127, 128, (40, k), dtype=np.int16).astype(np.int8)
    a[0] = 127
    b = rng.integers(-127, 128, (70, k), dtype=np.int16).astype(np.int8)
    b[0] = 127
    say(f"linear_matmul 40 x 70 x {k}")
    c = i8.linear_matmul(dev(a), dev(b))
    torch.cuda.synchronize()
    ref = oracle.int8_linear_matmul(a, b)
    assert ref[0, 0] == 2147479576
    assert_equal(c, ref, "C")


@pytest.mark.parametrize("m", [1, 3, 300])
def test_linear_forward_largest_k(m):
    """The fused forward at k = 133144: x = 1 and w = 2^-10 everywhere give
    all-127 codes on both sides (C = (k - o) * 127^2 near 2^31), plus three
    outlier columns of 7.0 in the fp16 part."""
    k, n = i8.I8MP_MAX_K, 64
    x = np.ones((m, k), np.float16)
    x[:, [5, 70000, k - 1]] = np.float16(7.0)
    w = np.full((n, k), np.float16(2.0 ** -10))
    w[1::2, ::3] = np.float16(-(2.0 ** -10))
    wq, ws = oracle.quantize_weight(w)
    ref = oracle.linear_forward(x, wq, ws, None, TAU)
    assert ref.c[0, 0] == (k - 3) * 127 * 127
    say(f"linear_forward m={m} k={k}")
    wsp = i8.LinearWorkspace.create(m, n, k, 8, "cuda")
    out = i8.linear(dev(x), dev(wq), dev(ws), None, TAU, 8, wsp)
    torch.cuda.synchronize()
    _check_workspace(wsp, x, ref.quant, 8)
    assert_fp16_close(out, ref.out)


@pytest.mark.parametrize("m,k", [(64, 2048), (40, 300), (300, 20000), (1100, 512), (8, 300), (16, 13824)])
def test_quant_row_max_inside_outlier_columns(m, k):
    """Rows whose largest element below the threshold sits in an outlier column
    (large in another row): the row scale must come from the other columns.
    Row 5: max 5.5 in outlier column 3, next 4.0 elsewhere; row 6: 5.5 in the
    outlier column and 5.5 in an ordinary column (tie); row 7: every ordinary
    element 0 (zero scale)."""
    L = make_inputs(m, k, 1, seed=(88, m, k), with_weight=False)
    x = (L.x.astype(np.float32) * 0.5).astype(np.float16)
    x[0, 3] = np.float16(50.0)
    x[1, k - 2] = np.float16(-7.0)
    x[5] = np.clip(x[5], -3.5, 3.5)
    x[5, 3] = np.float16(5.5)
    x[5, 10] = np.float16(-4.0)
    x[6] = np.clip(x[6], -3.5, 3.5)
    x[6, 3] = np.float16(-5.5)
    x[6, k - 1] = np.float16(5.5)
    x[7] = 0
    x[7, 3] = np.float16(2.0)
    x[7, k - 2] = np.float16(1.0)
    ref = oracle.vectorwise_quant(x, TAU)
    assert ref.cols.tolist() == [3, k - 2]
    assert ref.absmax[5] == np.float32(4.0) and ref.absmax[6] == np.float32(5.5) and ref.absmax[7] == 0
    say(f"vectorwise_quant row max inside outlier columns m={m} k={k}")
    q, s, bm = i8.vectorwise_quant(dev(x), TAU)
    torch.cuda.synchronize()
    assert_equal(q, ref.q, "codes")
    assert_equal(s, ref.absmax, "absmax")
    assert_equal(bm.view(torch.int32), ref.bitmap.view(np.int32), "bitmap")
    wsp = i8.LinearWorkspace.create(m, 8, k, 1, "cuda")
    i8.linear_quantize(dev(x), wsp, TAU)
    torch.cuda.synchronize()
    _check_workspace(wsp, x, ref, 1)


def test_decode_gemm_repeats():
    """The decode GEMM half run three times on one quantized workspace gives the
    same output each time, and the oracle's (nothing in the workspace is
    consumed by a GEMM launch)."""
    m, k, n = 12, 13824, 900
    L = make_inputs(m, k, n, n_outlier=6, bias_std=0.01, seed=(91, m, k), outlier_row_frac=0.7)
    wq, ws = oracle.quantize_weight(L.w)
    ref = oracle.linear_forward(L.x, wq, ws, L.bias, TAU)
    say(f"decode GEMM repeated m={m} k={k} n={n}")
    xd = dev(L.x)
    wsp = i8.LinearWorkspace.create(m, n, k, 64, "cuda")
    i8.linear_quantize(xd, wsp, TAU)
    outs = []
    for _ in range(3):
        out = torch.empty((m, n), dtype=torch.float16, device="cuda")
        i8.linear_matmul_dequant(xd, wsp, dev(wq), dev(ws), dev(L.bias), out)
        outs.append(out)
    torch.cuda.synchronize()
    for out in outs:
        assert torch.equal(out, outs[0])
    assert_fp16_close(outs[0], ref.out)
