"""GPU parity of the backward pass (column-wise quantization, both gradients)
against the CPU oracle.

Bit-exact: column-wise codes and column absmax (also the zero padding of the
transposed codes), the row-wise codes of the gradient, every GEMM operand the
backward leaves in its workspace.  Tolerance (fp16 outputs; fp32 epilogue and
fp32 sums of the outlier columns): |gpu - oracle| <= 1e-3 + 1e-2 |oracle|.
"""

import numpy as np
import pytest
import torch

import int8_mixed_precision_vectorwise_amd as i8
import oracle
from gpu_util import assert_equal, assert_fp16_close, dev, host, say
from synth import draw_grad, layer_specs, make_inputs, make_layer

pytestmark = pytest.mark.gpu

TAU = 6.0

COLQ_CASES = [
    # rows, cols, lda_extra, ldqt_extra, zero columns
    (1, 1, 0, 0, ()),
    (3, 5, 0, 0, ()),
    (16, 8, 0, 0, (3,)),
    (511, 64, 0, 1, ()),
    (513, 65, 0, 15, (0, 64)),
    (1000, 4096, 0, 24, (7, 100, 4095)),
    (777, 130, 3, 5, (129,)),          # unaligned columns and rows: element loads, byte stores
    (2048, 96, 8, 0, (0, 5, 95)),
    (5000, 24, 0, 0, ()),              # ten row blocks
    (0, 10, 0, 16, ()),                # no rows: zero scales, zero codes
]


@pytest.mark.parametrize("case", COLQ_CASES, ids=lambda c: "r%d_c%d_la%d_lq%d_z%d" % (c[:4] + (len(c[4]),)))
def test_colwise_quant_bit_exact(case):
    rows, cols, lda_x, ldq_x, zero = case
    L = make_inputs(rows, cols, 1, n_outlier=min(2, cols), seed=(80, rows % 97, cols % 89), with_weight=False)
    a = L.x.copy()
    if rows > 3 and cols > 2:
        a[:, 1] = 0                   # a zero column
    buf = np.zeros((rows, cols + lda_x), np.float16)
    buf[:, :cols] = a
    t = dev(buf)[:, :cols] if lda_x else dev(a)
    ldqt = rows + ldq_x
    zi = dev(np.array(list(zero) + [-1, -1], np.int32)) if zero else None
    zc = dev(np.array([len(zero)], np.int32)) if zero else None
    say(f"colwise_quant rows={rows} cols={cols} lda+{lda_x} ldqt={ldqt} zero={zero}")
    qt, s = i8.colwise_quant(t, zi, zc, ldqt=ldqt)
    torch.cuda.synchronize()
    ref_q, ref_s = oracle.colwise_quant(a, zero)
    assert_equal(s, ref_s, "column absmax")
    want = np.zeros((cols, ldqt), np.int8)
    want[:, :rows] = ref_q
    assert_equal(qt, want, "transposed codes")


def test_colwise_quant_count_above_cap():
    # only the first min(count, cap) listed columns are zeroed
    a = make_inputs(300, 40, 1, seed=(81, 0, 0), with_weight=False).x
    zi = dev(np.array([2, 9, 30], np.int32))
    zc = dev(np.array([7], np.int32))
    say("colwise_quant count above cap")
    qt, s = i8.colwise_quant(dev(a), zi, zc)
    torch.cuda.synchronize()
    ref_q, ref_s = oracle.colwise_quant(a, [2, 9, 30])
    assert_equal(qt, ref_q, "codes")
    zc2 = dev(np.array([2], np.int32))
    qt2, _ = i8.colwise_quant(dev(a), zi, zc2)
    torch.cuda.synchronize()
    assert_equal(qt2, oracle.colwise_quant(a, [2, 9])[0], "codes, count 2")


BWD_CASES = [
    # m, n, k, planted outlier columns, cap
    (1, 1, 1, 0, 0),
    (5, 7, 9, 1, 8),
    (16, 16, 16, 0, 8),
    (64, 96, 128, 3, 16),
    (130, 250, 300, 4, 32),
    (200, 33, 513, 5, 256),
    (512, 1024, 768, 7, 256),
    (333, 257, 1000, 12, 8),      # more outlier columns than cap: those past it summed from g and x
    (300, 200, 500, 20, 0),       # no gathered columns at all
    (1100, 640, 2048, 20, 32),    # three row blocks of the column maxima
    (700, 3000, 96, 2, 16),       # long grad_x contraction, short grad_w one
]


def _run_forward(x, n, k, cap):
    """The forward's quantization of x (the backward reads the outlier list it leaves)."""
    ws = i8.LinearWorkspace.create(x.shape[0], n, k, cap, "cuda")
    i8.linear_quantize(x, ws, threshold=TAU)
    return ws


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "m%d_n%d_k%d_o%d_cap%d" % c)
def test_linear_backward(case):
    m, n, k, o, cap = case
    L = make_inputs(m, k, n, n_outlier=o, seed=(82, m % 101, n % 103))
    x, w = L.x, L.w
    g = draw_grad(m, n, seed=(82, m % 101, n % 103))
    cols = oracle.outlier_columns(x, TAU)
    used = cols   # every outlier column takes the fp16 path, whatever cap
    say(f"linear_backward m={m} n={n} k={k} outliers={len(cols)} cap={cap}")
    xt, gt_, wt_ = dev(x), dev(g), dev(w)
    fws = _run_forward(xt, n, k, cap)
    bws = i8.BackwardWorkspace.create(m, n, k, cap, "cuda")
    gx, gw = i8.linear_backward(gt_, xt, wt_, fws, workspace=bws)
    torch.cuda.synchronize()
    ref = oracle.linear_backward(g, x, w, used)
    assert_equal(bws.g_q(), ref.g_q, "row-wise codes of g")
    assert_equal(bws.g_s(), ref.g_s, "row absmax of g")
    assert_equal(bws.wt_q(), ref.wt_q, "column-wise codes of W")
    assert_equal(bws.wt_s(), ref.wt_s, "column absmax of W")
    assert_equal(bws.gt_q(), ref.gt_q, "column-wise codes of g")
    assert_equal(bws.gt_s(), ref.gt_s, "column absmax of g")
    assert_equal(bws.xt_q(), ref.xt_q, "column-wise codes of x, outlier columns zeroed")
    assert_equal(bws.xt_s(), ref.xt_s, "column absmax of x")
    assert_fp16_close(gx, ref.gx, "grad_x")
    assert_fp16_close(gw, ref.gw, "grad_w")
    # the zero padding of the transposed codes past m (the GEMM reads it)
    lay = bws.layout
    if lay.ld_m > m:
        pad = bws.buf[lay.xtq_offset:lay.xtq_offset + k * lay.ld_m].view(k, lay.ld_m)[:, m:]
        assert not host(pad).any()


def test_linear_backward_one_gradient_and_no_outliers():
    m, n, k = 96, 80, 144
    L = make_inputs(m, k, n, n_outlier=3, seed=(83, 0, 0))
    g = draw_grad(m, n, seed=(83, 0, 0))
    say("linear_backward grad_x only / grad_w only / no forward workspace")
    gx, gw = i8.linear_backward(dev(g), dev(L.x), dev(L.w), None, need_grad_w=False)
    assert gw is None
    gx2, gw2 = i8.linear_backward(dev(g), dev(L.x), None, None, need_grad_x=False)
    assert gx2 is None
    torch.cuda.synchronize()
    ref = oracle.linear_backward(g, L.x, L.w, [])
    assert_fp16_close(gx, ref.gx, "grad_x")
    assert_fp16_close(gw2, ref.gw, "grad_w (pure int8)")


def test_linear_backward_empty_contractions():
    say("linear_backward n = 0 and m = 0")
    x = dev(make_inputs(8, 32, 1, seed=(84, 0, 0), with_weight=False).x)
    gx, _ = i8.linear_backward(torch.zeros((8, 0), dtype=torch.float16, device="cuda"), x,
                               torch.zeros((0, 32), dtype=torch.float16, device="cuda"), None, need_grad_w=False)
    _, gw = i8.linear_backward(torch.zeros((0, 5), dtype=torch.float16, device="cuda"),
                               torch.zeros((0, 32), dtype=torch.float16, device="cuda"), None, None,
                               need_grad_x=False)
    torch.cuda.synchronize()
    assert gx.shape == (8, 32) and not host(gx).any()
    assert gw.shape == (5, 32) and not host(gw).any()


def _sampled_backward(g, x, w, cols, rows_x, rows_w):
    """Oracle gradients on sampled rows of grad_x and grad_w (full operands)."""
    g_q, g_s = oracle.quantize_weight(g[rows_x])
    wt_q, wt_s = oracle.colwise_quant(w)
    c = g_q.astype(np.float64) @ wt_q.astype(np.float64).T
    gx = (wt_s.astype(np.float64)[None, :] / 127.0) * (c * g_s.astype(np.float64)[:, None] / 127.0)
    gt_q, gt_s = oracle.colwise_quant(g[:, rows_w])
    xt_q, xt_s = oracle.colwise_quant(x, cols)
    c2 = gt_q.astype(np.float64) @ xt_q.astype(np.float64).T
    gw = (xt_s.astype(np.float64)[None, :] / 127.0) * (c2 * gt_s.astype(np.float64)[:, None] / 127.0)
    if len(cols):
        gw[:, cols] += g[:, rows_w].astype(np.float64).T @ x[:, cols].astype(np.float64)
    return gx, gw


@pytest.mark.parametrize("layer", ["q", "gate", "down"])
def test_linear_backward_llama7b_full_size(layer):
    spec = next(s for s in layer_specs("llama7b_prefill_m2048") if s.name == layer)
    Lr = make_layer(spec)
    m, n, k = spec.m, spec.n, spec.k
    g = draw_grad(m, n, seed=(spec.config_id, spec.layer_id, spec.variant_id))
    cap = 256
    cols = oracle.outlier_columns(Lr.x, TAU)
    say(f"linear_backward full size 7B {layer} m={m} n={n} k={k} outliers={len(cols)}")
    xt = dev(Lr.x)
    fws = _run_forward(xt, n, k, cap)
    gx, gw = i8.linear_backward(dev(g), xt, dev(Lr.w), fws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(85)
    rows_x = np.sort(rng.choice(m, 24, replace=False))
    rows_w = np.sort(rng.choice(n, 24, replace=False))
    ref_x, ref_w = _sampled_backward(g, Lr.x, Lr.w, cols, rows_x, rows_w)
    assert_fp16_close(gx[torch.from_numpy(rows_x).cuda()], ref_x, "grad_x rows")
    assert_fp16_close(gw[torch.from_numpy(rows_w).cuda()], ref_w, "grad_w rows")


def test_backward_graph_replays_match_eager():
    # the backward is deterministic (fixed-order sums, no atomics): every
    # replay of a captured call equals the eager call bit for bit, whatever the
    # workspace held before
    m, n, k, cap = 300, 520, 640, 32
    L = make_inputs(m, k, n, n_outlier=6, seed=(86, 0, 0))
    g = draw_grad(m, n, seed=(86, 0, 0))
    xt, gt_, wt_ = dev(L.x), dev(g), dev(L.w)
    say("linear_backward graph capture")
    fws = _run_forward(xt, n, k, cap)
    bws = i8.BackwardWorkspace.create(m, n, k, cap, "cuda")
    ex, ew = i8.linear_backward(gt_, xt, wt_, fws, workspace=bws)
    ex, ew = ex.clone(), ew.clone()
    gx = torch.empty_like(ex)
    gw = torch.empty_like(ew)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(graph, stream=st):
            i8.linear_backward(gt_, xt, wt_, fws, True, True, bws, gx, gw)
    torch.cuda.synchronize()
    for rep in range(3):
        gx.fill_(7.0)
        gw.fill_(-3.0)
        bws.buf.fill_(0x5a)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(gx.view(torch.int16), ex.view(torch.int16)), rep
        assert torch.equal(gw.view(torch.int16), ew.view(torch.int16)), rep
    ref = oracle.linear_backward(g, L.x, L.w, oracle.outlier_columns(L.x, TAU))
    assert_fp16_close(gw, ref.gw, "grad_w after replays")


@pytest.mark.parametrize("tau", [6.0, 6.001])
def test_linear_backward_threshold_edge(tau):
    """The backward takes the forward's outlier list at the threshold's edge:
    a column whose only large element is exactly 6.0 is an outlier at tau = 6
    (zeroed in CAt, fp16 column of grad_w) and not at tau = 6.001; one at the
    largest fp16 below 6 never is."""
    m, n, k = 200, 96, 300
    L = make_inputs(m, k, n, seed=(87, 0, 0))
    L.x[17, 40] = np.float16(6.0)
    L.x[3, 41] = np.float16(-6.0)
    L.x[150, 99] = np.float16(5.99609375)
    L.x[151, 200] = np.float16(6.00390625)
    g = draw_grad(m, n, seed=(87, 0, 0))
    cols = oracle.outlier_columns(L.x, tau)
    assert cols.tolist() == ([40, 41, 200] if tau == 6.0 else [200])
    say(f"linear_backward threshold edge tau={tau}")
    xt = dev(L.x)
    fws = i8.LinearWorkspace.create(m, n, k, 32, "cuda")
    i8.linear_quantize(xt, fws, threshold=tau)
    bws = i8.BackwardWorkspace.create(m, n, k, 32, "cuda")
    gx, gw = i8.linear_backward(dev(g), xt, dev(L.w), fws, workspace=bws)
    torch.cuda.synchronize()
    ref = oracle.linear_backward(g, L.x, L.w, cols)
    assert_equal(bws.xt_q(), ref.xt_q, "column-wise codes of x, outlier columns zeroed")
    assert_fp16_close(gx, ref.gx, "grad_x")
    assert_fp16_close(gw, ref.gw, "grad_w")
