"""Parity at the workloads' full sizes, through the same entry point and launch
configuration the benchmark times (i8mp_linear_forward, cap 256).

The outlier set, row absmax, codes and weight codes are compared in full;
the int32 accumulators' consequence (the fp16 output) is compared on sampled
rows that the oracle computes one by one, with the outlier set taken from
the full input.
"""

import numpy as np
import pytest
import torch

import int8_mixed_precision_vectorwise_amd as i8
import oracle
from gpu_util import assert_equal, assert_fp16_close, dev, say
from synth import layer_specs, make_layer

pytestmark = pytest.mark.gpu

CAP = 256


def _sample_rows(m, count=48, seed=0):
    if m <= count:
        return np.arange(m)
    rng = np.random.default_rng(seed)
    rows = set([0, m - 1]) | set(rng.choice(m, count - 2, replace=False).tolist())
    return np.array(sorted(rows))


def _run_layer(spec):
    say(f"full-size {spec.config_id}/{spec.name} m={spec.m} k={spec.k} n={spec.n}")
    L = make_layer(spec)
    xd, wd = dev(L.x), dev(L.w)
    wq_g, ws_g = i8.quantize_weight(wd)
    del wd
    wsp = i8.LinearWorkspace.create(spec.m, spec.n, spec.k, CAP, "cuda")
    bias = dev(L.bias) if L.bias is not None else None
    out = i8.linear(xd, wq_g, ws_g, bias, spec.tau, CAP, wsp)
    torch.cuda.synchronize()

    wq, ws = oracle.quantize_weight(L.w)
    assert_equal(wq_g, wq, "weight codes")
    assert_equal(ws_g, ws, "weight absmax")
    qr = oracle.vectorwise_quant(L.x, spec.tau)
    assert qr.cols.tolist() == L.planted_cols.tolist()
    assert int(wsp.count().item()) == qr.cols.size
    assert_equal(wsp.bitmap().view(torch.int32), qr.bitmap.view(np.int32), "bitmap")
    assert_equal(wsp.absmax(), qr.absmax, "absmax")
    assert_equal(wsp.codes(), qr.q, "codes")

    rows = _sample_rows(spec.m, seed=spec.layer_id)
    xs = L.x[rows]
    s = oracle.row_absmax(xs, qr.cols)
    q = oracle.quantize_rows(xs, s, qr.cols)
    c = oracle.int8_linear_matmul(q, wq)
    p = oracle.outlier_matmul(xs, qr.cols, wq)
    ref = oracle.mm_dequant(c, s, ws, L.bias, p)
    assert_fp16_close(out[torch.from_numpy(rows).cuda()], ref, f"{spec.name} sampled rows")


def _ids(specs):
    return [f"{s.config_id}-{s.name}" for s in specs]


OPT = layer_specs("opt350m_mlp_pair_m512")
P7 = [s for s in layer_specs("llama7b_prefill_m2048") if s.name in ("q", "gate", "down")]
D13 = [s for s in layer_specs("llama13b_decode") if s.name.endswith("_o8") or s.name.endswith("_o0")]
P65 = layer_specs("llama65b_prefill_m4096")
TINY = layer_specs("tiny")


@pytest.mark.parametrize("spec", TINY + OPT, ids=_ids(TINY + OPT))
def test_small_workloads(spec):
    _run_layer(spec)


@pytest.mark.parametrize("spec", P7, ids=_ids(P7))
def test_llama7b_prefill(spec):
    _run_layer(spec)


@pytest.mark.parametrize("spec", D13, ids=_ids(D13))
def test_llama13b_decode(spec):
    _run_layer(spec)


@pytest.mark.parametrize("spec", P65, ids=_ids(P65))
def test_llama65b_prefill(spec):
    _run_layer(spec)


def test_vectorwise_dequant_65b_weight():
    """The int8 dequantize op on the 65B up-projection's weight (22016 x 8192
    codes, quantized on the GPU from a seeded fp16 weight): sampled rows
    against the oracle, fp16 output (one more rounding than fp32: half an fp16
    ulp)."""
    spec = [s for s in layer_specs("llama65b_prefill_m4096") if s.name == "up"][0]
    say(f"full-size dequant {spec.n}x{spec.k}")
    L = make_layer(spec, m=1)
    wq, ws = i8.quantize_weight(dev(L.w))
    out = i8.vectorwise_dequant(wq, ws, torch.float16)
    torch.cuda.synchronize()
    rows = _sample_rows(spec.n, seed=7)
    ridx = torch.from_numpy(rows).cuda()
    got = out[ridx].cpu().numpy().astype(np.float64)
    ref = oracle.vectorwise_dequant(wq[ridx].cpu().numpy(), ws[ridx].cpu().numpy())
    assert np.all(np.abs(got - ref) <= 2.0 ** -11 * np.abs(ref) * (1 + 2.0 ** -10) + 2.0 ** -24)
    # the weight codes themselves are the oracle's
    wq_ref, ws_ref = oracle.quantize_weight(L.w[rows])
    assert_equal(wq[ridx], wq_ref, "weight codes")


STRESS = layer_specs("llama65b_prefill_m4096_stress")


@pytest.mark.parametrize("spec,cap", [(STRESS[0], CAP), (STRESS[0], 8192), (STRESS[1], CAP)],
                         ids=["up-cap256", "up-capk", "down-cap256"])
def test_llama65b_stress_untruncated(spec, cap):
    """The 65B layers on their untruncated Student-t input: nearly every column
    is an outlier, so the linear is almost all fp16.  With cap 256 all but 256
    outlier columns read x through the index list; with cap = k all come from
    the gathered copy.  Codes, absmax, bitmap and the whole index list in full,
    the output on sampled rows (outlier set from the full input)."""
    say(f"stress {spec.name} m={spec.m} k={spec.k} n={spec.n} cap={cap}")
    L = make_layer(spec)
    qr = oracle.vectorwise_quant(L.x, spec.tau)
    assert qr.cols.size > 0.99 * spec.k
    xd = dev(L.x)
    wq_g, ws_g = i8.quantize_weight(dev(L.w))
    wsp = i8.LinearWorkspace.create(spec.m, spec.n, spec.k, cap, "cuda")
    out = i8.linear(xd, wq_g, ws_g, None, spec.tau, cap, wsp)
    torch.cuda.synchronize()
    assert int(wsp.count().item()) == qr.cols.size
    assert_equal(wsp.bitmap().view(torch.int32), qr.bitmap.view(np.int32), "bitmap")
    assert_equal(wsp.absmax(), qr.absmax, "absmax")
    assert_equal(wsp.codes(), qr.q, "codes")
    ridx, _, _ = oracle.outlier_extract(L.x, qr.cols, int(wsp.layout.idx_len))
    assert_equal(wsp.idx(), ridx, "idx")
    wq = wq_g.cpu().numpy()
    ws = ws_g.cpu().numpy()
    rows = _sample_rows(spec.m, count=24, seed=spec.layer_id + 11)
    xs = L.x[rows]
    s = oracle.row_absmax(xs, qr.cols)
    q = oracle.quantize_rows(xs, s, qr.cols)
    c = oracle.int8_linear_matmul(q, wq)
    p = oracle.outlier_matmul(xs, qr.cols, wq)
    ref = oracle.mm_dequant(c, s, ws, None, p)
    assert_fp16_close(out[torch.from_numpy(rows).cuda()], ref, f"{spec.name} stress sampled rows")
    wq_ref, ws_ref = oracle.quantize_weight(L.w[:64])
    assert_equal(wq_g[:64], wq_ref, "weight codes (first rows)")
