"""GPU parity of the blockwise 4-bit (FP4 E2M1) weight path against the CPU oracle.

Bit-exact: codes (unpacked), block absmax, double-quantized scales, the
dequantized weights (fp32, and fp16 rounded once from them).  Tolerance for
the 4-bit linear (fp32 sums on the GPU, float64 in the oracle):
|gpu - oracle| <= 1e-3 + 1e-2 |oracle|.
"""

import numpy as np
import pytest
import torch

import int8_mixed_precision_vectorwise_amd as i8
from gpu_util import assert_equal, assert_fp16_close, dev, host, say
from oracle import fp4
from synth import draw_weight, make_inputs

pytestmark = pytest.mark.gpu


def _weight(n, k, seed, ld_extra=0):
    w = draw_weight(n, k, seed=(90, seed, 0))
    if n > 2:
        w[1, :64] = 0                      # a zero block
        w[2, 5] = np.float16(-0.0)
    if ld_extra:
        buf = np.zeros((n, k + ld_extra), np.float16)
        buf[:, :k] = w
        return w, dev(buf)[:, :k]
    return w, dev(w)


QUANT_CASES = [(1, 64, 0), (3, 128, 0), (17, 640, 0), (256, 4096, 0), (1000, 5120, 0), (33, 192, 3), (7, 64, 8)]


@pytest.mark.parametrize("case", QUANT_CASES, ids=lambda c: "n%d_k%d_ld%d" % c)
def test_fp4_quantize_bit_exact(case):
    n, k, ldx = case
    w, wt = _weight(n, k, n % 50, ldx)
    say(f"fp4_quantize n={n} k={k} ld+{ldx}")
    fw = i8.fp4_quantize(wt)
    torch.cuda.synchronize()
    ref_c, ref_a = fp4.fp4_quantize(w)
    assert_equal(fw.absmax, ref_a, "block absmax")
    got = fp4.unpack_nibbles(host(fw.codes)[:, : k // 2])
    assert np.array_equal(got, ref_c), f"{int((got != ref_c).sum())} codes differ"
    # dequantize (fp32 bit-exact, fp16 rounded once from it)
    d32 = i8.fp4_dequantize(fw, torch.float32)
    d16 = i8.fp4_dequantize(fw, torch.float16)
    torch.cuda.synchronize()
    ref_d = fp4.fp4_dequantize(ref_c, ref_a)
    assert_equal(d32, ref_d, "dequantized fp32")
    assert_equal(d16, ref_d.astype(np.float16), "dequantized fp16")


@pytest.mark.parametrize("nb", [1, 255, 256, 257, 1000, 13824 * 5120 // 64])  # the last: a 13B up-projection
def test_fp4_double_quant_bit_exact(nb):
    rng = np.random.default_rng([91, nb])
    a = rng.uniform(0.0, 0.3, size=nb).astype(np.float32)
    a[rng.integers(nb)] = 0.0
    say(f"fp4_double_quant nb={nb}")
    fw = i8.Fp4Weight(torch.zeros((1, 32), dtype=torch.uint8, device="cuda"), 64, dev(a))
    dq = i8.fp4_double_quant(fw)
    torch.cuda.synchronize()
    ref_c8, ref_s2 = fp4.double_quant(a)
    assert_equal(dq.c8, ref_c8, "c8")
    assert_equal(dq.s2, ref_s2, "s2")


def test_fp4_dequantize_double_quantized():
    n, k = 300, 1024
    w, wt = _weight(n, k, 3)
    say("fp4_dequantize with double-quantized scales")
    fw = i8.fp4_quantize(wt, double_quant=True)
    d32 = i8.fp4_dequantize(fw, torch.float32)
    torch.cuda.synchronize()
    ref_c, ref_a = fp4.fp4_quantize(w)
    c8, s2 = fp4.double_quant(ref_a)
    assert_equal(fw.c8, c8, "c8")
    assert_equal(d32, fp4.fp4_dequantize(ref_c, fp4.double_dequant(c8, s2)), "dequantized fp32")


LINEAR_CASES = [
    # m, n, k, double quant, bias
    (1, 1, 64, False, False),
    (1, 5, 128, False, True),
    (2, 7, 192, True, False),
    (3, 13, 640, False, True),
    (4, 64, 4096, True, True),
    (5, 31, 2048, False, False),    # two launches: rows 0-3, then row 4
    (9, 100, 1024, True, True),
    (4, 50, 13824, False, False),   # more than 256 chunks of 32 weights per row: two segments
    (3, 37, 13824, True, True),     # two segments, the last group of four weight rows partial
    (2, 9, 9216, False, True),      # two segments at m = 2, the last group partial
    (1, 1000, 5120, True, False),
    # one row of x: x staged in LDS, 2 to 8 code chunks per lane (the fewest that cover a
    # row: 2 to 8 here, the last slot partly past the row; the first 1 to 3 slots' x held in
    # registers), rows past the grid's waves
    (1, 77, 13824, True, True),
    (1, 4100, 4096, False, True),
    (1, 50, 4160, False, False),
    (1, 300, 7168, True, True),
    (1, 37, 10240, False, True),
    (1, 129, 12224, True, False),
    (1, 9, 16384, False, False),
    (1, 5, 16448, True, False),     # past 16384: x from L2
    # two to four rows of x: x staged in LDS, the workgroups' shares of the weight rows
    (4, 9001, 1024, True, True),    # two tiles of 32 rows per workgroup, the last share partial
    (3, 4099, 13824, False, True),  # two segments of 256 chunks per row
    (2, 4098, 8192, True, False),   # one full segment
    # two to four rows of x on the matrix cores up to k = 14336 and n = 16384; past them
    # the four-row LDS-x kernel
    (4, 33, 16384, True, True),
    (2, 5000, 15360, False, False),
    (2, 16500, 1024, False, True),
    (3, 300, 64, True, False),      # one block per row: waves past the last block
    # past 16384 (x does not fit LDS): the kernel that reads x from L2 for 4 or 8 weight rows
    (4, 30, 16448, False, True),
    (3, 9, 16448, True, True),
    (2, 7, 16448, True, False),
]


@pytest.mark.parametrize("case", LINEAR_CASES, ids=lambda c: "m%d_n%d_k%d_dq%d_b%d" % c)
def test_fp4_linear(case):
    m, n, k, dq, with_bias = case
    L = make_inputs(m, k, n, seed=(92, n % 97, k % 89), bias_std=0.05 if with_bias else None)
    say(f"fp4_linear m={m} n={n} k={k} dq={dq} bias={with_bias}")
    fw = i8.fp4_quantize(dev(L.w), double_quant=dq)
    b = dev(L.bias) if with_bias else None
    out = i8.fp4_linear(dev(L.x), fw, b)
    torch.cuda.synchronize()
    ref_c, ref_a = fp4.fp4_quantize(L.w)
    scales = ref_a
    if dq:
        c8, s2 = fp4.double_quant(ref_a)
        scales = fp4.double_dequant(c8, s2)
    _, y = fp4.fp4_linear(L.x, ref_c, scales, L.bias)
    assert_fp16_close(out, y, "fp4 linear")


@pytest.mark.parametrize("layer", [("up", 5120, 13824), ("down", 13824, 5120)])
@pytest.mark.parametrize("m", [1, 4])
def test_fp4_linear_llama13b_decode_full_size(layer, m):
    name, k, n = layer
    L = make_inputs(m, k, n, seed=(93, m, k % 97))
    say(f"fp4_linear 13B {name} m={m} k={k} n={n}")
    fw = i8.fp4_quantize(dev(L.w), double_quant=True)
    out = i8.fp4_linear(dev(L.x), fw)
    torch.cuda.synchronize()
    rng = np.random.default_rng(94)
    rows = np.sort(rng.choice(n, 64, replace=False))
    ref_c, ref_a = fp4.fp4_quantize(L.w[rows])
    # the double quantization groups run over all n rows: take the scales from the full weight
    _, full_a = fp4.fp4_quantize(L.w)
    c8, s2 = fp4.double_quant(full_a)
    sc = fp4.double_dequant(c8, s2).reshape(n, k // 64)[rows]
    _, y = fp4.fp4_linear(L.x, ref_c, sc)
    assert_fp16_close(out[:, torch.from_numpy(rows).cuda()], y, "fp4 linear rows")


@pytest.mark.parametrize("m", [1, 3])
def test_fp4_linear_graph_replays_match_eager(m):
    n, k = 200, 1024
    L = make_inputs(m, k, n, seed=(95, m, 0), bias_std=0.05)
    say(f"fp4_linear graph capture m={m}")
    fw = i8.fp4_quantize(dev(L.w), double_quant=True)
    x, b = dev(L.x), dev(L.bias)
    eager = i8.fp4_linear(x, fw, b).clone()
    out = torch.empty_like(eager)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(graph, stream=st):
            i8.fp4_linear(x, fw, b, out)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), rep
