"""Host logic of the benchmark's counter summaries (no GPU): the dispatches of a
``--mode gemm`` run are grouped per layer at the fill kernel that follows each
layer's launches, so that a launch made of a main and a tail kernel counts once."""

import csv
import os

import bench

GEMM_MAIN = "void i8mp::gemm_pp_kernel<true>(i8mp::GemmArgs)"
GEMM_TAIL = "void i8mp::gemm_dtl_kernel<256, 128, 128, 4, true, 1, 2>(i8mp::GemmArgs)"
QUANT = "void i8mp::quant1_kernel<true, true, 16>(i8mp::QuantArgs, unsigned int*)"
MARK = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<int>, std::array<char*, 1ul> >"


def _write(tmp_path, folder, rows):
    d = tmp_path / folder / "host" / "123"
    os.makedirs(d)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_per_layer_groups_split_launches(tmp_path):
    launches = 3
    rows, d = [], 0

    def disp(name, value, counter="C"):
        nonlocal d
        d += 1
        # two rows per dispatch (one per XCD group, say): summed
        rows.append({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value / 2})
        rows.append({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value / 2})
        rows.append({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": "other", "Counter_Value": 1e9})

    disp(MARK, 5.0)              # a fill before the first layer: no group
    for i in range(launches):    # layer 0: main + tail per launch, one quantize
        if i == 0:
            disp(QUANT, 1e6)
        disp(GEMM_MAIN, 100.0)
        disp(GEMM_TAIL, 20.0)
    disp(MARK, 5.0)
    for i in range(launches):    # layer 1: one kernel per launch
        disp(GEMM_MAIN, 70.0 + i)
    disp(MARK, 5.0)
    _write(tmp_path, "gemm_x", rows)
    got = bench._per_layer(str(tmp_path), "gemm_x", "C", launches)
    assert got == [120.0, 71.0]


def test_per_layer_quant_kernels(tmp_path):
    """The quantize half's passes (zero, single read, finishing pass) count as one call."""
    rows, d = [], 0

    def disp(name, value):
        nonlocal d
        d += 1
        rows.append({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": "C", "Counter_Value": value})

    disp("void i8mp::quant_kernel<true, false, 4>(i8mp::QuantArgs)", 99.0)   # set-up: not counted
    disp(MARK, 0.0)
    for i in range(2):
        disp("i8mp::zero_words_kernel(unsigned int*, long)", 1.0)
        disp(QUANT, 10.0)
        disp("void i8mp::quant2_kernel<true>(i8mp::QuantArgs, unsigned int const*)", 3.0)
    disp(MARK, 0.0)
    for i in range(2):
        disp("void i8mp::cs1_kernel<true>(i8mp::QuantArgs, unsigned int*, float*)", 2.0)
        disp("void i8mp::cs2_kernel<true>(i8mp::QuantArgs, unsigned int const*, float const*, long)", 4.0)
    disp(MARK, 0.0)
    _write(tmp_path, "quant_x", rows)
    assert bench._per_layer(str(tmp_path), "quant_x", "C", 2, bench.QUANT_KERNELS) == [14.0, 6.0]
