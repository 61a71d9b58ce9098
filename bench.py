#!/usr/bin/env python3
"""Throughput of the int8 mixed-precision linear (LLM.int8()) on one MI355X.

A step is one pass of the whole hot path (outlier detection + calibration +
quantization, extraction, int8 MFMA GEMM with the fused dequant / outlier /
bias epilogue) over every layer of the workload, each layer on its own seeded
synthetic input.  Inputs and weights are resident in HBM before timing starts;
weight quantization (offline in the method) is done once, untimed.  Inputs,
weights, workspaces and outputs are rotated over enough copies that the
working set exceeds the last-level caches.

Prints ONE JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "int8 linear TOPS & % int8-MFMA peak (prefill); GB/s & % HBM peak (decode)"
PEAK_INT8_OPS = 5.0e15     # MI355X dense int8 MFMA
PEAK_HBM = 8.0e12          # MI355X HBM3E bytes/s
DEFAULT_WORKLOAD = "llama65b_prefill_m4096"
# sources of the GEMM-side kernels (prefill tiles, decode kernels, shared helpers)
GEMM_SRCS = [os.path.join(ROOT, "int8_mixed_precision_vectorwise_amd", "csrc", f)
             for f in ("gemm.hip", "decode.hip", "common.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic.json")
FP4_SRCS = [os.path.join(ROOT, "int8_mixed_precision_vectorwise_amd", "csrc", f)
            for f in ("fp4.hip", "fp4.h", "quant_util.h", "common.h")]
FP4_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fp4_traffic.json")
GEMM_KERNELS = ("i8mp::gemm", "i8mp::gemv")  # kernel-name parts of the fused GEMM launches
# kernel-name parts of the quantize half (every launch it makes)
QUANT_KERNELS = ("i8mp::quant", "i8mp::detect", "i8mp::zero_words", "i8mp::cs1", "i8mp::cs2")
QUANT_SRCS = [os.path.join(ROOT, "int8_mixed_precision_vectorwise_amd", "csrc", f)
              for f in ("quant.hip", "quant_util.h", "common.h")]
QUANT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "quant_traffic.json")
COPY_MB = 256              # calibration copy: 256 MiB read + 256 MiB written


def log(msg: str) -> None:
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def workload_specs(name: str):
    from synth import layer_specs
    if name.startswith("llama13b_decode_m"):
        m = int(name.rsplit("_m", 1)[1])
        specs = [s for s in layer_specs("llama13b_decode") if s.name.endswith(f"_m{m}_o8")]
        if not specs:
            raise SystemExit(f"unknown decode batch in {name}")
        return specs, "decode"
    specs = layer_specs(name)
    kind = "prefill"
    return specs, kind


def alg_bytes(s) -> int:
    """Bytes the method itself must move for one layer: x, w_q, w_absmax, out (+ bias)."""
    b = 2 * s.m * s.k + s.n * s.k + 4 * s.n + 2 * s.m * s.n
    if s.bias_std is not None:
        b += 2 * s.n
    return b


def gemm_alg_bytes(s) -> int:
    """Bytes of the fused GEMM kernel alone: codes, w_q, both absmax vectors, out (+ bias)."""
    b = s.m * s.k + s.n * s.k + 4 * (s.m + s.n) + 2 * s.m * s.n
    if s.bias_std is not None:
        b += 2 * s.n
    return b


def quant_alg_bytes(s) -> int:
    """Bytes of the quantize half alone: x read, codes and row absmax written."""
    return 2 * s.m * s.k + s.m * s.k + 4 * s.m


def _code_only(text: str) -> str:
    """The source without comments and blank lines: what a compiler sees."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).strip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def fp4_src_sha() -> str:
    h = hashlib.sha256()
    for f in FP4_SRCS:
        h.update(_code_only(open(f).read()).encode())
    return h.hexdigest()[:16]


def quant_src_sha() -> str:
    h = hashlib.sha256()
    for f in QUANT_SRCS:
        h.update(_code_only(open(f).read()).encode())
    return h.hexdigest()[:16]


def src_sha() -> str:
    """Hash of the GEMM-side kernel sources' code (comments and blank lines
    ignored), which the stored traffic counters must match."""
    h = hashlib.sha256()
    for f in GEMM_SRCS:
        h.update(_code_only(open(f).read()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("gemm_source_sha") != src_sha():
        return None
    return d.get("per_launch_bytes", {}).get(workload)


def cpu_baseline(specs, kind: str, budget_s: float):
    """The oracle as it stands, on a bounded sample of the same workload."""
    import oracle  # only this leg of the benchmark touches the oracle
    from synth import make_layer
    try:
        from threadpoolctl import threadpool_info
        threads = sum(p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas")
    except Exception:  # pragma: no cover
        threads = 1
    threads = max(threads, 1)
    rows_cap = 256 if kind == "prefill" else None
    prepared = []
    for s in specs:
        m = s.m if rows_cap is None else min(s.m, rows_cap)
        L = make_layer(s, m=m)
        wq, ws = oracle.quantize_weight(L.w)  # offline weight quantization: untimed
        prepared.append((s, m, L, wq, ws))
    done_units = 0.0
    reps = 0
    t0 = time.perf_counter()
    while True:
        for s, m, L, wq, ws in prepared:
            oracle.linear_forward(L.x, wq, ws, L.bias, s.tau)
            if kind == "prefill":
                done_units += 2.0 * m * s.n * s.k
            else:
                done_units += alg_bytes(s)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    if kind == "prefill":
        value, unit = done_units / el / 1e12, "TOPS"
        rows = ", ".join(f"{s.name}: {m} of {s.m} rows" for s, m, *_ in prepared)
        sample = f"{reps} passes over the workload's layers ({rows}; outlier set from the sampled rows)"
    else:
        value, unit = done_units / el / 1e9, "GB/s"
        sample = f"{reps} passes over the workload's layers (full size)"
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle", "sample": sample,
            "seconds": round(el, 2)}


def capture_gemm_graphs(torch, i8, sets, specs, copies):
    """One graph per layer: that layer's fused GEMM over every rotation copy."""
    for c in range(copies):
        for s, xc, wqc, wac, b, ws, out in sets[c]:
            i8.linear_quantize(xc, ws, s.tau)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(st):
        for li in range(len(specs)):
            for c in range(copies):  # eager warm-up of this layer's launches
                _, xc, wqc, wac, b, ws, out = sets[c][li]
                i8.linear_matmul_dequant(xc, ws, wqc, wac, b, out)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=st):
                for c in range(copies):
                    _, xc, wqc, wac, b, ws, out = sets[c][li]
                    i8.linear_matmul_dequant(xc, ws, wqc, wac, b, out)
            graphs.append(g)
    torch.cuda.synchronize()
    return graphs, st


def time_gemm_launches(torch, i8, sets, specs, copies, launches):
    """Average duration of one fused-GEMM launch per layer: HIP events on the
    replay stream around back-to-back graph replays of that layer's launches
    (no host work between launches)."""
    graphs, st = capture_gemm_graphs(torch, i8, sets, specs, copies)
    out = {}
    reps = max(1, launches // copies)
    for li, s in enumerate(specs):
        g = graphs[li]
        with torch.cuda.stream(st):
            g.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(reps):
                g.replay()
            e1.record(st)
        torch.cuda.synchronize()
        out[s.name] = e0.elapsed_time(e1) * 1e3 / (reps * copies)
    return out


# rocprofv3 --pmc passes behind the traffic and MFMA figures (one pass each; a
# pass holds at most 4 TCC and 8 SQ counters)
RD_COUNTERS = ("TCC_EA0_RDREQ_32B", "TCC_EA0_RDREQ_64B", "TCC_EA0_RDREQ_128B", "TCC_EA0_RDREQ")
WR_COUNTERS = ("TCC_EA0_WRREQ_64B", "TCC_EA0_WRREQ")
MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_I8", "GRBM_GUI_ACTIVE",
                 "SQ_WAVES", "SQ_CYCLES")
MFMA_FILE = os.path.join(ROOT, "profiles", "gemm_mfma.json")
N_CUS = 256


def _per_dispatch(directory: str, folder: str, counter: str, name_part: tuple):
    """Counter value per dispatch (summed over the rows rocprofv3 writes for it) of
    the kernels whose name contains one of name_part, in dispatch order."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(directory, folder, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and any(p in r["Kernel_Name"] for p in name_part):
                d = int(r["Dispatch_Id"])
                vals[d] = vals.get(d, 0.0) + float(r["Counter_Value"])
    return [vals[d] for d in sorted(vals)]


LAYER_MARK = "FillFunctor"   # the kernel --mode gemm runs after each layer's launches


def _per_layer(directory: str, folder: str, counter: str, launches: int, kernels=GEMM_KERNELS):
    """Counter value per launch of each layer, from a --mode gemm (or quant)
    run: the dispatches of `kernels` (several per call: a GEMM's main and tail
    launches, the quantizer's passes) between consecutive layer marks, summed
    and divided by the launches.  Dispatches before the first mark (the
    set-up's weight quantization) are not counted."""
    import csv
    import glob
    vals, names = {}, {}
    for f in glob.glob(os.path.join(directory, folder, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            names[d] = r["Kernel_Name"]
            vals[d] = vals.get(d, 0.0) + float(r["Counter_Value"])
    layers, cur, n, started = [], 0.0, 0, False
    for d in sorted(vals):
        if LAYER_MARK in names[d]:
            if n:
                layers.append(cur / launches)
            cur, n, started = 0.0, 0, True
        elif started and any(p in names[d] for p in kernels):
            cur += vals[d]
            n += 1
    return layers


def _read_bytes(directory, folder, name_part):
    """L2 -> fabric read bytes per dispatch: 32, 64 and 128-byte requests by size."""
    n32, n64, n128, nall = (_per_dispatch(directory, folder, c, name_part) for c in RD_COUNTERS)
    return [32 * a + 64 * b + 128 * c for a, b, c in zip(n32, n64, n128)], \
        [t - a - b - c for a, b, c, t in zip(n32, n64, n128, nall)]


def _write_bytes(directory, folder, name_part):
    """L2 -> fabric write bytes per dispatch: 64-byte requests and 32-byte ones."""
    n64, nall = (_per_dispatch(directory, folder, c, name_part) for c in WR_COUNTERS)
    return [64 * a + 32 * (t - a) for a, t in zip(n64, nall)]


def traffic_summary(directory: str, workload: str, launches: int) -> int:
    """Per-launch HBM (L2 -> fabric) bytes of the fused GEMM from rocprofv3 --pmc runs.

    ``directory`` holds four rocprofv3 output folders: gemm_rd, gemm_wr (``bench.py
    --mode gemm``) and copy_rd, copy_wr (``bench.py --mode copy``), with RD_COUNTERS
    and WR_COUNTERS.  Read bytes are the request counts by size times their sizes;
    the copy kernel, whose true bytes are known, checks the counting (its scale is
    reported and applied)."""
    specs, _ = workload_specs(workload)
    copy_bytes = COPY_MB * 2**20
    cr, c_other = _read_bytes(directory, "copy_rd", ("elementwise",))
    cw = _write_bytes(directory, "copy_wr", ("elementwise",))
    if not cr or not cw:
        raise SystemExit("no copy-kernel counters found")
    f_scale = copy_bytes / (sum(cr) / len(cr))
    w_scale = copy_bytes / (sum(cw) / len(cw))
    n32, n64, n128, nall = (_per_layer(directory, "gemm_rd", c, launches) for c in RD_COUNTERS)
    w64, wall = (_per_layer(directory, "gemm_wr", c, launches) for c in WR_COUNTERS)
    if min(len(n32), len(w64)) < len(specs):
        raise SystemExit(f"expected GEMM launches of {len(specs)} layers, got {len(n32)} / {len(w64)}")
    g_other = [t - a - b - c for a, b, c, t in zip(n32, n64, n128, nall)]
    layers = {}
    tot = 0.0
    for li, s in enumerate(specs):
        fb = (32 * n32[li] + 64 * n64[li] + 128 * n128[li]) * f_scale
        wb = (64 * w64[li] + 32 * (wall[li] - w64[li])) * w_scale
        layers[s.name] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                          "algorithmic_bytes": gemm_alg_bytes(s),
                          "ratio": round((fb + wb) / gemm_alg_bytes(s), 3)}
        tot += fb + wb
    try:
        d = json.load(open(TRAFFIC_FILE))
        if d.get("gemm_source_sha") != src_sha():
            d = {}
    except (OSError, ValueError):
        d = {}
    d["gemm_source_sha"] = src_sha()
    d.setdefault("per_launch_bytes", {})[workload] = round(tot)
    d.setdefault("layers", {})[workload] = layers
    d["calibration"] = {"copy_bytes": copy_bytes, "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
                        "counters": list(RD_COUNTERS + WR_COUNTERS),
                        "read_requests_of_other_sizes": [sum(c_other), sum(g_other)]}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(d, open(TRAFFIC_FILE, "w"), indent=1, sort_keys=True)
    print(json.dumps({"workload": workload, "traffic_bytes": round(tot), "layers": layers,
                      "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)}))
    return 0


def _copy_scales(directory: str):
    copy_bytes = COPY_MB * 2**20
    cr, _ = _read_bytes(directory, "copy_rd", ("elementwise",))
    cw = _write_bytes(directory, "copy_wr", ("elementwise",))
    if not cr or not cw:
        raise SystemExit("no copy-kernel counters found")
    return copy_bytes / (sum(cr) / len(cr)), copy_bytes / (sum(cw) / len(cw))


def quant_traffic_summary(directory: str, workload: str, launches: int) -> int:
    """Per-call HBM bytes of the quantize half (all of its launches) from the
    quant_rd / quant_wr folders of --mode quant runs, scaled like the GEMM's by
    the copy kernel's factors (copy_rd, copy_wr)."""
    specs, _ = workload_specs(workload)
    f_scale, w_scale = _copy_scales(directory)
    n32, n64, n128 = (_per_layer(directory, "quant_rd", c, launches, QUANT_KERNELS) for c in RD_COUNTERS[:3])
    w64, wall = (_per_layer(directory, "quant_wr", c, launches, QUANT_KERNELS) for c in WR_COUNTERS)
    if min(len(n32), len(w64)) < len(specs):
        raise SystemExit(f"expected quantize calls of {len(specs)} layers, got {len(n32)} / {len(w64)}")
    layers = {}
    for li, s in enumerate(specs):
        fb = (32 * n32[li] + 64 * n64[li] + 128 * n128[li]) * f_scale
        wb = (64 * w64[li] + 32 * (wall[li] - w64[li])) * w_scale
        layers[s.name] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                          "algorithmic_bytes": quant_alg_bytes(s),
                          "ratio": round((fb + wb) / quant_alg_bytes(s), 3)}
    try:
        d = json.load(open(QUANT_TRAFFIC_FILE))
        if d.get("quant_source_sha") != quant_src_sha():
            d = {}
    except (OSError, ValueError):
        d = {}
    d["quant_source_sha"] = quant_src_sha()
    d.setdefault("layers", {})[workload] = layers
    d["calibration"] = {"fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
                        "counters": list(RD_COUNTERS[:3] + WR_COUNTERS)}
    os.makedirs(os.path.dirname(QUANT_TRAFFIC_FILE), exist_ok=True)
    json.dump(d, open(QUANT_TRAFFIC_FILE, "w"), indent=1, sort_keys=True)
    print(json.dumps({"workload": workload, "quant_layers": layers}))
    return 0


STALL_COUNTERS = ("TA_BUSY_avr", "TA_ADDR_STALLED_BY_TC_CYCLES_sum", "GRBM_GUI_ACTIVE",
                  "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum", "TCC_HIT_sum", "TCC_MISS_sum",
                  "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES")
STALL_FILE = os.path.join(ROOT, "profiles", "gemm_stalls.json")


def stall_summary(directory: str, workload: str, launches: int) -> int:
    """Where the fused GEMM's memory side spends its time, from one rocprofv3
    --pmc pass with STALL_COUNTERS (folder gemm_stall, ``bench.py --mode gemm``):
    the texture addresser's busy share (TA_BUSY_avr, the mean over the 256 TA
    instances, against GRBM_GUI_ACTIVE / 8, the active cycles of one XCD), the
    share of it stalled by the L1 (TA_ADDR_STALLED_BY_TC_CYCLES summed over the
    TAs), the mean L1 -> L2 read latency in cycles, the L2 hit rate, and the
    share of wave cycles spent waiting on LDS instructions."""
    specs, _ = workload_specs(workload)
    vals = {c: _per_layer(directory, "gemm_stall", c, launches) for c in STALL_COUNTERS}
    if any(len(v) < len(specs) for v in vals.values()):
        raise SystemExit("missing stall counter dispatches")
    layers = {}
    for li, s in enumerate(specs):
        v = {c: x[li] for c, x in vals.items()}
        xcd_cycles = v["GRBM_GUI_ACTIVE"] / 8
        layers[s.name] = {
            "ta_busy": round(v["TA_BUSY_avr"] / xcd_cycles, 4),
            "ta_stalled_by_l1": round(v["TA_ADDR_STALLED_BY_TC_CYCLES_sum"] / N_CUS / xcd_cycles, 4),
            "l2_read_latency_cycles": round(v["TCP_TCC_READ_REQ_LATENCY_sum"] / max(v["TCP_TCC_READ_REQ_sum"], 1), 1),
            "l2_hit_rate": round(v["TCC_HIT_sum"] / max(v["TCC_HIT_sum"] + v["TCC_MISS_sum"], 1), 4),
            "lds_wait_share": round(v["SQ_WAIT_INST_LDS"] / max(v["SQ_WAVE_CYCLES"], 1), 4),
            "counters": {c: round(x) for c, x in v.items()}}
    try:
        d = json.load(open(STALL_FILE))
    except (OSError, ValueError):
        d = {}
    d[workload] = {"gemm_source_sha": src_sha(), "layers": layers}
    os.makedirs(os.path.dirname(STALL_FILE), exist_ok=True)
    json.dump(d, open(STALL_FILE, "w"), indent=1, sort_keys=True)
    print(json.dumps({"workload": workload, "stalls": layers}))
    return 0


def mfma_summary(directory: str, workload: str, launches: int) -> int:
    """MFMA utilisation of the fused GEMM from a rocprofv3 --pmc pass with
    MFMA_COUNTERS (folder gemm_mfma, ``bench.py --mode gemm``) and the bench line
    of a kernel-trace run of the same workload (trace_bench.json: per-launch us).

    SQ_VALU_MFMA_BUSY_CYCLES sums the matrix-core busy cycles of all 1024 SIMDs
    (each v_mfma_i32_32x32x32_i8 adds 32); GRBM_GUI_ACTIVE sums the GPU-active
    cycles of the 8 XCDs.  So the shader clock during the launch is
    GRBM_GUI_ACTIVE / 8 / duration, and the busy share of the SIMD-cycles is
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 * 1024).  ops =
    SQ_INSTS_VALU_MFMA_MOPS_I8 * 512, to match 2 m n k."""
    specs, _ = workload_specs(workload)
    vals = {c: _per_layer(directory, "gemm_mfma", c, launches) for c in MFMA_COUNTERS}
    if any(len(v) < len(specs) for v in vals.values()):
        raise SystemExit("missing MFMA counter dispatches")
    try:
        per_us = json.load(open(os.path.join(directory, "trace_bench.json")))["roofline"]["per_launch_us"]
    except (OSError, ValueError, KeyError):
        per_us = {}
    layers = {}
    for li, s in enumerate(specs):
        avg = {c: v[li] for c, v in vals.items()}
        xcd_cycles = avg["GRBM_GUI_ACTIVE"] / 8
        rec = {"mfma_busy": round(avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (xcd_cycles * 4 * N_CUS), 4),
               "mops_i8_x512": round(avg["SQ_INSTS_VALU_MFMA_MOPS_I8"] * 512),
               "two_mnk": 2 * s.m * s.n * s.k,
               "counters": {c: round(v) for c, v in avg.items()}}
        if s.name in per_us:
            us = per_us[s.name]
            clk = xcd_cycles / (us * 1e-6)
            rec.update({"launch_us": us, "clock_ghz": round(clk / 1e9, 3),
                        "int8_peak_at_clock_tops": round(N_CUS * 8192 * clk / 1e12, 1),
                        "achieved_tops": round(2 * s.m * s.n * s.k / (us * 1e-6) / 1e12, 1)})
        layers[s.name] = rec
    try:
        d = json.load(open(MFMA_FILE))
    except (OSError, ValueError):
        d = {}
    d[workload] = {"gemm_source_sha": src_sha(), "layers": layers,
                   "normalisation": "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs * 1024 SIMDs); "
                                    "clock = GRBM_GUI_ACTIVE / 8 / launch duration"}
    os.makedirs(os.path.dirname(MFMA_FILE), exist_ok=True)
    json.dump(d, open(MFMA_FILE, "w"), indent=1, sort_keys=True)
    print(json.dumps({"workload": workload, "layers": layers}))
    return 0


def dequant_run(steps: int, warmup: int) -> int:
    """The int8 vectorwise dequantize op on the 65B up-projection's weight
    (22016 x 8192 codes -> fp16), rotated over copies past the 256 MB MALL;
    one JSON line with its HBM roofline (bytes: codes + absmax + fp16 out)."""
    import torch
    import int8_mixed_precision_vectorwise_amd as i8
    from synth import layer_specs
    dev = torch.device("cuda:0")
    spec = [s for s in layer_specs("llama65b_prefill_m4096") if s.name == "up"][0]
    n, k = spec.n, spec.k
    gen = torch.Generator(device=dev)
    gen.manual_seed(spec.config_id * 1000 + spec.layer_id)
    copies = 4  # 4 x 180 MB codes + 4 x 360 MB out
    qs = [torch.randint(-127, 128, (n, k), device=dev, dtype=torch.int8, generator=gen) for _ in range(copies)]
    ss = [torch.rand(n, device=dev, generator=gen) + 0.01 for _ in range(copies)]
    outs = [torch.empty((n, k), device=dev, dtype=torch.float16) for _ in range(copies)]
    for i in range(max(warmup, copies)):
        i8.vectorwise_dequant(qs[i % copies], ss[i % copies], torch.float16, outs[i % copies])
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(steps):
        i8.vectorwise_dequant(qs[i % copies], ss[i % copies], torch.float16, outs[i % copies])
    e1.record(st)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    byts = n * k + 4 * n + 2 * n * k
    gbs = byts / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "int8 vectorwise dequant GB/s & % HBM peak", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i8->f16",
        "data": "synthetic (seeded codes and scales)",
        "config": {"workload": "dequant_65b_up_weight", "rows": n, "cols": k, "rotation_copies": copies},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": round(gbs / (PEAK_HBM / 1e9), 4), "traffic": None,
                     "kernel": "vectorwise_dequant_kernel", "per_launch_us": round(us, 3)},
        "cpu_baseline": None}), flush=True)
    return 0


def backward_run(args) -> int:
    """The backward through every layer of a prefill workload: grad_x and
    grad_w of each linear for a seeded upstream gradient, with the forward's
    outlier list (from its quantization of x, untimed) and the fp16 weight
    kept for training.  One JSON line; the dominant kernel is the fused int8
    GEMM (two per layer), timed alone on the same operands."""
    import torch
    import int8_mixed_precision_vectorwise_amd as i8
    from synth import draw_grad, make_layer
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    specs, kind = workload_specs(args.workload)
    if kind != "prefill":
        raise SystemExit("--mode backward takes a prefill workload")
    cap = args.cap
    base = []
    per_copy = 0
    for s in specs:
        log(f"layer {s.name}: m={s.m} k={s.k} n={s.n} outliers={s.n_outlier}")
        L = make_layer(s)
        x = torch.from_numpy(L.x).to(dev)
        w = torch.from_numpy(L.w).to(dev)
        g = torch.from_numpy(draw_grad(s.m, s.n, seed=(s.config_id, s.layer_id, s.variant_id))).to(dev)
        fws = i8.LinearWorkspace.create(s.m, s.n, s.k, cap, dev)
        i8.linear_quantize(x, fws, s.tau)
        bws = i8.BackwardWorkspace.create(s.m, s.n, s.k, cap, dev)
        base.append((s, x, w, g, fws))
        per_copy += 2 * (x.numel() + w.numel() + g.numel()) + bws.buf.numel() + 2 * (s.m + s.n) * s.k
    copies = int(min(64, max(2, math.ceil(args.rotate_mb * 2**20 / per_copy))))
    log(f"rotation copies: {copies} ({per_copy / 2**20:.1f} MiB each)")
    sets = []
    for c in range(copies):
        layer_sets = []
        for s, x, w, g, fws in base:
            if c > 0:
                x, w, g = x.clone(), w.clone(), g.clone()
                fws2 = i8.LinearWorkspace.create(s.m, s.n, s.k, cap, dev)
                i8.linear_quantize(x, fws2, s.tau)
                fws = fws2
            bws = i8.BackwardWorkspace.create(s.m, s.n, s.k, cap, dev)
            bws2 = i8.BackwardWorkspace.create(s.m, s.n, s.k, cap, dev) if args.bwd_streams == 2 else None
            gx = torch.empty((s.m, s.k), dtype=torch.float16, device=dev)
            gw = torch.empty((s.n, s.k), dtype=torch.float16, device=dev)
            layer_sets.append((s, x, w, g, fws, bws, gx, gw, bws2))
        sets.append(layer_sets)
    torch.cuda.synchronize()
    for s, x, w, g, fws, *_ in sets[0]:
        if fws.outliers_past_cap():
            log(f"layer {s.name}: more outlier columns than cap={cap} (those past it take the slow path)")

    side = torch.cuda.Stream() if args.bwd_streams == 2 else None  # default priority

    def step(c: int) -> None:
        if side is None:
            for s, x, w, g, fws, bws, gx, gw, _ in sets[c]:
                i8.linear_backward(g, x, w, fws, True, True, bws, gx, gw)
            return
        # grad_x of every layer on the current stream, grad_w on a second one
        # (own workspaces), joined at the end of the step
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        for s, x, w, g, fws, bws, gx, gw, bws2 in sets[c]:
            i8.linear_backward(g, x, w, fws, True, False, bws, gx, None)
            with torch.cuda.stream(side):
                i8.linear_backward(g, x, None, fws, False, True, bws2, None, gw)
        main.wait_stream(side)

    for i in range(max(args.warmup, copies)):
        step(i % copies)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(i % copies)
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / args.steps
    log(f"eager: {eager_ms * 1e3:.2f} us/step")
    ms, launch, graph_ms = eager_ms, "eager", None
    if args.graph == "on":
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())

        def capture(nsteps):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.stream(st):
                with torch.cuda.graph(gr, stream=st):
                    for c in range(nsteps):
                        step(c)
            return gr

        g_all = capture(copies)
        rem = args.steps % copies
        g_rem = capture(rem) if rem else None
        torch.cuda.synchronize()
        for _ in range(max(1, args.warmup // copies)):
            g_all.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps // copies):
            g_all.replay()
        if g_rem is not None:
            g_rem.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / args.steps
        log(f"graph replay: {graph_ms * 1e3:.2f} us/step")
        if graph_ms < ms:
            ms, launch = graph_ms, "hipGraph replay"

    # the two gradient GEMMs of each layer alone: the same fused kernel on the
    # same operands, reached through the forward's quantize -> matmul-dequant
    # entries (the row-wise codes of g^T are the column-wise codes of g)
    gemm_sets = []
    for s, x, w, g, fws, bws, gx, gw, _ in sets[0]:
        wt_q, wt_s = i8.colwise_quant(w)
        ws_x = i8.LinearWorkspace.create(s.m, s.k, s.n, 0, dev)
        i8.linear_quantize(g, ws_x, 0.0)
        xt_q, xt_s = i8.colwise_quant(x, fws.idx(), fws.count())
        ws_w = i8.LinearWorkspace.create(s.n, s.k, s.m, 0, dev)
        gt = g.t().contiguous()
        i8.linear_quantize(gt, ws_w, 0.0)
        gemm_sets.append((s, (g, ws_x, wt_q, wt_s, gx), (gt, ws_w, xt_q, xt_s, gw)))
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    gemm_us = {}
    reps = max(10, args.steps // 2)
    with torch.cuda.stream(st):
        for s, gx_args, gw_args in gemm_sets:
            for tag, (xq, wsq, bq, bs, out) in (("grad_x", gx_args), ("grad_w", gw_args)):
                for _ in range(3):
                    i8.linear_matmul_dequant(xq, wsq, bq, bs, None, out)
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr, stream=st):
                    for _ in range(4):
                        i8.linear_matmul_dequant(xq, wsq, bq, bs, None, out)
                gr.replay()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                for _ in range(reps):
                    gr.replay()
                e1.record(st)
                torch.cuda.synchronize()
                gemm_us[f"{s.name}.{tag}"] = e0.elapsed_time(e1) * 1e3 / (reps * 4)
                log(f"gemm {s.name} {tag}: {gemm_us[f'{s.name}.{tag}']:.2f} us/launch")

    ops = sum(4 * s.m * s.n * s.k for s in specs)
    value = ops / (ms * 1e-3) / 1e12
    g_time = sum(gemm_us.values()) * 1e-6
    achieved = ops / g_time / 1e12
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_INT8_OPS / 1e12, "unit": "TFLOP/s",
            "frac": round(achieved / (PEAK_INT8_OPS / 1e12), 4), "traffic": None,
            "kernel": "fused int8 GEMM + dequant epilogue (gemm_pp_kernel / gemm_dtl_kernel by shape), grad_x and grad_w launches",
            "per_launch_us": {k: round(v, 3) for k, v in gemm_us.items()},
            "timing": "HIP events around graph replays of each gradient GEMM's launches"}

    cpu = None
    if not args.no_cpu:
        import oracle  # only this leg of the benchmark touches the oracle
        log(f"cpu oracle for ~{args.cpu_seconds:.0f} s")
        rows = 256
        prepared = []
        for s in specs:
            L = make_layer(s, m=rows)
            gg = draw_grad(s.m, s.n, seed=(s.config_id, s.layer_id, s.variant_id))[:rows]
            prepared.append((s, L, gg, oracle.outlier_columns(L.x, s.tau)))
        done, reps_c, t0 = 0.0, 0, time.perf_counter()
        while True:
            for s, L, gg, cols in prepared:
                oracle.linear_backward(gg, L.x, L.w, cols)
                done += 4.0 * rows * s.n * s.k
            reps_c += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or reps_c >= 1000:
                break
        try:
            from threadpoolctl import threadpool_info
            threads = sum(p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas")
        except Exception:  # pragma: no cover
            threads = 1
        cpu = {"value": done / el / 1e12, "unit": "TOPS", "cores": max(threads, 1), "kind": "oracle",
               "sample": f"{reps_c} passes of the backward over the workload's layers with {rows} of each "
                         f"layer's rows (outlier set from the sampled rows)", "seconds": round(el, 2)}

    print(json.dumps({
        "metric": "int8 linear backward TOPS (grad_x + grad_w, 4*m*n*k per layer) & % int8-MFMA peak",
        "value": round(value, 4), "unit": "TOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8+f16", "data": "synthetic (seeded layers and upstream gradients)",
        "config": {"workload": args.workload + "_backward",
                   "layers": [{"name": s.name, "m": s.m, "k": s.k, "n": s.n, "outlier_cols": s.n_outlier}
                              for s in specs],
                   "threshold": specs[0].tau, "cap": cap, "launch": launch,
                   "streams": args.bwd_streams,
                   "eager_ms_per_step": round(eager_ms, 6),
                   "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 6),
                   "rotation_copies": copies, "device": torch.cuda.get_device_name(dev)},
        "roofline": roof, "cpu_baseline": cpu}), flush=True)
    return 0


def fp4_counter_run(args) -> int:
    """--mode fp4gemv: args.launches 4-bit decode linears per layer of a decode
    workload, each layer between two marks (for rocprofv3 --pmc runs)."""
    import torch
    import int8_mixed_precision_vectorwise_amd as i8
    from synth import make_layer
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    specs, kind = workload_specs(args.workload)
    if kind != "decode":
        raise SystemExit("--mode fp4gemv takes a decode workload (llama13b_decode_m1, _m4, _m16)")
    layers = []
    for s in specs:
        L = make_layer(s)
        fw = i8.fp4_quantize(torch.from_numpy(L.w).to(dev), double_quant=True)
        fws = [fw, i8.Fp4Weight(fw.codes.clone(), fw.k, None, fw.c8.clone(), fw.s2.clone())]
        out = torch.empty((s.m, s.n), dtype=torch.float16, device=dev)
        layers.append((s, torch.from_numpy(L.x).to(dev), fws, out))
    torch.cuda.synchronize()
    torch.full((1,), -1, dtype=torch.int32, device=dev)
    for li, (s, x, fws, out) in enumerate(layers):
        for i in range(args.launches):
            i8.fp4_linear(x, fws[i % 2], None, out)
        torch.full((1,), li, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    print(json.dumps({"workload": args.workload, "fp4_launches_per_layer": args.launches}))
    return 0


def fp4_traffic_summary(directory: str, workload: str, launches: int) -> int:
    """Per-launch HBM bytes of the 4-bit decode linear from the fp4_rd / fp4_wr
    folders of --mode fp4gemv runs, counted and scaled as the GEMM's (copy_rd,
    copy_wr give the factors)."""
    specs, _ = workload_specs(workload)
    f_scale, w_scale = _copy_scales(directory)
    k4 = ("fp4_gemv_kernel", "fp4_rows_kernel", "fp4_rows4_kernel", "fp4_mfma16_kernel")
    n32, n64, n128 = (_per_layer(directory, "fp4_rd", c, launches, k4) for c in RD_COUNTERS[:3])
    w64, wall = (_per_layer(directory, "fp4_wr", c, launches, k4) for c in WR_COUNTERS)
    if min(len(n32), len(w64)) < len(specs):
        raise SystemExit(f"expected 4-bit launches of {len(specs)} layers, got {len(n32)} / {len(w64)}")
    per_launch = {}
    tot = 0.0
    for li, s in enumerate(specs):
        fb = (32 * n32[li] + 64 * n64[li] + 128 * n128[li]) * f_scale
        wb = (64 * w64[li] + 32 * (wall[li] - w64[li])) * w_scale
        per_launch[s.name] = {"fetch_bytes": round(fb), "write_bytes": round(wb)}
        tot += fb + wb
    d = {"fp4_source_sha": fp4_src_sha(), "workload": workload,
         "calibration": {"fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
                         "counters": list(RD_COUNTERS[:3] + WR_COUNTERS)},
         "per_launch": per_launch, "per_step_bytes": {workload: round(tot)}}
    os.makedirs(os.path.dirname(FP4_TRAFFIC_FILE), exist_ok=True)
    json.dump(d, open(FP4_TRAFFIC_FILE, "w"), indent=1, sort_keys=True)
    print(json.dumps(d))
    return 0


def fp4_run(args) -> int:
    """The 4-bit (FP4 E2M1, double-quantized block scales) decode linear over
    a decode workload's layers (the same shapes as the int8 decode workload);
    one JSON line with its HBM roofline.  Bytes per layer: packed codes,
    8-bit scales and their group maxima, x and the fp16 output."""
    import torch
    import int8_mixed_precision_vectorwise_amd as i8
    from synth import make_layer
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    specs, kind = workload_specs(args.workload)
    if kind != "decode":
        raise SystemExit("--mode fp4 takes a decode workload (llama13b_decode_m1, _m4, _m16)")
    base = []
    per_copy = 0
    for s in specs:
        L = make_layer(s)
        fw = i8.fp4_quantize(torch.from_numpy(L.w).to(dev), double_quant=True)
        x = torch.from_numpy(L.x).to(dev)
        base.append((s, x, fw))
        per_copy += fw.codes.numel() + fw.c8.numel() + 4 * fw.s2.numel()
    copies = int(min(64, max(2, math.ceil(args.rotate_mb * 2**20 / per_copy))))
    log(f"rotation copies: {copies} ({per_copy / 2**20:.1f} MiB of 4-bit weights each)")
    sets = []
    for c in range(copies):
        layer_sets = []
        for s, x, fw in base:
            fwc = fw if c == 0 else i8.Fp4Weight(fw.codes.clone(), fw.k, None, fw.c8.clone(), fw.s2.clone())
            out = torch.empty((s.m, s.n), dtype=torch.float16, device=dev)
            layer_sets.append((s, x, fwc, out))
        sets.append(layer_sets)
    torch.cuda.synchronize()

    def step(c: int) -> None:
        for s, x, fwc, out in sets[c]:
            i8.fp4_linear(x, fwc, None, out)

    for i in range(max(args.warmup, copies)):
        step(i % copies)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            for c in range(copies):
                step(c)
        g.replay()
        reps = max(1, args.steps // copies)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(reps):
            g.replay()
        e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * copies)
    # per-layer launch time (same stream, graph replays of that layer alone)
    per_us = {}
    with torch.cuda.stream(st):
        for li, s in enumerate(specs):
            gl = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gl, stream=st):
                for c in range(copies):
                    _, x, fwc, out = sets[c][li]
                    i8.fp4_linear(x, fwc, None, out)
            gl.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(reps):
                gl.replay()
            e1.record(st)
            torch.cuda.synchronize()
            per_us[s.name] = e0.elapsed_time(e1) * 1e3 / (reps * copies)
            log(f"fp4 linear {s.name}: {per_us[s.name]:.2f} us/launch")

    def layer_bytes(s, fw):
        return fw.n * fw.k // 2 + fw.c8.numel() + 4 * fw.s2.numel() + 2 * s.m * s.k + 2 * s.m * s.n

    byts = sum(layer_bytes(s, fw) for s, _, fw in base)
    gbs = byts / (ms * 1e-3) / 1e9
    k_time = sum(per_us.values()) * 1e-6
    achieved = byts / k_time / 1e9
    cpu = None
    if not args.no_cpu:
        from oracle import fp4 as fp4_oracle  # only this leg of the benchmark touches the oracle
        rows = 1024
        prepared = []
        for s in specs:
            L = make_layer(s)
            c, a = fp4_oracle.fp4_quantize(L.w[:rows])
            c8, s2 = fp4_oracle.double_quant(a)
            prepared.append((s, L.x, c, fp4_oracle.double_dequant(c8, s2)))
        done, reps_c, t0 = 0.0, 0, time.perf_counter()
        while True:
            for s, x, c, sc in prepared:
                fp4_oracle.fp4_linear(x, c, sc)
                done += rows * s.k // 2 + rows * s.k // 64 + 2 * s.m * s.k + 2 * s.m * rows
            reps_c += 1
            el = time.perf_counter() - t0
            if el >= min(args.cpu_seconds, 10.0) or reps_c >= 1000:
                break
        try:
            from threadpoolctl import threadpool_info
            threads = sum(p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas")
        except Exception:  # pragma: no cover
            threads = 1
        cpu = {"value": done / el / 1e9, "unit": "GB/s", "cores": max(threads, 1), "kind": "oracle",
               "sample": f"{reps_c} passes over the layers with {rows} weight rows each (scales from those rows)",
               "seconds": round(el, 2)}
    traffic = None
    try:
        t = json.load(open(FP4_TRAFFIC_FILE))
        if t.get("fp4_source_sha") == fp4_src_sha():
            traffic = t.get("per_step_bytes", {}).get(args.workload)
    except (OSError, ValueError):
        pass
    print(json.dumps({
        "metric": "4-bit (FP4 E2M1, blocks of 64, double-quantized scales) decode linear GB/s & % HBM peak",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": reps * copies, "warmup": args.warmup,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4+f16", "data": "synthetic (seeded layers)",
        "config": {"workload": args.workload + "_fp4",
                   "layers": [{"name": s.name, "m": s.m, "k": s.k, "n": s.n} for s in specs],
                   "rotation_copies": copies, "launch": "hipGraph replay",
                   "device": torch.cuda.get_device_name(dev)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": round(achieved / (PEAK_HBM / 1e9), 4), "traffic": traffic,
                     "kernel": "fp4_rows_kernel (one row of x, k <= 16384) / fp4_mfma16_kernel (two to four, "
                               "k <= 14336) / fp4_rows4_kernel / fp4_gemv_kernel (k > 16384)", "per_launch_us": {k: round(v, 3) for k, v in per_us.items()},
                     "timing": "HIP events around graph replays of each layer's launches"},
        "cpu_baseline": cpu}), flush=True)
    return 0


def copy_run(launches: int) -> int:
    """A plain copy of known size (COPY_MB MiB read, COPY_MB MiB written) for counter calibration."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_MB * 2**20 // 2, dtype=torch.float16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(launches):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_mib": COPY_MB, "launches": launches}))
    return 0


def prepare_sets(torch, i8, specs, cap, rotate_mb, dev):
    """Inputs resident in HBM and weights quantized once (untimed), rotated over
    enough copies that the working set exceeds the last-level caches."""
    from synth import make_layer
    base = []
    per_copy = 0
    for s in specs:
        log(f"layer {s.name}: m={s.m} k={s.k} n={s.n} planted outliers={s.n_outlier}")
        L = make_layer(s)
        x = torch.from_numpy(L.x).to(dev)
        w = torch.from_numpy(L.w).to(dev)
        wq, wabs = i8.quantize_weight(w)
        del w
        b = torch.from_numpy(L.bias).to(dev) if L.bias is not None else None
        ws = i8.LinearWorkspace.create(s.m, s.n, s.k, cap, dev)
        base.append((s, x, wq, wabs, b))
        per_copy += x.numel() * 2 + wq.numel() + ws.buf.numel() + s.m * s.n * 2
    copies = int(min(64, max(2, math.ceil(rotate_mb * 2**20 / per_copy))))
    log(f"rotation copies: {copies} ({per_copy / 2**20:.1f} MiB each)")
    sets = []
    for c in range(copies):
        layer_sets = []
        for s, x, wq, wabs, b in base:
            if c == 0:
                xc, wqc, wac = x, wq, wabs
            else:
                xc, wqc, wac = x.clone(), wq.clone(), wabs.clone()
            ws = i8.LinearWorkspace.create(s.m, s.n, s.k, cap, dev)
            out = torch.empty((s.m, s.n), dtype=torch.float16, device=dev)
            layer_sets.append((s, xc, wqc, wac, b, ws, out))
        sets.append(layer_sets)
    torch.cuda.synchronize()
    return sets, copies


def time_steps(torch, i8, sets, cap, copies, steps, warmup, graph):
    """Eager and hipGraph-replay time per step (ms), the faster labelled."""
    def step(c: int) -> None:
        for s, xc, wqc, wac, b, ws, out in sets[c]:
            i8.linear(xc, wqc, wac, b, s.tau, cap, ws, out)

    for c in range(copies):
        step(c)
    torch.cuda.synchronize()
    for s, xc, wqc, wac, b, ws, out in sets[0]:
        n_out = int(ws.count().item())
        log(f"layer {s.name}: {n_out} outlier columns" + (" (past cap: the slower path)" if n_out > cap else ""))

    for i in range(warmup):
        step(i % copies)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i % copies)
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / steps
    log(f"eager: {eager_ms * 1e3:.2f} us/step")
    ms, launch, graph_ms = eager_ms, "eager", None
    if graph:
        # one graph holds a whole rotation (steps over copies 0 .. copies-1),
        # so a replay costs one graph launch per `copies` steps; a second graph
        # holds the remainder, so exactly `steps` steps run in the timed region
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())

        def capture(nsteps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(st):
                with torch.cuda.graph(g, stream=st):
                    for c in range(nsteps):
                        step(c)
            return g

        g_all = capture(copies)
        rem = steps % copies
        g_rem = capture(rem) if rem else None
        torch.cuda.synchronize()
        for _ in range(max(1, warmup // copies)):
            g_all.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps // copies):
            g_all.replay()
        if g_rem is not None:
            g_rem.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / steps
        log(f"graph replay: {graph_ms * 1e3:.2f} us/step ({copies} steps per graph)")
        if graph_ms < ms:
            ms, launch = graph_ms, "hipGraph replay"
    return ms, eager_ms, graph_ms, launch


def gemm_roofline(specs, gemm_us, workload):
    """Roofline of the fused GEMM kernel over the step's launches."""
    g_ops = sum(2 * s.m * s.n * s.k for s in specs)
    g_bytes = sum(gemm_alg_bytes(s) for s in specs)
    g_time = sum(gemm_us[s.name] for s in specs) * 1e-6
    if g_ops / PEAK_INT8_OPS >= g_bytes / PEAK_HBM:
        achieved = g_ops / g_time / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_INT8_OPS / 1e12,
                "unit": "TFLOP/s", "frac": round(achieved / (PEAK_INT8_OPS / 1e12), 4)}
    else:
        achieved = g_bytes / g_time / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": round(achieved / (PEAK_HBM / 1e9), 4)}
    roof["kernel"] = ("fused int8 GEMM + dequant epilogue, the GEMM half of the linear run alone "
                      "(gemm_pp_kernel / gemm_dtl_kernel for prefill; gemv_kernel for m <= 2, "
                      "gemm_decode_kernel for m <= 16)")
    roof["per_launch_us"] = {k: round(v, 3) for k, v in gemm_us.items()}
    roof["timing"] = "HIP events around graph replays of the layer's GEMM launches"
    roof["traffic"] = read_traffic(workload)
    return roof


def decode_record(torch, i8, dev, args):
    """13B decode layers (up and down, 8 outlier columns) at m = 1, 4 and 16:
    whole-linear GB/s of algorithmic bytes and the fraction of 8 TB/s."""
    out = {}
    for m in (1, 4, 16):
        wl = f"llama13b_decode_m{m}"
        specs, _ = workload_specs(wl)
        sets, copies = prepare_sets(torch, i8, specs, 256, args.rotate_mb, dev)
        ms, _, _, launch = time_steps(torch, i8, sets, 256, copies, max(args.steps, 100), args.warmup,
                                      args.graph == "on")
        byts = sum(alg_bytes(s) for s in specs)
        gbs = byts / (ms * 1e-3) / 1e9
        out[f"m{m}"] = {"value": round(gbs, 1), "unit": "GB/s", "frac": round(gbs / (PEAK_HBM / 1e9), 4),
                        "ms_per_step": round(ms, 6), "launch": launch, "workload": wl}
        log(f"decode m={m}: {gbs:.0f} GB/s ({ms * 1e3:.2f} us/step)")
        del sets
        torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cap", type=int, default=None,
                    help="outlier capacity of the workspaces (default 256; the stress workload: k)")
    ap.add_argument("--rotate-mb", type=float, default=1024.0)
    ap.add_argument("--graph", choices=("on", "off"), default="on")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--decode", choices=("on", "off"), default="on",
                    help="with a prefill workload: also measure the 13B decode layers at m = 1, 4, 16")
    ap.add_argument("--mode", choices=("bench", "gemm", "quant", "copy", "dequant", "backward", "fp4", "fp4gemv"),
                    default="bench",
                    help="gemm: only the fused GEMM launches (for rocprofv3 --pmc); quant: only the quantize "
                         "calls; copy: calibration copy; "
                         "dequant: the int8 dequantize op on a 65B weight; backward: both gradients of "
                         "every layer of a prefill workload; fp4: the 4-bit decode linear on a decode workload; "
                         "fp4gemv: only its launches (for rocprofv3 --pmc)")
    ap.add_argument("--launches", type=int, default=20, help="launches per layer in --mode gemm / quant / copy")
    ap.add_argument("--bwd-streams", type=int, choices=(1, 2), default=2,
                    help="--mode backward: grad_x and grad_w on one stream, or on two")
    ap.add_argument("--traffic-summary", metavar="DIR",
                    help="write profiles/gemm_traffic.json from rocprofv3 --pmc outputs in DIR")
    ap.add_argument("--mfma-summary", metavar="DIR",
                    help="write profiles/gemm_mfma.json from a rocprofv3 --pmc output in DIR")
    ap.add_argument("--stall-summary", metavar="DIR",
                    help="write profiles/gemm_stalls.json from a rocprofv3 --pmc output in DIR")
    ap.add_argument("--fp4-traffic-summary", metavar="DIR",
                    help="write profiles/fp4_traffic.json from rocprofv3 --pmc outputs in DIR")
    ap.add_argument("--quant-traffic-summary", metavar="DIR",
                    help="write profiles/quant_traffic.json from rocprofv3 --pmc outputs in DIR")
    args = ap.parse_args()

    if args.stall_summary:
        return stall_summary(args.stall_summary, args.workload, args.launches)
    if args.fp4_traffic_summary:
        return fp4_traffic_summary(args.fp4_traffic_summary, args.workload, args.launches)
    if args.quant_traffic_summary:
        return quant_traffic_summary(args.quant_traffic_summary, args.workload, args.launches)
    if args.traffic_summary:
        return traffic_summary(args.traffic_summary, args.workload, args.launches)
    if args.mfma_summary:
        return mfma_summary(args.mfma_summary, args.workload, args.launches)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the multi-GPU path is not built (one GPU per box); "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import int8_mixed_precision_vectorwise_amd as i8

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.cap is None:
        # the stress input makes nearly every column an outlier: capacity k
        # keeps them all on the gathered (fast) path
        stress = args.workload.endswith("_stress")
        args.cap = max(s.k for s in workload_specs(args.workload)[0]) if stress else 256
    if args.mode == "copy":
        return copy_run(args.launches)
    if args.mode == "dequant":
        return dequant_run(args.steps, args.warmup)
    if args.mode == "backward":
        return backward_run(args)
    if args.mode == "fp4gemv":
        return fp4_counter_run(args)
    if args.mode == "fp4":
        return fp4_run(args)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    specs, kind = workload_specs(args.workload)
    cap = args.cap
    sets, copies = prepare_sets(torch, i8, specs, cap, args.rotate_mb, dev)

    if args.mode == "quant":
        # args.launches quantize calls per layer, each layer between two marks
        torch.full((1,), -1, dtype=torch.int32, device=dev)
        for li, s in enumerate(specs):
            for i in range(args.launches):
                _, xc, wqc, wac, b, ws, out = sets[i % copies][li]
                i8.linear_quantize(xc, ws, s.tau)
            torch.full((1,), li, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        print(json.dumps({"workload": args.workload, "quantize_calls_per_layer": args.launches}))
        return 0

    if args.mode == "gemm":
        # exactly args.launches GEMM launches per layer, layer after layer, each
        # layer between two one-element fills (the marks the counter summaries
        # split the dispatches at: a launch may be two kernels)
        torch.full((1,), -1, dtype=torch.int32, device=dev)
        for li, s in enumerate(specs):
            for i in range(args.launches):
                _, xc, wqc, wac, b, ws, out = sets[i % copies][li]
                if i < copies:
                    i8.linear_quantize(xc, ws, s.tau)
                i8.linear_matmul_dequant(xc, ws, wqc, wac, b, out)
            torch.full((1,), li, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        print(json.dumps({"workload": args.workload, "gemm_launches_per_layer": args.launches}))
        return 0

    ms, eager_ms, graph_ms, launch = time_steps(torch, i8, sets, cap, copies, args.steps, args.warmup,
                                                args.graph == "on")

    # ---- dominant kernel: the fused GEMM, timed alone with events on its stream -----
    gemm_us = time_gemm_launches(torch, i8, sets, specs, copies, max(args.steps, 50))
    for s in specs:
        log(f"gemm {s.name}: {gemm_us[s.name]:.2f} us/launch")
    del sets
    torch.cuda.empty_cache()

    ops = sum(2 * s.m * s.n * s.k for s in specs)
    byts = sum(alg_bytes(s) for s in specs)
    if kind == "prefill":
        value, unit = ops / (ms * 1e-3) / 1e12, "TOPS"
    else:
        value, unit = byts / (ms * 1e-3) / 1e9, "GB/s"
    roof = gemm_roofline(specs, gemm_us, args.workload)

    decode = None
    if kind == "prefill" and args.decode == "on" and not args.workload.endswith("_stress"):
        decode = decode_record(torch, i8, dev, args)

    cpu = None
    if not args.no_cpu:
        log(f"cpu oracle for ~{args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(specs, kind, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8+f16",
        "data": "synthetic (seeded layers; no datasets or trained weights)",
        "config": {
            "workload": args.workload,
            "layers": [{"name": s.name, "m": s.m, "k": s.k, "n": s.n, "planted_outlier_cols": s.n_outlier,
                        "bias": s.bias_std is not None} for s in specs],
            "threshold": specs[0].tau,
            "cap": cap,
            "launch": launch,
            "eager_ms_per_step": round(eager_ms, 6),
            "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 6),
            "rotation_copies": copies,
            "device": torch.cuda.get_device_name(dev),
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if kind == "prefill":
        line["int8_peak_frac"] = round(value / (PEAK_INT8_OPS / 1e12), 4)
    if decode is not None:
        line["decode"] = decode
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
