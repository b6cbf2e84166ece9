#!/usr/bin/env python3
"""Benchmark of row-wise safe softmax on one MI355X.

One step = one ``softmax_fwd`` call (dispatch + kernel) over the whole
workload, inputs already resident in HBM.  The default workload is the fp16
attention-score softmax [4,32,512,512] (65536 rows x 512 cols).  The metric is
effective bandwidth: (bytes read + bytes written) / time, bytes = one read of
the input plus one write of the output (GB = 1e9).

Timing: >= 100 ms of the 16-byte copy kernel to bring the GPU clocks up, W
untimed warm-up steps, then a window of exactly K steps bracketed by
torch.cuda.synchronize() and HIP events recorded on the stream the kernels run
on, repeated 5 times; the reported time per step is the median window's (the
five, their minimum and maximum are in the JSON line).  The input/output pairs rotate over enough buffers that the inputs alone fill
1 GiB (4x the 256 MB last-level cache), so reads come from HBM; a
single-buffer ("hot") figure is reported separately.

Also reported: the roofline of the dominant kernel (HBM, 8 TB/s), the 16-byte
copy ceiling over the same bytes, and the CPU oracle's throughput on the host
(a baseline, not a target).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--kernel FAMILY]
    python bench.py --summarize-rocprof DIR   # turn rocprofv3 output into profiles/ text
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
PEAK_HBM_GBPS = 8000.0  # MI355X published HBM3E bandwidth
REPEATS = 5  # timed windows of K steps; the median window is reported
HEADLINE_METRIC = "effective HBM GB/s (read+write) and \u00b5s/call, fp16 softmax [4,32,512,512]"
# The pages' own figure for this metric and workload: 0.62 ms per call for
# fp16 [4,32,512,512] on a 60-CU DCU (DCU case-study page, section 5.3),
# i.e. 134217728 B / 0.62 ms.  Another machine: context only.
PAGES_FP16_ATTN_GBPS = 134217728 / 0.62e-3 / 1e9
# Profile summaries live in profiles/<key>_<workload>.txt.  The key is the
# kernel family for plain softmax, else the operation.  A summary is valid
# while the sources that define its kernels are unchanged (the copy kernel
# used for the counter calibration lives in rws_reference.hip).
_SOFTMAX_COMMON = ["rws_device.hpp", "rws_pre.hpp", "rws_kernels.hpp", "rws_variants.hpp",
                   "rws_reference.hip"]
KERNEL_SOURCES = {
    "wave_row": _SOFTMAX_COMMON + ["rws_wave_row.hip"],
    "block_onepass": _SOFTMAX_COMMON + ["rws_block_onepass.hip"],
    "two_pass": _SOFTMAX_COMMON + ["rws_two_pass.hip"],
    "splitk": _SOFTMAX_COMMON + ["rws_splitk.hip"],
    "splitk_fused": _SOFTMAX_COMMON + ["rws_ordered.hpp", "rws_splitk_fused.hip"],
    "splitk_ordered": _SOFTMAX_COMMON + ["rws_ordered.hpp", "rws_splitk_ordered.hip"],
    "tile_rows": _SOFTMAX_COMMON + ["rws_launch.hpp", "rws_tile.hpp", "rws_tile_rows.hip"],
    "masked": _SOFTMAX_COMMON + ["rws_masked.hip", "rws_launch.hpp", "rws_tile.hpp",
                                 "rws_tile_rows.hip"],
    "backward": _SOFTMAX_COMMON + ["rws_launch.hpp", "rws_ordered.hpp", "rws_backward.hip",
                                   "rws_tile.hpp", "rws_tile_rows.hip"],
    "layernorm": _SOFTMAX_COMMON + ["rws_launch.hpp", "rws_ordered.hpp", "rws_norm.hpp",
                                    "rws_norm_wave.hip", "rws_norm_block.hip", "rws_tile.hpp",
                                    "rws_tile_rows.hip"],
}
KERNEL_SOURCES["rmsnorm"] = KERNEL_SOURCES["layernorm"]
# Substring (or substrings) that name the step's kernels in a trace.
KERNEL_SYMBOL = {"wave_row": "k_wave_row", "block_onepass": "k_block_onepass",
                 "two_pass": "k_two_pass", "splitk": "k_splitk_stage",
                 "splitk_fused": "k_splitk_fused", "splitk_ordered": "k_splitk_ordered",
                 "tile_rows": "k_tile_rows",
                 "masked": ("MaskPre", "k_tile_rows_masked"), "backward": "k_bwd_",
                 "layernorm": "k_norm_", "rmsnorm": "k_norm_"}


def kernel_source_hash(family: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, "row_wise_safe_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------
# rocprofv3 summaries
# --------------------------------------------------------------------------
def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def summarize_rocprof(directory: str, workload: str, kernel: str, command: str) -> None:
    """Write profiles/<kernel>_<workload>_*.txt from rocprofv3 output in `directory`.

    Expects sub-directories 'trace' (--kernel-trace --stats), 'fetch'
    (--pmc FETCH_SIZE) and 'write' (--pmc WRITE_SIZE), and optionally
    'occupancy' (--pmc MeanOccupancyPerCU) and 'valu' (--pmc VALUBusy), each
    holding the CSVs rocprofv3 wrote.  FETCH_SIZE / WRITE_SIZE are KiB per dispatch; they are
    scaled by what the same counter reads for the 16-byte copy kernel, whose
    true traffic is known (its bytes read and written).
    """
    syms = KERNEL_SYMBOL[kernel]
    syms = syms if isinstance(syms, tuple) else (syms,)

    def step_kernel(name):
        return any(s in name for s in syms)

    lines = [f"# rocprofv3 summary: {kernel} on {workload}", f"# command: {command}", ""]
    stats = glob.glob(os.path.join(directory, "trace", "**", "*kernel_stats.csv"), recursive=True)
    if stats:
        rows = _read_csv(stats[0])
        lines.append("## kernel stats (--kernel-trace --stats)")
        lines.append("name | calls | total_ns | average_ns | min_ns | max_ns | percentage")
        for r in rows:
            lines.append(" | ".join(str(r.get(k, "")) for k in
                                    ("Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs",
                                     "MaxNs", "Percentage")))
        lines.append("")
    meta = {}
    counters = {}
    for which, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        files = glob.glob(os.path.join(directory, which, "**", "*counter_collection.csv"),
                          recursive=True)
        if not files:
            continue
        per = {}
        for r in _read_csv(files[0]):
            if r.get("Counter_Name") != counter:
                continue
            name = r.get("Kernel_Name", "")
            per.setdefault(name, []).append(float(r.get("Counter_Value", 0.0)))
        counters[counter] = per
    copy_bytes = None
    meta_path = os.path.join(directory, "bench_meta.json")
    if os.path.exists(meta_path):
        with open(meta_path) as f:
            meta = json.load(f)
        copy_bytes = meta.get("copy_bytes")
    traffic = None
    if counters.get("FETCH_SIZE") and counters.get("WRITE_SIZE") and copy_bytes:
        def avg(vs):
            return sum(vs) / len(vs) if vs else None
        fetch, write = counters["FETCH_SIZE"], counters["WRITE_SIZE"]
        copy_name = next((n for n in fetch if "k_copy16" in n), None)
        f_c = avg(fetch.get(copy_name, [])) if copy_name else None
        w_c = avg(write.get(copy_name, [])) if copy_name else None
        names = sorted(n for n in fetch if step_kernel(n))
        lines.append("## HBM traffic (--pmc FETCH_SIZE, then --pmc WRITE_SIZE; KiB per dispatch)")
        lines.append(f"copy kernel k_copy16 ({copy_bytes} B read + {copy_bytes} B written): "
                     f"FETCH_SIZE {f_c} KiB, WRITE_SIZE {w_c} KiB")
        if names and f_c and w_c:
            sf = copy_bytes / (f_c * 1024.0)
            sw = copy_bytes / (w_c * 1024.0)
            lines.append(f"scale factors (true bytes / counter bytes): fetch {sf:.4f}, write {sw:.4f}")
            traffic = 0.0
            for n in names:
                f_k, w_k = avg(fetch[n]), avg(write.get(n, []))
                lines.append(f"kernel {n}: FETCH_SIZE {f_k:.1f} KiB, WRITE_SIZE {w_k:.1f} KiB "
                             f"-> {f_k * 1024.0 * sf + w_k * 1024.0 * sw:.0f} B")
                traffic += f_k * 1024.0 * sf + w_k * 1024.0 * sw
            lines.append(f"traffic_bytes_per_launch: {traffic:.0f}"
                         + ("  (sum of the step's kernels)" if len(names) > 1 else ""))
            if meta.get("bytes_per_call"):
                lines.append(f"algorithmic_bytes_per_launch: {meta['bytes_per_call']}")
                lines.append(f"traffic / algorithmic: {traffic / meta['bytes_per_call']:.4f}")
        lines.append("")
    # absolute traffic from the L2-to-memory (EA) request counters, by request
    # size, beside the copy-calibrated figure above
    ea = {}
    for which in ("ea_rd", "ea_wr", "ea_stall", "hits", "levels"):
        files = glob.glob(os.path.join(directory, which, "**", "*counter_collection.csv"),
                          recursive=True)
        if not files:
            continue
        for r in _read_csv(files[0]):
            name = r.get("Kernel_Name", "")
            per = ea.setdefault(name, {})
            per.setdefault(r.get("Counter_Name"), []).append(float(r.get("Counter_Value", 0.0)))
    if ea:
        def mean(per, c):
            v = per.get(c)
            return sum(v) / len(v) if v else None
        lines.append("## absolute EA traffic (--pmc TCC_EA0_RDREQ{,_128B,_64B,_32B}_sum; "
                     "--pmc TCC_EA0_WRREQ{,_64B}_sum TCC_EA0_{RD,WR}REQ_DRAM_sum; "
                     "--pmc TCC_EA0_{RD,WR}REQ_DRAM_CREDIT_STALL_sum TCC_EA0_WRREQ_STALL_sum "
                     "GRBM_GUI_ACTIVE; --pmc TCC_HIT_sum TCC_MISS_sum; --pmc "
                     "TCC_EA0_{RD,WR}REQ_LEVEL_sum TCC_EA0_{RD,WR}REQ_sum GRBM_GUI_ACTIVE; "
                     "per dispatch)")
        lines.append("read bytes = 128*RDREQ_128B + 64*RDREQ_64B + 32*RDREQ_32B; write bytes = "
                     "64*WRREQ_64B + 32*(WRREQ - WRREQ_64B); stalls are cycles summed over the "
                     "L2 channels, per GRBM_GUI_ACTIVE cycle; latency = LEVEL / requests "
                     "(cycles), in flight = LEVEL / GRBM_GUI_ACTIVE (requests, all channels)")
        abs_total = None
        for n in sorted(ea):
            if not (step_kernel(n) or "k_copy16" in n):
                continue
            per = ea[n]
            rq, r128, r64, r32 = (mean(per, c) for c in (
                "TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_128B_sum", "TCC_EA0_RDREQ_64B_sum",
                "TCC_EA0_RDREQ_32B_sum"))
            wq, w64 = mean(per, "TCC_EA0_WRREQ_sum"), mean(per, "TCC_EA0_WRREQ_64B_sum")
            parts = [f"kernel {n}:"]
            rd = wr = None
            if None not in (rq, r128, r64, r32):
                rd = 128 * r128 + 64 * r64 + 32 * r32
                parts.append(f"RDREQ {rq:.0f} (128B {r128:.0f}, 64B {r64:.0f}, 32B {r32:.0f}) "
                             f"-> read {rd:.0f} B")
            if None not in (wq, w64):
                wr = 64 * w64 + 32 * (wq - w64)
                parts.append(f"WRREQ {wq:.0f} (64B {w64:.0f}) -> write {wr:.0f} B")
            for c in ("TCC_EA0_RDREQ_DRAM_sum", "TCC_EA0_WRREQ_DRAM_sum"):
                if mean(per, c) is not None:
                    parts.append(f"{c[8:-4]} {mean(per, c):.0f}")
            gui = mean(per, "GRBM_GUI_ACTIVE")
            for c in ("TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum", "TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum",
                      "TCC_EA0_WRREQ_STALL_sum"):
                v = mean(per, c)
                if v is not None and gui:
                    parts.append(f"{c[8:-4]} {v:.0f} ({v / gui:.3f}/cycle)")
            for kind in ("RD", "WR"):
                lvl = mean(per, f"TCC_EA0_{kind}REQ_LEVEL_sum")
                req = mean(per, f"TCC_EA0_{kind}REQ_sum")
                if lvl is not None and req and gui:
                    parts.append(f"{kind} latency {lvl / req:.0f} cycles, in flight "
                                 f"{lvl / gui:.0f}")
            hit, miss = mean(per, "TCC_HIT_sum"), mean(per, "TCC_MISS_sum")
            if hit is not None and miss is not None and hit + miss > 0:
                parts.append(f"L2 hit {hit:.0f} miss {miss:.0f} ({hit / (hit + miss):.3f})")
            lines.append(" ".join(parts))
            if rd is not None and wr is not None and step_kernel(n):
                abs_total = (abs_total or 0.0) + rd + wr
        if abs_total is not None:
            lines.append(f"absolute_bytes_per_launch: {abs_total:.0f}"
                         + (f"  (/ algorithmic {abs_total / meta['bytes_per_call']:.4f}"
                            if meta.get("bytes_per_call") else "")
                         + (f", / copy-calibrated {abs_total / traffic:.4f})" if traffic
                            else ")" if meta.get("bytes_per_call") else "")
                         + ("  (sum of the step's kernels)" if sum(step_kernel(n) for n in ea) > 1
                            else ""))
        lines.append("")
    # occupancy and vector-ALU activity (one derived metric per pass)
    extra = []
    for which, metric, unit in (("occupancy", "MeanOccupancyPerCU",
                                 "mean resident waves per CU over the kernel (max 32)"),
                                ("valu", "VALUBusy", "% of kernel time the vector ALUs issue")):
        files = glob.glob(os.path.join(directory, which, "**", "*counter_collection.csv"),
                          recursive=True)
        if not files:
            continue
        per = {}
        for r in _read_csv(files[0]):
            if r.get("Counter_Name") == metric and step_kernel(r.get("Kernel_Name", "")):
                per.setdefault(r["Kernel_Name"], []).append(float(r.get("Counter_Value", 0.0)))
        for n in sorted(per):
            extra.append(f"kernel {n}: {metric} {sum(per[n]) / len(per[n]):.2f} ({unit})")
    if extra:
        lines.append("## occupancy and VALU activity (--pmc MeanOccupancyPerCU, then --pmc VALUBusy)")
        lines.extend(extra)
        lines.append("")
    lines.append(f"kernel_source_sha: {kernel_source_hash(kernel)}")
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, f"{kernel}_{workload}.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def read_traffic(workload: str, kernel: str):
    """Counter-derived HBM bytes per launch from profiles/, or None when the
    summary is missing or the kernel sources changed since it was taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    traffic = sha = None
    with open(path) as f:
        for line in f:
            if line.startswith("traffic_bytes_per_launch:"):
                # "<bytes>" or "<bytes>  (sum of the step's kernels)"
                traffic = float(line.split(":", 1)[1].split()[0])
            elif line.startswith("kernel_source_sha:"):
                sha = line.split(":")[1].strip()
    if traffic is None or sha != kernel_source_hash(kernel):
        return None
    return traffic


# --------------------------------------------------------------------------
# HIP runtime queries used only for reporting (device HBM figures, the
# runtime's own device-to-device copy as a second reference)
# --------------------------------------------------------------------------
_HIP_ATTR_MEMORY_BUS_WIDTH = 59   # hipDeviceAttributeMemoryBusWidth (bits)
_HIP_ATTR_MEMORY_CLOCK_RATE = 60  # hipDeviceAttributeMemoryClockRate (kHz)


def _hip_runtime():
    import ctypes
    lib = ctypes.CDLL("libamdhip64.so")
    lib.hipDeviceGetAttribute.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]
    lib.hipDeviceGetAttribute.restype = ctypes.c_int
    lib.hipMemcpyDtoDAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]
    lib.hipMemcpyDtoDAsync.restype = ctypes.c_int
    return lib


def device_hbm(device: int = 0) -> dict:
    """Memory clock and bus width as the runtime reports them, next to the
    published peak the roofline uses: the transfers per reported clock that
    the published 8 TB/s implies over that bus (MI355X reports a 2 GHz
    memory clock and an 8192-bit bus, so 8 TB/s is ~3.9 transfers per clock,
    i.e. ~7.8 Gb/s per pin)."""
    import ctypes
    lib = _hip_runtime()
    vals = {}
    for key, attr in (("memory_clock_khz", _HIP_ATTR_MEMORY_CLOCK_RATE),
                      ("bus_width_bits", _HIP_ATTR_MEMORY_BUS_WIDTH)):
        v = ctypes.c_int(0)
        vals[key] = v.value if lib.hipDeviceGetAttribute(ctypes.byref(v), attr, device) == 0 \
            else None
    vals["published_peak_GBps"] = PEAK_HBM_GBPS
    if vals["memory_clock_khz"] and vals["bus_width_bits"]:
        bus_bytes_per_clock = vals["memory_clock_khz"] * 1e3 * vals["bus_width_bits"] / 8
        vals["published_peak_transfers_per_clock"] = round(PEAK_HBM_GBPS * 1e9
                                                           / bus_bytes_per_clock, 3)
    return vals


# --------------------------------------------------------------------------
# CPU baseline: the oracle on the host cores
# --------------------------------------------------------------------------
def cpu_baseline(w, x_stored_f64, target_s: float = 10.0, threads: int | None = None) -> dict:
    import oracle
    if threads is None:
        threads = max(1, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
                      else (os.cpu_count() or 1))
    rows = x_stored_f64.shape[0]
    t0 = time.perf_counter()
    passes = 0
    used = threads
    while True:
        _, used = oracle.safe_softmax_threads(x_stored_f64, threads)
        passes += 1
        if time.perf_counter() - t0 >= target_s:
            break
    dt = time.perf_counter() - t0
    nbytes = 2 * rows * w.cols * w.elem_bytes * passes
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(used),
            "kind": "oracle",
            "sample": f"{passes} passes of the full {rows}x{w.cols} workload "
                      f"(fp16 values widened to float64, fp64 libm exp), rows split over "
                      f"{used} host threads; bytes counted as fp16 in+out, {dt:.1f} s"}


def norm_cpu_baseline(w, x_stored_f64, mode: str, target_s: float = 10.0) -> dict:
    """The oracle's layernorm / rmsnorm (one host thread) over a row sample."""
    import oracle
    rows = min(x_stored_f64.shape[0], 16384)
    sample = x_stored_f64[:rows]
    fn = oracle.layernorm if mode == "layernorm" else oracle.rmsnorm
    t0 = time.perf_counter()
    passes = 0
    while True:
        fn(sample, 1e-5)
        passes += 1
        if time.perf_counter() - t0 >= target_s:
            break
    dt = time.perf_counter() - t0
    nbytes = 2 * rows * w.cols * w.elem_bytes * passes
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} passes over the first {rows} rows of {w.rows}x{w.cols} "
                      f"({mode}, values widened to float64, one host thread); bytes counted "
                      f"in the workload's dtype, in+out, {dt:.1f} s"}


# --------------------------------------------------------------------------
# HBM ceilings: the copy, read-only and write-only references and the fp16
# softmax of rows of 512 over a sweep of sizes
# --------------------------------------------------------------------------
def ceilings(steps: int, warmup: int) -> dict:
    """Per-call time of the 16-byte copy, read-only and write-only kernels
    and of the fp16 [rows,512] softmax, for 16..256 MiB per direction, each
    over rotating buffers whose inputs fill 1 GiB, median of REPEATS windows
    of `steps` calls.  A least-squares line t = t0 + bytes / rate over the
    sizes >= 64 MiB separates the fixed cost of a launch (t0: ramp-up and
    drain) from the streaming rate."""
    import torch
    import row_wise_safe_amd as rws
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sh = int(stream.cuda_stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def median_us(call):
        for i in range(warmup):
            call(i)
        out = []
        for r in range(REPEATS):
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(steps):
                call(r * steps + i)
            e1.record(stream)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) * 1e3 / steps)
        return statistics.median(out)

    g = torch.Generator(device=dev)
    g.manual_seed(20260010)
    rows_out = []
    for mib in (16, 32, 64, 128, 256):
        nbytes = mib << 20
        nbuf = max(2, (1 << 30) // nbytes)
        xs = [torch.randn(nbytes // 2, generator=g, device=dev).mul_(8.0).to(torch.float16)
              for _ in range(nbuf)]
        ys = [torch.empty_like(x) for x in xs]
        rows = nbytes // 1024
        log(f"[bench] ceilings {mib} MiB, {nbuf} buffers")
        t = {
            "copy": median_us(lambda i: rws.softmax_copy_bytes(
                xs[i % nbuf].data_ptr(), ys[i % nbuf].data_ptr(), nbytes, sh)),
            "read_only": median_us(lambda i: rws.softmax_read_bytes(
                xs[i % nbuf].data_ptr(), nbytes, sh)),
            "write_only": median_us(lambda i: rws.softmax_write_bytes(
                ys[i % nbuf].data_ptr(), nbytes, sh)),
            "softmax_fp16_512": median_us(lambda i: rws.softmax_fwd(
                xs[i % nbuf].data_ptr(), ys[i % nbuf].data_ptr(), rows, 512, rws.RWS_F16, sh)),
        }
        moved = {"copy": 2 * nbytes, "read_only": nbytes, "write_only": nbytes,
                 "softmax_fp16_512": 2 * nbytes}
        entry = {"MiB_per_direction": mib}
        for k, us in t.items():
            gbps = moved[k] / (us * 1e-6) / 1e9
            entry[k] = {"us": round(us, 3), "GBps": round(gbps, 1),
                        "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4)}
        log("[bench]   " + ", ".join(f"{k} {v['us']} us ({v['frac_of_peak']:.3f})"
                                     for k, v in entry.items() if isinstance(v, dict)))
        rows_out.append(entry)
        del xs, ys
        torch.cuda.empty_cache()
    fit = {}
    big = [e for e in rows_out if e["MiB_per_direction"] >= 64]
    for k in ("copy", "read_only", "write_only", "softmax_fp16_512"):
        mult = 1 if k in ("read_only", "write_only") else 2
        xb = [mult * (e["MiB_per_direction"] << 20) for e in big]
        yt = [e[k]["us"] for e in big]
        mx, my = statistics.fmean(xb), statistics.fmean(yt)
        slope = sum((a - mx) * (b - my) for a, b in zip(xb, yt)) / sum((a - mx) ** 2 for a in xb)
        rate = 1e-3 / slope  # GB/s from us per byte
        fit[k] = {"fixed_us_per_launch": round(my - slope * mx, 3),
                  "streaming_GBps": round(rate, 1),
                  "streaming_frac_of_peak": round(rate / PEAK_HBM_GBPS, 4)}
    return {"ceilings": rows_out, "fit_over_64_to_256_MiB": fit,
            "protocol": f"median of {REPEATS} windows of {steps} calls after {warmup} warm-up "
                        "calls; inputs rotate over 1 GiB; bytes moved = read + written"}


# --------------------------------------------------------------------------
# main
# --------------------------------------------------------------------------
def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default="fp16_attn_4x32x512x512")
    ap.add_argument("--kernel", default="auto")
    ap.add_argument("--variant", type=int, default=-1,
                    help="with --kernel FAMILY: that entry of the family's compiled shapes "
                         "(softmax_fwd_variant) instead of the dispatcher's choice")
    ap.add_argument("--shape", default=None, metavar="ROWSxCOLS",
                    help="an N(0, 4^2) input of this shape instead of a named workload")
    ap.add_argument("--dtype", default="f16", choices=["f32", "f16", "bf16"],
                    help="with --shape: the element type")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--masked", action="store_true",
                    help="attention-score form: softmax(x/8 + mask[S,S] + causal) with S = cols "
                         "(softmax_fwd_masked)")
    ap.add_argument("--backward", action="store_true",
                    help="softmax backward dx = y*(dy - sum(dy*y)) on the workload's shape "
                         "(softmax_bwd): 2 reads + 1 write per element")
    ap.add_argument("--norm", choices=["layernorm", "rmsnorm"], default=None,
                    help="row normalisation instead of softmax (layernorm_fwd / rmsnorm_fwd, no "
                         "affine, eps 1e-5) on a normalisation workload (default "
                         "ln_fp16_131040x192)")
    ap.add_argument("--affine", action="store_true",
                    help="with --norm: per-column weight and bias (LayerNorm) or weight (RMSNorm), "
                         "read once per call")
    ap.add_argument("--graph", action="store_true",
                    help="also time the calls replayed from a HIP graph (no host-side cost)")
    ap.add_argument("--skip-hot", action="store_true",
                    help="skip the single-buffer figure (profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--meta-out", default=None, help="write bench metadata JSON (for rocprof)")
    ap.add_argument("--summarize-rocprof", default=None, metavar="DIR",
                    help="write profiles/<key>_<workload>.txt from rocprofv3 output; --kernel "
                         "names the key (a softmax family, or masked, backward, layernorm, "
                         "rmsnorm)")
    ap.add_argument("--profile-command", default="")
    ap.add_argument("--ceilings", action="store_true",
                    help="time the copy, read-only and write-only references and the fp16 "
                         "[rows,512] softmax over 16..256 MiB and fit fixed cost + streaming rate")
    args = ap.parse_args()

    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof, args.workload,
                          args.kernel if args.kernel != "auto" else "wave_row",
                          args.profile_command)
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(rows shard across GPUs with no communication; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import row_wise_safe_amd as rws
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    rws.load_library()
    if args.ceilings:
        print(json.dumps(ceilings(args.steps, args.warmup)), flush=True)
        return 0
    if args.norm and (args.masked or args.backward):
        print("--norm excludes --masked and --backward", file=sys.stderr)
        return 2
    if args.norm and not args.shape:
        name = args.workload if args.workload in workloads.NORM_WORKLOADS else "ln_fp16_131040x192"
        w = workloads.NORM_WORKLOADS[name]
    elif args.shape:
        r, c = (int(v) for v in args.shape.lower().split("x"))
        w = workloads.Workload(f"{args.dtype}_{r}x{c}", args.dtype, r, c, 20260020, "normal",
                               dict(sigma=4.0), f"{args.dtype} [{r},{c}] N(0,4^2)")
    else:
        w = (workloads.WORKLOADS.get(args.workload)
             or workloads.LONG_ROW_WORKLOADS[args.workload])
    dev = torch.device("cuda:0")
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    code = rws.dtype_code(tdt)
    kid = rws.KERNEL_IDS[args.kernel]

    log(f"[bench] generating {w.name} {w.rows}x{w.cols} {w.dtype}")
    x64 = w.generate()
    x_host = torch.from_numpy(x64).to(tdt)
    del x64
    nbytes = w.algorithmic_bytes
    in_bytes = nbytes // 2
    # Rotate over enough input/output pairs that the inputs alone fill 1 GiB,
    # 4x the 256 MB last-level cache, so every call reads its input from HBM.
    # (The output stores are non-temporal and do not displace inputs from
    # that cache: a rotation sized on input + output bytes left earlier
    # inputs cache-resident -- a 64 MiB copy measured 19.7 us with 4 pairs and
    # 23.1 us with 8 or more.)
    nbuf = min(4096, max(2, -(-(1 << 30) // in_bytes)))
    xs = [x_host.to(dev) for _ in range(nbuf)]
    ys = [torch.empty_like(xs[0]) for _ in range(nbuf)]
    stream = torch.cuda.current_stream(dev)
    sh = int(stream.cuda_stream)
    if args.variant >= 0:
        if kid == 0 or args.masked or args.backward or args.norm:
            print("--variant needs --kernel FAMILY of the plain forward", file=sys.stderr)
            return 2
        desc = rws.softmax_describe_variant(w.rows, w.cols, code, xs[0].data_ptr(),
                                            ys[0].data_ptr(), kid, args.variant)
    else:
        desc = rws.softmax_describe_launch(w.rows, w.cols, code, xs[0].data_ptr(),
                                           ys[0].data_ptr(), kid, masked=args.masked)
    family = desc.split("<")[0]
    if args.norm:
        desc = f"{args.norm} {args.kernel}"
    dys = None
    if args.backward:
        # y = the forward output of each input, dy ~ N(0, 1); dx goes to ys[i]
        g = np.random.Generator(np.random.PCG64(w.seed + 200))
        dy_host = torch.from_numpy(g.standard_normal((w.rows, w.cols))).to(tdt)
        dys = [dy_host.to(dev) for _ in range(nbuf)]
        for i in range(nbuf):
            rws.softmax(xs[i], out=xs[i])  # xs now hold y
        torch.cuda.synchronize()
        nbytes = 3 * w.rows * w.cols * w.elem_bytes
        desc = "backward " + desc.split("<")[0]
    mask = None
    if args.masked:
        if w.rows % w.cols:
            print("--masked needs rows to be a multiple of cols (square score blocks)",
                  file=sys.stderr)
            return 2
        g = np.random.Generator(np.random.PCG64(w.seed + 100))
        mask = torch.from_numpy(g.normal(0.0, 1.0, (w.cols, w.cols))).to(tdt).to(dev)
        nbytes += mask.numel() * mask.element_size()  # the mask is read once per call
        desc = "masked " + desc
    wptr = bptr = 0
    if args.affine:
        if not args.norm:
            print("--affine needs --norm", file=sys.stderr)
            return 2
        g = np.random.Generator(np.random.PCG64(w.seed + 300))
        weight = torch.from_numpy(g.uniform(0.5, 1.5, w.cols)).to(tdt).to(dev)
        wptr = weight.data_ptr()
        nbytes += weight.numel() * weight.element_size()
        if args.norm == "layernorm":
            bias = torch.from_numpy(g.normal(0.0, 1.0, w.cols)).to(tdt).to(dev)
            bptr = bias.data_ptr()
            nbytes += bias.numel() * bias.element_size()
        desc += " affine"
    log(f"[bench] launch: {desc}; {nbuf} rotating buffer pairs")

    def step(i, sh=sh):
        if args.norm == "layernorm":
            st = rws.layernorm_fwd_kernel(xs[i % nbuf].data_ptr(), ys[i % nbuf].data_ptr(), w.rows,
                                          w.cols, code, 1e-5, wptr, bptr, 0, 0, sh, kid)
        elif args.norm == "rmsnorm":
            st = rws.rmsnorm_fwd_kernel(xs[i % nbuf].data_ptr(), ys[i % nbuf].data_ptr(), w.rows,
                                        w.cols, code, 1e-5, wptr, 0, sh, kid)
        elif dys is not None:
            st = rws.softmax_bwd_kernel(xs[i % nbuf].data_ptr(), dys[i % nbuf].data_ptr(),
                                        ys[i % nbuf].data_ptr(), w.rows, w.cols, code, sh, kid)
        elif mask is None and args.variant >= 0:
            st = rws.softmax_fwd_variant(xs[i % nbuf].data_ptr(), ys[i % nbuf].data_ptr(), w.rows,
                                         w.cols, code, sh, kid, args.variant)
        elif mask is None:
            st = rws.softmax_fwd_kernel(xs[i % nbuf].data_ptr(), ys[i % nbuf].data_ptr(), w.rows,
                                        w.cols, code, sh, kid)
        else:
            st = rws.softmax_fwd_masked(xs[i % nbuf].data_ptr(), ys[i % nbuf].data_ptr(), w.rows,
                                        w.cols, code, 0.125, mask.data_ptr(), w.cols, w.cols, sh,
                                        kid)
        if st != rws.RWS_OK:
            raise rws.SoftmaxError(st, rws.softmax_last_error())

    # Device warm-up before the warm-up steps: after the host-side input
    # generation the GPU has idled for seconds, and its clocks take ~15 ms of
    # load to come back (measured: the first 500 masked calls of a fresh
    # process ran 24 us instead of 20.4).  The 16-byte copy over the same
    # buffers keeps it busy for >= 100 ms; it is not a step of the method.
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < 0.1:
        for i in range(nbuf):
            rws.softmax_copy_bytes(xs[i].data_ptr(), ys[i].data_ptr(), in_bytes, sh)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def windows(call, steps):
        """Per-step ms of REPEATS windows of exactly `steps` calls each."""
        out = []
        for r in range(REPEATS):
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(steps):
                call(r * steps + i)
            e1.record(stream)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / steps)
        return out

    rot = windows(step, args.steps)
    ms = statistics.median(rot)
    gbps = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] {ms * 1e3:.2f} us/call (median of {REPEATS} windows of {args.steps} steps: "
        + ", ".join(f"{t * 1e3:.2f}" for t in rot) + f"), {gbps:.1f} GB/s (rotating)")

    # single buffer: the same input and output every call.  The kernels load
    # their input non-temporally and store their output past the caches, so
    # the input is not kept in the last-level cache between calls and this
    # figure is not expected to beat the rotating one (measured within 1% of
    # it either way: 21.6 against 21.7 us, 22.2 against 21.9 us).
    hot = None
    if not args.skip_hot:
        for i in range(args.warmup):
            step(0)
        hot_w = windows(lambda i: step(0), args.steps)
        hot_ms = statistics.median(hot_w)
        hot = {"us_per_call": round(hot_ms * 1e3, 3),
               "GBps": round(nbytes / (hot_ms * 1e-3) / 1e9, 2),
               "us_per_call_windows": [round(t * 1e3, 3) for t in hot_w]}

    # the same calls replayed from a HIP graph (one graph of gcalls calls over
    # the rotating buffers, captured on a stream of its own after eager calls
    # there): the per-call time without host-side cost
    graph = None
    if args.graph:
        gstream = torch.cuda.Stream(device=dev)
        gsh = int(gstream.cuda_stream)
        gcalls = 256
        with torch.cuda.stream(gstream):
            for i in range(nbuf):
                step(i, gsh)  # sizes any split-k workspace of this stream
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gstream):
            for i in range(gcalls):
                step(i, gsh)
        reps = max(2, args.steps // gcalls)
        with torch.cuda.stream(gstream):
            for _ in range(3):
                g.replay()
            gstream.synchronize()
            e0.record(gstream)
            for _ in range(reps):
                g.replay()
            e1.record(gstream)
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / (reps * gcalls)
        graph = {"us_per_call": round(graph_ms * 1e3, 3),
                 "GBps": round(nbytes / (graph_ms * 1e-3) / 1e9, 2),
                 "calls_per_graph": gcalls, "replays": reps}
        log(f"[bench] graph replay {graph_ms * 1e3:.2f} us/call")
        del g

    # copy ceiling: 16-byte copy of the input bytes, same rotation
    def copy(i):
        rws.softmax_copy_bytes(xs[i % nbuf].data_ptr(), ys[i % nbuf].data_ptr(), in_bytes, sh)

    for i in range(args.warmup):
        copy(i)
    copy_ms = statistics.median(windows(copy, args.steps))
    copy_gbps = 2 * in_bytes / (copy_ms * 1e-3) / 1e9
    log(f"[bench] copy ceiling {copy_ms * 1e3:.2f} us, {copy_gbps:.1f} GB/s")

    # the runtime's device-to-device copy of the same bytes, same rotation
    hip = _hip_runtime()
    def memcpy(i):
        hip.hipMemcpyDtoDAsync(ys[i % nbuf].data_ptr(), xs[i % nbuf].data_ptr(), in_bytes, sh)

    for i in range(min(args.warmup, 200)):
        memcpy(i)
    memcpy_ms = statistics.median(windows(memcpy, args.steps))
    memcpy_gbps = 2 * in_bytes / (memcpy_ms * 1e-3) / 1e9
    log(f"[bench] hipMemcpyDtoDAsync {memcpy_ms * 1e3:.2f} us, {memcpy_gbps:.1f} GB/s")

    if args.meta_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.meta_out)), exist_ok=True)
        with open(args.meta_out, "w") as f:
            json.dump({"workload": w.name, "bytes_per_call": nbytes, "copy_bytes": in_bytes,
                       "launch": desc}, f)

    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        stored = x_host.to(torch.float64).numpy()
        cpu = (norm_cpu_baseline(w, stored, args.norm, args.cpu_seconds) if args.norm
               else cpu_baseline(w, stored, args.cpu_seconds))
        log(f"[bench] cpu oracle {cpu['value']} GB/s on {cpu['cores']} threads")
        if not args.norm and cpu["cores"] > 1:
            cpu1 = cpu_baseline(w, stored, args.cpu_seconds / 3, threads=1)
            log(f"[bench] cpu oracle {cpu1['value']} GB/s on 1 thread")

    profile_key = (args.norm if args.norm else "masked" if mask is not None
                   else "backward" if dys is not None else family)
    # the committed profiles cover the forms without weight and bias
    traffic = None if args.affine else read_traffic(w.name, profile_key)
    achieved = nbytes / (ms * 1e-3) / 1e9
    headline = (w.name == "fp16_attn_4x32x512x512" and mask is None and dys is None
                and args.variant < 0
                and not args.norm)
    vs = round(gbps / PAGES_FP16_ATTN_GBPS, 3) if headline else None
    result = {
        "metric": (HEADLINE_METRIC if headline else
                   f"effective HBM GB/s (read+write) and µs/call, {w.description}"
                   + (", softmax(x/8 + mask + causal)" if mask is not None else "")
                   + (", backward dx = y*(dy - sum(dy*y))" if dys is not None else "")
                   + (f", {args.norm} forward (eps 1e-5, "
                      f"{'weight and bias' if args.affine else 'no affine'})" if args.norm else "")),
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "us_per_call": round(ms * 1e3, 3),
        "timing": {"windows": REPEATS, "steps_per_window": args.steps,
                   "us_per_call_windows": [round(t * 1e3, 3) for t in rot],
                   "us_per_call_min": round(min(rot) * 1e3, 3),
                   "us_per_call_max": round(max(rot) * 1e3, 3),
                   "reported": "median window"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": vs,
        # the arithmetic type: every kernel widens its inputs to fp32 and
        # computes in fp32; the tensors' storage type is config.io_dtype
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "io_dtype": w.dtype,
                   "rows": w.rows, "cols": w.cols,
                   "bytes_per_call": nbytes, "launch": desc, "rotating_buffers": nbuf,
                   "device_warmup": ">= 100 ms of the 16-byte copy before the warm-up steps",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic},
        "hot_single_buffer": hot,
        "graph_replay": graph,
        "copy_ceiling": {"us_per_call": round(copy_ms * 1e3, 3), "GBps": round(copy_gbps, 2),
                         "frac_of_peak": round(copy_gbps / PEAK_HBM_GBPS, 4)},
        "hip_memcpy_dtod": {"us_per_call": round(memcpy_ms * 1e3, 3),
                            "GBps": round(memcpy_gbps, 2)},
        "device_hbm": device_hbm(dev.index or 0),
        "cpu_baseline": cpu,
        "cpu_baseline_single_thread": cpu1,
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
