#!/usr/bin/env python3
"""Benchmark of C = ReLU(A @ B) on one MI355X.

One step is one call of the library's gemm_relu (every step of the path: tile
loads, MFMA contraction, ReLU, cast, store) on one batch of synthetic input
already resident in HBM.  The default workload is the 8192^3 fp16 GEMM with
inputs N(0, 1) * 0.1; three separately allocated input/output sets are rotated
so that repeated reads are not served from the 256 MB MALL.

Timing follows the method of "TileLang Guide: Composable Tiled AI Kernel
Programming" (Step 2, the benchmark script): warm-up calls, then timed calls
between GPU events, throughput = 2*M*N*K / t.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import re
import subprocess
import sys
import threading
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import tiled_dense_gemm_relu_amd as gr  # noqa: E402
from tiled_dense_gemm_relu_amd import binding, inputs  # noqa: E402
from tiled_dense_gemm_relu_amd.build import kernel_source_digest  # noqa: E402

PEAK_TFLOPS = {"fp16": 2500.0, "bf16": 2500.0}     # MI355X dense MFMA, published
PEAK_HBM_GBS = 8000.0                               # MI355X HBM3E, published
METRIC = "TFLOP/s and % of MI355X dense fp16 MFMA peak, ReLU(A@B) 8192³"


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "dma256_square_8192_fp16_traffic.json")


def measured_traffic(workload_name, kernel_name):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs, scaled by the
    copy-kernel calibration; None unless they were taken on this workload, this kernel and the
    current kernel sources."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            prof = json.load(f)
    except (OSError, ValueError):
        return None
    if not prof.get("workload", "").startswith(workload_name) or kernel_name != "dma_256x256x64_2stage":
        return None
    if prof.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return int(prof["traffic_bytes_per_launch"])


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def make_sets(w, n_sets, device, b_layout=binding.B_KN):
    sets = []
    for i in range(n_sets):
        g_seed = w.seed + 1000 * i
        a, b = inputs.normal_pair(w.M, w.N, w.K, w.torch_dtype, w.scale, g_seed)
        if b_layout == binding.B_NK:
            b = b.t().contiguous()          # handed over as B^T, (N, K)
        c = torch.empty((w.M, w.N), dtype=w.torch_dtype, device=device)
        sets.append((a.to(device), b.to(device), c))
    return sets


def sample_clocks(launch, seconds):
    """Keep the GPU busy with `launch` for about `seconds` while rocm-smi samples the shader
    and memory clocks (and the package power where the board reports it).  Returns medians
    over the samples after the first, or None if rocm-smi is unavailable."""
    samples, stop = [], threading.Event()

    def smi():
        while not stop.is_set():
            try:
                out = subprocess.run(["rocm-smi", "--showclocks", "--showpower"], capture_output=True,
                                     text=True, timeout=10).stdout
            except (OSError, subprocess.SubprocessError):
                return
            clk = re.search(r"sclk clock level: \d+: \((\d+)Mhz\)", out)
            mclk = re.search(r"mclk clock level: \d+: \((\d+)Mhz\)", out)
            pwr = re.search(r"(?<!Max )Graphics Package Power \(W\): ([0-9.]+)", out)
            samples.append((int(clk.group(1)) if clk else None, float(pwr.group(1)) if pwr else None,
                            int(mclk.group(1)) if mclk else None))

    th = threading.Thread(target=smi, daemon=True)
    th.start()
    t0, i = time.time(), 0
    while time.time() - t0 < seconds:
        for _ in range(8):
            launch(i)
            i += 1
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    clks = sorted(c for c, _, _ in samples[1:] if c is not None)
    pwrs = sorted(p for _, p, _ in samples[1:] if p is not None)
    mclks = sorted(m for _, _, m in samples[1:] if m is not None)
    if not clks:
        return None
    return {"sclk_mhz_median": clks[len(clks) // 2], "sclk_mhz_min": clks[0], "sclk_mhz_max": clks[-1],
            "mclk_mhz_median": mclks[len(mclks) // 2] if mclks else None,
            "power_w_median": pwrs[len(pwrs) // 2] if pwrs else None, "samples": len(clks),
            "seconds": round(time.time() - t0, 2), "source": "rocm-smi --showclocks --showpower"}


def time_workload(w, steps, warmup, n_sets, device, config=binding.CONFIG_AUTO, b_layout=binding.B_KN,
                  splits=None, clock_seconds=0.0):
    """Returns (ms per step over the timed region of K back-to-back launches, mean ms per launch
    between per-launch events in a second pass, clock samples or None).  splits: None for gemm_relu / gemm_relu_ex, else the split-K entry point with
    that many parts.  clock_seconds > 0: after the timed region, keep launching for that long while
    rocm-smi samples the clock (outside the timed region)."""
    sets = make_sets(w, n_sets, device, b_layout)
    stream = torch.cuda.current_stream(device)
    dt = binding.F16 if w.dtype == "fp16" else binding.BF16
    lib = gr.load_library()
    ws, ws_bytes = None, 0
    if splits is not None:
        cfg = gr.selected_splitk_config(w.M, w.N, w.K, dt, config, splits, b_layout=b_layout)
        log(f"[bench] {w.name} split-K: {cfg}")
        if cfg["workspace_bytes"]:
            ws = binding.splitk_workspace(device, stream, cfg["workspace_bytes"])
            ws_bytes = ws.numel()

    def launch(i):
        a, b, c = sets[i % n_sets]
        if splits is None:
            rc = binding.gemm_relu_raw(a.data_ptr(), b.data_ptr(), c.data_ptr(), w.M, w.N, w.K, dt,
                                       stream.cuda_stream, config, b_layout)
        else:
            rc = lib.gemm_relu_splitk(a.data_ptr(), b.data_ptr(), c.data_ptr(), w.M, w.N, w.K, dt, b_layout,
                                      config, splits, ws.data_ptr() if ws is not None else None, ws_bytes,
                                      stream.cuda_stream or None)
        if rc != 0:
            raise binding.GemmReluError(rc, gr.strerror(rc))

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize(device)

    # Timed region: K back-to-back launches between two events, nothing else on the
    # stream.  In the kernel trace they follow each other with no gap and no
    # overlap, so the region's length over K is both the time per step and each
    # launch's average duration.
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(device)
    t0.record(stream)
    for i in range(steps):
        launch(i)
    t1.record(stream)
    torch.cuda.synchronize(device)
    step_ms = t0.elapsed_time(t1) / steps
    # Then the same K launches once more, each between its own pair of events on
    # the launch stream: the per-launch durations.  The event records add host
    # time to every launch and leave about 10 us between launches on the GPU
    # (which sets the pace of small shapes), so this pass is reported beside the
    # step time, not used as it.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        launch(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize(device)
    kernel_ms = sum(s.elapsed_time(e) for s, e in ev) / steps
    clocks = sample_clocks(launch, clock_seconds) if clock_seconds > 0 else None
    del sets
    return step_ms, kernel_ms, clocks


def time_vendor(w, steps, warmup, n_sets, device):
    """The same workload through the vendor library in one process: torch.mm (hipBLASLt on
    ROCm) alone, and followed by an in-place ReLU (two kernels).  Mean ms per step between GPU
    events.  For context only: nothing in the library uses it."""
    sets = make_sets(w, n_sets, device)
    stream = torch.cuda.current_stream(device)
    out = {}
    for name, relu in (("mm_ms", False), ("mm_relu_ms", True)):
        def step(i):
            a, b, c = sets[i % n_sets]
            torch.mm(a, b, out=c)
            if relu:
                torch.relu_(c)
        for i in range(warmup):
            step(i)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(device)
        t0.record(stream)
        for i in range(steps):
            step(i)
        t1.record(stream)
        torch.cuda.synchronize(device)
        out[name] = round(t0.elapsed_time(t1) / steps, 5)
    out["mm_tflops"] = round(w.flop / (out["mm_ms"] * 1e-3) / 1e12, 1)
    out["mm_relu_tflops"] = round(w.flop / (out["mm_relu_ms"] * 1e-3) / 1e12, 1)
    del sets
    return out


def cpu_baseline(w, target_s):
    """The CPU oracle on a bounded sample of the workload: whole rows of C."""
    import oracle
    a, b = inputs.workload_inputs(w)
    threads = len(os.sched_getaffinity(0))
    # Grow the row count until one run takes at least half the target time
    # (the first runs are short; only the last, longest run is reported).
    rows = max(1, threads)
    while True:
        t = time.perf_counter()
        ref_rows = oracle.gemm_relu_rows(a, b, w.dtype, 0, rows, threads=threads)
        dt = time.perf_counter() - t
        if dt >= 0.5 * target_s or rows >= w.M:
            break
        rows = int(min(w.M, max(rows + 1, rows * target_s / max(dt, 1e-3))))
    rows_target = rows
    flop = 2.0 * rows_target * w.N * w.K
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"rows 0..{rows_target - 1} of C ({rows_target} x {w.N} x {w.K}), "
                      f"{dt:.1f} s wall, fp64 accumulation",
            "seconds": dt}, ref_rows


def parity_rows(w, ref_rows, device, b_layout):
    """The GPU's C for the workload's seeded inputs (the oracle's), compared with the oracle's
    rows from the CPU baseline: errors and the tolerance the tests use."""
    a, b = inputs.workload_inputs(w)
    if b_layout == binding.B_NK:
        b = b.t().contiguous()
    c = binding.gemm_relu_ex(a.to(device), b.to(device), b_layout=b_layout)
    torch.cuda.synchronize(device)
    rows = ref_rows.shape[0]
    got_bits = c[:rows].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    def values(bits):
        if w.dtype == "fp16":
            return bits.view(np.float16).astype(np.float64)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    g, r = values(got_bits), values(ref_rows)
    err = np.abs(g - r)
    tol = 1e-2 + 1e-2 * np.abs(r)
    big = np.abs(r) >= 1e-2          # relative error where it means something
    return {"rows_checked": int(rows), "elements": int(err.size), "max_abs_err": float(err.max()),
            "max_rel_err_ref_ge_1e-2": float((err[big] / np.abs(r[big])).max()) if big.any() else 0.0,
            "max_err_over_tolerance": round(float((err / tol).max()), 4),
            "within_1e-2_tolerance": bool((err <= tol).all()),
            "bit_identical_fraction": round(float((got_bits == ref_rows).mean()), 6)}


def cpu_small(names=("small_256", "square_1024")):
    """The CPU oracle on the small whole workloads, with one thread and with all host cores
    (seconds of CPU in all): for scale beside the GPU's launch-bound small shapes."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    out = {}
    for name in names:
        w = inputs.WORKLOADS[name]
        a, b = inputs.workload_inputs(w)
        entry = {}
        for label, n in (("threads_1", 1), (f"threads_{threads}", threads)):
            t = time.perf_counter()
            oracle.gemm_relu(a, b, w.dtype, threads=n)
            entry[label + "_ms"] = round((time.perf_counter() - t) * 1e3, 2)
        out[name] = entry
    return out


def copy_calibration(device, n_bytes=1 << 30, reps=5):
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE per dispatch give the
    factor between those counters and true HBM bytes."""
    src = torch.ones(n_bytes // 2, dtype=torch.float16, device=device)
    dst = torch.empty_like(src)
    torch.cuda.synchronize(device)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize(device)
    ms = t0.elapsed_time(t1) / reps
    print(json.dumps({"copy_bytes_read": n_bytes, "copy_bytes_written": n_bytes, "reps": reps,
                      "ms": round(ms, 4), "GB/s": round(2 * n_bytes / (ms * 1e-3) / 1e9, 1)}), flush=True)


def main():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="square_8192", choices=sorted(inputs.WORKLOADS))
    p.add_argument("--sets", type=int, default=3, help="rotated input/output sets")
    p.add_argument("--config", type=int, default=binding.CONFIG_AUTO)
    p.add_argument("--b-layout", choices=["kn", "nk"], default="kn",
                   help="B handed over as (K, N) or as B^T, (N, K)")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true", help="skip the other workloads' timings")
    p.add_argument("--no-vendor", action="store_true",
                   help="skip timing the same workload through torch.mm (+ torch.relu_)")
    p.add_argument("--clock-seconds", type=float, default=2.0,
                   help="after the timed steps, sustain the workload this long while rocm-smi samples the "
                        "shader clock (0: skip)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    args = p.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    if args.copy_calibration:
        copy_calibration(device)
        return
    gr.load_library()

    w = inputs.WORKLOADS[args.workload]
    b_layout = binding.B_NK if args.b_layout == "nk" else binding.B_KN
    cfg = gr.selected_config(w.M, w.N, w.K, binding.F16 if w.dtype == "fp16" else binding.BF16, args.config,
                             b_layout=b_layout)
    log(f"[bench] {w.name}: config {cfg}")
    ms_step, kernel_ms_events, clocks = time_workload(w, args.steps, args.warmup, args.sets, device, args.config,
                                                      b_layout, clock_seconds=args.clock_seconds)
    log(f"[bench] clocks under sustained load: {clocks}")
    # One launch per step, back to back with no gap: the step time is the kernel's
    # average launch duration over the timed region.
    tflops = w.flop / (ms_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    log(f"[bench] {w.name}: {ms_step:.4f} ms/step, {tflops:.1f} TFLOP/s; "
        f"{kernel_ms_events:.4f} ms per launch between per-launch events")

    secondary = {}
    if not args.no_secondary:
        # (workload, B layout, kernel config, split-K parts or None for the plain entry point)
        runs = [("small_256", binding.B_KN, binding.CONFIG_AUTO, None),
                ("square_1024", binding.B_KN, binding.CONFIG_AUTO, None),
                ("square_1024", binding.B_KN, binding.CONFIG_DMA_128, None),     # the pages' 128x128x64 tile
                ("square_1024", binding.B_KN, binding.CONFIG_DMA_128, 4),
                ("ragged_4000x11000x4100", binding.B_KN, binding.CONFIG_AUTO, None),
                ("skinny_64x16384x8192", binding.B_KN, binding.CONFIG_AUTO, None),
                ("skinny_64x16384x8192", binding.B_KN, binding.CONFIG_DMA_64x256, 4),
                ("deep_512x512x16384", binding.B_KN, binding.CONFIG_AUTO, None),
                ("deep_512x512x16384", binding.B_KN, binding.CONFIG_AUTO, 0),
                ("square_8192", binding.B_NK, binding.CONFIG_AUTO, None),
                ("square_8192_bf16", binding.B_KN, binding.CONFIG_AUTO, None),
                ("square_8192", binding.B_KN, binding.CONFIG_DMA_256x128_WS, None)]
        for name, s_layout, s_config, s_splits in runs:
            sw = inputs.WORKLOADS[name]
            if (sw.name == w.name and s_splits is None and s_config == binding.CONFIG_AUTO and
                    args.b_layout == ("nk" if s_layout == binding.B_NK else "kn")):
                continue
            s_ms, s_kms, _ = time_workload(sw, 50 if sw.flop < 1e12 else 20, 50, 3, device, config=s_config,
                                           b_layout=s_layout, splits=s_splits)
            if s_layout == binding.B_NK:
                name += "_b_nk"
            if s_splits is not None:
                name += "_splitk" if s_config == binding.CONFIG_AUTO else f"_splitk{s_splits}_config{s_config}"
            elif s_config != binding.CONFIG_AUTO:
                name += "_" + binding.CONFIG_NAMES[s_config]
            entry = {"ms": round(s_kms, 5), "ms_per_step_batch": round(s_ms, 5),
                     "TFLOP/s": round(sw.flop / (s_kms * 1e-3) / 1e12, 2),
                     "frac_mfma_peak": round(sw.flop / (s_kms * 1e-3) / 1e12 / PEAK_TFLOPS[sw.dtype], 4),
                     "GB/s": round(sw.bytes_once / (s_kms * 1e-3) / 1e9, 1)}
            entry["frac_hbm_peak"] = round(entry["GB/s"] / PEAK_HBM_GBS, 4)
            if not args.no_vendor and s_layout == binding.B_KN and s_config == binding.CONFIG_AUTO and s_splits is None:
                # The same workload through torch.mm + torch.relu_ in this process, per step
                # (back-to-back launches, launch gaps included on both sides, no per-launch
                # events on either): context, not a target.
                v = time_vendor(sw, 50 if sw.flop < 1e12 else 20, 50, 3, device)
                entry["vendor_mm_relu_ms"] = v["mm_relu_ms"]
                entry["fused_step_vs_mm_relu"] = round(v["mm_relu_ms"] / s_ms, 3)
            secondary[name] = entry
            log(f"[bench] {name}: {entry}")

    vendor = None
    if not args.no_vendor:
        vendor = time_vendor(w, args.steps, args.warmup, args.sets, device)
        # Both timed the same way: back-to-back steps, no per-launch events.
        vendor["fused_step_vs_mm_relu"] = round(vendor["mm_relu_ms"] / ms_step, 3)
        log(f"[bench] vendor library (torch.mm, then torch.relu_): {vendor}")

    cpu = parity = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        cpu, ref_rows = cpu_baseline(w, args.cpu_seconds)
        log(f"[bench] CPU oracle: {cpu}")
        cpu.pop("seconds", None)
        parity = parity_rows(w, ref_rows, device, b_layout)
        log(f"[bench] GPU against the oracle's rows: {parity}")
        cpu["small_workloads"] = cpu_small()
        log(f"[bench] CPU oracle, small whole workloads: {cpu['small_workloads']}")

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_per_launch_between_events": round(kernel_ms_events, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "accumulate": "fp32",
                   "input_dist": f"N(0,1)*{w.scale}", "kernel": binding.CONFIG_NAMES.get(cfg["config_id"]),
                   "block": [cfg["block_m"], cfg["block_n"], cfg["block_k"]], "stages": cfg["stages"],
                   "grid": cfg["grid"], "rotated_sets": args.sets, "b_layout": args.b_layout},
        "frac_of_peak": round(tflops / peak, 4),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4),
                     "traffic": (measured_traffic(w.name, binding.CONFIG_NAMES.get(cfg["config_id"]))
                                 if b_layout == binding.B_KN else None)},
        "cpu_baseline": cpu,
        "parity": parity,
        "kernel_source_sha256": kernel_source_digest(),
        "clocks": clocks,
        "vendor_reference": vendor,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
