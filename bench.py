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
    """Bytes per launch beyond L2 (FETCH_SIZE: what the L2s fetch on misses, from the MALL or HBM,
    plus WRITE_SIZE) from the committed rocprofv3 runs, scaled by the copy-kernel calibration;
    None unless they were taken on this workload, this kernel and the current kernel sources."""
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


def make_sets(w, n_sets, device, b_layout=binding.B_KN, data="normal"):
    sets = []
    for i in range(n_sets):
        if data == "integer":
            a, b = inputs.integer_pair(w.M, w.N, w.K, w.torch_dtype, w.int_seed + 1000 * i)
        elif data == "zero":
            a = torch.zeros((w.M, w.K), dtype=w.torch_dtype)
            b = torch.zeros((w.K, w.N), dtype=w.torch_dtype)
        else:
            a, b = inputs.normal_pair(w.M, w.N, w.K, w.torch_dtype, w.scale, w.seed + 1000 * i)
        if b_layout == binding.B_NK:
            b = b.t().contiguous()          # handed over as B^T, (N, K)
        c = torch.empty((w.M, w.N), dtype=w.torch_dtype, device=device)
        sets.append((a.to(device), b.to(device), c))
    return sets


def _gpu_sysfs_dir(pci_addr=None, root="/sys/class/drm"):
    """The sysfs device directory of the measured GPU: among the AMD cards with a shader-clock
    table, the one whose PCI address ("dddd:bb:dd.f", the name of the device directory the card's
    link points to) is `pci_addr`, else the first of them; None if there is none."""
    import glob
    cards = []
    for d in sorted(glob.glob(os.path.join(root, "card*", "device"))):
        try:
            if open(os.path.join(d, "vendor")).read().strip() == "0x1002" and \
                    os.path.exists(os.path.join(d, "pp_dpm_sclk")):
                cards.append(d)
        except OSError:
            continue
    if pci_addr:
        for d in cards:
            if os.path.basename(os.path.realpath(d)).lower() == pci_addr.lower():
                return d
    return cards[0] if cards else None


def _device_pci_addr():
    """The PCI address of the current GPU as sysfs names it, from torch's device properties, or None
    (no GPU, or a torch without those fields)."""
    try:
        if not torch.cuda.is_available():
            return None
        p = torch.cuda.get_device_properties(torch.cuda.current_device())
        return f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
    except (AttributeError, RuntimeError):
        return None


_SYSFS = None


def read_clocks():
    """Current shader and memory clock (MHz) and package power (W) from the driver's sysfs files:
    the active level of pp_dpm_sclk / pp_dpm_mclk (the level marked '*'; on these boards the
    middle level carries the live frequency) and hwmon power1_average or power1_input.  A field
    the board does not report is "unavailable"."""
    global _SYSFS
    if _SYSFS is None:
        _SYSFS = _gpu_sysfs_dir(_device_pci_addr()) or ""
    out = {"sclk_mhz": "unavailable", "mclk_mhz": "unavailable", "power_w": "unavailable"}
    if not _SYSFS:
        return out
    for key, name in (("sclk_mhz", "pp_dpm_sclk"), ("mclk_mhz", "pp_dpm_mclk")):
        try:
            for line in open(os.path.join(_SYSFS, name)):
                if line.rstrip().endswith("*"):
                    m = re.search(r"(\d+)\s*Mhz", line, re.I)
                    if m:
                        out[key] = int(m.group(1))
        except OSError:
            pass
    import glob
    for f in sorted(glob.glob(os.path.join(_SYSFS, "hwmon", "hwmon*", "power1_average")) +
                    glob.glob(os.path.join(_SYSFS, "hwmon", "hwmon*", "power1_input"))):
        try:
            uw = int(open(f).read().strip())
        except (OSError, ValueError):
            continue
        if uw > 0:
            out["power_w"] = round(uw / 1e6, 1)
            break
    return out


def read_power_cap():
    """The board's package power limit in W (hwmon power1_cap), or "unavailable"."""
    import glob
    global _SYSFS
    if _SYSFS is None:
        _SYSFS = _gpu_sysfs_dir(_device_pci_addr()) or ""
    if not _SYSFS:
        return "unavailable"
    for f in sorted(glob.glob(os.path.join(_SYSFS, "hwmon", "hwmon*", "power1_cap"))):
        try:
            return round(int(open(f).read().strip()) / 1e6, 1)
        except (OSError, ValueError):
            continue
    return "unavailable"


def power_clock_context(tflops, peak, sustained):
    """The throughput against the MFMA peak at the shader clock the board sustained on this workload
    (peak x sclk / 2400 MHz), beside the package power and its cap: on normal fp16 data the board
    lowers the clock to hold its power limit."""
    if not sustained or isinstance(sustained.get("sclk_mhz"), str):
        return {"sustained_sclk_mhz": "unavailable", "power_cap_w": read_power_cap()}
    sclk = sustained["sclk_mhz"]["median"]
    pw = sustained["power_w"]
    return {"sustained_sclk_mhz": sclk, "peak_at_sustained_sclk": round(peak * sclk / 2400.0, 1),
            "frac_of_peak_at_sustained_sclk": round(tflops / (peak * sclk / 2400.0), 4),
            "sustained_power_w": pw["median"] if isinstance(pw, dict) else pw, "power_cap_w": read_power_cap()}


def sample_clocks(launch, seconds, interval=0.02):
    """Keep the GPU busy with `launch` for about `seconds` while the clocks (and power, where the
    board reports it) are read every `interval` s.  Returns medians and ranges over the samples."""
    samples, stop = [], threading.Event()

    def reader():
        while not stop.is_set():
            samples.append(read_clocks())
            time.sleep(interval)

    th = threading.Thread(target=reader, daemon=True)
    th.start()
    t0, i = time.time(), 0
    while time.time() - t0 < seconds:
        for _ in range(8):
            launch(i)
            i += 1
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=5)
    n_skip = len(samples) // 10                  # the first tenth: the clock still settling
    body = samples[n_skip:] or samples

    def summary(key):
        vals = sorted(v[key] for v in body if not isinstance(v[key], str))
        if not vals:
            return "unavailable"
        return {"median": vals[len(vals) // 2], "min": vals[0], "max": vals[-1]}

    return {"sclk_mhz": summary("sclk_mhz"), "mclk_mhz": summary("mclk_mhz"), "power_w": summary("power_w"),
            "samples": len(body), "seconds": round(time.time() - t0, 2),
            "source": "sysfs pp_dpm_sclk / pp_dpm_mclk, hwmon power1_*"}


def time_workload(w, steps, warmup, n_sets, device, config=binding.CONFIG_AUTO, b_layout=binding.B_KN,
                  splits=None, repeats=1, per_launch_pass=False, clock_seconds=0.0, data="normal",
                  warmup_seconds=0.0):
    """Time one workload.  After `warmup` untimed launches, `repeats` timed regions of exactly
    `steps` back-to-back launches each, every region bracketed by a device synchronisation and a
    pair of GPU events on the launch stream.  Returns a dict with the median region's ms per step
    and every region's, the clocks read right before the first and right after the last region,
    optionally the mean ms per launch of a pass with a pair of events around every launch, and,
    with clock_seconds > 0, clocks sampled while the workload runs on for that long (outside the
    timed regions).  splits: None for gemm_relu / gemm_relu_ex, else the split-K entry point with
    that many parts.  data: "normal" (the workload's N(0, 1) * scale inputs), "integer" (its
    integer-valued variant) or "zero".  warmup_seconds > 0: after the `warmup` launches, further
    untimed launches in batches of `steps` until that much wall time has passed, so that the
    shader clock has settled at this workload's level before the first timed region."""
    sets = make_sets(w, n_sets, device, b_layout, data)
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

    t_warm = time.perf_counter()
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize(device)
    warmup_launches = warmup
    while time.perf_counter() - t_warm < warmup_seconds:
        for i in range(steps):
            launch(i)
        torch.cuda.synchronize(device)
        warmup_launches += steps

    # Timed regions: K back-to-back launches between two events, nothing else on the stream.
    # In the kernel trace they follow each other with no gap and no overlap, so a region's
    # length over K is both the time per step and each launch's average duration.
    # The clocks are read from the host while the first and the last region run on the GPU
    # (after their launches are queued, before the synchronisation that ends them).
    region_ms, before, after = [], None, None
    for r in range(repeats):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(device)
        t0.record(stream)
        for i in range(steps):
            launch(i)
        t1.record(stream)
        if r == 0:
            before = read_clocks()
        if r == repeats - 1:
            after = read_clocks()
        torch.cuda.synchronize(device)
        region_ms.append(t0.elapsed_time(t1) / steps)
    out = {"ms_per_step": sorted(region_ms)[len(region_ms) // 2], "region_ms_per_step": region_ms,
           "clocks_first_region": before, "clocks_last_region": after, "warmup_launches": warmup_launches}
    if per_launch_pass:
        # The same K launches once more, each between its own pair of events on the launch
        # stream.  The event records add host time to every launch and leave about 10 us
        # between launches on the GPU, which sets the pace of the small shapes.
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record(stream)
            launch(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize(device)
        out["ms_per_launch_between_events"] = sum(s.elapsed_time(e) for s, e in ev) / steps
    if clock_seconds > 0:
        out["clocks_sustained"] = sample_clocks(launch, clock_seconds)
    del sets
    return out


def cpu_baseline(w, target_s, data="normal"):
    """The CPU oracle on a bounded sample of the workload: whole rows of C."""
    import oracle
    a, b = inputs.workload_inputs(w, data == "integer")
    if data == "zero":
        a, b = torch.zeros_like(a), torch.zeros_like(b)
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


def parity_rows(w, ref_rows, device, b_layout, config=binding.CONFIG_AUTO, splits=None, data="normal"):
    """The GPU's C for the workload's seeded inputs (the oracle's), through the entry point and
    kernel the bench timed, compared with the oracle's rows from the CPU baseline: errors and the
    tolerance the tests use."""
    a, b = inputs.workload_inputs(w, data == "integer")
    if data == "zero":
        a, b = torch.zeros_like(a), torch.zeros_like(b)
    if b_layout == binding.B_NK:
        b = b.t().contiguous()
    if splits is None:
        c = binding.gemm_relu_ex(a.to(device), b.to(device), b_layout=b_layout, config=config)
    else:
        c = binding.gemm_relu_splitk(a.to(device), b.to(device), b_layout=b_layout, config=config, splits=splits)
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
    p.add_argument("--repeats", type=int, default=5,
                   help="timed regions of --steps launches each; the median region is reported")
    p.add_argument("--workload", default="square_8192", choices=sorted(inputs.WORKLOADS))
    p.add_argument("--sets", type=int, default=3, help="rotated input/output sets")
    p.add_argument("--config", type=int, default=binding.CONFIG_AUTO)
    p.add_argument("--b-layout", choices=["kn", "nk"], default="kn",
                   help="B handed over as (K, N) or as B^T, (N, K)")
    p.add_argument("--splits", type=int, default=None,
                   help="time the split-K entry point with this many parts (0: the library chooses) "
                        "instead of gemm_relu")
    p.add_argument("--data", choices=["normal", "integer", "zero"], default="normal",
                   help="the workload's N(0, 1) * scale inputs, its integer-valued variant, or zeros (the "
                        "last two draw less power: for clock and power comparisons, not the metric)")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true", help="skip the other workloads' timings")
    p.add_argument("--clock-seconds", type=float, default=2.0,
                   help="after the timed steps, sustain the workload this long while the shader clock "
                        "is sampled (0: skip)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    args = p.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; "
              "run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.repeats < 1 or args.warmup < 0:
        print("bench.py: --steps and --repeats must be >= 1, --warmup >= 0", file=sys.stderr)
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
    dt = binding.F16 if w.dtype == "fp16" else binding.BF16
    if args.splits is None:
        cfg = gr.selected_config(w.M, w.N, w.K, dt, args.config, b_layout=b_layout)
    else:
        cfg = gr.selected_splitk_config(w.M, w.N, w.K, dt, args.config, args.splits, b_layout=b_layout)
    log(f"[bench] {w.name}: config {cfg}")
    head = time_workload(w, args.steps, args.warmup, args.sets, device, args.config, b_layout,
                         splits=args.splits, repeats=args.repeats, clock_seconds=args.clock_seconds,
                         data=args.data)
    ms_step = head["ms_per_step"]
    # One launch per step, back to back with no gap: the step time is the kernel's
    # average launch duration over the timed region.
    tflops = w.flop / (ms_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    log(f"[bench] {w.name}: median {ms_step:.4f} ms/step over {args.repeats} regions "
        f"{[round(x, 4) for x in head['region_ms_per_step']]}, {tflops:.1f} TFLOP/s; "
        f"clocks in the first region {head['clocks_first_region']}, in the last {head['clocks_last_region']}")
    log(f"[bench] clocks under sustained load: {head.get('clocks_sustained')}")

    secondary = {}
    if not args.no_secondary:
        # (workload, B layout, kernel config, split-K parts or None for the plain entry point)
        runs = [("small_256", binding.B_KN, binding.CONFIG_AUTO, None),
                ("square_1024", binding.B_KN, binding.CONFIG_AUTO, None),
                ("square_1024", binding.B_KN, binding.CONFIG_DMA_128, None),     # the pages' 128x128x64 tile
                ("ragged_4000x11000x4100", binding.B_KN, binding.CONFIG_AUTO, None),
                ("skinny_64x16384x8192", binding.B_KN, binding.CONFIG_AUTO, None),
                ("skinny_64x16384x8192", binding.B_NK, binding.CONFIG_AUTO, None),
                ("skinny_64x16384x8192", binding.B_KN, binding.CONFIG_DMA_64x256, 4),
                ("wide_decode_64x65536x2048", binding.B_KN, binding.CONFIG_AUTO, None),
                ("wide_decode_64x65536x2048", binding.B_NK, binding.CONFIG_AUTO, None),
                ("deep_512x512x16384", binding.B_KN, binding.CONFIG_AUTO, None),
                ("deep_512x512x16384", binding.B_KN, binding.CONFIG_AUTO, 0),
                ("square_2048", binding.B_KN, binding.CONFIG_AUTO, None),
                ("square_8192", binding.B_NK, binding.CONFIG_AUTO, None),
                ("square_8192_bf16", binding.B_KN, binding.CONFIG_AUTO, None)]
        for name, s_layout, s_config, s_splits in runs:
            sw = inputs.WORKLOADS[name]
            if (sw.name == w.name and s_splits == args.splits and s_config == args.config and
                    args.b_layout == ("nk" if s_layout == binding.B_NK else "kn") and args.data == "normal"):
                continue
            r = time_workload(sw, 50 if sw.flop < 1e12 else 20, 50, 3, device, config=s_config,
                              b_layout=s_layout, splits=s_splits, repeats=3, per_launch_pass=True,
                              warmup_seconds=0.25)
            s_ms, s_kms = r["ms_per_step"], r["ms_per_launch_between_events"]
            if s_layout == binding.B_NK:
                name += "_b_nk"
            if s_splits is not None:
                name += "_splitk" if s_config == binding.CONFIG_AUTO else f"_splitk{s_splits}_config{s_config}"
            elif s_config != binding.CONFIG_AUTO:
                name += "_" + binding.CONFIG_NAMES[s_config]
            # Rates from the back-to-back step time (the median of 3 regions).  On the small
            # shapes the gap between back-to-back launches is part of it; the per-launch time
            # between events is given beside it.
            entry = {"ms_per_step": round(s_ms, 5), "ms_per_launch_between_events": round(s_kms, 5),
                     "TFLOP/s": round(sw.flop / (s_ms * 1e-3) / 1e12, 2),
                     "frac_mfma_peak": round(sw.flop / (s_ms * 1e-3) / 1e12 / PEAK_TFLOPS[sw.dtype], 4),
                     "GB/s": round(sw.bytes_once / (s_ms * 1e-3) / 1e9, 1),
                     "sclk_mhz_last_region": r["clocks_last_region"]["sclk_mhz"],
                     "warmup_launches": r["warmup_launches"]}
            entry["frac_hbm_peak"] = round(entry["GB/s"] / PEAK_HBM_GBS, 4)
            secondary[name] = entry
            log(f"[bench] {name}: {entry}")

    cpu = parity = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        cpu, ref_rows = cpu_baseline(w, args.cpu_seconds, args.data)
        log(f"[bench] CPU oracle: {cpu}")
        cpu.pop("seconds", None)
        parity = parity_rows(w, ref_rows, device, b_layout, args.config, args.splits, args.data)
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
        "repeats": args.repeats,
        "ms_per_step": round(ms_step, 5),
        "region_ms_per_step": [round(x, 5) for x in head["region_ms_per_step"]],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "accumulate": "fp32",
                   "input_dist": {"normal": f"N(0,1)*{w.scale}", "integer": "integers uniform in [-2, 2]",
                                  "zero": "zeros"}[args.data],
                   "kernel": binding.CONFIG_NAMES.get(cfg["config_id"]), "splits": cfg["splits"],
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
        "clocks": {"first_timed_region": head["clocks_first_region"],
                   "last_timed_region": head["clocks_last_region"], "sustained": head.get("clocks_sustained")},
        "power_clock": power_clock_context(tflops, peak, head.get("clocks_sustained")),
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
