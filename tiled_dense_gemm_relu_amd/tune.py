"""Offline tile-configuration search and the per-shape table the library compiles in.

For each shape (M, N, K, dtype, B layout) this times every kernel configuration
the library can run for it -- the plain entry point's configurations and the
split-K ones with 2 to 16 parts -- and records the fastest of each kind.  The
search follows the two steps the TileLang GEMM article on zwxr.cn describes for
its autotuner (its section 4.3): a short benchmark of every candidate as a
prefilter, then a longer one of the few best.  Each benchmark times back-to-back
launches on three rotated input sets, as the bench does, so that a choice holds
for calls that follow each other; the candidates of a stage run their timed
regions in alternating rounds, so that the shader clock's drift reaches all of
them alike, and each is given its median region.

Output:
  * ``csrc/tuned_table.inc``: one C initialiser per shape, included by
    gemm_relu_api.hip; GEMM_RELU_CONFIG_AUTO uses it for an exact shape match
    (with pointers aligned as the tuner's were), the heuristics otherwise;
  * a JSON report with every timing (``--report``).

Run it on the GPU the table is for (an MI355X, gfx950), then rebuild:
    python -m tiled_dense_gemm_relu_amd.tune --report tuning.json
    python -m tiled_dense_gemm_relu_amd.build
"""
from __future__ import annotations

import argparse
import datetime
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
TABLE = os.path.join(PKG, "csrc", "tuned_table.inc")

SPLIT_CONFIGS = (4, 5, 6)          # the kernels that have split-K variants
SPLIT_PARTS = (2, 4, 8, 16)
PREFILTER_LAUNCHES = 5
PREFILTER_REGIONS = 3
FINAL_LAUNCHES = 30
FINAL_REGIONS = 7
BEAM = 3
# A split-K entry is kept only if it beats the plain choice by this factor
# (it costs a workspace).
SPLIT_MARGIN = 0.97
# The plain configuration AUTO resolves to before the search (the table entry
# or, for a new shape, the size rules) is kept unless another one beats it by
# this factor, so that re-tuning does not flip choices on noise.
PLAIN_MARGIN = 0.98
MAX_WORKSPACE = 256 << 20          # split-K candidates needing more are not tried


def default_shapes():
    from . import inputs
    shapes = []
    for w in inputs.WORKLOADS.values():
        for layout in (0, 1):
            shapes.append((w.M, w.N, w.K, w.dtype, layout))
    for n in (512, 2048, 4096):
        if (n, n, n, "fp16", 0) not in shapes:
            shapes.append((n, n, n, "fp16", 0))
    return shapes


def parse_shape(text):
    parts = text.split(",")
    M, N, K = (int(p) for p in parts[:3])
    dtype = parts[3] if len(parts) > 3 else "fp16"
    layout = {"kn": 0, "nk": 1}[parts[4]] if len(parts) > 4 else 0
    return M, N, K, dtype, layout


def candidates(M, N, K, dt, layout):
    """Distinct (config_id, splits) pairs the library resolves requests to."""
    from . import binding
    seen = {}
    for cfg in range(0, binding.CONFIG_DMA_128x128_WS + 1):
        r = binding.selected_config(M, N, K, dt, cfg, b_layout=layout)
        if r["config_id"] == binding.CONFIG_DIRECT and cfg != binding.CONFIG_DIRECT:
            continue
        seen[(r["config_id"], 1)] = cfg
    for cfg in SPLIT_CONFIGS:
        for s in SPLIT_PARTS:
            r = binding.selected_splitk_config(M, N, K, dt, cfg, s, b_layout=layout)
            if r["splits"] > 1 and r["workspace_bytes"] <= MAX_WORKSPACE:
                seen[(r["config_id"], r["splits"])] = cfg
    # The direct kernel only competes when nothing else can run.
    if len(seen) > 1:
        seen.pop((binding.CONFIG_DIRECT, 1), None)
    return sorted(seen)


def make_launcher(sets, M, N, K, dt, layout, config, splits, ws):
    """One call of the candidate on input set i % len(sets), on the current stream."""
    import torch
    from . import binding
    lib = binding.load_library()
    stream = torch.cuda.current_stream()

    def launch(i):
        a, b, c = sets[i % len(sets)]
        if splits == 1:
            rc = lib.gemm_relu_ex(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, dt, layout, config,
                                  stream.cuda_stream or None)
        else:
            rc = lib.gemm_relu_splitk(a.data_ptr(), b.data_ptr(), c.data_ptr(), M, N, K, dt, layout, config,
                                      splits, ws.data_ptr(), ws.numel(), stream.cuda_stream or None)
        if rc != 0:
            raise binding.GemmReluError(rc, binding.strerror(rc))
    return launch


def time_region(launch, launches):
    """`launches` back-to-back launches between two events on the launch stream, as the bench
    times a step; returns the time per launch, ms."""
    import torch
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(launches):
        launch(i)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / launches


def time_alternating(launchers, launches, regions):
    """Every candidate warmed up, then `regions` rounds in which each candidate runs one timed
    region in turn, so that clock and power drift reach all of them alike.  Returns each
    candidate's median region, ms per launch."""
    for launch in launchers.values():
        for i in range(launches):
            launch(i)
    times = {c: [] for c in launchers}
    for _ in range(regions):
        for c, launch in launchers.items():
            times[c].append(time_region(launch, launches))
    return {c: sorted(t)[len(t) // 2] for c, t in times.items()}


def choose_plain(final, incumbent, margin=PLAIN_MARGIN):
    """The plain (unsplit) configuration to record, from the final timings
    {(config, parts): ms}: the fastest, unless the incumbent configuration was
    timed and the fastest does not beat it by `margin`.  Returns (ms, (config, 1))."""
    best = min((t, c) for c, t in final.items() if c[1] == 1)
    inc = (incumbent, 1)
    if inc in final and best[0] >= margin * final[inc]:
        return final[inc], inc
    return best


def tune_shape(M, N, K, dtype, layout, log):
    import torch
    from . import binding, inputs
    dt = binding.F16 if dtype == "fp16" else binding.BF16
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    sets = []
    for seed in (1, 2, 3):
        a, b = inputs.normal_pair(M, N, K, tdt, 0.1, seed)
        if layout == 1:
            b = b.t().contiguous()
        sets.append((a.cuda(), b.cuda(), torch.empty((M, N), dtype=tdt, device="cuda")))
    cands = candidates(M, N, K, dt, layout)
    need = max([binding.selected_splitk_config(M, N, K, dt, c, s, b_layout=layout)["workspace_bytes"]
                for c, s in cands if s > 1] + [256])
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    launchers = {c: make_launcher(sets, M, N, K, dt, layout, c[0], c[1], ws) for c in cands}
    pre = time_alternating(launchers, PREFILTER_LAUNCHES, PREFILTER_REGIONS)
    finalists = set()
    for kind in (lambda c: c[1] == 1, lambda c: c[1] > 1):
        finalists.update(c for _, c in sorted((t, c) for c, t in pre.items() if kind(c))[:BEAM])
    # the current AUTO choice is always timed in the final rounds, so that it can be kept
    incumbent = binding.selected_config(M, N, K, dt, binding.CONFIG_AUTO, b_layout=layout)["config_id"]
    if (incumbent, 1) in pre:
        finalists.add((incumbent, 1))
    final = time_alternating({c: launchers[c] for c in sorted(finalists)}, FINAL_LAUNCHES, FINAL_REGIONS)
    plain = choose_plain(final, incumbent)
    split = min(((t, c) for c, t in final.items() if c[1] > 1), default=None)
    entry = {"M": M, "N": N, "K": K, "dtype": dtype, "b_layout": layout, "config": plain[1][0],
             "config_ms": plain[0], "splitk_config": plain[1][0], "splits": 1, "splitk_ms": plain[0],
             "incumbent": incumbent,
             "prefilter_ms": {f"{c}x{s}": round(t, 5) for (c, s), t in pre.items()},
             "final_ms": {f"{c}x{s}": round(t, 5) for (c, s), t in final.items()}}
    if split is not None and split[0] < SPLIT_MARGIN * plain[0]:
        entry.update(splitk_config=split[1][0], splits=split[1][1], splitk_ms=split[0])
    log(f"[tune] {M}x{N}x{K} {dtype} layout={layout}: plain config {entry['config']} "
        f"{entry['config_ms'] * 1e3:.1f} us; split-K config {entry['splitk_config']} x{entry['splits']} "
        f"{entry['splitk_ms'] * 1e3:.1f} us ({len(cands)} candidates)")
    del sets, ws
    return entry


def write_table(entries, device_name, path=TABLE):
    dcode = {"fp16": 0, "bf16": 1}
    lines = [f"// Generated by tiled_dense_gemm_relu_amd/tune.py on {device_name}, "
             f"{datetime.date.today().isoformat()}; regenerate rather than edit.",
             "// {M, N, K, dtype, b_layout, config, split-K config, split-K parts}"]
    for e in entries:
        lines.append(f"{{{e['M']}, {e['N']}, {e['K']}, {dcode[e['dtype']]}, {e['b_layout']}, {e['config']}, "
                     f"{e['splitk_config']}, {e['splits']}}},")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--shape", action="append", default=[], help="M,N,K[,fp16|bf16[,kn|nk]] (repeatable)")
    p.add_argument("--out", default=TABLE, help="C table to write")
    p.add_argument("--report", default=None, help="JSON report with every timing")
    args = p.parse_args()
    import torch
    if not torch.cuda.is_available():
        sys.exit("tune.py needs the GPU the table is for")
    name = torch.cuda.get_device_properties(0).gcnArchName
    if not name.startswith("gfx950"):
        sys.exit(f"tune.py tunes for gfx950, found {name}")
    shapes = [parse_shape(s) for s in args.shape] or default_shapes()
    log = lambda m: print(m, file=sys.stderr, flush=True)
    entries = [tune_shape(*s, log) for s in shapes]
    write_table(entries, f"{torch.cuda.get_device_name(0)} ({name})", args.out)
    if args.report:
        with open(args.report, "w") as f:
            json.dump({"device": torch.cuda.get_device_name(0), "arch": name, "entries": entries}, f, indent=1)
    log(f"[tune] wrote {args.out}")


if __name__ == "__main__":
    main()
