"""The measurement programs.  The layout-ablation program: the 256x256x64 LDS-DMA kernel with and without
its XOR swizzle, and without its XCD remap, must give bit-identical C (the
swizzle moves bytes within LDS, never values between them; the remap changes
only which workgroup computes which tile)."""
import json
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

PROGRAM = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tiled_dense_gemm_relu_amd",
                       "layout_ablation")


def test_layout_ablation_outputs_identical():
    if not os.path.exists(PROGRAM):
        pytest.fail(f"{PROGRAM} is missing: build it with python -m tiled_dense_gemm_relu_amd.build")
    res = subprocess.run([PROGRAM], capture_output=True, text=True, timeout=180)
    assert res.returncode == 0, res.stderr
    lines = [json.loads(l) for l in res.stdout.splitlines() if l.startswith("{")]
    rounds = [l for l in lines if "round" in l]
    assert len(rounds) == 4
    assert all(r[f"{v}_tflops"] > 0 for r in rounds for v in ("product", "unswizzled", "no_remap"))
    assert lines[-1] == {"outputs_identical": True}


def test_lds_read_rates():
    """The LDS read-rate mode: each of the three fragment reads reports a rate, and a 16-byte read
    moves more bytes per second than the 8-byte transposed read that B stored (K, N) needs."""
    if not os.path.exists(PROGRAM):
        pytest.fail(f"{PROGRAM} is missing: build it with python -m tiled_dense_gemm_relu_amd.build")
    res = subprocess.run([PROGRAM, "--lds-rates"], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    lines = [json.loads(l) for l in res.stdout.splitlines() if l.startswith("{")]
    assert sorted({l["lds_read"] for l in lines}) == ["ds_read_b128", "ds_read_b64", "ds_read_b64_tr_b16"]
    best = {name: max(l["gb_per_s_per_cu"] for l in lines if l["lds_read"] == name) for name in
            ("ds_read_b128", "ds_read_b64", "ds_read_b64_tr_b16")}
    assert all(v > 0 for v in best.values())
    assert best["ds_read_b128"] > best["ds_read_b64_tr_b16"]


MFMA_FORM = os.path.join(os.path.dirname(PROGRAM), "mfma_form")


def test_mfma_form_program():
    """The MFMA-form measurement program: the library's 256 tile (16x16x32) and the same tile on
    32x32x16 MFMAs give bit-identical C on integer inputs, equal to exact host sums on sampled
    entries; every run reports a positive rate."""
    if not os.path.exists(MFMA_FORM):
        pytest.fail(f"{MFMA_FORM} is missing: build it with python -m tiled_dense_gemm_relu_amd.build")
    res = subprocess.run([MFMA_FORM, "--mode", "all", "--seconds", "0.3", "--rounds", "1"], capture_output=True,
                         text=True, timeout=240)
    assert res.returncode == 0, (res.stdout[-2000:], res.stderr[-2000:])
    lines = [json.loads(l) for l in res.stdout.splitlines() if l.startswith("{")]
    check = [l["check"] for l in lines if "check" in l]
    assert check == [{"bit_identical": True, "sampled": 2000, "sampled_mismatches": 0}]
    loops = [l for l in lines if l["mode"] == "mfma"]
    assert sorted((l["data"], l["shape"]) for l in loops) == [("normal", "16x16x32"), ("normal", "32x32x16"),
                                                              ("zero", "16x16x32"), ("zero", "32x32x16")]
    tiles = [l for l in lines if l["mode"] == "tile" and "form" in l]
    assert sorted(l["form"] for l in tiles) == ["16x16x32", "32x32x16"]
    assert all(l["tflops"] > 0 and l["launches"] > 0 for l in loops + tiles)


STREAM_CEILING = os.path.join(os.path.dirname(PROGRAM), "stream_ceiling")


def test_stream_ceiling_program():
    """The skinny shape's streaming-ceiling program: three LDS-DMA read patterns and the library's
    64x64 kernel (B stored (K, N) and (N, K)) each report a positive B rate, and each timed kernel's
    C matches fp64 sums on sampled entries."""
    if not os.path.exists(STREAM_CEILING):
        pytest.fail(f"{STREAM_CEILING} is missing: build it with python -m tiled_dense_gemm_relu_amd.build")
    res = subprocess.run([STREAM_CEILING, "--reps", "5"], capture_output=True, text=True, timeout=180)
    assert res.returncode == 0, (res.stdout[-2000:], res.stderr[-2000:])
    lines = [json.loads(l) for l in res.stdout.splitlines() if l.startswith("{")]
    patterns = [l for l in lines if "pattern" in l]
    assert [l["pattern"] for l in patterns] == ["contiguous", "strips", "strips_a", "strips_pitch_plus_128"]
    kernels = [l for l in lines if "kernel" in l]
    assert [(l["b_layout"], l["workgroups"]) for l in kernels] == [("kn", 256), ("nk", 256)]
    assert all(l["b_tbs"] > 0 for l in patterns + kernels)
    assert [l["check"] for l in lines if "check" in l] == [{"b_layout": "kn", "sampled": 256, "mismatches": 0},
                                                          {"b_layout": "nk", "sampled": 256, "mismatches": 0}]


KERNEL_TIMELINE = os.path.join(os.path.dirname(PROGRAM), "kernel_timeline")


def test_kernel_timeline_program():
    """The kernel-timeline program times, per shape, the configuration AUTO picks for it; every
    workgroup records every launch, the phases are non-negative and fit inside the launch span,
    workgroup w runs on XCD w % 8 (the premise of the tile remap), and each shape's C matches
    fp64 sums on sampled entries."""
    from tiled_dense_gemm_relu_amd import binding as b
    if not os.path.exists(KERNEL_TIMELINE):
        pytest.fail(f"{KERNEL_TIMELINE} is missing: build it with python -m tiled_dense_gemm_relu_amd.build")
    res = subprocess.run([KERNEL_TIMELINE, "--reps", "5"], capture_output=True, text=True, timeout=240)
    assert res.returncode == 0, (res.stdout[-2000:], res.stderr[-2000:])
    lines = [json.loads(l) for l in res.stdout.splitlines() if l.startswith("{")]
    shapes = [l for l in lines if "shape" in l]
    assert [l["shape"] for l in shapes] == ["square_256", "square_1024", "square_2048", "skinny_64x16384x8192",
                                            "square_8192"]
    for l in shapes:
        dt = b.F16 if l["dtype"] == "fp16" else b.BF16
        chosen = b.selected_config(l["M"], l["N"], l["K"], dt)["config_id"]
        assert l["config"].startswith(f"{chosen}:"), (l["shape"], chosen, l["config"])
        phases = [l[k] for k in ("ramp_us", "first_stage_us", "k_loop_us", "epilogue_us", "store_drain_us")]
        assert all(p >= 0 for p in phases) and l["gap_us"] >= 0, l
        assert l["first_stage_us"] + l["k_loop_us"] + l["epilogue_us"] + l["store_drain_us"] <= l["span_us"] * 1.05 + 0.05
        assert 0 < l["span_us"] <= l["event_us"] * 1.5, l
        # the tile remap's premise: the hardware dispatches workgroup w to XCD w % 8
        assert l["xcd_is_wg_mod_8"] is True, l["shape"]
        assert len(l["slowest_se_per_xcd"]) == 8
    assert lines[-1]["checked"] is True
