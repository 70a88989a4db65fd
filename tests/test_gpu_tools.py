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
