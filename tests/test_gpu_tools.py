"""The layout-ablation program: the 256x256x64 LDS-DMA kernel with and without
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
