"""gemm_relu_splitk_noalloc (split-K with the library's static device scratch) against
gemm_relu_splitk (split-K with a caller-owned workspace), through the C ABI.

Both run the same kernels with the same number of parts, so their results must be
bit-identical on any input; on integer-valued inputs both must also equal the oracle.
Two calls in a row share the scratch, the second with a smaller input, so stale
counters or partials of the first would show in the second.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import tiled_dense_gemm_relu_amd as gr
from tiled_dense_gemm_relu_amd import binding, inputs

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def with_workspace(a, b, layout, config, splits):
    return bits(gr.gemm_relu_splitk(a, b, b_layout=layout, config=config, splits=splits))


def without_workspace(a, b, layout, config, splits):
    return bits(gr.gemm_relu_splitk_noalloc(a, b, b_layout=layout, config=config, splits=splits))


# (M, N, K, dtype, config, parts): the first of each pair is the larger call.
CASES = [
    [(512, 512, 16384, "fp16", binding.CONFIG_AUTO, 0), (256, 320, 4160, "fp16", binding.CONFIG_AUTO, 0)],
    [(64, 16384, 8192, "bf16", binding.CONFIG_DMA_64x256, 4), (64, 4096, 2048, "bf16", binding.CONFIG_DMA_64x256, 2)],
    [(1024, 1024, 1024, "fp16", binding.CONFIG_DMA_128, 4), (520, 392, 1000, "fp16", binding.CONFIG_DMA_128, 3)],
]
DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


@pytest.mark.parametrize("layout", [binding.B_KN, binding.B_NK])
@pytest.mark.parametrize("pair", range(len(CASES)))
def test_noalloc_matches_workspace_entry_point_twice(pair, layout):
    for integer in (True, False):
        for (M, N, K, dt, config, parts) in CASES[pair]:
            code = gr.F16 if dt == "fp16" else gr.BF16
            cfg = gr.selected_splitk_config(M, N, K, dtype=code, config=config, splits=parts, b_layout=layout)
            assert cfg["splits"] > 1 and cfg["workspace_bytes"] <= binding.NOALLOC_SCRATCH_BYTES
            say(f"[noalloc] {M}x{N}x{K} {dt} layout={layout} config={cfg['config_id']} "
                f"parts={cfg['splits']} integer={integer}")
            if integer:
                a, b = inputs.integer_pair(M, N, K, DT[dt], seed=M + N + K)
            else:
                a, b = inputs.normal_pair(M, N, K, DT[dt], 0.05, M + N + K)
            bd = b.t().contiguous() if layout == binding.B_NK else b
            ad, bd = a.cuda(), bd.cuda()
            got = without_workspace(ad, bd, layout, config, parts)
            want = with_workspace(ad, bd, layout, config, parts)
            bad = np.argwhere(got != want)
            assert bad.size == 0, f"{len(bad)} differ from gemm_relu_splitk, first at {tuple(bad[0])}"
            if integer:
                rows = [0, M // 2, M - 1]
                ref = np.concatenate([oracle.gemm_relu_rows(a, b, dt, r, r + 1) for r in rows])
                assert np.array_equal(got[rows], ref)


def test_noalloc_unsplit_and_refused_calls_leave_c_as_documented():
    # A shape that resolves to one part runs gemm_relu_ex; a call beyond the scratch is refused
    # before launch and leaves C untouched.
    a, b = inputs.integer_pair(300, 264, 96, torch.float16, seed=5)
    want = oracle.gemm_relu(a, b, "fp16")
    c = gr.gemm_relu_splitk_noalloc(a.cuda(), b.cuda(), splits=1)
    assert np.array_equal(bits(c), want)
    M, N, K = 8192, 8192, 1024
    ad = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    bd = torch.zeros((K, N), dtype=torch.float16, device="cuda")
    cd = torch.full((M, N), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(binding.GemmReluError) as e:
        gr.gemm_relu_splitk_noalloc(ad, bd, out=cd, config=binding.CONFIG_DMA_128, splits=2)
    assert e.value.code == -11
    torch.cuda.synchronize()
    assert bool((cd == 7.0).all())
