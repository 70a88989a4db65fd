"""GPU parity for split-K (gemm_relu_splitk): each output tile's K range is cut
into parts, the parts' fp32 partial tiles are added in part order by the last
part to finish, and ReLU is applied once, after the sum (ReLU does not
distribute over a sum).  The split/combine structure follows the num_split
parameter and combine step of the MLA decode section of "Writing
High-Performance Kernels in TileLang"; the operation is still ReLU(A @ B).

Bars as for gemm_relu: bit-exact on integer-valued inputs, |C_gpu - C_ref| <=
1e-2 + 1e-2 * |C_ref| on real-valued ones; plus: the workspace counters are
back at zero after every call, and repeated calls are bit-identical.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_dense_gemm_relu_amd as gr
from tiled_dense_gemm_relu_amd import binding, inputs

from test_gpu_parity import DT, assert_within_tolerance, bits, check_relu_invariants, say

pytestmark = pytest.mark.gpu

SPLIT_CONFIGS = [binding.CONFIG_AUTO, binding.CONFIG_DMA_128, binding.CONFIG_DMA_64, binding.CONFIG_DMA_64x256]


def run_splitk(a, b, b_layout, config, splits, workspace=None):
    bb = b.t().contiguous() if b_layout == gr.B_NK else b
    c = gr.gemm_relu_splitk(a.cuda(), bb.cuda(), b_layout=b_layout, config=config, splits=splits,
                            workspace=workspace)
    torch.cuda.synchronize()
    return bits(c)


def counters_zero(ws, cfg):
    """The per-tile counters at the start of the workspace are all zero."""
    n = cfg["workspace_bytes"] - cfg["grid"] * cfg["block_m"] * cfg["block_n"] * 4
    return bool((ws[:n] == 0).all().item())


SHAPES = [(64, 64, 64), (64, 512, 1024), (100, 300, 520), (37, 1000, 776), (256, 256, 200), (130, 270, 4104),
          (64, 2048, 2048)]


@pytest.mark.parametrize("b_layout", [gr.B_KN, gr.B_NK])
@pytest.mark.parametrize("splits", [0, 2, 3, 5, 16])
@pytest.mark.parametrize("config", SPLIT_CONFIGS)
@pytest.mark.parametrize("shape", SHAPES)
def test_splitk_integer_inputs_bit_exact(shape, config, splits, b_layout):
    M, N, K = shape
    dtype = "bf16" if (M + N + K) % 2 else "fp16"
    a, b = inputs.integer_pair(M, N, K, DT[dtype], seed=M * 3 + N * 7 + K + splits)
    want = oracle.gemm_relu(a, b, dtype)
    got = run_splitk(a, b, b_layout, config, splits)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("config", SPLIT_CONFIGS)
def test_splitk_real_inputs_and_workspace_reuse(config):
    M, N, K = 96, 1536, 2048
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    outs = []
    for seed in (1, 2, 1):
        a, b = inputs.normal_pair(M, N, K, torch.float16, 0.5, seed)
        got = run_splitk(a, b, gr.B_KN, config, 4, workspace=ws)
        cfg = gr.selected_splitk_config(M, N, K, config=config, splits=4)
        assert cfg["splits"] == 4
        assert counters_zero(ws, cfg)
        check_relu_invariants(got, "fp16")
        assert_within_tolerance(got, oracle.gemm_relu(a, b, "fp16"), "fp16")
        outs.append(got)
    assert np.array_equal(outs[0], outs[2])          # same inputs, same bits


def test_splitk_workspace_shared_across_shapes():
    # One workspace for calls whose tile counts grow and shrink: the partial
    # tiles of one call must never be taken for another call's counters.
    ws = torch.zeros(32 << 20, dtype=torch.uint8, device="cuda")
    for M, N, K, config in [(64, 512, 1024, 4), (64, 2048, 2048, 5), (64, 256, 512, 6), (128, 4096, 512, 5),
                            (64, 2048, 2048, 5), (200, 296, 1000, 4)]:
        a, b = inputs.integer_pair(M, N, K, torch.float16, seed=M + N + K)
        cfg = gr.selected_splitk_config(M, N, K, config=config)
        assert cfg["splits"] > 1 and cfg["workspace_bytes"] <= ws.numel()
        assert np.array_equal(run_splitk(a, b, gr.B_KN, config, 0, workspace=ws), oracle.gemm_relu(a, b, "fp16"))
        assert counters_zero(ws, cfg)


def test_splitk_matches_integer_results_of_the_plain_kernel():
    a, b = inputs.integer_pair(64, 4096, 4096, torch.bfloat16, seed=5)
    plain = bits(gr.gemm_relu(a.cuda(), b.cuda()))
    for splits in (2, 4, 8, 32):
        assert np.array_equal(run_splitk(a, b, gr.B_KN, binding.CONFIG_AUTO, splits), plain)


@pytest.mark.parametrize("integer", [False, True])
@pytest.mark.parametrize("b_layout", [gr.B_KN, gr.B_NK])
def test_splitk_skinny_64x16384x8192_bf16_full(integer, b_layout):
    w = inputs.WORKLOADS["skinny_64x16384x8192"]
    cfg = gr.selected_splitk_config(w.M, w.N, w.K, dtype=gr.BF16, config=binding.CONFIG_DMA_64x256,
                                    b_layout=b_layout)
    assert (cfg["config_id"], cfg["splits"]) == (binding.CONFIG_DMA_64x256, 4)
    a, b = inputs.workload_inputs(w, integer)
    got = run_splitk(a, b, b_layout, binding.CONFIG_DMA_64x256, 0)
    say(f"[{w.name} split-K layout={b_layout} integer={integer}] full oracle")
    want = oracle.gemm_relu(a, b, w.dtype)
    check_relu_invariants(got, w.dtype)
    if integer:
        assert np.array_equal(got, want)
    else:
        assert_within_tolerance(got, want, w.dtype)


def test_splitk_nothing_written_outside_c():
    M, N, K = 70, 600, 1000
    guard = 4096
    a, b = inputs.normal_pair(M, N, K, torch.float16, 1.0, 9)
    buf = torch.full((M * N + 2 * guard,), float("nan"), dtype=torch.float16, device="cuda")
    c = buf[guard:guard + M * N].view(M, N)
    gr.gemm_relu_splitk(a.cuda(), b.cuda(), out=c, splits=4)
    torch.cuda.synchronize()
    raw = bits(buf)
    nan_bits = bits(torch.tensor([float("nan")], dtype=torch.float16))[0]
    assert (raw[:guard] == nan_bits).all() and (raw[guard + M * N:] == nan_bits).all()
    assert_within_tolerance(raw[guard:guard + M * N].reshape(M, N), oracle.gemm_relu(a, b, "fp16"), "fp16")


def test_splitk_workspace_errors():
    a = torch.ones((64, 512), dtype=torch.float16, device="cuda")
    b = torch.ones((512, 512), dtype=torch.float16, device="cuda")
    need = gr.selected_splitk_config(64, 512, 512, splits=4)["workspace_bytes"]
    assert need > 0
    small = torch.zeros(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(binding.GemmReluError) as e:
        gr.gemm_relu_splitk(a, b, splits=4, workspace=small)
    assert e.value.code == -10
    big = torch.zeros(need + 1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(binding.GemmReluError) as e:
        gr.gemm_relu_splitk(a, b, splits=4, workspace=big[16:])      # not 256-byte aligned
    assert e.value.code == -10
    # splits == 1 needs no workspace
    c = gr.gemm_relu_splitk(a, b, splits=1)
    torch.cuda.synchronize()
    assert (c == 512).all()


@pytest.mark.parametrize("integer", [False, True])
def test_splitk_deep_512x512x16384_full(integer):
    w = inputs.WORKLOADS["deep_512x512x16384"]
    cfg = gr.selected_splitk_config(w.M, w.N, w.K)
    assert (cfg["config_id"], cfg["splits"]) == (binding.CONFIG_DMA_64, 4)
    a, b = inputs.workload_inputs(w, integer)
    got = run_splitk(a, b, gr.B_KN, binding.CONFIG_AUTO, 0)
    want = oracle.gemm_relu(a, b, w.dtype)
    check_relu_invariants(got, w.dtype)
    if integer:
        assert np.array_equal(got, want)
    else:
        assert_within_tolerance(got, want, w.dtype)


def test_splitk_on_two_streams_uses_two_workspaces():
    # The binding keeps one cached workspace per stream: two streams running
    # split-K at the same time never share counters or partials.
    M, N, K = 64, 4096, 4096
    pairs = [inputs.integer_pair(M, N, K, torch.float16, seed=s) for s in (31, 32)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    dev_pairs = [(a.cuda(), b.cuda()) for a, b in pairs]
    torch.cuda.synchronize()
    outs = []
    for rep in range(3):
        for (a, b), st in zip(dev_pairs, streams):
            with torch.cuda.stream(st):
                outs.append(gr.gemm_relu_splitk(a, b, config=binding.CONFIG_DMA_64x256, splits=8))
    torch.cuda.synchronize()
    for i, c in enumerate(outs):
        a, b = pairs[i % 2]
        assert np.array_equal(bits(c), oracle.gemm_relu(a, b, "fp16")), i
    keys = [k for k in binding._workspaces if k[1] in (streams[0].cuda_stream, streams[1].cuda_stream)]
    assert len(keys) == 2
