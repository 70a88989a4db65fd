"""Launch-bound callers capture the library's calls in HIP graphs: the entry
points issue only kernel launches on the caller's stream (no allocation, no
memset), and split-K's counters return to zero after every call (the
no-allocation variant clears its own with a fill kernel), so a captured call
can be replayed.  Each replay is checked against the oracle, with new
inputs copied in between replays."""
import numpy as np
import pytest
import torch

import oracle
import tiled_dense_gemm_relu_amd as gr
from tiled_dense_gemm_relu_amd import binding, inputs

from test_gpu_parity import bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", ["plain", "b_nk", "dma256", "dma256_b_nk", "splitk", "splitk_noalloc"])
def test_graph_replays_match_the_oracle(kind):
    M, N, K = 192, 320, 512
    dev = torch.device("cuda:0")
    a = torch.empty((M, K), dtype=torch.float16, device=dev)
    nk = kind in ("b_nk", "dma256_b_nk")
    b = torch.empty((N, K) if nk else (K, N), dtype=torch.float16, device=dev)
    c = torch.empty((M, N), dtype=torch.float16, device=dev)
    ws = torch.zeros(gr.selected_splitk_config(M, N, K, splits=4)["workspace_bytes"], dtype=torch.uint8,
                     device=dev)

    def call():
        if kind == "plain":
            gr.gemm_relu(a, b, out=c)
        elif kind == "b_nk":
            gr.gemm_relu_ex(a, b, out=c, b_layout=gr.B_NK)
        elif kind.startswith("dma256"):
            # the 256 tile (16x16x32 MFMAs, early refill), forced at this small shape
            gr.gemm_relu_ex(a, b, out=c, b_layout=gr.B_NK if nk else gr.B_KN, config=binding.CONFIG_DMA_256)
        elif kind == "splitk":
            gr.gemm_relu_splitk(a, b, out=c, splits=4, workspace=ws)
        else:
            # the static scratch: its counters are cleared by a fill kernel inside the graph
            gr.gemm_relu_splitk_noalloc(a, b, out=c, splits=4)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                                  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for seed in (11, 12, 13):
        ah, bh = inputs.integer_pair(M, N, K, torch.float16, seed=seed)
        a.copy_(ah)
        b.copy_(bh.t() if nk else bh)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(c), oracle.gemm_relu(ah, bh, "fp16")), (kind, seed)
    if kind == "splitk":
        assert (ws[:65536] == 0).all()          # the counter region is back at zero
