"""GPU parity for B stored as B^T, an (N, K) row-major array (gemm_relu_ex with
GEMM_RELU_B_NK): the "transpose_B" GEMM whose B buffer is declared (N, K) in
"TileLang Guide: Composable Tiled AI Kernel Programming" (sections "Tiles as
First-Class Language Primitives" and "Step 1: Defining the Composable Kernel").

The oracle computes ReLU(A @ B) from B itself; the GPU is handed the bytes of
B^T.  Bars as for the (K, N) layout: bit-exact on integer-valued inputs,
|C_gpu - C_ref| <= 1e-2 + 1e-2 * |C_ref| on real-valued ones.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_dense_gemm_relu_amd as gr
from tiled_dense_gemm_relu_amd import binding, inputs

from test_gpu_parity import (CONFIGS, DT, assert_within_tolerance, bits, check_relu_invariants, sample_rows,
                             say)

pytestmark = pytest.mark.gpu


def run_nk(a, b, config=binding.CONFIG_AUTO):
    """C = ReLU(a @ b) on the GPU, with b handed over as b^T (N, K)."""
    bt = b.t().contiguous()
    c = gr.gemm_relu_ex(a.cuda(), bt.cuda(), b_layout=gr.B_NK, config=config)
    torch.cuda.synchronize()
    return bits(c)


NK_SHAPES = [(1, 1, 1), (33, 65, 17), (32, 32, 16), (64, 64, 8), (255, 257, 64), (256, 256, 40),
             (300, 520, 200), (257, 263, 96), (129, 131, 200), (512, 256, 192), (64, 1000, 1024),
             (520, 776, 1064),
             # K even but not a multiple of 8: 4-byte DMA lanes for both operands
             (200, 264, 100), (260, 262, 66), (300, 270, 4098)]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("config", CONFIGS)
@pytest.mark.parametrize("shape", NK_SHAPES)
def test_b_nk_integer_inputs_bit_exact(shape, config, dtype):
    M, N, K = shape
    a, b = inputs.integer_pair(M, N, K, DT[dtype], seed=3 * M + 5 * N + 11 * K)
    want = oracle.gemm_relu(a, b, dtype)
    assert np.array_equal(run_nk(a, b, config), want)


@pytest.mark.parametrize("name", ["small_256", "square_1024"])
@pytest.mark.parametrize("config", CONFIGS)
def test_b_nk_workloads_within_tolerance(name, config):
    w = inputs.WORKLOADS[name]
    a, b = inputs.workload_inputs(w)
    want = oracle.gemm_relu(a, b, w.dtype)
    got = run_nk(a, b, config)
    check_relu_invariants(got, w.dtype)
    assert_within_tolerance(got, want, w.dtype)


@pytest.mark.parametrize("config", [binding.CONFIG_DMA_256, binding.CONFIG_DMA_128, binding.CONFIG_DMA_64])
def test_b_nk_matches_b_kn_bit_for_bit(config):
    # Same tile, same MFMA k order: the two layouts give identical fp32 sums.
    a, b = inputs.normal_pair(700, 520, 1000, torch.float16, 1.0, 21)
    kn = bits(gr.gemm_relu(a.cuda(), b.cuda(), config=config))
    torch.cuda.synchronize()
    assert np.array_equal(run_nk(a, b, config), kn)


@pytest.mark.parametrize("integer", [False, True])
def test_b_nk_square_8192_sampled(integer):
    w = inputs.WORKLOADS["square_8192"]
    a, b = inputs.workload_inputs(w, integer)
    say(f"[{w.name} B (N,K) integer={integer}] GPU run")
    got = run_nk(a, b)
    check_relu_invariants(got, w.dtype)
    rows = sample_rows(w.M)
    say(f"[{w.name} B (N,K) integer={integer}] oracle on rows {rows}")
    want_rows = np.concatenate([oracle.gemm_relu_rows(a, b, w.dtype, r, r + 1) for r in rows])
    rng = np.random.default_rng(w.seed + 1)
    ii, jj = rng.integers(0, w.M, 1024), rng.integers(0, w.N, 1024)
    want_entries = oracle.gemm_relu_entries(a, b, w.dtype, ii, jj)
    if integer:
        assert np.array_equal(got[rows], want_rows)
        assert np.array_equal(got[ii, jj], want_entries)
    else:
        assert_within_tolerance(got[rows], want_rows, w.dtype)
        assert_within_tolerance(got[ii, jj], want_entries, w.dtype)


@pytest.mark.parametrize("a_off,b_off,c_off", [(1, 0, 0), (0, 1, 0), (0, 0, 1), (2, 2, 0), (4, 4, 0)])
@pytest.mark.parametrize("config", CONFIGS)
def test_b_nk_unaligned_pointers(a_off, b_off, c_off, config):
    M, N, K = 130, 270, 104
    a, b = inputs.integer_pair(M, N, K, torch.float16, seed=77)
    want = oracle.gemm_relu(a, b, "fp16")
    abuf = torch.zeros(M * K + a_off, dtype=torch.float16, device="cuda")
    bbuf = torch.zeros(N * K + b_off, dtype=torch.float16, device="cuda")
    cbuf = torch.zeros(M * N + c_off, dtype=torch.float16, device="cuda")
    av, btv, cv = abuf[a_off:].view(M, K), bbuf[b_off:].view(N, K), cbuf[c_off:].view(M, N)
    av.copy_(a)
    btv.copy_(b.t())
    gr.gemm_relu_ex(av, btv, out=cv, b_layout=gr.B_NK, config=config)
    torch.cuda.synchronize()
    assert np.array_equal(bits(cv), want)


@pytest.mark.parametrize("a_off,b_off", [(0, 0), (2, 2), (0, 2)])
@pytest.mark.parametrize("shape", [(300, 264, 2), (257, 520, 36), (520, 776, 70), (513, 1032, 764),
                                   (300, 270, 4098), (4100, 4360, 70)])
def test_b_nk_k_straddling_pieces(shape, a_off, b_off):
    # B^T rows hold K elements like A rows.  With K even but not a multiple of 8
    # the 256 LDS-DMA kernel loads both with 16-byte lanes, and the last K-step's
    # piece holding element K - 1 of a row also covers the start of the next row,
    # in A and in B^T; past K, those two would multiply each other.  The kernel
    # rewrites both pieces with zeros past K.  +inf and NaN at the start of rows
    # of both operands must reach only the outputs whose sums contain them.
    # A and B^T may start 4 bytes into a buffer (rows 4-byte aligned only).
    M, N, K = shape
    for dtype in ("fp16", "bf16"):
        a, b = inputs.integer_pair(M, N, K, DT[dtype], seed=M + N + K + 1)
        a[1::3, 0] = float("inf")
        a[2::5, 1] = float("nan")
        b[0, 1::4] = float("inf")          # B^T rows 1, 5, 9, ... start with +inf
        b[1, 3::7] = float("nan")
        want = oracle.gemm_relu(a, b, dtype)
        assert np.isinf(torch.from_numpy(want.view(np.int16)).view(DT[dtype]).float().numpy()).any()
        abuf = torch.zeros(M * K + a_off, dtype=DT[dtype], device="cuda")
        bbuf = torch.zeros(N * K + b_off, dtype=DT[dtype], device="cuda")
        av, btv = abuf[a_off:].view(M, K), bbuf[b_off:].view(N, K)
        av.copy_(a)
        btv.copy_(b.t())
        for config in (binding.CONFIG_AUTO, binding.CONFIG_DMA_256):
            cfg = gr.selected_config(M, N, K, dtype=gr.F16 if dtype == "fp16" else gr.BF16, config=config,
                                     a_ptr=av.data_ptr(), b_ptr=btv.data_ptr(), b_layout=gr.B_NK)
            assert (cfg["config_id"], cfg["vec_a"], cfg["vec_b"], cfg["block_k"]) == (3, 8, 8, 64)
            say(f"B (N, K) straddling pieces: {shape} offsets {a_off},{b_off} {dtype} config={config}")
            c = gr.gemm_relu_ex(av, btv, b_layout=gr.B_NK, config=config)
            torch.cuda.synchronize()
            got = bits(c)
            bad = np.argwhere(got != want)
            assert bad.size == 0, (dtype, config, f"{len(bad)} differ, first at {tuple(bad[0])}")


@pytest.mark.parametrize("config", CONFIGS)
def test_b_nk_nothing_written_outside_c(config):
    M, N, K = 250, 300, 72
    guard = 4096
    a, b = inputs.normal_pair(M, N, K, torch.bfloat16, 1.0, 6)
    buf = torch.full((M * N + 2 * guard,), float("nan"), dtype=torch.bfloat16, device="cuda")
    c = buf[guard:guard + M * N].view(M, N)
    gr.gemm_relu_ex(a.cuda(), b.t().contiguous().cuda(), out=c, b_layout=gr.B_NK, config=config)
    torch.cuda.synchronize()
    raw = bits(buf)
    nan_bits = bits(torch.tensor([float("nan")], dtype=torch.bfloat16))[0]
    assert (raw[:guard] == nan_bits).all() and (raw[guard + M * N:] == nan_bits).all()
    assert_within_tolerance(raw[guard:guard + M * N].reshape(M, N), oracle.gemm_relu(a, b, "bf16"), "bf16")


@pytest.mark.parametrize("integer", [False, True])
@pytest.mark.parametrize("shape", [(64, 65536, 2048), (40, 65800, 1000)])
def test_b_nk_wide_decode_shapes(shape, integer):
    # At most 64 rows with B^T: AUTO takes the 64x64 producer tile whatever the tile count (the
    # second shape has M, N and K tails).  Sampled rows and entries against the oracle.
    M, N, K = shape
    assert gr.selected_config(M, N, K, dtype=gr.BF16, b_layout=gr.B_NK)["config_id"] == binding.CONFIG_DMA_64x64_WS
    if integer:
        a, b = inputs.integer_pair(M, N, K, torch.bfloat16, seed=M + N + K + 1)
    else:
        a, b = inputs.normal_pair(M, N, K, torch.bfloat16, scale=0.05, seed=M + N + K + 1)
    say(f"[B^T wide decode {shape} integer={integer}] GPU run")
    got = run_nk(a, b)
    check_relu_invariants(got, "bf16")
    rows = [0, 1, M // 2, M - 1]
    want_rows = np.concatenate([oracle.gemm_relu_rows(a, b, "bf16", r, r + 1) for r in rows])
    rng = np.random.default_rng(M + N + K + 1)
    ii = np.concatenate([rng.integers(0, M, 1024), np.full(64, M - 1)])
    jj = np.concatenate([rng.integers(0, N, 1024), rng.integers(N - 64, N, 64)])
    want_entries = oracle.gemm_relu_entries(a, b, "bf16", ii, jj)
    if integer:
        assert np.array_equal(got[rows], want_rows)
        assert np.array_equal(got[ii, jj], want_entries)
    else:
        assert_within_tolerance(got[rows], want_rows, "bf16")
        assert_within_tolerance(got[ii, jj], want_entries, "bf16")


@pytest.mark.parametrize("config", [binding.CONFIG_DMA_64x64_WS, binding.CONFIG_DMA_32x32_WS])
@pytest.mark.parametrize("integer", [False, True])
def test_b_nk_k_rotation(config, integer):
    # With at most 64 rows, the 64x64 and 32x32 producer tiles walk each tile's K-steps from a
    # column-dependent start, wrapping round.  313 tiles of 64x64 (more than the CUs, so workgroups
    # move on to tiles with another start) and K = 1000 (a partial last K-step, met anywhere in the
    # order): bit-exact on integer inputs, within tolerance on real ones.
    M, N, K = 48, 20032, 1000
    if integer:
        a, b = inputs.integer_pair(M, N, K, torch.bfloat16, seed=4848)
    else:
        a, b = inputs.normal_pair(M, N, K, torch.bfloat16, scale=0.05, seed=4848)
    say(f"[B^T K rotation, config {config}, integer={integer}] GPU run")
    got = run_nk(a, b, config)
    want = oracle.gemm_relu(a, b, "bf16")
    check_relu_invariants(got, "bf16")
    if integer:
        assert np.array_equal(got, want)
    else:
        assert_within_tolerance(got, want, "bf16")


def test_b_nk_k_zero_and_empty():
    a = torch.empty((37, 0), dtype=torch.float16, device="cuda")
    bt = torch.empty((53, 0), dtype=torch.float16, device="cuda")
    c = torch.full((37, 53), float("nan"), dtype=torch.float16, device="cuda")
    gr.gemm_relu_ex(a, bt, out=c, b_layout=gr.B_NK)
    torch.cuda.synchronize()
    assert (bits(c) == 0).all()
    assert gr.gemm_relu_ex(torch.ones((4, 16), dtype=torch.float16, device="cuda"),
                           torch.empty((0, 16), dtype=torch.float16, device="cuda"),
                           b_layout=gr.B_NK).shape == (4, 0)


def test_b_nk_wrapper_checks_shapes():
    a = torch.ones((4, 8), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        gr.gemm_relu_ex(a, torch.ones((8, 5), dtype=torch.float16, device="cuda"), b_layout=gr.B_NK)
    with pytest.raises(ValueError):
        gr.gemm_relu_ex(a, torch.ones((5, 8), dtype=torch.float16, device="cuda"), b_layout=7)
    assert gr.gemm_relu_ex(a, torch.ones((5, 8), dtype=torch.float16, device="cuda"),
                           b_layout=gr.B_NK).shape == (4, 5)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("shape", [(300, 520, 201), (700, 900, 1031), (4100, 264, 77)])
def test_b_nk_odd_k_takes_the_register_staged_kernel(shape, dtype):
    # With odd K, B^T rows are only 2-byte aligned: no LDS-DMA lane width fits, and AUTO takes the
    # register-staged kernel, which loads B^T like A (elements along K), over several tiles.
    M, N, K = shape
    a, b = inputs.integer_pair(M, N, K, DT[dtype], seed=M + 3 * N + 7 * K)
    want = oracle.gemm_relu(a, b, dtype)
    code = gr.F16 if dtype == "fp16" else gr.BF16
    bt = b.t().contiguous().cuda()
    cfg = gr.selected_config(M, N, K, dtype=code, b_layout=gr.B_NK, a_ptr=1 << 20, b_ptr=1 << 21)
    assert cfg["config_id"] in (binding.CONFIG_TILE_256, binding.CONFIG_TILE_128) and cfg["vec_b"] == 1
    for config in (binding.CONFIG_AUTO, binding.CONFIG_TILE_256, binding.CONFIG_TILE_128, binding.CONFIG_DMA_256,
                   binding.CONFIG_DIRECT):
        c = gr.gemm_relu_ex(a.cuda(), bt, b_layout=gr.B_NK, config=config)
        torch.cuda.synchronize()
        got = bits(c)
        bad = np.argwhere(got != want)
        assert bad.size == 0, (config, f"{len(bad)} differ, first at {tuple(bad[0])}")
