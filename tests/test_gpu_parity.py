"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars:
- integer-valued inputs (entries in {-2..2}): every fp32 partial sum is an exact
  integer, so the GPU result must equal the oracle's bit for bit;
- real-valued inputs: |C_gpu - C_ref| <= 1e-2 + 1e-2 * |C_ref| elementwise
  (the acceptance rule of the GEMM + ReLU example in "Writing High-Performance
  Kernels in TileLang", section "Let's write a GEMM": rtol = atol = 1e-2);
- always: C >= 0, no -0.0, no NaN; nothing written outside C.

Full-size workloads the oracle cannot finish in seconds are checked on sampled
rows (each a complete row of C, spread over first, middle and last tiles) and
sampled elements, in the launch configuration the benchmark times.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import tiled_dense_gemm_relu_amd as gr
from tiled_dense_gemm_relu_amd import binding, inputs

pytestmark = pytest.mark.gpu

RTOL = ATOL = 1e-2
CONFIGS = [binding.CONFIG_DIRECT, binding.CONFIG_TILE_256, binding.CONFIG_TILE_128, binding.CONFIG_DMA_256,
           binding.CONFIG_DMA_128, binding.CONFIG_DMA_64, binding.CONFIG_DMA_64x256, binding.CONFIG_DMA_256x128_WS,
           binding.CONFIG_DMA_32x32_WS, binding.CONFIG_DMA_64x64_WS, binding.CONFIG_DMA_128x128_WS]
DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def values(b: np.ndarray, dtype) -> np.ndarray:
    return torch.from_numpy(b.view(np.int16)).view(DT[dtype]).to(torch.float64).numpy()


def run_gpu(a, b, config=binding.CONFIG_AUTO):
    c = gr.gemm_relu(a.cuda(), b.cuda(), config=config)
    torch.cuda.synchronize()
    return bits(c)


def check_relu_invariants(got_bits, dtype):
    v = values(got_bits, dtype)
    assert not np.isnan(v).any(), "NaN in output"
    assert (v >= 0).all(), "negative output"
    assert not (got_bits == 0x8000).any(), "-0.0 in output"


def assert_within_tolerance(got_bits, want_bits, dtype):
    g, w = values(got_bits, dtype), values(want_bits, dtype)
    err = np.abs(g - w)
    bound = ATOL + RTOL * np.abs(w)
    bad = err > bound
    assert not bad.any(), (f"{int(bad.sum())} elements out of tolerance; worst at "
                           f"{np.unravel_index(np.argmax(err - bound), err.shape)}")


# ------------------------------------------------------------- integer inputs

INT_SHAPES = [(1, 1, 1), (32, 32, 16), (33, 65, 17), (255, 257, 63), (257, 255, 65),
              (300, 520, 130), (129, 131, 200), (512, 256, 192), (64, 1000, 1024),
              # 16-byte-loadable shapes for the LDS-DMA kernel: a K tail (K % 32 != 0),
              # fewer K-steps than pipeline stages, and M / N tails
              (300, 520, 200), (256, 256, 40), (64, 64, 8), (257, 264, 96), (520, 776, 1064),
              # 4-byte DMA lanes: A rows of an even length, B rows of an even length, both
              (200, 264, 100), (260, 262, 64), (256, 300, 66), (300, 270, 4098)]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("config", CONFIGS)
@pytest.mark.parametrize("shape", INT_SHAPES)
def test_integer_inputs_bit_exact(shape, config, dtype):
    M, N, K = shape
    a, b = inputs.integer_pair(M, N, K, DT[dtype], seed=M + 7 * N + 13 * K)
    want = oracle.gemm_relu(a, b, dtype)
    got = run_gpu(a, b, config)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("config", CONFIGS)
def test_small_256_workload(config):
    w = inputs.WORKLOADS["small_256"]
    for integer in (False, True):
        a, b = inputs.workload_inputs(w, integer)
        want = oracle.gemm_relu(a, b, w.dtype)
        got = run_gpu(a, b, config)
        check_relu_invariants(got, w.dtype)
        if integer:
            assert np.array_equal(got, want)
        else:
            assert_within_tolerance(got, want, w.dtype)


@pytest.mark.parametrize("config", [binding.CONFIG_AUTO] + CONFIGS[1:])
def test_square_1024_workload(config):
    w = inputs.WORKLOADS["square_1024"]
    for integer in (False, True):
        a, b = inputs.workload_inputs(w, integer)
        want = oracle.gemm_relu(a, b, w.dtype)
        got = run_gpu(a, b, config)
        check_relu_invariants(got, w.dtype)
        if integer:
            assert np.array_equal(got, want)
        else:
            assert_within_tolerance(got, want, w.dtype)


# ------------------------------------------------------- full-size workloads


def sample_rows(M, tile=256):
    rows = {0, 1, M // 2, M - 2, M - 1}
    last_tile = (M - 1) // tile * tile
    rows |= {tile - 1, tile, last_tile, min(M - 1, last_tile + 1)}
    return sorted(r for r in rows if 0 <= r < M)


def check_sampled(w, integer, n_entries=2048):
    a, b = inputs.workload_inputs(w, integer)
    say(f"[{w.name} integer={integer}] GPU run")
    c = gr.gemm_relu(a.cuda(), b.cuda())
    torch.cuda.synchronize()
    got = bits(c)
    check_relu_invariants(got, w.dtype)
    rows = sample_rows(w.M)
    say(f"[{w.name} integer={integer}] oracle on rows {rows}")
    want_rows = np.concatenate([oracle.gemm_relu_rows(a, b, w.dtype, r, r + 1) for r in rows])
    rng = np.random.default_rng(w.seed)
    ii, jj = rng.integers(0, w.M, n_entries), rng.integers(0, w.N, n_entries)
    want_entries = oracle.gemm_relu_entries(a, b, w.dtype, ii, jj)
    if integer:
        assert np.array_equal(got[rows], want_rows)
        assert np.array_equal(got[ii, jj], want_entries)
    else:
        assert_within_tolerance(got[rows], want_rows, w.dtype)
        assert_within_tolerance(got[ii, jj], want_entries, w.dtype)
    return got


@pytest.mark.parametrize("integer", [False, True])
def test_ragged_4000x11000x4100_sampled(integer):
    w = inputs.WORKLOADS["ragged_4000x11000x4100"]
    got = check_sampled(w, integer)
    if not integer:
        frac_zero = (got == 0).mean()
        assert 0.4 < frac_zero < 0.6                # about half the sums are negative


@pytest.mark.parametrize("name", ["square_8192", "square_8192_bf16"])
@pytest.mark.parametrize("integer", [False, True])
def test_square_8192_sampled(integer, name):
    w = inputs.WORKLOADS[name]
    got = check_sampled(w, integer, n_entries=1024)
    if not integer:
        assert 0.45 < (got == 0).mean() < 0.55


def test_k_of_a_million():
    # K = 2^20 + 40 (a K tail), M and N tails: offsets along K up to 2 MiB per
    # A row and B bands of 64 rows x N, through the plain and the split-K
    # entry points.  Integer inputs: every fp32 partial sum is exact (< 2^24).
    M, N, K = 264, 264, (1 << 20) + 40
    a, b = inputs.integer_pair(M, N, K, torch.float16, seed=77)
    rows = [0, 1, 127, 128, 255, 256, M - 1]
    want = np.concatenate([oracle.gemm_relu_rows(a, b, "fp16", r, r + 1) for r in rows])
    say("[K = 2^20 + 40] GPU runs")
    ad, bd = a.cuda(), b.cuda()
    c1 = gr.gemm_relu(ad, bd)
    c2 = gr.gemm_relu_splitk(ad, bd, splits=0)
    torch.cuda.synchronize()
    for c in (c1, c2):
        assert np.array_equal(bits(c)[rows], want)


@pytest.mark.parametrize("config", [binding.CONFIG_AUTO, binding.CONFIG_DMA_128])
def test_c_larger_than_4_gib(config):
    # C of 32800 x 65544 fp16 = 4.3 GB: element offsets past 2^31, and C stored
    # through one buffer descriptor per 32-row strip.  Only sampled entries, the
    # last rows and the last column come back to the host.
    M, N, K = 32800, 65544, 16
    a, b = inputs.integer_pair(M, N, K, torch.float16, seed=4242)
    say(f"[C > 4 GiB, config {config}] GPU run")
    c = gr.gemm_relu(a.cuda(), b.cuda(), config=config)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4242)
    ii = np.concatenate([rng.integers(0, M, 4096), [M - 1] * 64, rng.integers(M - 40, M, 64)])
    jj = np.concatenate([rng.integers(0, N, 4096), rng.integers(0, N, 64), [N - 1] * 64])
    got = bits(c[torch.from_numpy(ii).cuda(), torch.from_numpy(jj).cuda()])
    assert np.array_equal(got, oracle.gemm_relu_entries(a, b, "fp16", ii, jj))
    last_rows = bits(c[M - 2:])
    assert np.array_equal(last_rows, oracle.gemm_relu_rows(a, b, "fp16", M - 2, M))
    last_col = bits(c[:, N - 1])
    assert np.array_equal(last_col, oracle.gemm_relu_entries(a, b, "fp16", np.arange(M), np.full(M, N - 1)))
    del c
    torch.cuda.empty_cache()


@pytest.mark.parametrize("integer", [False, True])
def test_skinny_64x16384x8192_bf16_full(integer):
    w = inputs.WORKLOADS["skinny_64x16384x8192"]
    a, b = inputs.workload_inputs(w, integer)
    got = run_gpu(a, b)
    say(f"[{w.name} integer={integer}] full oracle")
    want = oracle.gemm_relu(a, b, w.dtype)
    check_relu_invariants(got, w.dtype)
    if integer:
        assert np.array_equal(got, want)
    else:
        assert_within_tolerance(got, want, w.dtype)


@pytest.mark.parametrize("integer", [False, True])
@pytest.mark.parametrize("shape", [(64, 65536, 2048), (40, 65800, 1000)])
def test_wide_decode_shapes(shape, integer):
    # At most 64 rows over 256 or more 64x256 tiles: AUTO runs the 64x256 tile unsplit (4 stages,
    # C staged through LDS).  The second shape has M, N and K tails (a partial last column tile and
    # K % 32 != 0).  Sampled rows and entries against the oracle.
    M, N, K = shape
    assert gr.selected_config(M, N, K, dtype=gr.BF16)["config_id"] == binding.CONFIG_DMA_64x256
    if integer:
        a, b = inputs.integer_pair(M, N, K, torch.bfloat16, seed=M + N + K)
    else:
        a, b = inputs.normal_pair(M, N, K, torch.bfloat16, scale=0.05, seed=M + N + K)
    say(f"[wide decode {shape} integer={integer}] GPU run")
    got = run_gpu(a, b)
    check_relu_invariants(got, "bf16")
    rows = [0, 1, M // 2, M - 1]
    want_rows = np.concatenate([oracle.gemm_relu_rows(a, b, "bf16", r, r + 1) for r in rows])
    rng = np.random.default_rng(M + N + K)
    ii = np.concatenate([rng.integers(0, M, 1024), np.full(64, M - 1)])
    jj = np.concatenate([rng.integers(0, N, 1024), rng.integers(N - 256, N, 64)])
    want_entries = oracle.gemm_relu_entries(a, b, "bf16", ii, jj)
    if integer:
        assert np.array_equal(got[rows], want_rows)
        assert np.array_equal(got[ii, jj], want_entries)
    else:
        assert_within_tolerance(got[rows], want_rows, "bf16")
        assert_within_tolerance(got[ii, jj], want_entries, "bf16")


# ------------------------------------------------------------------ edge cases


@pytest.mark.parametrize("config", CONFIGS)
def test_k_zero_fills_positive_zero(config):
    a = torch.empty((37, 0), dtype=torch.float16, device="cuda")
    b = torch.empty((0, 53), dtype=torch.float16, device="cuda")
    c = torch.full((37, 53), float("nan"), dtype=torch.float16, device="cuda")
    gr.gemm_relu(a, b, out=c, config=config)
    torch.cuda.synchronize()
    assert (bits(c) == 0).all()


def test_empty_m_or_n():
    a = torch.empty((0, 16), dtype=torch.float16, device="cuda")
    b = torch.ones((16, 8), dtype=torch.float16, device="cuda")
    assert gr.gemm_relu(a, b).shape == (0, 8)
    a = torch.ones((4, 16), dtype=torch.float16, device="cuda")
    b = torch.empty((16, 0), dtype=torch.float16, device="cuda")
    assert gr.gemm_relu(a, b).shape == (4, 0)


@pytest.mark.parametrize("a_off,b_off,c_off", [(1, 0, 0), (0, 1, 0), (0, 0, 1), (3, 5, 7), (4, 4, 0)])
@pytest.mark.parametrize("config", CONFIGS)
def test_unaligned_pointers(a_off, b_off, c_off, config):
    # Views starting a few elements into a buffer: 2-byte aligned only.
    M, N, K = 130, 270, 100
    a, b = inputs.integer_pair(M, N, K, torch.float16, seed=99)
    want = oracle.gemm_relu(a, b, "fp16")
    abuf = torch.zeros(M * K + a_off, dtype=torch.float16, device="cuda")
    bbuf = torch.zeros(K * N + b_off, dtype=torch.float16, device="cuda")
    cbuf = torch.zeros(M * N + c_off, dtype=torch.float16, device="cuda")
    av = abuf[a_off:].view(M, K)
    bv = bbuf[b_off:].view(K, N)
    cv = cbuf[c_off:].view(M, N)
    av.copy_(a)
    bv.copy_(b)
    gr.gemm_relu(av, bv, out=cv, config=config)
    torch.cuda.synchronize()
    assert np.array_equal(bits(cv), want)


@pytest.mark.parametrize("K", [1, 2, 3, 5, 7, 9, 63, 65, 127])
def test_odd_k(K):
    M, N = 70, 90
    for dtype in ("fp16", "bf16"):
        a, b = inputs.integer_pair(M, N, K, DT[dtype], seed=K)
        want = oracle.gemm_relu(a, b, dtype)
        for config in CONFIGS:
            assert np.array_equal(run_gpu(a, b, config), want), (dtype, config)


@pytest.mark.parametrize("a_off", [0, 2])
@pytest.mark.parametrize("shape", [(300, 264, 2), (257, 520, 36), (64, 64, 6), (520, 776, 70),
                                   (300, 264, 1030), (513, 1032, 764),
                                   # more tiles than CUs: with one K-step per tile every step is a
                                   # last K-step, so consecutive tiles each rewrite their piece
                                   (4100, 4360, 6), (4100, 4360, 70)])
def test_k_straddling_piece(shape, a_off):
    # K even but not a multiple of 8, B rows of 8-element multiples: the 256
    # LDS-DMA kernel loads A with 16-byte lanes, so the last K-step's piece
    # holding element K - 1 of a row also covers the first elements of the
    # next row.  The kernel rewrites that piece with zeros past K.  +inf and
    # NaN placed at the start of rows would otherwise reach the row above as
    # inf * 0 = NaN.  A may also start 4 bytes into a buffer (rows 4-byte
    # aligned only).
    M, N, K = shape
    for dtype in ("fp16", "bf16"):
        a, b = inputs.integer_pair(M, N, K, DT[dtype], seed=M + N + K)
        a[1::3, 0] = float("inf")
        a[2::5, 1] = float("nan")
        b[0][b[0] == 0] = 1
        want = oracle.gemm_relu(a, b, dtype)
        assert np.isinf(values(want, dtype)).any()
        abuf = torch.zeros(M * K + a_off, dtype=DT[dtype], device="cuda")
        av = abuf[a_off:].view(M, K)
        av.copy_(a)
        for config in (binding.CONFIG_AUTO, binding.CONFIG_DMA_256):
            cfg = gr.selected_config(M, N, K, dtype=gr.F16 if dtype == "fp16" else gr.BF16, config=config,
                                     a_ptr=av.data_ptr(), b_ptr=1 << 20)
            if config == binding.CONFIG_DMA_256:
                assert (cfg["config_id"], cfg["vec_a"], cfg["block_k"]) == (3, 8, 64)
            say(f"straddling piece: {shape} a_off={a_off} {dtype} config={config} -> {cfg['config_id']}")
            c = gr.gemm_relu(av, b.cuda(), config=config)
            torch.cuda.synchronize()
            got = bits(c)
            bad = np.argwhere(got != want)
            assert bad.size == 0, (dtype, config, f"{len(bad)} differ, first at {tuple(bad[0])}")


@pytest.mark.parametrize("b_layout", [binding.B_KN, binding.B_NK])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_producer_wave_tiles_with_more_tiles_than_cus(dtype, b_layout):
    # The producer-wave configs with more output tiles than persistent workgroups: every
    # workgroup runs several tiles, so the producer waves set up the next tile's loads while
    # the compute waves run the last tile's epilogue (staged through LDS for the 128x128
    # tile).  M, N and K tails (K % 64 = 8).  AUTO picks the 128x128 producer tile here.
    M, N, K = 2056, 2312, 200
    a, b = inputs.integer_pair(M, N, K, DT[dtype], seed=M + N + K + b_layout)
    want = oracle.gemm_relu(a, b, dtype)
    bd = (b.t().contiguous() if b_layout == binding.B_NK else b).cuda()
    ad = a.cuda()
    code = gr.F16 if dtype == "fp16" else gr.BF16
    for config in (binding.CONFIG_DMA_32x32_WS, binding.CONFIG_DMA_64x64_WS, binding.CONFIG_DMA_128x128_WS,
                   binding.CONFIG_AUTO):
        cfg = gr.selected_config(M, N, K, dtype=code, config=config, b_layout=b_layout)
        if config == binding.CONFIG_AUTO:
            assert cfg["config_id"] == binding.CONFIG_DMA_128x128_WS
        else:
            assert cfg["config_id"] == config
        assert cfg["grid"] > 256, cfg
        say(f"[producer tiles] {M}x{N}x{K} {dtype} layout={b_layout} config={cfg['config_id']} tiles={cfg['grid']}")
        c = gr.gemm_relu_ex(ad, bd, b_layout=b_layout, config=config)
        torch.cuda.synchronize()
        got = bits(c)
        bad = np.argwhere(got != want)
        assert bad.size == 0, (config, f"{len(bad)} differ, first at {tuple(bad[0])}")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("config", CONFIGS)
def test_subnormal_inputs(config, dtype):
    # A holds only subnormals of its dtype: integers in {-2..2} times 2^-20 (fp16: below
    # 2^-14) or 2^-130 (bf16: below 2^-126).  B holds integers times a power of two, so
    # every product and partial sum is exact in fp32 and the oracle's exact result is
    # what the GPU must give, bit for bit.  In fp16, sums of a few units come out as
    # subnormals (below 2^-14) too.  A kernel that flushed subnormal inputs would give 0.
    M, N, K = 256, 264, 136
    ia, ib = inputs.integer_pair(M, N, K, torch.float32, seed=77)
    a_scale, b_scale = (2.0 ** -20, 2.0 ** 4) if dtype == "fp16" else (2.0 ** -130, 2.0 ** 100)
    a = (ia * a_scale).to(DT[dtype])
    b = (ib * b_scale).to(DT[dtype])
    av = a.to(torch.float64)
    assert ((av == 0) | (av.abs() < (2.0 ** -14 if dtype == "fp16" else 2.0 ** -126))).all()
    assert (av != 0).any() and torch.equal(av, ia.to(torch.float64) * a_scale)
    want = oracle.gemm_relu(a, b, dtype)
    wv = values(want, dtype)
    assert (wv > 0).sum() > M * N // 4
    if dtype == "fp16":
        assert ((wv > 0) & (wv < 2.0 ** -14)).any()     # subnormal outputs are part of the check
    got = run_gpu(a, b, config)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} differ, first at {tuple(bad[0])}"


@pytest.mark.parametrize("config", CONFIGS)
def test_nothing_written_outside_c(config):
    M, N, K = 250, 300, 70
    guard = 4096
    a, b = inputs.normal_pair(M, N, K, torch.float16, 1.0, 5)
    buf = torch.full((M * N + 2 * guard,), float("nan"), dtype=torch.float16, device="cuda")
    c = buf[guard:guard + M * N].view(M, N)
    gr.gemm_relu(a.cuda(), b.cuda(), out=c, config=config)
    torch.cuda.synchronize()
    raw = bits(buf)
    nan_bits = bits(torch.tensor([float("nan")], dtype=torch.float16))[0]
    assert (raw[:guard] == nan_bits).all() and (raw[guard + M * N:] == nan_bits).all()
    assert_within_tolerance(raw[guard:guard + M * N].reshape(M, N), oracle.gemm_relu(a, b, "fp16"), "fp16")


def _random_staged_shapes(n=16, seed=2024):
    # Seeded shapes with N % 8 == 0 (C in 16-byte row pieces, the staged
    # epilogue) and ragged M and K: rows past M inside a 32-row strip, M below
    # one strip, K tails of every residue mod 64.
    import random
    rng = random.Random(seed)
    shapes = []
    for _ in range(n):
        M = rng.choice([rng.randint(1, 40), rng.randint(33, 700)])
        N = 8 * rng.randint(1, 100)
        K = rng.choice([rng.randint(1, 130), 8 * rng.randint(1, 64)])
        shapes.append((M, N, K))
    return shapes


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("shape", _random_staged_shapes())
def test_random_shapes_staged_epilogue(shape, dtype):
    M, N, K = shape
    a, b = inputs.integer_pair(M, N, K, DT[dtype], seed=M * 131 + N * 7 + K)
    want = oracle.gemm_relu(a, b, dtype)
    for config in (binding.CONFIG_AUTO, binding.CONFIG_DMA_256, binding.CONFIG_DMA_128, binding.CONFIG_DMA_256x128_WS):
        assert np.array_equal(run_gpu(a, b, config), want), (shape, dtype, config)


@pytest.mark.parametrize("c_off", [0, 4, 2, 1])
@pytest.mark.parametrize("config", CONFIGS)
def test_c_store_paths(c_off, config):
    # N % 8 == 0 with M and N tails.  C starting c_off elements into a buffer
    # selects the store path: 0 gives 16-byte aligned rows (16-byte pieces; the
    # LDS-DMA kernels stage them through LDS), 4 gives 8-byte pieces, and 2
    # and 1 give element stores.  NaN guards on both sides must survive.
    M, N, K = 300, 264, 96
    guard = 4096
    a, b = inputs.integer_pair(M, N, K, torch.float16, seed=300 + c_off)
    want = oracle.gemm_relu(a, b, "fp16")
    buf = torch.full((M * N + 2 * guard + c_off,), float("nan"), dtype=torch.float16, device="cuda")
    c = buf[guard + c_off:guard + c_off + M * N].view(M, N)
    gr.gemm_relu(a.cuda(), b.cuda(), out=c, config=config)
    torch.cuda.synchronize()
    raw = bits(buf)
    nan_bits = bits(torch.tensor([float("nan")], dtype=torch.float16))[0]
    assert (raw[:guard + c_off] == nan_bits).all() and (raw[guard + c_off + M * N:] == nan_bits).all()
    assert np.array_equal(raw[guard + c_off:guard + c_off + M * N].reshape(M, N), want)


def test_run_to_run_bit_identical():
    w = inputs.WORKLOADS["ragged_4000x11000x4100"]
    a, b = inputs.workload_inputs(w)
    a, b = a.cuda(), b.cuda()
    c1 = bits(gr.gemm_relu(a, b))
    c2 = bits(gr.gemm_relu(a, b))
    assert np.array_equal(c1, c2)


def test_all_configs_agree_on_integer_inputs():
    a, b = inputs.integer_pair(777, 555, 333, torch.bfloat16, seed=4)
    outs = [run_gpu(a, b, cfg) for cfg in CONFIGS]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_side_stream():
    a, b = inputs.integer_pair(300, 200, 100, torch.float16, seed=8)
    want = oracle.gemm_relu(a, b, "fp16")
    s = torch.cuda.Stream()
    a, b = a.cuda(), b.cuda()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        c = gr.gemm_relu(a, b)
    s.synchronize()
    assert np.array_equal(bits(c), want)


def test_alias_is_rejected_and_c_untouched():
    a = torch.ones((64, 64), dtype=torch.float16, device="cuda")
    b = torch.ones((64, 64), dtype=torch.float16, device="cuda")
    before = bits(a).copy()
    with pytest.raises(binding.GemmReluError) as e:
        gr.gemm_relu(a, b, out=a)
    assert e.value.code == -3
    assert np.array_equal(bits(a), before)


def test_python_wrapper_rejects_bad_tensors():
    a = torch.ones((4, 8), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        gr.gemm_relu(a, a)                                  # inner dims differ
    with pytest.raises(ValueError):
        gr.gemm_relu(a.t(), a.t().contiguous())             # non-contiguous
    with pytest.raises(TypeError):
        gr.gemm_relu(a.float(), a.t().contiguous().float())
    with pytest.raises(ValueError):
        gr.gemm_relu(a.cpu(), a.t().contiguous().cpu())


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("b_layout", [binding.B_KN, binding.B_NK])
@pytest.mark.parametrize("c_off", [0, 4, 1])
@pytest.mark.parametrize("shape", [(300, 264, 128), (300, 264, 136), (260, 260, 192)])
def test_dma256_c_store_paths(shape, c_off, b_layout, dtype):
    """The 256 tile's three ways of storing C: staged through LDS (N % 8 == 0, C 16-byte aligned),
    8-byte pieces (N % 4 == 0, C 8-byte aligned) and single elements, with K % 64 == 0 and a K tail,
    for both B layouts."""
    M, N, K = shape
    if b_layout == binding.B_KN and N % 8:
        pytest.skip("B stored (K, N) with N % 8 != 0 takes the 4-byte-lane instance")
    dt = gr.F16 if dtype == "fp16" else gr.BF16
    a, b = inputs.integer_pair(M, N, K, DT[dtype], seed=7 + c_off)
    want = oracle.gemm_relu(a, b, dtype)
    cbuf = torch.full((M * N + c_off,), float("nan"), dtype=DT[dtype], device="cuda")
    cv = cbuf[c_off:].view(M, N)
    bdev = (b.t().contiguous() if b_layout == binding.B_NK else b).cuda()
    cfg = gr.selected_config(M, N, K, dtype=dt, config=binding.CONFIG_DMA_256, c_ptr=cv.data_ptr(),
                             b_layout=b_layout)
    assert cfg["config_id"] == binding.CONFIG_DMA_256
    say(f"[256 tile C stores] {shape} c_off={c_off} layout={b_layout} {dtype}")
    gr.gemm_relu_ex(a.cuda(), bdev, out=cv, b_layout=b_layout, config=binding.CONFIG_DMA_256)
    torch.cuda.synchronize()
    assert np.array_equal(bits(cv), want)
    assert torch.isnan(cbuf[:c_off]).all()          # nothing written before C
