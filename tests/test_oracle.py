"""Pins for the CPU oracle: each check rests on something other than the oracle itself.

- the fp16/bf16 codec against numpy's and torch's conversions (library routines
  that round to nearest even), over every bit pattern and a million doubles;
- hand-worked examples (tests/golden/hand_examples.json);
- exact integer and exact rational (fractions.Fraction) arithmetic;
- textbook special cases and invariants of ReLU(A @ B);
- planted mistakes: mutated copies of the oracle source must fail these pins.
"""
import json
import os
import re
import subprocess
import ctypes
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tiled_dense_gemm_relu_amd import inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def f16_bits(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def bf16_bits_from_f32(x):
    """torch's float32 -> bfloat16 cast (round to nearest even) as bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_torch(bits, dtype):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dtype)


# ------------------------------------------------------------------ codec


def test_decode_every_f16_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode(bits, "fp16")
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signs of zeros too
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_decode_every_bf16_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode(bits, "bf16")
    want = to_torch(bits, torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def _random_doubles(n, lo_exp, hi_exp, seed):
    rng = np.random.default_rng(seed)
    mant = rng.uniform(1.0, 2.0, n)
    exp = rng.integers(lo_exp, hi_exp, n)
    sign = rng.choice([-1.0, 1.0], n)
    return sign * np.ldexp(mant, exp)


def test_encode_f16_matches_numpy_on_a_million_doubles():
    x = _random_doubles(1_000_000, -30, 18, 7)   # subnormal, normal and overflow ranges
    assert np.array_equal(oracle.encode(x, "fp16"), f16_bits(x))


def test_encode_f16_boundaries_match_numpy():
    ulp_sub = 2.0 ** -24
    cases = [0.0, -0.0, ulp_sub, ulp_sub / 2, ulp_sub * 1.5, ulp_sub * 2.5, ulp_sub / 2 * 1.0000001,
             2.0 ** -14, 2.0 ** -14 - ulp_sub / 2, 2.0 ** -14 - ulp_sub / 4,
             65504.0, 65519.0, 65519.999, 65520.0, 65536.0, 1e30, -65520.0,
             1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0, 1024.5, 1025.5,
             float("inf"), float("-inf")]
    for k in range(-24, 16):                    # 2^k plus/minus half an ulp of its binade
        for sgn in (1.0, -1.0):
            p = 2.0 ** k
            cases += [sgn * p, sgn * (p + p * 2.0 ** -11), sgn * (p - p * 2.0 ** -12)]
    x = np.array(cases)
    assert np.array_equal(oracle.encode(x, "fp16"), f16_bits(x))


def test_encode_bf16_matches_torch_on_float32_values():
    # float32-representable doubles: torch's float32 -> bf16 cast is then a single rounding
    with np.errstate(over="ignore"):
        x = _random_doubles(1_000_000, -140, 130, 8).astype(np.float32)
    x = x[np.isfinite(x)].astype(np.float64)
    assert np.array_equal(oracle.encode(x, "bf16"), bf16_bits_from_f32(x))


def _bf16_nearest_by_search(x):
    """Round doubles to bf16 bit patterns by search: the nearest entry of the table of every finite
    bf16 value (decoded by torch), ties to the pattern with an even fraction, and past the largest
    finite value by half its spacing or more to infinity.  It uses none of the oracle's arithmetic
    (no binade, quantum or rint): only the value table and exact float64 comparisons.  The midpoint
    of two neighbouring bf16 values has at most 9 significant bits, so it is an exact double and
    x < mid, x == mid, x > mid decide the rounding exactly."""
    pos_bits = np.arange(0, 0x7F80, dtype=np.uint16)            # +0 .. largest finite, increasing
    vals = to_torch(pos_bits, torch.bfloat16).to(torch.float64).numpy()
    top = 2.0 ** 128                                            # the next value past the largest
    hi_vals = np.append(vals[1:], top)
    hi_bits = np.append(pos_bits[1:], np.uint16(0x7F80))
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    i = np.searchsorted(vals, ax, side="right") - 1             # vals[i] <= ax < vals[i + 1]
    lo, hi = vals[i], hi_vals[i]
    mid = (lo + hi) / 2
    up = (ax > mid) | ((ax == mid) & (pos_bits[i] & 1 == 1))
    out = np.where(up, hi_bits[i], pos_bits[i]).astype(np.uint16)
    out[ax >= top] = 0x7F80
    return out | np.where(np.signbit(x), np.uint16(0x8000), np.uint16(0)).astype(np.uint16)


def test_encode_bf16_of_any_double_is_a_single_rounding():
    # Doubles with all 53 significant bits, and doubles within 2^-9 .. 2^-40 of a bf16 rounding
    # midpoint on either side (bits far below float32's last place): rounding through float32 first
    # would move many of them onto the midpoint.
    x = _random_doubles(200_000, -140, 128, 21)
    rng = np.random.default_rng(22)
    v = rng.integers(0x0001, 0x7F7F, 20_000).astype(np.uint16)
    vals = to_torch(v, torch.bfloat16).to(torch.float64).numpy()
    nxt = to_torch(v + 1, torch.bfloat16).to(torch.float64).numpy()
    mid = (vals + nxt) / 2
    eps = np.ldexp(nxt - vals, -rng.integers(9, 40, v.size))
    near = np.concatenate([mid, mid + eps, mid - eps])
    x = np.concatenate([x, near, -near])
    assert np.array_equal(oracle.encode(x, "bf16"), _bf16_nearest_by_search(x))


def test_bf16_search_agrees_with_torch_on_float32_values():
    # The search itself, against torch's float32 -> bf16 cast where that is a single rounding.
    with np.errstate(over="ignore"):
        x = _random_doubles(100_000, -140, 130, 23).astype(np.float32)
    x = x[np.isfinite(x)].astype(np.float64)
    assert np.array_equal(_bf16_nearest_by_search(x), bf16_bits_from_f32(x))


def test_encode_bf16_ties_and_edges():
    # Worked by hand: bf16 keeps 8 significant bits.
    table = {
        257.0: 0x4380,      # tie 256/258 -> 256 (even fraction)
        259.0: 0x4382,      # tie 258/260 -> 260
        1.0 + 2.0 ** -8: 0x3F80,    # tie -> 1.0
        1.0 + 3 * 2.0 ** -8: 0x3F82,
        -1.0 - 2.0 ** -8: 0xBF80,
        (2 - 2.0 ** -7) * 2.0 ** 127: 0x7F7F,   # largest finite bf16
        (2 - 2.0 ** -8) * 2.0 ** 127: 0x7F80,   # halfway to 2^128 -> +inf (odd fraction)
        2.0 ** -133: 0x0001,             # smallest subnormal
        2.0 ** -134: 0x0000,             # tie with zero -> 0
        3 * 2.0 ** -134: 0x0002,         # 1.5 quanta -> 2 quanta
    }
    x = np.array(list(table.keys()))
    assert oracle.encode(x, "bf16").tolist() == list(table.values())


# ----------------------------------------------------------- hand examples


def test_hand_worked_examples():
    data = json.load(open(os.path.join(HERE, "golden", "hand_examples.json")))
    for ex in data["examples"]:
        dt = ex["dtype"]
        A = np.array(ex["A"], dtype=np.float64)
        N = ex.get("N")
        if A.size == 0:
            M, K = len(ex["A"]), 0
            A = np.zeros((M, 0))
            B = np.zeros((0, N))
        else:
            B = np.array(ex["B"], dtype=np.float64)
        enc = oracle.encode
        a_bits, b_bits = enc(A, dt).reshape(A.shape), enc(B, dt).reshape(B.shape)
        # the inputs are exact in their dtype
        assert np.array_equal(oracle.decode(a_bits, dt), A), ex["name"]
        assert np.array_equal(oracle.decode(b_bits, dt), B), ex["name"]
        got = oracle.gemm_relu(a_bits, b_bits, dt)
        want = np.array([[int(h, 16) for h in row] for row in ex["C_bits"]], dtype=np.uint16)
        assert np.array_equal(got, want), (ex["name"], got, want)


# -------------------------------------------------------- exact arithmetic


@pytest.mark.parametrize("shape", [(1, 1, 1), (3, 5, 7), (17, 9, 33), (64, 48, 256), (5, 130, 96)])
def test_integer_inputs_match_exact_integer_matmul_f16(shape):
    M, N, K = shape
    a, b = inputs.integer_pair(M, N, K, torch.float16, seed=M * 1000 + N * 10 + K)
    exact = a.to(torch.int64).numpy() @ b.to(torch.int64).numpy()      # |s| <= 4K <= 1024: exact in fp16
    want = f16_bits(np.maximum(exact, 0).astype(np.float64))
    got = oracle.gemm_relu(a, b, "fp16")
    assert np.array_equal(got, want)
    assert np.array_equal(oracle.decode(got, "fp16"), np.maximum(exact, 0))


@pytest.mark.parametrize("K", [300, 1000, 4100])
def test_integer_inputs_beyond_exact_fp16_range_round_once(K):
    # Sums beyond 2048 are not all fp16 values: the exact integer is rounded once (numpy, RNE).
    M, N = 9, 11
    a, b = inputs.integer_pair(M, N, K, torch.float16, seed=K)
    a = a * 8                                  # entries in {-16..16}: larger sums, more rounding
    exact = a.to(torch.int64).numpy() @ b.to(torch.int64).numpy()
    want = f16_bits(np.maximum(exact, 0).astype(np.float64))
    assert np.array_equal(oracle.gemm_relu(a, b, "fp16"), want)


@pytest.mark.parametrize("K", [8, 64, 512, 8192])
def test_integer_inputs_match_exact_integer_matmul_bf16(K):
    M, N = 6, 13
    a, b = inputs.integer_pair(M, N, K, torch.bfloat16, seed=K + 5)
    exact = a.to(torch.int64).numpy() @ b.to(torch.int64).numpy()      # < 2^24: exact in float32
    want = bf16_bits_from_f32(np.maximum(exact, 0).astype(np.float32))
    assert np.array_equal(oracle.gemm_relu(a, b, "bf16"), want)


def _rne_via_library(x: Fraction, dtype):
    """Round an exact rational when it is an exact double (else None): numpy's double -> fp16
    cast, or for bf16 the search over torch's bf16 value table (any double, not only float32
    values)."""
    d = float(x)
    if Fraction(d) != x:
        return None
    if dtype == "fp16":
        return int(f16_bits(d))
    return int(_bf16_nearest_by_search(np.array([d]))[0])


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_real_valued_tiny_shapes_match_exact_rational_sums(dtype):
    checked = 0
    for seed in range(80):
        M, N, K = 1 + seed % 4, 1 + (seed // 4) % 5, 1 + seed % 8
        tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
        a, b = inputs.normal_pair(M, N, K, tdt, 1.0, seed)
        A = oracle.decode(a, dtype)
        B = oracle.decode(b, dtype)
        got = oracle.gemm_relu(a, b, dtype)
        for i in range(M):
            for j in range(N):
                s = sum((Fraction(A[i, k]) * Fraction(B[k, j]) for k in range(K)), Fraction(0))
                r = s if s > 0 else Fraction(0)
                want = _rne_via_library(r, dtype)
                if want is None:
                    continue
                assert int(got[i, j]) == want, (seed, i, j, s)
                checked += 1
    assert checked >= 500


# ------------------------------------------------- invariants and special cases


def test_relu_invariant_no_negative_no_minus_zero_no_nan():
    a, b = inputs.normal_pair(33, 47, 65, torch.float16, 1.0, 3)
    c = oracle.gemm_relu(a, b, "fp16")
    v = oracle.decode(c, "fp16")
    assert (v >= 0).all() and not np.isnan(v).any()
    assert not (c == 0x8000).any()
    assert (c == 0).sum() > 0.3 * c.size           # about half the sums are negative


def test_complement_identity_recovers_the_pre_relu_product():
    # relu(s) - relu(-s) = s: the negative part that ReLU hides is pinned through -A.
    M, N, K = 20, 30, 200
    a, b = inputs.integer_pair(M, N, K, torch.float16, seed=11)
    pos = oracle.decode(oracle.gemm_relu(a, b, "fp16"), "fp16")
    neg = oracle.decode(oracle.gemm_relu(-a, b, "fp16"), "fp16")
    exact = a.to(torch.int64).numpy() @ b.to(torch.int64).numpy()
    assert np.array_equal(pos - neg, exact)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_identity_b_gives_relu_of_a(dtype):
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    a, _ = inputs.normal_pair(25, 1, 40, tdt, 3.0, 5)
    eye = torch.eye(40, dtype=tdt)
    got = oracle.gemm_relu(a, eye, dtype)
    want = torch.relu(a).view(torch.int16).numpy().view(np.uint16).copy()
    want[want == 0x8000] = 0
    assert np.array_equal(got, want)


def test_zero_a_gives_positive_zero():
    a = torch.zeros(7, 9, dtype=torch.float16)
    _, b = inputs.normal_pair(1, 5, 9, torch.float16, 1.0, 6)
    assert (oracle.gemm_relu(a, b, "fp16") == 0).all()
    assert (oracle.gemm_relu(-a, b, "fp16") == 0).all()     # -0.0 inputs still give +0.0


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_k_equal_one_is_a_rounded_outer_product(dtype):
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    a, b = inputs.normal_pair(31, 29, 1, tdt, 2.0, 9)
    A, B = oracle.decode(a, dtype), oracle.decode(b, dtype)
    prod = np.maximum(A @ B, 0.0)                  # one exact product per element
    if dtype == "fp16":
        want = f16_bits(prod)
    else:
        # the product of two bf16 values has <= 16 significant bits: exact in float32
        assert np.array_equal(prod.astype(np.float32).astype(np.float64), prod)
        want = bf16_bits_from_f32(prod)
    assert np.array_equal(oracle.gemm_relu(a, b, dtype), want)


def test_transpose_identity_pins_the_axes():
    # ReLU(A B)^T = ReLU(B^T A^T): same products in the same k order.
    a, b = inputs.normal_pair(13, 21, 17, torch.float16, 1.0, 12)
    c = oracle.gemm_relu(a, b, "fp16")
    ct = oracle.gemm_relu(b.t().contiguous(), a.t().contiguous(), "fp16")
    assert np.array_equal(c.T, ct)


def test_row_permutation_of_a_permutes_rows_of_c():
    a, b = inputs.normal_pair(19, 8, 23, torch.float16, 1.0, 13)
    perm = torch.randperm(19, generator=torch.Generator().manual_seed(1))
    c = oracle.gemm_relu(a, b, "fp16")
    cp = oracle.gemm_relu(a[perm].contiguous(), b, "fp16")
    assert np.array_equal(c[perm.numpy()], cp)


def test_degenerate_shapes():
    e = torch.zeros
    assert oracle.gemm_relu(e(0, 4, dtype=torch.float16), e(4, 3, dtype=torch.float16), "fp16").shape == (0, 3)
    assert oracle.gemm_relu(e(2, 4, dtype=torch.float16), e(4, 0, dtype=torch.float16), "fp16").shape == (2, 0)
    c = oracle.gemm_relu(e(3, 0, dtype=torch.float16), e(0, 5, dtype=torch.float16), "fp16")
    assert c.shape == (3, 5) and (c == 0).all()


def test_rows_entries_and_thread_count_agree_with_full_oracle():
    a, b = inputs.normal_pair(40, 70, 90, torch.bfloat16, 1.0, 14)
    full = oracle.gemm_relu(a, b, "bf16", threads=1)
    assert np.array_equal(full, oracle.gemm_relu(a, b, "bf16", threads=4))
    assert np.array_equal(full[7:29], oracle.gemm_relu_rows(a, b, "bf16", 7, 29))
    rng = np.random.default_rng(0)
    ii, jj = rng.integers(0, 40, 200), rng.integers(0, 70, 200)
    assert np.array_equal(full[ii, jj], oracle.gemm_relu_entries(a, b, "bf16", ii, jj))


# ---------------------------------------------------------- planted mistakes

MUTANTS = {
    # a dropped term: the last k is skipped
    "drops_last_k": ("for (int64_t k = 0; k < K; ++k) {\n                    uint16_t abits",
                     "for (int64_t k = 0; k + 1 < K; ++k) {\n                    uint16_t abits"),
    # a wrong column index of B
    "mirrors_b_columns": ("acc[j] += a * brow[j];", "acc[j] += a * brow[N - 1 - j];"),
    # a wrong sign handling: |s| instead of max(s, 0)
    "abs_instead_of_relu": ("double r = s > 0.0 ? s : 0.0;", "double r = s > 0.0 ? s : -s;"),
    # truncation instead of round-to-nearest-even
    "truncating_cast": ("double n = rint(", "double n = trunc("),
    # ReLU applied to the wrong sign
    "keeps_negative_part": ("double r = s > 0.0 ? s : 0.0;", "double r = s < 0.0 ? -s : 0.0;"),
    # double rounding: the fp64 sum rounded to float32 before the bf16 cast
    "bf16_through_float32": ("uint16_t oracle_f64_to_bf16(double x) { return encode_rne(x,",
                             "uint16_t oracle_f64_to_bf16(double x) { return encode_rne((double)(float)x,"),
}


def _build_mutant(tmp_path, name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "gemm_relu_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"{name}.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", str(path), "-o", str(so), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    u16p = ctypes.POINTER(ctypes.c_uint16)
    i64 = ctypes.c_int64
    lib.oracle_gemm_relu.argtypes = [u16p, u16p, u16p, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    return lib


def _pins_pass(lib):
    """The core pins, run against a given oracle library; False if any of them fails."""
    u16p = ctypes.POINTER(ctypes.c_uint16)

    def run(a, b):
        ab = a.contiguous().view(torch.int16).numpy().view(np.uint16)
        bb = b.contiguous().view(torch.int16).numpy().view(np.uint16)
        M, K = ab.shape
        N = bb.shape[1]
        c = np.zeros((M, N), dtype=np.uint16)
        dt = 1 if a.dtype == torch.bfloat16 else 0
        lib.oracle_gemm_relu(ab.ctypes.data_as(u16p), bb.ctypes.data_as(u16p), c.ctypes.data_as(u16p),
                             M, N, K, dt, 0)
        return c

    a, b = inputs.integer_pair(9, 7, 33, torch.float16, seed=2)
    exact = a.to(torch.int64).numpy() @ b.to(torch.int64).numpy()
    if not np.array_equal(run(a, b), f16_bits(np.maximum(exact, 0).astype(np.float64))):
        return False
    data = json.load(open(os.path.join(HERE, "golden", "hand_examples.json")))
    for ex in data["examples"]:
        if not ex["B"]:
            continue
        tdt = torch.float16 if ex["dtype"] == "fp16" else torch.bfloat16
        A, B = np.array(ex["A"], dtype=np.float64), np.array(ex["B"], dtype=np.float64)
        got = run(torch.from_numpy(A).to(tdt), torch.from_numpy(B).to(tdt))
        want = np.array([[int(h, 16) for h in row] for row in ex["C_bits"]], dtype=np.uint16)
        if not np.array_equal(got, want):
            return False
    return True


def test_pins_accept_the_oracle(tmp_path):
    lib = ctypes.CDLL(oracle.build())
    u16p = ctypes.POINTER(ctypes.c_uint16)
    lib.oracle_gemm_relu.argtypes = [u16p, u16p, u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_int, ctypes.c_int]
    assert _pins_pass(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistakes(tmp_path, name):
    assert not _pins_pass(_build_mutant(tmp_path, name)), name
