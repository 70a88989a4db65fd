"""Host-side checks of the C ABI: the library loads, exports every declared entry
point, and validates arguments before touching a device.  No GPU is needed and
no kernel is launched: every call below returns from argument checking, or is
the pure-host configuration query.
"""
import ctypes
import os
import re

import pytest

import tiled_dense_gemm_relu_amd as gr
from tiled_dense_gemm_relu_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_relu.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gemm_relu\w*)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return gr.load_library()


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted([
        "gemm_relu", "gemm_relu_with_config", "gemm_relu_query_config", "gemm_relu_strerror",
        "gemm_relu_version", "gemm_relu_ex", "gemm_relu_query_config_ex", "gemm_relu_splitk",
        "gemm_relu_query_splitk", "gemm_relu_selected_config", "gemm_relu_splitk_noalloc"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_strerror(lib):
    assert lib.gemm_relu_version() >= 100
    for code in list(binding.ERRORS) + [-99]:
        assert isinstance(gr.strerror(code), str) and gr.strerror(code)
    assert gr.strerror(0) == "ok"


# Fake, well separated addresses: the calls below must fail argument checks
# before any device work, so these are never dereferenced.
A_PTR, B_PTR, C_PTR = 1 << 32, 2 << 32, 3 << 32


@pytest.mark.parametrize("args,code", [
    ((A_PTR, B_PTR, C_PTR, 4, 4, 4, 7), -2),                 # bad dtype
    ((A_PTR, B_PTR, C_PTR, -1, 4, 4, 0), -1),                # negative M
    ((A_PTR, B_PTR, C_PTR, 4, -1, 4, 0), -1),
    ((A_PTR, B_PTR, C_PTR, 4, 4, -1, 0), -1),
    ((A_PTR, B_PTR, 0, 4, 4, 4, 0), -1),                     # null C with work to do
    ((0, B_PTR, C_PTR, 4, 4, 4, 0), -1),                     # null A with K > 0
    ((A_PTR, 0, C_PTR, 4, 4, 4, 0), -1),
    ((A_PTR + 1, B_PTR, C_PTR, 4, 4, 4, 0), -4),             # odd address
    ((A_PTR, B_PTR, C_PTR + 1, 4, 4, 4, 1), -4),
    ((A_PTR, B_PTR, A_PTR + 6, 4, 4, 4, 0), -3),             # C overlaps A
    ((A_PTR, B_PTR, B_PTR - 8, 4, 4, 4, 0), -3),             # C overlaps B
    ((A_PTR, B_PTR, C_PTR, (1 << 24) + 1, 4, 4, 0), -7),     # beyond the size limits
    ((A_PTR, B_PTR, C_PTR, 4, 4, (1 << 22) + 1, 0), -7),
])
def test_invalid_arguments_are_rejected_before_launch(lib, args, code):
    a, b, c, M, N, K, dt = args
    assert lib.gemm_relu(a, b, c, M, N, K, dt, None) == code
    assert lib.gemm_relu_query_config(a, b, c, M, N, K, dt, -1, None) == code
    # B stored (N, K) occupies the same bytes: the same checks apply
    for b_layout in (gr.B_KN, gr.B_NK):
        assert lib.gemm_relu_ex(a, b, c, M, N, K, dt, b_layout, -1, None) == code
        assert lib.gemm_relu_query_config_ex(a, b, c, M, N, K, dt, b_layout, -1, None) == code


def test_unknown_b_layout_is_rejected(lib):
    for b_layout in (2, -1):
        assert lib.gemm_relu_ex(A_PTR, B_PTR, C_PTR, 4, 4, 4, 0, b_layout, -1, None) == -9
        assert lib.gemm_relu_query_config_ex(A_PTR, B_PTR, C_PTR, 4, 4, 4, 0, b_layout, -1, None) == -9
    assert "layout" in gr.strerror(-9)


def test_unknown_config_is_rejected(lib):
    assert lib.gemm_relu_with_config(A_PTR, B_PTR, C_PTR, 4, 4, 4, 0, 11, None) == -8
    assert lib.gemm_relu_with_config(A_PTR, B_PTR, C_PTR, 4, 4, 4, 0, -2, None) == -8


def test_empty_outputs_are_a_no_op(lib):
    # M == 0 or N == 0: nothing to write, OK without touching a device (null pointers allowed).
    assert lib.gemm_relu(0, 0, 0, 0, 5, 5, 0, None) == 0
    assert lib.gemm_relu(0, 0, 0, 5, 0, 5, 1, None) == 0


def test_k_zero_needs_no_inputs():
    cfg = gr.selected_config(3, 5, 0, a_ptr=0, b_ptr=0)
    assert cfg["grid"] >= 1 and cfg["threads"] == 256


def test_config_choice_for_the_workload_shapes():
    big = gr.selected_config(8192, 8192, 8192)
    assert (big["config_id"], big["block_m"], big["block_n"], big["block_k"]) == (3, 256, 256, 64)
    # the 128 KiB ring plus 8 waves x 4 KiB of C staging: the whole 160 KiB
    assert (big["stages"], big["vec_a"], big["vec_b"], big["grid"], big["lds_bytes"]) == (2, 8, 8, 1024, 163840)
    small = gr.selected_config(1024, 1024, 1024)
    # 64x64x64 tiles with 4 producer waves in 4 stages (the tuned choice)
    assert (small["config_id"], small["block_m"], small["stages"], small["threads"], small["grid"]) == (9, 64, 4, 512, 256)
    mid = gr.selected_config(2048, 2048, 2048)
    assert (mid["config_id"], mid["block_m"], mid["threads"], mid["grid"]) == (10, 128, 512, 256)   # producer waves
    ragged = gr.selected_config(4000, 11000, 4100)
    assert ragged["config_id"] == 3 and ragged["grid"] == 16 * 43
    # K % 8 == 4: 16-byte A DMA lanes, BK = 64 in 2 stages; the piece straddling K is rewritten in LDS
    assert (ragged["vec_a"], ragged["vec_b"], ragged["block_k"], ragged["stages"]) == (8, 8, 64, 2)
    odd = gr.selected_config(4000, 11000, 4101)
    assert (odd["config_id"], odd["vec_a"]) == (1, 1)               # odd K: register-staged kernel
    skinny = gr.selected_config(64, 16384, 8192, dtype=gr.BF16)
    assert (skinny["config_id"], skinny["grid"]) == (9, 256)


@pytest.mark.parametrize("K,N,a_off,b_off,want", [
    (8, 8, 0, 0, (8, 8)), (12, 8, 0, 0, (4, 8)), (8, 12, 0, 0, (8, 4)), (6, 6, 0, 0, (2, 2)),
    (7, 8, 0, 0, (1, 1)), (8, 8, 8, 0, (4, 8)), (8, 8, 2, 2, (1, 1)),
])
def test_load_width_follows_row_length_and_alignment(K, N, a_off, b_off, want):
    cfg = gr.selected_config(512, N, K, config=1, a_ptr=4096 + a_off, b_ptr=(1 << 20) + b_off)
    assert (cfg["vec_a"], cfg["vec_b"]) == want


def test_dma_config_falls_back_without_suitable_loads():
    assert gr.selected_config(512, 512, 512, config=3)["config_id"] == 3
    cfg = gr.selected_config(512, 512, 516, config=3)            # K % 8 != 0: still 16-byte A lanes
    assert (cfg["config_id"], cfg["vec_a"], cfg["vec_b"], cfg["block_k"]) == (3, 8, 8, 64)
    cfg = gr.selected_config(512, 518, 512, config=3)            # N % 8 != 0: 4-byte B lanes
    assert (cfg["config_id"], cfg["vec_a"], cfg["vec_b"], cfg["block_k"]) == (3, 8, 2, 32)
    cfg = gr.selected_config(512, 518, 516, config=3)            # ... and then 4-byte A lanes too
    assert (cfg["config_id"], cfg["vec_a"], cfg["vec_b"]) == (3, 2, 2)
    cfg = gr.selected_config(512, 512, 515, config=3)            # odd K: register-staged kernel
    assert (cfg["config_id"], cfg["vec_a"]) == (1, 1)
    cfg = gr.selected_config(512, 512, 512, config=3, a_ptr=4096 + 8)   # A only 8-byte aligned: 16-byte lanes
    assert (cfg["config_id"], cfg["vec_a"]) == (3, 8)
    cfg = gr.selected_config(512, 512, 512, config=3, a_ptr=4096 + 4)   # ... or 4-byte aligned
    assert (cfg["config_id"], cfg["vec_a"]) == (3, 8)
    cfg = gr.selected_config(512, 512, 512, config=4, a_ptr=4096 + 8)   # other DMA tiles need 16-byte rows
    assert cfg["config_id"] == 2
    assert gr.selected_config(512, 512, 512, config=3, a_ptr=4096 + 2)["config_id"] == 1
    for dma in (4, 5):
        assert gr.selected_config(512, 512, 512, config=dma)["config_id"] == dma
        assert gr.selected_config(512, 512, 516, config=dma)["config_id"] == 2


def test_direct_config_geometry():
    cfg = gr.selected_config(100, 70, 9, config=0)
    assert (cfg["block_m"], cfg["block_n"], cfg["threads"], cfg["grid"]) == (32, 32, 64, 4 * 3)


def nt_config(M, N, K, **kw):
    return gr.selected_config(M, N, K, b_layout=gr.B_NK, **kw)


def test_few_tiles_deep_k_takes_32x32_producer_tiles():
    # 64x64 tiles would leave at least half the CUs idle: the plain entry point
    # takes 32x32 tiles with producer waves (4 times as many tiles)
    cfg = gr.selected_config(512, 512, 2048)
    assert (cfg["config_id"], cfg["block_m"], cfg["block_n"], cfg["threads"], cfg["grid"]) == (8, 32, 32, 320, 256)
    assert gr.selected_config(512, 512, 2048, b_layout=gr.B_NK)["config_id"] == 8
    assert gr.selected_config(512, 520, 1024)["config_id"] == 8         # any K
    assert gr.selected_config(1024, 1024, 4096)["config_id"] == 9       # 256 tiles of 64x64, producer waves
    # split-K entry: 256 tiles do not split, so the producer tiles too; asked for parts, the 64x64
    # tile without producers (it has split-K instances)
    assert (gr.selected_splitk_config(1024, 1024, 4096)["config_id"], gr.selected_splitk_config(1024, 1024, 4096)["splits"]) == (9, 1)
    sk4 = gr.selected_splitk_config(1024, 1024, 4096, splits=4)
    assert (sk4["config_id"], sk4["splits"]) == (5, 4)
    # the split-K entry point keeps the 64x64 tile and splits K instead
    sk = gr.selected_splitk_config(512, 512, 2048 + 64)
    assert (sk["config_id"], sk["splits"] > 1) == (5, True)
    # forced, it runs unsplit on either entry point; without 16-byte loads it falls back
    assert gr.selected_splitk_config(512, 512, 4096, config=8)["splits"] == 1
    assert gr.selected_config(512, 512, 2052, config=8)["config_id"] == 2
    assert gr.selected_config(512, 512, 2052, config=8, b_layout=gr.B_NK)["config_id"] == 3


def test_wide_decode_shapes_take_the_64x256_tile():
    # at most 64 rows over 256 or more 64x256 tiles: the 64x256 tile, unsplit, 4 stages, staged C
    cfg = gr.selected_config(64, 65536, 2048, dtype=gr.BF16)
    assert (cfg["config_id"], cfg["block_m"], cfg["block_n"], cfg["block_k"], cfg["stages"], cfg["grid"],
            cfg["splits"]) == (6, 64, 256, 32, 4, 256, 1)
    assert cfg["lds_bytes"] == 4 * (64 + 256) * 32 * 2 + 4 * 4096
    assert gr.selected_config(32, 65536, 4096, dtype=gr.BF16)["config_id"] == 6
    assert gr.selected_config(1, 131072, 64)["config_id"] == 6
    # 255 such tiles or more than 64 rows: the other rules
    assert gr.selected_config(64, 65280, 2048, dtype=gr.BF16)["config_id"] == 3
    assert gr.selected_config(65, 65536, 2048, dtype=gr.BF16)["config_id"] == 3
    assert gr.selected_config(64, 32768, 4096, dtype=gr.BF16)["config_id"] == 10
    # B stored (N, K), at most 64 rows: the 64x64 producer tile (32x32 when 64x64 tiles are few)
    assert gr.selected_config(64, 65536, 2048, dtype=gr.BF16, b_layout=gr.B_NK)["config_id"] == 9
    assert gr.selected_config(16, 32768, 8192, dtype=gr.BF16, b_layout=gr.B_NK)["config_id"] == 9
    assert gr.selected_config(64, 4096, 8192, dtype=gr.BF16, b_layout=gr.B_NK)["config_id"] == 8
    assert gr.selected_config(65, 65536, 2048, dtype=gr.BF16, b_layout=gr.B_NK)["config_id"] == 3
    # without 16-byte loads of B: the 256 tile's 4-byte lanes (N even), else the register-staged tiles
    assert gr.selected_config(64, 65538, 2048, dtype=gr.BF16)["config_id"] == 3
    assert gr.selected_config(64, 65537, 2048, dtype=gr.BF16)["config_id"] in (1, 2)


def test_b_nk_config_choice():
    big = nt_config(8192, 8192, 8192)
    assert (big["config_id"], big["vec_a"], big["vec_b"], big["b_layout"]) == (3, 8, 8, gr.B_NK)
    assert gr.selected_config(8192, 8192, 8192)["b_layout"] == gr.B_KN
    assert nt_config(1024, 1024, 1024)["config_id"] == 9
    assert nt_config(2048, 2048, 2048)["config_id"] == 10
    assert nt_config(64, 16384, 8192, dtype=gr.BF16)["config_id"] == 9
    # B^T rows have length K: N no longer matters for the load width
    assert nt_config(1024, 1000, 1024)["config_id"] == 9
    assert nt_config(4000, 11003, 4096)["vec_b"] == 8
    # K even but not a multiple of 8: the 256 kernel, 16-byte lanes for both operands, the
    # pieces straddling K rewritten in LDS (BK = 64 in 2 stages)
    cfg = nt_config(1024, 1024, 1030)
    assert (cfg["config_id"], cfg["vec_a"], cfg["vec_b"], cfg["block_k"], cfg["stages"]) == (3, 8, 8, 64, 2)
    cfg = nt_config(8192, 8192, 8192, b_ptr=(1 << 20) + 4)           # B^T only 4-byte aligned
    assert (cfg["config_id"], cfg["vec_a"], cfg["vec_b"], cfg["block_k"]) == (3, 8, 8, 64)
    # odd K, or 2-byte alignment: the register-staged kernels, which load B^T like A
    cfg = nt_config(1024, 1024, 1031)
    assert (cfg["config_id"], cfg["vec_a"], cfg["vec_b"]) == (2, 1, 1)
    cfg = nt_config(8192, 8192, 8192, a_ptr=4096 + 2)                # (1, 8) has no instance: (1, 1)
    assert (cfg["config_id"], cfg["vec_a"], cfg["vec_b"]) == (1, 1, 1)
    cfg = nt_config(8192, 8192, 8190, b_ptr=(1 << 20) + 2)           # B^T rows of an even length, 2-byte aligned
    assert (cfg["config_id"], cfg["vec_b"]) == (1, 1)


def test_b_nk_forced_configs():
    # the register-staged kernels read B^T too (TILE_* means them in both layouts)
    assert nt_config(512, 512, 512, config=1)["config_id"] == 1
    assert nt_config(512, 512, 512, config=2)["config_id"] == 2
    for dma in (3, 4, 5):
        assert nt_config(512, 512, 512, config=dma)["config_id"] == dma
        assert nt_config(512, 512, 516, config=dma)["config_id"] == 3      # K even: the 256 DMA tile
    assert nt_config(512, 512, 515, config=3)["config_id"] == 1             # odd K: register-staged
    for dma in (4, 5, 8, 9, 10):
        assert nt_config(512, 512, 515, config=dma)["config_id"] == 2
    assert nt_config(512, 512, 515, config=0)["config_id"] == 0
    cfg = nt_config(512, 512, 516, config=1)
    assert (cfg["config_id"], cfg["vec_a"], cfg["vec_b"]) == (1, 4, 4)     # K % 8 == 4: 4-element loads


def test_splitk_config_choice():
    # an untuned skinny shape: the 64x256 tile with enough parts for 256 units
    skinny = gr.selected_splitk_config(64, 16384, 8192 + 64, dtype=gr.BF16)
    assert (skinny["config_id"], skinny["splits"], skinny["grid"]) == (6, 4, 256)
    skinny = gr.selected_splitk_config(64, 16384, 8192, dtype=gr.BF16, config=6)
    # the fixed 64 KiB counter region + 4 fp32 partial tiles per tile
    assert skinny["workspace_bytes"] == 65536 + 64 * 4 * 64 * 256 * 4
    # enough tiles already: no split, no workspace
    big = gr.selected_splitk_config(8192, 8192, 8192)
    assert (big["config_id"], big["splits"], big["workspace_bytes"]) == (3, 1, 0)
    # explicit parts, capped by the K-steps
    cfg = gr.selected_splitk_config(1024, 1024, 1024, config=4, splits=4)
    assert (cfg["splits"], cfg["grid"]) == (4, 256)
    assert gr.selected_splitk_config(128, 128, 128, config=4, splits=8)["splits"] == 2
    assert gr.selected_splitk_config(1024, 1024, 1024, config=4, splits=64)["splits"] == 16
    # the 256 tile and the register-staged kernels do not split
    assert gr.selected_splitk_config(512, 512, 512, config=3, splits=4)["splits"] == 1
    assert gr.selected_splitk_config(64, 512, 514, splits=4)["splits"] == 1          # K % 8 != 0
    # more tiles than the counter region holds (16384 counters, 4 waves per tile): no split
    assert gr.selected_splitk_config(64 * 4097, 64, 1024, config=5, splits=2)["splits"] == 1
    assert gr.selected_splitk_config(64 * 4096, 64, 1024, config=5, splits=2)["splits"] == 2
    # the plain entry points never split
    assert gr.selected_config(64, 16384, 8192)["splits"] == 1


def test_splitk_argument_errors(lib):
    args = (A_PTR, B_PTR, C_PTR, 64, 512, 512, 0, 0, -1)
    assert lib.gemm_relu_query_splitk(*args, -1, None) == -1
    assert lib.gemm_relu_query_splitk(*args, 65, None) == -1
    assert lib.gemm_relu_splitk(*args, 4, None, 0, None) == -10                   # no workspace
    need = gr.selected_splitk_config(64, 512, 512, splits=4)["workspace_bytes"]
    ws = 5 << 32
    assert lib.gemm_relu_splitk(*args, 4, ws, need - 1, None) == -10              # too small
    assert lib.gemm_relu_splitk(*args, 4, ws + 16, need, None) == -10             # misaligned
    assert lib.gemm_relu_splitk(*args, 4, C_PTR, need, None) == -3                # overlaps C
    assert lib.gemm_relu_splitk(A_PTR, B_PTR, C_PTR, 64, 512, 512, 0, 2, -1, 4, ws, need, None) == -9


def tuned_table():
    """Rows of the compiled-in table, parsed from its source."""
    path = os.path.join(ROOT, "tiled_dense_gemm_relu_amd", "csrc", "tuned_table.inc")
    rows = []
    for line in open(path):
        m = re.match(r"\{(.*)\},\s*$", line.strip())
        if m:
            rows.append(tuple(int(v) for v in m.group(1).split(",")))
    return rows


def test_tuned_table_rows_are_what_auto_selects():
    rows = tuned_table()
    assert len(rows) >= 10
    assert len({r[:5] for r in rows}) == len(rows)                       # one row per shape
    for M, N, K, dt, layout, config, sk_config, splits in rows:
        assert 0 <= config <= 10 and 0 <= sk_config <= 10 and 1 <= splits <= 64
        plain = gr.selected_config(M, N, K, dtype=dt, b_layout=layout)
        assert (plain["config_id"], plain["splits"]) == (config, 1), (M, N, K, layout)
        sk = gr.selected_splitk_config(M, N, K, dtype=dt, b_layout=layout)
        assert (sk["config_id"], sk["splits"]) == (sk_config, splits), (M, N, K, layout)


def test_tuned_table_needs_the_tuners_alignment():
    # The deep shape is tuned to split in 4 (and to 32x32 producer tiles without
    # split-K); with B only 4-byte aligned the table does not apply and the
    # heuristics choose (the register-staged 128 tile).
    rows = {r[:5]: r for r in tuned_table()}
    assert rows[(512, 512, 16384, 0, 0)][5:] == (8, 5, 4)
    sk = gr.selected_splitk_config(512, 512, 16384, b_ptr=(1 << 20) + 4)
    assert (sk["config_id"], sk["splits"]) == (2, 1)


def test_wave_specialised_config():
    cfg = gr.selected_config(8192, 8192, 8192, config=7)
    assert (cfg["config_id"], cfg["block_m"], cfg["block_n"], cfg["block_k"], cfg["threads"]) == (7, 256, 128, 32, 768)
    assert (cfg["grid"], cfg["lds_bytes"]) == (32 * 64, 4 * 384 * 32 * 2 + 8 * 4096)
    assert gr.selected_config(8192, 8192, 8192, config=7, b_layout=gr.B_NK)["config_id"] == 7
    # needs 16-byte loads: else the 256 tile of the layout's fallback family
    assert gr.selected_config(512, 512, 516, config=7)["config_id"] == 1
    assert gr.selected_config(512, 512, 516, config=7, b_layout=gr.B_NK)["config_id"] == 3
    # never split
    assert gr.selected_splitk_config(512, 512, 4096, config=7, splits=4)["splits"] == 1


@pytest.mark.parametrize("shape", [
    (256, 256, 256, 0), (1024, 1024, 1024, 0), (2048, 2048, 2048, 0), (8192, 8192, 8192, 0),
    (4000, 11000, 4100, 0), (64, 16384, 8192, 1), (512, 512, 16384, 0), (8192, 8192, 8192, 1),
    (100, 70, 9, 0), (4000, 11000, 4101, 0), (512, 518, 516, 0), (3, 5, 0, 0), (1, 1, 1, 1)])
def test_selected_config_agrees_with_the_full_query(lib, shape):
    # gemm_relu_selected_config (the block sizes and stage count the pages' kernel factory takes)
    # reports what gemm_relu_query_config gives for separate, 256-byte aligned buffers.
    M, N, K, dt = shape
    base = 1 << 32
    a, b, c = base, base + (1 << 36), base + (2 << 36)
    q = gr.selected_config(M, N, K, dtype=dt, a_ptr=a, b_ptr=b, c_ptr=c)
    assert gr.selected_block_config(M, N, K, dt) == (q["block_m"], q["block_n"], q["block_k"], q["stages"])


def test_selected_config_values_and_errors(lib):
    assert gr.selected_block_config(8192, 8192, 8192) == (256, 256, 64, 2)
    assert gr.selected_block_config(1024, 1024, 1024) == (64, 64, 64, 4)
    out = [ctypes.c_int(-7) for _ in range(4)]
    refs = [ctypes.byref(v) for v in out]
    assert lib.gemm_relu_selected_config(4, 4, 4, 5, *refs) == -2              # bad dtype
    assert lib.gemm_relu_selected_config(-1, 4, 4, 0, *refs) == -1             # negative M
    assert lib.gemm_relu_selected_config(4, 4, (1 << 22) + 1, 0, *refs) == -7  # too large
    assert [v.value for v in out] == [-7] * 4                                  # untouched on error
    assert lib.gemm_relu_selected_config(64, 64, 64, 0, None, None, None, None) == 0


def test_explicit_parts_are_never_dropped_by_the_tuned_table():
    # 2048^3 is tuned to the 128x128 producer-wave tile, which has no split-K kernels: asked for
    # 4 parts, AUTO takes the 128x128 tile that splits, as for an untuned shape of that size.
    sk = gr.selected_splitk_config(2048, 2048, 2048, splits=4)
    assert (sk["config_id"], sk["splits"]) == (4, 4)
    untuned = gr.selected_splitk_config(2048, 2048, 2048 + 8, splits=4)
    assert (untuned["config_id"], untuned["splits"]) == (4, 4)
    # the skinny shape with B stored (N, K) is tuned unsplit on the 64x64 producer tile; asked for
    # 2 parts it takes the 64x64 tile that splits (the 64x256 rule for M <= 64 is for B (K, N))
    sk = gr.selected_splitk_config(64, 16384, 8192, dtype=gr.BF16, splits=2, b_layout=gr.B_NK)
    assert (sk["config_id"], sk["splits"]) == (5, 2)
    sk = gr.selected_splitk_config(64, 16384, 8192 + 64, dtype=gr.BF16, b_layout=gr.B_NK)
    assert (sk["config_id"], sk["splits"]) == (9, 1)   # untuned: 256 tiles of 64x64 need no parts
    # with the parts left to the library, the table still decides
    sk = gr.selected_splitk_config(64, 16384, 8192, dtype=gr.BF16, b_layout=gr.B_NK)
    assert (sk["config_id"], sk["splits"]) == (9, 1)
    # a tuned row whose split-K tile does split keeps it for explicit parts (deep K: 64x64, 4 parts)
    sk = gr.selected_splitk_config(512, 512, 16384, splits=2)
    assert (sk["config_id"], sk["splits"]) == (5, 2)


def test_noalloc_rejects_calls_beyond_its_scratch(lib):
    # gemm_relu_splitk_noalloc keeps partials in a static device array; a call needing more is
    # refused on the host before anything is launched (no device is touched here).
    args = (A_PTR, B_PTR, C_PTR, 8192, 8192, 1024, 0, 0, 4)      # 128x128 tiles, forced
    need = gr.selected_splitk_config(8192, 8192, 1024, config=4, splits=2)
    assert need["splits"] == 2 and need["workspace_bytes"] > binding.NOALLOC_SCRATCH_BYTES
    assert lib.gemm_relu_splitk_noalloc(*args, 2, None) == -11
    assert "scratch" in gr.strerror(-11)
    # the usual argument errors come first
    assert lib.gemm_relu_splitk_noalloc(A_PTR, B_PTR, C_PTR, 64, 512, 512, 9, 0, -1, 4, None) == -2
    assert lib.gemm_relu_splitk_noalloc(A_PTR, B_PTR, C_PTR, 64, 512, 512, 0, 0, -1, 65, None) == -1
    assert lib.gemm_relu_splitk_noalloc(A_PTR, B_PTR, A_PTR + 2, 64, 512, 512, 0, 0, -1, 4, None) == -3
    # M == 0: nothing to do, no device needed
    assert lib.gemm_relu_splitk_noalloc(0, 0, 0, 0, 512, 512, 0, 0, -1, 4, None) == 0
    # the header's size is the binding's
    text = open(HEADER).read()
    assert "#define GEMM_RELU_NOALLOC_SCRATCH_BYTES ((int64_t)65536 + ((int64_t)32 << 20))" in text
    # every split the library chooses by itself fits: fewer than 192 tiles, parts for about 256
    # units, so at most 447 partial tiles of at most 64 KiB
    sizes = [64, 128, 192, 256, 320, 512, 640, 1024, 1536, 1792, 2048, 2304]
    split_seen = 0
    for M in sizes:
        for N in sizes + [16384]:
            for dt in (0, 1):
                for layout in (gr.B_KN, gr.B_NK):
                    cfg = gr.selected_splitk_config(M, N, 4096, dtype=dt, b_layout=layout)
                    assert cfg["workspace_bytes"] <= binding.NOALLOC_SCRATCH_BYTES, (M, N, dt, layout, cfg)
                    split_seen += cfg["splits"] > 1
    assert split_seen > 50
