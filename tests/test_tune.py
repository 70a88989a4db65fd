"""Host-side checks of the offline tile-configuration search (no GPU: the
candidate enumeration is pure configuration queries, and the table writer is
plain text)."""
import re

import tiled_dense_gemm_relu_amd as gr
from tiled_dense_gemm_relu_amd import tune


def test_parse_shape():
    assert tune.parse_shape("64,16384,8192,bf16,nk") == (64, 16384, 8192, "bf16", 1)
    assert tune.parse_shape("512,512,512") == (512, 512, 512, "fp16", 0)


def test_default_shapes_cover_the_workloads_in_both_layouts():
    shapes = tune.default_shapes()
    assert (8192, 8192, 8192, "fp16", 0) in shapes and (8192, 8192, 8192, "fp16", 1) in shapes
    assert (64, 16384, 8192, "bf16", 0) in shapes
    assert len(set(shapes)) == len(shapes)


def test_candidates_are_distinct_resolved_configurations():
    cands = tune.candidates(512, 512, 16384, gr.F16, gr.B_KN)
    assert len(cands) == len(set(cands))
    assert all(0 <= c <= 10 and 1 <= s <= 16 for c, s in cands)
    assert (5, 4) in cands and (3, 1) in cands           # split-K on the 64 tile, the 256 tile
    assert (8, 1) in cands                               # 32x32 tiles with producer waves
    assert (0, 1) not in cands                           # the direct kernel only when nothing else runs
    # every candidate is what the library resolves a request to
    for c, s in cands:
        r = gr.selected_splitk_config(512, 512, 16384, config=c, splits=s) if s > 1 else \
            gr.selected_config(512, 512, 16384, config=c)
        assert (r["config_id"], r["splits"]) == (c, s)
    # odd K: only the kernels that take 2-byte loads remain, the register-staged ones in both layouts
    assert tune.candidates(100, 100, 101, gr.F16, gr.B_NK) == [(1, 1), (2, 1)]
    assert tune.candidates(100, 100, 101, gr.F16, gr.B_KN) == [(1, 1), (2, 1)]


def test_split_candidates_respect_the_workspace_cap():
    for c, s in tune.candidates(8192, 8192, 8192, gr.F16, gr.B_KN):
        if s > 1:
            assert gr.selected_splitk_config(8192, 8192, 8192, config=c, splits=s)["workspace_bytes"] <= \
                tune.MAX_WORKSPACE


def test_write_table_round_trips(tmp_path):
    entries = [{"M": 8, "N": 16, "K": 24, "dtype": "bf16", "b_layout": 1, "config": 5, "splitk_config": 6,
                "splits": 4}]
    path = tmp_path / "t.inc"
    tune.write_table(entries, "test device", str(path))
    rows = [tuple(int(v) for v in m.group(1).split(","))
            for m in (re.match(r"\{(.*)\},\s*$", l.strip()) for l in path.read_text().splitlines()) if m]
    assert rows == [(8, 16, 24, 1, 1, 5, 6, 4)]


def test_choose_plain_keeps_the_incumbent_within_the_margin():
    final = {(9, 1): 0.0610, (5, 1): 0.0609, (5, 2): 0.0594}
    # 5 is faster than the incumbent 9 by 0.2%: not enough to replace it
    assert tune.choose_plain(final, incumbent=9) == (0.0610, (9, 1))
    # a candidate more than 2% faster replaces it
    final[(10, 1)] = 0.0590
    assert tune.choose_plain(final, incumbent=9) == (0.0590, (10, 1))
    # an incumbent that was not timed (or is not a plain candidate) does not count
    assert tune.choose_plain({(9, 1): 0.05, (5, 1): 0.0499}, incumbent=3) == (0.0499, (5, 1))
    # split candidates never become the plain choice
    assert tune.choose_plain({(9, 1): 0.05, (5, 4): 0.01}, incumbent=9) == (0.05, (9, 1))


def test_time_alternating_takes_turns_and_medians(monkeypatch):
    """Finalists are timed region by region in turn (a drifting clock reaches each alike), each
    warmed up first, and each gets the median of its own regions."""
    warm, calls = [], []
    launchers = {name: (lambda i, name=name: warm.append(name)) for name in ("a", "b")}
    name_of = {id(f): name for name, f in launchers.items()}
    scripted = {"a": iter([3.0, 1.0, 2.0]), "b": iter([5.0, 9.0, 4.0])}

    def fake_region(launch, launches):
        calls.append(name_of[id(launch)])
        return next(scripted[name_of[id(launch)]])

    monkeypatch.setattr(tune, "time_region", fake_region)
    assert tune.time_alternating(launchers, launches=4, regions=3) == {"a": 2.0, "b": 5.0}
    assert calls == ["a", "b", "a", "b", "a", "b"]
    assert warm == ["a"] * 4 + ["b"] * 4
