"""The build's kernel-source digest, which stamps every profile: comments do not change it, code does."""
import os
import shutil

from tiled_dense_gemm_relu_amd import build


def test_strip_comments_keeps_literals():
    src = ('int a; // line\n/* block\n over lines */ int b = 1;\n\n'
           'asm volatile("s_mov_b32 m0, %0\\n\\tbuffer_load // inside a string");\n'
           "char q = '/'; char r = '\\''; const char* s = \"/* not a comment */\";\n")
    out = build.strip_comments(src)
    assert "line" not in out and "block" not in out and "over lines" not in out
    assert '"s_mov_b32 m0, %0\\n\\tbuffer_load // inside a string"' in out
    assert "'/'" in out and "'\\''" in out and '"/* not a comment */"' in out
    assert "\n\n" not in out and out.startswith("int a;")


def test_digest_ignores_comments_but_not_code(tmp_path, monkeypatch):
    csrc = tmp_path / "csrc"
    shutil.copytree(build.CSRC, csrc)
    monkeypatch.setattr(build, "CSRC", str(csrc))
    base = build.kernel_source_digest()
    kernels = csrc / "gemm_relu_kernels.hpp"
    text = kernels.read_text()
    kernels.write_text("// a new comment\n" + text.replace("#pragma once", "#pragma once  /* note */", 1) + "\n\n")
    assert build.kernel_source_digest() == base
    kernels.write_text(text.replace("constexpr int kBufferFlags = 0x00020000;", "constexpr int kBufferFlags = 0x00020001;"))
    assert build.kernel_source_digest() != base
