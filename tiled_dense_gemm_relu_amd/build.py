"""Ahead-of-time build of libgemm_relu.so for gfx950 with hipcc.

Each .hip translation unit is compiled to an object in parallel, then linked
into ``tiled_dense_gemm_relu_amd/libgemm_relu.so`` (in-tree, so it travels with
the source tree).  Run ``python -m tiled_dense_gemm_relu_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libgemm_relu.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ABLATION_PATH = os.path.join(PKG, "layout_ablation")
MFMA_FORM_PATH = os.path.join(PKG, "mfma_form")
STREAM_CEILING_PATH = os.path.join(PKG, "stream_ceiling")
KERNEL_TIMELINE_PATH = os.path.join(PKG, "kernel_timeline")
ARCH = "gfx950"

SOURCES = ["gemm_relu_api.hip", "kernels_f16.hip", "kernels_bf16.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # No packed fp32 arithmetic (v_pk_*_f32) in generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


KERNEL_SOURCES = ["gemm_relu_kernels.hpp", "kernel_instances.hpp", "kernels_f16.hip", "kernels_bf16.hip"]


def strip_comments(src: str) -> str:
    """C/C++ source without its comments and blank lines; string and character literals are kept
    as they are (inline assembly strings hold sequences such as "\\n\\t")."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":                               # literal: copy through its closing quote
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):                 # line comment: drop to the end of the line
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):                 # block comment
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (line.rstrip() for line in "".join(out).split("\n"))
    return "\n".join(line for line in lines if line)


def kernel_source_digest() -> str:
    """SHA-256 over the kernel sources with comments and blank lines removed: identifies the kernels
    a profile was taken on, and stays the same when only comments change."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + strip_comments(f.read()).encode())
    return h.hexdigest()


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libgemm_relu.so")
    return path


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every HIP source and link the shared library.  Returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra or [])
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    # The measurement programs: layout ablations (XOR swizzle, XCD remap on / off),
    # the power and clock of the two MFMA forms, the skinny shape's streaming ceiling
    # and the per-workgroup phase timeline of a launch.
    programs = (("layout_ablation.hip", ABLATION_PATH), ("mfma_form.hip", MFMA_FORM_PATH),
                ("stream_ceiling.hip", STREAM_CEILING_PATH), ("kernel_timeline.hip", KERNEL_TIMELINE_PATH))
    for src, path in programs:
        tmp = path + f".tmp{os.getpid()}"
        cmd = [hipcc(), *HIPCC_FLAGS, *extra, os.path.join(CSRC, src), "-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
        os.replace(tmp, path)
    if verbose:
        print(f"built {LIB_PATH} and " + ", ".join(path for _, path in programs))
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
