"""CPU oracle for C = ReLU(A @ B) -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP product path
(``tiled_dense_gemm_relu_amd``) never imports it, and the two share no code.

The arithmetic lives in ``gemm_relu_oracle.c`` (plain C, OpenMP over rows,
fp64 sums in ascending k); this module builds it with gcc and wraps it with
ctypes.  What it computes follows the GEMM + ReLU example of "Writing
High-Performance Kernels in TileLang" (atlascloud.ai, section "Let's write a
GEMM"): C[i, j] = cast(max(sum_k A[i, k] * B[k, j], 0)), cast = round to
nearest even into the input dtype, max(s, 0) = +0.0 for s <= 0.

Every function here is pinned by ``tests/test_oracle.py`` against library
conversions, exact integer and rational arithmetic and hand-worked examples.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_relu_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

F16 = 0
BF16 = 1
_DTYPES = {"float16": F16, "fp16": F16, "f16": F16, "bfloat16": BF16, "bf16": BF16}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2 -fopenmp).  Returns the .so path."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            u16p = ctypes.POINTER(ctypes.c_uint16)
            f64p = ctypes.POINTER(ctypes.c_double)
            i64p = ctypes.POINTER(ctypes.c_int64)
            i64 = ctypes.c_int64
            lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
            lib.oracle_f16_to_f64.restype = ctypes.c_double
            lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
            lib.oracle_bf16_to_f64.restype = ctypes.c_double
            lib.oracle_f64_to_f16.argtypes = [ctypes.c_double]
            lib.oracle_f64_to_f16.restype = ctypes.c_uint16
            lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
            lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
            lib.oracle_decode.argtypes = [u16p, f64p, i64, ctypes.c_int]
            lib.oracle_decode.restype = None
            lib.oracle_encode.argtypes = [f64p, u16p, i64, ctypes.c_int]
            lib.oracle_encode.restype = None
            lib.oracle_gemm_relu.argtypes = [u16p, u16p, u16p, i64, i64, i64, ctypes.c_int, ctypes.c_int]
            lib.oracle_gemm_relu.restype = ctypes.c_int
            lib.oracle_gemm_relu_rows.argtypes = [u16p, u16p, u16p, i64, i64, i64, i64, i64,
                                                  ctypes.c_int, ctypes.c_int]
            lib.oracle_gemm_relu_rows.restype = ctypes.c_int
            lib.oracle_gemm_relu_entries.argtypes = [u16p, u16p, i64, i64, i64, i64p, i64p, i64,
                                                     u16p, ctypes.c_int]
            lib.oracle_gemm_relu_entries.restype = ctypes.c_int
            lib.oracle_max_threads.argtypes = []
            lib.oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def _dtype_code(dtype) -> int:
    name = str(dtype).replace("torch.", "")
    if name not in _DTYPES:
        raise ValueError(f"oracle: unsupported dtype {dtype!r}")
    return _DTYPES[name]


def _bits(x) -> np.ndarray:
    """16-bit patterns of a torch tensor or numpy array, as a C-contiguous uint16 array."""
    if hasattr(x, "view") and hasattr(x, "numpy") and hasattr(x, "dtype") and "torch" in type(x).__module__:
        import torch
        x = x.detach().cpu().contiguous().view(torch.int16).numpy()
    arr = np.ascontiguousarray(x)
    if arr.dtype.itemsize != 2:
        raise TypeError("oracle: expected 16-bit elements")
    return arr.view(np.uint16)


def _u16p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def decode(bits, dtype) -> np.ndarray:
    """Exact fp64 values of 16-bit patterns of ``dtype``."""
    b = _bits(bits)
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_decode(_u16p(b), out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), b.size,
                          _dtype_code(dtype))
    return out


def encode(values, dtype) -> np.ndarray:
    """Round fp64 values to ``dtype`` bit patterns (nearest, ties to even)."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().oracle_encode(v.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), _u16p(out), v.size,
                          _dtype_code(dtype))
    return out


def _shapes(a, b):
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"oracle: bad shapes {a.shape} @ {b.shape}")
    return a.shape[0], b.shape[1], a.shape[1]


def gemm_relu(a, b, dtype, threads: int = 0) -> np.ndarray:
    """C = ReLU(A @ B) as ``dtype`` bit patterns (uint16 array of shape (M, N))."""
    ab, bb = _bits(a), _bits(b)
    M, N, K = _shapes(ab, bb)
    c = np.zeros((M, N), dtype=np.uint16)
    rc = _load().oracle_gemm_relu(_u16p(ab), _u16p(bb), _u16p(c), M, N, K, _dtype_code(dtype), threads)
    if rc != 0:
        raise RuntimeError("oracle_gemm_relu failed")
    return c


def gemm_relu_rows(a, b, dtype, row0: int, row1: int, threads: int = 0) -> np.ndarray:
    """Rows [row0, row1) of ReLU(A @ B) as bit patterns, shape (row1 - row0, N)."""
    ab, bb = _bits(a), _bits(b)
    M, N, K = _shapes(ab, bb)
    if not (0 <= row0 <= row1 <= M):
        raise ValueError("oracle: bad row range")
    # Only the selected rows of A are passed, as a (row1-row0, K) matrix.
    sub = np.ascontiguousarray(ab[row0:row1])
    c = np.zeros((row1 - row0, N), dtype=np.uint16)
    rc = _load().oracle_gemm_relu_rows(_u16p(sub), _u16p(bb), _u16p(c), row1 - row0, N, K,
                                       0, row1 - row0, _dtype_code(dtype), threads)
    if rc != 0:
        raise RuntimeError("oracle_gemm_relu_rows failed")
    return c


def gemm_relu_entries(a, b, dtype, ii, jj) -> np.ndarray:
    """C[ii[t], jj[t]] of ReLU(A @ B) for every t, as bit patterns."""
    ab, bb = _bits(a), _bits(b)
    M, N, K = _shapes(ab, bb)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    if ii.shape != jj.shape:
        raise ValueError("oracle: index arrays differ in shape")
    out = np.zeros(ii.shape, dtype=np.uint16)
    i64p = ctypes.POINTER(ctypes.c_int64)
    rc = _load().oracle_gemm_relu_entries(_u16p(ab), _u16p(bb), M, N, K, ii.ctypes.data_as(i64p),
                                          jj.ctypes.data_as(i64p), ii.size, _u16p(out),
                                          _dtype_code(dtype))
    if rc != 0:
        raise RuntimeError("oracle_gemm_relu_entries failed (index out of range?)")
    return out


def max_threads() -> int:
    return int(_load().oracle_max_threads())
