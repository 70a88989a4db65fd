"""Thin ctypes binding over libgemm_relu.so (the C ABI in include/gemm_relu.h).

Argument marshalling only: every step of ReLU(A @ B) runs in the library's
HIP kernels.  torch supplies device memory and the current stream.  There is
no fallback: if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

F16 = 0
BF16 = 1

# How B is stored: (K, N) row-major, or B^T as an (N, K) row-major array.
B_KN = 0
B_NK = 1

CONFIG_AUTO = -1
CONFIG_DIRECT = 0
CONFIG_TILE_256 = 1
CONFIG_TILE_128 = 2
CONFIG_DMA_256 = 3
CONFIG_DMA_128 = 4
CONFIG_DMA_64 = 5
CONFIG_DMA_64x256 = 6
CONFIG_DMA_256x128_WS = 7
CONFIG_DMA_32x32_WS = 8
CONFIG_DMA_64x64_WS = 9
CONFIG_DMA_128x128_WS = 10
CONFIG_NAMES = {CONFIG_DIRECT: "direct_32x32", CONFIG_TILE_256: "tile_256x256x64",
                CONFIG_TILE_128: "tile_128x128x64", CONFIG_DMA_256: "dma_256x256x64_2stage",
                CONFIG_DMA_128: "dma_128x128x64_4stage", CONFIG_DMA_64: "dma_64x64x64_8stage",
                CONFIG_DMA_64x256: "dma_64x256x32_4stage", CONFIG_DMA_256x128_WS: "dma_256x128x32_4stage_ws",
                CONFIG_DMA_32x32_WS: "dma_32x32x64_4stage_ws", CONFIG_DMA_64x64_WS: "dma_64x64x64_4stage_ws",
                CONFIG_DMA_128x128_WS: "dma_128x128x64_4stage_ws"}

ERRORS = {
    0: "OK", -1: "INVALID_ARG", -2: "BAD_DTYPE", -3: "ALIAS", -4: "MISALIGNED", -5: "NO_DEVICE",
    -6: "LAUNCH", -7: "TOO_LARGE", -8: "BAD_CONFIG", -9: "BAD_LAYOUT", -10: "WORKSPACE", -11: "SCRATCH",
}

# GEMM_RELU_NOALLOC_SCRATCH_BYTES: the static device array gemm_relu_splitk_noalloc works in.
NOALLOC_SCRATCH_BYTES = 65536 + (32 << 20)

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libgemm_relu.so")
_lock = threading.Lock()
_lib = None


class GemmReluError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"gemm_relu failed: {ERRORS.get(code, code)} ({code}): {msg}")
        self.code = code


class _Config(ctypes.Structure):
    _fields_ = [("config_id", ctypes.c_int), ("block_m", ctypes.c_int), ("block_n", ctypes.c_int),
                ("block_k", ctypes.c_int), ("stages", ctypes.c_int), ("threads", ctypes.c_int),
                ("vec_a", ctypes.c_int), ("vec_b", ctypes.c_int), ("grid", ctypes.c_int64),
                ("lds_bytes", ctypes.c_int), ("b_layout", ctypes.c_int), ("splits", ctypes.c_int),
                ("workspace_bytes", ctypes.c_int64)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libgemm_relu.so (built in-tree by tiled_dense_gemm_relu_amd.build); raise if absent."""
    global _lib
    if _lib is not None:          # loaded (the reference is only ever set once, under the lock)
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                                   "`python -m tiled_dense_gemm_relu_amd.build` (needs hipcc)")
            lib = ctypes.CDLL(_LIB_PATH)
            vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
            lib.gemm_relu.argtypes = [vp, vp, vp, i64, i64, i64, ci, vp]
            lib.gemm_relu.restype = ci
            lib.gemm_relu_with_config.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, vp]
            lib.gemm_relu_with_config.restype = ci
            lib.gemm_relu_query_config.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, ctypes.POINTER(_Config)]
            lib.gemm_relu_query_config.restype = ci
            lib.gemm_relu_ex.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, ci, vp]
            lib.gemm_relu_ex.restype = ci
            lib.gemm_relu_query_config_ex.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, ci,
                                                      ctypes.POINTER(_Config)]
            lib.gemm_relu_query_config_ex.restype = ci
            lib.gemm_relu_splitk.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, ci, ci, vp, i64, vp]
            lib.gemm_relu_splitk.restype = ci
            lib.gemm_relu_query_splitk.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, ci, ci,
                                                   ctypes.POINTER(_Config)]
            lib.gemm_relu_query_splitk.restype = ci
            lib.gemm_relu_splitk_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, ci, ci, vp]
            lib.gemm_relu_splitk_noalloc.restype = ci
            ip = ctypes.POINTER(ci)
            lib.gemm_relu_selected_config.argtypes = [i64, i64, i64, ci, ip, ip, ip, ip]
            lib.gemm_relu_selected_config.restype = ci
            lib.gemm_relu_strerror.argtypes = [ci]
            lib.gemm_relu_strerror.restype = ctypes.c_char_p
            lib.gemm_relu_version.argtypes = []
            lib.gemm_relu_version.restype = ci
            _lib = lib
    return _lib


def strerror(code: int) -> str:
    return load_library().gemm_relu_strerror(code).decode()


def _check(code: int):
    if code != 0:
        raise GemmReluError(code, strerror(code))


def gemm_relu_raw(a_ptr: int, b_ptr: int, c_ptr: int, M: int, N: int, K: int, dtype: int,
                  stream: int = 0, config: int = CONFIG_AUTO, b_layout: int = B_KN) -> int:
    """Call the C ABI with raw device pointers; returns the library's status code."""
    lib = load_library()
    if b_layout != B_KN:
        return lib.gemm_relu_ex(a_ptr, b_ptr, c_ptr, M, N, K, dtype, b_layout, config, stream or None)
    if config == CONFIG_AUTO:
        return lib.gemm_relu(a_ptr, b_ptr, c_ptr, M, N, K, dtype, stream or None)
    return lib.gemm_relu_with_config(a_ptr, b_ptr, c_ptr, M, N, K, dtype, config, stream or None)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"gemm_relu: dtype must be float16 or bfloat16, got {t.dtype}")


def _check_tensors(a, b, out, b_layout=B_KN) -> int:
    """Argument checks of the tensor entry points; returns the device index."""
    import torch
    for name, t in (("a", a), ("b", b)) + ((("out", out),) if out is not None else ()):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"gemm_relu: {name} must be a torch.Tensor")
        if not t.is_cuda:
            raise ValueError(f"gemm_relu: {name} must be a GPU tensor, got {t.device}")
        if t.dim() != 2:
            raise ValueError(f"gemm_relu: {name} must be 2-D, got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"gemm_relu: {name} must be contiguous (row-major)")
    if a.dtype != b.dtype or (out is not None and out.dtype != a.dtype):
        raise TypeError("gemm_relu: a, b and out must share one dtype")
    k_b, n = (b.shape[1], b.shape[0]) if b_layout == B_NK else (b.shape[0], b.shape[1])
    if a.shape[1] != k_b:
        raise ValueError(f"gemm_relu: inner dimensions differ: a {tuple(a.shape)}, b {tuple(b.shape)}"
                         f" stored {'(N, K)' if b_layout == B_NK else '(K, N)'}")
    dev = a.get_device()
    if b.get_device() != dev or (out is not None and out.get_device() != dev):
        raise ValueError("gemm_relu: a, b and out must be on one device")
    if out is not None and (out.shape[0] != a.shape[0] or out.shape[1] != n):
        raise ValueError(f"gemm_relu: out must have shape {(a.shape[0], n)}, got {tuple(out.shape)}")
    return dev


def _stream_handle(stream, dev: int) -> int:
    """The HIP stream handle to enqueue on: ``stream``'s, else the device's current one."""
    import torch
    if stream is not None:
        return stream.cuda_stream
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(dev)
    return torch.cuda.current_stream(dev).cuda_stream


def gemm_relu(a, b, out=None, config: int = CONFIG_AUTO, stream=None):
    """C = ReLU(a @ b) for row-major fp16/bf16 GPU tensors a (M, K) and b (K, N).

    ``out`` (M, N) is written if given, else allocated.  The kernel is enqueued
    on ``stream`` (a torch.cuda.Stream), by default torch's current stream.
    """
    return gemm_relu_ex(a, b, out=out, b_layout=B_KN, config=config, stream=stream)


def gemm_relu_ex(a, b, out=None, b_layout: int = B_KN, config: int = CONFIG_AUTO, stream=None):
    """C = ReLU(a @ B) with B stored as ``b_layout`` says.

    B_KN: ``b`` is B, (K, N) row-major.  B_NK: ``b`` is B^T, an (N, K)
    row-major tensor (e.g. a weight stored output-major), so C = ReLU(a @ b.T).
    """
    import torch
    if b_layout not in (B_KN, B_NK):
        raise ValueError(f"gemm_relu: b_layout must be B_KN or B_NK, got {b_layout}")
    dev = _check_tensors(a, b, out, b_layout)
    dtype = _dtype_code(a)
    M, K = a.shape
    N = b.shape[0] if b_layout == B_NK else b.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    handle = _stream_handle(stream, dev)
    args = (a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, dtype, handle, config, b_layout)
    # The library launches on the current device: make it the tensors' one.
    if torch.cuda.current_device() == dev:
        rc = gemm_relu_raw(*args)
    else:
        with torch.cuda.device(dev):
            rc = gemm_relu_raw(*args)
    _check(rc)
    return out


_workspaces = {}
_workspaces_lock = threading.Lock()


def splitk_workspace(device, stream, nbytes: int):
    """A zero-filled workspace of at least ``nbytes`` for split-K calls on ``stream``.

    One buffer per (device, stream), grown when needed and kept for later calls
    until the process ends: the library leaves its counters at zero after every
    completed call.  Calls on one stream are ordered, so they may share it;
    other streams get their own.  A buffer that is replaced by a larger one is
    released through torch's stream-ordered allocator, after the work already
    queued on that stream.
    """
    import torch
    key = (device, stream.cuda_stream)
    with _workspaces_lock:
        ws = _workspaces.get(key)
        if ws is None or ws.numel() < nbytes:
            with torch.cuda.stream(stream):
                ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
            _workspaces[key] = ws
    return ws


def gemm_relu_splitk(a, b, out=None, b_layout: int = B_KN, config: int = CONFIG_AUTO, splits: int = 0,
                     workspace=None, stream=None):
    """C = ReLU(a @ B) with each output tile's K range split into ``splits`` parts (0: the library
    chooses).  ``workspace``: a zero-filled uint8 GPU tensor of at least the queried size, or None
    for a cached one per stream.  B as for gemm_relu_ex."""
    import torch
    if b_layout not in (B_KN, B_NK):
        raise ValueError(f"gemm_relu: b_layout must be B_KN or B_NK, got {b_layout}")
    _check_tensors(a, b, out, b_layout)
    dtype = _dtype_code(a)
    M, K = a.shape
    N = b.shape[0] if b_layout == B_NK else b.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    s = stream if stream is not None else torch.cuda.current_stream(a.device)
    lib = load_library()
    cfg = _Config()
    _check(lib.gemm_relu_query_splitk(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, dtype, b_layout,
                                      config, splits, ctypes.byref(cfg)))
    ws_ptr, ws_bytes = None, 0
    if cfg.workspace_bytes > 0:
        if workspace is None:
            workspace = splitk_workspace(a.device, s, cfg.workspace_bytes)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(a.device):
        rc = lib.gemm_relu_splitk(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, dtype, b_layout, config,
                                  splits, ws_ptr, ws_bytes, s.cuda_stream or None)
    _check(rc)
    return out


def gemm_relu_splitk_noalloc(a, b, out=None, b_layout: int = B_KN, config: int = CONFIG_AUTO, splits: int = 0,
                             stream=None):
    """gemm_relu_splitk with the library's static device scratch instead of a workspace (the C
    entry point allocates nothing; here ``out`` is allocated if not given).  Calls that may overlap
    in time on one device share that scratch and race: keep them on one stream."""
    import torch
    if b_layout not in (B_KN, B_NK):
        raise ValueError(f"gemm_relu: b_layout must be B_KN or B_NK, got {b_layout}")
    dev = _check_tensors(a, b, out, b_layout)
    dtype = _dtype_code(a)
    M, K = a.shape
    N = b.shape[0] if b_layout == B_NK else b.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    handle = _stream_handle(stream, dev)
    with torch.cuda.device(a.device):
        rc = load_library().gemm_relu_splitk_noalloc(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, dtype,
                                                     b_layout, config, splits, handle or None)
    _check(rc)
    return out


def selected_splitk_config(M: int, N: int, K: int, dtype: int = F16, config: int = CONFIG_AUTO, splits: int = 0,
                           a_ptr: int = 256, b_ptr: int = 256, c_ptr: int = 1 << 40, b_layout: int = B_KN) -> dict:
    """The configuration gemm_relu_splitk would use, with ``splits`` and ``workspace_bytes`` (host only)."""
    cfg = _Config()
    _check(load_library().gemm_relu_query_splitk(a_ptr, b_ptr, c_ptr, M, N, K, dtype, b_layout, config, splits,
                                                 ctypes.byref(cfg)))
    return {f: getattr(cfg, f) for f, _ in _Config._fields_}


def selected_config(M: int, N: int, K: int, dtype: int = F16, config: int = CONFIG_AUTO,
                    a_ptr: int = 256, b_ptr: int = 256, c_ptr: int = 1 << 40, b_layout: int = B_KN) -> dict:
    """The kernel configuration the library would pick (host logic only, no device needed)."""
    cfg = _Config()
    lib = load_library()
    if b_layout == B_KN:
        rc = lib.gemm_relu_query_config(a_ptr, b_ptr, c_ptr, M, N, K, dtype, config, ctypes.byref(cfg))
    else:
        rc = lib.gemm_relu_query_config_ex(a_ptr, b_ptr, c_ptr, M, N, K, dtype, b_layout, config,
                                           ctypes.byref(cfg))
    _check(rc)
    return {f: getattr(cfg, f) for f, _ in _Config._fields_}


def selected_block_config(M: int, N: int, K: int, dtype: int = F16) -> tuple:
    """(block_m, block_n, block_k, stages) that gemm_relu picks for dense, 256-byte aligned buffers
    (gemm_relu_selected_config; host logic only)."""
    out = [ctypes.c_int(-1) for _ in range(4)]
    _check(load_library().gemm_relu_selected_config(M, N, K, dtype, *(ctypes.byref(v) for v in out)))
    return tuple(v.value for v in out)
