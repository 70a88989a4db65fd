"""Seeded synthetic inputs for ReLU(A @ B) workloads.

This module only draws random matrices; it holds none of the GEMM's
arithmetic.  It is the one module the HIP path's tests and the CPU oracle both
use, so that both see the same input bytes.

The pages benchmark on plain normally distributed fp16 matrices (the GEMM +
ReLU example of "Writing High-Performance Kernels in TileLang", section
"Let's write a GEMM", and the benchmark script of "TileLang Guide: Composable
Tiled AI Kernel Programming", Step 2).  The workloads below keep that recipe,
with a per-workload scale so that outputs stay well inside the fp16 range, plus
an integer-valued variant (entries uniform in {-2, ..., 2}) whose every partial
sum is exact in fp32.

All draws happen on the CPU with ``torch.Generator().manual_seed(seed)``; A is
drawn first, then B, from the same generator, so the bytes are identical on
every machine.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

_DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dtype: str          # "fp16" or "bf16"; inputs and output share it
    scale: float        # A, B ~ N(0, 1) * scale before rounding to dtype
    seed: int           # seed of the real-valued variant
    int_seed: int       # seed of the integer-valued variant

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.dtype]

    @property
    def flop(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def bytes_once(self) -> int:
        """A, B read once and C written once, 2 bytes per element."""
        return 2 * (self.M * self.K + self.K * self.N + self.M * self.N)


# The workload shapes: a small correctness case, the 1024^3 example shape with
# 128x128x64 tiles, the 8192^3 compute-bound headline, a shape with ragged M, N
# and K tails, a skinny decode-like bf16 shape that is HBM-bound, a deep-K
# shape with few output tiles, the headline shape in bf16, a mid-size square
# and a decode-like shape with many columns.
WORKLOADS = {
    "small_256": Workload("small_256", 256, 256, 256, "fp16", 1.0, 1001, 1011),
    "square_1024": Workload("square_1024", 1024, 1024, 1024, "fp16", 1.0, 1002, 1012),
    "square_8192": Workload("square_8192", 8192, 8192, 8192, "fp16", 0.1, 1003, 1013),
    "ragged_4000x11000x4100": Workload("ragged_4000x11000x4100", 4000, 11000, 4100, "fp16", 0.05,
                                       1004, 1014),
    "skinny_64x16384x8192": Workload("skinny_64x16384x8192", 64, 16384, 8192, "bf16", 0.05,
                                     1005, 1015),
    # few output tiles over a long K: the case split-K is for
    "deep_512x512x16384": Workload("deep_512x512x16384", 512, 512, 16384, "fp16", 0.05, 1006, 1016),
    # the headline shape in bf16
    "square_8192_bf16": Workload("square_8192_bf16", 8192, 8192, 8192, "bf16", 0.1, 1007, 1017),
    # a mid-size square: 128x128 tiles fill the CUs, 256x256 ones do not
    "square_2048": Workload("square_2048", 2048, 2048, 2048, "fp16", 0.1, 1008, 1018),
    # decode-like with many columns (256 tiles of 64x256): HBM-bound on B, like the skinny shape
    "wide_decode_64x65536x2048": Workload("wide_decode_64x65536x2048", 64, 65536, 2048, "bf16", 0.05,
                                          1009, 1019),
}


def normal_pair(M: int, N: int, K: int, dtype: torch.dtype, scale: float, seed: int):
    """A (M, K) and B (K, N) with entries N(0, 1) * scale rounded to ``dtype`` (CPU tensors)."""
    g = torch.Generator().manual_seed(seed)
    a = (torch.randn((M, K), generator=g, dtype=torch.float32) * scale).to(dtype)
    b = (torch.randn((K, N), generator=g, dtype=torch.float32) * scale).to(dtype)
    return a, b


def integer_pair(M: int, N: int, K: int, dtype: torch.dtype, seed: int, lo: int = -2, hi: int = 2):
    """A (M, K) and B (K, N) with integer entries uniform in [lo, hi] (CPU tensors)."""
    g = torch.Generator().manual_seed(seed)
    a = torch.randint(lo, hi + 1, (M, K), generator=g, dtype=torch.int32).to(dtype)
    b = torch.randint(lo, hi + 1, (K, N), generator=g, dtype=torch.int32).to(dtype)
    return a, b


def workload_inputs(w: Workload, integer: bool = False):
    """The seeded (A, B) CPU pair of a workload, real-valued or integer-valued."""
    if integer:
        return integer_pair(w.M, w.N, w.K, w.torch_dtype, w.int_seed)
    return normal_pair(w.M, w.N, w.K, w.torch_dtype, w.scale, w.seed)
