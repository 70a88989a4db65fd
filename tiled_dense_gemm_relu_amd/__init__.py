"""MI355X-native fused GEMM + ReLU: C = ReLU(A @ B) on gfx950 MFMA."""
from .binding import (  # noqa: F401
    gemm_relu,
    gemm_relu_ex,
    gemm_relu_splitk,
    gemm_relu_splitk_noalloc,
    selected_splitk_config,
    gemm_relu_raw,
    selected_config,
    selected_block_config,
    strerror,
    library_path,
    load_library,
    GemmReluError,
    F16,
    BF16,
    B_KN,
    B_NK,
)
