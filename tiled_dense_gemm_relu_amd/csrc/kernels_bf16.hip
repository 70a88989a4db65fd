// Instances of the gfx950 GEMM + ReLU kernels for the bf16 dtype.
#include "kernel_instances.hpp"

namespace gemm_relu_hip {

const DtypeKernels& kernels_bf16()
{
    static const DtypeKernels table = instances::make_table<kBF16>();
    return table;
}

}  // namespace gemm_relu_hip
