// Instances of the gfx950 GEMM + ReLU kernels for the f16 dtype.
#include "kernel_instances.hpp"

namespace gemm_relu_hip {

const DtypeKernels& kernels_f16()
{
    static const DtypeKernels table = instances::make_table<kF16>();
    return table;
}

const void* zero_fill_kernel() { return (const void*)&gemm_relu_zero_fill<uint16_t>; }

}  // namespace gemm_relu_hip
