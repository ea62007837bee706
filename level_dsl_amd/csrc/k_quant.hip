// k_quant.hip -- the MX block quantization kernel.
#include "mxgemm_launch.h"

namespace mxg {

hipError_t launch_quant(int sel, const quant::QuantArgs &a, dim3 grid, dim3 block, hipStream_t stream)
{
    switch (sel) {
    case 0: hipLaunchKernelGGL((quant::kernel<0, 0>), grid, block, 0, stream, a); break;
    case 1: hipLaunchKernelGGL((quant::kernel<0, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((quant::kernel<1, 0>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((quant::kernel<1, 1>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((quant::kernel<4, 0>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((quant::kernel<4, 1>), grid, block, 0, stream, a); break;
    }
    return hipGetLastError();
}

} // namespace mxg
