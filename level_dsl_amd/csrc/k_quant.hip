// k_quant.hip -- the MX block quantization kernel and the streaming copy.
#include <algorithm>

#include "mxcopy.h"
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

hipError_t launch_copy(const uint8_t *src, uint8_t *dst, uint64_t bytes, hipStream_t stream)
{
    // two workgroups per CU (measured best on 1 GiB), but no more than there
    // are pieces
    const uint64_t pieces = (bytes + copy::PIECE - 1) / copy::PIECE;
    const uint64_t per_block = copy::THREADS / 64;
    const uint64_t blocks = std::min<uint64_t>((pieces + per_block - 1) / per_block, 256 * 2);
    hipLaunchKernelGGL(copy::kernel, dim3((unsigned)blocks), dim3(copy::THREADS), 0, stream, src, dst,
                       bytes);
    return hipGetLastError();
}

} // namespace mxg
