// k_quant.hip -- the MX block quantization kernel, the streaming copy, the
// conversion of scale bytes to the preshuffled layout and the rewrite of
// sub-byte operand codes as e4m3 bytes.
#include <algorithm>

#include "mxcopy.h"
#include "mxgemm_launch.h"
#include "mxwiden.h"

namespace mxg {

hipError_t launch_quant(int sel, const quant::QuantArgs &a, dim3 grid, dim3 block, hipStream_t stream)
{
    switch (sel) {
    case 0: hipLaunchKernelGGL((quant::kernel<0, 0>), grid, block, 0, stream, a); break;
    case 1: hipLaunchKernelGGL((quant::kernel<0, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((quant::kernel<1, 0>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((quant::kernel<1, 1>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((quant::kernel<2, 0>), grid, block, 0, stream, a); break;
    case 5: hipLaunchKernelGGL((quant::kernel<2, 1>), grid, block, 0, stream, a); break;
    case 6: hipLaunchKernelGGL((quant::kernel<3, 0>), grid, block, 0, stream, a); break;
    case 7: hipLaunchKernelGGL((quant::kernel<3, 1>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((quant::kernel<4, 0>), grid, block, 0, stream, a); break;
    case 9: hipLaunchKernelGGL((quant::kernel<4, 1>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_widen(int fmt, const uint8_t *src, uint8_t *dst, uint64_t n, hipStream_t stream)
{
    // one thread per 16 codes; at most 8 workgroups per CU, each thread then
    // loops over its share
    const uint64_t groups = n / widen::CODES;
    const uint64_t blocks = std::min<uint64_t>((groups + widen::THREADS - 1) / widen::THREADS, 256 * 8);
    const dim3 grid((unsigned)std::max<uint64_t>(blocks, 1)), block(widen::THREADS);
    switch (fmt) {
    case 4: hipLaunchKernelGGL((widen::kernel<4>), grid, block, 0, stream, src, dst, n); break;
    case 2: hipLaunchKernelGGL((widen::kernel<2>), grid, block, 0, stream, src, dst, n); break;
    case 3: hipLaunchKernelGGL((widen::kernel<3>), grid, block, 0, stream, src, dst, n); break;
    default: return hipErrorInvalidValue;
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

namespace {

// Row-major scale bytes (rows x KB) to the preshuffled layout: thread t
// writes word t of dst, which is word w = u % (KB / 4) of row 32 g + t % 32
// for unit u = t / 32 of group g = u / (KB / 4) (mxgemm_common.h, scale_at);
// rows past `rows` (the last group's padding) are written as zeros.
__global__ __launch_bounds__(256) void preshuffle_kernel(const uint8_t *src, uint32_t *dst,
                                                         uint64_t rows, uint32_t KB, uint64_t words)
{
    const uint64_t t = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    if (t >= words) return;
    const uint32_t W = KB / 4;
    const uint64_t u = t >> 5;
    const uint64_t g = u / W;
    const uint32_t w = (uint32_t)(u - g * W);
    const uint64_t r = 32 * g + (t & 31u);
    uint32_t v = 0;
    if (r < rows) {
        const uint8_t *s = src + r * KB + 4 * w;
        v = (uint32_t)s[0] | ((uint32_t)s[1] << 8) | ((uint32_t)s[2] << 16) | ((uint32_t)s[3] << 24);
    }
    dst[t] = v;
}

} // namespace

hipError_t launch_preshuffle(const uint8_t *src, uint8_t *dst, uint64_t rows, int KB, hipStream_t stream)
{
    const uint64_t words = (rows + 31) / 32 * 32 * (uint64_t)KB / 4;
    hipLaunchKernelGGL(preshuffle_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                       src, (uint32_t *)dst, rows, (uint32_t)KB, words);
    return hipGetLastError();
}

} // namespace mxg
