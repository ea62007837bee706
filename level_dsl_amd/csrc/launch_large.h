// launch_large.h -- launch templates of the 256 x 256-tile kernel, shared by
// its translation units (k_large_*.hip).
#pragma once

#include "mxgemm_large.h"

namespace mxg {
namespace {

template <int FA, int FB, bool NATIVE, bool SPLIT>
hipError_t launch_large_s(const mxg::GemmArgs &a, hipStream_t s)
{
    const int blocks = a.tiles_m * a.tiles_n * a.splits;
    // 16-byte scale windows (in registers for the exact mode, through LDS for
    // the scaled-MFMA modes) need K % 512 == 0 and 16-byte aligned row-major
    // scale rows; preshuffled scales take one coalesced dword per stage
    if (a.scale_dword == 2 && !a.scale_ps) {
        hipLaunchKernelGGL((mxg::large::kernel<FA, FB, NATIVE, true, SPLIT>), dim3(blocks),
                           dim3(mxg::large::THREADS), 0, s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((mxg::large::kernel<FA, FB, NATIVE, false, SPLIT>), dim3(blocks),
                       dim3(mxg::large::THREADS), 0, s, a);
    return hipGetLastError();
}

// Split launches use their own instantiation, so that the split epilogue
// adds nothing to the register budget of the unsplit kernel.
template <int FA, int FB, bool NATIVE>
hipError_t launch_large(const mxg::GemmArgs &a, hipStream_t s)
{
    return a.splits > 1 ? launch_large_s<FA, FB, NATIVE, true>(a, s)
                        : launch_large_s<FA, FB, NATIVE, false>(a, s);
}

} // namespace
} // namespace mxg
