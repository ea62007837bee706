// launch_skinny.h -- launch templates of the small-M scaled-MFMA kernel,
// shared by its translation units (k_skinny_*.hip).
#pragma once

#include "mxgemm_skinny.h"

namespace mxg {
namespace {

template <int FA, int FB, int MT, bool SPLIT>
hipError_t launch_skinny_s(const mxg::GemmArgs &a, hipStream_t s)
{
    namespace sk = mxg::skinny;
    const int blocks = a.tiles_m * a.tiles_n * a.splits;
    // scale table in LDS when the scale rows are 16-byte multiples, aligned,
    // and all of K fits; else (e2m1, row-major scales) 8-byte loads per
    // stage, or byte loads
    if (a.scale_dword == 2 && sk::table_fits(a.KB)) {
        hipLaunchKernelGGL((sk::kernel<FA, FB, sk::SCALES_TABLE, MT, SPLIT>), dim3(blocks),
                           dim3(sk::THREADS), 0, s, a);
        return hipGetLastError();
    }
    if constexpr (FA == 4) {
        if (a.scale_dword == 2 && !a.scale_ps) {
            hipLaunchKernelGGL((sk::kernel<FA, FB, sk::SCALES_VEC, MT, SPLIT>), dim3(blocks),
                               dim3(sk::THREADS), 0, s, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((sk::kernel<FA, FB, sk::SCALES_BYTES, MT, SPLIT>), dim3(blocks),
                       dim3(sk::THREADS), 0, s, a);
    return hipGetLastError();
}

// split launches use their own instantiation, as for the 256 x 256 kernel
template <int FA, int FB, int MT>
hipError_t launch_skinny_mt(const mxg::GemmArgs &a, hipStream_t s)
{
    return a.splits > 1 ? launch_skinny_s<FA, FB, MT, true>(a, s)
                        : launch_skinny_s<FA, FB, MT, false>(a, s);
}

// e2m1 and e2m3 run only ceil(M/16) tiles of A; the fp8 native variant (an opt-in)
// keeps all four, which holds down the number of kernels built
template <int FA, int FB>
hipError_t launch_skinny(const mxg::GemmArgs &a, hipStream_t s)
{
    if constexpr (FA == 4 || FA == 2) {
        switch ((a.M + 15) / 16) {
        case 1: return launch_skinny_mt<FA, FB, 1>(a, s);
        case 2: return launch_skinny_mt<FA, FB, 2>(a, s);
        case 3: return launch_skinny_mt<FA, FB, 3>(a, s);
        default: break;
        }
    }
    return launch_skinny_mt<FA, FB, 4>(a, s);
}

} // namespace
} // namespace mxg
