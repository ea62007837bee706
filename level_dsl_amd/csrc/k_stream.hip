// k_stream.hip -- the exact small-M kernel (M <= 64), e4m3 / e5m2 operands.
#include "mxgemm_launch.h"
#include "mxgemm_stream.h"

namespace mxg {
namespace {

template <int FA, int FB, int MT>
hipError_t launch_stream_mt(const mxg::GemmArgs &a, hipStream_t s)
{
    const dim3 grid(a.tiles_n * a.splits), block(mxg::stream::threads_for<MT>());
    if (a.scale_dword)
        hipLaunchKernelGGL((mxg::stream::kernel<FA, FB, true, MT>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((mxg::stream::kernel<FA, FB, false, MT>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int FA, int FB>
hipError_t launch_stream(const mxg::GemmArgs &a, hipStream_t s)
{
    switch ((a.M + 15) / 16) {
    case 1: return launch_stream_mt<FA, FB, 1>(a, s);
    case 2: return launch_stream_mt<FA, FB, 2>(a, s);
    case 3: return launch_stream_mt<FA, FB, 3>(a, s);
    default: return launch_stream_mt<FA, FB, 4>(a, s);
    }
}

} // namespace

hipError_t launch_stream_exact(int f, const GemmArgs &a, hipStream_t s)
{
    switch (f) {
    case 0: return launch_stream<0, 0>(a, s);
    case 1: return launch_stream<0, 1>(a, s);
    case 2: return launch_stream<1, 0>(a, s);
    default: return launch_stream<1, 1>(a, s);
    }
}

} // namespace mxg
