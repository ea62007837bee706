// k_large_native.hip -- the 256 x 256-tile kernel on the scaled MFMA,
// e4m3 / e5m2 operands (the native opt-in).
#include "launch_large.h"
#include "mxgemm_launch.h"

namespace mxg {

hipError_t launch_large_native(int f, const GemmArgs &a, hipStream_t s)
{
    switch (f) {
    case 0: return launch_large<0, 0, true>(a, s);
    case 1: return launch_large<0, 1, true>(a, s);
    case 2: return launch_large<1, 0, true>(a, s);
    default: return launch_large<1, 1, true>(a, s);
    }
}

} // namespace mxg
