// k_skinny_fp8.hip -- the small-M scaled-MFMA kernel, e4m3 / e5m2 operands
// (the native opt-in).
#include "launch_skinny.h"
#include "mxgemm_launch.h"

namespace mxg {

hipError_t launch_skinny_native(int f, const GemmArgs &a, hipStream_t s)
{
    switch (f) {
    case 0: return launch_skinny<0, 0>(a, s);
    case 1: return launch_skinny<0, 1>(a, s);
    case 2: return launch_skinny<1, 0>(a, s);
    default: return launch_skinny<1, 1>(a, s);
    }
}

} // namespace mxg
