// k_large_exact.hip -- the 256 x 256-tile kernel, exact mode (decode to
// bf16), e4m3 A operands (k_large_exact_b.hip: e5m2 A).
#include "launch_large.h"
#include "mxgemm_launch.h"

namespace mxg {

hipError_t launch_large_exact(int f, const GemmArgs &a, hipStream_t s)
{
    switch (f) {
    case 0: return launch_large<0, 0, false>(a, s);
    case 1: return launch_large<0, 1, false>(a, s);
    default: return launch_large_exact_b(f, a, s);
    }
}

} // namespace mxg
