// k_large_exact_b.hip -- the 256 x 256-tile kernel, exact mode, e5m2 A
// operands (a translation unit of its own so that the library builds in
// parallel).
#include "launch_large.h"
#include "mxgemm_launch.h"

namespace mxg {

hipError_t launch_large_exact_b(int f, const GemmArgs &a, hipStream_t s)
{
    return f == 2 ? launch_large<1, 0, false>(a, s) : launch_large<1, 1, false>(a, s);
}

} // namespace mxg
