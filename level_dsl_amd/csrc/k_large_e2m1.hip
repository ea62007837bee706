// k_large_e2m1.hip -- the 256 x 256-tile kernel, e2m1 x e2m1 on the scaled
// MFMA.
#include "launch_large.h"
#include "mxgemm_launch.h"

namespace mxg {

hipError_t launch_large_e2m1(const GemmArgs &a, hipStream_t s) { return launch_large<4, 4, true>(a, s); }

} // namespace mxg
