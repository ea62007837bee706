// k_large_e2m1.hip -- the 256 x 256-tile kernel on the scaled MFMA for the
// sub-byte formats: e2m1 x e2m1 and e2m3 x e2m3.
#include "launch_large.h"
#include "mxgemm_launch.h"

namespace mxg {

hipError_t launch_large_e2m1(const GemmArgs &a, hipStream_t s) { return launch_large<4, 4, true>(a, s); }
hipError_t launch_large_e2m3(const GemmArgs &a, hipStream_t s) { return launch_large<2, 2, true>(a, s); }

} // namespace mxg
