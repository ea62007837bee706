// k_skinny_e2m1.hip -- the small-M scaled-MFMA kernel, e2m1 x e2m1 and e2m3 x e2m3.
#include "launch_skinny.h"
#include "mxgemm_launch.h"

namespace mxg {

hipError_t launch_skinny_e2m1(const GemmArgs &a, hipStream_t s) { return launch_skinny<4, 4>(a, s); }
hipError_t launch_skinny_e2m3(const GemmArgs &a, hipStream_t s) { return launch_skinny<2, 2>(a, s); }

} // namespace mxg
