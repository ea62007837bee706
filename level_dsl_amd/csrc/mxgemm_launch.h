// mxgemm_launch.h -- the kernel launchers that mxgemm.hip (the host side of
// the C ABI) calls.  Each is defined in its own translation unit (k_*.hip),
// which holds that kernel's template instantiations, so that the library
// builds in parallel.  All launch on the caller's stream and return
// hipGetLastError() of the launch.
#pragma once

#include <hip/hip_runtime.h>

#include "mxgemm_common.h"
#include "mxquant.h"

namespace mxg {

// f = 2 fmtA + fmtB for e4m3 (0) / e5m2 (1) operands
hipError_t launch_large_exact(int f, const GemmArgs &a, hipStream_t s);   // k_large_exact.hip
hipError_t launch_large_exact_b(int f, const GemmArgs &a, hipStream_t s); // k_large_exact_b.hip (f = 2, 3)
hipError_t launch_large_native(int f, const GemmArgs &a, hipStream_t s);  // k_large_native.hip
hipError_t launch_large_e2m1(const GemmArgs &a, hipStream_t s);           // k_large_e2m1.hip
hipError_t launch_large_e2m3(const GemmArgs &a, hipStream_t s);           // k_large_e2m1.hip
hipError_t launch_stream_exact(int f, const GemmArgs &a, hipStream_t s);  // k_stream.hip
hipError_t launch_skinny_native(int f, const GemmArgs &a, hipStream_t s); // k_skinny_fp8.hip
hipError_t launch_skinny_e2m1(const GemmArgs &a, hipStream_t s);          // k_skinny_e2m1.hip
hipError_t launch_skinny_e2m3(const GemmArgs &a, hipStream_t s);          // k_skinny_e2m1.hip
// sel = 2 fmt + (x_dtype == bf16), fmt in {0, 1, 2, 3, 4}
hipError_t launch_quant(int sel, const quant::QuantArgs &a, dim3 grid, dim3 block,
                        hipStream_t s);                                    // k_quant.hip
hipError_t launch_copy(const uint8_t *src, uint8_t *dst, uint64_t bytes, hipStream_t s);  // k_quant.hip
// n codes of format fmt (4 e2m1, 2 e2m3, 3 e3m2; n % 16 == 0) -> n e4m3 bytes
hipError_t launch_widen(int fmt, const uint8_t *src, uint8_t *dst, uint64_t n, hipStream_t s);  // k_quant.hip
// row-major scale bytes (rows x KB, KB % 4 == 0) to the preshuffled layout
hipError_t launch_preshuffle(const uint8_t *src, uint8_t *dst, uint64_t rows, int KB,
                             hipStream_t s);                               // k_quant.hip

} // namespace mxg
