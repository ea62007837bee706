// mxcopy.h -- plain streaming copy through raw buffer loads and stores, the
// measured ceiling ("achievable HBM") that the HBM-bound kernels are compared
// against.  It is the buffer_load / buffer_store pattern of the TLX
// global-memory page ("Example: buffer load and store"): scalar base plus
// 32-bit per-lane offsets, the tail masked by the descriptor's range check.
//
// Each wave moves pieces of UNROLL KiB: lane l loads 16-byte chunks
// u * 64 + l (u < UNROLL) with the non-temporal cache policy (the data is
// read once), then stores them the same way; waves stride over the pieces.
#pragma once

#include "mxgemm_common.h"

namespace mxg {
namespace copy {

constexpr int THREADS = 256;
// 16-byte chunks in flight per lane.  Measured on 1 GiB (read + write):
// 4 chunks with 2 workgroups per CU reached 6.02 TB/s, 8 chunks 5.7-5.96,
// 16 chunks 5.4-5.5; plain (cached) loads and stores lost 5-10%.
constexpr int UNROLL = 4;
constexpr uint32_t PIECE = UNROLL * 64 * 16;  // bytes per wave and iteration

__global__ __launch_bounds__(THREADS) void kernel(const uint8_t *src, uint8_t *dst, uint64_t bytes)
{
    constexpr int kNT = 2;
    const int lane = threadIdx.x & 63;
    const uint64_t waves = (uint64_t)gridDim.x * (THREADS / 64);
    for (uint64_t base = ((uint64_t)blockIdx.x * (THREADS / 64) + (threadIdx.x >> 6)) * PIECE;
         base < bytes; base += waves * PIECE) {
        const uint64_t left = bytes - base;
        const uint32_t n = left < PIECE ? (uint32_t)left : PIECE;
        const rsrc_t rs = make_rsrc(src + base, n), rd = make_rsrc(dst + base, n);
        v4i x[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            x[u] = __builtin_bit_cast(
                v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(u * 64 + lane) * 16, 0, kNT));
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            __builtin_amdgcn_raw_buffer_store_b128(x[u], rd, (uint32_t)(u * 64 + lane) * 16, 0, kNT);
    }
}

} // namespace copy
} // namespace mxg
