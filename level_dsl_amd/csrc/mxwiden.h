// mxwiden.h -- rewrite sub-byte MX operand codes (e2m1, e2m3, e3m2) as e4m3
// bytes.
//
// Every value of the three sub-byte members of the F8F6F4 operand family
// that the scaled dot of the TLX pages accepts ("Scaled dot" on the
// async-compute page) is an e4m3 value: their magnitudes run from 2^-4
// (e3m2's smallest subnormal) to 28 (e3m2's largest), with at most three
// mantissa bits (e2m3), and e4m3 holds 2^-6 .. 448 as normals with three
// mantissa bits.  So the rewrite is exact, keeps the block scales as they
// are, and an operand pair that the scaled MFMA cannot multiply exactly
// (e3m2, or a sub-byte format beside fp8 or beside another sub-byte format)
// runs on the exact fp8 path with unchanged results.
//
// Layout: an operand of `n` codes (rows x K, K a multiple of 32) is one flat
// code string, since every row is a whole number of 32-code blocks.  Thread
// t rewrites codes 16t .. 16t+15: 8 source bytes for e2m1 (two codes per
// byte, the even code in the low nibble), 12 for e2m3 / e3m2 (code k at bits
// 6k .. 6k+5 of the little-endian bit string), and one 16-byte store of
// e4m3 bytes, so a wave's loads and stores are contiguous.
//
// The byte of each code comes from a table of the format's 16 or 64 codes
// in LDS, filled once per workgroup: a computed conversion costs about 15
// VALU operations a code, which held the kernel near 3 TB/s on VALU issue;
// the lookup is one conflict-free LDS byte read (the 64-byte table spans 16
// distinct banks) between the bit extract and the merge.  Loads and stores
// are non-temporal, as in the streaming copy: every byte is touched once
// (measured 69.5 against 73.6 us for a 28672 x 8192 e3m2 operand).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace mxg::widen {

typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int THREADS = 256;
constexpr int CODES = 16;  // per thread

// One code (sign bit above EB exponent bits above MB mantissa bits, exponent
// bias BIAS, no inf / NaN encodings) -> the e4m3 byte of the same value.
// Normal codes keep their unbiased exponent (rebiased by 7) and their
// mantissa, shifted up to three bits; a subnormal m * 2^(1-BIAS-MB) is
// normalised at its leading bit p: 2^(p+1-BIAS-MB) * (1 + (m - 2^p) / 2^p).
// Both land in e4m3's normal range for the three formats (exponent fields
// 3 .. 11), and a signed zero stays a signed zero.
template <int EB, int MB, int BIAS>
__device__ __forceinline__ uint32_t to_e4m3(uint32_t c)
{
    const uint32_t s = (c >> (EB + MB)) & 1u;
    const uint32_t e = (c >> MB) & ((1u << EB) - 1u);
    const uint32_t m = c & ((1u << MB) - 1u);
    uint32_t mag;
    if (e != 0u) {
        mag = ((e + 7u - BIAS) << 3) | (m << (3 - MB));
    } else if (m == 0u) {
        mag = 0u;
    } else {
        const uint32_t p = 31u - (uint32_t)__builtin_clz(m);
        mag = ((p + 8u - BIAS - MB) << 3) | ((m - (1u << p)) << (3u - p));
    }
    return (s << 7) | mag;
}

// FMT: 4 = e2m1, 2 = e2m3, 3 = e3m2 (the library's format numbers)
template <int FMT>
__global__ __launch_bounds__(THREADS) void kernel(const uint8_t *__restrict__ src,
                                                  uint8_t *__restrict__ dst, uint64_t n)
{
    static_assert(FMT == 4 || FMT == 2 || FMT == 3, "sub-byte formats only");
    constexpr int EB = FMT == 4 ? 2 : FMT == 2 ? 2 : 3;
    constexpr int MB = FMT == 4 ? 1 : FMT == 2 ? 3 : 2;
    constexpr int BIAS = FMT == 3 ? 3 : 1;
    constexpr int NCODES = 1 << (1 + EB + MB);
    static_assert(NCODES <= THREADS, "one table entry per thread");
    __shared__ uint8_t lut[NCODES];
    if (threadIdx.x < NCODES) lut[threadIdx.x] = (uint8_t)to_e4m3<EB, MB, BIAS>(threadIdx.x);
    __syncthreads();
    const uint64_t groups = n / CODES;
    const uint64_t stride = (uint64_t)gridDim.x * THREADS;
    for (uint64_t t = (uint64_t)blockIdx.x * THREADS + threadIdx.x; t < groups; t += stride) {
        uint32_t out[4] = {0u, 0u, 0u, 0u};
        if constexpr (FMT == 4) {
            const v2u w = __builtin_nontemporal_load(reinterpret_cast<const v2u *>(src + 8 * t));
#pragma unroll
            for (int j = 0; j < CODES; ++j) {
                const uint32_t word = j < 8 ? w.x : w.y;
                const uint32_t c = (word >> (4 * (j & 7))) & 15u;
                out[j >> 2] |= (uint32_t)lut[c] << (8 * (j & 3));
            }
        } else {
            // 12 bytes at a 4-byte aligned offset: three dwords
            const uint32_t *p = reinterpret_cast<const uint32_t *>(src + 12 * t);
            const uint32_t p0 = __builtin_nontemporal_load(p), p1 = __builtin_nontemporal_load(p + 1);
            const uint64_t lo = (uint64_t)p0 | ((uint64_t)p1 << 32);
            const uint32_t hi = __builtin_nontemporal_load(p + 2);
#pragma unroll
            for (int j = 0; j < CODES; ++j) {
                const int b = 6 * j;  // first bit of code j
                uint32_t c;
                if (b + 6 <= 64)
                    c = (uint32_t)(lo >> b) & 63u;
                else if (b >= 64)
                    c = (hi >> (b - 64)) & 63u;
                else
                    c = ((uint32_t)(lo >> b) | (hi << (64 - b))) & 63u;
                out[j >> 2] |= (uint32_t)lut[c] << (8 * (j & 3));
            }
        }
        const v4u o = {out[0], out[1], out[2], out[3]};
        __builtin_nontemporal_store(o, reinterpret_cast<v4u *>(dst + 16 * t));
    }
}

}  // namespace mxg::widen
