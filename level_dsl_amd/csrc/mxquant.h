// mxquant.h -- MX block quantization for gfx950: fp32 or bf16 values to fp8
// codes (e4m3 / e5m2) with one e8m0 scale byte per 32 consecutive elements
// of a row (the operand layout of the scaled multiply: a uint8 scale tile
// whose K extent is BLOCK_K // 32, TLX async-compute page, "TMEM-backed MX
// Scales").  Per block: the scale is the smallest power of two 2^e with
// max|x| <= MAX * 2^e (MAX = 448 for e4m3, 57344 for e5m2; an all-zero
// block takes the smallest scale), stored as e + 127 clamped to 0..254, and
// each code is x * 2^-e rounded to nearest even.  e2m1 (format 4: MAX = 6,
// codes packed two per byte along K, the even k in the low nibble), e2m3
// (format 2: MAX = 7.5) and e3m2 (format 3: MAX = 28; both packed four codes
// per three bytes, code k at bits 6k .. 6k+5 of the row's little-endian bit
// string) follow the same recipe.
//
// The work is a flat stream (K % 32 == 0, so blocks never straddle rows):
//   * a wave owns 4 x 64 consecutive 16-byte chunks of X; lane l loads
//     chunks l, 64 + l, 128 + l, 192 + l (every load instruction reads 1 KiB
//     of contiguous memory), so a block is 8 lanes of fp32 or 4 lanes of
//     bf16;
//   * the block maximum is an integer max over the magnitude bits (IEEE
//     order for finite values), reduced across the block's lanes with
//     cross-lane shuffles; the scale byte is read off its exponent and
//     mantissa fields: max|x| = 1.f * 2^(E-127) <= 0.875 * 2^(e+9) for e4m3
//     gives e + 127 = E - 8 + (f > 0.75), for e5m2 E - 15 + (f > 0.75), for
//     e2m1 (6 = 1.5 * 2^2) E - 2 + (f > 0.5), for e2m3 (7.5 = 1.875 * 2^2)
//     E - 2 + (f > 0.875), for e3m2 (28 = 1.75 * 2^4) E - 4 + (f > 0.75);
//   * x * 2^(127 - scale) is exact (a power-of-two product whose magnitude
//     is at most MAX), and v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 /
//     v_cvt_scalef32_pk_fp4_f32 (scale 1) round it to nearest even, two
//     values per instruction; the 6-bit formats round in software
//     (fp6_code): one fp32 add of a power of two rounds the value to its
//     binade's grid, half to even, and leaves the grid index in the sum's
//     mantissa;
//   * codes leave as one 4-byte (fp32 input) or 8-byte (bf16 input) store
//     per lane and chunk -- e2m1: 2 or 4 bytes, e2m3 / e3m2: 3 or 6 bytes
//     (4 or 8 codes, whole bytes) -- contiguous across the
//     wave; the first lane of each block stores its scale byte, at its
//     place in the row-major or the preshuffled scale layout
//     (mxgemm_common.h, scale_at).
// Descriptors are rebased per wave, so every offset stays far below 2^32 and
// the tail of the stream is masked by the descriptors' range checks.
#pragma once

#include "mxgemm_common.h"

namespace mxg {
namespace quant {

constexpr int THREADS = 256;
constexpr int CHUNKS = 4;                 // 16-byte chunks per lane
constexpr int WAVE_BYTES = CHUNKS * 64 * 16;  // input bytes per wave

struct QuantArgs {
    const uint8_t *X;
    uint8_t *codes;
    uint8_t *scales;
    uint64_t n;  // elements (R * K, a multiple of 32)
    int KB;      // K / 32, scale bytes per row
    int ps;      // 1: preshuffled scale layout (KB % 4 == 0)
    uint64_t scale_bytes;  // of the whole scale buffer (preshuffled: rows padded to 32)
};

template <int FMT>
__device__ __forceinline__ uint32_t cvt_pair(float a, float b, uint32_t old, bool hi)
{
    if constexpr (FMT == 0)
        return (uint32_t)(hi ? __builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, true)
                             : __builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, false));
    else
        return (uint32_t)(hi ? __builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, true)
                             : __builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, false));
}

// e2m1: two values into byte B of `old` (round to nearest even)
template <int B>
__device__ __forceinline__ uint32_t cvt_fp4_pair(uint32_t old, float a, float b)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, B);
}

// e2m3 (MB = 3, BIAS = 1) / e3m2 (MB = 2, BIAS = 3): the 6-bit code of x *
// 2^sh rounded to nearest even, for |x| * 2^sh <= the format's largest
// value.  The grid spacing at magnitude y is q = 2^(k-MB) in binade 2^k,
// and 2^(1-BIAS-MB) below the smallest normal 2^(1-BIAS).  Adding C = 2^23
// q to y makes the fp32 adder round y to a multiple of q, half to even (C's
// ulp is q and y < C), and leaves the multiple's index n in the sum's
// mantissa field.  Below the smallest normal the code is n; in binade k it
// is ((k + BIAS - 1) << MB) + n, n running from 2^MB (the binade's first
// value) to 2^(MB+1) (rounded up into the next binade), which is the same
// formula with k clamped to 1 - BIAS.  The sign is x's (a negative value
// that rounds to zero gives -0).
template <int MB, int BIAS>
__device__ __forceinline__ uint32_t fp6_code(float x, int sh)
{
    const uint32_t xb = __builtin_bit_cast(uint32_t, x);
    const float y = __builtin_ldexpf(__builtin_bit_cast(float, xb & 0x7fffffffu), sh);
    const uint32_t e = max(__builtin_bit_cast(uint32_t, y) >> 23, (uint32_t)(128 - BIAS));  // biased k, clamped
    const float c = __builtin_bit_cast(float, (e - MB + 23) << 23);
    const uint32_t n = __builtin_bit_cast(uint32_t, y + c) & 0x7fffffu;
    return ((xb >> 31) << 5) | (((e - (128 - BIAS)) << MB) + n);
}

template <int FMT, int XBF16>
__global__ __launch_bounds__(THREADS) void kernel(QuantArgs p)
{
    constexpr bool FP4 = FMT == 4;
    constexpr bool FP6 = FMT == 2 || FMT == 3;
    constexpr int EPL = XBF16 ? 8 : 4;    // elements per 16-byte chunk
    constexpr int LPB = 32 / EPL;         // lanes per block
    constexpr int ESZ = XBF16 ? 2 : 4;
    constexpr int WAVE_ELEMS = WAVE_BYTES / ESZ;
    // scale byte = E - OFF + (f > THR / 2^23)
    constexpr uint32_t OFF = FMT == 0 ? 8 : FMT == 1 ? 15 : FMT == 3 ? 4 : 2;
    constexpr uint32_t THR = FP4 ? 0x400000u : FMT == 2 ? 0x700000u : 0x600000u;

    const int lane = threadIdx.x & 63;
    const uint64_t e0 = ((uint64_t)blockIdx.x * (THREADS / 64) + (threadIdx.x >> 6)) * WAVE_ELEMS;
    if (e0 >= p.n) return;  // whole wave past the end
    const uint64_t left = p.n - e0;
    const uint32_t ne = left < (uint64_t)WAVE_ELEMS ? (uint32_t)left : (uint32_t)WAVE_ELEMS;
    const rsrc_t rX = make_rsrc(p.X + e0 * ESZ, ne * ESZ);
    const rsrc_t rQ = FP4   ? make_rsrc(p.codes + e0 / 2, ne / 2)
                      : FP6 ? make_rsrc(p.codes + e0 * 3 / 4, ne * 3 / 4)
                            : make_rsrc(p.codes + e0, ne);
    // row-major scales: this wave's bytes from block e0 / 32 on; preshuffled:
    // from the 32-row group of the wave's first block (row r0 = sr0 + 32 g0,
    // block kb0 of it) to the end of the buffer
    const uint64_t b0 = e0 / 32;
    const uint64_t row0 = b0 / (uint64_t)p.KB;
    const uint32_t kb0 = (uint32_t)(b0 - row0 * (uint64_t)p.KB), sr0 = (uint32_t)(row0 & 31u);
    const uint64_t sbase = p.ps ? (row0 - sr0) * (uint64_t)p.KB : b0;
    const uint64_t sleft = p.ps ? p.scale_bytes - sbase : ne / 32;
    const rsrc_t rS = make_rsrc(p.scales + sbase, (uint32_t)(sleft < kOob ? sleft : kOob));

    v4i x[CHUNKS];
#pragma unroll
    // X is read once: non-temporal loads (measured 2% faster than plain ones
    // on the 28672 x 8192 fp32 weight; the same hint on the small-M GEMMs'
    // B stream measured no gain)
    for (int j = 0; j < CHUNKS; ++j) x[j] = load16_nt(rX, (uint32_t)(64 * j + lane) * 16);

#pragma unroll
    for (int j = 0; j < CHUNKS; ++j) {
        // the chunk's elements as fp32, and their largest magnitude (bits)
        float f[EPL];
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            uint32_t b;
            if constexpr (XBF16)
                b = ((uint32_t)x[j][i / 2] >> (16 * (i & 1))) << 16;
            else
                b = (uint32_t)x[j][i];
            f[i] = __builtin_bit_cast(float, b);
            m = max(m, b & 0x7fffffffu);
        }
#pragma unroll
        for (int d = 1; d < LPB; d <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d, 64));
        const int E = (int)(m >> 23);
        int s = E - (int)OFF + ((m & 0x7fffffu) > THR ? 1 : 0);
        s = s < 0 ? 0 : (s > 254 ? 254 : s);
        const int sh = 127 - s;
        const uint32_t c = (uint32_t)(64 * j + lane);  // chunk index within the wave
        if constexpr (FP6) {
            // EPL codes -> 3 EPL / 4 bytes: four codes fill three bytes
            constexpr int MB = FMT == 2 ? 3 : 2, BIAS = FMT == 2 ? 1 : 3;
            uint32_t w[EPL / 4];
#pragma unroll
            for (int q = 0; q < EPL / 4; ++q) {
                w[q] = 0u;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[q] |= fp6_code<MB, BIAS>(f[4 * q + i], sh) << (6 * i);
            }
            if constexpr (XBF16) {
                // 48 bits: w[0] in bytes 0..2, w[1] in bytes 3..5, as three
                // 2-byte stores
                const uint32_t b = c * 6;
                __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(w[0] & 0xffffu), rQ, b, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b16(
                    (unsigned short)((w[0] >> 16) | ((w[1] & 0xffu) << 8)), rQ, b + 2, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(w[1] >> 8), rQ, b + 4, 0, 0);
            } else {
                const uint32_t b = c * 3;
#pragma unroll
                for (int i = 0; i < 3; ++i)
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(w[0] >> (8 * i)), rQ, b + i, 0, 0);
            }
        } else if constexpr (FP4) {
            // EPL codes -> EPL / 2 bytes, the even element in the low nibble
            uint32_t w = cvt_fp4_pair<0>(0u, __builtin_ldexpf(f[0], sh), __builtin_ldexpf(f[1], sh));
            w = cvt_fp4_pair<1>(w, __builtin_ldexpf(f[2], sh), __builtin_ldexpf(f[3], sh));
            if constexpr (XBF16) {
                w = cvt_fp4_pair<2>(w, __builtin_ldexpf(f[4], sh), __builtin_ldexpf(f[5], sh));
                w = cvt_fp4_pair<3>(w, __builtin_ldexpf(f[6], sh), __builtin_ldexpf(f[7], sh));
                store4(rQ, c * 4, w);
            } else {
                __builtin_amdgcn_raw_buffer_store_b16((unsigned short)w, rQ, c * 2, 0, 0);
            }
        } else {
            uint32_t w[EPL / 4];
#pragma unroll
            for (int q = 0; q < EPL / 4; ++q) {
                uint32_t v = cvt_pair<FMT>(__builtin_ldexpf(f[4 * q], sh), __builtin_ldexpf(f[4 * q + 1], sh), 0u, false);
                w[q] = cvt_pair<FMT>(__builtin_ldexpf(f[4 * q + 2], sh), __builtin_ldexpf(f[4 * q + 3], sh), v, true);
            }
            if constexpr (XBF16)
                store8(rQ, c * 8, v2i{(int)w[0], (int)w[1]});
            else
                store4(rQ, c * 4, w[0]);
        }
        if (lane % LPB == 0) {
            uint32_t so = c / LPB;
            if (p.ps) {
                // block so of the wave: block (kb0 + so) % KB of row sr0 +
                // (kb0 + so) / KB of the range (a store past the stream's end
                // is masked)
                const uint32_t q = kb0 + so, dr = q / (uint32_t)p.KB;
                so = so < ne / 32 ? scale_at(sr0 + dr, q - dr * (uint32_t)p.KB, p.KB, 1) : kOob;
            }
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)s, rS, so, 0, 0);
        }
    }
}

} // namespace quant
} // namespace mxg
