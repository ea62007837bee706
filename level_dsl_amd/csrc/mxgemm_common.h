// mxgemm_common.h -- device-side building blocks shared by the gfx950 kernels.
//
// Raw buffer loads and stores through a resource descriptor: the hardware
// drops stores and returns zero for loads whose byte offset lies beyond the
// descriptor's record count, which is how every tile edge is masked (TLX
// global-memory page, "Global memory access": buffer operations take a
// scalar base and 32-bit offsets and let the hardware do the
// out-of-bounds check).  Offsets inside a row that must be masked (K and N
// tails) are pushed to kOob, far past any record count built here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxg {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Word 3 of a gfx9-family raw buffer descriptor (32-bit data format, no
// swizzle, no stride).
constexpr int kRsrcWord3 = 0x00020000;
// A voffset beyond every record count used (all descriptors built below
// cover < 2^31 bytes).
constexpr uint32_t kOob = 0x80000000u;

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

__device__ __forceinline__ v4i load16(rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ uint32_t load4(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

__device__ __forceinline__ uint32_t load1(rsrc_t r, uint32_t off)
{
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

__device__ __forceinline__ void store16(rsrc_t r, uint32_t off, v4f v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v), r, off, 0, 0);
}

__device__ __forceinline__ void store8(rsrc_t r, uint32_t off, v2i v)
{
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}

__device__ __forceinline__ void store4(rsrc_t r, uint32_t off, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}

__device__ __forceinline__ void store2(rsrc_t r, uint32_t off, uint16_t v)
{
    __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}

// fp32 -> bf16 bit pattern, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_bits(float f)
{
    __bf16 h = (__bf16)f;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16)
{
    return __builtin_bit_cast(float, bits16 << 16);
}

// One 32x32x64 scaled MFMA: D = (X * 2^(sx-127)) @ (Y * 2^(sy-127)) + C where
// X supplies the 32 output rows and Y the 32 output columns; each lane holds
// 32 consecutive K bytes of one row of X (lane % 32) in K half (lane / 32),
// and byte 0 of sx / sy is the scale of that row's 32-element K block.
template <int FX, int FY>
__device__ __forceinline__ v16f mfma_scaled(v8i x, v8i y, v16f c, uint32_t sx, uint32_t sy)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, FX, FY, 0, (int)sx, 0,
                                                           (int)sy);
}

} // namespace mxg
