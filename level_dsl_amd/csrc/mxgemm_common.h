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

// Lambdas in the kernels carry this so that the K loop is one straight-line
// body (an outlined call would move the accumulators through scratch).
#define MXG_INLINE __attribute__((always_inline))

namespace mxg {

template <int V>
struct int_c {
    static constexpr int value = V;
};
// Calls f(int_c<0>{}), ..., f(int_c<N-1>{}) (compile-time loop index).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(int_c<I>{});
        static_for<N, I + 1>(f);
    }
}

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Word 3 of a gfx9-family raw buffer descriptor (32-bit data format, no
// swizzle, no stride).
constexpr int kRsrcWord3 = 0x00020000;
// A voffset beyond every record count used (all descriptors built below
// cover < 2^31 bytes).
constexpr uint32_t kOob = 0x80000000u;

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void *lds_ptr_t;

// Arguments shared by every kernel (validated on the host).
struct GemmArgs {
    const uint8_t *A;
    const uint8_t *As;
    const uint8_t *B;
    const uint8_t *Bs;
    void *C;
    int M, N, K, KB;       // KB = K / 32
    int tiles_m, tiles_n;
    int use_acc;           // 0 / 1
    int out_bf16;          // 0 fp32, 1 bf16
    int scale_dword;       // 2: KB % 16 == 0 and scale bases 16-byte aligned (preshuffled:
                           // KB % 16 == 0); 1: KB % 4 == 0 and 4-byte aligned; 0: neither
    int scale_ps;          // 1: scales in the preshuffled layout (scale_at), else row-major
    int c_vec;             // 1: N % 4 == 0 (aligned vector stores of C); 2: also N % 8 == 0
                           // (16-byte stores of 8 bf16)
    int splits;            // small-M exact path: K splits per column tile (1: none)
    float *ws;             // split-K partial tiles (splits > 1)
    uint32_t *cnt;         // split-K arrival counters, zero between calls
};

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

__device__ __forceinline__ v4i load16(rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// non-temporal (the NT cache-policy bit) 16-byte load, for data read once
__device__ __forceinline__ v4i load16_nt(rsrc_t r, uint32_t off)
{
    constexpr int kNT = 2;
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNT));
}

__device__ __forceinline__ uint32_t load4(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

__device__ __forceinline__ uint32_t load1(rsrc_t r, uint32_t off)
{
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

// 16 bytes per lane straight into LDS: lane i of the wave writes
// lds_base + 16 i .. + 15 (buffer_load_dwordx4 ... lds; lds_base must be
// the same for the whole wave).  Out-of-range lanes write zeros.
__device__ __forceinline__ void load16_lds(rsrc_t r, void *lds_base, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_base, 16, off, 0, 0, 0);
}

// x itself, hidden from the optimizer's reassociation of address arithmetic
// (an empty asm statement: no instruction is emitted).  v: a per-lane
// value, s: a wave-uniform one.
__device__ __forceinline__ uint32_t opaque_v(uint32_t x)
{
    asm("" : "+v"(x));
    return x;
}
__device__ __forceinline__ uint32_t opaque_s(uint32_t x)
{
    asm("" : "+s"(x));
    return x;
}

// Wait until every vector-memory operation of this wave has completed,
// including loads that write LDS directly, which the compiler does not
// track (s_waitcnt vmcnt(0)).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Workgroup barrier without a memory fence (__syncthreads' release fence
// would also wait for every direct-to-LDS load in flight).  For LDS data
// that each wave has already waited for itself; the signal fences keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void barrier_nofence()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until at most N of this wave's vector-memory operations are in
// flight (s_waitcnt vmcnt(N)); they complete in issue order.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// ---- scale layouts ---------------------------------------------------------
// Row-major: scale byte (r, kb) of an operand with KB = K/32 blocks per row
// at r * KB + kb.  Preshuffled (KB % 4 == 0): rows in groups of 32 and blocks
// in groups of 4; the pair of groups (r / 32, kb / 4) is one 128-byte unit
// at (r / 32) * 32 KB + (kb / 4) * 128 that holds the 32 rows' 4-byte words
// in row order, so the word that lane l of a 32-row MFMA fragment needs is
// byte 4 l of the unit and one wave's load of it is one 128-byte line.  A
// group of 32 rows spans 32 KB bytes in both layouts: a row offset that is
// a multiple of 32 moves the base pointer alike.  The last group is padded
// to 32 rows (bytes of rows past the operand are never used for an output).
// The offset is a row part plus a block part.
__device__ __forceinline__ uint32_t scale_row(uint32_t r, int KB, int ps)
{
    return ps ? (r & ~31u) * (uint32_t)KB + (r & 31u) * 4u : r * (uint32_t)KB;
}
__device__ __forceinline__ uint32_t scale_col(uint32_t kb, int ps)
{
    return ps ? (kb & ~3u) * 32u + (kb & 3u) : kb;
}
__device__ __forceinline__ uint32_t scale_at(uint32_t r, uint32_t kb, int KB, int ps)
{
    return scale_row(r, KB, ps) + scale_col(kb, ps);
}
// bytes of `rows` scale rows from a multiple of 32 (preshuffled: whole groups)
__device__ __forceinline__ uint32_t scale_span(int rows, int KB, int ps)
{
    return (uint32_t)(ps ? (rows + 31) & ~31 : rows) * (uint32_t)KB;
}

// Scale bytes kb0 .. kb0+3 of scale row r as one little-endian dword; bytes
// past KB read as zero.  `dword` selects one aligned 4-byte load (KB % 4 == 0
// and a 4-byte aligned base; always so when preshuffled), else four byte
// loads.
__device__ __forceinline__ uint32_t load_scale4(rsrc_t rs, uint32_t r, int KB, int kb0, int dword,
                                                int ps)
{
    if (dword) return __builtin_amdgcn_raw_buffer_load_b32(rs, scale_at(r, kb0, KB, ps), 0, 0);
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
        v |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(
                 rs, kb0 + b < KB ? r * KB + kb0 + b : kOob, 0, 0)
             << (8 * b);
    return v;
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

// Two floats rounded to bf16 (RNE) and packed, a in the low half: one
// v_cvt_pk_bf16_f32 (two scalar conversions cost a shift and an OR more).
typedef float v2f_pack __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_pack __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    const v2bf_pack h = __builtin_convertvector((v2f_pack){a, b}, v2bf_pack);
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16)
{
    return __builtin_bit_cast(float, bits16 << 16);
}

// Epilogue store of 4 consecutive columns n..n+3 of one row of C, element
// index e0 = row * N + n relative to the descriptor rC.  use_acc adds the
// previous C (fp32, or bf16 widened) before the single rounding to the
// output type.  With c_vec (N % 4 == 0) one 16-byte (fp32) or 8-byte (bf16)
// store; otherwise per-element stores with columns >= N masked.  Rows past
// the descriptor's range are dropped by the hardware.
__device__ __forceinline__ void store_c4(rsrc_t rC, uint32_t e0, int n, int N, v4f v, int out_bf16,
                                         int use_acc, int c_vec)
{
    const int esz = out_bf16 ? 2 : 4;
    if (c_vec) {
        const uint32_t off = n < N ? e0 * esz : kOob;
        if (!out_bf16) {
            if (use_acc) v += __builtin_bit_cast(v4f, load16(rC, off));
            store16(rC, off, v);
        } else {
            if (use_acc) {
                v2i old = __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(rC, off, 0, 0));
                v[0] += bf16_to_f32((uint32_t)old[0] & 0xffffu);
                v[1] += bf16_to_f32((uint32_t)old[0] >> 16);
                v[2] += bf16_to_f32((uint32_t)old[1] & 0xffffu);
                v[3] += bf16_to_f32((uint32_t)old[1] >> 16);
            }
            v2i o = {(int)pack_bf16x2(v[0], v[1]), (int)pack_bf16x2(v[2], v[3])};
            store8(rC, off, o);
        }
        return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t off = (n + e) < N ? (e0 + e) * esz : kOob;
        float x = v[e];
        if (!out_bf16) {
            if (use_acc) x += __builtin_bit_cast(float, load4(rC, off));
            store4(rC, off, __builtin_bit_cast(uint32_t, x));
        } else {
            if (use_acc)
                x += bf16_to_f32((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rC, off, 0, 0));
            store2(rC, off, (uint16_t)bf16_bits(x));
        }
    }
}

// Epilogue store of 8 consecutive columns n..n+7 of one row of C as bf16,
// element index e0 = row * N + n (N % 8 == 0 and n % 8 == 0, so the 16
// bytes are aligned): use_acc adds the previous C (bf16 widened) before the
// single rounding; one 16-byte store (buffer_store_dwordx4).  Columns at
// or past N are dropped (off = kOob), rows past the descriptor by the
// hardware.
__device__ __forceinline__ void store_bf16x8(rsrc_t rC, uint32_t e0, int n, int N, v4f lo, v4f hi,
                                             int use_acc)
{
    const uint32_t off = n < N ? e0 * 2 : kOob;
    if (use_acc) {
        const v4i old = load16(rC, off);
        lo[0] += bf16_to_f32((uint32_t)old[0] & 0xffffu);
        lo[1] += bf16_to_f32((uint32_t)old[0] >> 16);
        lo[2] += bf16_to_f32((uint32_t)old[1] & 0xffffu);
        lo[3] += bf16_to_f32((uint32_t)old[1] >> 16);
        hi[0] += bf16_to_f32((uint32_t)old[2] & 0xffffu);
        hi[1] += bf16_to_f32((uint32_t)old[2] >> 16);
        hi[2] += bf16_to_f32((uint32_t)old[3] & 0xffffu);
        hi[3] += bf16_to_f32((uint32_t)old[3] >> 16);
    }
    const v4i o = {(int)pack_bf16x2(lo[0], lo[1]), (int)pack_bf16x2(lo[2], lo[3]),
                   (int)pack_bf16x2(hi[0], hi[1]), (int)pack_bf16x2(hi[2], hi[3])};
    __builtin_amdgcn_raw_buffer_store_b128(o, rC, off, 0, 0);
}

// One 32x32x64 scaled MFMA: D = (X * 2^(sx-127)) @ (Y * 2^(sy-127)) + C where
// X supplies the 32 output rows and Y the 32 output columns.  Operand layout
// of gfx950 (measured on the device with one-hot inputs): lane l holds row
// l % 32; with h = l / 32, its register bytes 0..15 carry K 16h..16h+15 and
// bytes 16..31 carry K 32+16h..32+16h+15; lane half h supplies the scale of
// the row's K block h (K 32h..32h+31), taken from byte OP of sx / sy.
// Accumulator register r of lane l is D[8 (r/4) + 4 (l/32) + r%4][l % 32].
template <int FX, int FY, int OP>
__device__ __forceinline__ v16f mfma_scaled(v8i x, v8i y, v16f c, uint32_t sx, uint32_t sy)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, FX, FY, OP, (int)sx, OP,
                                                           (int)sy);
}

// e8m0 scale byte s -> the fp32 value 2^(s-127): byte 0 is the fp32
// subnormal 2^-127, byte 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s)
{
    const uint32_t bits = s == 0u ? 0x00400000u : (s == 255u ? 0x7fc00000u : s << 23);
    return __builtin_bit_cast(float, bits);
}

// Byte `b` of the scale dword d as the fp32 2^(s-127), valid for s in
// 1..254 (one shift).  The fast loops of the exact kernels only use it for
// bytes inside the format's scale window (below); a wave that meets any
// other byte recomputes its outputs on the fallback path, which decodes with
// clamped scales.
template <int b>
__device__ __forceinline__ float scale_f32(uint32_t d)
{
    return __builtin_bit_cast(float, ((d >> (8 * b)) & 0xffu) << 23);
}

// ---- scale windows of the exact (decode-to-bf16) path ----------------------
// A code of format F (0 e4m3, 1 e5m2) times 2^(s-127) is a bf16 normal
// number (or zero, or the code's own inf/NaN) for every code exactly when the
// scale byte s lies in [scale_lo<F>, scale_hi<F>]: the smallest nonzero
// magnitude (e4m3 2^-9, e5m2 2^-16) must reach 2^-126 and the largest (448 =
// 1.75 * 2^8, 57344 = 1.75 * 2^15) must stay below 2^128.  Inside the window
// the decode is exact and the bf16 MFMA forms exact products.
template <int F>
__device__ __forceinline__ constexpr int scale_lo() { return F == 0 ? 10 : 17; }
template <int F>
__device__ __forceinline__ constexpr int scale_hi() { return F == 0 ? 246 : 239; }

typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

// Running check of the scale bytes one lane has seen against a window
// [lo, hi], in one register: bytes 0, 2 and bytes 1, 3 of each dword are
// spread into two packed-u16 pairs (v_perm_b32), lo is subtracted with u16
// wrap-around (a byte below lo becomes 65536 - lo + byte, far above any
// window width), and the packed maximum is kept.  A byte lies outside the
// window exactly when its value exceeds hi - lo.  lo2 is lo in each u16 half.
struct ScaleRange {
    v2u16 mx;
    __device__ __forceinline__ void init() { mx = v2u16{0, 0}; }
    __device__ __forceinline__ void add(uint32_t d, v2u16 lo2)
    {
        // selector bytes: 0x0c is the constant 0x00, 0..3 are the bytes of d
        const v2u16 e = __builtin_bit_cast(v2u16, __builtin_amdgcn_perm(0u, d, 0x0c020c00u));
        const v2u16 o = __builtin_bit_cast(v2u16, __builtin_amdgcn_perm(0u, d, 0x0c030c01u));
        mx = __builtin_elementwise_max(mx, __builtin_elementwise_max(e - lo2, o - lo2));
    }
    // width = hi - lo of the window the bytes were checked against
    __device__ __forceinline__ bool outside(int width) const
    {
        const int m = mx[0] > mx[1] ? mx[0] : mx[1];
        return m > width;
    }
};

// The window of format F as (lo in each u16 half, hi - lo).
template <int F>
__device__ __forceinline__ constexpr v2u16 window_lo2()
{
    return v2u16{(unsigned short)scale_lo<F>(), (unsigned short)scale_lo<F>()};
}
template <int F>
__device__ __forceinline__ constexpr int window_width() { return scale_hi<F>() - scale_lo<F>(); }

// Bytes of dword d at or past byte `valid` (0..4) replaced by 127, a byte
// inside every window (scale bytes past the end of a row are not data).
__device__ __forceinline__ uint32_t mask_scale_tail(uint32_t d, int valid)
{
    const uint32_t keep = valid >= 4 ? 0xffffffffu : ((1u << (8 * valid)) - 1u);
    return (d & keep) | (0x7f7f7f7fu & ~keep);
}

// The fallback's decode scale and remainder for scale byte s of format F: the
// operand is decoded with the clamped byte c (exact, inside the window), and
// the block's partial sum is later multiplied by 2^(s - c) (ldexp), which is
// exact unless the true contribution leaves the fp32 range.  Byte 255 (NaN)
// is returned through `nan` (NaN, else 0), to be added to the result.
template <int F>
__device__ __forceinline__ void clamp_scale(uint32_t s, float &dec, int &rem, float &nan)
{
    const int c = (int)s < scale_lo<F>() ? scale_lo<F>() : ((int)s > scale_hi<F>() ? scale_hi<F>() : (int)s);
    dec = __builtin_bit_cast(float, (uint32_t)c << 23);
    rem = (int)s - c;
    nan = s == 255u ? __builtin_nanf("") : 0.0f;
}

// Two fp8 codes (bytes 2*hi, 2*hi+1 of w) -> two bf16 equal to the codes' values
// times `scale`, rounded to nearest even (v_cvt_scalef32_pk_bf16_fp8 / _bf8).
// For every code and every power-of-two scale 2^-127..2^127 this was checked
// on the device to equal round-to-nearest-even of the exact product; it is
// exact whenever that product is a bf16 number.
template <int F, bool HI>
__device__ __forceinline__ v2bf cvt2(uint32_t w, float scale)
{
    if constexpr (F == 0)
        return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, HI);
    else
        return __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, scale, HI);
}

// 16 fp8 codes (one 16-byte chunk, byte order) scaled -> 16 bf16 as two
// 8-element MFMA operands (bytes 0..7 and 8..15).
template <int F>
__device__ __forceinline__ void decode16(v4i x, float scale, v8bf &lo, v8bf &hi)
{
    const v2bf a0 = cvt2<F, false>((uint32_t)x[0], scale), a1 = cvt2<F, true>((uint32_t)x[0], scale);
    const v2bf b0 = cvt2<F, false>((uint32_t)x[1], scale), b1 = cvt2<F, true>((uint32_t)x[1], scale);
    const v2bf c0 = cvt2<F, false>((uint32_t)x[2], scale), c1 = cvt2<F, true>((uint32_t)x[2], scale);
    const v2bf d0 = cvt2<F, false>((uint32_t)x[3], scale), d1 = cvt2<F, true>((uint32_t)x[3], scale);
    lo = v8bf{a0[0], a0[1], a1[0], a1[1], b0[0], b0[1], b1[0], b1[1]};
    hi = v8bf{c0[0], c0[1], c1[0], c1[1], d0[0], d0[1], d1[0], d1[1]};
}

// 8 fp8 codes (bytes 0..7 of x) scaled -> 8 bf16, one MFMA operand.
template <int F>
__device__ __forceinline__ v8bf decode8(v2i x, float scale)
{
    const v2bf a0 = cvt2<F, false>((uint32_t)x[0], scale), a1 = cvt2<F, true>((uint32_t)x[0], scale);
    const v2bf b0 = cvt2<F, false>((uint32_t)x[1], scale), b1 = cvt2<F, true>((uint32_t)x[1], scale);
    return v8bf{a0[0], a0[1], a1[0], a1[1], b0[0], b0[1], b1[0], b1[1]};
}

// bf16 MFMAs: products of bf16 operands are exact and, as measured on the
// device, summed without the narrow per-group alignment of the fp8 MFMAs, so
// an fp8 x fp8 x 2^s x 2^t product sum decoded to bf16 is accumulated at fp32
// precision.  32x32x16: accumulator layout as in mfma_scaled; 16x16x32:
// register r of lane l is D[4 (l/16) + r][l % 16].
__device__ __forceinline__ v16f mfma_bf16_32(v8bf x, v8bf y, v16f c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_bf16_16(v8bf x, v8bf y, v4f c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
}

} // namespace mxg
