// mxgemm_skinny.h -- small-M (M <= 64) MX GEMM kernel for gfx950 on the
// scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4): the native variant for
// e4m3 / e5m2 operands, and the e2m1 x e2m1 path (exact for e2m1).  The
// exact small-M variant for fp8 is mxgemm_stream.h.
//
// With M <= 64 the multiply is bound by reading B once from HBM (about 120
// flop per byte at M = 64, far below the chip's MFMA-to-HBM balance), so
// the kernel is organised around streaming B:
//   * one workgroup per 112 columns of C (N = 28672 gives exactly 256
//     workgroups, one per CU); the four waves split K, wave w taking the
//     128-byte K stages w, w+4, w+8, ... counted from a per-workgroup start
//     stage (workgroup n starts n stages in, wrapping around).  Without the
//     rotation every workgroup reads its B rows at the same K offset at the
//     same time; with a power-of-two row pitch those addresses crowd onto a
//     few memory channels (measured: 4.5 vs 5.5+ TB/s for the bare stream);
//   * operands go straight from global memory into registers, so no LDS
//     staging is needed; each wave keeps a ring of RING stage buffers, so
//     RING - 1 of its stages are loading while it multiplies one.  Lane l
//     works on row l % 16; with g = l / 16 it loads K bytes 16g..16g+15 and
//     64+16g..64+16g+15 of each 128-byte stage (each load instruction reads
//     64 contiguous bytes of 16 rows).  fp8: the two chunks are the 32 codes
//     lane group g contributes to one 16x16x128 step (the instruction's
//     operand layout, measured on the device) and the lane supplies the
//     scale of block g.  e2m1 (two codes per byte): a stage is 256 codes,
//     two steps; each chunk is the 32 codes of one scale block, and the
//     measured e2m1 layout is lane group g holding block g of the step, so
//     the low chunk feeds step 0 (block g) and the high chunk step 1 (block
//     4 + g), with both scale bytes in one dword selected by op_sel;
//   * A (at most 64 x K bytes) is re-read by every workgroup and stays in L2;
//   * at the end the four per-wave partial tiles are summed in a fixed order
//     through LDS (deterministic), use_acc adds the old C, and C is written
//     with coalesced 16-byte (fp32) or 8-byte (bf16) buffer stores;
//   * with few column tiles (N up to 128 tiles of 112) K is split over
//     several workgroups per tile, whose partial tiles are added in split
//     order through a caller-owned workspace.
#pragma once

#include "mxgemm_common.h"

namespace mxg {
namespace skinny {

constexpr int MAX_M = 64;
constexpr int BN = 112;
constexpr int BK = 128;
constexpr int THREADS = 256;
constexpr int WAVES = THREADS / 64;
constexpr int SUB_M = MAX_M / 16, SUB_N = BN / 16;

template <int FX, int FY, int OP = 0>
__device__ __forceinline__ v4f mfma16(v8i x, v8i y, v4f c, uint32_t sx, uint32_t sy)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, FX, FY, OP, (int)sx, OP,
                                                           (int)sy);
}

template <int MT>  // 16-row tiles of A (M <= 16 MT)
struct Stage {
    v8i b[SUB_N];
    v8i a[MT];
    uint32_t sb[SUB_N];  // fp8: block g; e2m1: blocks g (byte 0) and 4 + g (byte 1)
    uint32_t sa[MT];
    int kt;              // the K stage (scale table mode reads its scales at multiply time)
};

// scale modes: how a stage's scale bytes reach the MFMA
enum { SCALES_BYTES = 0,  // byte loads per row and stage
       SCALES_VEC = 1,    // e2m1: one 8-byte load per row and stage
       SCALES_TABLE = 2 }; // the workgroup's whole scale table, loaded once into LDS
constexpr int TABLE_ROWS = MAX_M + BN;  // A rows 0..63, then this workgroup's B rows
// table row pitch for K/32 = kb scale bytes (kb % 16 == 0): an odd number of
// dwords, so that the 16 rows of one read fall in different banks
__host__ __device__ constexpr int table_pitch(int kb) { return kb + 4; }
constexpr int TABLE_BYTES = WAVES * MAX_M * BN * 4;  // shares the reduction buffer
__host__ __device__ constexpr bool table_fits(int kb) { return TABLE_ROWS * table_pitch(kb) <= TABLE_BYTES; }

constexpr int RING = 3;  // stage buffers per wave: RING - 1 loading, one multiplied

// SMODE (the host picks it): SCALES_TABLE when K/32 % 16 == 0 with 16-byte
// aligned scale rows and the table fits: every workgroup loads its scale
// rows (all of K) into LDS with coalesced 16-byte loads once, and reads a
// stage's bytes from there (scattered per-row scale loads had cost about as
// much as A's loads: measured 41 -> 31 us at e2m1, M = 64, N = 28672,
// K = 8192 without them).  Else SCALES_VEC for e2m1 (one 8-byte load per row
// and stage) or byte loads.  (For fp8 a per-stage dword load plus a per-lane
// shift measured slower: it pushes the kernel into register spills.)
// MT: 16-row tiles of A loaded and multiplied (M <= 16 MT), so a
// decode-size M pays only for its own rows.
// SPLIT: workgroup tile + tiles_n * sp runs K split sp of p.splits and the
// splits' partial tiles are summed in split order through the workspace.
template <int FA, int FB, int SMODE, int MT, bool SPLIT>
__global__ __launch_bounds__(THREADS) void kernel(GemmArgs p)
{
    static_assert(MT >= 1 && MT <= SUB_M, "M tiles");
    using Stage = mxg::skinny::Stage<MT>;
    constexpr bool FP4 = FA == 4;  // e2m1 x e2m1; K is the row pitch in bytes
    static_assert(FP4 == (FB == 4), "e2m1 pairs only with e2m1");
    // e2m3 x e2m3 (four codes per three bytes): a stage is 128 codes, 96
    // bytes of a row, one 16x16x128 step; lane group g loads the 24 bytes of
    // block g (16 + 8 bytes) into operand dwords 0..5 and supplies its scale,
    // as for fp8
    constexpr bool FP6 = FA == 2;
    static_assert(FP6 == (FB == 2), "e2m3 pairs only with e2m3");
    static_assert(SMODE != SCALES_VEC || FP4, "vector scale loads are for e2m1");
    constexpr bool SVEC = SMODE == SCALES_VEC, STAB = SMODE == SCALES_TABLE;
    constexpr int SPS = FP4 ? 8 : BK / 32;  // scale bytes per row and stage
    constexpr int SB = FP6 ? 96 : BK;       // bytes of a row per stage
    __shared__ __attribute__((aligned(16))) float red[WAVES][MAX_M][BN];
    static_assert(sizeof(red) == TABLE_BYTES, "the scale table shares the reduction buffer");
    uint8_t *const tab = reinterpret_cast<uint8_t *>(&red[0][0][0]);

    const int tile = SPLIT ? (int)(blockIdx.x % (unsigned)p.tiles_n) : (int)blockIdx.x;
    const int sp = SPLIT ? (int)(blockIdx.x / (unsigned)p.tiles_n) : 0;
    const int n0 = tile * BN;
    const int rows_b = min(BN, p.N - n0);
    const int M = p.M, N = p.N, K = p.K, KB = p.KB;
    // this workgroup's K stages [kbeg, kbeg + nk) of nk_all
    const int nk_all = (K + SB - 1) / SB;
    const int kbeg = SPLIT ? (int)((int64_t)sp * nk_all / p.splits) : 0;
    const int nk = SPLIT ? (int)((int64_t)(sp + 1) * nk_all / p.splits) - kbeg : nk_all;

    const rsrc_t rA = make_rsrc(p.A, (uint32_t)M * K);
    const rsrc_t rB = make_rsrc(p.B + (size_t)n0 * K, (uint32_t)rows_b * K);
    // Scale rows: A from row 0; B from row n0, or with preshuffled scales
    // from the 32-row group that holds it (row n0 is row nsb of the range)
    const int ps = p.scale_ps;
    const int nsb = ps ? n0 & 31 : 0;
    const rsrc_t rAs = make_rsrc(p.As, scale_span(M, KB, ps));
    const rsrc_t rBs = make_rsrc(p.Bs + (size_t)(n0 - nsb) * KB, scale_span(nsb + rows_b, KB, ps));

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, kq = lane >> 4;

    uint32_t boff[SUB_N], aoff[MT], bsrow[SUB_N], asrow[MT];
    // chunks K bytes 16g.. and 64+16g.. of each stage (e2m3: bytes 24g..
    // and 24g+16.. of block g); scale rows
    constexpr int LO = FP6 ? 24 : 16, HI = FP6 ? 16 : 64;
#pragma unroll
    for (int j = 0; j < SUB_N; ++j) {
        boff[j] = (uint32_t)(16 * j + r16) * K + kq * LO;
        bsrow[j] = scale_row((uint32_t)(nsb + 16 * j + r16), KB, ps);
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        aoff[i] = (uint32_t)(16 * i + r16) * K + kq * LO;
        asrow[i] = scale_row((uint32_t)(16 * i + r16), KB, ps);
    }

    // the stage's scale bytes of one row (`row`: the row part of its scale
    // offsets): fp8 block g in byte 0; e2m1 blocks g and 4 + g in bytes 0 and 1
    auto scales_of = [&](rsrc_t rs, uint32_t row, int kb0, bool s0_in, bool s1_in) MXG_INLINE {
        if constexpr (SVEC) {  // row-major scales only
            const v2i v = __builtin_bit_cast(
                v2i, __builtin_amdgcn_raw_buffer_load_b64(rs, s0_in ? row + kb0 : kOob, 0, 0));
            return (((uint32_t)v[0] >> (8 * kq)) & 0xffu) | ((((uint32_t)v[1] >> (8 * kq)) & 0xffu) << 8);
        } else {
            uint32_t v = load1(rs, s0_in ? row + scale_col(kb0 + kq, ps) : kOob);
            if constexpr (FP4) v |= load1(rs, s1_in ? row + scale_col(kb0 + kq + 4, ps) : kOob) << 8;
            return v;
        }
    };

    // table mode: the workgroup's scale rows into LDS (row r < 64: A row r;
    // else B row r - 64 of this workgroup; missing rows read zero), the
    // 16-byte pieces that cover this workgroup's stages, at their places in
    // the row
    const int tpitch = table_pitch(KB);
    if constexpr (STAB) {
        const int c_lo = kbeg * SPS / 16, c_hi = min(KB / 16, ((kbeg + nk) * SPS + 15) / 16);
        const int per_row = c_hi - c_lo;  // 16-byte pieces per row
        if (ps) {
            // a 16-byte piece is one word (4 blocks) of 4 consecutive rows;
            // consecutive threads take consecutive row quads of one word
            constexpr int QUADS = TABLE_ROWS / 4;
            static_assert(MAX_M % 32 == 0 && TABLE_ROWS % 4 == 0, "quads stay within A or B");
            for (int q = tid; q < QUADS * 4 * per_row; q += THREADS) {
                const int r = 4 * (q % QUADS), w = 4 * c_lo + q / QUADS;
                const bool is_a = r < MAX_M;
                const v4i v = load16(is_a ? rAs : rBs,
                                     scale_row((uint32_t)(is_a ? r : r - MAX_M + nsb), KB, 1) + 128u * w);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    *reinterpret_cast<uint32_t *>(tab + (r + e) * tpitch + 4 * w) = (uint32_t)v[e];
            }
        } else {
            for (int q = tid; q < TABLE_ROWS * per_row; q += THREADS) {
                const int r = q / per_row, c = (c_lo + q % per_row) * 16;
                const bool is_a = r < MAX_M;
                const v4i v = load16(is_a ? rAs : rBs, (uint32_t)((is_a ? r : r - MAX_M) * KB + c));
                uint32_t *d = reinterpret_cast<uint32_t *>(tab + r * tpitch + c);
                d[0] = (uint32_t)v[0];
                d[1] = (uint32_t)v[1];
                d[2] = (uint32_t)v[2];
                d[3] = (uint32_t)v[3];
            }
        }
        __syncthreads();
    }
    // table mode: the stage's scale bytes of table row r (fp8: block g;
    // e2m1: blocks g and 4 + g)
    auto table_scales = [&](int r, int kt) MXG_INLINE {
        const uint8_t *t = tab + r * tpitch + kt * SPS + kq;
        return FP4 ? (uint32_t)t[0] | ((uint32_t)t[4] << 8) : (uint32_t)t[0];
    };

    // every call issues the same loads; a dead stage (kt < 0) reads zeros
    auto load_stage = [&](int kt, Stage &s) MXG_INLINE {
        const bool live = kt >= 0;
        s.kt = kt;
        const int k0 = (live ? kt : 0) * SB;
        // e2m3: both pieces belong to block g, which lies in the row or not
        const bool lo_in = live && k0 + kq * LO < K, hi_in = FP6 ? lo_in : live && k0 + kq * LO + HI < K;
        const int kb0 = (live ? kt : 0) * SPS;
        // scale bytes: fp8, block g (in range when its 32 codes are);
        // e2m1, blocks g and 4 + g (each the block of one chunk).  The vector
        // form needs only the stage to exist (its rows hold whole stages).
        const bool s0_in = SVEC ? live : (FP4 || FP6 ? lo_in : live && k0 + kq * 32 < K);
        const bool s1_in = hi_in;
        // two pieces per row: 16 + 16 bytes (e2m3: 16 + 8, operand dwords 6, 7 zero)
        auto piece = [&](rsrc_t r, uint32_t off) MXG_INLINE {
            const v4i lo = load16(r, lo_in ? off + k0 : kOob);
            if constexpr (FP6) {
                const v2i hi = __builtin_bit_cast(
                    v2i, __builtin_amdgcn_raw_buffer_load_b64(r, hi_in ? off + k0 + HI : kOob, 0, 0));
                return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], 0, 0};
            } else {
                const v4i hi = load16(r, hi_in ? off + k0 + HI : kOob);
                return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
        };
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) {
            s.b[j] = piece(rB, boff[j]);
            if constexpr (!STAB) s.sb[j] = scales_of(rBs, bsrow[j], kb0, s0_in, s1_in);
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            s.a[i] = piece(rA, aoff[i]);
            if constexpr (!STAB) s.sa[i] = scales_of(rAs, asrow[i], kb0, s0_in, s1_in);
        }
    };

    v4f acc[MT][SUB_N];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) acc[i][j] = v4f{};

    auto multiply = [&](const Stage &cur_) MXG_INLINE {
        Stage cur = cur_;
        if constexpr (STAB) {
#pragma unroll
            for (int j = 0; j < SUB_N; ++j) cur.sb[j] = table_scales(MAX_M + 16 * j + r16, cur.kt);
#pragma unroll
            for (int i = 0; i < MT; ++i) cur.sa[i] = table_scales(16 * i + r16, cur.kt);
        }
        if constexpr (FP4) {
            // step 0: the low chunks (blocks g, scale byte 0); step 1: the high
            // chunks (blocks 4 + g, scale byte 1)
#pragma unroll
            for (int j = 0; j < SUB_N; ++j)
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const v8i b0 = {cur.b[j][0], cur.b[j][1], cur.b[j][2], cur.b[j][3], 0, 0, 0, 0};
                    const v8i a0 = {cur.a[i][0], cur.a[i][1], cur.a[i][2], cur.a[i][3], 0, 0, 0, 0};
                    acc[i][j] = mfma16<FB, FA, 0>(b0, a0, acc[i][j], cur.sb[j], cur.sa[i]);
                }
#pragma unroll
            for (int j = 0; j < SUB_N; ++j)
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const v8i b1 = {cur.b[j][4], cur.b[j][5], cur.b[j][6], cur.b[j][7], 0, 0, 0, 0};
                    const v8i a1 = {cur.a[i][4], cur.a[i][5], cur.a[i][6], cur.a[i][7], 0, 0, 0, 0};
                    acc[i][j] = mfma16<FB, FA, 1>(b1, a1, acc[i][j], cur.sb[j], cur.sa[i]);
                }
        } else {
#pragma unroll
            for (int j = 0; j < SUB_N; ++j)
#pragma unroll
                for (int i = 0; i < MT; ++i)
                    acc[i][j] = mfma16<FB, FA>(cur.b[j], cur.a[i], acc[i][j], cur.sb[j], cur.sa[i]);
        }
    };

    const int s0 = tile % nk;  // this workgroup's first stage, counted from kbeg
    auto stage_of = [&](int t) MXG_INLINE { const int s = t + s0; return kbeg + (s < nk ? s : s - nk); };
    // wave w runs its stages t = w, w + WAVES, ...; the i-th of them lives in
    // ring slot i % RING (static indices only: the ring stays in registers)
    // Loads are issued unconditionally (dead stages read zeros) so that the
    // compiler's wait counting stays exact across the ring.
    auto kt_of = [&](int t) MXG_INLINE { return t < nk ? stage_of(t) : -1; };
    Stage ring[RING];
    static_for<RING - 1>([&](auto P) MXG_INLINE {
        load_stage(kt_of(wave + decltype(P)::value * WAVES), ring[decltype(P)::value]);
    });
    for (int t0 = wave; t0 < nk; t0 += RING * WAVES) {
        static_for<RING>([&](auto P) MXG_INLINE {
            constexpr int pp = decltype(P)::value;
            const int t = t0 + pp * WAVES;
            // loads into the slot multiplied last, RING - 1 stages ahead
            load_stage(kt_of(t + (RING - 1) * WAVES), ring[(pp + RING - 1) % RING]);
            if (t < nk) multiply(ring[pp]);
        });
    }

    // acc[i][j] register r of lane l: m = 16 i + l % 16, n = 16 j + 4 (l / 16) + r.
    if constexpr (STAB) __syncthreads();  // every wave is done with the scale table
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < SUB_N; ++j)
            *reinterpret_cast<v4f *>(&red[wave][16 * i + r16][16 * j + 4 * kq]) = acc[i][j];
    __syncthreads();

    const rsrc_t rC = make_rsrc((uint8_t *)p.C, (uint32_t)M * N * (p.out_bf16 ? 2 : 4));
    constexpr int Q = MAX_M * BN / 4;  // float4 groups in the tile
    // bf16 output with N % 8 == 0: rows of 8 columns, one 16-byte store each
    const bool wide_bf16 = p.out_bf16 && p.c_vec == 2;
    static_assert(BN % 8 == 0, "whole 8-column groups");
    if constexpr (SPLIT) {
        // Every split leaves its fp32 partial tile in the workspace
        // ([split][tile][64 rows][112 columns]); a counter per tile counts the
        // splits that are done, and the workgroup that completes the count
        // adds the partials in split order 0, 1, ..., so the result does not
        // depend on which split finishes last, and resets the counter for the
        // next call.  Partials are written and read with device-scope
        // coherent (sc1) buffer accesses, which bypass the per-XCD L2s'
        // non-coherent copies: the wait for the stores to complete, then the
        // barrier, is the whole release (no L2 writeback).
        constexpr int TILE_F = MAX_M * BN;
        constexpr int SC1 = 16;  // cache-policy bit of the buffer intrinsics
        __shared__ uint32_t last;
        const rsrc_t rW = make_rsrc(p.ws, (uint32_t)(p.splits * p.tiles_n * TILE_F * 4));
        const uint32_t tile_off = (uint32_t)(tile * TILE_F) * 4;
        const uint32_t split_pitch = (uint32_t)(p.tiles_n * TILE_F) * 4;
        for (int q = tid; q < Q; q += THREADS) {
            const int m = q / (BN / 4), nl = (q % (BN / 4)) * 4;
            if (m >= M) continue;
            v4f v = *reinterpret_cast<const v4f *>(&red[0][m][nl]);
#pragma unroll
            for (int w = 1; w < WAVES; ++w) v += *reinterpret_cast<const v4f *>(&red[w][m][nl]);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v), rW,
                                                   tile_off + sp * split_pitch + (uint32_t)(m * BN + nl) * 4,
                                                   0, SC1);
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this thread's stores are complete
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __syncthreads();                     // ... and so are every thread's
        if (tid == 0) {
            uint32_t *cnt = p.cnt + tile;
            const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = old == (uint32_t)(p.splits - 1);
            if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!last) return;
        // up to QB splits' partials in flight at once (a split past the last
        // reads zeros through the range check and is not added)
        constexpr int QB = 8;
        auto split_sum = [&](uint32_t off) MXG_INLINE {
            v4f v = {};
            for (int q0 = 0; q0 < p.splits; q0 += QB) {
                v4f part[QB];
#pragma unroll
                for (int qq = 0; qq < QB; ++qq)
                    part[qq] = __builtin_bit_cast(
                        v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                 rW, q0 + qq < p.splits ? off + (q0 + qq) * split_pitch : kOob, 0, SC1));
#pragma unroll
                for (int qq = 0; qq < QB; ++qq) {
                    if (q0 + qq == 0)
                        v = part[qq];
                    else if (q0 + qq < p.splits)
                        v += part[qq];
                }
            }
            return v;
        };
        if (wide_bf16) {
            for (int q = tid; q < Q / 2; q += THREADS) {
                const int m = q / (BN / 8), nl = (q % (BN / 8)) * 8;
                if (m >= M) continue;
                const uint32_t off = tile_off + (uint32_t)(m * BN + nl) * 4;
                const v4f lo = split_sum(off), hi = split_sum(off + 16);
                const int n = n0 + nl;
                store_bf16x8(rC, (uint32_t)m * N + n, n, N, lo, hi, p.use_acc);
            }
            return;
        }
        for (int q = tid; q < Q; q += THREADS) {
            const int m = q / (BN / 4), nl = (q % (BN / 4)) * 4;
            if (m >= M) continue;
            const v4f v = split_sum(tile_off + (uint32_t)(m * BN + nl) * 4);
            const int n = n0 + nl;
            store_c4(rC, (uint32_t)m * N + n, n, N, v, p.out_bf16, p.use_acc, p.c_vec);
        }
        return;
    }
    auto tile_sum = [&](int m, int nl) MXG_INLINE {
        v4f v = *reinterpret_cast<const v4f *>(&red[0][m][nl]);
#pragma unroll
        for (int w = 1; w < WAVES; ++w) v += *reinterpret_cast<const v4f *>(&red[w][m][nl]);
        return v;
    };
    if (wide_bf16) {
        for (int q = tid; q < Q / 2; q += THREADS) {
            const int m = q / (BN / 8), nl = (q % (BN / 8)) * 8;
            if (m >= M) continue;
            const int n = n0 + nl;
            store_bf16x8(rC, (uint32_t)m * N + n, n, N, tile_sum(m, nl), tile_sum(m, nl + 4), p.use_acc);
        }
        return;
    }
    for (int q = tid; q < Q; q += THREADS) {
        const int m = q / (BN / 4), nl = (q % (BN / 4)) * 4;
        if (m >= M) continue;
        const int n = n0 + nl;
        store_c4(rC, (uint32_t)m * N + n, n, N, tile_sum(m, nl), p.out_bf16, p.use_acc, p.c_vec);
    }
}

} // namespace skinny
} // namespace mxg
