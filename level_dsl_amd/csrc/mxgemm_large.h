// mxgemm_large.h -- 256x256-tile MX-FP8 GEMM kernel for gfx950 (MFMA-bound shapes).
//
// One workgroup of four waves (one per SIMD) computes a 256 (M) x 256 (N)
// tile of C; each wave owns a 128 x 128 quarter held as 4 x 4 accumulators
// of a 32x32 MFMA (256 fp32 per lane, in the accumulator registers), which
// leaves the 256 ordinary VGPRs for a software pipeline.
//
// Data flow per stage of BK = 128 bytes of K (two LDS stages of 2 x 32 KiB):
//   * global -> LDS: 16-byte raw buffer loads that write LDS directly
//     (buffer_load_dwordx4 ... lds); one wave instruction fills one
//     contiguous 1 KiB LDS segment (8 tile rows), lane i writing bytes
//     16i..16i+15; the swizzle is applied by choosing which global chunk each
//     lane fetches.  K and row tails read as zero through the descriptor's
//     range check.  Stage kt+2's A tile is loaded right after the barrier
//     that retires stage kt's buffer and (exact mode) its B tile one block
//     later, about one stage before they are needed.  The scaled-MFMA
//     modes, whose stages are half as long, issue both tiles right after the
//     barrier (measured 5-8% faster there; the exact mode measured better
//     with the split, which keeps a 64-load burst from stalling its longer
//     MFMA stream).
//   * scales: with row-major scales and K % 512 == 0 they come in 16-byte
//     windows per row (four stages' worth; two for e2m1), prefetched a window
//     ahead: the exact mode loads each lane's windows of its 8 fragment rows
//     into registers (one dwordx4 per row); the scaled-MFMA modes load the
//     windows of all 512 tile rows into LDS once per workgroup (one coalesced
//     16-byte direct-to-LDS load per row) and read each stage's dwords from
//     there.  Otherwise (and with preshuffled scales, where a wave's dword
//     load is one 128-byte line) one dword (or four bytes) per row per stage,
//     prefetched one stage ahead.
//   * blocks: a stage is split into blocks (exact mode: the four 32-byte K
//     blocks; native mode: the two 64-byte MFMA K steps).  While the MFMAs of
//     block g run, the fragments of block g+1 are read from LDS (ds_read_b128)
//     and, in exact mode, decoded to bf16 -- the intra-wave interleave of
//     memory and MFMA work described for gfx950 on the TLX warp-
//     specialization page ("Warp pipeline", intra-wave scheduling).  The
//     stage barrier sits where the last fragment of a stage has been read,
//     so the next stage's first block is read while the last block's MFMAs
//     still run.
//   * the multiply:
//       exact mode (default): lane half h of a row takes 16-byte chunk
//       2p + h of K block p, decodes the 16 codes with the row's block-p
//       scale into 16 bf16 (v_cvt_scalef32_pk_bf16_fp8/bf8) and feeds two
//       32x32x16 bf16 MFMAs;
//       native mode: lane half h takes chunks 4kk+h and 4kk+2+h for the
//       kk-th 64-byte step and one v_mfma_scale_f32_32x32x64_f8f6f4 consumes
//       them with the scale bytes selected by op_sel;
//     MFMAs are issued K-major, then N, then M, so consecutive MFMAs update
//     independent accumulators (the issue order of amd_scheduled_mfma on the
//     TLX async-compute page, "Explicit MFMA scheduling").
// LDS rows are 128 bytes; 16-byte chunk c of row r sits at chunk position
// c ^ swz(r), swz(r) = (r & 7) ^ ((r >> 3) & 1), so the lanes of one
// ds_read_b128 pass (consecutive rows, same chunk) hit distinct banks.
//
// Roles in the MFMA: the B tile supplies the instruction's rows and the A
// tile its columns, so each lane's accumulator registers hold 4 consecutive
// n of one m -- one 16-byte fp32 (or 8-byte bf16) store per group (the
// "transposed" MFMA layout that the TLX global-memory page pairs with
// vectorised buffer_store).
#pragma once

#include "mxgemm_common.h"

#include <type_traits>

namespace mxg {
namespace large {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int WAVES = 4, THREADS = 64 * WAVES;
constexpr int WAVE_M = 128, WAVE_N = 128;     // per-wave tile
constexpr int SUB_M = WAVE_M / 32, SUB_N = WAVE_N / 32;
constexpr int TILE_BYTES = BM * BK;           // one operand, one stage (32 KiB)
constexpr int SEG = 1024;                     // bytes one wave load instruction fills
constexpr int SEGS_PER_WAVE = TILE_BYTES / SEG / WAVES;  // 8 per operand per stage
// stages per 16-byte scale window: 128-byte stages of e2m1 (256 codes) hold
// 8 scale blocks, all other stages 4
__host__ __device__ constexpr int window_stages(bool fp4) { return fp4 ? 2 : 4; }

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Workgroup -> tile.  Workgroups are dealt round-robin to the 8 XCDs, so the
// ids that land on one XCD are made consecutive in tile order; tiles are then
// walked in groups of 8 tile-rows so that the workgroups resident on one XCD
// share A rows and B columns in that XCD's L2.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int nb = tiles_m * tiles_n;
    const int q = nb >> 3, r = nb & 7, x = bid & 7, i = bid >> 3;
    const int t = x * q + (x < r ? x : r) + i;
    constexpr int G = 8;
    const int per_group = G * tiles_n;
    const int g = t / per_group;
    const int first_m = g * G;
    const int gs = (tiles_m - first_m) < G ? (tiles_m - first_m) : G;
    const int w = t - g * per_group;
    tm = first_m + w % gs;
    tn = w / gs;
}

// Fragments of one block: exact mode keeps 16 bf16 (two MFMA operands) per
// fragment, native mode the 32 raw codes.
template <bool NATIVE>
struct Frags;
template <>
struct Frags<false> {
    v8bf a[SUB_M][2], b[SUB_N][2];
};
template <>
struct Frags<true> {
    v8i a[SUB_M], b[SUB_N];
};
template <bool NATIVE>
struct Raw;
template <>
struct Raw<false> {
    v4i a[SUB_M], b[SUB_N];
};
template <>
struct Raw<true> {};  // native fragments are read straight into the operand registers

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int SG_VALU = 0x002, SG_SALU = 0x004, SG_MFMA = 0x008, SG_VMEM_RD = 0x020,
              SG_DS_RD = 0x100;

// ---- epilogue ---------------------------------------------------------------
// Store a wave's 128 x 128 accumulators acc (fp32 or bf16 C, optionally
// accumulating into it).  Split K (p.splits > 1): the partial goes to the
// workspace and the last split to arrive adds them up.  slow: the wave
// recomputes its outputs with slow_tile(i, j) instead (exact mode's
// fallback for scale bytes outside the decode window).
template <bool SPLIT, class SlowTile>
__device__ __forceinline__ void store_tile(const GemmArgs &p, v16f (&acc)[SUB_M][SUB_N], int tile, int sp,
                                           int ntiles, int m0, int n0, int rows_a, int wm, int wn,
                                           int lrow, int khalf, bool slow, SlowTile &&slow_tile)
{
    // acc[i][j] register r of lane l: m = 32 i + (l % 32),
    // n = 32 j + 8 (r / 4) + 4 (l / 32) + (r % 4), relative to the wave tile.
    // Group x = 4 (SUB_N i + j) + g of a lane is registers 4g..4g+3 of acc[i][j].
    const int esz = p.out_bf16 ? 2 : 4;
    const rsrc_t rC = make_rsrc((uint8_t *)p.C + ((size_t)m0 * p.N) * esz,
                                (uint32_t)rows_a * p.N * esz);
    const int N = p.N;
    auto store_group = [&](int i, int j, int g, v4f v) MXG_INLINE {
        const int m = wm * WAVE_M + i * 32 + lrow;                      // tile-local row
        const int n = n0 + wn * WAVE_N + j * 32 + 8 * g + 4 * khalf;  // global column
        store_c4(rC, (uint32_t)m * N + n, n, N, v, p.out_bf16, p.use_acc, p.c_vec);
    };
    constexpr int GROUPS = SUB_M * SUB_N * 4;  // 16-byte groups per lane
    // bf16 output with N % 8 == 0: groups g (even) and g + 1 of a sub-tile
    // are stored as 16-byte rows of 8 bf16.  Lane l holds columns 8g + 4 kh
    // .. + 3 of both groups (kh = l / 32) and the lane l ^ 32 the other four
    // of each, so the two lane halves swap one group: the lower half keeps
    // group g and takes its partner's half of it, the upper half group g + 1.
    const bool wide_bf16 = p.out_bf16 && p.c_vec == 2;
    auto store_pair = [&](int i, int j, int g, v4f x, v4f y) MXG_INLINE {  // groups g, g + 1
        const int kh = (int)(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) >> 5);
        const int lr = (int)(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) & 31);
        // v_permlane32_swap: the upper lane half of x trades places with
        // the lower half of y, so the lower half ends with (its x, the upper
        // lane's x) and the upper half with (the lower lane's y, its y)
        v4f lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // (the elements are copied out first: a bit cast of x[e] itself
            // compiled to a read of element 0 for every e)
            const float xe = x[e], ye = y[e];
            const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, xe),
                                                            __builtin_bit_cast(uint32_t, ye), false, false);
            lo[e] = __builtin_bit_cast(float, (uint32_t)r[0]);
            hi[e] = __builtin_bit_cast(float, (uint32_t)r[1]);
        }
        const int m = wm * WAVE_M + i * 32 + lr;                       // tile-local row
        const int n = n0 + wn * WAVE_N + j * 32 + 8 * (g + kh);      // global column
        store_bf16x8(rC, (uint32_t)m * N + n, n, N, lo, hi, p.use_acc);
    };

    if constexpr (SPLIT) {
        // Split K (p.splits > 1): every split stores its wave's fp32 partial
        // (the 64 groups of each lane, 1 KiB per store instruction) with
        // device-coherent (sc1) buffer stores; per (tile, wave) an arrival
        // counter counts the splits that are done, and the wave that
        // completes the count adds all partials in split order 0, 1, ...
        // (deterministic), PER groups at a time, writes them to C and resets
        // the counter.  The sc1 accesses bypass the per-XCD L2s'
        // non-coherent copies, so waiting for the stores to complete is the
        // whole release (no L2 writeback).
        constexpr int SC1 = 16;
        constexpr uint32_t WAVE_PART = GROUPS * 64 * 16;  // one wave's partial, bytes
        // the lane index again (mbcnt), so that nothing lane-dependent has to
        // stay live across the main loop for this path
        const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
        const rsrc_t rW = make_rsrc(p.ws, (uint32_t)p.splits * ntiles * WAVES * WAVE_PART);
        const uint32_t lane_off = (uint32_t)(tile * WAVES + wave) * WAVE_PART + lane * 16;
        const uint32_t split_pitch = (uint32_t)ntiles * WAVES * WAVE_PART;
        // group x = 4 (SUB_N i + j) + g of the partial
        auto put = [&](int i, int j, const v16f &v) MXG_INLINE {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const v4f q = {v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(v4i, q), rW,
                    lane_off + sp * split_pitch + (4 * (SUB_N * i + j) + g) * 1024, 0, SC1);
            }
        };
        if (slow) {
            for (int t = 0; t < SUB_M * SUB_N; ++t) put(t / SUB_N, t % SUB_N, slow_tile(t / SUB_N, t % SUB_N));
        } else {
            static_for<SUB_M * SUB_N>([&](auto T) MXG_INLINE {
                constexpr int t = decltype(T)::value;
                put(t / SUB_N, t % SUB_N, acc[t / SUB_N][t % SUB_N]);
            });
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the partial has reached the coherent level
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        uint32_t *cnt = p.cnt + tile * WAVES + wave;
        uint32_t old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = (uint32_t)__shfl((int)old, 0, 64);
        if (old != (uint32_t)(p.splits - 1)) return;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        constexpr int PER = 8;  // groups summed at a time (loads in flight per split)
        static_for<GROUPS / PER>([&](auto Bt) MXG_INLINE {
            constexpr int b = decltype(Bt)::value;
            v4f sum[PER];
            for (int q = 0; q < p.splits; ++q) {
                v4f part[PER];
                static_for<PER>([&](auto Y) MXG_INLINE {
                    constexpr int y = decltype(Y)::value;
                    part[y] = __builtin_bit_cast(
                        v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                 rW, lane_off + q * split_pitch + (b * PER + y) * 1024, 0, SC1));
                });
#pragma unroll
                for (int y = 0; y < PER; ++y) sum[y] = q == 0 ? part[y] : sum[y] + part[y];
            }
            if (wide_bf16) {
                static_for<PER / 2>([&](auto Y) MXG_INLINE {
                    constexpr int y = 2 * decltype(Y)::value, x = b * PER + y;
                    store_pair(x / (SUB_N * 4), (x / 4) % SUB_N, x % 4, sum[y], sum[y + 1]);
                });
            } else {
                static_for<PER>([&](auto Y) MXG_INLINE {
                    constexpr int x = b * PER + decltype(Y)::value;
                    store_group(x / (SUB_N * 4), (x / 4) % SUB_N, x % 4, sum[decltype(Y)::value]);
                });
            }
        });

    } else {
        auto put = [&](int i, int j, const v16f &v) MXG_INLINE {
            if (wide_bf16) {
#pragma unroll
                for (int g = 0; g < 4; g += 2)
                    store_pair(i, j, g, v4f{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]},
                               v4f{v[4 * g + 4], v[4 * g + 5], v[4 * g + 6], v[4 * g + 7]});
            } else {
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    store_group(i, j, g, v4f{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]});
            }
        };
        if (slow) {
            for (int t = 0; t < SUB_M * SUB_N; ++t) put(t / SUB_N, t % SUB_N, slow_tile(t / SUB_N, t % SUB_N));
        } else {
            static_for<SUB_M * SUB_N>([&](auto T) MXG_INLINE {
                constexpr int t = decltype(T)::value;
                put(t / SUB_N, t % SUB_N, acc[t / SUB_N][t % SUB_N]);
            });
        }
    }
}

template <int FA, int FB, bool NATIVE, bool SCALE16, bool SPLIT>
__global__ __launch_bounds__(THREADS) void kernel(GemmArgs p)
{
    // e2m1 operands (format 4, two codes per byte along K): the scaled MFMA
    // sums e2m1 products exactly (every product of a 32-element block fits
    // its 8-product window), so they always run on it, with 8 scale bytes
    // per row and 128-byte stage and per-stage scale loads
    constexpr bool FP4 = FA == 4;
    static_assert(FP4 == (FB == 4), "e2m1 pairs only with e2m1");
    static_assert(!FP4 || NATIVE, "e2m1 runs on the scaled MFMA");
    // e2m3 operands (format 2, four codes per three bytes): every product of
    // a 32-element block fits the scaled MFMA's 8-product window as well, so
    // they too run on it.  A stage is 128 codes, 96 bytes of a row: its four
    // 24-byte blocks sit in LDS padded to 32 bytes (LDS chunks 2b and 2b + 1
    // hold bytes 24b .. 24b + 15 and 24b + 16 .. 24b + 31 of the stage, the
    // last 8 unused), so that the lane half taking block b reads one whole
    // chunk and the first half of the next.  Scales and MFMA steps are laid
    // out as in the fp8 native mode (two 64-code steps per stage).
    constexpr bool FP6 = FA == 2;
    static_assert(FP6 == (FB == 2), "e2m3 pairs only with e2m3");
    static_assert(!FP6 || NATIVE, "e2m3 runs on the scaled MFMA");
    constexpr int SB = FP6 ? 96 : BK;                     // bytes of a row per stage
    constexpr int SPS = FP4 ? 8 : 4;                     // scale bytes per row and stage
    constexpr int BLOCKS = NATIVE && !FP4 ? 2 : 4;        // blocks per stage
    constexpr int MF = NATIVE ? SUB_M * SUB_N : 2 * SUB_M * SUB_N;  // MFMAs per block
    // SCALE16 (row-major scales, K % 512 == 0): the scale bytes of a row come
    // in 16-byte windows of WIN stages.  Exact mode holds a lane's windows in
    // registers (SREG).  The scaled-MFMA modes stage them through LDS (SLDS):
    // the workgroup loads the windows of its 512 tile rows once, one
    // coalesced 16-byte direct-to-LDS load per row, a window ahead, and each
    // stage reads its dwords from there.  (Per-row dword loads from global
    // memory cost each wave instruction 32 cache lines and were what held
    // these modes back.)
    constexpr bool SREG = SCALE16 && !NATIVE, SLDS = SCALE16 && NATIVE;
    constexpr int WIN = SCALE16 ? window_stages(FP4) : 1;  // stages per window
    static_assert(!SCALE16 || WIN * SPS == 16, "a window is 16 scale bytes");
    static_assert(WIN % 2 == 0 || !SCALE16, "stage parity follows the window position");
    // Main loops that run two stages per iteration (compile-time buffer
    // parity), where they fit in the registers: e2m3 and the fp8 scaled-MFMA
    // loop with per-stage scale loads spill in them and keep one stage per
    // iteration.
    constexpr bool PAIR = !SREG && !FP6 && (SLDS || FP4 || !NATIVE);
    // The two stage buffers are separate LDS objects ([A/B] each): a read of
    // one can then be told apart from direct-to-LDS loads into the other, and
    // the compiler does not drain those loads before it.
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[2][TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[2][TILE_BYTES];
    auto lbuf = [&](int st, int op) MXG_INLINE -> uint8_t * { return st ? lds1[op] : lds0[op]; };
    // SLDS: [window buffer][tile row (A rows 0..255, then B rows)][16 bytes]
    constexpr int SWIN_BYTES = (BM + BN) * 16;
    __shared__ __attribute__((aligned(16))) uint8_t slds[SLDS ? 2 * SWIN_BYTES : 16];

    // workgroup -> (tile, K split); split sp runs stages [ks0, ks0 + nk) of
    // the nk_all stages (whole scale windows when SCALE16)
    const int ntiles = p.tiles_m * p.tiles_n;
    const int tile = SPLIT ? (int)(blockIdx.x % (unsigned)ntiles) : (int)blockIdx.x;
    const int sp = SPLIT ? (int)(blockIdx.x / (unsigned)ntiles) : 0;
    int tm, tn;
    tile_of(tile, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int rows_a = min(BM, p.M - m0), rows_b = min(BN, p.N - n0);
    const int K = p.K, KB = p.KB;

    const rsrc_t rA = make_rsrc(p.A + (size_t)m0 * K, (uint32_t)rows_a * K);
    const rsrc_t rB = make_rsrc(p.B + (size_t)n0 * K, (uint32_t)rows_b * K);
    // tiles start at multiples of 32 rows: the same base in both scale layouts
    const int ps = p.scale_ps;
    const rsrc_t rAs = make_rsrc(p.As + (size_t)m0 * KB, scale_span(rows_a, KB, ps));
    const rsrc_t rBs = make_rsrc(p.Bs + (size_t)n0 * KB, scale_span(rows_b, KB, ps));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int lrow = lane & 31, khalf = lane >> 5;
    const int nk_all = (K + SB - 1) / SB;
    constexpr int SPLIT_UNIT = WIN;                   // stages a split boundary is a multiple of
    const int nu_all = nk_all / SPLIT_UNIT;           // SCALE16 needs K % 512 == 0: no remainder
    const int ks0 = SPLIT ? (int)((int64_t)sp * nu_all / p.splits) * SPLIT_UNIT : 0;
    const int nk = SPLIT ? (int)((int64_t)(sp + 1) * nu_all / p.splits) * SPLIT_UNIT - ks0 : nk_all;

    // ---- global -> LDS, one stage ---------------------------------------
    // A stage's two operands are loaded at different points of the K loop
    // (A right after the barrier that frees the buffer, B one block later),
    // so that a wave never issues all of its loads in one burst: a burst of
    // 64 loads per CU backs up the address path and stalls the in-order MFMA
    // stream behind it.
    // segment s = SEGS_PER_WAVE*wave + j holds tile rows 8s..8s+7; lane i
    // writes row 8s + i/8 at chunk position i%8, i.e. global chunk
    // (i%8) ^ swz(row) = (i%8) ^ (i/8) ^ (s & 1).  Stages past the end of K
    // read as zero (every offset is out of range), so the call needs no guard.
    const int gc0 = (lane & 7) ^ (lane >> 3);  // chunk for even segments; odd: gc0 ^ 1
    const uint32_t grow = (uint32_t)(8 * SEGS_PER_WAVE * wave + (lane >> 3)) * K;
    // operand OP (0: A, 1: B) of local stage kt into LDS stage st
    auto gload = [&](int st, int kt, auto OP) MXG_INLINE {
        constexpr int op = decltype(OP)::value;
        const int k0 = (kt + ks0) * SB;
#pragma unroll
        for (int j = 0; j < SEGS_PER_WAVE; ++j) {
            const int s = SEGS_PER_WAVE * wave + j;
            const int c = gc0 ^ (j & 1);
            // byte of the stage that LDS chunk c starts with, and whether its
            // data exist (e2m3: the chunk's 24-byte block lies in the row)
            const int g = FP6 ? 24 * (c >> 1) + 16 * (c & 1) : 16 * c;
            const bool in = FP6 ? k0 + 24 * (c >> 1) < K : k0 + g < K;
            const uint32_t off = in ? grow + (uint32_t)(8 * j) * K + g + k0 : kOob;
            load16_lds(op == 0 ? rA : rB, lbuf(st, op) + s * SEG, off);
        }
    };

    // ---- scales ---------------------------------------------------------
    // Fragment rows of this lane: A rows wm*128 + 32i + lrow, B rows
    // wn*128 + 32j + lrow.  SREG: 16 bytes (4 stages) per row and load;
    // SLDS: a stage's dwords from the LDS window; otherwise one dword (or
    // four bytes) per row and stage.  SCALE16 reads
    // row-major scales only; preshuffled scales take the per-stage dword
    // loads, each one 128-byte line for the wave's 32 rows.
    const uint32_t sra = (uint32_t)(wm * WAVE_M + lrow), srb = (uint32_t)(wn * WAVE_N + lrow);
    auto srow_a = [&](int i) MXG_INLINE { return sra + 32 * i; };
    auto srow_b = [&](int j) MXG_INLINE { return srb + 32 * j; };
    auto scale16 = [&](int kt, v4i *xa, v4i *xb) MXG_INLINE {  // window starting at local stage kt
        const int kb0 = (ks0 + kt) * (BK / 32);
        const bool in = kb0 < KB;
#pragma unroll
        for (int i = 0; i < SUB_M; ++i) xa[i] = load16(rAs, in ? srow_a(i) * KB + kb0 : kOob);
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) xb[j] = load16(rBs, in ? srow_b(j) * KB + kb0 : kOob);
    };
    // local stage kt: its first 4 scale bytes per row into xa/xb, and for
    // e2m1 the next 4 into xa2/xb2 (a dword past the row's end reads zero)
    auto scale4 = [&](int kt, uint32_t *xa, uint32_t *xb, uint32_t *xa2, uint32_t *xb2) MXG_INLINE {
        const int kb0 = (ks0 + kt) * SPS;
#pragma unroll
        for (int i = 0; i < SUB_M; ++i) xa[i] = load_scale4(rAs, srow_a(i), KB, kb0, p.scale_dword, ps);
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) xb[j] = load_scale4(rBs, srow_b(j), KB, kb0, p.scale_dword, ps);
        if constexpr (FP4) {
            const int kb1 = kb0 + 4;
            const bool in = kb1 < KB;
#pragma unroll
            for (int i = 0; i < SUB_M; ++i)
                xa2[i] = in ? load_scale4(rAs, sra + 32 * i, KB, kb1, p.scale_dword, ps) : 0u;
#pragma unroll
            for (int j = 0; j < SUB_N; ++j)
                xb2[j] = in ? load_scale4(rBs, srb + 32 * j, KB, kb1, p.scale_dword, ps) : 0u;
        }
    };
    // SLDS: the window starting at local stage kt into LDS buffer (kt / WIN) & 1.
    // Wave w loads tile rows 128 w .. 128 w + 127 (waves 0, 1: A; 2, 3: B), 64
    // rows per instruction; rows past the tile and windows past K read zero
    // or are never used.
    auto swin = [&](int kt) MXG_INLINE {
        if constexpr (SLDS) {
            const int kb0 = (ks0 + kt) * SPS;
            const bool in = kb0 < KB;
            const bool isa = wave < 2;
            const rsrc_t rs = isa ? rAs : rBs;
            uint8_t *dst = slds + ((kt / WIN) & 1) * SWIN_BYTES;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r0 = 128 * wave + 64 * h;  // first tile row of the instruction
                const uint32_t row = (uint32_t)((isa ? r0 : r0 - BM) + lane);
                load16_lds(rs, dst + r0 * 16, in ? row * KB + kb0 : kOob);
            }
        }
    };
    // SLDS: local stage kt's scale dwords from its window (as scale4)
    // Each address is the base plus a stage offset plus a lane offset (plus
    // a constant), both kept whole: a longer chain of address steps loses
    // the compiler's record of which LDS object is read, and with it the
    // knowledge that the direct-to-LDS loads in flight write other objects
    // (it would wait for them all before the read).
    const uint32_t soff_a = opaque_v(sra * 16), soff_b = opaque_v((BM + srb) * 16);
    auto scale_lds = [&](int kt, uint32_t *xa, uint32_t *xb, uint32_t *xa2, uint32_t *xb2) MXG_INLINE {
        if constexpr (SLDS) {
            const uint8_t *w = slds + opaque_s((uint32_t)(((kt / WIN) & 1) * SWIN_BYTES + (kt % WIN) * SPS));
#pragma unroll
            for (int i = 0; i < SUB_M; ++i) {
                const uint8_t *q = w + soff_a + i * 32 * 16;
                if constexpr (FP4) {
                    const v2i v = *reinterpret_cast<const v2i *>(q);
                    xa[i] = (uint32_t)v[0];
                    xa2[i] = (uint32_t)v[1];
                } else {
                    xa[i] = *reinterpret_cast<const uint32_t *>(q);
                }
            }
#pragma unroll
            for (int j = 0; j < SUB_N; ++j) {
                const uint8_t *q = w + soff_b + j * 32 * 16;
                if constexpr (FP4) {
                    const v2i v = *reinterpret_cast<const v2i *>(q);
                    xb[j] = (uint32_t)v[0];
                    xb2[j] = (uint32_t)v[1];
                } else {
                    xb[j] = *reinterpret_cast<const uint32_t *>(q);
                }
            }
        }
    };
    // Exact mode: every scale byte the fast loop decodes with passes
    // through this check; a byte outside its format's window (where the
    // bf16 decode would round, overflow or misread byte 0 / 255) sends the
    // wave to the fallback after the loop.  The two lane halves hold the same
    // rows' scales, so the lower half checks the A rows and the upper half
    // the B rows.  Rows past the tile's end and bytes past the end of K are
    // not data: they read as zero and are replaced by an in-window byte.
    ScaleRange rg;
    rg.init();
    const bool chk_b = khalf != 0;
    const v2u16 chk_lo2 = chk_b ? window_lo2<FB == 1 ? 1 : 0>() : window_lo2<FA == 1 ? 1 : 0>();
    bool live[SUB_M];
    static_assert(SUB_M == SUB_N, "one check per fragment row of A or B");
#pragma unroll
    for (int i = 0; i < SUB_M; ++i) live[i] = chk_b ? (int)srow_b(i) < rows_b : (int)srow_a(i) < rows_a;
    auto track4 = [&](int kt, const uint32_t *xa, const uint32_t *xb) MXG_INLINE {  // local stage kt
        if constexpr (!NATIVE) {
            const int valid = KB - (ks0 + kt) * (BK / 32);
#pragma unroll
            for (int i = 0; i < SUB_M; ++i) {
                uint32_t d = chk_b ? xb[i] : xa[i];
                if constexpr (!SREG) d = mask_scale_tail(d, valid);  // SREG: KB % 16 == 0
                rg.add(live[i] ? d : 0x7f7f7f7fu, chk_lo2);
            }
        }
    };

    // native mode: the upper lane half supplies the odd K blocks (fp8: of
    // each 64-element MFMA step; e2m1: each lane half holds one block)
    // (a shift by 8 khalf, not a branch on khalf: a lane-divergent branch
    // would split the MFMA block's scheduling region, and the interleave of
    // LDS reads with MFMAs would be lost)
    auto native_shift = [&](uint32_t *xa, uint32_t *xb) MXG_INLINE {
        if constexpr (NATIVE) {
            const uint32_t sh = 8u * (uint32_t)khalf;
#pragma unroll
            for (int i = 0; i < SUB_M; ++i) xa[i] >>= sh;
#pragma unroll
            for (int j = 0; j < SUB_N; ++j) xb[j] >>= sh;
        }
    };

    // ---- fragments --------------------------------------------------------
    const int sw = swz(lrow);
    const uint32_t fa_off = (wm * WAVE_M + lrow) * BK, fb_off = (wn * WAVE_N + lrow) * BK;
    // read block `blk` of LDS stage `st` (exact: into raw; native: straight
    // into the MFMA operands f)
    auto read_block = [&](int st, int blk, Raw<NATIVE> &r, Frags<NATIVE> &f) MXG_INLINE {
        const uint8_t *la = lbuf(st, 0) + fa_off, *lb = lbuf(st, 1) + fb_off;
        if constexpr (FP4) {
            // block blk = MFMA step blk: lane half h takes chunk 2 blk + h,
            // the 32 codes of one scale block (the operand layout of the
            // e2m1 scaled MFMA, as measured on the device)
            const uint32_t o = (((2 * blk + khalf) ^ sw) << 4);
#pragma unroll
            for (int i = 0; i < SUB_M; ++i) {
                const v4i x = *reinterpret_cast<const v4i *>(la + i * 32 * BK + o);
                f.a[i] = v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
            }
#pragma unroll
            for (int j = 0; j < SUB_N; ++j) {
                const v4i x = *reinterpret_cast<const v4i *>(lb + j * 32 * BK + o);
                f.b[j] = v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
            }
        } else if constexpr (FP6) {
            // step blk: lane half h takes block 2 blk + h, LDS chunk 2 (2 blk + h)
            // (16 bytes) and the first 8 bytes of the next: its 32 codes in
            // operand dwords 0..5
            const int pc = 2 * (2 * blk + khalf);
            const uint32_t o0 = ((pc ^ sw) << 4), o1 = (((pc + 1) ^ sw) << 4);
#pragma unroll
            for (int i = 0; i < SUB_M; ++i) {
                const v4i lo = *reinterpret_cast<const v4i *>(la + i * 32 * BK + o0);
                const v2i hi = *reinterpret_cast<const v2i *>(la + i * 32 * BK + o1);
                f.a[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], 0, 0};
            }
#pragma unroll
            for (int j = 0; j < SUB_N; ++j) {
                const v4i lo = *reinterpret_cast<const v4i *>(lb + j * 32 * BK + o0);
                const v2i hi = *reinterpret_cast<const v2i *>(lb + j * 32 * BK + o1);
                f.b[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], 0, 0};
            }
        } else if constexpr (NATIVE) {
            const int c0 = blk * 4 + khalf;  // K 64blk+16h .. +15; chunk c0 + 2: K +32
            const uint32_t o0 = ((c0 ^ sw) << 4), o1 = (((c0 + 2) ^ sw) << 4);
#pragma unroll
            for (int i = 0; i < SUB_M; ++i) {
                const v4i lo = *reinterpret_cast<const v4i *>(la + i * 32 * BK + o0);
                const v4i hi = *reinterpret_cast<const v4i *>(la + i * 32 * BK + o1);
                f.a[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
#pragma unroll
            for (int j = 0; j < SUB_N; ++j) {
                const v4i lo = *reinterpret_cast<const v4i *>(lb + j * 32 * BK + o0);
                const v4i hi = *reinterpret_cast<const v4i *>(lb + j * 32 * BK + o1);
                f.b[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
        } else {
            const uint32_t o = (((2 * blk + khalf) ^ sw) << 4);
#pragma unroll
            for (int i = 0; i < SUB_M; ++i) r.a[i] = *reinterpret_cast<const v4i *>(la + i * 32 * BK + o);
#pragma unroll
            for (int j = 0; j < SUB_N; ++j) r.b[j] = *reinterpret_cast<const v4i *>(lb + j * 32 * BK + o);
        }
    };
    // exact mode: decode raw block `blk` (scale dwords sa/sb of its stage)
    // into the bf16 MFMA operands; native mode: nothing to do
    auto prep_block = [&](auto BLK, const Raw<NATIVE> &r, const uint32_t *sa_, const uint32_t *sb_,
                          Frags<NATIVE> &f) MXG_INLINE {
        constexpr int blk = decltype(BLK)::value;
        if constexpr (!NATIVE) {
#pragma unroll
            for (int i = 0; i < SUB_M; ++i)
                decode16<FA>(r.a[i], scale_f32<blk>(sa_[i]), f.a[i][0], f.a[i][1]);
#pragma unroll
            for (int j = 0; j < SUB_N; ++j)
                decode16<FB>(r.b[j], scale_f32<blk>(sb_[j]), f.b[j][0], f.b[j][1]);
        }
    };

    v16f acc[SUB_M][SUB_N];
#pragma unroll
    for (int i = 0; i < SUB_M; ++i)
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) acc[i][j] = v16f{};

    // MFMAs t = T0 .. T0+CNT-1 of a block, in K-major, N, M order
    auto mfma_range = [&](auto BLK, auto T0, auto CNT, const Frags<NATIVE> &f, const uint32_t *sa_,
                          const uint32_t *sb_, const uint32_t *sa2_, const uint32_t *sb2_) MXG_INLINE {
        constexpr int blk = decltype(BLK)::value;
        constexpr int t0 = decltype(T0)::value, cnt = decltype(CNT)::value;
        static_for<cnt>([&](auto TT) MXG_INLINE {
            constexpr int t = t0 + decltype(TT)::value;
            if constexpr (FP4) {
                // step blk uses scale blocks 2 blk + h: dword blk / 2, byte 2 (blk % 2) + h
                constexpr int j = t / SUB_M, i = t % SUB_M;
                const uint32_t *sa = blk < 2 ? sa_ : sa2_, *sb = blk < 2 ? sb_ : sb2_;
                acc[i][j] = mfma_scaled<FB, FA, 2 * (blk % 2)>(f.b[j], f.a[i], acc[i][j], sb[j], sa[i]);
            } else if constexpr (NATIVE) {
                constexpr int j = t / SUB_M, i = t % SUB_M;
                acc[i][j] = mfma_scaled<FB, FA, 2 * blk>(f.b[j], f.a[i], acc[i][j], sb_[j], sa_[i]);
            } else {
                constexpr int hh = t / (SUB_M * SUB_N), j = (t / SUB_M) % SUB_N, i = t % SUB_M;
                acc[i][j] = mfma_bf16_32(f.b[j][hh], f.a[i][hh], acc[i][j]);
            }
        });
    };

    // Interleave for the block that crosses into the next stage (after its
    // barrier): the next stage's first LDS reads, then the SEGS_PER_WAVE
    // direct-to-LDS loads of stage kt+2's A tile spread over the remaining
    // MFMAs, then the decode.
    auto sched_cross = [&]() MXG_INLINE {
        constexpr int rest = MF - MF / 4;  // MFMAs after the barrier
        constexpr int nld = SEGS_PER_WAVE;
        __builtin_amdgcn_sched_group_barrier(SG_DS_RD, NATIVE ? 4 : SUB_M + SUB_N, 0);
        static_for<(nld < rest ? nld : rest)>([&](auto) MXG_INLINE {
            __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
            __builtin_amdgcn_sched_group_barrier(SG_SALU, 2, 0);
        });
        if constexpr (!NATIVE) {
            static_for<(rest > nld ? rest - nld : 0)>([&](auto) MXG_INLINE {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_VALU, 4, 0);
            });
        } else {
            static_for<(rest > nld ? rest - nld : 0)>([&](auto) MXG_INLINE {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
            });
        }
    };

    // Interleave for a block: the next block's LDS reads first, a few MFMAs
    // to cover their latency, then one MFMA per three VALU (decode) slots.
    auto sched_block = [&]() MXG_INLINE {
        if constexpr (NATIVE) {
            __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 4, 0);
            static_for<MF>([&](auto) MXG_INLINE {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
            });
        } else {
            __builtin_amdgcn_sched_group_barrier(SG_DS_RD, SUB_M + SUB_N, 0);
            __builtin_amdgcn_sched_group_barrier(SG_MFMA, 4, 0);
            static_for<MF - 4>([&](auto) MXG_INLINE {
                __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
                __builtin_amdgcn_sched_group_barrier(SG_VALU, 3, 0);
            });
        }
    };

    // Block 0 of a stage also issues the SEGS_PER_WAVE loads of the next
    // stage's B tile, one per MFMA after the LDS reads' head start.
    auto sched_block_ld = [&]() MXG_INLINE {
        __builtin_amdgcn_sched_group_barrier(SG_DS_RD, NATIVE ? 4 : SUB_M + SUB_N, 0);
        if constexpr (!NATIVE) __builtin_amdgcn_sched_group_barrier(SG_MFMA, 4, 0);
        static_for<SEGS_PER_WAVE>([&](auto) MXG_INLINE {
            __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 1, 0);
            __builtin_amdgcn_sched_group_barrier(SG_SALU, 2, 0);
            if constexpr (NATIVE)
                __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
            else
                __builtin_amdgcn_sched_group_barrier(SG_VALU, 3, 0);
        });
        static_for<MF - (NATIVE ? 0 : 4) - SEGS_PER_WAVE>([&](auto) MXG_INLINE {
            __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
            if constexpr (NATIVE)
                __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
            else
                __builtin_amdgcn_sched_group_barrier(SG_VALU, 3, 0);
        });
    };

    Raw<NATIVE> raw;
    Frags<NATIVE> f0, f1;
    uint32_t csa[SUB_M], csb[SUB_N];  // scale dwords of the stage being decoded
    uint32_t csa2[SUB_M], csb2[SUB_N], sa2_1[SUB_M], sb2_1[SUB_N];  // e2m1: bytes 4..7 of a stage
    v4i wa[SUB_M], wb[SUB_N], na[SUB_M], nb[SUB_N];  // SREG windows (current, next)
    uint32_t sa1[SUB_M], sb1[SUB_N];  // !SREG: next stage's scale dwords

    // One stage.  SS: the stage's position in its scale window (SREG),
    // CROSS: whether the last block continues into stage kt+1.
    auto stage = [&](int kt, auto SS, auto CROSS, auto PAR) MXG_INLINE {
        constexpr int ss = decltype(SS)::value;
        constexpr bool cross = decltype(CROSS)::value;
        // stage buffer: a compile-time parity where the loop is unrolled by
        // two (PAR 0 / 1), else kt & 1 (PAR -1)
        constexpr int par = decltype(PAR)::value;
        const int st = par >= 0 ? par : (kt & 1);
        if constexpr (SREG) {
            if constexpr (ss == 0) scale16(kt + WIN, na, nb);  // next window, 4 stages ahead
        } else if constexpr (SLDS) {
            // next stage's scale dwords, then the next window into the other
            // buffer (a wave-uniform test: the stage loop is not unrolled by
            // windows here, which measured register spills).  The reads come
            // first: the compiler orders LDS reads of the window buffers
            // after any direct-to-LDS load into them, with a vmcnt wait that
            // would also drain the operand loads in flight.
            scale_lds(kt + 1, sa1, sb1, sa2_1, sb2_1);
            if (kt % WIN == 0) swin(kt + WIN);
        } else {
            scale4(kt + 1, sa1, sb1, sa2_1, sb2_1);               // next stage
        }
        uint32_t ksa[SUB_M], ksb[SUB_N];  // this stage's scale dwords (native MFMAs need them)
        uint32_t ksa2[SUB_M], ksb2[SUB_N];
#pragma unroll
        for (int i = 0; i < SUB_M; ++i) ksa[i] = csa[i];
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) ksb[j] = csb[j];
        if constexpr (FP4) {
#pragma unroll
            for (int i = 0; i < SUB_M; ++i) ksa2[i] = csa2[i];
#pragma unroll
            for (int j = 0; j < SUB_N; ++j) ksb2[j] = csb2[j];
        }
        static_for<BLOCKS>([&](auto BLK) MXG_INLINE {
            constexpr int blk = decltype(BLK)::value;
            Frags<NATIVE> &cur = (blk & 1) ? f1 : f0;
            Frags<NATIVE> &nxt = (blk & 1) ? f0 : f1;
            if constexpr (blk + 1 < BLOCKS) {
                read_block(st, blk + 1, raw, nxt);
                // B tile of stage kt+1 (its buffer was freed at the last barrier)
                if constexpr (blk == 0 && !NATIVE) gload(st ^ 1, kt + 1, int_c<1>{});
                mfma_range(BLK, int_c<0>{}, int_c<MF>{}, cur, ksa, ksb, ksa2, ksb2);
                prep_block(int_c<blk + 1>{}, raw, csa, csb, nxt);
                if constexpr (blk == 0 && !NATIVE)
                    sched_block_ld();
                else
                    sched_block();
                __builtin_amdgcn_sched_barrier(0);
            } else if constexpr (cross) {
                // MFMAs that keep the matrix pipe busy across the barrier
                mfma_range(BLK, int_c<0>{}, int_c<MF / 4>{}, cur, ksa, ksb, ksa2, ksb2);
                // every wave has read all of stage kt's buffer; stage kt+1 has
                // landed once this wave's loads are done and all waves pass
                wait_vmem();
                __syncthreads();
                read_block(st ^ 1, 0, raw, nxt);
                gload(st, kt + 2, int_c<0>{});  // A tile of stage kt+2
                if constexpr (NATIVE) gload(st, kt + 2, int_c<1>{});  // and its B tile
                // scale dwords of stage kt+1
                if constexpr (SREG) {
                    if constexpr (ss == WIN - 1) {
#pragma unroll
                        for (int i = 0; i < SUB_M; ++i) wa[i] = na[i];
#pragma unroll
                        for (int j = 0; j < SUB_N; ++j) wb[j] = nb[j];
                    }
                    constexpr int nx = (ss + 1) % WIN;
#pragma unroll
                    for (int i = 0; i < SUB_M; ++i) csa[i] = (uint32_t)wa[i][nx];
#pragma unroll
                    for (int j = 0; j < SUB_N; ++j) csb[j] = (uint32_t)wb[j][nx];
                    track4(kt + 1, csa, csb);
                } else {
#pragma unroll
                    for (int i = 0; i < SUB_M; ++i) csa[i] = sa1[i];
#pragma unroll
                    for (int j = 0; j < SUB_N; ++j) csb[j] = sb1[j];
                    track4(kt + 1, csa, csb);
                    if constexpr (FP4) {
#pragma unroll
                        for (int i = 0; i < SUB_M; ++i) csa2[i] = sa2_1[i];
#pragma unroll
                        for (int j = 0; j < SUB_N; ++j) csb2[j] = sb2_1[j];
                    }
                }
                native_shift(csa, csb);
                if constexpr (FP4) native_shift(csa2, csb2);
                mfma_range(BLK, int_c<MF / 4>{}, int_c<MF - MF / 4>{}, cur, ksa, ksb, ksa2, ksb2);
                prep_block(int_c<0>{}, raw, csa, csb, nxt);
                sched_cross();
                __builtin_amdgcn_sched_barrier(0);
            } else {
                mfma_range(BLK, int_c<0>{}, int_c<MF>{}, cur, ksa, ksb, ksa2, ksb2);
            }
        });
    };

    // ---- prologue ---------------------------------------------------------
    // Stage 0 and its scales, then stage 1's tiles right behind them (buffer
    // 1 is free; exact mode: stage 1's B tile follows in stage 0's first
    // block).  The wait lets stage 1's loads stay in flight: direct-to-LDS
    // loads issue in program order and complete in issue order (the scale
    // registers the compiler guards itself).
    gload(0, 0, int_c<0>{});
    gload(0, 0, int_c<1>{});
    if constexpr (SREG) {
        scale16(0, wa, wb);
    } else if constexpr (SLDS) {
        swin(0);
    } else {
        scale4(0, sa1, sb1, sa2_1, sb2_1);
    }
    gload(1, 1, int_c<0>{});
    if constexpr (NATIVE) gload(1, 1, int_c<1>{});
    wait_vmcnt<(NATIVE ? 2 : 1) * SEGS_PER_WAVE>();
    barrier_nofence();
    if constexpr (SLDS) scale_lds(0, sa1, sb1, sa2_1, sb2_1);
    if constexpr (SREG) {
#pragma unroll
        for (int i = 0; i < SUB_M; ++i) csa[i] = (uint32_t)wa[i][0];
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) csb[j] = (uint32_t)wb[j][0];
        track4(0, csa, csb);
    } else {
#pragma unroll
        for (int i = 0; i < SUB_M; ++i) csa[i] = sa1[i];
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) csb[j] = sb1[j];
        track4(0, csa, csb);
        if constexpr (FP4) {
#pragma unroll
            for (int i = 0; i < SUB_M; ++i) csa2[i] = sa2_1[i];
#pragma unroll
            for (int j = 0; j < SUB_N; ++j) csb2[j] = sb2_1[j];
        }
    }
    native_shift(csa, csb);
    if constexpr (FP4) native_shift(csa2, csb2);
    read_block(0, 0, raw, f0);
    prep_block(int_c<0>{}, raw, csa, csb, f0);

    // ---- main loop --------------------------------------------------------
    if constexpr (SREG) {
        // nk is a multiple of the window; the last window's last stage ends
        const int nw = nk / WIN;
        for (int w = 0; w + 1 < nw; ++w)
            static_for<WIN>([&](auto SS) MXG_INLINE {
                constexpr int ss = decltype(SS)::value;
                stage(WIN * w + ss, SS, std::true_type{}, int_c<ss & 1>{});
            });
        static_for<WIN - 1>([&](auto SS) MXG_INLINE {
            constexpr int ss = decltype(SS)::value;
            stage(WIN * (nw - 1) + ss, SS, std::true_type{}, int_c<ss & 1>{});
        });
        stage(nk - 1, int_c<WIN - 1>{}, std::false_type{}, int_c<1>{});
    } else if constexpr (PAIR) {
        // two stages per iteration, so that each copy names its stage buffer
        // at compile time and the compiler does not drain the direct-to-LDS
        // loads into one buffer before reading the other
        int kt = 0;
        for (; kt + 2 < nk; kt += 2) {
            stage(kt, int_c<0>{}, std::true_type{}, int_c<0>{});
            stage(kt + 1, int_c<0>{}, std::true_type{}, int_c<1>{});
        }
        if constexpr (SLDS) {  // nk is even
            stage(kt, int_c<0>{}, std::true_type{}, int_c<0>{});
            stage(kt + 1, int_c<0>{}, std::false_type{}, int_c<1>{});
        } else {
            if (kt + 1 < nk) stage(kt++, int_c<0>{}, std::true_type{}, int_c<-1>{});
            stage(kt, int_c<0>{}, std::false_type{}, int_c<-1>{});
        }
    } else {
        for (int kt = 0; kt + 1 < nk; ++kt) stage(kt, int_c<0>{}, std::true_type{}, int_c<-1>{});
        stage(nk - 1, int_c<0>{}, std::false_type{}, int_c<-1>{});
    }

    // every accumulator is complete here (keeps the last stage's MFMAs out
    // of the epilogue's branches, where their operands would stay live)
#pragma unroll
    for (int i = 0; i < SUB_M; ++i)
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) asm volatile("" : "+a"(acc[i][j]));

    // ---- fallback for scale bytes outside the window (exact mode) ---------
    // A wave whose A rows or B rows carry a scale byte outside its format's
    // window (over its K range) recomputes its 128 x 128 outputs here, one
    // 32 x 32 sub-tile at a time, straight from global memory: each 32-K
    // block is decoded with clamped scale bytes (exact), its two bf16 MFMAs
    // are summed into a fresh block partial t, and t * 2^(remainder of the
    // A row + remainder of the B row) is added to the sub-tile's sum.  Byte
    // 255 makes its row's (column's) outputs NaN, as in the definition.
    bool slow = false;
    if constexpr (!NATIVE) {
        constexpr int wa = window_width<FA == 1 ? 1 : 0>(), wb = window_width<FB == 1 ? 1 : 0>();
        slow = __builtin_amdgcn_ballot_w64(rg.outside(chk_b ? wb : wa)) != 0;
    }
    auto slow_tile = [&](int i, int j) MXG_INLINE {
        v16f s = {};
        if constexpr (!NATIVE) {
            const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
            const int lr = ln & 31, kh = ln >> 5;
            const uint32_t ar = (uint32_t)(wm * WAVE_M + 32 * i + lr);
            const uint32_t br = (uint32_t)(wn * WAVE_N + 32 * j + lr);
            const int kb0 = ks0 * (BK / 32), kb1 = min(KB, (ks0 + nk) * (BK / 32));
            constexpr int kNanCode = 4096;  // a B remainder that marks scale byte 255
            for (int kb = kb0; kb < kb1; ++kb) {
                const v4i xa = load16(rA, ar * K + 32 * kb + 16 * kh);  // rows past the tile read 0
                const v4i xb = load16(rB, br * K + 32 * kb + 16 * kh);
                const uint32_t ba = load1(rAs, scale_at(ar, kb, KB, p.scale_ps)),
                               bb = load1(rBs, scale_at(br, kb, KB, p.scale_ps));
                float da, db, na, nb;
                int ea, eb;
                clamp_scale<FA>(ba, da, ea, na);
                clamp_scale<FB>(bb, db, eb, nb);
                v8bf a0, a1, b0, b1;
                decode16<FA>(xa, da, a0, a1);
                decode16<FB>(xb, db, b0, b1);
                v16f t = mfma_bf16_32(b0, a0, v16f{});
                t = mfma_bf16_32(b1, a1, t);
                // register r holds output row n = 8 (r/4) + 4 kh + r%4 of
                // the sub-tile, whose B remainder sits in lane n
                const int code = bb == 255u ? kNanCode : eb;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int c = __shfl(code, 8 * (r / 4) + 4 * kh + (r % 4), 64);
                    const float nbr = c == kNanCode ? __builtin_nanf("") : 0.0f;
                    s[r] += __builtin_amdgcn_ldexpf(t[r], ea + (c == kNanCode ? 0 : c)) + (na + nbr);
                }
            }
        }
        return s;
    };

    store_tile<SPLIT>(p, acc, tile, sp, ntiles, m0, n0, rows_a, wm, wn, lrow, khalf, slow, slow_tile);
}

} // namespace large
} // namespace mxg
