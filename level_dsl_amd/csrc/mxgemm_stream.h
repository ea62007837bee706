// mxgemm_stream.h -- small-M (M <= 64) MX-FP8 GEMM, exact mode, for gfx950.
//
// With M <= 64 the multiply is bound by reading B once from HBM (about 120
// flop per byte at M = 64, far below the chip's MFMA-to-HBM balance).  The
// kernel streams B with as little else in its way as possible, using four
// producer waves and seven consumer waves per workgroup (the producer /
// consumer split of warp specialization on the TLX warp-specialization page,
// with one workgroup barrier per stage standing in for the full/empty
// barrier pair of the pipelined GEMM pattern in the TLX API Quick Reference):
//
//   * a workgroup owns 112 columns of C (N = 28672 gives exactly 256
//     workgroups, one per CU) and all of K, in stages of 128 bytes of K;
//     workgroup n starts at stage n (mod the stage count) and wraps around,
//     so that the workgroups do not all read their B rows at the same K
//     offset (with a power-of-two row pitch those addresses crowd onto a few
//     memory channels);
//   * consumer wave w (0..6) owns columns 16w..16w+15: lane l holds B row
//     16w + l%16 and, with g = l/16, loads K 16g..16g+15 and 64+16g..64+16g+15
//     of each stage straight into registers (each load instruction reads 64
//     contiguous bytes of 16 rows), seven stages ahead in an eight-slot
//     register ring (about 100 KiB of B in flight per CU, enough to cover the
//     loaded HBM latency); it decodes its codes with their block scales to bf16
//     (v_cvt_scalef32_pk_bf16_fp8/bf8) and runs sixteen 16x16x32 bf16 MFMAs
//     per stage against A;
//   * one producer wave per 16-row tile of M (MT = ceil(M/16) of them, so
//     that at M = 64 every SIMD carries a similar share of the decode) fetch
//     the A tile (at most 64 rows x 128 bytes per stage, from L2) seven
//     stages ahead with direct-to-LDS loads into an eight-slot fp8 ring,
//     decode it once for the whole workgroup into bf16 with its scales
//     folded in, and write it to a two-slot LDS ring; a barrier per stage
//     publishes the slot.  The consumers run MT row tiles of MFMAs, so a
//     decode-size M pays for its own rows only;
//   * the scale dwords of A and of this workgroup's B rows for 64 stages at a
//     time are loaded by all waves into LDS at the start of each 64-stage
//     chunk (for K <= 8192, once), instead of a scattered load per row and
//     stage;
//   * every output element is summed by one lane over all of K in a fixed
//     order (deterministic); C is written with 16-byte (fp32) or 8-byte
//     (bf16) buffer stores;
//   * split K (when N leaves most CUs idle): workgroup (tile, split) streams
//     a contiguous range of K stages and leaves an fp32 partial tile in a
//     caller-owned workspace; the last split of each consumer wave's 16
//     columns to arrive (an arrival counter) adds the partials in split
//     order and writes C, so the result is still deterministic.
#pragma once

#include "mxgemm_common.h"

namespace mxg {
namespace stream {

constexpr int MAX_M = 64;
constexpr int BN = 112;
constexpr int BK = 128;
constexpr int CONSUMERS = 7;
constexpr int PROWS = 16;                // rows of A each producer wave decodes per stage
constexpr int MAX_SPLITS_TILES = 256;    // split-K: at most this many (tile, split) workgroups
// one producer wave per 16-row M tile: MT = ceil(M / 16) tiles, 1..4
template <int MT>
constexpr int threads_for() { return 64 * (CONSUMERS + MT); }
constexpr int RING = 8;                  // consumer register ring: the current stage + 7 ahead
constexpr int ADEPTH = 8;                // producer's fp8 A ring in LDS: the current stage + 7 ahead
constexpr int A8 = MAX_M * BK;           // bytes of one fp8 A stage (8 KiB)
constexpr int AROW = 2 * BK;             // bytes of one decoded (bf16) A row per stage
constexpr int A_SLOT = MAX_M * AROW;     // 16 KiB
constexpr int SCH = 64;                  // stages whose scale dwords sit in LDS at a time
constexpr int SPITCH = SCH + 1;          // LDS row pitch of the scale table (dwords): rows of one
                                         // column fall in different banks
constexpr int SROWS = MAX_M + BN;        // scale rows: A rows 0..63, then the B rows

// Workgroup barrier that orders LDS only: this wave's LDS reads and writes
// complete (lgkmcnt(0)), then s_barrier; the signal fences keep the compiler
// from moving LDS accesses across it.  Outstanding global loads stay in
// flight, including the producers' loads that write LDS directly: an LDS
// memory fence would wait for those too (vmcnt(0)) and drain the producers'
// prefetch every stage.  Each producer wave reads back only the rows its own
// direct loads wrote, after waiting for them with vmcnt.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// bf16 A rows in LDS: 16 chunks of 16 bytes, chunk c of row r at position
// c ^ (r & 15), so the 16 lanes of a fragment read (16 consecutive rows, one
// chunk) hit distinct banks.
__device__ __forceinline__ uint32_t a_addr(int r, int c) { return r * AROW + ((c ^ (r & 15)) << 4); }

// Scale dword of row r for stage kt (4 bytes, one per 32-element block):
// SDW selects one aligned dword load, else four byte loads; a dead stage or
// row reads zeros through an out-of-range offset.
template <bool SDW>
__device__ __forceinline__ uint32_t scale_dword(rsrc_t rs, uint32_t r, int KB, int kb0, bool live,
                                                int ps)
{
    if constexpr (SDW) {  // always so with preshuffled scales
        return __builtin_amdgcn_raw_buffer_load_b32(rs, live ? scale_at(r, kb0, KB, ps) : kOob, 0, 0);
    } else {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b)
            v |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(
                     rs, live && kb0 + b < KB ? r * KB + kb0 + b : kOob, 0, 0)
                 << (8 * b);
        return v;
    }
}

// s_waitcnt vmcnt(n) (other counters untouched); n < 64
template <int n>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0f70);
}

template <int FA, int FB, bool SDW, int MT>
__global__ __launch_bounds__(threads_for<MT>()) void kernel(GemmArgs p)
{
    static_assert(MT >= 1 && MT * 16 <= MAX_M, "M tiles");
    constexpr int THREADS = threads_for<MT>();
    __shared__ __attribute__((aligned(1024))) uint8_t a8_lds[ADEPTH][A8];   // raw A, row-major
    __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][A_SLOT];       // decoded A (bf16)
    __shared__ __attribute__((aligned(16))) uint32_t s_lds[SROWS][SPITCH];  // scale dwords
    __shared__ uint32_t slow_lds;  // nonzero: a scale byte outside its window (fallback)

    // workgroup -> (column tile, K split): split sp takes stages
    // [sp * nk / splits, (sp + 1) * nk / splits)
    const int tile = (int)(blockIdx.x % (unsigned)p.tiles_n);
    const int sp = (int)(blockIdx.x / (unsigned)p.tiles_n);
    const int n0 = tile * BN;
    const int rows_b = min(BN, p.N - n0);
    const int M = p.M, N = p.N, K = p.K, KB = p.KB;
    const int nk_all = (K + BK - 1) / BK;
    const int kbeg = (int)((int64_t)sp * nk_all / p.splits);
    const int nk = (int)((int64_t)(sp + 1) * nk_all / p.splits) - kbeg;  // this split's stages, >= 1
    static_assert(RING == ADEPTH && SCH % RING == 0, "producer and consumers run the same iterations");
    // iterations, padded to whole rings; a padding iteration loads nothing
    // (its offsets fail the range check) and adds products of zeros.  Testing
    // each stage instead costs more (measured: 15% at M <= 16), and a tested
    // copy of the last ring alone makes the kernel spill.
    const int nu = (nk + RING - 1) / RING * RING;
    const int s0 = tile % nk;
    auto kt_of = [&](int u) MXG_INLINE { const int s = u + s0; return kbeg + (s < nk ? s : s - nk); };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // Scale rows: A from row 0; B from row n0, or with preshuffled scales
    // from the 32-row group that holds it (row n0 is row nsb of the range)
    const int ps = p.scale_ps;
    const int nsb = ps ? n0 & 31 : 0;
    const rsrc_t rAs = make_rsrc(p.As, scale_span(M, KB, ps));
    const rsrc_t rBs = make_rsrc(p.Bs + (size_t)(n0 - nsb) * KB, scale_span(nsb + rows_b, KB, ps));
    // All waves: the scale dwords of iterations u0 .. u0+SCH-1 into s_lds
    // (row r < 64: A row r; else B row r - 64 of this workgroup), column u - u0.
    // (all loads are issued before the first LDS write, so the chunk costs one
    // round trip)
    //
    // Every scale byte of real data loaded here is also checked against its
    // format's window (mxgemm_common.h, scale_lo / scale_hi): a byte outside
    // it (where the fast loop's bf16 decode would round, overflow or misread
    // byte 0 / 255) sets slow_lds, and the consumers then recompute their
    // outputs on the fallback path after the loop.  Dead stages, rows past M
    // or past this workgroup's columns, and bytes past the end of K are not
    // data and are not checked.
    auto load_scales = [&](int u0) MXG_INLINE {
        constexpr int PER = (SROWS * SCH + THREADS - 1) / THREADS;
        uint32_t v[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = min(tid + THREADS * i, SROWS * SCH - 1);
            const int r = e / SCH, uu = e % SCH, u = u0 + uu;
            const bool live = u < nk;
            const int kb0 = (live ? kt_of(u) : 0) * (BK / 32);
            // rows 0..63 are A rows, the rest B rows: pick the descriptor
            const bool is_a = r < MAX_M;
            v[i] = scale_dword<SDW>(is_a ? rAs : rBs, (uint32_t)(is_a ? r : r - MAX_M + nsb), KB, kb0,
                                    live, ps);
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + THREADS * i;
            if (e < SROWS * SCH) s_lds[e / SCH][e % SCH] = v[i];
        }
        // the check reads this thread's entries back from LDS, so that the
        // loaded registers are free by then (the fence keeps the compiler
        // from forwarding the stored values)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        ScaleRange rga, rgb;
        rga.init();
        rgb.init();
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + THREADS * i;
            const int r = e / SCH, u = u0 + e % SCH;
            const bool live = u < nk && e < SROWS * SCH;
            const bool is_a = r < MAX_M;
            const bool data = live && (is_a ? r < M : r - MAX_M < rows_b);
            // valid bytes of the dword (0: none)
            const uint32_t d = mask_scale_tail(live ? s_lds[r][e % SCH] : 0u,
                                               data ? KB - kt_of(u) * (BK / 32) : 0);
            if (is_a)
                rga.add(d, window_lo2<FA == 1 ? 1 : 0>());
            else
                rgb.add(d, window_lo2<FB == 1 ? 1 : 0>());
        }
        if (rga.outside(window_width<FA == 1 ? 1 : 0>()) || rgb.outside(window_width<FB == 1 ? 1 : 0>()))
            slow_lds = 1u;
    };
    if (tid == 0) slow_lds = 0u;
    lds_barrier();  // the flag is clear before any wave checks its scales

    if (wave >= CONSUMERS) {
        // ----------------------------------------------------------- producers
        const rsrc_t rA = make_rsrc(p.A, (uint32_t)M * K);
        // fp8 A of stage u, direct to LDS: producer pw (one per M tile)
        // handles rows PROWS*pw .. +PROWS-1; its instruction j fills rows
        // PROWS*pw + 8j..+7
        // (lane l: row ... + l/8, 16-byte chunk l%8)
        const int pw = wave - CONSUMERS;
        const int c = lane & 7, r0 = PROWS * pw + (lane >> 3);
        constexpr int NJ = PROWS / 8;
        auto fetch = [&](int u) MXG_INLINE {
            const int k0 = (u < nk ? kt_of(u) : 0) * BK;
            const bool cin = u < nk && k0 + 16 * c < K;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const uint32_t r = 8 * j + r0;
                load16_lds(rA, &a8_lds[u % ADEPTH][1024 * (NJ * pw + j)],
                           cin ? r * K + k0 + 16 * c : kOob);
            }
        };
        // decode stage u (landed in a8_lds) with its A scales into a_lds[u & 1]
        auto publish = [&](int u) MXG_INLINE {
            const uint8_t *src = a8_lds[u % ADEPTH] + 1024 * NJ * pw;
            uint8_t *dst = a_lds[u & 1];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int r = 8 * j + r0;
                const v4i x = *reinterpret_cast<const v4i *>(src + 1024 * j + 16 * lane);
                const uint32_t sd = s_lds[r][u % SCH];
                const float sc = __builtin_bit_cast(float, ((sd >> (8 * (c >> 1))) & 0xffu) << 23);
                v8bf lo, hi;
                decode16<FA>(x, sc, lo, hi);
                *reinterpret_cast<v8bf *>(dst + a_addr(r, 2 * c)) = lo;
                *reinterpret_cast<v8bf *>(dst + a_addr(r, 2 * c + 1)) = hi;
            }
        };
        for (int u0 = 0; u0 < nu; u0 += SCH) {
            load_scales(u0);
            if (u0 == 0)
                for (int u = 0; u < ADEPTH - 1; ++u) fetch(u);
            lds_barrier();  // scales of this chunk in place
            for (int u1 = u0; u1 < min(u0 + SCH, nu); u1 += ADEPTH) {
                static_for<ADEPTH>([&](auto P) MXG_INLINE {
                    const int u = u1 + decltype(P)::value;
                    fetch(u + ADEPTH - 1);
                    wait_vmcnt<NJ * (ADEPTH - 1)>();  // stage u has landed
                    publish(u);
                    lds_barrier();
                });
            }
            lds_barrier();  // every wave is done with this chunk's scales
        }
        return;
    }

    // ------------------------------------------------------------- consumers
    const int w = wave;
    const int r16 = lane & 15, g = lane >> 4;
    const rsrc_t rB = make_rsrc(p.B + (size_t)n0 * K, (uint32_t)rows_b * K);
    const uint32_t brow = (uint32_t)(16 * w + r16) * K + 16 * g;
    v4i blo[RING], bhi[RING];
    auto fetch = [&](int u, auto SLOT) MXG_INLINE {
        constexpr int sl = decltype(SLOT)::value;
        const int k0 = (u < nk ? kt_of(u) : 0) * BK;
        const bool live = u < nk;
        blo[sl] = load16(rB, live && k0 + 16 * g < K ? brow + k0 : kOob);
        bhi[sl] = load16(rB, live && k0 + 64 + 16 * g < K ? brow + k0 + 64 : kOob);
    };
    v4f acc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i] = v4f{};

    static_for<RING - 1>([&](auto P) MXG_INLINE { fetch(decltype(P)::value, P); });
    for (int u0 = 0; u0 < nu; u0 += SCH) {
        load_scales(u0);
        lds_barrier();  // scales of this chunk in place
        for (int u1 = u0; u1 < min(u0 + SCH, nu); u1 += RING) {
            static_for<RING>([&](auto P) MXG_INLINE {
                constexpr int pp = decltype(P)::value;
                const int u = u1 + pp;
                fetch(u + RING - 1, int_c<(pp + RING - 1) % RING>{});
                lds_barrier();
                // B: K 16g.. (block g/2) and 64+16g.. (block 2+g/2) of this stage
                const uint32_t sd = s_lds[MAX_M + 16 * w + r16][u % SCH];
                const float slo = __builtin_bit_cast(float, ((sd >> (8 * (g >> 1))) & 0xffu) << 23);
                const float shi = __builtin_bit_cast(float, ((sd >> (8 * (2 + (g >> 1)))) & 0xffu) << 23);
                v8bf bq[4];
                decode16<FB>(blo[pp], slo, bq[0], bq[1]);
                decode16<FB>(bhi[pp], shi, bq[2], bq[3]);
                // A operand (i, q): row 16i + l%16, K 16g + 8(q%2) + 64(q/2), i.e.
                // bf16 chunk 2g + q%2 + 8(q/2) of the row
                const uint8_t *al = a_lds[u & 1];
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int i = 0; i < MT; ++i) {
                        const v8bf a = *reinterpret_cast<const v8bf *>(
                            al + a_addr(16 * i + r16, 2 * g + (q & 1) + 8 * (q >> 1)));
                        acc[i] = mfma_bf16_16(bq[q], a, acc[i]);
                    }
            });
        }
        lds_barrier();  // every wave is done with this chunk's scales
    }

    // Fallback (a scale byte outside its window somewhere in this
    // workgroup's rows): recompute acc over this split's K blocks straight
    // from global memory.  Per 32-K block, lane group g decodes K 8g..8g+7 of
    // its B row and of its A row with clamped scale bytes (exact), one
    // 16x16x32 bf16 MFMA forms the block's partial t, and t * 2^(A row
    // remainder + B column remainder) is added; byte 255 makes the row's or
    // column's outputs NaN.
    if (__builtin_amdgcn_readfirstlane(slow_lds)) {
        const rsrc_t rA = make_rsrc(p.A, (uint32_t)M * K);
        const int kb0 = kbeg * (BK / 32), kb1 = min(KB, (kbeg + nk) * (BK / 32));
        constexpr int kNanCode = 4096;  // a B remainder that marks scale byte 255
        const uint32_t bro = (uint32_t)(16 * w + r16);  // this lane's B row in the workgroup
        const uint32_t bsr = scale_row(bro + nsb, KB, ps);  // its scale row part
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[i] = v4f{};
        for (int kb = kb0; kb < kb1; ++kb) {
            const v2i xb = __builtin_bit_cast(
                v2i, __builtin_amdgcn_raw_buffer_load_b64(rB, bro * K + 32 * kb + 8 * g, 0, 0));
            const uint32_t bb = load1(rBs, bsr + scale_col(kb, ps));
            float db, nb;
            int eb;
            clamp_scale<FB>(bb, db, eb, nb);
            const v8bf b8 = decode8<FB>(xb, db);
            const int code = bb == 255u ? kNanCode : eb;
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const uint32_t aro = (uint32_t)(16 * i + r16);  // rows past M read as zero
                const v2i xa = __builtin_bit_cast(
                    v2i, __builtin_amdgcn_raw_buffer_load_b64(rA, aro * K + 32 * kb + 8 * g, 0, 0));
                const uint32_t ba = load1(rAs, scale_at(aro, kb, KB, ps));
                float da, na;
                int ea;
                clamp_scale<FA>(ba, da, ea, na);
                const v4f t = mfma_bf16_16(b8, decode8<FA>(xa, da), v4f{});
                // register r holds column 4 g + r, whose B remainder sits in lane 4 g + r
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int c = __shfl(code, 4 * g + r, 64);
                    const float nbr = c == kNanCode ? __builtin_nanf("") : 0.0f;
                    acc[i][r] += __builtin_amdgcn_ldexpf(t[r], ea + (c == kNanCode ? 0 : c)) + (na + nbr);
                }
            }
        }
    }

    // acc[i] register r of lane l: m = 16 i + l % 16, n = 16 w + 4 (l / 16) + r.
    const rsrc_t rC = make_rsrc((uint8_t *)p.C, (uint32_t)M * N * (p.out_bf16 ? 2 : 4));
    const int n = n0 + 16 * w + 4 * g;
    if (p.splits > 1) {
        // Split K: every split leaves its fp32 partial tile in the workspace
        // ([split][tile][64 rows][112 columns]); per consumer wave (16
        // columns of the tile) a counter counts the splits that are done, and
        // the wave that completes the count adds the partials in split order
        // 0, 1, ..., so the result does not depend on which split finishes
        // last.  That wave also resets the counter for the next call.
        // Partials are written and read with device-scope coherent (sc1)
        // buffer accesses, the encoding of agent-scope atomic loads and
        // stores, so they bypass the per-XCD L2s' non-coherent copies: the
        // wait for this wave's stores to complete is the whole release, and
        // no L2 writeback or invalidate is needed (a full agent-scope fence
        // writes back the whole L2 and costs tens of microseconds here).
        constexpr int TILE_F = MAX_M * BN;
        constexpr int SC1 = 16;  // cache-policy bit of the buffer intrinsics
        const rsrc_t rW = make_rsrc(p.ws, (uint32_t)(p.splits * p.tiles_n * TILE_F * 4));
        const uint32_t lane_off = (uint32_t)(tile * TILE_F + r16 * BN + 16 * w + 4 * g) * 4;
        const uint32_t split_pitch = (uint32_t)(p.tiles_n * TILE_F) * 4;
#pragma unroll
        for (int i = 0; i < MT; ++i)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, acc[i]), rW,
                                                   lane_off + sp * split_pitch + i * 16 * BN * 4,
                                                   0, SC1);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the partial has reached the coherent level
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        uint32_t *cnt = p.cnt + tile * CONSUMERS + w;
        uint32_t old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = (uint32_t)__shfl((int)old, 0, 64);
        if (old != (uint32_t)(p.splits - 1)) return;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the partials of up to QB splits are in flight at once (a split
        // past the last reads zeros through the range check and is not
        // added); they are summed in split order
        constexpr int QB = 8;
        for (int q0 = 0; q0 < p.splits; q0 += QB) {
            v4f part[QB][MT];
#pragma unroll
            for (int qq = 0; qq < QB; ++qq)
#pragma unroll
                for (int i = 0; i < MT; ++i)
                    part[qq][i] = __builtin_bit_cast(
                        v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                 rW,
                                 q0 + qq < p.splits
                                     ? lane_off + (q0 + qq) * split_pitch + i * 16 * BN * 4
                                     : kOob,
                                 0, SC1));
#pragma unroll
            for (int qq = 0; qq < QB; ++qq)
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    if (q0 + qq == 0)
                        acc[i] = part[qq][i];
                    else if (q0 + qq < p.splits)
                        acc[i] += part[qq][i];
                }
        }
    }
    if (p.out_bf16 && p.c_vec == 2) {
        // bf16 output with N % 8 == 0: lane groups g and g ^ 1 hold the two
        // halves of one 8-column group of the same row; the even group takes
        // its partner's four columns and stores all eight with one 16-byte
        // store (the odd group stores nothing)
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            v4f hi;
#pragma unroll
            for (int e = 0; e < 4; ++e) hi[e] = __shfl_xor(acc[i][e], 16, 64);
            const int m = 16 * i + r16;
            const int n8 = (g & 1) ? N : n;  // odd groups: dropped
            store_bf16x8(rC, (uint32_t)m * N + n, n8, N, acc[i], hi, p.use_acc);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int m = 16 * i + r16;
        store_c4(rC, (uint32_t)m * N + n, n, N, acc[i], p.out_bf16, p.use_acc, p.c_vec);
    }
}

} // namespace stream
} // namespace mxg
