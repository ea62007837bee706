// mxgemm_large.h -- 256x256-tile MX-FP8 GEMM kernel for gfx950 (MFMA-bound shapes).
//
// One workgroup of eight waves computes a 256 (M) x 256 (N) tile of C.  Each
// SIMD runs two of the waves, so while one issues MFMAs the other decodes,
// reads LDS or waits on memory; each wave owns a 128 (M) x 64 (N) block held
// as 4 x 2 accumulators of a 32x32 MFMA (128 fp32 per lane).
//
// K loop (BK = 128 bytes of K per stage, two LDS stages of 2 x 32 KiB):
//   * global -> LDS: 16-byte raw buffer loads that write LDS directly
//     (buffer_load_dwordx4 ... lds); each wave instruction fills one
//     contiguous 1 KiB LDS segment (8 tile rows), lane i writing bytes
//     16i..16i+15; the swizzle is applied by choosing which global chunk each
//     lane fetches.  K and row tails read as zero through the descriptor's
//     range check.  The next stage's loads are issued before the current
//     stage's MFMAs and waited for (vmcnt(0)) just before the stage barrier;
//   * scale dwords (4 blocks = one stage) go straight to registers, one per
//     lane per 32-row fragment, also one stage ahead;
//   * LDS -> registers: ds_read_b128 fragments, then the multiply:
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

namespace mxg {
namespace large {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int WAVES = 8, THREADS = 64 * WAVES;
constexpr int WAVE_M = 128, WAVE_N = 64;      // per-wave tile
constexpr int SUB_M = WAVE_M / 32, SUB_N = WAVE_N / 32;
constexpr int TILE_BYTES = BM * BK;           // one operand, one stage (32 KiB)
constexpr int SEG = 1024;                     // bytes one wave load instruction fills
constexpr int SEGS_PER_WAVE = TILE_BYTES / SEG / WAVES;  // 4 per operand per stage

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

template <int FA, int FB, bool NATIVE>
__global__ __launch_bounds__(THREADS) void kernel(GemmArgs p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2][2][TILE_BYTES];  // [stage][A/B]

    int tm, tn;
    tile_of(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int rows_a = min(BM, p.M - m0), rows_b = min(BN, p.N - n0);
    const int K = p.K, KB = p.KB;

    const rsrc_t rA = make_rsrc(p.A + (size_t)m0 * K, (uint32_t)rows_a * K);
    const rsrc_t rB = make_rsrc(p.B + (size_t)n0 * K, (uint32_t)rows_b * K);
    const rsrc_t rAs = make_rsrc(p.As + (size_t)m0 * KB, (uint32_t)rows_a * KB);
    const rsrc_t rBs = make_rsrc(p.Bs + (size_t)n0 * KB, (uint32_t)rows_b * KB);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int lrow = lane & 31, khalf = lane >> 5;

    // ---- global -> LDS, one stage ---------------------------------------
    // segment s = SEGS_PER_WAVE*wave + j holds tile rows 8s..8s+7; lane i
    // writes row 8s + i/8 at chunk position i%8, i.e. global chunk
    // (i%8) ^ swz(row) = (i%8) ^ (i/8) ^ (s & 1).
    uint32_t goff[SEGS_PER_WAVE], gk[SEGS_PER_WAVE];
#pragma unroll
    for (int j = 0; j < SEGS_PER_WAVE; ++j) {
        const int s = SEGS_PER_WAVE * wave + j;
        const int r = 8 * s + (lane >> 3);
        const int c = (lane & 7) ^ (lane >> 3) ^ (s & 1);
        gk[j] = 16 * c;
        goff[j] = (uint32_t)r * K + 16 * c;
    }
    auto gload = [&](int st, int k0) {
#pragma unroll
        for (int j = 0; j < SEGS_PER_WAVE; ++j) {
            const int s = SEGS_PER_WAVE * wave + j;
            const uint32_t off = (int)(k0 + gk[j]) < K ? goff[j] + k0 : kOob;
            load16_lds(rA, &lds[st][0][s * SEG], off);
            load16_lds(rB, &lds[st][1][s * SEG], off);
        }
    };

    // ---- scales: one dword (4 blocks = one stage) per lane per fragment --
    uint32_t sa[SUB_M], sb[SUB_N];
    auto sload = [&](int k0) {
        const int kb0 = k0 >> 5;
#pragma unroll
        for (int i = 0; i < SUB_M; ++i)
            sa[i] = load_scale4(rAs, (uint32_t)(wm * WAVE_M + i * 32 + lrow), KB, kb0,
                                p.scale_dword);
#pragma unroll
        for (int j = 0; j < SUB_N; ++j)
            sb[j] = load_scale4(rBs, (uint32_t)(wn * WAVE_N + j * 32 + lrow), KB, kb0,
                                p.scale_dword);
    };

    // ---- fragment addresses --------------------------------------------
    const int sw = swz(lrow);
    uint32_t fa_off[SUB_M], fb_off[SUB_N];
#pragma unroll
    for (int i = 0; i < SUB_M; ++i) fa_off[i] = (wm * WAVE_M + i * 32 + lrow) * BK;
#pragma unroll
    for (int j = 0; j < SUB_N; ++j) fb_off[j] = (wn * WAVE_N + j * 32 + lrow) * BK;

    v16f acc[SUB_M][SUB_N];
#pragma unroll
    for (int i = 0; i < SUB_M; ++i)
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) acc[i][j] = v16f{};

    const int nk = (K + BK - 1) / BK;

    gload(0, 0);
    sload(0);
    wait_vmem();
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        uint32_t csa[SUB_M], csb[SUB_N];
#pragma unroll
        for (int i = 0; i < SUB_M; ++i) csa[i] = (NATIVE && khalf) ? sa[i] >> 8 : sa[i];
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) csb[j] = (NATIVE && khalf) ? sb[j] >> 8 : sb[j];

        const bool more = kt + 1 < nk;
        if (more) {
            gload(st ^ 1, (kt + 1) * BK);
            sload((kt + 1) * BK);
        }

        const uint8_t *la = lds[st][0], *lb = lds[st][1];
        if constexpr (NATIVE) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int c0 = kk * 4 + khalf;  // K 64kk+16h .. +15; chunk c0 + 2: K +32
                const uint32_t o0 = ((c0 ^ sw) << 4), o1 = (((c0 + 2) ^ sw) << 4);
                v8i fa[SUB_M], fb[SUB_N];
#pragma unroll
                for (int i = 0; i < SUB_M; ++i) {
                    v4i lo = *reinterpret_cast<const v4i *>(la + fa_off[i] + o0);
                    v4i hi = *reinterpret_cast<const v4i *>(la + fa_off[i] + o1);
                    fa[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
#pragma unroll
                for (int j = 0; j < SUB_N; ++j) {
                    v4i lo = *reinterpret_cast<const v4i *>(lb + fb_off[j] + o0);
                    v4i hi = *reinterpret_cast<const v4i *>(lb + fb_off[j] + o1);
                    fb[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
#pragma unroll
                for (int j = 0; j < SUB_N; ++j)
#pragma unroll
                    for (int i = 0; i < SUB_M; ++i) {
                        if (kk == 0)
                            acc[i][j] = mfma_scaled<FB, FA, 0>(fb[j], fa[i], acc[i][j], csb[j], csa[i]);
                        else
                            acc[i][j] = mfma_scaled<FB, FA, 2>(fb[j], fa[i], acc[i][j], csb[j], csa[i]);
                    }
            }
        } else {
#pragma unroll
            for (int pb = 0; pb < BK / 32; ++pb) {
                const uint32_t o = (((2 * pb + khalf) ^ sw) << 4);
                v8bf fa[SUB_M][2], fb[SUB_N][2];
#pragma unroll
                for (int i = 0; i < SUB_M; ++i) {
                    const v4i x = *reinterpret_cast<const v4i *>(la + fa_off[i] + o);
                    decode16<FA>(x, e8m0_to_f32((csa[i] >> (8 * pb)) & 0xffu), fa[i][0], fa[i][1]);
                }
#pragma unroll
                for (int j = 0; j < SUB_N; ++j) {
                    const v4i x = *reinterpret_cast<const v4i *>(lb + fb_off[j] + o);
                    decode16<FB>(x, e8m0_to_f32((csb[j] >> (8 * pb)) & 0xffu), fb[j][0], fb[j][1]);
                }
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int j = 0; j < SUB_N; ++j)
#pragma unroll
                        for (int i = 0; i < SUB_M; ++i)
                            acc[i][j] = mfma_bf16_32(fb[j][hh], fa[i][hh], acc[i][j]);
            }
        }

        if (more) wait_vmem();
        __syncthreads();
    }

    // ---- epilogue ---------------------------------------------------------
    // acc[i][j] register r of lane l: m = 32 i + (l % 32),
    // n = 32 j + 8 (r / 4) + 4 (l / 32) + (r % 4), relative to the wave tile.
    const int esz = p.out_bf16 ? 2 : 4;
    const rsrc_t rC = make_rsrc((uint8_t *)p.C + ((size_t)m0 * p.N) * esz,
                                (uint32_t)rows_a * p.N * esz);
    const int N = p.N;
#pragma unroll
    for (int i = 0; i < SUB_M; ++i) {
        const int m = wm * WAVE_M + i * 32 + lrow;  // tile-local row
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * WAVE_N + j * 32 + 8 * g + 4 * khalf;  // global column
                const uint32_t e0 = (uint32_t)m * N + n;                        // element index
                v4f v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                         acc[i][j][4 * g + 3]};
                store_c4(rC, e0, n, N, v, p.out_bf16, p.use_acc, p.c_vec);
            }
        }
    }
}

} // namespace large
} // namespace mxg
