// mxgemm_large.h -- 256x256-tile MX-FP8 GEMM kernel for gfx950 (MFMA-bound shapes).
//
// One workgroup of four waves computes a 256 (M) x 256 (N) tile of C; each
// wave owns a 128 x 128 quarter held as 4 x 4 accumulators of the 32x32
// scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4), i.e. 256 fp32 per lane.
//
// K loop (BK = 128 bytes of K per stage, two LDS stages):
//   * global -> registers: raw 16-byte buffer loads of the next A and B
//     tiles (256 rows x 128 bytes each) plus, straight into registers, the
//     scale dwords each lane needs for the next stage;
//   * LDS -> registers: two ds_read_b128 per operand fragment, in the
//     scaled-MFMA operand layout (lane half h of row r takes 16-byte chunks
//     h and h+2 of each 64-byte K step);
//   * 32 scaled MFMAs per wave per stage, issued K-major, then N, then M,
//     so that consecutive MFMAs update independent accumulators (the issue
//     order of amd_scheduled_mfma on the TLX async-compute page, "Explicit
//     MFMA scheduling");
//   * the prefetched registers are written to the other LDS stage, then
//     one workgroup barrier.
// LDS rows are 128 bytes; 16-byte chunk c of row r is stored at chunk
// position c ^ swz(r), swz(r) = (r & 7) ^ ((r >> 3) & 1), so that the lanes
// of one ds_read_b128 pass (consecutive rows, same chunk) and of one
// ds_write_b128 pass hit distinct banks.
//
// Roles in the MFMA: the B tile supplies the instruction's rows and the A
// tile its columns, so each lane's accumulator registers hold 4 consecutive
// n of one m -- one 16-byte fp32 (or 8-byte bf16) store per group (the
// "transposed" MFMA layout that the TLX global-memory page pairs with
// vectorised buffer_store).
#pragma once

#include "mxgemm_common.h"

namespace mxg {

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
    int scale_dword;       // 1: KB % 4 == 0 and scale bases 4-byte aligned
    int c_vec;             // 1: N % 4 == 0 (aligned vector stores of C)
};

namespace large {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int THREADS = 256;
constexpr int WAVE_M = 128, WAVE_N = 128;     // per-wave tile
constexpr int SUB_M = WAVE_M / 32, SUB_N = WAVE_N / 32;
constexpr int TILE_BYTES = BM * BK;           // one operand, one stage (32 KiB)
constexpr int LOADS_PER_THREAD = TILE_BYTES / 16 / THREADS;  // 8 per operand

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
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][TILE_BYTES];  // [stage][A/B]

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
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lrow = lane & 31, khalf = lane >> 5;

    // ---- global -> register loads of one stage --------------------------
    // chunk c = tid + 256*i: tile row c / 8, 16-byte chunk c % 8 of the row.
    uint32_t goff[LOADS_PER_THREAD];
    uint32_t lds_w[LOADS_PER_THREAD];
#pragma unroll
    for (int i = 0; i < LOADS_PER_THREAD; ++i) {
        const int c = tid + THREADS * i;
        const int r = c >> 3, ch = c & 7;
        goff[i] = (uint32_t)r * K + ch * 16;
        lds_w[i] = r * BK + ((ch ^ swz(r)) << 4);
    }
    const int ch_lane = (tid & 7) * 16;  // K byte of this thread's chunk within a stage

    v4i ga[LOADS_PER_THREAD], gb[LOADS_PER_THREAD];
    auto gload = [&](int k0) {
        const bool kin = k0 + ch_lane < K;
#pragma unroll
        for (int i = 0; i < LOADS_PER_THREAD; ++i) {
            const uint32_t off = kin ? goff[i] + k0 : kOob;
            ga[i] = load16(rA, off);
            gb[i] = load16(rB, off);
        }
    };
    auto lstore = [&](int st) {
#pragma unroll
        for (int i = 0; i < LOADS_PER_THREAD; ++i) {
            *reinterpret_cast<v4i *>(&lds[st][0][lds_w[i]]) = ga[i];
            *reinterpret_cast<v4i *>(&lds[st][1][lds_w[i]]) = gb[i];
        }
    };

    // ---- scales: one dword (4 blocks = one stage) per lane per subtile ---
    // lane half khalf of a row supplies block 2*kk + khalf of the stage to
    // MFMA k-step kk; lanes of the upper half shift their dword down one byte
    // so that the instruction's byte select is 0 for kk = 0 and 2 for kk = 1.
    uint32_t sa[SUB_M], sb[SUB_N];
    auto sload = [&](int k0) {
        const int kb0 = k0 >> 5;
#pragma unroll
        for (int i = 0; i < SUB_M; ++i) {
            const int r = wm * WAVE_M + i * 32 + lrow;
            sa[i] = 0;
            if (p.scale_dword) {
                sa[i] = load4(rAs, (uint32_t)r * KB + kb0);
            } else {
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    sa[i] |= load1(rAs, kb0 + b < KB ? (uint32_t)r * KB + kb0 + b : kOob) << (8 * b);
            }
        }
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) {
            const int r = wn * WAVE_N + j * 32 + lrow;
            sb[j] = 0;
            if (p.scale_dword) {
                sb[j] = load4(rBs, (uint32_t)r * KB + kb0);
            } else {
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    sb[j] |= load1(rBs, kb0 + b < KB ? (uint32_t)r * KB + kb0 + b : kOob) << (8 * b);
            }
        }
    };

    // ---- fragment reads -------------------------------------------------
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

    gload(0);
    sload(0);
    lstore(0);
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
            gload((kt + 1) * BK);
            sload((kt + 1) * BK);
        }

        if constexpr (NATIVE) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int c0 = kk * 4 + khalf;  // K 64kk+16h .. +15; chunk c0 + 2: K +32
                const uint32_t o0 = ((c0 ^ sw) << 4), o1 = (((c0 + 2) ^ sw) << 4);
                v8i fa[SUB_M], fb[SUB_N];
#pragma unroll
                for (int i = 0; i < SUB_M; ++i) {
                    v4i lo = *reinterpret_cast<const v4i *>(&lds[st][0][fa_off[i] + o0]);
                    v4i hi = *reinterpret_cast<const v4i *>(&lds[st][0][fa_off[i] + o1]);
                    fa[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
#pragma unroll
                for (int j = 0; j < SUB_N; ++j) {
                    v4i lo = *reinterpret_cast<const v4i *>(&lds[st][1][fb_off[j] + o0]);
                    v4i hi = *reinterpret_cast<const v4i *>(&lds[st][1][fb_off[j] + o1]);
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
            // Exact path: K block p (32 bytes) of the stage; lane half h takes
            // its 16-byte chunk 2p + h, decodes it with the row's block-p scale
            // into 16 bf16 and feeds two 32x32x16 bf16 MFMAs.
#pragma unroll
            for (int pb = 0; pb < BK / 32; ++pb) {
                const uint32_t o = (((2 * pb + khalf) ^ sw) << 4);
                v8bf fa[SUB_M][2], fb[SUB_N][2];
#pragma unroll
                for (int i = 0; i < SUB_M; ++i) {
                    const v4i x = *reinterpret_cast<const v4i *>(&lds[st][0][fa_off[i] + o]);
                    decode16<FA>(x, e8m0_to_f32((csa[i] >> (8 * pb)) & 0xffu), fa[i][0], fa[i][1]);
                }
#pragma unroll
                for (int j = 0; j < SUB_N; ++j) {
                    const v4i x = *reinterpret_cast<const v4i *>(&lds[st][1][fb_off[j] + o]);
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

        if (more) lstore(st ^ 1);
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
                if (p.c_vec) {
                    const uint32_t off = n < N ? e0 * esz : kOob;
                    if (!p.out_bf16) {
                        if (p.use_acc) v += __builtin_bit_cast(v4f, load16(rC, off));
                        store16(rC, off, v);
                    } else {
                        if (p.use_acc) {
                            v2i old = __builtin_bit_cast(
                                v2i, __builtin_amdgcn_raw_buffer_load_b64(rC, off, 0, 0));
                            v[0] += bf16_to_f32((uint32_t)old[0] & 0xffffu);
                            v[1] += bf16_to_f32((uint32_t)old[0] >> 16);
                            v[2] += bf16_to_f32((uint32_t)old[1] & 0xffffu);
                            v[3] += bf16_to_f32((uint32_t)old[1] >> 16);
                        }
                        v2i o = {(int)(bf16_bits(v[0]) | (bf16_bits(v[1]) << 16)),
                                 (int)(bf16_bits(v[2]) | (bf16_bits(v[3]) << 16))};
                        store8(rC, off, o);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t off = (n + e) < N ? (e0 + e) * esz : kOob;
                        float x = v[e];
                        if (!p.out_bf16) {
                            if (p.use_acc) x += __builtin_bit_cast(float, load4(rC, off));
                            store4(rC, off, __builtin_bit_cast(uint32_t, x));
                        } else {
                            if (p.use_acc)
                                x += bf16_to_f32((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(
                                    rC, off, 0, 0));
                            store2(rC, off, (uint16_t)bf16_bits(x));
                        }
                    }
                }
            }
        }
    }
}

} // namespace large
} // namespace mxg
