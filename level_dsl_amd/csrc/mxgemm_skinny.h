// mxgemm_skinny.h -- small-M (M <= 64) MX-FP8 GEMM kernel for gfx950,
// native scaled-MFMA variant (the exact variant is mxgemm_stream.h).
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
//     staging is needed, and the next stage's loads are in flight while the
//     current stage's MFMAs run.  Lane l works on row l % 16; with
//     g = l / 16 it loads K 16g..16g+15 and 64+16g..64+16g+15 of each
//     128-byte stage (each load instruction reads 64 contiguous bytes of 16
//     rows).  Exact mode (default): the two chunks are decoded with the
//     scales of their K blocks (g/2 and 2 + g/2) into 32 bf16 that feed four
//     16x16x32 bf16 MFMAs.  Native mode: this is the operand layout of
//     v_mfma_scale_f32_16x16x128_f8f6f4 (as measured on the device) and the
//     lane supplies the scale of block g to it;
//   * A (at most 64 x K bytes) is re-read by every workgroup and stays in L2;
//   * at the end the four per-wave partial tiles are summed in a fixed order
//     through LDS (deterministic), use_acc adds the old C, and C is written
//     with coalesced 16-byte (fp32) or 8-byte (bf16) buffer stores.
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

template <int FX, int FY>
__device__ __forceinline__ v4f mfma16(v8i x, v8i y, v4f c, uint32_t sx, uint32_t sy)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, FX, FY, 0, (int)sx, 0,
                                                           (int)sy);
}

struct Stage {
    v8i b[SUB_N];
    v8i a[SUB_M];
    uint32_t sb[SUB_N];  // exact: blocks g/2 (byte 0) and 2 + g/2 (byte 1); native: block g
    uint32_t sa[SUB_M];
};

template <int FA, int FB, bool NATIVE>
__global__ __launch_bounds__(THREADS) void kernel(GemmArgs p)
{
    __shared__ __attribute__((aligned(16))) float red[WAVES][MAX_M][BN];

    const int n0 = blockIdx.x * BN;
    const int rows_b = min(BN, p.N - n0);
    const int M = p.M, N = p.N, K = p.K, KB = p.KB;

    const rsrc_t rA = make_rsrc(p.A, (uint32_t)M * K);
    const rsrc_t rB = make_rsrc(p.B + (size_t)n0 * K, (uint32_t)rows_b * K);
    const rsrc_t rAs = make_rsrc(p.As, (uint32_t)M * KB);
    const rsrc_t rBs = make_rsrc(p.Bs + (size_t)n0 * KB, (uint32_t)rows_b * KB);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, kq = lane >> 4;

    uint32_t boff[SUB_N], aoff[SUB_M], bsoff[SUB_N], asoff[SUB_M];
    // chunks K 16g.. and 64+16g.. of each stage
    constexpr int LO = 16, HI = 64;
    const int sb0 = NATIVE ? kq : kq / 2;  // scale block of the low chunk (exact)
#pragma unroll
    for (int j = 0; j < SUB_N; ++j) {
        boff[j] = (uint32_t)(16 * j + r16) * K + kq * LO;
        bsoff[j] = (uint32_t)(16 * j + r16) * KB + sb0;
    }
#pragma unroll
    for (int i = 0; i < SUB_M; ++i) {
        aoff[i] = (uint32_t)(16 * i + r16) * K + kq * LO;
        asoff[i] = (uint32_t)(16 * i + r16) * KB + sb0;
    }

    auto load_stage = [&](int kt, Stage &s) {
        const int k0 = kt * BK;
        const bool lo_in = k0 + kq * LO < K, hi_in = k0 + kq * LO + HI < K;
        const int kb0 = kt * (BK / 32);
        // scale bytes: native, block g; exact, blocks g/2 (low chunk) and 2 + g/2
        const bool s0_in = NATIVE ? k0 + kq * 32 < K : lo_in, s1_in = hi_in;
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) {
            v4i lo = load16(rB, lo_in ? boff[j] + k0 : kOob);
            v4i hi = load16(rB, hi_in ? boff[j] + k0 + HI : kOob);
            s.b[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            s.sb[j] = load1(rBs, s0_in ? bsoff[j] + kb0 : kOob);
            if (!NATIVE) s.sb[j] |= load1(rBs, s1_in ? bsoff[j] + kb0 + 2 : kOob) << 8;
        }
#pragma unroll
        for (int i = 0; i < SUB_M; ++i) {
            v4i lo = load16(rA, lo_in ? aoff[i] + k0 : kOob);
            v4i hi = load16(rA, hi_in ? aoff[i] + k0 + HI : kOob);
            s.a[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            s.sa[i] = load1(rAs, s0_in ? asoff[i] + kb0 : kOob);
            if (!NATIVE) s.sa[i] |= load1(rAs, s1_in ? asoff[i] + kb0 + 2 : kOob) << 8;
        }
    };

    v4f acc[SUB_M][SUB_N];
#pragma unroll
    for (int i = 0; i < SUB_M; ++i)
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) acc[i][j] = v4f{};

    const int nk = (K + BK - 1) / BK;
    const int s0 = (int)(blockIdx.x % (unsigned)nk);  // this workgroup's first stage
    auto stage_of = [&](int t) { const int s = t + s0; return s < nk ? s : s - nk; };
    Stage cur, nxt;
    if (wave < nk) load_stage(stage_of(wave), cur);
    for (int t = wave; t < nk; t += WAVES) {
        const bool more = t + WAVES < nk;
        if (more) load_stage(stage_of(t + WAVES), nxt);
        if constexpr (NATIVE) {
#pragma unroll
            for (int j = 0; j < SUB_N; ++j)
#pragma unroll
                for (int i = 0; i < SUB_M; ++i)
                    acc[i][j] = mfma16<FB, FA>(cur.b[j], cur.a[i], acc[i][j], cur.sb[j], cur.sa[i]);
        } else {
            // decode each lane's 32 codes with its block scale into 4 x 8 bf16,
            // then four 16x16x32 bf16 MFMAs per (i, j)
            v8bf fa[SUB_M][4], fb[SUB_N][4];
#pragma unroll
            for (int i = 0; i < SUB_M; ++i) {
                decode16<FA>(v4i{cur.a[i][0], cur.a[i][1], cur.a[i][2], cur.a[i][3]},
                             scale_f32<0>(cur.sa[i]), fa[i][0], fa[i][1]);
                decode16<FA>(v4i{cur.a[i][4], cur.a[i][5], cur.a[i][6], cur.a[i][7]},
                             scale_f32<1>(cur.sa[i]), fa[i][2], fa[i][3]);
            }
#pragma unroll
            for (int j = 0; j < SUB_N; ++j) {
                decode16<FB>(v4i{cur.b[j][0], cur.b[j][1], cur.b[j][2], cur.b[j][3]},
                             scale_f32<0>(cur.sb[j]), fb[j][0], fb[j][1]);
                decode16<FB>(v4i{cur.b[j][4], cur.b[j][5], cur.b[j][6], cur.b[j][7]},
                             scale_f32<1>(cur.sb[j]), fb[j][2], fb[j][3]);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int j = 0; j < SUB_N; ++j)
#pragma unroll
                    for (int i = 0; i < SUB_M; ++i)
                        acc[i][j] = mfma_bf16_16(fb[j][q], fa[i][q], acc[i][j]);
        }
        if (more) cur = nxt;
    }

    // acc[i][j] register r of lane l: m = 16 i + l % 16, n = 16 j + 4 (l / 16) + r.
#pragma unroll
    for (int i = 0; i < SUB_M; ++i)
#pragma unroll
        for (int j = 0; j < SUB_N; ++j)
            *reinterpret_cast<v4f *>(&red[wave][16 * i + r16][16 * j + 4 * kq]) = acc[i][j];
    __syncthreads();

    const rsrc_t rC = make_rsrc((uint8_t *)p.C, (uint32_t)M * N * (p.out_bf16 ? 2 : 4));
    constexpr int Q = MAX_M * BN / 4;  // float4 groups in the tile
    for (int q = tid; q < Q; q += THREADS) {
        const int m = q / (BN / 4), nl = (q % (BN / 4)) * 4;
        if (m >= M) continue;
        v4f v = *reinterpret_cast<const v4f *>(&red[0][m][nl]);
#pragma unroll
        for (int w = 1; w < WAVES; ++w) v += *reinterpret_cast<const v4f *>(&red[w][m][nl]);
        const int n = n0 + nl;
        store_c4(rC, (uint32_t)m * N + n, n, N, v, p.out_bf16, p.use_acc, p.c_vec);
    }
}

} // namespace skinny
} // namespace mxg
