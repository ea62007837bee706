// mxgemm.hip -- host side of the C ABI declared in include/mxgemm.h.
//
// Argument checking, variant selection and the launch on the caller's
// stream.  Everything the multiply computes runs in the gfx950 kernels
// (mxgemm_large.h, mxgemm_skinny.h, mxgemm_stream.h, mxquant.h, launched
// from the k_*.hip translation units); this file does no arithmetic on the
// operands.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <new>

#include "mxgemm.h"
#include "mxgemm_large.h"
#include "mxgemm_launch.h"
#include "mxgemm_skinny.h"
#include "mxgemm_stream.h"

static_assert(mxg::stream::BN == mxg::skinny::BN && mxg::stream::MAX_M == mxg::skinny::MAX_M,
              "both small-M kernels tile N and bound M alike");

struct mxgemm_ctx {
    uint32_t magic;
    int device;
    int variant;
    int splits;      // 0 automatic, 1 never, S >= 2 forced
    uint8_t *ws;     // caller's split-K workspace, or NULL
    size_t ws_bytes;
    int scale_layout;  // MXGEMM_SCALES_*
    uint8_t *opbuf;    // caller's buffer for widened operands, or NULL
    size_t opbuf_bytes;
};

// The split-K scratch of mxgemm_run_noalloc: 4 KiB of arrival counters, then
// partial tiles, laid out like a caller's workspace of the same size.  Each
// GPU the library runs on holds its own copy until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: its
// device address is resolved once per device (scratch_setup) and only that
// address is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[MXGEMM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr uint32_t kMagic = 0x4d584732u;  // "MXG2"
constexpr uint32_t kDead = 0xdeadbeefu;

bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

__global__ void zero_words(uint32_t *p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

constexpr size_t kCounterBytes = 4096;

constexpr size_t kScratchBytes = MXGEMM_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes >= MXGEMM_WORKSPACE_BYTES, "the scratch holds every small-M split");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t *g_scratch[kMaxDevices];  // device address of `scratch` on each device, or NULL
static_assert(MXGEMM_WORKSPACE_BYTES ==
                  kCounterBytes + (size_t)mxg::stream::MAX_SPLITS_TILES * mxg::stream::MAX_M *
                                      mxg::stream::BN * sizeof(float),
              "workspace layout");
static_assert((256 / 2) * mxg::stream::CONSUMERS * sizeof(uint32_t) <= kCounterBytes,
              "one counter per consumer wave of every split tile");
static_assert((256 / 2) * mxg::large::WAVES * sizeof(uint32_t) <= kCounterBytes,
              "one counter per wave of every split tile");
constexpr size_t kLargePartial = (size_t)mxg::large::BM * mxg::large::BN * sizeof(float);
static_assert(MXGEMM_WORKSPACE_BYTES_LARGE ==
                  kCounterBytes + (size_t)mxg::stream::MAX_SPLITS_TILES * kLargePartial,
              "large workspace layout");

// Once per device, with that device current: resolve the device address of
// its copy of `scratch` and clear the arrival counters (every split-K call
// leaves them at zero again).  The clearing is a kernel on the null stream,
// waited for here, at set-up, outside any caller's stream work.
int scratch_setup(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) return MXGEMM_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev]) return MXGEMM_OK;
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MXGEMM_ERR_HIP;
    constexpr int words = (int)(kCounterBytes / 4);
    hipLaunchKernelGGL(zero_words, dim3((words + 255) / 256), dim3(256), 0, nullptr, (uint32_t *)p,
                       words);
    if (hipGetLastError() != hipSuccess || hipStreamSynchronize(nullptr) != hipSuccess)
        return MXGEMM_ERR_HIP;
    g_scratch[dev] = (uint8_t *)p;
    return MXGEMM_OK;
}

// K splits of a small-M call: none unless asked for or the column tiles
// leave more than half of the 256 CUs idle; then the largest power of two
// that keeps every split at least kMinStages 128-byte K stages long, tiles_n
// * S within one workgroup per CU, and S <= 8 (measured: more splits cost
// more in the reduction than they gain in streaming).  The exact kernel
// takes kMinStages = 8: with K a multiple of 1 KiB * S every split is a whole
// number of its 8-stage rings.  The scaled-MFMA kernel takes 4, one stage per wave
// (measured at N = 3584, K = 8192: 12.0 us at 8 splits, 12.7 at 4, 23.8 unsplit).
int choose_splits(int forced, int tiles_n, int nk, int kMinStages)
{
    constexpr int kTarget = mxg::stream::MAX_SPLITS_TILES, kMaxAuto = 8;
    int s;
    if (forced >= 1) {
        s = forced;
    } else if (tiles_n > kTarget / 2) {
        s = 1;
    } else {
        const int cap = std::min(kMaxAuto, std::min(kTarget / tiles_n, nk / kMinStages));
        s = 1;
        while (2 * s <= cap) s *= 2;
    }
    s = std::min(s, std::min(nk, kTarget / tiles_n));
    return std::max(s, 1);
}

// K splits of a large-kernel call, in the same way over its split units
// (4-stage scale windows when it reads 16-byte scale windows, else stages),
// further limited by how many 256 KiB partial tiles the workspace holds.
int choose_splits_large(int forced, int tiles, int units, int unit_stages, size_t ws_bytes)
{
    constexpr int kTarget = mxg::stream::MAX_SPLITS_TILES, kMinStages = 8, kMaxAuto = 8;
    const int fit = ws_bytes > kCounterBytes
                        ? (int)std::min<size_t>((ws_bytes - kCounterBytes) / ((size_t)tiles * kLargePartial),
                                                (size_t)kTarget)
                        : 0;
    int s;
    if (forced >= 1) {
        s = forced;
    } else if (tiles > kTarget / 2) {
        s = 1;
    } else {
        const int per = (kMinStages + unit_stages - 1) / unit_stages;  // units per split, at least
        const int cap = std::min(kMaxAuto, std::min(kTarget / tiles, units / per));
        s = 1;
        while (2 * s <= cap) s *= 2;
    }
    s = std::min(s, std::min(units, kTarget / tiles));
    // with a workspace attached, never more splits than it holds partials for
    // (ws_bytes == 0: none attached; the caller turns a forced split into an error)
    if (ws_bytes) s = std::min(s, fit);
    return std::max(s, 1);
}

// Bytes of an operand row of K codes: e2m1 packs two codes per byte, e2m3
// and e3m2 four codes per three bytes, e4m3 / e5m2 one per byte.
int64_t row_bytes(int fmt, int64_t K)
{
    return fmt == MXGEMM_FMT_E2M1                                 ? K / 2
           : fmt == MXGEMM_FMT_E2M3 || fmt == MXGEMM_FMT_E3M2 ? 3 * K / 4
                                                                  : K;
}

bool known_fmt(int f)
{
    return f == MXGEMM_FMT_E4M3 || f == MXGEMM_FMT_E5M2 || f == MXGEMM_FMT_E2M3 ||
           f == MXGEMM_FMT_E3M2 || f == MXGEMM_FMT_E2M1;
}

bool sub_byte(int f)
{
    return f == MXGEMM_FMT_E2M1 || f == MXGEMM_FMT_E2M3 || f == MXGEMM_FMT_E3M2;
}

// Whether an operand of format f, multiplied with one of format `other`, is
// rewritten as e4m3 first: e3m2 always (the scaled MFMA's window cannot hold
// its products' range), e2m1 and e2m3 unless beside themselves.
bool widened(int f, int other)
{
    return sub_byte(f) && (f == MXGEMM_FMT_E3M2 || f != other);
}

bool shape_ok(int64_t M, int64_t N, int64_t K)
{
    return M >= 1 && N >= 1 && K >= 32 && M <= MXGEMM_MAX_M && N <= MXGEMM_MAX_N &&
           K <= MXGEMM_MAX_K && (K % 32) == 0 && M * N <= MXGEMM_MAX_MN;
}

constexpr int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

// f: 2 fmtA + fmtB for the fp8 pairs (0..3), kF4 for e2m1 x e2m1, kF6 for
// e2m3 x e2m3 (both always on the scaled MFMA)
constexpr int kF4 = 4, kF6 = 5;

hipError_t dispatch(bool native, bool skinny, int f, const mxg::GemmArgs &a, hipStream_t s)
{
    if (skinny) {
        if (f == kF4) return mxg::launch_skinny_e2m1(a, s);
        if (f == kF6) return mxg::launch_skinny_e2m3(a, s);
        return native ? mxg::launch_skinny_native(f, a, s) : mxg::launch_stream_exact(f, a, s);
    }
    if (f == kF4) return mxg::launch_large_e2m1(a, s);
    if (f == kF6) return mxg::launch_large_e2m3(a, s);
    return native ? mxg::launch_large_native(f, a, s) : mxg::launch_large_exact(f, a, s);
}

} // namespace

extern "C" {

int mxgemm_version(void) { return 1; }

const char *mxgemm_status_string(int code)
{
    switch (code) {
    case MXGEMM_OK: return "ok";
    case MXGEMM_ERR_NULL: return "a required pointer is NULL";
    case MXGEMM_ERR_FMT:
        return "operand format must be e4m3 (0), e5m2 (1), e2m3 (2), e3m2 (3) or e2m1 (4)";
    case MXGEMM_ERR_DTYPE: return "out_dtype must be f32 (0) or bf16 (1) and use_acc 0 or 1";
    case MXGEMM_ERR_SHAPE:
        return "M, N, K out of range or K not a multiple of 32 (of 128 with preshuffled scales)";
    case MXGEMM_ERR_ALIGN: return "A, B, C (and preshuffled scales) must be 16-byte aligned";
    case MXGEMM_ERR_DEVICE: return "device is not gfx950 or not the handle's device";
    case MXGEMM_ERR_HIP: return "HIP runtime error";
    case MXGEMM_ERR_HANDLE: return "invalid handle";
    case MXGEMM_ERR_ALIAS: return "C overlaps an input";
    case MXGEMM_ERR_VARIANT: return "unknown kernel variant or scale layout";
    case MXGEMM_ERR_WORKSPACE:
        return "split-K workspace or operand buffer missing, too small or misaligned";
    default: return "unknown status";
    }
}

int mxgemm_create(mxgemm_t *out)
{
    if (!out) return MXGEMM_ERR_NULL;
    *out = nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MXGEMM_ERR_HIP;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MXGEMM_ERR_HIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MXGEMM_ERR_DEVICE;
    const int rs = scratch_setup(dev);
    if (rs != MXGEMM_OK) return rs;
    mxgemm_ctx *h = new (std::nothrow) mxgemm_ctx;
    if (!h) return MXGEMM_ERR_HIP;
    h->magic = kMagic;
    h->device = dev;
    h->variant = MXGEMM_VARIANT_AUTO;
    h->splits = 0;
    h->ws = nullptr;
    h->ws_bytes = 0;
    h->scale_layout = MXGEMM_SCALES_ROW_MAJOR;
    h->opbuf = nullptr;
    h->opbuf_bytes = 0;
    *out = h;
    return MXGEMM_OK;
}

int mxgemm_destroy(mxgemm_t h)
{
    if (!h) return MXGEMM_OK;
    if (h->magic != kMagic) return MXGEMM_ERR_HANDLE;
    h->magic = kDead;
    delete h;
    return MXGEMM_OK;
}

int mxgemm_set_variant(mxgemm_t h, int variant)
{
    if (!h || h->magic != kMagic) return MXGEMM_ERR_HANDLE;
    if (variant < MXGEMM_VARIANT_AUTO || variant > MXGEMM_VARIANT_SKINNY_NATIVE)
        return MXGEMM_ERR_VARIANT;
    h->variant = variant;
    return MXGEMM_OK;
}

int mxgemm_set_workspace(mxgemm_t h, void *ws, size_t bytes, hipStream_t stream)
{
    if (!h || h->magic != kMagic) return MXGEMM_ERR_HANDLE;
    if (!ws) {
        h->ws = nullptr;
        h->ws_bytes = 0;
        return MXGEMM_OK;
    }
    if (bytes < MXGEMM_WORKSPACE_BYTES || ((uintptr_t)ws & 255u)) return MXGEMM_ERR_WORKSPACE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MXGEMM_ERR_HIP;
    if (dev != h->device) return MXGEMM_ERR_DEVICE;
    constexpr int words = (int)(kCounterBytes / 4);
    hipLaunchKernelGGL(zero_words, dim3((words + 255) / 256), dim3(256), 0, stream,
                       (uint32_t *)ws, words);
    if (hipGetLastError() != hipSuccess) return MXGEMM_ERR_HIP;
    h->ws = (uint8_t *)ws;
    h->ws_bytes = bytes;
    return MXGEMM_OK;
}

int mxgemm_set_splits(mxgemm_t h, int splits)
{
    if (!h || h->magic != kMagic) return MXGEMM_ERR_HANDLE;
    if (splits < 0) return MXGEMM_ERR_SHAPE;
    h->splits = splits;
    return MXGEMM_OK;
}

int mxgemm_set_scale_layout(mxgemm_t h, int layout)
{
    if (!h || h->magic != kMagic) return MXGEMM_ERR_HANDLE;
    if (layout != MXGEMM_SCALES_ROW_MAJOR && layout != MXGEMM_SCALES_PRESHUFFLED)
        return MXGEMM_ERR_VARIANT;
    h->scale_layout = layout;
    return MXGEMM_OK;
}

int64_t mxgemm_scale_bytes(int layout, int64_t rows, int64_t K)
{
    if (rows < 1 || K < 32 || K % 32 != 0 || rows > MXGEMM_MAX_M || K > MXGEMM_MAX_K) return 0;
    if (layout == MXGEMM_SCALES_ROW_MAJOR) return rows * (K / 32);
    if (layout == MXGEMM_SCALES_PRESHUFFLED && K % 128 == 0) return (rows + 31) / 32 * 32 * (K / 32);
    return 0;
}

int mxgemm_preshuffle_scales(mxgemm_t h, const uint8_t *src, uint8_t *dst, int64_t rows, int64_t K,
                             hipStream_t stream)
{
    if (!h || h->magic != kMagic) return MXGEMM_ERR_HANDLE;
    if (!src || !dst) return MXGEMM_ERR_NULL;
    if (rows < 1 || K < 128 || rows > MXGEMM_MAX_M || K > MXGEMM_MAX_K || K % 128 != 0 ||
        rows * K > MXGEMM_MAX_QELEMS)
        return MXGEMM_ERR_SHAPE;
    if ((uintptr_t)dst & 15u) return MXGEMM_ERR_ALIGN;
    if (overlaps(src, (uint64_t)(rows * (K / 32)), dst,
                 (uint64_t)mxgemm_scale_bytes(MXGEMM_SCALES_PRESHUFFLED, rows, K)))
        return MXGEMM_ERR_ALIAS;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MXGEMM_ERR_HIP;
    if (dev != h->device) return MXGEMM_ERR_DEVICE;
    return mxg::launch_preshuffle(src, dst, (uint64_t)rows, (int)(K / 32), stream) == hipSuccess
               ? MXGEMM_OK
               : MXGEMM_ERR_HIP;
}

int mxgemm_validate_args(const void *A, const uint8_t *A_scale, int fmtA, const void *B,
                         const uint8_t *B_scale, int fmtB, const void *C, int64_t M, int64_t N,
                         int64_t K, int use_acc, int out_dtype)
{
    if (!A || !A_scale || !B || !B_scale || !C) return MXGEMM_ERR_NULL;
    if (!known_fmt(fmtA) || !known_fmt(fmtB)) return MXGEMM_ERR_FMT;
    if ((out_dtype != MXGEMM_OUT_F32 && out_dtype != MXGEMM_OUT_BF16) ||
        (use_acc != 0 && use_acc != 1))
        return MXGEMM_ERR_DTYPE;
    if (!shape_ok(M, N, K)) return MXGEMM_ERR_SHAPE;
    if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)C) & 15u) return MXGEMM_ERR_ALIGN;
    const uint64_t csize = (uint64_t)M * (uint64_t)N * (out_dtype == MXGEMM_OUT_F32 ? 4u : 2u);
    if (overlaps(C, csize, A, (uint64_t)M * (uint64_t)row_bytes(fmtA, K)) ||
        overlaps(C, csize, B, (uint64_t)N * (uint64_t)row_bytes(fmtB, K)) ||
        overlaps(C, csize, A_scale, (uint64_t)M * (K / 32)) ||
        overlaps(C, csize, B_scale, (uint64_t)N * (K / 32)))
        return MXGEMM_ERR_ALIAS;
    return MXGEMM_OK;
}

int64_t mxgemm_operand_buffer_bytes(int fmtA, int fmtB, int64_t M, int64_t N, int64_t K)
{
    if (!known_fmt(fmtA) || !known_fmt(fmtB) || !shape_ok(M, N, K)) return -1;
    return (widened(fmtA, fmtB) ? round256(M * K) : 0) + (widened(fmtB, fmtA) ? N * K : 0);
}

int mxgemm_set_operand_buffer(mxgemm_t h, void *buf, size_t bytes)
{
    if (!h || h->magic != kMagic) return MXGEMM_ERR_HANDLE;
    if (buf && ((uintptr_t)buf & 255u)) return MXGEMM_ERR_WORKSPACE;
    h->opbuf = buf ? (uint8_t *)buf : nullptr;
    h->opbuf_bytes = buf ? bytes : 0;
    return MXGEMM_OK;
}

int mxgemm_widen(mxgemm_t h, const void *src, int fmt, int64_t rows, int64_t K, uint8_t *dst,
                 hipStream_t stream)
{
    if (!h || h->magic != kMagic) return MXGEMM_ERR_HANDLE;
    if (!src || !dst) return MXGEMM_ERR_NULL;
    if (!sub_byte(fmt)) return MXGEMM_ERR_FMT;
    if (rows < 1 || K < 32 || rows > MXGEMM_MAX_M || K > MXGEMM_MAX_K || K % 32 != 0 ||
        rows * K > MXGEMM_MAX_QELEMS)
        return MXGEMM_ERR_SHAPE;
    if (((uintptr_t)src | (uintptr_t)dst) & 15u) return MXGEMM_ERR_ALIGN;
    if (overlaps(src, (uint64_t)(rows * row_bytes(fmt, K)), dst, (uint64_t)(rows * K)))
        return MXGEMM_ERR_ALIAS;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MXGEMM_ERR_HIP;
    if (dev != h->device) return MXGEMM_ERR_DEVICE;
    return mxg::launch_widen(fmt, (const uint8_t *)src, dst, (uint64_t)(rows * K), stream) == hipSuccess
               ? MXGEMM_OK
               : MXGEMM_ERR_HIP;
}

} // extern "C"

namespace {

// The multiply behind mxgemm_run and mxgemm_run_noalloc: ws / ws_bytes is
// the split-K workspace (NULL / 0: none), and `strict` turns a forced split
// count that the workspace cannot hold into MXGEMM_ERR_WORKSPACE instead of
// fewer splits.  With launch = false it makes every check of the call and
// launches nothing.
int run_impl(mxgemm_t h, const void *A, const uint8_t *A_scale, int fmtA, const void *B,
             const uint8_t *B_scale, int fmtB, void *C, int64_t M, int64_t N, int64_t K, int use_acc,
             int out_dtype, hipStream_t stream, uint8_t *ws, size_t ws_bytes, bool strict,
             bool launch)
{
    if (!h || h->magic != kMagic) return MXGEMM_ERR_HANDLE;
    const int rc = mxgemm_validate_args(A, A_scale, fmtA, B, B_scale, fmtB, C, M, N, K, use_acc,
                                        out_dtype);
    if (rc != MXGEMM_OK) return rc;
    const bool ps = h->scale_layout == MXGEMM_SCALES_PRESHUFFLED;
    if (ps) {
        // the preshuffled layout's own conditions (mxgemm_set_scale_layout)
        if (K % 128 != 0) return MXGEMM_ERR_SHAPE;
        if (((uintptr_t)A_scale | (uintptr_t)B_scale) & 15u) return MXGEMM_ERR_ALIGN;
        const uint64_t csize = (uint64_t)M * (uint64_t)N * (out_dtype == MXGEMM_OUT_F32 ? 4u : 2u);
        if (overlaps(C, csize, A_scale, (uint64_t)mxgemm_scale_bytes(MXGEMM_SCALES_PRESHUFFLED, M, K)) ||
            overlaps(C, csize, B_scale, (uint64_t)mxgemm_scale_bytes(MXGEMM_SCALES_PRESHUFFLED, N, K)))
            return MXGEMM_ERR_ALIAS;
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MXGEMM_ERR_HIP;
    if (dev != h->device) return MXGEMM_ERR_DEVICE;

    // A widened pair: each sub-byte operand rewritten as e4m3 into the
    // operand buffer (A at 0, B after it), then the fp8 pair multiplied.
    // Every check of that multiply comes first, so that an error launches
    // nothing.
    const bool wa = widened(fmtA, fmtB), wb = widened(fmtB, fmtA);
    if (wa || wb) {
        const int64_t need = mxgemm_operand_buffer_bytes(fmtA, fmtB, M, N, K);
        if (!h->opbuf || need <= 0 || (uint64_t)need > h->opbuf_bytes) return MXGEMM_ERR_WORKSPACE;
        const uint64_t csize = (uint64_t)M * (uint64_t)N * (out_dtype == MXGEMM_OUT_F32 ? 4u : 2u);
        const int layout = ps ? MXGEMM_SCALES_PRESHUFFLED : MXGEMM_SCALES_ROW_MAJOR;
        const uint8_t *ob = h->opbuf;
        if (overlaps(ob, (uint64_t)need, A, (uint64_t)(M * row_bytes(fmtA, K))) ||
            overlaps(ob, (uint64_t)need, B, (uint64_t)(N * row_bytes(fmtB, K))) ||
            overlaps(ob, (uint64_t)need, A_scale, (uint64_t)mxgemm_scale_bytes(layout, M, K)) ||
            overlaps(ob, (uint64_t)need, B_scale, (uint64_t)mxgemm_scale_bytes(layout, N, K)) ||
            overlaps(ob, (uint64_t)need, C, csize))
            return MXGEMM_ERR_ALIAS;
        uint8_t *const wA = h->opbuf;
        uint8_t *const wB = h->opbuf + (wa ? round256(M * K) : 0);
        const void *A2 = wa ? (const void *)wA : A;
        const void *B2 = wb ? (const void *)wB : B;
        const int fa2 = wa ? (int)MXGEMM_FMT_E4M3 : fmtA, fb2 = wb ? (int)MXGEMM_FMT_E4M3 : fmtB;
        const int rc2 = run_impl(h, A2, A_scale, fa2, B2, B_scale, fb2, C, M, N, K, use_acc,
                                 out_dtype, stream, ws, ws_bytes, strict, false);
        if (rc2 != MXGEMM_OK || !launch) return rc2;
        if (wa && mxg::launch_widen(fmtA, (const uint8_t *)A, wA, (uint64_t)(M * K), stream) != hipSuccess)
            return MXGEMM_ERR_HIP;
        if (wb && mxg::launch_widen(fmtB, (const uint8_t *)B, wB, (uint64_t)(N * K), stream) != hipSuccess)
            return MXGEMM_ERR_HIP;
        return run_impl(h, A2, A_scale, fa2, B2, B_scale, fb2, C, M, N, K, use_acc, out_dtype,
                        stream, ws, ws_bytes, strict, true);
    }

    // 64 < M <= 192 under AUTO: the small-M kernel (exact, or e2m1's) on
    // rows 0..63, 64..127, ..., streaming B once per 64 rows, instead of the
    // 256 x 256 kernel.  Measured at K = 8192: two launches are faster for
    // M <= 128 at N = 3584 to 28672 (e4m3: 34.1 vs 65.2 us at M = 80,
    // N = 3584, 110.1 vs 114.6 us at M = 128, N = 28672; e2m1: 27.1 vs 57.8
    // and 69.6 vs 79.0 us); three are faster for M <= 192 only while N gives
    // at most 64 column tiles (e4m3 M = 160, N = 3584: 57.0 vs 67.2 us; at
    // N = 14336: 96.0 vs 78.9 us); four never were.
    if (h->variant == MXGEMM_VARIANT_AUTO && M > mxg::skinny::MAX_M) {
        constexpr int64_t H = mxg::skinny::MAX_M;
        const int64_t tiles_n = (N + mxg::skinny::BN - 1) / mxg::skinny::BN;
        if (M <= 2 * H || (M <= 3 * H && tiles_n <= 64)) {
            const int64_t rb = row_bytes(fmtA, K);
            const size_t esz = out_dtype == MXGEMM_OUT_F32 ? 4 : 2;
            // every chunk checked before the first one launches
            for (int pass = 0; pass < (launch ? 2 : 1); ++pass) {
                for (int64_t r = 0; r < M; r += H) {
                    // 64-row steps: whole 32-row groups, the same scale offset in both layouts
                    const int rc_r = run_impl(h, (const uint8_t *)A + r * rb,
                                              A_scale + r * (K / 32), fmtA, B, B_scale, fmtB,
                                              (uint8_t *)C + (size_t)r * N * esz,
                                              std::min(H, M - r), N, K, use_acc, out_dtype, stream,
                                              ws, ws_bytes, strict, pass == 1);
                    if (rc_r != MXGEMM_OK) return rc_r;
                }
            }
            return MXGEMM_OK;
        }
    }

    mxg::GemmArgs a;
    a.A = (const uint8_t *)A;
    a.As = A_scale;
    a.B = (const uint8_t *)B;
    a.Bs = B_scale;
    a.C = C;
    // sub-byte codes are packed along K; the kernels see K as the row pitch in bytes
    const bool fp4 = fmtA == MXGEMM_FMT_E2M1, fp6 = fmtA == MXGEMM_FMT_E2M3;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)row_bytes(fmtA, K);
    const int stage_bytes = fp6 ? 96 : 128;  // bytes of a row per K stage of the scaled-MFMA kernels
    a.KB = (int)(K / 32);
    a.use_acc = use_acc;
    a.out_bf16 = out_dtype == MXGEMM_OUT_BF16;
    const uintptr_t salign = ((uintptr_t)A_scale) | ((uintptr_t)B_scale);
    a.scale_dword = (a.KB % 16 == 0 && (salign & 15u) == 0) ? 2
                    : (a.KB % 4 == 0 && (salign & 3u) == 0) ? 1 : 0;
    a.scale_ps = ps ? 1 : 0;  // then KB % 4 == 0 and 16-byte aligned: scale_dword >= 1
    a.c_vec = N % 8 == 0 ? 2 : (N % 4 == 0 ? 1 : 0);

    int variant = h->variant;
    bool native = variant == MXGEMM_VARIANT_LARGE_NATIVE ||
                  variant == MXGEMM_VARIANT_SKINNY_NATIVE;
    bool skinny;
    if (variant == MXGEMM_VARIANT_AUTO)
        skinny = M <= mxg::skinny::MAX_M;
    else
        skinny = variant == MXGEMM_VARIANT_SKINNY || variant == MXGEMM_VARIANT_SKINNY_NATIVE;
    if (skinny && M > mxg::skinny::MAX_M) return MXGEMM_ERR_VARIANT;
    if (fp4 || fp6) {
        // e2m1 x e2m1 and e2m3 x e2m3 run on the scaled MFMA, which is exact
        // for them; for M <= 64 on the small-M kernel's native mode (measured
        // faster than the 256 x 256 kernel for e2m1, split or not, from
        // N = 3584 to 28672)
        native = true;
    }
    a.splits = 1;
    a.ws = nullptr;
    a.cnt = nullptr;
    if (skinny) {
        a.tiles_m = 1;
        a.tiles_n = (int)((N + mxg::skinny::BN - 1) / mxg::skinny::BN);
        const int nk = native ? (a.K + stage_bytes - 1) / stage_bytes
                              : (int)((K + mxg::stream::BK - 1) / mxg::stream::BK);
        a.splits = choose_splits(h->splits, a.tiles_n, nk, native ? 4 : 8);
        if (a.splits > 1 && !ws) {
            if (h->splits >= 2) return MXGEMM_ERR_WORKSPACE;
            a.splits = 1;
        }
        if (a.splits > 1) {
            a.cnt = (uint32_t *)ws;
            a.ws = (float *)(ws + kCounterBytes);
        }
    } else {
        a.tiles_m = (int)((M + mxg::large::BM - 1) / mxg::large::BM);
        a.tiles_n = (int)((N + mxg::large::BN - 1) / mxg::large::BN);
        const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
        if (tiles <= mxg::stream::MAX_SPLITS_TILES / 2) {
            // stages as the kernel counts them (bytes of a row per stage)
            const int nk = (a.K + stage_bytes - 1) / stage_bytes;
            // the kernel's SCALE16: 16-byte scale windows of 16 / (scale bytes
            // per stage) stages, whole windows per split
            const bool scale16 = a.scale_dword == 2 && !ps;
            const int unit = scale16 ? mxg::large::window_stages(fp4) : 1;
            a.splits = choose_splits_large(h->splits, (int)tiles, nk / unit, unit, ws_bytes);
            if (strict && h->splits >= 2 &&
                a.splits < choose_splits_large(h->splits, (int)tiles, nk / unit, unit, 0))
                return MXGEMM_ERR_WORKSPACE;  // the forced split needs more partials than fit
            if (a.splits > 1 && !ws) {
                if (h->splits >= 2) return MXGEMM_ERR_WORKSPACE;
                a.splits = 1;
            }
            if (a.splits > 1) {
                a.cnt = (uint32_t *)ws;
                a.ws = (float *)(ws + kCounterBytes);
            }
        }
    }
    if (!launch) return MXGEMM_OK;
    const int f = fp4 ? kF4 : fp6 ? kF6 : fmtA * 2 + fmtB;
    const hipError_t e = dispatch(native, skinny, f, a, stream);
    return e == hipSuccess ? MXGEMM_OK : MXGEMM_ERR_HIP;
}

} // namespace

extern "C" {

int mxgemm_run(mxgemm_t h, const void *A, const uint8_t *A_scale, int fmtA, const void *B,
               const uint8_t *B_scale, int fmtB, void *C, int64_t M, int64_t N, int64_t K,
               int use_acc, int out_dtype, hipStream_t stream)
{
    if (!h || h->magic != kMagic) return MXGEMM_ERR_HANDLE;
    return run_impl(h, A, A_scale, fmtA, B, B_scale, fmtB, C, M, N, K, use_acc, out_dtype, stream,
                    h->ws, h->ws_bytes, false, true);
}

int mxgemm_run_noalloc(mxgemm_t h, const void *A, const uint8_t *A_scale, int fmtA, const void *B,
                       const uint8_t *B_scale, int fmtB, void *C, int64_t M, int64_t N, int64_t K,
                       int use_acc, int out_dtype, hipStream_t stream)
{
    if (!h || h->magic != kMagic) return MXGEMM_ERR_HANDLE;
    uint8_t *const sp = h->device >= 0 && h->device < kMaxDevices ? g_scratch[h->device] : nullptr;
    if (!sp) return MXGEMM_ERR_HIP;  // set-up in mxgemm_create did not resolve the array
    return run_impl(h, A, A_scale, fmtA, B, B_scale, fmtB, C, M, N, K, use_acc, out_dtype, stream,
                    sp, kScratchBytes, true, true);
}


int mxgemm_validate_quantize(const void *X, int x_dtype, int64_t R, int64_t K, int fmt,
                             const uint8_t *codes, const uint8_t *scales)
{
    if (!X || !codes || !scales) return MXGEMM_ERR_NULL;
    if (!known_fmt(fmt)) return MXGEMM_ERR_FMT;
    if (x_dtype != MXGEMM_X_F32 && x_dtype != MXGEMM_X_BF16) return MXGEMM_ERR_DTYPE;
    if (R < 1 || K < 32 || R > MXGEMM_MAX_M || K > MXGEMM_MAX_K || (K % 32) != 0 ||
        R * K > MXGEMM_MAX_QELEMS)
        return MXGEMM_ERR_SHAPE;
    if (((uintptr_t)X | (uintptr_t)codes) & 15u) return MXGEMM_ERR_ALIGN;
    const uint64_t n = (uint64_t)R * (uint64_t)K;
    const uint64_t xbytes = n * (x_dtype == MXGEMM_X_F32 ? 4u : 2u);
    const uint64_t cbytes = (uint64_t)row_bytes(fmt, (int64_t)n);  // packed sub-byte codes
    if (overlaps(X, xbytes, codes, cbytes) || overlaps(X, xbytes, scales, n / 32) ||
        overlaps(codes, cbytes, scales, n / 32))
        return MXGEMM_ERR_ALIAS;
    return MXGEMM_OK;
}

int mxgemm_quantize(mxgemm_t h, const void *X, int x_dtype, int64_t R, int64_t K, int fmt,
                    uint8_t *codes, uint8_t *scales, hipStream_t stream)
{
    if (!h || h->magic != kMagic) return MXGEMM_ERR_HANDLE;
    const int rc = mxgemm_validate_quantize(X, x_dtype, R, K, fmt, codes, scales);
    if (rc != MXGEMM_OK) return rc;
    const bool ps = h->scale_layout == MXGEMM_SCALES_PRESHUFFLED;
    const uint64_t sbytes = (uint64_t)mxgemm_scale_bytes(h->scale_layout, R, K);
    if (ps) {
        // the padded scale buffer must hold no byte of X or the codes
        if (K % 128 != 0) return MXGEMM_ERR_SHAPE;
        const uint64_t n = (uint64_t)R * (uint64_t)K;
        const uint64_t xbytes = n * (x_dtype == MXGEMM_X_F32 ? 4u : 2u);
        const uint64_t cbytes = (uint64_t)row_bytes(fmt, (int64_t)n);
        if (overlaps(X, xbytes, scales, sbytes) || overlaps(codes, cbytes, scales, sbytes))
            return MXGEMM_ERR_ALIAS;
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MXGEMM_ERR_HIP;
    if (dev != h->device) return MXGEMM_ERR_DEVICE;

    mxg::quant::QuantArgs a;
    a.X = (const uint8_t *)X;
    a.codes = codes;
    a.scales = scales;
    a.n = (uint64_t)R * (uint64_t)K;
    a.KB = (int)(K / 32);
    a.ps = ps ? 1 : 0;
    a.scale_bytes = sbytes;
    const uint64_t esz = x_dtype == MXGEMM_X_F32 ? 4 : 2;
    const uint64_t per_block = (uint64_t)(mxg::quant::THREADS / 64) * mxg::quant::WAVE_BYTES / esz;
    const dim3 grid((unsigned)((a.n + per_block - 1) / per_block));
    const dim3 block(mxg::quant::THREADS);
    const int sel = fmt * 2 + (x_dtype == MXGEMM_X_BF16 ? 1 : 0);
    return mxg::launch_quant(sel, a, grid, block, stream) == hipSuccess ? MXGEMM_OK : MXGEMM_ERR_HIP;
}

int mxgemm_validate_copy(const void *dst, const void *src, uint64_t bytes)
{
    if (!dst || !src) return MXGEMM_ERR_NULL;
    if (bytes < 16 || bytes > MXGEMM_MAX_COPY_BYTES || (bytes & 15u)) return MXGEMM_ERR_SHAPE;
    if (((uintptr_t)dst | (uintptr_t)src) & 15u) return MXGEMM_ERR_ALIGN;
    if (overlaps(dst, bytes, src, bytes)) return MXGEMM_ERR_ALIAS;
    return MXGEMM_OK;
}

int mxgemm_copy(mxgemm_t h, void *dst, const void *src, uint64_t bytes, hipStream_t stream)
{
    if (!h || h->magic != kMagic) return MXGEMM_ERR_HANDLE;
    const int rc = mxgemm_validate_copy(dst, src, bytes);
    if (rc != MXGEMM_OK) return rc;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MXGEMM_ERR_HIP;
    if (dev != h->device) return MXGEMM_ERR_DEVICE;
    return mxg::launch_copy((const uint8_t *)src, (uint8_t *)dst, bytes, stream) == hipSuccess
               ? MXGEMM_OK
               : MXGEMM_ERR_HIP;
}

} // extern "C"
