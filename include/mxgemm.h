/*
 * mxgemm.h -- C ABI of the MI355X (gfx950) microscaled FP8 matrix multiply.
 *
 * The operation is the scaled dot listed as async_dot_scaled in the TLX API
 * Quick Reference ("Matrix Multiply (MMA)" table): D = (A*scale_A) @
 * (B*scale_B) + D with FP8 operands, accumulating in fp32 (TLX async-compute
 * page, "TMEM-backed MX Scales": fp32 accumulator, uint8 scale tiles of K
 * extent BLOCK_K // 32).  Written out:
 *
 *   C[m,n] (+)= sum_k dec(A[m,k]) * 2^(As[m,k/32]-127) * dec(B[k,n]) * 2^(Bs[n,k/32]-127)
 *
 * with the operand formats named "e4m3" / "e5m2" (TLX API Quick Reference,
 * Utility table, get_fp8_format_name) and the argument order of the
 * synchronous form, dot_scaled(lhs, lhs_scale, lhs_format, rhs, rhs_scale,
 * rhs_format, acc, ..., out_dtype=float32) (TLX async-compute page,
 * "Scaled dot").
 *
 * Encodings (the pages give the names only): e4m3 is OCP E4M3 "FN"
 * (bias 7, no infinities, S.1111.111 = NaN, max 448); e5m2 is OCP E5M2
 * (bias 15, IEEE inf/NaN, max 57344); a scale byte s is E8M0, 2^(s-127),
 * with 255 = NaN (every product of its block is NaN, also for code 0).
 *
 * Memory layout (all dense, no leading-dimension arguments):
 *   A        M x K codes, row-major (byte A[m*K + k]); e2m1: M x K/2 bytes,
 *            e2m3 / e3m2: M x 3K/4 bytes (packed along K, see the formats
 *            below).
 *   B        N x K codes, K contiguous ("K-major"): byte B[n*K + k] = B[k,n];
 *            e2m1: N x K/2 bytes, e2m3 / e3m2: N x 3K/4 bytes.
 *   A_scale  M x (K/32) bytes, row-major (or preshuffled, see
 *            mxgemm_set_scale_layout).
 *   B_scale  N x (K/32) bytes, row-major (or preshuffled).
 *   C        M x N, row-major, fp32 or bf16 (bit pattern in uint16).
 *
 * Ownership: the caller owns every buffer, including the optional split-K
 * workspace (mxgemm_set_workspace); all pointers given to mxgemm_run are
 * device pointers on the handle's device.  The library allocates no device
 * memory and keeps no state between calls beyond the handle and the
 * workspace's arrival counters, which every call leaves at zero.
 *
 * Errors: every entry point returns an MXGEMM_* status.  On an error nothing
 * is launched and no output is touched.  Nothing throws across this ABI.
 */
#ifndef MXGEMM_H
#define MXGEMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mxgemm_ctx *mxgemm_t;

/* operand formats (format strings "e4m3" / "e5m2" / "e2m1").
 *
 * e2m1 is a reading (the pages name the F8F6F4 operand family of the scaled
 * MMA lowering, ScaledBlockedToScaledWMMAF8F6F4, and the sub-byte packing
 * switch lhs_k_pack / rhs_k_pack of dot_scaled, but give no encoding): OCP
 * FP4 E2M1 (sign, 2-bit exponent with bias 1, 1-bit mantissa; magnitudes 0,
 * 0.5, 1, 1.5, 2, 3, 4, 6; no inf/NaN), packed two codes per byte along K,
 * the even k in the low nibble (k_pack = True), so an e2m1 operand row is
 * K/2 bytes.  e2m1 x e2m1 runs on the gfx950 scaled MFMA, whose 8-product
 * windows hold every e2m1 product of a block exactly (measured), so it
 * meets the same 1e-5 * sum|ab| bound as the exact variants at the fp4 MFMA
 * rate.  e2m1 beside another format runs widened (below). */
/* e2m3 is the 6-bit member of the same family (a reading as well): OCP FP6
 * E2M3 (sign, 2-bit exponent with bias 1, 3-bit mantissa; magnitudes 0 to
 * 7.5 in steps of 1/8 below 1; no inf/NaN), packed four codes per three
 * bytes along K, code k at bits 6k .. 6k+5 of the row read as one
 * little-endian bit string, so an e2m3 operand row is 3K/4 bytes.  e2m3 x
 * e2m3 runs on the scaled MFMA, whose 8-product windows hold every e2m3
 * product of a block exactly (0.125^2 to 7.5^2 spans less than the
 * window), so it too meets the exact variants' bound.  The other FP6
 * member, e3m2 (format 3; sign, 3-bit exponent with bias 3, 2-bit
 * mantissa; magnitudes 0.0625 to 28; no inf/NaN), is packed like e2m3.  Its
 * products span about 17 binades, more than the window holds, so it always
 * runs widened.
 *
 * Widened pairs: e3m2 with any format, and e2m1 or e2m3 beside any format
 * but itself.  Every e2m1, e2m3 and e3m2 value is an e4m3 value (2^-4 to
 * 28, at most three mantissa bits), so the call first rewrites each
 * sub-byte operand as e4m3 bytes (mxgemm_widen) into the handle's operand
 * buffer (mxgemm_set_operand_buffer), keeps the scales, and multiplies the
 * resulting fp8 pair on the variant selected, with that variant's results
 * and error bound for an fp8 pair. */
enum {
    MXGEMM_FMT_E4M3 = 0,
    MXGEMM_FMT_E5M2 = 1,
    MXGEMM_FMT_E2M3 = 2,
    MXGEMM_FMT_E3M2 = 3,
    MXGEMM_FMT_E2M1 = 4
};

/* output types of C (out_dtype); bf16 is rounded to nearest even from the
 * fp32 accumulator */
enum { MXGEMM_OUT_F32 = 0, MXGEMM_OUT_BF16 = 1 };

/* input types of mxgemm_quantize */
enum { MXGEMM_X_F32 = 0, MXGEMM_X_BF16 = 1 };

/* kernel variants (mxgemm_set_variant).
 *
 * Exact variants (AUTO, LARGE, SKINNY) decode every code with its block
 * scale to bf16 and multiply on the bf16 MFMA, which forms exact products
 * and rounds once to fp32 per instruction (16 or 32 K).  The decode is
 * exact for every code when the scale byte lies in the format's window,
 * 10..246 for e4m3 and 17..239 for e5m2; a wave that meets any other byte
 * (0, 255 and the bytes near them are legal) recomputes its outputs on a
 * slower fallback that decodes with the byte clamped into the window and
 * scales each 32-K block's partial sum by the rest (exactly, by a power of
 * two), so every scale byte 0..255 gives the defined result.  Error bound:
 * |err| <= (K/16 + S) * 2^-24 * sum_k |a_k b_k| (S = K splits, 1 without),
 * which is within 1e-5 * sum|ab| for K <= 2684; at larger K the rounding
 * errors of random-sign data cancel, and the measured error stays far
 * inside 1e-5 * sum|ab| (about 6e-7 at K = 8192, 1e-6 at K = 16384).
 * Outputs whose sum|ab| exceeds the fp32 range may be +-inf or NaN (an fp32
 * partial sum overflows), and outputs below the fp32 normal range
 * (2^-126) may lose subnormal bits.
 *
 * Native variants feed the codes and scales to the gfx950 scaled MFMA
 * (v_mfma_scale_f32_*_f8f6f4) at twice the bf16 rate, for every scale byte.
 * That instruction sums each aligned group of 8 products in a fixed-point
 * window reaching 13 bits below the group's largest product and drops the
 * rest (toward zero; measured), so its error is bounded only by about
 * 2^-10 of each group's largest |product|: a product 2^-14 below the
 * largest of its group is lost outright (6e-5 * sum|ab|), and on N(0,1)
 * data at K = 256 about 1% of outputs miss 1e-5 * sum|ab|.
 *
 * e2m1 x e2m1 operands run on the scaled MFMA under every variant: for them
 * the window holds every product of a block, so the result meets the exact
 * variants' bound (see MXGEMM_FMT_E2M1). */
enum {
    MXGEMM_VARIANT_AUTO = 0,          /* exact; skinny for M <= 64, one skinny launch
                                         per 64 rows for M <= 128 (M <= 192 when N
                                         gives at most 64 tiles of 112), else large */
    MXGEMM_VARIANT_LARGE = 1,         /* exact, 256x256 tiles (MFMA-bound shapes) */
    MXGEMM_VARIANT_SKINNY = 2,        /* exact, M <= 64, streams B once (HBM-bound) */
    MXGEMM_VARIANT_LARGE_NATIVE = 3,  /* native scaled-MFMA accumulation, 256x256 tiles */
    MXGEMM_VARIANT_SKINNY_NATIVE = 4  /* native scaled-MFMA accumulation, M <= 64 */
};

enum {
    MXGEMM_OK = 0,
    MXGEMM_ERR_NULL = 1,    /* a required pointer is NULL */
    MXGEMM_ERR_FMT = 2,     /* fmtA / fmtB not e4m3, e5m2, e2m3, e3m2 or e2m1 */
    MXGEMM_ERR_DTYPE = 3,   /* out_dtype not f32/bf16, or use_acc not 0/1 */
    MXGEMM_ERR_SHAPE = 4,   /* M, N, K out of range or K % 32 != 0 */
    MXGEMM_ERR_ALIGN = 5,   /* A, B or C not 16-byte aligned */
    MXGEMM_ERR_DEVICE = 6,  /* not a gfx950 device, or not the handle's device */
    MXGEMM_ERR_HIP = 7,     /* the HIP runtime reported an error */
    MXGEMM_ERR_HANDLE = 8,  /* NULL or destroyed handle */
    MXGEMM_ERR_ALIAS = 9,   /* C overlaps an input buffer */
    MXGEMM_ERR_VARIANT = 10, /* unknown variant */
    MXGEMM_ERR_WORKSPACE = 11 /* workspace missing for a forced split, too small or
                                 misaligned, or the operand buffer of a widened pair
                                 missing or too small */
};

/* Limits of one call. */
#define MXGEMM_MAX_M ((int64_t)1 << 30)
#define MXGEMM_MAX_N ((int64_t)1 << 20)
#define MXGEMM_MAX_K ((int64_t)1 << 21)
#define MXGEMM_MAX_MN ((int64_t)1 << 36) /* M * N: C up to 256 GiB of fp32 */
#define MXGEMM_MAX_QELEMS ((int64_t)1 << 38) /* R * K of one mxgemm_quantize call */

/* Bytes of a split-K workspace: 4 KiB of arrival counters, then partial
 * tiles.  MXGEMM_WORKSPACE_BYTES (the minimum) holds 256 fp32 partials of
 * 64 x 112, enough for every small-M split; the 256 x 256 tiles of larger M
 * take 256 KiB each, and MXGEMM_WORKSPACE_BYTES_LARGE holds 256 of them, so
 * that no large-M split count is cut short by the workspace. */
#define MXGEMM_WORKSPACE_BYTES ((size_t)4096 + (size_t)256 * 64 * 112 * 4)
#define MXGEMM_WORKSPACE_BYTES_LARGE ((size_t)4096 + (size_t)256 * 256 * 256 * 4)

/* Library ABI version (this header: 1). */
int mxgemm_version(void);

/* Create a handle bound to the current HIP device.  Fails with
 * MXGEMM_ERR_DEVICE if that device is not gfx950, MXGEMM_ERR_NULL if out is
 * NULL, MXGEMM_ERR_HIP if the runtime fails.  The handle owns only host
 * memory.  The first handle on a device also sets up that device's copy of
 * the library's fixed scratch array (mxgemm_run_noalloc): it resolves the
 * array's address and clears its counters with a kernel on the null
 * stream, which it waits for. */
int mxgemm_create(mxgemm_t *out);

/* Destroy a handle (NULL is accepted and ignored).  Work already launched
 * with it is unaffected. */
int mxgemm_destroy(mxgemm_t h);

/* Select the kernel variant used by later mxgemm_run calls on this handle
 * (MXGEMM_VARIANT_*).  Exact variants differ from each other only in fp32
 * summation order.  Forcing a skinny variant makes mxgemm_run return
 * MXGEMM_ERR_VARIANT for M > 64.  e2m1 operands always run on the scaled
 * MFMA (exact for them): LARGE and LARGE_NATIVE on the 256 x 256 kernel,
 * SKINNY and SKINNY_NATIVE on the small-M kernel, AUTO on the small-M
 * kernel when M <= 64, in one launch of it per 64 rows when 64 < M <= 128
 * or, with N <= 7168, M <= 192 (as for e4m3 / e5m2), else on the 256 x 256
 * kernel.  Not synchronised with mxgemm_run calls
 * running on the same handle in other threads. */
int mxgemm_set_variant(mxgemm_t h, int variant);

/* Attach a caller-owned device buffer of at least MXGEMM_WORKSPACE_BYTES
 * (256-byte aligned) to the handle, or detach it with ws = NULL.  With a
 * workspace attached, calls that leave most of the 256 CUs idle split K
 * over several workgroups: small-M calls (M <= 64, every variant) whose N
 * gives at most 128 column tiles of 112, and M > 64 calls with at most 128 output
 * tiles of 256 x 256 (as many splits as the workspace holds partials for,
 * `bytes` counting; MXGEMM_WORKSPACE_BYTES_LARGE never limits them).  The TLX
 * global-memory page offers an atomic buffer add (tlx.buffer_atomic_add) for
 * such partial sums; here instead every split writes an fp32 partial tile to
 * the workspace and the last split of each tile to finish adds the partials
 * in split order, so results are deterministic (and within the exact
 * variants' bound).
 * Attaching zeroes the counter area with a kernel on `stream`; later calls
 * must be ordered after it.  Calls that use one workspace must not overlap
 * on the GPU (order them on one stream, or give each stream its own handle
 * and workspace).  MXGEMM_ERR_WORKSPACE for a short or misaligned buffer. */
int mxgemm_set_workspace(mxgemm_t h, void *ws, size_t bytes, hipStream_t stream);

/* Bytes of the operand buffer that a call with this format pair and shape
 * needs (see "Widened pairs" above): 0 when the pair runs as it is (e4m3 /
 * e5m2 with each other, e2m1 x e2m1, e2m3 x e2m3); else M * K rounded up to
 * a multiple of 256 when A is widened, plus N * K when B is.  -1 for an
 * unknown format or M, N, K out of the ranges of mxgemm_validate_args. */
int64_t mxgemm_operand_buffer_bytes(int fmtA, int fmtB, int64_t M, int64_t N, int64_t K);

/* Attach a caller-owned device buffer (256-byte aligned) that calls of
 * widened pairs rewrite their sub-byte operands into, or detach it with buf
 * = NULL.  A widened call whose buffer is missing or shorter than
 * mxgemm_operand_buffer_bytes returns MXGEMM_ERR_WORKSPACE, one whose
 * needed bytes of it overlap an operand, a scale buffer or C returns
 * MXGEMM_ERR_ALIAS; calls of other pairs never touch it.  Widened A sits
 * at offset 0 (when A is widened), widened B after it.  The rewrite runs
 * on the call's stream before the multiply, so widened calls that share one
 * buffer must not overlap on the GPU (order them on one stream).
 * mxgemm_run_noalloc uses it too: it is caller memory, so such a call still
 * allocates nothing.  MXGEMM_ERR_WORKSPACE for a misaligned buffer. */
int mxgemm_set_operand_buffer(mxgemm_t h, void *buf, size_t bytes);

/* Rewrite rows x K codes of a sub-byte format (fmt e2m1, e2m3 or e3m2,
 * packed as for mxgemm_run) as rows x K e4m3 bytes, each the code's value
 * exactly (signed zeros kept), asynchronously on `stream`: the step a
 * widened call takes, for callers that widen an operand once and reuse it
 * (the scales stay as they are, and the e4m3 operand multiplies to the same
 * result).  src and dst are device pointers on the handle's device, both
 * 16-byte aligned and disjoint; 1 <= rows <= MXGEMM_MAX_M, 32 <= K <=
 * MXGEMM_MAX_K with K % 32 == 0, rows * K <= MXGEMM_MAX_QELEMS.  Errors:
 * MXGEMM_ERR_FMT (fmt not sub-byte), _SHAPE, _ALIGN, _ALIAS, _NULL,
 * _DEVICE, _HANDLE; on an error nothing is launched. */
int mxgemm_widen(mxgemm_t h, const void *src, int fmt, int64_t rows, int64_t K, uint8_t *dst,
                 hipStream_t stream);

/* Number of K splits: 0 (default) chooses it from the shape, 1 never
 * splits, S >= 2 forces S splits, reduced to at most the number of 128-byte
 * K stages (of whole 16-byte scale windows -- 4 stages, 2 for e2m1 -- where
 * the large kernel reads row-major scales with K % 512 == 0), to 256 /
 * output tiles, and to the partials the workspace holds.  Applies to every kernel.  A forced S >= 2
 * that survives this makes mxgemm_run return MXGEMM_ERR_WORKSPACE when no
 * workspace is attached.  MXGEMM_ERR_SHAPE for S < 0. */
int mxgemm_set_splits(mxgemm_t h, int splits);

/* Layout of the scale bytes that mxgemm_run / mxgemm_run_noalloc read and
 * mxgemm_quantize writes with this handle (default row-major).
 *
 * The pages name preshuffled MXFP scales only as what the tiles_per_warp
 * option of the scaled dot serves (each warp holding 2 x 2 WMMA tiles for
 * better reuse of scale registers, on gfx1250; TLX async-compute page,
 * "Scaled dot") and give no byte order.
 * The layout here is a reading: the order in which the MFMA's lanes
 * consume scales.  A 32 x 32 fragment gives lane l (l < 32) row l of the
 * tile and takes one scale word (4 consecutive K blocks) per lane, so:
 *   rows are taken in groups of 32 and K blocks in groups of 4, and the
 *   pair of groups (r / 32, kb / 4) is one 128-byte unit holding the 32
 *   rows' 4-byte words in row order:
 *     byte(r, kb) = (r / 32) * 32 * (K/32) + (kb / 4) * 128 + (r % 32) * 4 + kb % 4.
 * A wave then reads a stage's scales of 32 rows as one 128-byte line
 * instead of 32 scattered words.  The buffer holds ceil(rows / 32) * 32 rows
 * (mxgemm_scale_bytes); bytes of the padding rows are never used for an
 * output.  A group of 32 rows is the same byte range in both layouts.
 *
 * With MXGEMM_SCALES_PRESHUFFLED, mxgemm_run also requires K % 128 == 0
 * (MXGEMM_ERR_SHAPE), 16-byte aligned scale pointers (MXGEMM_ERR_ALIGN),
 * and C disjoint from the padded scale buffers (MXGEMM_ERR_ALIAS);
 * mxgemm_quantize requires K % 128 == 0 and writes only the bytes of real
 * rows.  MXGEMM_ERR_VARIANT for another layout value. */
#define MXGEMM_SCALES_ROW_MAJOR 0
#define MXGEMM_SCALES_PRESHUFFLED 1
int mxgemm_set_scale_layout(mxgemm_t h, int layout);

/* Bytes of the scale buffer of a rows x K operand in `layout`: rows * K/32
 * (row-major) or ceil(rows / 32) * 32 * K/32 (preshuffled); 0 if rows < 1,
 * K < 32, K % 32 != 0 (preshuffled: K % 128 != 0) or the layout is unknown. */
int64_t mxgemm_scale_bytes(int layout, int64_t rows, int64_t K);

/* Convert the row-major scale bytes of a rows x K operand (src,
 * rows x K/32 bytes, any alignment) to the preshuffled layout (dst,
 * mxgemm_scale_bytes(MXGEMM_SCALES_PRESHUFFLED, rows, K) bytes, 16-byte
 * aligned), asynchronously on `stream`; the padding rows are written as
 * zeros.  Both are device pointers on the handle's device, owned by the
 * caller.  Errors: MXGEMM_ERR_NULL, MXGEMM_ERR_SHAPE (1 <= rows <=
 * MXGEMM_MAX_M, 128 <= K <= MXGEMM_MAX_K with K % 128 == 0, rows * K <=
 * MXGEMM_MAX_QELEMS), MXGEMM_ERR_ALIGN, MXGEMM_ERR_ALIAS (src and dst
 * overlap); on an error nothing is launched. */
int mxgemm_preshuffle_scales(mxgemm_t h, const uint8_t *src, uint8_t *dst, int64_t rows, int64_t K,
                             hipStream_t stream);

/* Check the arguments of mxgemm_run without touching the GPU: pointers
 * non-NULL, formats, out_dtype, use_acc in {0,1}, 1 <= M <= MXGEMM_MAX_M,
 * 1 <= N <= MXGEMM_MAX_N, M * N <= MXGEMM_MAX_MN, 32 <= K <= MXGEMM_MAX_K
 * with K % 32 == 0,
 * A, B, C 16-byte aligned, and C not overlapping A, B or the scales
 * (byte ranges A[M*rowA], B[N*rowB], A_scale[M*K/32], B_scale[N*K/32],
 * C[M*N*sizeof(out)], with row bytes K for e4m3 / e5m2, K/2 for e2m1, 3K/4
 * for e2m3 / e3m2).  Scales need no alignment.  These are the checks for
 * row-major scales; a handle set to preshuffled scales adds those of
 * mxgemm_set_scale_layout in mxgemm_run, and a widened pair those of
 * mxgemm_set_operand_buffer. */
int mxgemm_validate_args(const void *A, const uint8_t *A_scale, int fmtA,
                         const void *B, const uint8_t *B_scale, int fmtB,
                         const void *C, int64_t M, int64_t N, int64_t K,
                         int use_acc, int out_dtype);

/* C (+)= (A * 2^(A_scale-127)) @ (B * 2^(B_scale-127)), asynchronously on
 * `stream` (0 = the null stream).  With use_acc = 0, C is overwritten and
 * its previous contents are never read; with use_acc = 1 the previous C
 * (fp32, or bf16 widened to fp32) is added to the fp32 accumulator before
 * the single rounding to out_dtype.  Buffers must stay valid until the
 * stream reaches this point; the caller synchronises.  Thread-safe: a
 * handle without a workspace may be used from several host threads on
 * different streams (see mxgemm_set_workspace for one with), except for
 * widened pairs, whose calls share the handle's operand buffer and must be
 * ordered (mxgemm_set_operand_buffer). */
int mxgemm_run(mxgemm_t h,
               const void *A, const uint8_t *A_scale, int fmtA,
               const void *B, const uint8_t *B_scale, int fmtB,
               void *C, int64_t M, int64_t N, int64_t K,
               int use_acc, int out_dtype, hipStream_t stream);

/* mxgemm_run for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * operation, arguments, results and errors are those of mxgemm_run on a
 * handle with a workspace of MXGEMM_NOALLOC_SCRATCH_BYTES attached (a
 * workspace attached to h is not used).  The split-K scratch is a fixed
 * array inside the library instead, one per GPU, resolved when the handle is
 * created and held until the process ends, so the call allocates nothing and
 * needs no workspace.  Every call on one GPU shares that array: calls that
 * overlap on one GPU (several streams, several host threads) race, and the
 * caller must order them.  A forced split count (mxgemm_set_splits) whose
 * partial tiles do not fit in the array returns MXGEMM_ERR_WORKSPACE
 * (automatic splits are chosen to fit); MXGEMM_ERR_HIP if the handle's
 * set-up could not resolve the array. */
#define MXGEMM_NOALLOC_SCRATCH_BYTES MXGEMM_WORKSPACE_BYTES
int mxgemm_run_noalloc(mxgemm_t h,
                       const void *A, const uint8_t *A_scale, int fmtA,
                       const void *B, const uint8_t *B_scale, int fmtB,
                       void *C, int64_t M, int64_t N, int64_t K,
                       int use_acc, int out_dtype, hipStream_t stream);

/* MX block quantization: the step that produces the multiply's operands.
 * X is R x K, row-major, fp32 or bf16 (x_dtype MXGEMM_X_*); each row is cut
 * into blocks of 32 consecutive elements, one e8m0 scale byte per block
 * (the uint8 scale tile of K extent BLOCK_K // 32, TLX async-compute page,
 * "TMEM-backed MX Scales"), laid out like the operands of mxgemm_run:
 *   codes   R x K bytes, row-major (an A operand, or B stored K-contiguous);
 *           e2m1: R x K/2 bytes, two codes per byte, the even k in the low
 *           nibble; e2m3 / e3m2: R x 3K/4 bytes, four codes per three bytes;
 *   scales  R x (K/32) bytes, row-major, or in the handle's preshuffled
 *           layout (mxgemm_set_scale_layout).
 * The scale rule (a reading; the pages do not fix it): with MAX = 448
 * (e4m3), 57344 (e5m2), 6 (e2m1), 7.5 (e2m3) or 28 (e3m2), e is the
 * smallest integer with
 * max|x| <= MAX * 2^e over the block (an all-zero block takes the smallest
 * scale), the scale byte is e + 127 clamped to 0..254, and each code is
 * x * 2^(127 - scale byte) rounded to the nearest value of the format, ties
 * to even, -0 kept as negative zero (0x80; e2m1 0x8; e2m3 / e3m2 0x20).  Inputs must be finite; for a block holding a NaN
 * or an infinity the output is unspecified.
 *
 * Checks (pure host): pointers non-NULL, fmt e4m3/e5m2/e2m3/e3m2/e2m1, x_dtype, 1 <= R <=
 * MXGEMM_MAX_M, 32 <= K <= MXGEMM_MAX_K with K % 32 == 0, R * K <=
 * MXGEMM_MAX_QELEMS, X and codes 16-byte aligned, and X, codes and scales
 * pairwise disjoint.  Same status codes as mxgemm_validate_args. */
int mxgemm_validate_quantize(const void *X, int x_dtype, int64_t R, int64_t K, int fmt,
                             const uint8_t *codes, const uint8_t *scales);

/* Quantize as above, asynchronously on `stream`; all pointers are device
 * pointers on the handle's device, owned by the caller.  Nothing is
 * allocated.  On an error nothing is launched. */
int mxgemm_quantize(mxgemm_t h, const void *X, int x_dtype, int64_t R, int64_t K, int fmt,
                    uint8_t *codes, uint8_t *scales, hipStream_t stream);

/* Streaming copy of `bytes` bytes from src to dst with raw buffer loads and
 * stores (the buffer_load / buffer_store example of the TLX global-memory
 * page), asynchronously on `stream`; both are device pointers on the
 * handle's device, owned by the caller.  It computes nothing: its rate is
 * the measured "achievable HBM" bandwidth that the memory-bound kernels are
 * compared with.  mxgemm_validate_copy is its pure host check: pointers
 * non-NULL, both 16-byte aligned, 16 <= bytes <= MXGEMM_MAX_COPY_BYTES with
 * bytes % 16 == 0, and the two ranges disjoint (MXGEMM_ERR_ALIAS).  On an
 * error nothing is launched. */
#define MXGEMM_MAX_COPY_BYTES ((uint64_t)1 << 40)
int mxgemm_validate_copy(const void *dst, const void *src, uint64_t bytes);
int mxgemm_copy(mxgemm_t h, void *dst, const void *src, uint64_t bytes, hipStream_t stream);

/* Static text for a status code ("unknown status" for others). */
const char *mxgemm_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* MXGEMM_H */
