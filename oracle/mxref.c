/*
 * mxref.c -- CPU oracle for the microscaled (MX) FP8 matrix multiply.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library,
 * its Python binding) may link, load or call this file; only the tests, the
 * package's smoke check and the benchmark's CPU-baseline leg do.  It shares
 * no code, header, table or constant with the GPU path.
 *
 * What it computes (TLX API Quick Reference, "Matrix Multiply (MMA)" table,
 * row async_dot_scaled: D = (A*scale_A) @ (B*scale_B) + D with FP8 inputs;
 * TLX async-compute page, "TMEM-backed MX Scales": uint8 scales whose K
 * extent is BLOCK_K // 32, i.e. one scale byte per 32 K-elements;
 * "Scaled dot": accumulator / out_dtype float32 by default):
 *
 *   C[m,n] (+)= sum_k  dec(A[m,k]) * 2^(sa[m,k/32]-127)
 *                    * dec(B[k,n]) * 2^(sb[n,k/32]-127)
 *
 * Readings that the pages leave open (stated, not quoted):
 *   - e4m3 is the OCP "FN" variant (bias 7, S.1111.111 is NaN, no inf,
 *     max 448); e5m2 is OCP (bias 15, IEEE-like inf/NaN, max 57344).
 *     The pages give only the names "e4m3"/"e5m2".
 *   - a scale byte s is e8m0: 2^(s-127) for s in 0..254, NaN for 255.
 *   - e2m1 (the 4-bit member of the F8F6F4 operand family that the pages
 *     name for the scaled WMMA) is OCP FP4 E2M1: sign | 2-bit exponent,
 *     bias 1 | 1-bit mantissa, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6, no
 *     inf or NaN.  Its codes are packed two per byte along K (the default
 *     lhs_k_pack / rhs_k_pack = True of dot_scaled): element k of a row is
 *     the low nibble of byte k/2 when k is even, the high nibble when odd,
 *     so a row of K elements takes ceil(K/2) bytes.
 *   - e2m3 and e3m2 (the 6-bit members of that family) are OCP FP6 E2M3
 *     (sign | 2-bit exponent, bias 1 | 3-bit mantissa; max 7.5) and E3M2
 *     (sign | 3-bit exponent, bias 3 | 2-bit mantissa; max 28), neither with
 *     inf or NaN.  Their codes are packed four per three bytes along K:
 *     element k of a row occupies bits 6k .. 6k+5 of the row read as one
 *     little-endian bit string, so a row of K elements takes ceil(6K/8)
 *     bytes.
 *   - memory layout: A is M x K row-major bytes; B is stored K-contiguous
 *     ("K-major"), B_mem[n*K + k] = B[k,n]; scales are row-major
 *     M x KB and N x KB bytes with KB = ceil(K/32).
 *   - use_acc adds the incoming C (fp32, or bf16 widened) as one more addend.
 *
 * Method: the plain definition.  Every factor is decoded exactly to double;
 * every product of two 8-bit floats and two powers of two is exact in
 * binary64 (at most 8 significant bits, exponents within +-286), and the K
 * products are summed in ascending k with one double accumulator, then
 * rounded once to fp32 (and, for bf16 output, once more fp32 -> bf16 with
 * round-to-nearest-even).  The sum of |products| is returned alongside so
 * the caller can apply a relative tolerance.  Compile with
 * -ffp-contract=off and without fast-math.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MXREF_FMT_E4M3 0
#define MXREF_FMT_E5M2 1
#define MXREF_FMT_E2M3 2
#define MXREF_FMT_E3M2 3
#define MXREF_FMT_E2M1 4
#define MXREF_FMT_E8M0 8
#define MXREF_NTAB 9

/* ---- format decoders, written from the OCP 8-bit float / MX definitions -- */

/* e4m3 (OCP FN): sign | 4-bit exponent, bias 7 | 3-bit mantissa.
 * exponent field 0 is subnormal: (m/8) * 2^(1-7); S.1111.111 is NaN. */
static double dec_e4m3(unsigned c)
{
    unsigned s = (c >> 7) & 1u, e = (c >> 3) & 15u, m = c & 7u;
    double v;
    if (e == 15u && m == 7u)
        return NAN;
    if (e == 0u)
        v = ldexp((double)m, 1 - 7 - 3);          /* m/8 * 2^-6 */
    else
        v = ldexp((double)(8u + m), (int)e - 7 - 3); /* (1+m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* e5m2 (OCP): sign | 5-bit exponent, bias 15 | 2-bit mantissa.
 * exponent field 31: mantissa 0 is +-inf, otherwise NaN. */
static double dec_e5m2(unsigned c)
{
    unsigned s = (c >> 7) & 1u, e = (c >> 2) & 31u, m = c & 3u;
    double v;
    if (e == 31u)
        v = (m == 0u) ? INFINITY : NAN;
    else if (e == 0u)
        v = ldexp((double)m, 1 - 15 - 2);          /* m/4 * 2^-14 */
    else
        v = ldexp((double)(4u + m), (int)e - 15 - 2); /* (1+m/4) * 2^(e-15) */
    if (isnan(v))
        return v;
    return s ? -v : v;
}

/* e2m1 (OCP FP4): sign | 2-bit exponent, bias 1 | 1-bit mantissa.
 * exponent field 0 is subnormal: (m/2) * 2^(1-1); codes above 15 do not
 * exist (NaN here). */
static double dec_e2m1(unsigned c)
{
    if (c > 15u)
        return NAN;
    unsigned s = (c >> 3) & 1u, e = (c >> 1) & 3u, m = c & 1u;
    double v;
    if (e == 0u)
        v = ldexp((double)m, 1 - 1 - 1);            /* m/2 */
    else
        v = ldexp((double)(2u + m), (int)e - 1 - 1); /* (1+m/2) * 2^(e-1) */
    return s ? -v : v;
}

/* e2m3 (OCP FP6): sign | 2-bit exponent, bias 1 | 3-bit mantissa.
 * exponent field 0 is subnormal: (m/8) * 2^(1-1); codes above 63 do not
 * exist (NaN here). */
static double dec_e2m3(unsigned c)
{
    if (c > 63u)
        return NAN;
    unsigned s = (c >> 5) & 1u, e = (c >> 3) & 3u, m = c & 7u;
    double v;
    if (e == 0u)
        v = ldexp((double)m, 1 - 1 - 3);            /* m/8 */
    else
        v = ldexp((double)(8u + m), (int)e - 1 - 3); /* (1+m/8) * 2^(e-1) */
    return s ? -v : v;
}

/* e3m2 (OCP FP6): sign | 3-bit exponent, bias 3 | 2-bit mantissa.
 * exponent field 0 is subnormal: (m/4) * 2^(1-3); codes above 63 do not
 * exist (NaN here). */
static double dec_e3m2(unsigned c)
{
    if (c > 63u)
        return NAN;
    unsigned s = (c >> 5) & 1u, e = (c >> 2) & 7u, m = c & 3u;
    double v;
    if (e == 0u)
        v = ldexp((double)m, 1 - 3 - 2);            /* m/4 * 2^-2 */
    else
        v = ldexp((double)(4u + m), (int)e - 3 - 2); /* (1+m/4) * 2^(e-3) */
    return s ? -v : v;
}

/* e8m0 scale: unsigned biased exponent, 2^(s-127); 255 is NaN. */
static double dec_e8m0(unsigned s)
{
    if (s == 255u)
        return NAN;
    return ldexp(1.0, (int)s - 127);
}

static double TAB[MXREF_NTAB][256];
static pthread_once_t tab_once = PTHREAD_ONCE_INIT;

static void build_tables(void)
{
    for (unsigned c = 0; c < 256u; ++c) {
        TAB[MXREF_FMT_E4M3][c] = dec_e4m3(c);
        TAB[MXREF_FMT_E5M2][c] = dec_e5m2(c);
        TAB[MXREF_FMT_E2M3][c] = dec_e2m3(c);
        TAB[MXREF_FMT_E3M2][c] = dec_e3m2(c);
        TAB[MXREF_FMT_E2M1][c] = dec_e2m1(c);
        TAB[5][c] = TAB[6][c] = TAB[7][c] = NAN; /* no formats 5..7 */
        TAB[MXREF_FMT_E8M0][c] = dec_e8m0(c);
    }
}

static const double *table(int fmt)
{
    pthread_once(&tab_once, build_tables);
    return TAB[fmt];
}

int mxref_version(void) { return 1; }

/* Decoded value of one code: fmt 0 = e4m3, 1 = e5m2, 2 = e2m3 and
 * 3 = e3m2 (codes 0..63), 4 = e2m1 (codes 0..15), 8 = e8m0 scale.  Returns
 * NaN for an unknown format or code. */
double mxref_decode(int fmt, int code)
{
    if (fmt < 0 || fmt >= MXREF_NTAB || (fmt > 4 && fmt != MXREF_FMT_E8M0) || code < 0 ||
        code > 255)
        return NAN;
    return table(fmt)[code];
}

/* Bits per code of an operand format (8, 6 or 4), 0 for an unknown one. */
static int code_bits(int fmt)
{
    switch (fmt) {
    case MXREF_FMT_E4M3:
    case MXREF_FMT_E5M2: return 8;
    case MXREF_FMT_E2M3:
    case MXREF_FMT_E3M2: return 6;
    case MXREF_FMT_E2M1: return 4;
    default: return 0;
    }
}

/* Bytes per operand row of K codes of `bits` bits each. */
static int64_t row_bytes(int64_t K, int bits) { return (K * bits + 7) / 8; }

/* Code k of a row of `bits`-bit codes: bits bits*k .. bits*k+bits-1 of the
 * row read as one little-endian bit string. */
static unsigned code_at(const uint8_t *row, int64_t k, int bits)
{
    if (bits == 8)
        return row[k];
    const int64_t bit = k * bits;
    const unsigned sh = (unsigned)(bit % 8);
    unsigned v = row[bit / 8] >> sh;
    if (sh + (unsigned)bits > 8u)
        v |= (unsigned)row[bit / 8 + 1] << (8u - sh);
    return v & ((1u << bits) - 1u);
}

/* Store code c as code k of a row of `bits`-bit codes (the row must start
 * zeroed: bits are OR-ed in). */
static void put_code(uint8_t *row, int64_t k, int bits, unsigned c)
{
    if (bits == 8) {
        row[k] = (uint8_t)c;
        return;
    }
    const int64_t bit = k * bits;
    const unsigned sh = (unsigned)(bit % 8);
    row[bit / 8] |= (uint8_t)(c << sh);
    if (sh + (unsigned)bits > 8u)
        row[bit / 8 + 1] |= (uint8_t)(c >> (8u - sh));
}

/* fp32 -> bf16 bit pattern, round to nearest, ties to even; NaN stays a
 * (quiet) NaN with its sign; overflow rounds to +-inf as IEEE requires. */
uint16_t mxref_bf16_rne(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

static double bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* ---- the GEMM at a list of output points --------------------------------- */

struct job {
    const uint8_t *A, *As, *B, *Bs;
    const void *Cin;
    int cin_dtype;               /* 0 fp32, 1 bf16 */
    const double *ta, *tb, *te;
    int bitsA, bitsB;            /* bits per code: 8, 6 (packed 4 per 3 bytes) or 4 */
    int64_t ldA, ldB;            /* bytes per operand row */
    int64_t M, N, K, KB;
    const int64_t *rows, *cols;
    int64_t p0, p1;
    double *sum_out, *mag_out;
    float *ref32_out;
    uint16_t *refbf16_out;
};

static void *run_job(void *arg)
{
    const struct job *j = (const struct job *)arg;
    for (int64_t p = j->p0; p < j->p1; ++p) {
        const int64_t m = j->rows[p], n = j->cols[p];
        const uint8_t *a = j->A + m * j->ldA, *b = j->B + n * j->ldB;
        const uint8_t *sa = j->As + m * j->KB, *sb = j->Bs + n * j->KB;
        double s = 0.0, mag = 0.0;
        for (int64_t k = 0; k < j->K; ++k) {
            /* decode(A[m,k]) * 2^(sa-127) and decode(B[k,n]) * 2^(sb-127) */
            const unsigned ca = code_at(a, k, j->bitsA);
            const unsigned cb = code_at(b, k, j->bitsB);
            double av = j->ta[ca] * j->te[sa[k / 32]];
            double bv = j->tb[cb] * j->te[sb[k / 32]];
            double prod = av * bv;
            s += prod;
            mag += fabs(prod);
        }
        if (j->Cin) {
            double c;
            if (j->cin_dtype == 0)
                c = (double)((const float *)j->Cin)[m * j->N + n];
            else
                c = bf16_to_double(((const uint16_t *)j->Cin)[m * j->N + n]);
            s += c;
            mag += fabs(c);
        }
        float r32 = (float)s; /* IEEE round to nearest even */
        if (j->sum_out) j->sum_out[p] = s;
        if (j->mag_out) j->mag_out[p] = mag;
        if (j->ref32_out) j->ref32_out[p] = r32;
        if (j->refbf16_out) j->refbf16_out[p] = mxref_bf16_rne(r32);
    }
    return NULL;
}

/*
 * Compute npts outputs C[rows[p], cols[p]].
 *   A: M*K codes, As: M*KB bytes, B: N*K codes (K-contiguous), Bs: N*KB,
 *   KB = ceil(K/32); fmtA/fmtB: 0 e4m3, 1 e5m2, 2 e2m3, 3 e3m2, 4 e2m1
 *   (a row of sub-byte codes holds ceil(bits*K/8) bytes, packed as
 *   code_at reads them).
 *   Cin: NULL (use_acc off) or the M*N incoming C, fp32 (cin_dtype 0) or
 *   bf16 bits (cin_dtype 1).
 *   Outputs (each may be NULL): sum_out/mag_out the double sum and sum of
 *   |products|; ref32_out the fp32 rounding; refbf16_out its bf16 rounding.
 *   nthreads: number of POSIX threads (>= 1); the result does not depend on it.
 * Returns 0, or -1 on bad arguments.  A thread that cannot be started has
 * its share computed on the calling thread instead.
 */
int mxref_gemm_points(const uint8_t *A, const uint8_t *As, int fmtA,
                      const uint8_t *B, const uint8_t *Bs, int fmtB,
                      const void *Cin, int cin_dtype,
                      int64_t M, int64_t N, int64_t K,
                      const int64_t *rows, const int64_t *cols, int64_t npts,
                      double *sum_out, double *mag_out, float *ref32_out,
                      uint16_t *refbf16_out, int nthreads)
{
    if (!A || !As || !B || !Bs || !rows || !cols || M < 1 || N < 1 || K < 1 ||
        npts < 0 || code_bits(fmtA) == 0 || code_bits(fmtB) == 0 ||
        (Cin && cin_dtype != 0 && cin_dtype != 1))
        return -1;
    for (int64_t p = 0; p < npts; ++p)
        if (rows[p] < 0 || rows[p] >= M || cols[p] < 0 || cols[p] >= N)
            return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > npts)
        nthreads = npts > 0 ? (int)npts : 1;

    struct job base;
    base.A = A; base.As = As; base.B = B; base.Bs = Bs;
    base.Cin = Cin; base.cin_dtype = cin_dtype;
    base.ta = table(fmtA); base.tb = table(fmtB); base.te = table(MXREF_FMT_E8M0);
    base.bitsA = code_bits(fmtA); base.bitsB = code_bits(fmtB);
    base.ldA = row_bytes(K, base.bitsA); base.ldB = row_bytes(K, base.bitsB);
    base.M = M; base.N = N; base.K = K; base.KB = (K + 31) / 32;
    base.rows = rows; base.cols = cols;
    base.sum_out = sum_out; base.mag_out = mag_out;
    base.ref32_out = ref32_out; base.refbf16_out = refbf16_out;

    struct job jobs[256];
    pthread_t tids[256];
    int started[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].p0 = npts * t / nthreads;
        jobs[t].p1 = npts * (t + 1) / nthreads;
        started[t] = 0;
    }
    for (int t = 1; t < nthreads; ++t) {
        started[t] = pthread_create(&tids[t], NULL, run_job, &jobs[t]) == 0;
    }
    run_job(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) {
        if (started[t])
            pthread_join(tids[t], NULL);
        else
            run_job(&jobs[t]); /* still produce every output */
    }
    return 0;
}

/* ---- MX block quantization ------------------------------------------------ */
/*
 * The step that produces the multiply's operands: each row of X is cut into
 * blocks of 32 consecutive K-elements (the last block may be shorter), and
 * every block gets one e8m0 scale byte and 32 codes (the uint8 scale tile
 * whose K extent is BLOCK_K // 32, TLX async-compute page, "TMEM-backed MX
 * Scales").  The pages do not say how the scale is chosen; the reading taken
 * here is the recipe that makes the block's largest magnitude fit the
 * format: with MAX the format's largest finite value (448 for e4m3, 57344
 * for e5m2),
 *   e     = the smallest integer with max|x| <= MAX * 2^e
 *           (an all-zero block takes the smallest scale),
 *   scale = e + 127, clamped to 0..254,
 *   code  = x * 2^(127 - scale) rounded to the nearest value of the format,
 *           ties to the code whose mantissa field is even (round to nearest
 *           even), saturating at +-MAX; the sign is kept (-0 gives 0x80).
 * Written from that definition: the exponent by exact comparisons with
 * ldexp, the rounding by exhaustive search over the format's codes.
 */
static double fmt_max(int fmt)
{
    switch (fmt) {
    case MXREF_FMT_E4M3: return 448.0;
    case MXREF_FMT_E5M2: return 57344.0;
    case MXREF_FMT_E2M3: return 7.5;
    case MXREF_FMT_E3M2: return 28.0;
    default: return 6.0; /* e2m1 */
    }
}

/* Nearest code of `fmt` to v, ties to an even mantissa field (the lowest
 * bit of the code), largest finite magnitude if |v| exceeds it. */
static uint8_t nearest_code(int fmt, double v)
{
    const double *t = table(fmt);
    const double a = fabs(v);
    const int bits = code_bits(fmt);
    const int ncodes = 1 << (bits - 1); /* the non-negative codes: below the sign bit */
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c < ncodes; ++c) {
        if (!isfinite(t[c]))
            continue;
        const double d = fabs(t[c] - a);
        if (d < bd || (d == bd && (c & 1) == 0)) {
            bd = d;
            best = c;
        }
    }
    return (uint8_t)(best | (signbit(v) ? ncodes : 0));
}

/* Smallest integer e with amax <= MAX * 2^e, for finite amax > 0. */
static int block_exponent(int fmt, double amax)
{
    const double mx = fmt_max(fmt);
    int e = (int)floor(log2(amax / mx));
    while (amax > ldexp(mx, e))
        ++e;
    while (amax <= ldexp(mx, e - 1))
        --e;
    return e;
}

/*
 * Quantize the R x K matrix X (row-major; x_dtype 0: fp32, 1: bf16 bit
 * patterns) to codes (R x K) and scales (R x ceil(K/32)) of format fmt
 * (0 e4m3, 1 e5m2, 2 e2m3, 3 e3m2, 4 e2m1; sub-byte codes packed along K as
 * the operands are).  Returns 0; -1 on bad arguments; -2 if X holds a NaN
 * or an infinity (the recipe is defined for finite inputs only).
 */
int mxref_quantize(const void *X, int x_dtype, int64_t R, int64_t K, int fmt, uint8_t *codes,
                   uint8_t *scales)
{
    if (!X || !codes || !scales || R < 1 || K < 1 || (x_dtype != 0 && x_dtype != 1) ||
        code_bits(fmt) == 0)
        return -1;
    const int64_t KB = (K + 31) / 32;
    /* sub-byte codes are packed along K as the operands are (code_at) */
    const int bits = code_bits(fmt);
    const int64_t ldc = row_bytes(K, bits);
    if (bits < 8)
        memset(codes, 0, (size_t)(R * ldc));
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t b = 0; b < KB; ++b) {
            const int64_t k0 = 32 * b, k1 = k0 + 32 < K ? k0 + 32 : K;
            double x[32];
            double amax = 0.0;
            for (int64_t k = k0; k < k1; ++k) {
                const int64_t i = r * K + k;
                x[k - k0] = x_dtype == 0 ? (double)((const float *)X)[i]
                                         : bf16_to_double(((const uint16_t *)X)[i]);
                if (!isfinite(x[k - k0]))
                    return -2;
                if (fabs(x[k - k0]) > amax)
                    amax = fabs(x[k - k0]);
            }
            int s = 0;
            if (amax > 0.0) {
                s = block_exponent(fmt, amax) + 127;
                s = s < 0 ? 0 : (s > 254 ? 254 : s);
            }
            scales[r * KB + b] = (uint8_t)s;
            for (int64_t k = k0; k < k1; ++k) {
                const uint8_t c = nearest_code(fmt, ldexp(x[k - k0], 127 - s));
                put_code(codes + r * ldc, k, bits, c);
            }
        }
    }
    return 0;
}
