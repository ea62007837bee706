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
#define MXREF_FMT_E8M0 2

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

/* e8m0 scale: unsigned biased exponent, 2^(s-127); 255 is NaN. */
static double dec_e8m0(unsigned s)
{
    if (s == 255u)
        return NAN;
    return ldexp(1.0, (int)s - 127);
}

static double TAB[3][256];
static pthread_once_t tab_once = PTHREAD_ONCE_INIT;

static void build_tables(void)
{
    for (unsigned c = 0; c < 256u; ++c) {
        TAB[MXREF_FMT_E4M3][c] = dec_e4m3(c);
        TAB[MXREF_FMT_E5M2][c] = dec_e5m2(c);
        TAB[MXREF_FMT_E8M0][c] = dec_e8m0(c);
    }
}

static const double *table(int fmt)
{
    pthread_once(&tab_once, build_tables);
    return TAB[fmt];
}

int mxref_version(void) { return 1; }

/* Decoded value of one code: fmt 0 = e4m3, 1 = e5m2, 2 = e8m0 scale.
 * Returns NaN for an unknown format. */
double mxref_decode(int fmt, int code)
{
    if (fmt < 0 || fmt > 2 || code < 0 || code > 255)
        return NAN;
    return table(fmt)[code];
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
        const uint8_t *a = j->A + m * j->K, *b = j->B + n * j->K;
        const uint8_t *sa = j->As + m * j->KB, *sb = j->Bs + n * j->KB;
        double s = 0.0, mag = 0.0;
        for (int64_t k = 0; k < j->K; ++k) {
            /* decode(A[m,k]) * 2^(sa-127) and decode(B[k,n]) * 2^(sb-127) */
            double av = j->ta[a[k]] * j->te[sa[k / 32]];
            double bv = j->tb[b[k]] * j->te[sb[k / 32]];
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
 *   KB = ceil(K/32); fmtA/fmtB: 0 e4m3, 1 e5m2.
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
        npts < 0 || (fmtA != 0 && fmtA != 1) || (fmtB != 0 && fmtB != 1) ||
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
