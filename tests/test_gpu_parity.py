"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Exact cases (bitwise): permutation and pairwise-product probes, the
integer matrix product and the scale-doubling invariant.  Random cases:
the agreement rule in gpu_helpers (1e-5 * sum|ab|, plus one bf16 ulp for
bf16 output), on full outputs at sizes the oracle finishes in seconds
(several tiles plus ragged tails) and on 65,536 sampled outputs plus the
edge tiles at the five named workload sizes, in the launch configuration
the benchmark times.
"""
import numpy as np
import pytest
import torch

import level_dsl_amd as L
import mxinputs as mi
import oracle
from gpu_helpers import (alloc_c, c_numpy, compare, compare_native, log, native_group_extra,
                         oracle_full, oracle_points, run, to_dev)

pytestmark = pytest.mark.gpu

LARGE, SKINNY, AUTO = L.MXGEMM_VARIANT_LARGE, L.MXGEMM_VARIANT_SKINNY, L.MXGEMM_VARIANT_AUTO
LARGE_NATIVE, SKINNY_NATIVE = L.MXGEMM_VARIANT_LARGE_NATIVE, L.MXGEMM_VARIANT_SKINNY_NATIVE
ALL_VARIANTS = [LARGE, SKINNY, LARGE_NATIVE, SKINNY_NATIVE]
VNAME = {AUTO: "auto", LARGE: "large", SKINNY: "skinny", LARGE_NATIVE: "large_native",
         SKINNY_NATIVE: "skinny_native"}


@pytest.fixture(scope="module")
def gemm():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    g = L.Gemm()
    yield g
    g.close()


def _variants_for(M, native=False):
    v = [LARGE, SKINNY] if M <= 64 else [LARGE]
    if native:
        v += [LARGE_NATIVE, SKINNY_NATIVE] if M <= 64 else [LARGE_NATIVE]
    return v


def _is_skinny(v):
    return v in (SKINNY, SKINNY_NATIVE)


# ------------------------------------------------------------ exact probes --

@pytest.mark.parametrize("variant", ALL_VARIANTS, ids=lambda v: VNAME[v])
@pytest.mark.parametrize("which", ["A", "B"])
def test_permutation_probe_exact(gemm, variant, which):
    """One 1.0 per row of A (or of B): every output is a single scaled
    element of the other operand, so the result is exact; a wrong fragment,
    lane or scale mapping shows up as a wrong source element."""
    M = 64 if _is_skinny(variant) else 320
    N, K = 288, 512
    g = np.random.Generator(np.random.PCG64(21))
    p = mi.random_problem(M, N, K, seed=31, fmtA=0, fmtB=1, scale_lo=100, scale_hi=150)
    if which == "A":
        pi = np.array([g.integers(0, K) for _ in range(M)])
        p.A[:] = 0
        p.A[np.arange(M), pi] = 0x38
    else:
        sg = np.array([g.integers(0, K) for _ in range(N)])
        p.B[:] = 0
        p.B[np.arange(N), sg] = 0x38
    log(f"permutation probe {which} variant={variant} M={M} N={N} K={K}")
    got = run(gemm, p, variant)
    ref = oracle_full(p)
    assert np.array_equal(got, ref["ref32"]), f"{np.sum(got != ref['ref32'])} mismatches"


# scale-byte pairs: the middle, the edges of the e4m3 window (10..246) and of
# the e5m2 window (17..239), bytes outside both, 0 (2^-127), 254 (2^127),
# skewed pairs whose product is moderate, pairs that overflow or underflow
# fp32, and 255 (NaN)
PAIR_SCALES = [(127, 127), (10, 239), (140, 100), (1, 254), (0, 254), (254, 0), (0, 0),
               (254, 254), (2, 3), (9, 17), (16, 238), (247, 5), (240, 240), (246, 10),
               (255, 127), (127, 255)]


@pytest.mark.parametrize("variant", ALL_VARIANTS, ids=lambda v: VNAME[v])
@pytest.mark.parametrize("fa,fb", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("sa,sb", PAIR_SCALES, ids=lambda x: str(x))
def test_pairwise_products_exact(gemm, variant, fa, fb, sa, sb):
    """A[m,0] = code m, B[0,n] = code n (finite codes only), all else zero:
    C[m,n] = dec(m) dec(n) 2^(sa+sb-254) exactly, for every pair and every
    scale byte.  Results in the fp32 normal range (and infinities) must be
    bit-identical to the oracle's, zeros must be zero, NaN (scale byte 255)
    must be NaN; fp32-subnormal results are not graded.  Small-M variants run
    the 256 rows as four calls of 64."""
    M = N = 256
    K = 32
    tab = {f: oracle.decode_table(f) for f in (0, 1)}
    A = np.zeros((M, K), np.uint8)
    B = np.zeros((N, K), np.uint8)
    ca = np.arange(256, dtype=np.uint8)
    ca[~np.isfinite(tab[fa])] = 0
    cb = np.arange(256, dtype=np.uint8)
    cb[~np.isfinite(tab[fb])] = 0
    A[:, 0] = ca
    B[:, 0] = cb
    p = mi.Problem(M, N, K, fa, fb, A, np.full((M, 1), sa, np.uint8), B,
                   np.full((N, 1), sb, np.uint8), mi.OUT_F32, False)
    log(f"pairwise fa={fa} fb={fb} sa={sa} sb={sb} variant={VNAME[variant]}")
    if _is_skinny(variant):
        parts = []
        for r0 in range(0, M, 64):
            q = mi.Problem(64, N, K, fa, fb, A[r0:r0 + 64].copy(), p.As[r0:r0 + 64].copy(), B,
                           p.Bs, mi.OUT_F32, False)
            parts.append(run(gemm, q, variant))
        got = np.concatenate(parts)
    else:
        got = run(gemm, p, variant)
    ref = oracle_full(p)
    r = ref["ref32"]
    assert np.array_equal(np.isnan(got), np.isnan(r)), \
        f"NaN pattern differs: {np.isnan(got).sum()} vs {np.isnan(r).sum()}"
    graded = ~np.isnan(r) & (np.abs(r) >= np.float32(2.0**-126))  # normal or inf
    assert np.array_equal(got[graded], r[graded]), f"{np.sum(got[graded] != r[graded])} mismatches"
    zero = r == 0
    assert np.all(got[zero] == 0)


def _extreme_problem(M, N, K, fa, fb, seed, normal_rows, normal_cols, out=mi.OUT_F32, acc=False):
    """Scale bytes outside the decode windows, with every product moderate.
    Even 32-K blocks carry the 'normal' rows and columns (scales U{120..134});
    odd blocks carry the others, whose scales sit outside the windows with
    the A and B bytes of a block summing to about 254 (blocks 1 mod 4: A low,
    B high; 3 mod 4: A high, B low).  A row's codes are zero in the blocks of
    the other kind, and normal rows keep byte 127 there, so normal x normal
    outputs see only in-window bytes, other x other outputs only extreme ones,
    and mixed outputs are exactly zero."""
    p = mi.random_problem(M, N, K, seed=seed, fmtA=fa, fmtB=fb, out_dtype=out, use_acc=acc)
    g = np.random.Generator(np.random.PCG64(seed + 17))
    lo = {0: (0, 9), 1: (0, 16)}
    hi = {0: (247, 254), 1: (240, 254)}
    kb = K // 32
    ra = np.arange(M) < normal_rows
    cb = np.arange(N) < normal_cols
    for b in range(kb):
        rows_k = slice(32 * b, 32 * b + 32)
        if b % 2 == 0:
            p.A[~ra, rows_k] = 0
            p.B[~cb, rows_k] = 0
            continue
        p.A[ra, rows_k] = 0
        p.B[cb, rows_k] = 0
        p.As[ra, b] = 127
        p.Bs[cb, b] = 127
        (al, ah), (bl, bh) = (lo[fa], hi[fb]) if b % 4 == 1 else (hi[fa], lo[fb])
        p.As[~ra, b] = g.integers(al, ah + 1, size=(~ra).sum())
        p.Bs[~cb, b] = g.integers(bl, bh + 1, size=(~cb).sum())
    return p


EXTREME_CASES = [
    # M, N, K, fmtA, fmtB, normal rows, normal cols, out, use_acc
    (300, 280, 1024, 0, 0, 128, 128, mi.OUT_F32, False),   # 16-byte scale windows
    (300, 280, 1056, 0, 0, 128, 128, mi.OUT_F32, False),   # a partial last scale dword
    (270, 260, 512, 1, 0, 200, 64, mi.OUT_BF16, False),
    (256, 300, 640, 1, 1, 0, 0, mi.OUT_F32, True),         # every wave on the fallback
    (64, 300, 1024, 0, 1, 32, 200, mi.OUT_F32, False),
    (40, 520, 1056, 1, 0, 40, 100, mi.OUT_BF16, True),
]


@pytest.mark.parametrize("case", EXTREME_CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"_f{c[3]}{c[4]}")
def test_extreme_scales(gemm, case):
    """Scale bytes outside the bf16 decode windows (0..9 and 247..254 for
    e4m3, 0..16 and 240..254 for e5m2) in some waves of a launch: those waves
    recompute on the fallback path, the others keep the fast loop; every
    output meets the agreement rule, with and without split K."""
    M, N, K, fa, fb, nr, nc, out, acc = case
    p = _extreme_problem(M, N, K, fa, fb, seed=M + N + K + fa, normal_rows=nr, normal_cols=nc,
                         out=out, acc=acc)
    ref = oracle_full(p)
    dev = to_dev(p)
    gemm.enable_split_k()
    try:
        for v in _variants_for(M) + [AUTO]:
            for splits in (1, 2):
                gemm.set_splits(splits)
                log(f"extreme {case} variant={VNAME[v]} splits={splits}")
                got = run(gemm, p, v, guard=64, dev_inputs=dev)
                compare(got, ref, out, f"extreme {case} {VNAME[v]} splits={splits}")
    finally:
        gemm.set_splits(0)
        gemm.disable_split_k()


def test_quantized_tiny_blocks(gemm):
    """A quantized operand whose blocks are tiny gets scale byte 0 (2^-127)
    from the quantizer; multiplying it with an operand of large scales
    (moderate products) matches the oracle."""
    g = np.random.Generator(np.random.PCG64(404))
    M, N, K = 96, 160, 512
    X = (g.standard_normal((M, K)) * 1e-39).astype(np.float32)
    X[:, :32] = g.standard_normal((M, 32)).astype(np.float32)  # one ordinary block per row
    xd = torch.from_numpy(X).to("cuda:0")
    codes, scales = gemm.quantize(xd, L.MXGEMM_FMT_E4M3)
    torch.cuda.synchronize()
    As = scales.cpu().numpy()
    assert (As[:, 1:] <= 2).all() and (As[:, 1:] == 0).any(), "expected scale bytes at the bottom"
    p = mi.random_problem(M, N, K, seed=405, scale_lo=230, scale_hi=254)
    p.A = codes.cpu().numpy()
    p.As = As
    p.Bs[:, 0] = 127
    ref = oracle_full(p)
    for v in (LARGE, AUTO):
        log(f"quantized tiny blocks variant={VNAME[v]}")
        compare(run(gemm, p, v), ref, mi.OUT_F32, f"quantized tiny blocks {VNAME[v]}")


@pytest.mark.parametrize("M,N,K", [(300, 260, 544), (64, 200, 1024), (1, 5, 32)])
def test_integer_gemm_bitexact(gemm, M, N, K):
    """Integer-valued codes with unit scales: every partial sum is an integer
    below 2^24, so the GPU result is the exact integer product, bit for bit."""
    g = np.random.Generator(np.random.PCG64(M * 7 + N))
    ia = g.integers(-16, 17, size=(M, K))
    ib = g.integers(-8, 9, size=(N, K))
    A = mi.quantize(ia.astype(np.float32), 0)
    B = mi.quantize(ib.astype(np.float32), 1)
    p = mi.Problem(M, N, K, 0, 1, A, np.full((M, K // 32), 127, np.uint8), B,
                   np.full((N, K // 32), 127, np.uint8), mi.OUT_F32, False)
    want = (ia @ ib.T).astype(np.float32)
    for v in _variants_for(M, native=True):
        log(f"integer gemm M={M} N={N} K={K} variant={v}")
        got = run(gemm, p, v)
        assert np.array_equal(got, want), f"variant {v}: {np.sum(got != want)} mismatches"


@pytest.mark.parametrize("M", [200, 48])
def test_scale_doubling_bitexact(gemm, M):
    """Raising every scale byte of A row m by one doubles row m exactly and
    leaves the other rows bit-identical (same kernel, same order)."""
    N, K = 136, 640
    p = mi.random_problem(M, N, K, seed=41)
    for v in _variants_for(M, native=True):
        log(f"scale doubling M={M} variant={v}")
        base = run(gemm, p, v)
        q = mi.Problem(**{**p.__dict__})
        q.As = p.As.copy()
        q.As[M // 2, :] += 1
        q.Bs = p.Bs.copy()
        q.Bs[N - 1, :] += 1
        got = run(gemm, q, v)
        rows = np.ones(M, bool)
        rows[M // 2] = False
        cols = np.ones(N, bool)
        cols[N - 1] = False
        assert np.array_equal(got[M // 2, :-1], 2 * base[M // 2, :-1])
        assert np.array_equal(got[:, N - 1][rows], 2 * base[:, N - 1][rows])
        assert got[M // 2, N - 1] == 4 * base[M // 2, N - 1]
        assert np.array_equal(got[np.ix_(rows, cols)], base[np.ix_(rows, cols)])


# --------------------------------------------------- random, full outputs --

RANDOM_CASES = [
    # M, N, K, fmtA, fmtB, out, use_acc
    (256, 256, 256, 0, 0, mi.OUT_F32, False),
    (517, 389, 1056, 0, 0, mi.OUT_F32, False),   # ragged M/N, N % 4 != 0, K % 128 != 0
    (300, 512, 640, 1, 0, mi.OUT_BF16, False),
    (1, 1, 32, 0, 0, mi.OUT_F32, False),
    (7, 9, 64, 1, 1, mi.OUT_F32, False),
    (130, 260, 384, 0, 1, mi.OUT_F32, True),
    (257, 255, 512, 1, 1, mi.OUT_BF16, True),
    (512, 768, 2048, 0, 0, mi.OUT_BF16, False),
    (64, 448, 1024, 0, 0, mi.OUT_F32, False),
    (1, 113, 96, 0, 0, mi.OUT_F32, False),
    (33, 300, 2048, 1, 0, mi.OUT_BF16, True),
    (64, 1000, 4128, 0, 0, mi.OUT_F32, False),
    (17, 1234, 160, 1, 0, mi.OUT_F32, True),
    # bf16 output with N % 8 == 0 (16-byte stores of 8 bf16), with and without use_acc
    (300, 520, 1024, 0, 0, mi.OUT_BF16, True),
    (64, 448, 1024, 1, 0, mi.OUT_BF16, True),
    (20, 1000, 512, 0, 1, mi.OUT_BF16, False),
]


@pytest.mark.parametrize("case", RANDOM_CASES, ids=lambda c: "x".join(map(str, c[:3])) +
                         f"_f{c[3]}{c[4]}_o{c[5]}_acc{int(c[6])}")
def test_random_full(gemm, case):
    M, N, K, fa, fb, out, acc = case
    p = mi.random_problem(M, N, K, seed=M * 131 + N * 7 + K, fmtA=fa, fmtB=fb, out_dtype=out,
                          use_acc=acc)
    ref = oracle_full(p)
    for v in _variants_for(M) + [AUTO]:
        log(f"random full {case} variant={v}")
        got = run(gemm, p, v, guard=64)
        compare(got, ref, out, f"{case} variant {v}")


def test_deterministic(gemm):
    p = mi.random_problem(333, 444, 1536, seed=9, out_dtype=mi.OUT_BF16)
    for v in (LARGE, LARGE_NATIVE):
        log(f"determinism variant={v}")
        a = run(gemm, p, v)
        b = run(gemm, p, v)
        assert np.array_equal(a, b)
    q = mi.random_problem(40, 700, 1536, seed=10)
    for v in (SKINNY, SKINNY_NATIVE):
        log(f"determinism {VNAME[v]}")
        assert np.array_equal(run(gemm, q, v), run(gemm, q, v))


NATIVE_CASES = [(256, 256, 256, 0, 0, mi.OUT_F32, False), (517, 389, 1056, 1, 0, mi.OUT_F32, True),
                (64, 448, 1024, 0, 1, mi.OUT_BF16, False), (33, 300, 2048, 1, 1, mi.OUT_F32, True),
                (16, 120, 24576, 0, 0, mi.OUT_F32, False)]  # small-M scales without the LDS table


@pytest.mark.parametrize("case", NATIVE_CASES, ids=lambda c: "x".join(map(str, c[:3])))
def test_native_within_group_window_bound(gemm, case):
    """The native variants sum each aligned group of 8 products in a window
    reaching 13 bits below the group's largest product (measured on the
    device).  Bound checked here: |err| <= 1e-5 * sum|ab| + 8 * sum_g
    2^(E_g - 13), E_g = floor(log2 max_{k in g} |a_k b_k|)."""
    M, N, K, fa, fb, out, acc = case
    p = mi.random_problem(M, N, K, seed=M + N + K, fmtA=fa, fmtB=fb, out_dtype=out, use_acc=acc)
    ref = oracle_full(p)
    extra = native_group_extra(p)
    for v in ([LARGE_NATIVE, SKINNY_NATIVE] if M <= 64 else [LARGE_NATIVE]):
        log(f"native bound {case} variant={VNAME[v]}")
        got = run(gemm, p, v)
        compare_native(got, ref, out, extra, f"native {case} {VNAME[v]}")


# ------------------------------------------------ the five named workloads --

def _workload_check(gemm, wid, full: bool):
    p = mi.workload(wid)
    log(f"workload {wid} ({p.name}) generated")
    dev = to_dev(p)
    buf, c = alloc_c(p)
    gemm.set_variant(AUTO)
    log(f"workload {wid} run")
    gemm(*dev[:2], p.fmtA, *dev[2:], p.fmtB, c, use_acc=p.use_acc, out_dtype=p.out_dtype)
    torch.cuda.synchronize()
    log(f"workload {wid} done on GPU")
    if full:
        got = c_numpy(c, p.out_dtype)
        ref = oracle_full(p)
        compare(got, ref, p.out_dtype, p.name)
        return
    rows, cols = mi.sample_points(p.M, p.N, 65536, seed=wid)
    ref = oracle_points(p, rows, cols)
    got = c_numpy(c, p.out_dtype)[rows, cols]
    compare(got, ref, p.out_dtype, p.name)


def test_workload_256cube_full(gemm):
    _workload_check(gemm, 0, full=True)


def test_workload_4096cube_sampled(gemm):
    _workload_check(gemm, 1, full=False)


def test_workload_8192cube_bf16_sampled(gemm):
    _workload_check(gemm, 2, full=False)


def test_workload_skinny_m64_sampled(gemm):
    _workload_check(gemm, 3, full=False)


def test_workload_16384cube_acc_sampled(gemm):
    _workload_check(gemm, 4, full=False)


# ------------------------------------------------------------- edge cases --

EDGE_CASES = [
    # M, N, K, fmtA, fmtB, out, use_acc
    (37, 250, 20576, 0, 0, mi.OUT_F32, False),   # 161 K stages: three scale chunks, a ragged last stage
    (64, 224, 16384, 1, 1, mi.OUT_BF16, True),   # two full scale chunks, e5m2 x e5m2, bf16 accumulate
    (96, 130, 9248, 0, 1, mi.OUT_F32, False),    # K % 128 == 32: per-byte scale path of the large kernel
    (2, 3, 1 << 21, 0, 0, mi.OUT_F32, False),    # the largest K (16384 stages)
    (3, 1 << 20, 64, 0, 0, mi.OUT_F32, False),   # the largest N (9363 small-M workgroups)
    (70000, 40, 64, 1, 0, mi.OUT_BF16, False),   # many row tiles, ragged last tile
]


@pytest.mark.parametrize("case", EDGE_CASES, ids=lambda c: "x".join(map(str, c[:3])))
def test_edge_full(gemm, case):
    M, N, K, fa, fb, out, acc = case
    p = mi.random_problem(M, N, K, seed=(M * 7 + N * 3 + K) % 100003, fmtA=fa, fmtB=fb,
                          out_dtype=out, use_acc=acc)
    ref = oracle_full(p)
    dev = to_dev(p)
    for v in _variants_for(M):
        log(f"edge {case} variant={VNAME[v]}")
        got = run(gemm, p, v, guard=64, dev_inputs=dev)
        compare(got, ref, out, f"edge {case} variant {VNAME[v]}")


def test_invalid_call_launches_nothing(gemm):
    """Every rejected call returns its status and leaves C untouched."""
    p = mi.random_problem(64, 64, 128, seed=5)
    A, As, B, Bs = to_dev(p)
    buf, c = alloc_c(p)  # NaN-filled
    h = gemm.h
    bad = [
        (dict(M=0), "MXGEMM_ERR_SHAPE"), (dict(K=48), "MXGEMM_ERR_SHAPE"),
        (dict(fmtA=5), "MXGEMM_ERR_FMT"), (dict(fmtB=9), "MXGEMM_ERR_FMT"),
        (dict(out_dtype=7), "MXGEMM_ERR_DTYPE"),
        (dict(C=c.data_ptr() + 4), "MXGEMM_ERR_ALIGN"), (dict(C=A.data_ptr()), "MXGEMM_ERR_ALIAS"),
    ]
    for kw, status in bad:
        args = dict(A=A, A_scale=As, fmtA=0, B=B, B_scale=Bs, fmtB=0, C=c, M=64, N=64, K=128,
                    use_acc=0, out_dtype=0)
        args.update(kw)
        with pytest.raises(L.MxgemmError) as e:
            L.mxgemm_run(h, **args)
        assert e.value.code == L.STATUS_CODE[status], kw
    q = mi.random_problem(65, 8, 32, seed=6)
    qA, qAs, qB, qBs = to_dev(q)
    qbuf, qc = alloc_c(q)
    gemm.set_variant(SKINNY)
    with pytest.raises(L.MxgemmError) as e:  # a forced small-M variant with M > 64
        L.mxgemm_run(h, qA, qAs, 0, qB, qBs, 0, qc, 65, 8, 32, 0, 0)
    assert e.value.code == L.STATUS_CODE["MXGEMM_ERR_VARIANT"]
    gemm.set_variant(AUTO)
    torch.cuda.synchronize()
    assert bool(torch.isnan(buf).all()) and bool(torch.isnan(qbuf).all()), "a rejected call wrote C"


# ------------------------------------------------ non-finite codes, scales --

@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 1), (1, 0)])
def test_nonfinite_pattern(gemm, fa, fb):
    """NaN and infinity codes and NaN scale bytes (255) are outside every
    workload; the exact variants still put NaN and +-inf exactly where the
    oracle's IEEE arithmetic does (the decode turns them into bf16 NaN/inf,
    which the bf16 MFMA propagates), and the finite outputs of the same
    problem meet the usual tolerance."""
    p = mi.random_problem(70, 72, 256, seed=77 + fa * 2 + fb, fmtA=fa, fmtB=fb)
    nan_a = 0x7F if fa == 0 else 0x7E
    p.A[3, 5] = nan_a                 # NaN code in row 3
    p.As[10, 2] = 255                 # NaN scale for row 10, block 2
    p.A[20, 64:96] = 0x38             # row 20, block 2: all +1.0 ...
    p.As[20, 2] = 255                 # ... with a NaN scale: NaN, not +inf
    p.Bs[50, 5] = 255                 # NaN scale for column 50, block 5
    if fb == 1:
        p.B[7, 40] = 0x7C             # +inf in column 7
        p.B[8, 41] = 0xFC             # -inf in column 8
    ref = oracle_full(p)
    for v in _variants_for(p.M):
        got = run(gemm, p, v)
        r = ref["ref32"]
        assert np.array_equal(np.isnan(got), np.isnan(r)), \
            f"NaN pattern differs ({VNAME[v]}): {np.isnan(got).sum()} vs {np.isnan(r).sum()}"
        fin = np.isfinite(r)
        inf = np.isinf(r)
        assert np.array_equal(got[inf], r[inf]), f"infinities differ ({VNAME[v]})"
        compare(got[fin], {k: a[fin] for k, a in ref.items()}, mi.OUT_F32, f"finite part {VNAME[v]}")


BF16_RNE_CASES = [
    # M, N, K, fmtA, fmtB, variants
    (300, 520, 1024, 0, 0, (LARGE, LARGE_NATIVE)),          # N % 8 == 0: 16-byte bf16 stores; scale windows
    (300, 516, 1056, 1, 0, (LARGE, LARGE_NATIVE)),          # N % 8 != 0: 8-byte stores; per-stage scales
    (48, 520, 1024, 0, 1, (SKINNY, SKINNY_NATIVE, LARGE)),  # the small-M kernels
    (300, 520, 1024, 4, 4, (AUTO,)),                        # e2m1 on the 256 x 256 kernel
    (300, 520, 1024, 2, 2, (AUTO,)),                        # e2m3
    (300, 520, 1024, 3, 0, (AUTO, LARGE_NATIVE)),           # e3m2 x e4m3: widened, then fp8
    (48, 516, 1024, 0, 4, (SKINNY, SKINNY_NATIVE)),         # e4m3 x e2m1: widened B, small-M kernels
]


@pytest.mark.parametrize("case", BF16_RNE_CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"_f{c[3]}{c[4]}")
def test_bf16_output_is_rne_of_f32_output(gemm, case):
    """bf16 output is bit for bit the f32 output of the same call rounded to
    nearest even (the sums are the same; the bf16 epilogue's lane-half
    exchange and pairwise packing must leave every value in its place,
    rounded once)."""
    M, N, K, fa, fb, variants = case
    seed = 4400 + M + N + K + fa
    p32 = mi.random_problem(M, N, K, seed=seed, fmtA=fa, fmtB=fb, out_dtype=mi.OUT_F32)
    p16 = mi.random_problem(M, N, K, seed=seed, fmtA=fa, fmtB=fb, out_dtype=mi.OUT_BF16)
    dev = to_dev(p32)
    for v in variants:
        log(f"bf16 = RNE(f32) {case[:5]} variant={VNAME[v]}")
        c32 = run(gemm, p32, v, guard=64, dev_inputs=dev)
        c16 = run(gemm, p16, v, guard=64, dev_inputs=dev)
        assert np.isfinite(c32).all()
        want = torch.from_numpy(c32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        bad = np.flatnonzero(c16 != want)
        assert bad.size == 0, (f"{case[:5]} variant {VNAME[v]}: {bad.size} bf16 outputs differ from "
                               f"RNE of the f32 output, e.g. flat index {bad[:5]}")
    gemm.set_variant(AUTO)
