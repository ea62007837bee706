"""GPU parity of e2m3 (FP6) operands, four codes per three bytes along K,
against the CPU oracle.

e2m3 x e2m3 runs on the scaled MFMA of both kernels (every product of a
32-element block, 2^-6 .. 56.25, fits the instruction's 8-product window,
so the sum is exact up to the fp32 accumulation) and is held to the same
agreement rule as the exact variants:
  * one-hot rows (a single 1.0 per row of A, or of B): every output names
    its source element, which pins the 6-bit operand layout (bit order
    inside a block, lane halves, blocks of a step) of both kernels;
  * every pair of the 64 codes at several scale pairs, 0, 254 and 255
    included, bit for bit;
  * random problems on full outputs: ragged M, N and K (a partial last
    stage), use_acc, bf16 output, every small-M tile count, and both
    kernels;
  * split-K, forced, on both kernels;
  * the 8192 x 8192 x 8192 shape on sampled outputs;
  * e2m3 beside another format, and e3m2, rejected without an operand
    buffer (they run widened; tests/test_gpu_widen.py).
"""
import numpy as np
import pytest
import torch

import level_dsl_amd as L
import mxinputs as mi
from gpu_helpers import compare, log, oracle_full, oracle_points, run, to_dev, alloc_c, c_numpy

pytestmark = pytest.mark.gpu

E2M3 = L.MXGEMM_FMT_E2M3
AUTO, LARGE, LARGE_NATIVE = L.MXGEMM_VARIANT_AUTO, L.MXGEMM_VARIANT_LARGE, L.MXGEMM_VARIANT_LARGE_NATIVE
SKINNY, SKINNY_NATIVE = L.MXGEMM_VARIANT_SKINNY, L.MXGEMM_VARIANT_SKINNY_NATIVE
ONE = 8  # the e2m3 code of 1.0 (exponent field 1, mantissa 0)


@pytest.fixture(scope="module")
def gemm():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    g = L.Gemm()
    yield g
    g.close()


def _variants(M):
    return (AUTO, LARGE) + ((SKINNY,) if M <= 64 else ())


@pytest.mark.parametrize("which", ["A", "B"])
@pytest.mark.parametrize("M", [320, 64, 16])
def test_fp6_one_hot_rows(gemm, which, M):
    """A single 1.0 per row of A (or of B) at a random K: every output is one
    scaled element of the other operand, exactly."""
    N, K = 288, 512
    g = np.random.Generator(np.random.PCG64(1300 + M))
    p = mi.random_problem(M, N, K, seed=1310 + M, fmtA=E2M3, fmtB=E2M3, scale_lo=100,
                          scale_hi=150, sigma=2.0)
    if which == "A":
        codes = np.zeros((M, K), np.uint8)
        codes[np.arange(M), g.integers(0, K, size=M)] = ONE
        p.A = mi.pack_bits(codes, 6)
    else:
        codes = np.zeros((N, K), np.uint8)
        codes[np.arange(N), g.integers(0, K, size=N)] = ONE
        p.B = mi.pack_bits(codes, 6)
    ref = oracle_full(p)["ref32"]
    for v in _variants(M):
        log(f"fp6 one-hot {which} M={M} variant={v}")
        got = run(gemm, p, v)
        assert np.array_equal(got, ref), f"variant {v}: {np.sum(got != ref)} mismatches"
    gemm.set_variant(AUTO)


@pytest.mark.parametrize("sa,sb", [(127, 127), (100, 150), (1, 254), (0, 254), (254, 0), (255, 127)])
def test_fp6_pairwise_products_exact(gemm, sa, sb):
    """A[m, 0] = code m, B[n, 0] = code n (64 x 64 codes, K = 32): every
    C[m, n] is dec(m) dec(n) 2^(sa+sb-254); fp32-normal results and zeros
    bit for bit, NaN where a scale byte is 255."""
    M = N = 64
    K = 32
    a = np.zeros((M, K), np.uint8)
    b = np.zeros((N, K), np.uint8)
    a[:, 0] = np.arange(64)
    b[:, 0] = np.arange(64)
    p = mi.Problem(M, N, K, E2M3, E2M3, mi.pack_bits(a, 6), np.full((M, 1), sa, np.uint8),
                   mi.pack_bits(b, 6), np.full((N, 1), sb, np.uint8), mi.OUT_F32, False)
    ref = oracle_full(p)["ref32"]
    for v in (LARGE, SKINNY):
        log(f"fp6 pairwise sa={sa} sb={sb} variant={v}")
        got = run(gemm, p, v)
        assert np.array_equal(np.isnan(got), np.isnan(ref))
        graded = ~np.isnan(ref) & ((np.abs(ref) >= np.float32(2.0**-126)) | (ref == 0))
        assert np.array_equal(got[graded], ref[graded]), f"{np.sum(got[graded] != ref[graded])} mismatches"
    gemm.set_variant(AUTO)


FP6_CASES = [
    # M, N, K, use_acc, out
    (300, 260, 4096, False, mi.OUT_F32),
    (257, 300, 2048, True, mi.OUT_BF16),
    (129, 513, 1056, False, mi.OUT_F32),     # 33 blocks: a partial last stage
    (64, 200, 8192, True, mi.OUT_F32),
    (1, 5, 32, False, mi.OUT_F32),
    (517, 389, 1120, True, mi.OUT_BF16),
    (33, 1000, 640, False, mi.OUT_BF16),
    (16, 120, 24576, False, mi.OUT_F32),     # M <= 64 with K too long for the LDS scale table
    (20, 333, 2080, True, mi.OUT_BF16),      # two 16-row tiles of A on the small-M kernel
    (48, 250, 4096, False, mi.OUT_F32),      # three
    (96, 700, 3072, False, mi.OUT_F32),      # AUTO: two small-M launches
]


@pytest.mark.parametrize("M,N,K,acc,out", FP6_CASES, ids=lambda c: str(c))
def test_fp6_random_full(gemm, M, N, K, acc, out):
    p = mi.random_problem(M, N, K, seed=1400 + M + K, fmtA=E2M3, fmtB=E2M3, out_dtype=out,
                          use_acc=acc)
    ref = oracle_full(p)
    dev = to_dev(p)
    for v in _variants(M) + ((LARGE_NATIVE, SKINNY_NATIVE) if M <= 64 else (LARGE_NATIVE,)):
        log(f"fp6 random M={M} N={N} K={K} use_acc={acc} out={out} variant={v}")
        got = run(gemm, p, v, guard=64, dev_inputs=dev)
        compare(got, ref, out, f"fp6 {M}x{N}x{K} variant {v}")
    gemm.set_variant(AUTO)


@pytest.mark.parametrize("M,N,K,S", [(300, 260, 4096, 2), (512, 512, 2048, 3), (40, 700, 4096, 5),
                                     (64, 3584, 8192, 0)])
def test_fp6_split_k(M, N, K, S):
    """Split K, forced (S >= 2) or automatic (S = 0), through a workspace:
    within the rule and equal to the unsplit result within it."""
    p = mi.random_problem(M, N, K, seed=1500 + S + M, fmtA=E2M3, fmtB=E2M3,
                          out_dtype=mi.OUT_BF16, use_acc=True)
    rows, cols = mi.sample_points(M, N, 8192, seed=S, edge=64)
    ref = oracle_points(p, rows, cols)
    g = L.Gemm()
    g.enable_split_k()
    try:
        g.set_splits(S)
        log(f"fp6 split M={M} N={N} K={K} S={S}")
        got = run(g, p, AUTO)
        compare(got[rows, cols], ref, p.out_dtype, f"fp6 split S={S}")
    finally:
        g.close()


def test_fp6_8192cube_sampled(gemm):
    """The 8192^3 shape with e2m3 operands (N(0,1), scales U{120..134}, bf16
    out) on 65,536 sampled outputs plus the edge tiles."""
    p = mi.random_problem(8192, 8192, 8192, seed=860, fmtA=E2M3, fmtB=E2M3, out_dtype=mi.OUT_BF16)
    log("fp6 8192^3 generated")
    dev = to_dev(p)
    buf, c = alloc_c(p)
    gemm.set_variant(AUTO)
    gemm(*dev[:2], p.fmtA, *dev[2:], p.fmtB, c, out_dtype=p.out_dtype)
    torch.cuda.synchronize()
    rows, cols = mi.sample_points(p.M, p.N, 65536, seed=86)
    compare(c_numpy(c, p.out_dtype)[rows, cols], oracle_points(p, rows, cols), p.out_dtype,
            "fp6 8192^3")


def test_fp6_widened_pairs_need_the_operand_buffer():
    """e2m3 beside another format, and e3m2, run widened: on a handle
    without an operand buffer they are rejected before any launch, and an
    unknown format always is."""
    p = mi.random_problem(64, 64, 128, seed=1600, fmtA=E2M3, fmtB=E2M3)
    A, As, B, Bs = to_dev(p)
    buf, c = alloc_c(p)
    fresh = L.Gemm()
    try:
        for fa, fb in ((E2M3, 0), (1, E2M3), (E2M3, 4), (3, 3), (3, 0)):
            q = mi.random_problem(64, 64, 128, seed=1601 + fa + 8 * fb, fmtA=fa, fmtB=fb)
            qA, qAs, qB, qBs = to_dev(q)
            with pytest.raises(L.MxgemmError) as e:
                L.mxgemm_run(fresh.h, qA, qAs, fa, qB, qBs, fb, c, 64, 64, 128, 0, 0)
            assert e.value.code == L.STATUS_CODE["MXGEMM_ERR_WORKSPACE"], (fa, fb)
        with pytest.raises(L.MxgemmError) as e:
            L.mxgemm_run(fresh.h, A, As, E2M3, B, Bs, 6, c, 64, 64, 128, 0, 0)
        assert e.value.code == L.STATUS_CODE["MXGEMM_ERR_FMT"]
    finally:
        fresh.close()
    torch.cuda.synchronize()
    assert bool(torch.isnan(buf).all()), "a rejected call wrote C"
