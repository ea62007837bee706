"""GPU parity of e2m1 (FP4) operands, two codes per byte along K, against
the CPU oracle.

e2m1 x e2m1 runs on the 256 x 256 kernel's scaled MFMA (every product of a
32-element block fits the instruction's 8-product window, so it is exact up
to the fp32 accumulation), and is held to the same agreement rule as the
exact variants:
  * every pair of the 16 codes at several scale pairs, bit for bit;
  * random problems on full outputs: ragged M, N and K (a partial last
    stage, K not a multiple of 128 values), use_acc, bf16 output, M = 1 and
    small M, and both e2m1-capable variants;
  * a NaN scale at the start of the next row must not leak into a row
    whose last stage stops inside the scale dword (K = 1152);
  * 64 < M <= 128 under AUTO (two launches of the small-M kernel);
  * split-K, forced and automatic, on both kernels (the small-M kernel's
    split in its three scale modes, bitwise repeatable, its arrival
    counters shared with the other kernels' splits);
  * the 8192 x 8192 x 8192 benchmark shape on sampled outputs;
  * the limits of the C ABI: the largest K and N, many row tiles, and the
    row-chunked small-M launches at the largest N;
  * the error paths (e2m1 beside e4m3 on a handle without an operand
    buffer, an unknown format, a small-M variant with M > 64).
"""
import numpy as np
import pytest
import torch

import level_dsl_amd as L
import mxinputs as mi
import oracle
from gpu_helpers import alloc_c, compare, log, oracle_full, oracle_points, run, to_dev

pytestmark = pytest.mark.gpu

E2M1 = L.MXGEMM_FMT_E2M1
AUTO, LARGE, LARGE_NATIVE = L.MXGEMM_VARIANT_AUTO, L.MXGEMM_VARIANT_LARGE, L.MXGEMM_VARIANT_LARGE_NATIVE
SKINNY, SKINNY_NATIVE = L.MXGEMM_VARIANT_SKINNY, L.MXGEMM_VARIANT_SKINNY_NATIVE


@pytest.fixture(scope="module")
def gemm():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    g = L.Gemm()
    yield g
    g.close()


@pytest.mark.parametrize("sa,sb", [(127, 127), (100, 150), (1, 254), (200, 60)])
def test_fp4_pairwise_products_exact(gemm, sa, sb):
    """A[m, 0] = code m, B[n, 0] = code n (16 x 16, K = 32, the rest zero):
    every C[m, n] is the exact product dec(m) dec(n) 2^(sa+sb-254)."""
    M = N = 16
    K = 32
    A = np.zeros((M, K // 2), np.uint8)
    B = np.zeros((N, K // 2), np.uint8)
    A[:, 0] = np.arange(16, dtype=np.uint8)      # k = 0: the low nibble
    B[:, 0] = np.arange(16, dtype=np.uint8)
    p = mi.Problem(M, N, K, E2M1, E2M1, A, np.full((M, 1), sa, np.uint8), B,
                   np.full((N, 1), sb, np.uint8), mi.OUT_F32, False)
    log(f"fp4 pairwise sa={sa} sb={sb}")
    got = run(gemm, p, AUTO)
    ref = oracle_full(p)
    r = ref["ref32"]
    normal = (np.abs(r) >= np.float32(2.0**-126)) | (r == 0)
    assert np.array_equal(got[normal], r[normal]), f"{np.sum(got[normal] != r[normal])} mismatches"


FP4_CASES = [
    # M, N, K, use_acc, out
    (300, 260, 4096, False, mi.OUT_F32),
    (257, 300, 2048, True, mi.OUT_BF16),
    (129, 513, 1056, False, mi.OUT_F32),     # 528 bytes per row: a partial last stage
    (64, 200, 8192, True, mi.OUT_F32),
    (1, 5, 32, False, mi.OUT_F32),
    (517, 389, 1056, True, mi.OUT_BF16),
    (33, 1000, 640, False, mi.OUT_BF16),
    (16, 120, 24576, False, mi.OUT_F32),     # M <= 64 with K too long for the LDS scale table
    (20, 333, 2048, True, mi.OUT_BF16),      # two 16-row tiles of A on the small-M kernel
    (48, 250, 4096, False, mi.OUT_F32),      # three
]


@pytest.mark.parametrize("M,N,K,acc,out", FP4_CASES, ids=lambda c: str(c))
def test_fp4_random_full(gemm, M, N, K, acc, out):
    p = mi.random_problem(M, N, K, seed=800 + M + K, fmtA=E2M1, fmtB=E2M1, out_dtype=out,
                          use_acc=acc)
    ref = oracle_full(p)
    dev = to_dev(p)
    for v in (AUTO, LARGE_NATIVE) + ((SKINNY, SKINNY_NATIVE) if M <= 64 else ()):
        log(f"fp4 random M={M} N={N} K={K} use_acc={acc} out={out} variant={v}")
        got = run(gemm, p, v, guard=64, dev_inputs=dev)
        compare(got, ref, out, f"fp4 {M}x{N}x{K} variant {v}")
    gemm.set_variant(AUTO)


def test_fp4_scale_tail_does_not_read_the_next_row(gemm):
    """K = 1152: 36 scale bytes per row (a multiple of 4, so scales are read
    as dwords) and 576 code bytes, 4.5 stages; the last stage's second scale
    dword lies past the row.  Every other row starts with a NaN scale byte;
    a kernel that read the next row's first dword there would turn the
    zero-padded tail of a finite row into NaN."""
    M, N, K = 64, 96, 1152
    p = mi.random_problem(M, N, K, seed=820, fmtA=E2M1, fmtB=E2M1)
    p.As[1::2, 0] = 255
    p.Bs[1::2, 0] = 255
    ref = oracle_full(p)
    log("fp4 scale tail guard")
    got = run(gemm, p, AUTO)
    compare(got, ref, p.out_dtype, "fp4 scale tail")
    assert np.isnan(got[1::2]).all() and np.isnan(got[:, 1::2]).all()
    assert np.isfinite(got[0::2, 0::2]).all(), "NaN leaked into a finite row"


@pytest.mark.parametrize("S", [2, 4, 7])
def test_fp4_split_k_forced(S):
    M, N, K = 300, 260, 4096
    p = mi.random_problem(M, N, K, seed=830 + S, fmtA=E2M1, fmtB=E2M1, out_dtype=mi.OUT_BF16,
                          use_acc=True)
    g = L.Gemm()
    g.enable_split_k()
    try:
        g.set_splits(S)
        log(f"fp4 split-K S={S}")
        got = run(g, p, AUTO, guard=64)
        compare(got, oracle_full(p), p.out_dtype, f"fp4 split S={S}")
    finally:
        g.close()


SMALL_M_SPLIT_CASES = [
    # M, N, K, splits, use_acc, out  (scale mode the host picks)
    (16, 250, 8192, 8, False, mi.OUT_F32),     # LDS scale table
    (33, 130, 4160, 5, True, mi.OUT_BF16),     # 17 stages, the last partial; byte scale loads
    (64, 500, 2048, 3, False, mi.OUT_F32),     # four A tiles, table
    (1, 3, 1024, 8, False, mi.OUT_F32),        # 4 stages: asks for 8, runs 4
    (48, 112, 3072, 7, True, mi.OUT_F32),      # 12 stages over 7 splits (one or two each)
    (16, 120, 24576, 4, False, mi.OUT_BF16),   # K too long for the table: 8-byte scale loads
]


@pytest.mark.parametrize("M,N,K,S,acc,out", SMALL_M_SPLIT_CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}_s{c[3]}" for c in SMALL_M_SPLIT_CASES])
def test_fp4_small_m_split_k_forced(M, N, K, S, acc, out):
    """Split K on the small-M scaled-MFMA kernel (M <= 64), against the
    oracle on full outputs, with the guard bands around C intact."""
    p = mi.random_problem(M, N, K, seed=850 + S + M, fmtA=E2M1, fmtB=E2M1, out_dtype=out,
                          use_acc=acc)
    g = L.Gemm()
    g.enable_split_k()
    try:
        g.set_splits(S)
        log(f"fp4 small-M split-K S={S} M={M} N={N} K={K} use_acc={acc} out={out}")
        got = run(g, p, AUTO, guard=64)
        compare(got, oracle_full(p), out, f"fp4 small-M split S={S}")
    finally:
        g.close()


def test_fp4_small_m_split_k_repeatable_and_counters_reset():
    """Splits add their partials in split order: repeated calls give the
    same bits.  Calls of other shapes and kernels in between (the exact
    small-M kernel's split, the 256 x 256 kernel's split) share the arrival
    counters; each call leaves them at zero, so every result stays right."""
    g = L.Gemm()
    g.enable_split_k()
    try:
        p = mi.random_problem(64, 336, 8192, seed=860, fmtA=E2M1, fmtB=E2M1)
        dev = to_dev(p)
        g.set_splits(8)
        outs = [run(g, p, AUTO, dev_inputs=dev) for _ in range(3)]
        log("fp4 small-M split repeatability: 3 calls, S=8, 64x336x8192")
        for o in outs[1:]:
            assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
        compare(outs[0], oracle_full(p), p.out_dtype, "S=8")
        others = [mi.random_problem(40, 300, 2048, seed=861),
                  mi.random_problem(200, 300, 2048, seed=862, fmtA=E2M1, fmtB=E2M1),
                  mi.random_problem(16, 250, 4096, seed=863, fmtA=E2M1, fmtB=E2M1)]
        for S in (3, 5):
            g.set_splits(S)
            for q in others:
                log(f"fp4 counters: S={S} M={q.M} N={q.N} K={q.K} fmt={q.fmtA}")
                compare(run(g, q, AUTO, guard=16), oracle_full(q), q.out_dtype, f"S={S} M={q.M}")
            again = run(g, p, AUTO, dev_inputs=dev)
            compare(again, oracle_full(p), p.out_dtype, f"after S={S}")
    finally:
        g.close()


@pytest.mark.parametrize("M", [1, 16, 64])
def test_fp4_small_m_split_k_auto_sharded_decode(M):
    """One GPU's share of the decode shape split by columns over 8 GPUs:
    N = 3584 leaves 32 column tiles, so the automatic choice splits K 8 ways;
    sampled outputs against the oracle, and the unsplit call agrees."""
    N, K = 3584, 8192
    p = mi.random_problem(M, N, K, seed=870 + M, fmtA=E2M1, fmtB=E2M1)
    dev = to_dev(p)
    rows, cols = mi.sample_points(M, N, 8192, seed=870 + M, edge=64)
    ref = oracle_points(p, rows, cols)
    g = L.Gemm()
    g.enable_split_k()
    try:
        log(f"fp4 small-M auto split M={M} N={N} K={K}")
        got = run(g, p, AUTO, guard=64, dev_inputs=dev)
        compare(got[rows, cols], ref, p.out_dtype, "fp4 small-M auto split")
    finally:
        g.close()
    g = L.Gemm()
    try:
        plain = run(g, p, AUTO, dev_inputs=dev)
    finally:
        g.close()
    compare(plain[rows, cols], ref, p.out_dtype, "fp4 small-M unsplit")


@pytest.mark.parametrize("M,N,K,acc,out", [
    (65, 250, 2048, False, mi.OUT_F32),     # one row in the second launch
    (96, 130, 4160, True, mi.OUT_BF16),     # ragged K, byte scale loads
    (128, 336, 8192, False, mi.OUT_F32),    # two full halves
    (192, 200, 4096, True, mi.OUT_F32),     # three launches
])
def test_fp4_two_half_launches(M, N, K, acc, out):
    """e2m1 with 64 < M <= 128 under AUTO runs the small-M kernel on rows
    0..63 and then on the rest: full outputs against the oracle, and the
    guard bands around C intact."""
    p = mi.random_problem(M, N, K, seed=880 + M, fmtA=E2M1, fmtB=E2M1, out_dtype=out, use_acc=acc)
    g = L.Gemm()
    try:
        log(f"fp4 two half launches M={M} N={N} K={K} use_acc={acc} out={out}")
        got = run(g, p, AUTO, guard=64)
        compare(got, oracle_full(p), out, f"fp4 halves M={M}")
    finally:
        g.close()


def test_fp4_two_half_launches_split_sharded():
    """The same at one GPU's share of N (3584 columns) with a workspace: each
    half splits K 8 ways; sampled outputs against the oracle."""
    M, N, K = 112, 3584, 8192
    p = mi.random_problem(M, N, K, seed=890, fmtA=E2M1, fmtB=E2M1)
    g = L.Gemm()
    g.enable_split_k()
    try:
        log(f"fp4 two half launches with split M={M} N={N} K={K}")
        got = run(g, p, AUTO, guard=64)
        rows, cols = mi.sample_points(M, N, 8192, seed=890, edge=64)
        compare(got[rows, cols], oracle_points(p, rows, cols), p.out_dtype, "fp4 halves split")
    finally:
        g.close()


@pytest.mark.parametrize("M,variant", [(128, LARGE), (192, AUTO)])
def test_fp4_split_k_auto_medium_m(M, variant):
    """The 256 x 256 kernel's automatic split at medium M (56 output tiles):
    M = 128 with the variant forced (AUTO takes two small-M launches there),
    M = 192 under AUTO."""
    N, K = 14336, 8192
    p = mi.random_problem(M, N, K, seed=840, fmtA=E2M1, fmtB=E2M1)
    g = L.Gemm()
    g.enable_split_k()
    try:
        log(f"fp4 auto split at M={M}")
        got = run(g, p, variant)
        rows, cols = mi.sample_points(M, N, 8192, seed=840, edge=64)
        compare(got[rows, cols], oracle_points(p, rows, cols), p.out_dtype, "fp4 auto split")
    finally:
        g.close()


def test_fp4_8192_cube_sampled(gemm):
    """The e2m1 benchmark shape: 8192^3, N(0, 1) codes, scales U{120..134},
    bf16 out, 16384 sampled outputs plus the edges."""
    M = N = K = 8192
    p = mi.random_problem(M, N, K, seed=850, fmtA=E2M1, fmtB=E2M1, out_dtype=mi.OUT_BF16)
    log("fp4 8192^3 generated")
    got = run(gemm, p, AUTO)
    rows, cols = mi.sample_points(M, N, 16384, seed=850, edge=64)
    compare(got[rows, cols], oracle_points(p, rows, cols), p.out_dtype, "fp4 8192^3")


def test_fp4_decode_size_sampled(gemm):
    """M = 64, N = 28672, K = 8192 (the decode workload's shape in e2m1): the
    automatic choice is the small-M kernel; sampled outputs and the edges."""
    M, N, K = 64, 28672, 8192
    p = mi.random_problem(M, N, K, seed=870, fmtA=E2M1, fmtB=E2M1)
    log("fp4 decode shape generated")
    got = run(gemm, p, AUTO, guard=64)
    rows, cols = mi.sample_points(M, N, 16384, seed=870, edge=64)
    compare(got[rows, cols], oracle_points(p, rows, cols), p.out_dtype, "fp4 decode shape")


def test_fp4_error_paths(gemm):
    p = mi.random_problem(64, 64, 128, seed=860, fmtA=E2M1, fmtB=E2M1)
    A, As, B, Bs = to_dev(p)
    buf, c = alloc_c(p)
    # e2m1 with e4m3 runs widened: on a handle without an operand buffer it
    # is rejected before any launch; an unknown format always is
    w = mi.random_problem(64, 64, 128, seed=862, fmtA=E2M1, fmtB=0)
    wA, wAs, wB, wBs = to_dev(w)
    fresh = L.Gemm()
    try:
        for fb, name in ((0, "MXGEMM_ERR_WORKSPACE"), (5, "MXGEMM_ERR_FMT")):
            with pytest.raises(L.MxgemmError) as e:
                L.mxgemm_run(fresh.h, wA, wAs, E2M1, wB, wBs, fb, c, 64, 64, 128, 0, 0)
            assert e.value.code == L.STATUS_CODE[name], name
    finally:
        fresh.close()
    # a forced small-M variant with M > 64
    q = mi.random_problem(65, 64, 128, seed=861, fmtA=E2M1, fmtB=E2M1)
    qA, qAs, qB, qBs = to_dev(q)
    qbuf, qc = alloc_c(q)
    for v in (SKINNY, SKINNY_NATIVE):
        gemm.set_variant(v)
        with pytest.raises(L.MxgemmError) as e:
            L.mxgemm_run(gemm.h, qA, qAs, E2M1, qB, qBs, E2M1, qc, 65, 64, 128, 0, 0)
        assert e.value.code == L.STATUS_CODE["MXGEMM_ERR_VARIANT"]
    gemm.set_variant(AUTO)
    torch.cuda.synchronize()
    assert bool(torch.isnan(qbuf).all()), "a rejected call wrote C"
    torch.cuda.synchronize()
    assert bool(torch.isnan(buf).all()), "a rejected call wrote C"


E2M1_EDGE_CASES = [
    # M, N, K, out, variants
    (2, 3, 1 << 21, mi.OUT_F32, (AUTO, LARGE)),          # the largest K: 1 MiB packed rows
    (3, 1 << 20, 64, mi.OUT_BF16, (AUTO, LARGE)),        # the largest N (9363 small-M workgroups)
    (70000, 40, 64, mi.OUT_F32, (AUTO,)),                # many row tiles, ragged last tile
]


@pytest.mark.parametrize("case", E2M1_EDGE_CASES, ids=lambda c: "x".join(map(str, c[:3])))
def test_fp4_edge_full(gemm, case):
    """e2m1 at the limits of the C ABI, full outputs against the oracle on
    every variant listed, with the guard bands around C intact."""
    M, N, K, out, variants = case
    p = mi.random_problem(M, N, K, seed=(M * 7 + N * 3 + K) % 100003, fmtA=E2M1, fmtB=E2M1,
                          out_dtype=out)
    ref = oracle_full(p)
    dev = to_dev(p)
    for v in variants:
        log(f"fp4 edge {M}x{N}x{K} variant={v}")
        got = run(gemm, p, v, guard=64, dev_inputs=dev)
        compare(got, ref, out, f"fp4 edge {M}x{N}x{K} variant {v}")
    gemm.set_variant(AUTO)


def test_fp4_two_launches_largest_n_sampled(gemm):
    """AUTO's row-chunked small-M launches at the largest N (M = 100: rows
    0..63, then 64..99), sampled outputs against the oracle."""
    M, N, K = 100, 1 << 20, 64
    p = mi.random_problem(M, N, K, seed=895, fmtA=E2M1, fmtB=E2M1)
    log(f"fp4 two launches at the largest N: {M}x{N}x{K}")
    got = run(gemm, p, AUTO, guard=64)
    rows, cols = mi.sample_points(M, N, 16384, seed=895, edge=64)
    compare(got[rows, cols], oracle_points(p, rows, cols), p.out_dtype, "fp4 largest N halves")
