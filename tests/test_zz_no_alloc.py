"""mxgemm_run_noalloc (the entry point for callers that cannot allocate)
against mxgemm_run on a handle with a workspace of the same size: through the
C ABI, two calls in a row on the library's fixed scratch (the second with a
smaller problem, so that stale partials or counters of the first would
show), each bit-identical to mxgemm_run and within the agreement rule of the
oracle."""
import numpy as np
import pytest
import torch

import level_dsl_amd as L
import mxinputs as mi
from gpu_helpers import alloc_c, c_numpy, compare, log, oracle_full, oracle_points, to_dev

pytestmark = pytest.mark.gpu

# (first problem, second, smaller problem): M, N, K, fmtA, fmtB, out, use_acc
PAIRS = [
    # small-M kernel, split 8 then split 2
    ((64, 3584, 8192, 0, 0, mi.OUT_F32, False), (16, 1000, 2048, 1, 0, mi.OUT_F32, False)),
    # 256 x 256 kernel, 4 tiles split 4, then 1 tile split 2
    ((512, 512, 4096, 0, 0, mi.OUT_BF16, False), (256, 256, 2048, 0, 1, mi.OUT_F32, True)),
    # e2m1 small-M kernel with splits, then the AUTO row chunks of M = 100
    ((64, 3584, 8192, 4, 4, mi.OUT_F32, False), (100, 900, 4096, 0, 0, mi.OUT_BF16, True)),
]


def _check(p, got, ref_got, where):
    assert np.array_equal(got, ref_got), f"{where}: differs from mxgemm_run"
    if p.M * p.N * p.K <= (1 << 31):
        ref = oracle_full(p)
        compare(got, ref, p.out_dtype, where)
    else:
        rows, cols = mi.sample_points(p.M, p.N, 8192, seed=3, edge=64)
        compare(got[rows, cols], oracle_points(p, rows, cols), p.out_dtype, where)


@pytest.mark.parametrize("pair", PAIRS, ids=lambda c: f"{c[0][0]}x{c[0][1]}x{c[0][2]}_then_"
                         f"{c[1][0]}x{c[1][1]}x{c[1][2]}")
def test_noalloc_matches_run(pair):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    probs = []
    for k, (M, N, K, fa, fb, out, acc) in enumerate(pair):
        probs.append(mi.random_problem(M, N, K, seed=6100 + 7 * k + M + N, fmtA=fa, fmtB=fb,
                                       out_dtype=out, use_acc=acc))
    ref_h = L.Gemm()
    ws = torch.empty(L.MXGEMM_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda:0")
    L.mxgemm_set_workspace(ref_h.h, ws, L.MXGEMM_WORKSPACE_BYTES)
    na = L.Gemm()  # no workspace attached
    try:
        devs = [to_dev(p) for p in probs]
        # the reference results, one call at a time on the caller's workspace
        refs = []
        for p, (A, As, B, Bs) in zip(probs, devs):
            buf, c = alloc_c(p)
            log(f"noalloc reference {p.name}")
            L.mxgemm_run(ref_h.h, A, As, p.fmtA, B, Bs, p.fmtB, c, p.M, p.N, p.K, int(p.use_acc),
                         p.out_dtype)
            torch.cuda.synchronize()
            refs.append(c_numpy(c, p.out_dtype))
        # the same two problems through mxgemm_run_noalloc, back to back
        outs = []
        for p, (A, As, B, Bs) in zip(probs, devs):
            buf, c = alloc_c(p)
            outs.append(c)
            log(f"noalloc call {p.name}")
            L.mxgemm_run_noalloc(na.h, A, As, p.fmtA, B, Bs, p.fmtB, c, p.M, p.N, p.K,
                                 int(p.use_acc), p.out_dtype)
        torch.cuda.synchronize()
        for p, c, r in zip(probs, outs, refs):
            _check(p, c_numpy(c, p.out_dtype), r, f"noalloc {p.name}")
    finally:
        ref_h.close()
        na.close()


def test_noalloc_forced_split_beyond_scratch():
    """A forced split whose 256 x 256 partial tiles do not fit the fixed
    scratch is rejected, and C is left untouched."""
    p = mi.random_problem(1024, 1024, 8192, seed=6200)  # 16 tiles: 8 splits need 32 MiB
    A, As, B, Bs = to_dev(p)
    buf, c = alloc_c(p)  # NaN-filled
    g = L.Gemm()
    try:
        g.set_splits(8)
        with pytest.raises(L.MxgemmError) as e:
            L.mxgemm_run_noalloc(g.h, A, As, 0, B, Bs, 0, c, p.M, p.N, p.K, 0, 0)
        assert e.value.code == L.STATUS_CODE["MXGEMM_ERR_WORKSPACE"]
        g.set_splits(1)  # no split: fine
        L.mxgemm_run_noalloc(g.h, A, As, 0, B, Bs, 0, c, p.M, p.N, p.K, 0, 0)
        torch.cuda.synchronize()
        rows, cols = mi.sample_points(p.M, p.N, 4096, seed=4, edge=32)
        compare(c_numpy(c, 0)[rows, cols], oracle_points(p, rows, cols), 0, "noalloc unsplit")
    finally:
        g.close()
