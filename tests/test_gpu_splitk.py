"""GPU parity of the small-M exact path's decode-size tiling and split-K.

* M below 64 runs ceil(M/16) row tiles of 16 (and as many decoding waves);
  every M from 1 to 64 that changes the tile count, or sits on either side
  of a tile boundary, is compared with the oracle on full outputs.
* Split-K (a caller-owned workspace attached to the handle): forced split
  counts, ragged K, both formats, use_acc and bf16 output, against the
  oracle; the fixed-order reduction gives bitwise-equal results on repeated
  calls; the arrival counters are back at zero after every call, so calls
  of different shapes in a row stay correct; the automatic choice at one
  GPU's share of the M=64 decode workload (N = 3584) against sampled
  oracle outputs; and the error paths.
* 64 < M <= 128 under AUTO: two launches of the exact small-M kernel, on
  full outputs and, with a workspace, split.
* Split-K of the 256 x 256-tile kernel (M > 64): forced split counts over
  4-stage scale windows (K % 512 == 0) and over single stages (other K),
  both variants (the native one against its own bound), use_acc and bf16;
  the automatic choice at medium M and at few output tiles; bitwise
  repeatability; and a workspace too small for the asked-for split, which
  must cut the split count, not overrun the buffer.
"""
import numpy as np
import pytest
import torch

import level_dsl_amd as L
import mxinputs as mi
from gpu_helpers import (alloc_c, c_numpy, compare, compare_native, log, native_group_extra,
                         oracle_full, oracle_points, run, to_dev)

pytestmark = pytest.mark.gpu

SKINNY = L.MXGEMM_VARIANT_SKINNY
LARGE, LARGE_NATIVE = L.MXGEMM_VARIANT_LARGE, L.MXGEMM_VARIANT_LARGE_NATIVE


@pytest.fixture(scope="module")
def gemm():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    g = L.Gemm()
    yield g
    g.close()


@pytest.fixture(scope="module")
def gemm_ws():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    g = L.Gemm()
    g.enable_split_k()
    yield g
    g.close()


@pytest.mark.parametrize("M", [1, 2, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64])
def test_decode_size_m_full(gemm, M):
    N, K = 250, 1056  # three column tiles (the last ragged), 8.25 K stages
    p = mi.random_problem(M, N, K, seed=500 + M, fmtA=M % 2, fmtB=(M // 2) % 2)
    log(f"decode-size M={M} N={N} K={K} fmt={p.fmtA}{p.fmtB}")
    got = run(gemm, p, SKINNY, guard=64)
    compare(got, oracle_full(p), p.out_dtype, f"M={M}")


SPLIT_CASES = [
    # M, N, K, splits, fmtA, fmtB, use_acc, out
    (64, 250, 8192, 8, 0, 0, False, mi.OUT_F32),
    (17, 112, 4128, 5, 0, 1, True, mi.OUT_BF16),     # 33 stages, the last partial
    (1, 3, 1024, 8, 1, 0, False, mi.OUT_F32),        # one stage per split
    (33, 500, 2080, 3, 1, 1, True, mi.OUT_F32),
    (48, 130, 640, 64, 0, 0, False, mi.OUT_BF16),    # asks for 64, runs 5 (one per stage)
    (64, 14336, 512, 2, 0, 0, False, mi.OUT_F32),    # 128 tiles x 2 splits: the workspace's limit
]


@pytest.mark.parametrize("M,N,K,S,fa,fb,acc,out", SPLIT_CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}_s{c[3]}" for c in SPLIT_CASES])
def test_split_k_forced(gemm_ws, M, N, K, S, fa, fb, acc, out):
    p = mi.random_problem(M, N, K, seed=600 + S, fmtA=fa, fmtB=fb, out_dtype=out, use_acc=acc)
    log(f"split-K forced S={S} M={M} N={N} K={K} fmt={fa}{fb} use_acc={acc} out={out}")
    gemm_ws.set_splits(S)
    try:
        got = run(gemm_ws, p, SKINNY, guard=64)
    finally:
        gemm_ws.set_splits(0)
    if M * N <= 64 * 500:
        compare(got, oracle_full(p), out, f"S={S}")
    else:
        rows, cols = mi.sample_points(M, N, 8192, seed=S, edge=64)
        compare(got[rows, cols], oracle_points(p, rows, cols), out, f"S={S} sampled")


NATIVE_SPLIT_CASES = [
    # M, N, K, splits, fmtA, fmtB, use_acc, out
    (64, 250, 8192, 8, 0, 0, False, mi.OUT_F32),     # LDS scale table
    (17, 112, 4128, 5, 0, 1, True, mi.OUT_BF16),     # 33 stages, the last partial; byte scales
    (1, 3, 1024, 8, 1, 0, False, mi.OUT_F32),        # 8 stages, two per split
    (40, 3584, 8192, 0, 1, 1, False, mi.OUT_F32),    # automatic: 32 column tiles, 8 splits
]


@pytest.mark.parametrize("M,N,K,S,fa,fb,acc,out", NATIVE_SPLIT_CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}_s{c[3]}" for c in NATIVE_SPLIT_CASES])
def test_native_small_m_split_k(gemm_ws, M, N, K, S, fa, fb, acc, out):
    """Split K on the small-M scaled-MFMA kernel with fp8 operands (the
    native opt-in), held to the native variants' bound; the unsplit call
    meets it too."""
    p = mi.random_problem(M, N, K, seed=700 + S + M, fmtA=fa, fmtB=fb, out_dtype=out, use_acc=acc)
    log(f"native small-M split-K S={S} M={M} N={N} K={K} fmt={fa}{fb} use_acc={acc} out={out}")
    dev = to_dev(p)
    gemm_ws.set_splits(S)
    try:
        got = run(gemm_ws, p, L.MXGEMM_VARIANT_SKINNY_NATIVE, guard=64, dev_inputs=dev)
    finally:
        gemm_ws.set_splits(0)
        gemm_ws.set_variant(L.MXGEMM_VARIANT_AUTO)
    extra = native_group_extra(p)
    if M * N <= 64 * 500:
        ref = oracle_full(p)
        compare_native(got, ref, out, extra, f"native S={S}")
    else:
        rows, cols = mi.sample_points(M, N, 8192, seed=S + M, edge=64)
        ref = oracle_points(p, rows, cols)
        compare_native(got[rows, cols], ref, out, extra[rows, cols], f"native S={S} sampled")


def test_split_k_bitwise_repeatable(gemm_ws):
    """The partials are added in split order whatever order the splits
    finish in: repeated calls give identical bits."""
    p = mi.random_problem(64, 336, 8192, seed=611)
    dev = to_dev(p)
    gemm_ws.set_splits(8)
    try:
        outs = [run(gemm_ws, p, SKINNY, dev_inputs=dev) for _ in range(4)]
    finally:
        gemm_ws.set_splits(0)
    log("split-K repeatability: 4 calls, S=8, 64x336x8192")
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))
    compare(outs[0], oracle_full(p), p.out_dtype, "S=8")


def test_split_k_counters_reset_across_calls(gemm_ws):
    """Calls of different shapes and split counts in a row, without any
    host-side reset in between: each is right, so every call leaves the
    arrival counters at zero."""
    cases = [(64, 224, 2048, 4), (5, 700, 1024, 3), (64, 224, 2048, 7), (16, 10, 4096, 8),
             (64, 224, 2048, 2)]
    for i, (M, N, K, S) in enumerate(cases):
        p = mi.random_problem(M, N, K, seed=620 + i)
        log(f"counter reset case {i}: S={S} M={M} N={N} K={K}")
        gemm_ws.set_splits(S)
        try:
            got = run(gemm_ws, p, SKINNY, guard=16)
        finally:
            gemm_ws.set_splits(0)
        compare(got, oracle_full(p), p.out_dtype, f"case {i}")


def test_split_k_auto_sharded_decode(gemm_ws):
    """One GPU's share of the M=64, N=28672, K=8192 decode workload when its
    columns are split over 8 GPUs: N = 3584 gives 32 column tiles, so the
    automatic choice splits K 8 ways (256 workgroups)."""
    M, N, K = 64, 3584, 8192
    p = mi.random_problem(M, N, K, seed=630)
    log(f"auto split at M={M} N={N} K={K}")
    got = run(gemm_ws, p, L.MXGEMM_VARIANT_AUTO, guard=64)
    rows, cols = mi.sample_points(M, N, 16384, seed=630, edge=64)
    compare(got[rows, cols], oracle_points(p, rows, cols), p.out_dtype, "auto split")
    # the same call without a workspace (unsplit) agrees within the rule
    g = L.Gemm()
    try:
        plain = run(g, p, L.MXGEMM_VARIANT_AUTO)
    finally:
        g.close()
    compare(plain[rows, cols], oracle_points(p, rows, cols), p.out_dtype, "unsplit")


def test_forced_split_without_workspace_is_an_error(gemm):
    p = mi.random_problem(64, 200, 2048, seed=640)
    A, As, B, Bs = to_dev(p)
    buf, c = alloc_c(p)
    gemm.set_splits(4)
    try:
        with pytest.raises(L.MxgemmError) as e:
            L.mxgemm_run(gemm.h, A, As, p.fmtA, B, Bs, p.fmtB, c, p.M, p.N, p.K, 0, 0)
        assert e.value.code == L.STATUS_CODE["MXGEMM_ERR_WORKSPACE"]
    finally:
        gemm.set_splits(0)
    torch.cuda.synchronize()
    assert torch.isnan(c).all(), "C touched by a rejected call"


def test_set_workspace_rejects_short_or_misaligned():
    g = L.Gemm()
    try:
        ws = torch.empty(L.MXGEMM_WORKSPACE_BYTES + 256, dtype=torch.uint8, device="cuda:0")
        for ptr, n in ((ws.data_ptr(), L.MXGEMM_WORKSPACE_BYTES - 1),
                       (ws.data_ptr() + 16, L.MXGEMM_WORKSPACE_BYTES)):
            with pytest.raises(L.MxgemmError) as e:
                L.mxgemm_set_workspace(g.h, ptr, n)
            assert e.value.code == L.STATUS_CODE["MXGEMM_ERR_WORKSPACE"]
        with pytest.raises(L.MxgemmError) as e:
            L.mxgemm_set_splits(g.h, -1)
        assert e.value.code == L.STATUS_CODE["MXGEMM_ERR_SHAPE"]
    finally:
        g.close()


def test_split_k_alternating_problems_never_see_stale_partials(gemm_ws):
    """Two problems of the same shape alternate on one workspace, ten calls
    each: a partial left over from the other problem (a store not yet
    visible, or a stale cached copy) would change the bits of a result, so
    every call must reproduce the first result of its problem exactly."""
    M, N, K = 64, 3584, 8192
    probs = [mi.random_problem(M, N, K, seed=650 + j) for j in range(2)]
    devs = [to_dev(p) for p in probs]
    first = [None, None]
    for it in range(20):
        j = it % 2
        got = run(gemm_ws, probs[j], L.MXGEMM_VARIANT_AUTO, dev_inputs=devs[j])
        if first[j] is None:
            first[j] = got
            rows, cols = mi.sample_points(M, N, 4096, seed=650 + j, edge=32)
            compare(got[rows, cols], oracle_points(probs[j], rows, cols), probs[j].out_dtype,
                    f"problem {j}")
        else:
            assert np.array_equal(got.view(np.uint32), first[j].view(np.uint32)), f"call {it}"
    log("alternating split-K calls: 20 calls reproduced their first results")



LARGE_SPLIT_CASES = [
    # M, N, K, splits, fmtA, fmtB, use_acc, out
    (300, 260, 4096, 4, 0, 0, False, mi.OUT_F32),     # 4 tiles; 8 windows -> 2 each
    (257, 300, 2048, 3, 0, 1, True, mi.OUT_BF16),     # 4 windows over 3 splits (1, 1, 2)
    (129, 513, 1056, 3, 1, 0, False, mi.OUT_F32),     # K % 512 != 0: 9 stages, 3 each
    (80, 256, 640, 8, 1, 1, True, mi.OUT_F32),        # scale rows of 20 bytes: 5 stages, 5 splits
    (512, 512, 8192, 64, 0, 0, False, mi.OUT_BF16),   # asks for 64: 16 windows -> 16 splits
]


@pytest.mark.parametrize("M,N,K,S,fa,fb,acc,out", LARGE_SPLIT_CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}_s{c[3]}" for c in LARGE_SPLIT_CASES])
def test_large_split_k_forced(gemm_ws, M, N, K, S, fa, fb, acc, out):
    p = mi.random_problem(M, N, K, seed=700 + S + M, fmtA=fa, fmtB=fb, out_dtype=out, use_acc=acc)
    ref = oracle_full(p)
    dev = to_dev(p)
    gemm_ws.set_splits(S)
    try:
        log(f"large split-K forced S={S} M={M} N={N} K={K} fmt={fa}{fb} use_acc={acc} out={out}")
        got = run(gemm_ws, p, LARGE, guard=64, dev_inputs=dev)
        compare(got, ref, out, f"large S={S}")
        log(f"large native split-K forced S={S} M={M} N={N} K={K}")
        got = run(gemm_ws, p, LARGE_NATIVE, guard=64, dev_inputs=dev)
        compare_native(got, ref, out, native_group_extra(p), f"large native S={S}")
    finally:
        gemm_ws.set_splits(0)
        gemm_ws.set_variant(L.MXGEMM_VARIANT_AUTO)


@pytest.mark.parametrize("M,N,K", [(128, 28672, 8192), (1024, 1024, 8192), (200, 3000, 4096)])
def test_large_split_k_auto(gemm_ws, M, N, K):
    """Automatic split of the 256 x 256 kernel (variant LARGE: AUTO takes
    two small-M launches at M = 128) at medium M (one row of tiles) and at
    few output tiles, against sampled oracle outputs; the unsplit result
    agrees too."""
    p = mi.random_problem(M, N, K, seed=720 + M)
    dev = to_dev(p)
    rows, cols = mi.sample_points(M, N, 8192, seed=720 + M, edge=64)
    ref = oracle_points(p, rows, cols)
    log(f"large auto split M={M} N={N} K={K}")
    try:
        got = run(gemm_ws, p, LARGE, guard=64, dev_inputs=dev)
        compare(got[rows, cols], ref, p.out_dtype, "auto split")
        again = run(gemm_ws, p, LARGE, dev_inputs=dev)
        assert np.array_equal(got.view(np.uint32), again.view(np.uint32)), "not repeatable"
    finally:
        gemm_ws.set_variant(L.MXGEMM_VARIANT_AUTO)
    g = L.Gemm()
    try:
        plain = run(g, p, LARGE, dev_inputs=dev)
    finally:
        g.close()
    compare(plain[rows, cols], ref, p.out_dtype, "unsplit")


def test_large_split_k_small_workspace_is_respected():
    """A minimum-size workspace (room for 28 partial tiles of 256 x 256)
    with 16 output tiles and 8 splits asked for: the split count must drop
    to what fits (here 1), the bytes past the workspace stay untouched and
    the result is right."""
    M, N, K = 1024, 1024, 4096
    p = mi.random_problem(M, N, K, seed=740)
    guard = 1 << 20
    buf = torch.full((L.MXGEMM_WORKSPACE_BYTES + guard,), 0x5A, dtype=torch.uint8, device="cuda:0")
    g = L.Gemm()
    try:
        L.mxgemm_set_workspace(g.h, buf, L.MXGEMM_WORKSPACE_BYTES)
        g.set_splits(8)
        log("large split with a minimum-size workspace")
        got = run(g, p, LARGE, guard=64)
        torch.cuda.synchronize()
        assert bool((buf[L.MXGEMM_WORKSPACE_BYTES:] == 0x5A).all()), "write past the workspace"
        rows, cols = mi.sample_points(M, N, 4096, seed=740, edge=32)
        compare(got[rows, cols], oracle_points(p, rows, cols), p.out_dtype, "small workspace")
        # 4 tiles fit 7 partials each: a split of 4 is honoured and correct
        q = mi.random_problem(400, 400, 4096, seed=741)
        g.set_splits(4)
        got = run(g, q, LARGE, guard=64)
        compare(got, oracle_full(q), q.out_dtype, "small workspace, 4 tiles x 4 splits")
        assert bool((buf[L.MXGEMM_WORKSPACE_BYTES:] == 0x5A).all()), "write past the workspace"
    finally:
        g.close()


@pytest.mark.parametrize("M,N,K,fa,fb,acc,out", [
    (65, 250, 1056, 0, 0, False, mi.OUT_F32),     # one row in the second launch, ragged stages
    (100, 130, 2080, 1, 0, True, mi.OUT_BF16),
    (128, 336, 4096, 0, 1, False, mi.OUT_F32),    # two full halves
    (150, 250, 2048, 1, 1, True, mi.OUT_F32),     # three launches (3 column tiles)
    (192, 7168, 512, 0, 0, False, mi.OUT_BF16),   # three launches at 64 column tiles
])
def test_two_half_launches_exact(gemm, M, N, K, fa, fb, acc, out):
    """64 < M <= 128 (M <= 192 with at most 64 column tiles) under AUTO: the
    exact small-M kernel once per 64 rows; full outputs against the oracle,
    guard bands intact."""
    p = mi.random_problem(M, N, K, seed=740 + M, fmtA=fa, fmtB=fb, out_dtype=out, use_acc=acc)
    log(f"two half launches M={M} N={N} K={K} fmt={fa}{fb} use_acc={acc} out={out}")
    got = run(gemm, p, L.MXGEMM_VARIANT_AUTO, guard=64)
    compare(got, oracle_full(p), out, f"halves M={M}")


def test_two_half_launches_exact_split_sharded(gemm_ws):
    """The same at N = 3584 with a workspace, so that each half splits K."""
    M, N, K = 96, 3584, 8192
    p = mi.random_problem(M, N, K, seed=750)
    log(f"two half launches with split M={M} N={N} K={K}")
    got = run(gemm_ws, p, L.MXGEMM_VARIANT_AUTO, guard=64)
    rows, cols = mi.sample_points(M, N, 8192, seed=750, edge=64)
    compare(got[rows, cols], oracle_points(p, rows, cols), p.out_dtype, "halves split")
