"""GPU parity of the widened operand pairs against the CPU oracle.

e3m2 operands, and e2m1 or e2m3 beside any format but itself, are rewritten
as e4m3 bytes on the device (every value of the three sub-byte formats is
an e4m3 value) and multiplied on the fp8 path.  Checked here:
  * the rewrite itself, bit for bit: every code of each format, and a
    16 M-code operand that takes the kernel's grid-stride loop, against the
    e4m3 byte the oracle's decode tables name for each code's value (signed
    zeros included), with a canary past the end of the output;
  * mixed and e3m2 pairs through mxgemm_run on full outputs: both kernels,
    ragged M, N, K, use_acc, bf16 output, the row-chunked AUTO path, and
    the ABI's limits (the largest K, the largest N, many row tiles);
  * the native variants on a widened pair, to their bound;
  * preshuffled scales, split-K (automatic and forced) and
    mxgemm_run_noalloc on widened pairs;
  * the error paths (no operand buffer, a short one, one overlapping an
    operand or C, a bad format), none of which writes C.
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

E4M3, E5M2, E2M3, E3M2, E2M1 = (L.MXGEMM_FMT_E4M3, L.MXGEMM_FMT_E5M2, L.MXGEMM_FMT_E2M3,
                                L.MXGEMM_FMT_E3M2, L.MXGEMM_FMT_E2M1)
AUTO, LARGE, SKINNY = L.MXGEMM_VARIANT_AUTO, L.MXGEMM_VARIANT_LARGE, L.MXGEMM_VARIANT_SKINNY
LARGE_NATIVE, SKINNY_NATIVE = L.MXGEMM_VARIANT_LARGE_NATIVE, L.MXGEMM_VARIANT_SKINNY_NATIVE
BITS = {E2M1: 4, E2M3: 6, E3M2: 6}


@pytest.fixture(scope="module")
def gemm():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    g = L.Gemm()
    yield g
    g.close()


def e4m3_of(fmt):
    """For each code of `fmt`, the e4m3 byte of the same value, from the
    oracle's decode tables: the one byte whose value and sign match."""
    src = oracle.decode_table(fmt)[: 1 << BITS[fmt]]
    dst = oracle.decode_table(E4M3)
    out = np.empty(len(src), np.uint8)
    for c, v in enumerate(src):
        hits = [b for b in range(256) if dst[b] == v and np.signbit(dst[b]) == np.signbit(v)]
        assert len(hits) == 1, (fmt, c, v, hits)
        out[c] = hits[0]
    return out


def unpack_flat(packed: np.ndarray, fmt: int) -> np.ndarray:
    """All codes of a packed operand, in order (two per byte, the even code
    in the low nibble; or four per three bytes, code j at bits 6j .. 6j+5 of
    the little-endian group)."""
    b = np.ascontiguousarray(packed).reshape(-1)
    if fmt == E2M1:
        out = np.empty(2 * b.size, np.uint8)
        out[0::2], out[1::2] = b & 15, b >> 4
        return out
    g = b.reshape(-1, 3).astype(np.uint32)
    x = g[:, 0] | (g[:, 1] << 8) | (g[:, 2] << 16)
    return np.stack([(x >> (6 * j)) & 63 for j in range(4)], axis=1).astype(np.uint8).reshape(-1)


def widen_on_device(h, packed: np.ndarray, fmt: int, rows: int, K: int, canary: int = 256):
    src = torch.from_numpy(np.ascontiguousarray(packed).reshape(-1)).cuda()
    buf = torch.full((rows * K + canary,), 0xA5, dtype=torch.uint8, device="cuda")
    L.mxgemm_widen(h, src, fmt, rows, K, buf)
    torch.cuda.synchronize()
    out = buf.cpu().numpy()
    assert np.all(out[rows * K:] == 0xA5), "widen wrote past its output"
    return out[: rows * K]


@pytest.mark.parametrize("fmt", [E2M1, E2M3, E3M2])
def test_widen_every_code(gemm, fmt):
    """Every code of the format (several times, in every position of a
    16-code group) and a ragged tail of groups: each output byte is the e4m3
    byte of the code's value."""
    rows, K = 3, 1056
    g = np.random.Generator(np.random.PCG64(2100 + fmt))
    codes = g.integers(0, 1 << BITS[fmt], size=(rows, K), dtype=np.uint8)
    n = 1 << BITS[fmt]
    codes[0, :n] = np.arange(n)          # every code, in every position of a 16-code group
    codes[1, 5:5 + n] = np.arange(n)[::-1]
    packed = mi.pack_bits(codes, BITS[fmt])
    assert np.array_equal(unpack_flat(packed, fmt), codes.reshape(-1))
    log(f"widen every code fmt={fmt}")
    got = widen_on_device(gemm.h, packed, fmt, rows, K)
    assert np.array_equal(got, e4m3_of(fmt)[codes.reshape(-1)])


@pytest.mark.parametrize("fmt", [E2M1, E3M2])
def test_widen_grid_stride(gemm, fmt):
    """16 M codes (more than the launch's threads cover in one pass): random
    bytes are a valid packed operand of either format."""
    rows, K = 8, 1 << 21
    g = np.random.Generator(np.random.PCG64(2200 + fmt))
    packed = g.integers(0, 256, size=rows * L.row_bytes(fmt, K), dtype=np.uint8)
    log(f"widen grid-stride fmt={fmt}")
    got = widen_on_device(gemm.h, packed, fmt, rows, K)
    assert np.array_equal(got, e4m3_of(fmt)[unpack_flat(packed, fmt)])


def _variants(M):
    return (AUTO, LARGE) + ((SKINNY,) if M <= 64 else ())


WIDE_CASES = [
    # M, N, K, fmtA, fmtB, use_acc, out
    (300, 260, 1056, E2M1, E4M3, False, mi.OUT_F32),   # K % 128 != 0
    (300, 260, 1056, E5M2, E2M1, True, mi.OUT_BF16),
    (257, 300, 2048, E3M2, E3M2, True, mi.OUT_F32),
    (48, 520, 1024, E3M2, E4M3, False, mi.OUT_BF16),   # small-M kernel too
    (40, 333, 2080, E2M3, E5M2, True, mi.OUT_F32),
    (130, 700, 1024, E2M1, E2M3, False, mi.OUT_F32),   # AUTO: three small-M launches
    (64, 448, 4096, E4M3, E3M2, False, mi.OUT_BF16),
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=lambda c: "x".join(map(str, c[:3])) + f"_f{c[3]}{c[4]}")
def test_widened_pairs_full(gemm, case):
    M, N, K, fa, fb, acc, out = case
    p = mi.random_problem(M, N, K, seed=2300 + M + N + fa + 8 * fb, fmtA=fa, fmtB=fb,
                          use_acc=acc, out_dtype=out)
    ref = oracle_full(p)
    dev = to_dev(p)
    for v in _variants(M):
        log(f"widened {case} variant={v}")
        got = run(gemm, p, v, guard=64, dev_inputs=dev)
        compare(got, ref, out, f"widened {case} variant {v}")
    gemm.set_variant(AUTO)


@pytest.mark.parametrize("case", [(300, 260, 1056, E2M1, E4M3), (48, 520, 1024, E3M2, E3M2)],
                         ids=lambda c: "x".join(map(str, c[:3])))
def test_widened_pairs_native(gemm, case):
    """A native variant on a widened pair runs the fp8 pair on the scaled
    MFMA: the native bound."""
    M, N, K, fa, fb = case
    p = mi.random_problem(M, N, K, seed=2400 + M, fmtA=fa, fmtB=fb)
    ref = oracle_full(p)
    extra = native_group_extra(p)
    for v in ([LARGE_NATIVE, SKINNY_NATIVE] if M <= 64 else [LARGE_NATIVE]):
        log(f"widened native {case} variant={v}")
        got = run(gemm, p, v)
        compare_native(got, ref, p.out_dtype, extra, f"widened native {case} {v}")
    gemm.set_variant(AUTO)


def test_widened_preshuffled_scales():
    M, N, K = 300, 260, 1024
    p = mi.random_problem(M, N, K, seed=2500, fmtA=E2M1, fmtB=E5M2, out_dtype=mi.OUT_BF16)
    ref = oracle_full(p)
    g = L.Gemm()
    try:
        A, As, B, Bs = to_dev(p)
        g.set_scale_layout(L.MXGEMM_SCALES_PRESHUFFLED)
        Aps, Bps = g.preshuffle_scales(As), g.preshuffle_scales(Bs)
        buf, c = alloc_c(p)
        log("widened preshuffled")
        g(A, Aps, p.fmtA, B, Bps, p.fmtB, c, out_dtype=p.out_dtype)
        torch.cuda.synchronize()
        compare(c_numpy(c, p.out_dtype), ref, p.out_dtype, "widened preshuffled")
    finally:
        g.close()


@pytest.mark.parametrize("M,N,K,S,fa,fb", [(48, 700, 4096, 0, E2M1, E4M3), (300, 260, 2048, 4, E3M2, E5M2)])
def test_widened_split_k(M, N, K, S, fa, fb):
    p = mi.random_problem(M, N, K, seed=2600 + S, fmtA=fa, fmtB=fb, use_acc=True)
    rows, cols = mi.sample_points(M, N, 8192, seed=S, edge=64)
    ref = oracle_points(p, rows, cols)
    g = L.Gemm()
    g.enable_split_k()
    try:
        g.set_splits(S)
        log(f"widened split M={M} N={N} K={K} S={S}")
        got = run(g, p, AUTO)
        compare(got[rows, cols], ref, p.out_dtype, f"widened split S={S}")
    finally:
        g.close()


def test_widened_noalloc():
    """mxgemm_run_noalloc rewrites into the attached operand buffer (caller
    memory) and splits K in the library's scratch: within the rule, on two
    calls in a row, the second smaller."""
    g = L.Gemm()
    try:
        for M, N, K, fa, fb in ((300, 260, 1056, E3M2, E4M3), (40, 200, 512, E4M3, E2M1)):
            p = mi.random_problem(M, N, K, seed=2700 + M, fmtA=fa, fmtB=fb)
            A, As, B, Bs = to_dev(p)
            need = L.mxgemm_operand_buffer_bytes(fa, fb, M, N, K)
            assert need > 0
            ob = torch.empty(need, dtype=torch.uint8, device="cuda")
            L.mxgemm_set_operand_buffer(g.h, ob, need)
            buf, c = alloc_c(p, 64)
            log(f"widened noalloc {M}x{N}x{K}")
            L.mxgemm_run_noalloc(g.h, A, As, fa, B, Bs, fb, c, M, N, K, 0, p.out_dtype)
            torch.cuda.synchronize()
            g0, g1 = buf[:64].cpu().numpy(), buf[-64:].cpu().numpy()
            assert np.all(g0 == 1.5) and np.all(g1 == -2.25), "store outside C"
            compare(c_numpy(c, p.out_dtype), oracle_full(p), p.out_dtype, f"widened noalloc {M}")
    finally:
        g.close()


def test_widened_error_paths():
    """Widened pairs without a usable operand buffer, and bad formats, are
    rejected before any launch: C keeps its NaN fill."""
    M, N, K = 64, 64, 128
    p = mi.random_problem(M, N, K, seed=2800, fmtA=E3M2, fmtB=E4M3)
    A, As, B, Bs = to_dev(p)
    buf, c = alloc_c(p)
    g = L.Gemm()
    code = lambda name: L.STATUS_CODE[name]
    try:
        def rejected(name, fa=E3M2, fb=E4M3, C=c):
            with pytest.raises(L.MxgemmError) as e:
                L.mxgemm_run(g.h, A, As, fa, B, Bs, fb, C, M, N, K, 0, 0)
            assert e.value.code == code(name), (name, e.value.code)

        rejected("MXGEMM_ERR_WORKSPACE")                     # none attached
        need = L.mxgemm_operand_buffer_bytes(E3M2, E4M3, M, N, K)
        assert need == M * K
        short = torch.empty(need, dtype=torch.uint8, device="cuda")
        L.mxgemm_set_operand_buffer(g.h, short, need - 256)
        rejected("MXGEMM_ERR_WORKSPACE")                     # too short
        # a buffer whose needed bytes overlap C
        big = torch.full((M * N * 4 + need,), 0, dtype=torch.uint8, device="cuda")
        cb = big[: M * N * 4].view(torch.float32).view(M, N)
        cb.fill_(float("nan"))
        L.mxgemm_set_operand_buffer(g.h, big, need)
        rejected("MXGEMM_ERR_ALIAS", C=cb)
        assert bool(torch.isnan(cb).all())
        # one that overlaps A
        L.mxgemm_set_operand_buffer(g.h, A, need)
        rejected("MXGEMM_ERR_ALIAS")
        rejected("MXGEMM_ERR_FMT", fa=5)
        with pytest.raises(L.MxgemmError) as e:
            L.mxgemm_set_operand_buffer(g.h, big[16:], need)
        assert e.value.code == code("MXGEMM_ERR_WORKSPACE")
        # mxgemm_widen's own checks
        dst = torch.empty(M * K + 64, dtype=torch.uint8, device="cuda")
        for args, name in (((A, E4M3, M, K, dst), "MXGEMM_ERR_FMT"),
                           ((A, E3M2, M, 48, dst), "MXGEMM_ERR_SHAPE"),
                           ((A, E3M2, M, K, dst[8:]), "MXGEMM_ERR_ALIGN"),
                           ((A, E3M2, M, K, A), "MXGEMM_ERR_ALIAS")):
            with pytest.raises(L.MxgemmError) as e:
                L.mxgemm_widen(g.h, *args)
            assert e.value.code == code(name), name
        torch.cuda.synchronize()
        assert bool(torch.isnan(buf).all()), "a rejected call wrote C"
    finally:
        g.close()


WIDE_EDGE_CASES = [
    # M, N, K, fmtA, fmtB, variants
    (2, 3, 1 << 21, E3M2, E4M3, (AUTO, LARGE)),     # the largest K: a 1.5 MiB packed row of A
    (3, 1 << 20, 64, E4M3, E2M3, (AUTO, LARGE)),    # the largest N: B rewritten, 64 MiB of e4m3
    (70000, 40, 64, E2M1, E5M2, (AUTO,)),           # many row tiles, ragged last tile
]


@pytest.mark.parametrize("case", WIDE_EDGE_CASES, ids=lambda c: "x".join(map(str, c[:3])))
def test_widened_edge_full(gemm, case):
    """Widened pairs at the limits of the C ABI, full outputs against the
    oracle, with the guard bands around C intact."""
    M, N, K, fa, fb, variants = case
    p = mi.random_problem(M, N, K, seed=(M * 5 + N * 7 + K) % 100019, fmtA=fa, fmtB=fb)
    ref = oracle_full(p)
    dev = to_dev(p)
    for v in variants:
        log(f"widened edge {case[:5]} variant={v}")
        got = run(gemm, p, v, guard=64, dev_inputs=dev)
        compare(got, ref, p.out_dtype, f"widened edge {case[:5]} {v}")
    gemm.set_variant(AUTO)
