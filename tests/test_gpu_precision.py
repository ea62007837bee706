"""How each MFMA family sums: probes on the device, through the C ABI.

These pin the device readings behind the choice of the default path:

  d2  the gfx950 scaled MFMA (v_mfma_scale_f32_*_f8f6f4, the native
      variants) sums each aligned group of 8 consecutive K products in a
      fixed-point window that ends 13 bits below the group's largest
      product; bits below it are dropped (toward zero, whatever the sign).
      Products of different groups, and of different 32-K scale blocks of
      one instruction, are combined without that loss.
  d3  the bf16 MFMA (the exact variants, after the scaled decode) forms
      exact products and rounds once per instruction to fp32.
  f4  e2m1 x e2m1 products of one block all fit the window, so the scaled
      MFMA is exact for them, at every scale byte.

Together they show why the exact variants decode to bf16: a product
2^-14 below a group's largest is lost by the scaled MFMA, an error of
6.1e-5 * sum|ab| against the 1e-5 rule, while the bf16 path keeps it.
"""
import numpy as np
import pytest
import torch

import level_dsl_amd as L
import mxinputs as mi
import oracle
from gpu_helpers import log, oracle_full, run

pytestmark = pytest.mark.gpu

LARGE, SKINNY = L.MXGEMM_VARIANT_LARGE, L.MXGEMM_VARIANT_SKINNY
LARGE_NATIVE, SKINNY_NATIVE = L.MXGEMM_VARIANT_LARGE_NATIVE, L.MXGEMM_VARIANT_SKINNY_NATIVE
EXACT = [LARGE, SKINNY]
NATIVE = [LARGE_NATIVE, SKINNY_NATIVE]
VNAME = {LARGE: "large", SKINNY: "skinny", LARGE_NATIVE: "large_native",
         SKINNY_NATIVE: "skinny_native"}


@pytest.fixture(scope="module")
def gemm():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    g = L.Gemm()
    yield g
    g.close()


def e4m3_pow2(e):
    """e4m3 code of 2^-e, e = 0..9 (normal down to 2^-6, then subnormals)."""
    return (7 - e) << 3 if e <= 6 else {7: 0x04, 8: 0x02, 9: 0x01}[e]


def group_probe(j, sign):
    """C[e, f] = 1 + sign * 2^-(e + f): 1.0 * 1.0 at k = 0 and
    (sign 2^-e) * 2^-f at k = j, all scales 127, K = 64."""
    M = N = 10
    K = 64
    A = np.zeros((M, K), np.uint8)
    B = np.zeros((N, K), np.uint8)
    A[:, 0] = 0x38
    B[:, 0] = 0x38
    for e in range(10):
        A[e, j] = e4m3_pow2(e) | (0x80 if sign < 0 else 0)
        B[e, j] = e4m3_pow2(e)
    return mi.Problem(M, N, K, 0, 0, A, np.full((M, 2), 127, np.uint8), B,
                      np.full((N, 2), 127, np.uint8), mi.OUT_F32, False)


@pytest.mark.parametrize("sign", [1, -1])
@pytest.mark.parametrize("j", [1, 7, 8, 16, 32])
def test_group_window(gemm, j, sign):
    """A product 2^-t below the largest one: the exact variants keep it for
    every t up to 18; the native variants keep it up to t = 13 and drop it
    from t = 14 when it shares the largest product's group of 8 (k = 1..7),
    and keep it when it sits in another group (k = 8, 16) or block (k = 32).
    At t = 14..16 the drop breaks the 1e-5 * sum|ab| rule."""
    p = group_probe(j, sign)
    t = np.add.outer(np.arange(10), np.arange(10))
    exact = 1.0 + sign * np.ldexp(1.0, -t)
    for v in EXACT + NATIVE:
        log(f"group window j={j} sign={sign} {VNAME[v]}")
        got = run(gemm, p, v).astype(np.float64)
        if v in EXACT or j >= 8:
            assert np.array_equal(got, exact), f"{VNAME[v]}: {got[got != exact]} vs {exact[got != exact]}"
        else:
            want = np.where(t <= 13, exact, 1.0)
            assert np.array_equal(got, want), f"{VNAME[v]}: {got[got != want]} vs {want[got != want]}"
            err = np.abs(got - exact) / (1.0 + np.ldexp(1.0, -t))
            assert np.all(err[(t >= 14) & (t <= 16)] > 1e-5)


def test_scale_blocks_of_one_instruction(gemm):
    """1.0 in block 0 and 1.875 * 2^-t in block 1 (scale byte 127 - t,
    t = 10..40) of one 64-K MFMA: every variant returns the oracle's result
    bit for bit, so the scaled MFMA applies the block scales before it sums
    the blocks and loses nothing across them."""
    M = N = 64
    K = 64
    A = np.zeros((M, K), np.uint8)
    B = np.zeros((N, K), np.uint8)
    A[:, 0] = 0x38
    B[:, 0] = 0x38
    A[:, 32] = 0x3F  # 1.875
    B[:, 32] = 0x38
    As = np.full((M, 2), 127, np.uint8)
    ts = np.arange(10, 41)
    As[:len(ts), 1] = 127 - ts
    p = mi.Problem(M, N, K, 0, 0, A, As, B, np.full((N, 2), 127, np.uint8), mi.OUT_F32, False)
    ref = oracle_full(p)["ref32"]
    for v in EXACT + NATIVE:
        log(f"scale blocks {VNAME[v]}")
        got = run(gemm, p, v)
        assert np.array_equal(got, ref), f"{VNAME[v]}: {np.sum(got != ref)} mismatches"


def test_bf16_mfma_rounds_once(gemm):
    """2^16 + 2^-8 + 2^-8 inside one MFMA: rounded once, the sum is
    2^16 (1 + 2^-23) exactly (the exact variants); rounded after each add it
    would be 2^16; the scaled MFMA drops both small products (24 bits below
    the group's largest)."""
    M = N = 16
    K = 32
    A = np.zeros((M, K), np.uint8)
    B = np.zeros((N, K), np.uint8)
    A[:, 0] = B[:, 0] = 0x78          # 2^8
    A[:, 1:3] = B[:, 1:3] = 0x18      # 2^-4
    p = mi.Problem(M, N, K, 0, 0, A, np.full((M, 1), 127, np.uint8), B,
                   np.full((N, 1), 127, np.uint8), mi.OUT_F32, False)
    once = np.float32(65536.0 * (1 + 2.0**-23))
    for v in EXACT:
        assert np.all(run(gemm, p, v) == once), VNAME[v]
    for v in NATIVE:
        assert np.all(run(gemm, p, v) == np.float32(65536.0)), VNAME[v]


E2M1_VALUES = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


@pytest.mark.parametrize("sa,sb", [(127, 127), (1, 254), (0, 254), (254, 0), (0, 127),
                                   (254, 254), (255, 127), (127, 255)])
def test_e2m1_exact_at_every_scale(gemm, sa, sb):
    """e2m1: every product of two codes, at extreme scale bytes (0 is
    2^-127, 254 is 2^127, 255 is NaN), equals the oracle bit for bit on the
    scaled MFMA (256 x 256 kernel and small-M kernel)."""
    M = N = 16
    K = 64
    a = np.zeros((M, K), np.uint8)
    b = np.zeros((N, K), np.uint8)
    a[:, 0] = np.arange(16)
    b[:, 0] = np.arange(16)
    p = mi.Problem(M, N, K, 4, 4, mi.pack_e2m1(a), np.full((M, 2), sa, np.uint8), mi.pack_e2m1(b),
                   np.full((N, 2), sb, np.uint8), mi.OUT_F32, False)
    ref = oracle_full(p)["ref32"]
    for v in (LARGE, SKINNY):
        got = run(gemm, p, v)
        assert np.array_equal(np.isnan(got), np.isnan(ref)), VNAME[v]
        fin = ~np.isnan(ref)
        assert np.array_equal(got[fin], ref[fin]), VNAME[v]


def test_e2m1_group_spread_exact(gemm):
    """One group of 8 e2m1 products spanning the whole format range
    (6 * 6 = 36 down to 0.5 * 0.5 = 0.25): the sum is exact."""
    M = N = 8
    K = 64
    a = np.zeros((M, K), np.uint8)
    b = np.zeros((N, K), np.uint8)
    g = np.random.Generator(np.random.PCG64(77))
    a[:, :8] = g.integers(0, 16, size=(M, 8))
    b[:, :8] = g.integers(0, 16, size=(N, 8))
    a[:, 0] = b[:, 0] = 7             # 6.0
    a[:, 1] = b[:, 1] = 1             # 0.5
    p = mi.Problem(M, N, K, 4, 4, mi.pack_e2m1(a), np.full((M, 2), 127, np.uint8), mi.pack_e2m1(b),
                   np.full((N, 2), 127, np.uint8), mi.OUT_F32, False)
    ref = oracle_full(p)["ref32"]
    for v in (LARGE, SKINNY):
        assert np.array_equal(run(gemm, p, v), ref), VNAME[v]


def test_native_breaks_the_rule_on_random_data(gemm):
    """The 256^3 workload (e4m3 from N(0,1), scales U{123..131}): the native
    variant leaves hundreds of the 65,536 outputs outside 1e-5 * sum|ab|
    (538 when measured), the exact variant none."""
    p = mi.workload(0)
    ref = oracle_full(p)
    for v, want_bad in ((LARGE, False), (LARGE_NATIVE, True)):
        got = run(gemm, p, v).astype(np.float64)
        rel = np.abs(got - ref["ref32"]) / ref["mag"]
        n_bad = int(np.sum(rel > 1e-5))
        log(f"{VNAME[v]}: max |err| / sum|ab| = {rel.max():.3g}, {n_bad} outside 1e-5")
        assert (n_bad > 100) if want_bad else (n_bad == 0), (VNAME[v], n_bad)
