"""Pins of the CPU oracle to facts outside itself.

Each ``pin_*`` function takes a loaded oracle library (the real one, or a
mutant compiled by the planted-mistake test) and raises AssertionError if
the oracle disagrees with:
  * torch's own float8 / bf16 conversions (a library routine independent of
    the oracle's bit-field decoders),
  * the OCP spot values stored in tests/golden/,
  * exact rational arithmetic (fractions.Fraction) on tiny inputs,
  * closed forms, the integer matrix product, and exact invariants of the
    definition (power-of-two scale doubling, permutation inputs).

What is pinned is the definition of the scaled dot given as async_dot_scaled
in the TLX API Quick Reference ("Matrix Multiply (MMA)": D = (A*scale_A) @
(B*scale_B) + D) with one uint8 scale per 32 K-elements (TLX async-compute
page, "TMEM-backed MX Scales", K extent BLOCK_K // 32), and the block
quantization that produces such operands (the ``pin_quant_*`` functions:
torch's round-to-nearest-even float8 casts, the block exponent's defining
inequality evaluated directly, power-of-two invariance, and the input
generator's own torch-based quantizer).
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import torch

import oracle
import mxinputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
E8 = oracle.FMT_E8M0  # the scale format
FMT_NAMES = {"e4m3": 0, "e5m2": 1, "e8m0": E8}
_TORCH = {0: torch.float8_e4m3fn, 1: torch.float8_e5m2, E8: torch.float8_e8m0fnu}


def torch_decode(fmt: int) -> np.ndarray:
    codes = torch.arange(256, dtype=torch.uint8)
    return codes.view(_TORCH[fmt]).to(torch.float64).numpy()


def same(a, b, signed_zero: bool = False) -> bool:
    """Equal as floats with NaN equal to NaN; the sign of zero counts only
    when signed_zero is set (a sum that is exactly zero has no fixed sign)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = a == b
    if signed_zero:
        eq &= np.signbit(a) == np.signbit(b)
    return bool(np.all(both_nan | eq))


def bf16_bits_to_float(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def _parse_value(tok: str) -> float:
    if tok == "-0":
        return -0.0
    if tok.startswith("0x") or tok.startswith("-0x"):
        return float.fromhex(tok)
    return float(tok)


def golden_spot_values():
    out = []
    with open(os.path.join(GOLDEN, "ocp_fp8_spot_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fmt, code, val = line.split()
            out.append((FMT_NAMES[fmt], int(code, 16), _parse_value(val)))
    return out


# ---------------------------------------------------------------- formats --

def pin_tables_match_torch(lib):
    for fmt in (0, 1, E8):
        got = oracle.decode_table(fmt, lib)
        want = torch_decode(fmt)
        assert same(got, want, signed_zero=True), \
            f"format {fmt}: oracle table differs from torch's float8 view"


def pin_spot_values(lib):
    for fmt, code, val in golden_spot_values():
        got = lib.mxref_decode(fmt, code)
        assert same(got, val, signed_zero=True), f"format {fmt} code {code:#04x}: {got!r} != {val!r}"


def pin_special_counts(lib):
    e4 = oracle.decode_table(0, lib)
    e5 = oracle.decode_table(1, lib)
    e8 = oracle.decode_table(oracle.FMT_E8M0, lib)
    assert np.isnan(e4).sum() == 2 and np.isinf(e4).sum() == 0
    assert np.isnan(e5).sum() == 6 and np.isinf(e5).sum() == 2
    assert np.isnan(e8).sum() == 1 and np.isinf(e8).sum() == 0
    fin4, fin5 = e4[np.isfinite(e4)], e5[np.isfinite(e5)]
    assert fin4.max() == 448.0 and fin4.min() == -448.0
    assert fin5.max() == 57344.0 and fin5.min() == -57344.0
    # every finite positive value appears once (no duplicate encodings but +-0)
    assert len(np.unique(fin4[fin4 > 0])) == 126 and len(np.unique(fin5[fin5 > 0])) == 123


def pin_bf16_rne(lib):
    g = np.random.Generator(np.random.PCG64(4242))
    x = g.standard_normal(4000).astype(np.float32) * np.float32(3.0)
    bits = g.integers(0, 2**32, size=4000, dtype=np.uint64).astype(np.uint32)
    y = bits.view(np.float32)
    # exact ties: low 16 bits 0x8000, both parities of bit 16
    ties = (np.arange(64, dtype=np.uint32) * 0x10000 + 0x3f808000).view(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38,
                        1e-45, 1.17549435e-38, 65504.0], dtype=np.float32)
    allv = np.concatenate([x, y, ties, special])
    got = oracle.bf16_rne(allv, lib)
    want = torch.from_numpy(allv).to(torch.bfloat16).view(torch.uint16).numpy()
    fin = ~np.isnan(allv)
    assert np.array_equal(got[fin], want[fin]), "bf16 RNE differs from torch's cast"
    nanout = got[~fin]
    assert np.all((nanout & 0x7f80) == 0x7f80) and np.all((nanout & 0x007f) != 0)


# ------------------------------------------------------------ the product --

def _exact_value(code: int, fmt: int, dec) -> Fraction:
    return Fraction(float(dec[fmt][code]))


def pin_bruteforce_fraction(lib):
    """Tiny random problems: the oracle's double sum is within Higham's
    recursive-summation bound of the exact rational sum, its fp32 result is
    the correct rounding whenever the double sum is exact, and never more
    than one fp32 ulp away."""
    dec = {f: torch_decode(f) for f in (0, 1, E8)}
    cases = [(3, 4, 64, 0, 0, False, 0), (2, 3, 96, 1, 0, False, 0), (4, 2, 40, 0, 1, False, 0),
             (3, 3, 256, 1, 1, True, 0), (2, 2, 33, 0, 0, True, 1), (1, 1, 1, 1, 1, False, 0),
             (4, 4, 160, 0, 0, True, 0)]
    for i, (M, N, K, fa, fb, acc, cdt) in enumerate(cases):
        p = mxinputs.random_problem(M, N, K, seed=50 + i, fmtA=fa, fmtB=fb, scale_lo=110,
                                    scale_hi=140, use_acc=acc,
                                    out_dtype=mxinputs.OUT_BF16 if cdt else mxinputs.OUT_F32)
        r = oracle.gemm_full(p.A, p.As, fa, p.B, p.Bs, fb, M, N, K, cin=p.Cin, nthreads=2, lib=lib)
        for m in range(M):
            for n in range(N):
                exact = Fraction(0)
                mag = Fraction(0)
                for k in range(K):
                    t = (_exact_value(p.A[m, k], fa, dec) * _exact_value(p.As[m, k // 32], E8, dec)
                         * _exact_value(p.B[n, k], fb, dec) * _exact_value(p.Bs[n, k // 32], E8, dec))
                    exact += t
                    mag += abs(t)
                if acc:
                    if cdt == 0:
                        c = Fraction(float(p.Cin[m, n]))
                    else:
                        c = Fraction(float(bf16_bits_to_float(p.Cin[m, n])))
                    exact += c
                    mag += abs(c)
                s = r["sum"][m, n]
                bound = Fraction(K + 1) * Fraction(2) ** -53 * mag
                assert abs(Fraction(s) - exact) <= bound, f"case {i} ({m},{n}): sum off"
                assert float(mag) == r["mag"][m, n] or abs(Fraction(r["mag"][m, n]) - mag) <= bound
                want32 = np.float32(float(exact))  # double rounding only if exact not a double
                if Fraction(float(exact)) == exact:
                    assert r["ref32"][m, n] == want32, f"case {i} ({m},{n}): fp32 rounding"
                else:
                    ulp = np.spacing(np.float32(abs(want32)))
                    assert abs(float(r["ref32"][m, n]) - float(want32)) <= ulp


def _pairwise(lib, fa, fb, sa, sb):
    """M = N = 256, K = 32: A[m,0] = code m, B[0,n] = code n, all else 0."""
    M = N = 256
    K = 32
    A = np.zeros((M, K), np.uint8)
    B = np.zeros((N, K), np.uint8)
    A[:, 0] = np.arange(256, dtype=np.uint8)
    B[:, 0] = np.arange(256, dtype=np.uint8)
    As = np.full((M, 1), sa, np.uint8)
    Bs = np.full((N, 1), sb, np.uint8)
    return oracle.gemm_full(A, As, fa, B, Bs, fb, M, N, K, nthreads=4, lib=lib)


def pin_pairwise_products(lib):
    """Every pair of codes, for every format pair and several scale bytes:
    C[m,n] is exactly dec(m) * dec(n) * 2^(sa+sb-254)."""
    dec = {f: torch_decode(f) for f in (0, 1)}
    for fa in (0, 1):
        for fb in (0, 1):
            for sa, sb in ((127, 127), (0, 127), (127, 1), (126, 128), (253, 254), (254, 254),
                           (1, 0), (100, 140)):
                r = _pairwise(lib, fa, fb, sa, sb)
                scale = math.ldexp(1.0, sa - 127) * math.ldexp(1.0, sb - 127)
                want = np.outer(dec[fa], dec[fb])
                with np.errstate(invalid="ignore", over="ignore"):
                    want = want * scale  # a power of two times an exact product
                    # inf * 0 from the zero padding terms is NaN in the definition too
                    assert same(r["sum"], want), f"pairwise fa={fa} fb={fb} sa={sa} sb={sb}"
                    want32 = want.astype(np.float32)   # numpy's IEEE rounding to fp32
                assert same(r["ref32"], want32), f"pairwise fp32 fa={fa} fb={fb} sa={sa} sb={sb}"


def pin_closed_form(lib):
    """A = B = 1.0 (code 0x38) everywhere with constant scales:
    C = K * 2^(sa + sb - 254) exactly."""
    for K, sa, sb, fa, fb in ((32, 127, 127, 0, 0), (96, 130, 120, 0, 0), (1024, 140, 100, 0, 0),
                              (320, 127, 128, 1, 1), (4096, 5, 250, 0, 1)):
        M, N = 3, 5
        c1 = {0: 0x38, 1: 0x3C}
        A = np.full((M, K), c1[fa], np.uint8)
        B = np.full((N, K), c1[fb], np.uint8)
        As = np.full((M, K // 32), sa, np.uint8)
        Bs = np.full((N, K // 32), sb, np.uint8)
        r = oracle.gemm_full(A, As, fa, B, Bs, fb, M, N, K, nthreads=1, lib=lib)
        want = K * math.ldexp(1.0, sa + sb - 254)
        assert np.all(r["sum"] == want) and np.all(r["ref32"] == np.float32(want)), f"K={K}"
        assert np.all(r["mag"] == want)


def pin_integer_gemm(lib):
    """Codes restricted to integers (e4m3: -16..16, e5m2: -8..8), scales 1.0:
    C equals the int64 matrix product exactly."""
    for fa, fb, seed in ((0, 0, 1), (1, 0, 2), (0, 1, 3), (1, 1, 4)):
        g = np.random.Generator(np.random.PCG64(seed))
        M, N, K = 37, 29, 544
        lim = {0: 16, 1: 8}
        ia = g.integers(-lim[fa], lim[fa] + 1, size=(M, K))
        ib = g.integers(-lim[fb], lim[fb] + 1, size=(N, K))
        A = mxinputs.quantize(ia.astype(np.float32), fa)
        B = mxinputs.quantize(ib.astype(np.float32), fb)
        As = np.full((M, K // 32), 127, np.uint8)
        Bs = np.full((N, K // 32), 127, np.uint8)
        r = oracle.gemm_full(A, As, fa, B, Bs, fb, M, N, K, nthreads=3, lib=lib)
        want = ia.astype(np.int64) @ ib.astype(np.int64).T
        assert np.array_equal(r["sum"], want.astype(np.float64)), f"integer gemm {fa},{fb}"
        assert np.array_equal(r["ref32"], want.astype(np.float32))


def pin_scale_doubling(lib):
    """Adding 1 to every A-scale byte of row m (or B-scale byte of column n)
    doubles that row (column) exactly; bumping one block's byte changes only
    that block's contribution, by exactly its own value."""
    p = mxinputs.random_problem(9, 7, 256, seed=77)
    M, N, K = p.M, p.N, p.K
    base = oracle.gemm_full(p.A, p.As, 0, p.B, p.Bs, 0, M, N, K, lib=lib)
    As2 = p.As.copy(); As2[4, :] += 1
    r = oracle.gemm_full(p.A, As2, 0, p.B, p.Bs, 0, M, N, K, lib=lib)
    assert np.array_equal(r["sum"][4], 2 * base["sum"][4])
    assert np.array_equal(r["ref32"][4], 2 * base["ref32"][4])
    mask = np.ones(M, bool); mask[4] = False
    assert np.array_equal(r["sum"][mask], base["sum"][mask])
    Bs2 = p.Bs.copy(); Bs2[2, :] += 1
    r = oracle.gemm_full(p.A, p.As, 0, p.B, Bs2, 0, M, N, K, lib=lib)
    assert np.array_equal(r["ref32"][:, 2], 2 * base["ref32"][:, 2])
    # one block: the difference equals that block's partial sum
    As3 = p.As.copy(); As3[1, 3] += 1
    r = oracle.gemm_full(p.A, As3, 0, p.B, p.Bs, 0, M, N, K, lib=lib)
    blk = np.zeros((M, K), np.uint8); blk[:, 96:128] = p.A[:, 96:128]
    part = oracle.gemm_full(blk, p.As, 0, p.B, p.Bs, 0, M, N, K, lib=lib)
    assert np.allclose(r["sum"][1] - base["sum"][1], part["sum"][1], rtol=1e-12, atol=0)
    assert np.array_equal(r["sum"][0], base["sum"][0])


def pin_permutation(lib):
    """A a permutation matrix of 1.0 codes with scale bytes 127: C[m,n] is the
    scaled B element at K index pi(m); and the same with B a permutation."""
    dec = {f: torch_decode(f) for f in (0, 1, E8)}
    g = np.random.Generator(np.random.PCG64(11))
    M = N = 64
    K = 128
    pi = g.permutation(K)[:M]
    p = mxinputs.random_problem(M, N, K, seed=12, fmtB=1)
    A = np.zeros((M, K), np.uint8); A[np.arange(M), pi] = 0x38
    As = np.full((M, K // 32), 127, np.uint8)
    r = oracle.gemm_full(A, As, 0, p.B, p.Bs, 1, M, N, K, lib=lib)
    want = dec[1][p.B[:, pi].T] * dec[E8][p.Bs[:, pi // 32].T]
    assert same(r["sum"], want), "A = permutation"
    sigma = g.permutation(K)[:N]
    B = np.zeros((N, K), np.uint8); B[np.arange(N), sigma] = 0x38
    Bs = np.full((N, K // 32), 127, np.uint8)
    r = oracle.gemm_full(p.A, p.As, 0, B, Bs, 0, M, N, K, lib=lib)
    want = dec[0][p.A[:, sigma]] * dec[E8][p.As[:, sigma // 32]]
    assert same(r["sum"], want), "B = permutation"


def pin_numpy_matmul(lib):
    """Medium random problems, including a K that is not a multiple of 32 and
    use_acc with an fp32 and a bf16 C: the oracle agrees with numpy's float64
    matmul of the decoded, scaled operands (torch decode) within 1e-12 * mag."""
    for i, (M, N, K, fa, fb, acc, outd) in enumerate((
            (70, 53, 512, 0, 0, False, 0), (33, 65, 200, 1, 0, True, 0),
            (48, 17, 96, 0, 1, True, 1), (20, 20, 1000, 1, 1, False, 0))):
        p = mxinputs.random_problem(M, N, K, seed=300 + i, fmtA=fa, fmtB=fb, use_acc=acc,
                                    out_dtype=outd)
        dec = {f: torch_decode(f) for f in (0, 1, E8)}
        sa = np.repeat(dec[E8][p.As], 32, axis=1)[:, :K]
        sb = np.repeat(dec[E8][p.Bs], 32, axis=1)[:, :K]
        a = dec[fa][p.A] * sa
        b = dec[fb][p.B] * sb
        want = a @ b.T
        mag = np.abs(a) @ np.abs(b).T
        if acc:
            if outd == 0:
                c = p.Cin.astype(np.float64)
            else:
                c = bf16_bits_to_float(p.Cin).astype(np.float64)
            want = want + c
            mag = mag + np.abs(c)
        r = oracle.gemm_full(p.A, p.As, fa, p.B, p.Bs, fb, M, N, K, cin=p.Cin, lib=lib)
        assert np.all(np.abs(r["sum"] - want) <= 1e-12 * mag + 1e-300), f"case {i}"
        assert np.allclose(r["mag"], mag, rtol=1e-12, atol=0)
        if outd == 1:
            want_bf = torch.from_numpy(r["ref32"]).to(torch.bfloat16).view(torch.uint16).numpy()
            assert np.array_equal(r["refbf16"], want_bf)


def pin_nan_propagation(lib):
    """A NaN code or a NaN scale byte (255) poisons exactly the outputs it
    reaches; an e5m2 infinity times a nonzero value gives an infinity."""
    p = mxinputs.random_problem(6, 5, 64, seed=90)
    A = p.A.copy(); A[2, 17] = 0x7F                     # e4m3 NaN
    Bs = p.Bs.copy(); Bs[3, 1] = 255                   # NaN scale on column 3
    r = oracle.gemm_full(A, p.As, 0, p.B, Bs, 0, 6, 5, 64, lib=lib)
    nan = np.isnan(r["ref32"])
    want = np.zeros((6, 5), bool); want[2, :] = True; want[:, 3] = True
    assert np.array_equal(nan, want)
    A5 = np.full((1, 32), 0x3C, np.uint8); A5[0, 0] = 0x7C  # +inf in e5m2
    B = np.full((1, 32), 0x38, np.uint8)
    r = oracle.gemm_full(A5, np.full((1, 1), 127, np.uint8), 1, B,
                         np.full((1, 1), 127, np.uint8), 0, 1, 1, 32, lib=lib)
    assert r["ref32"][0, 0] == np.inf


def pin_thread_independence(lib):
    p = mxinputs.random_problem(31, 23, 320, seed=5)
    outs = [oracle.gemm_full(p.A, p.As, 0, p.B, p.Bs, 0, 31, 23, 320, nthreads=t, lib=lib)
            for t in (1, 3, 8)]
    for o in outs[1:]:
        assert np.array_equal(o["sum"].view(np.int64), outs[0]["sum"].view(np.int64))


def pin_scale_tile_extent(lib):
    """The page's scale tiles: (rows, K//32) bytes, one per 32 K-elements.
    With scale byte j of row 0 raised by one, only K-elements 32j..32j+31
    of that row are doubled."""
    with open(os.path.join(GOLDEN, "scale_tile_shapes.txt")) as f:
        tiles = [tuple(int(t) for t in ln.split()) for ln in f
                 if ln.strip() and not ln.startswith("#")]
    for nrows, cols, kcov in tiles:
        assert kcov == 32 * cols
        K, M, N = kcov, nrows, 2
        for j in range(cols):
            A = np.zeros((M, K), np.uint8)
            A[0, 32 * j: 32 * j + 32] = 0x38        # 1.0 inside block j only
            B = np.full((N, K), 0x38, np.uint8)
            Bs = np.full((N, cols), 127, np.uint8)
            As = np.full((M, cols), 127, np.uint8)
            As[0, j] = 128
            r = oracle.gemm_full(A, As, 0, B, Bs, 0, M, N, K, lib=lib)
            assert np.all(r["sum"][0] == 64.0) and np.all(r["sum"][1:] == 0.0)
            As[0, j] = 127
            As[0, (j + 1) % cols] = 128
            r = oracle.gemm_full(A, As, 0, B, Bs, 0, M, N, K, lib=lib)
            assert np.all(r["sum"][0] == 32.0)


# ------------------------------------------------------- block quantization --

QMAX = {0: 448.0, 1: 57344.0}


def _quant_probe_values(fmt: int, n: int, seed: int) -> np.ndarray:
    """Values with |v| <= MAX: log-uniform magnitudes down into the
    subnormal range, exact midpoints between neighbouring codes (ties), the
    fp32 neighbours of those midpoints, zeros of both signs."""
    g = np.random.Generator(np.random.PCG64(seed))
    mx = QMAX[fmt]
    mag = np.exp2(g.uniform(-22.0, np.log2(mx), n)).astype(np.float32)
    sgn = np.where(g.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
    tab = torch_decode(fmt)[:128]
    fin = np.sort(tab[np.isfinite(tab)])
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)       # exact in fp32
    up = np.nextafter(mids, np.float32(np.inf)).astype(np.float32)
    dn = np.nextafter(mids, np.float32(0)).astype(np.float32)
    extra = np.concatenate([mids, -mids, up, -up, dn, -dn, fin.astype(np.float32),
                            -fin.astype(np.float32), np.float32([0.0, -0.0])])
    return np.concatenate([mag * sgn, extra]).astype(np.float32)


def pin_quant_rne_vs_torch(lib):
    """Blocks whose largest magnitude is exactly MAX get scale 127 (2^0), so
    each code must be torch's RNE float8 cast of the value itself."""
    for fmt in (0, 1):
        v = _quant_probe_values(fmt, 20000, seed=11 + fmt)
        nb = (v.size + 30) // 31
        v = np.concatenate([v, np.zeros(nb * 31 - v.size, np.float32)])
        X = np.empty((nb, 32), np.float32)
        X[:, 0] = np.where(np.arange(nb) % 2 == 0, QMAX[fmt], -QMAX[fmt])
        X[:, 1:] = v.reshape(nb, 31)
        codes, scales = oracle.quantize(X, fmt, lib=lib)
        assert np.all(scales == 127), "scale of a block whose max is MAX"
        want = torch.from_numpy(X).to(_TORCH[fmt]).view(torch.uint8).numpy()
        assert np.array_equal(codes, want), f"{np.sum(codes != want)} codes differ from torch ({fmt})"


def pin_quant_block_exponent(lib):
    """scale byte b satisfies the definition: amax <= MAX*2^(b-127), and b is
    0 or amax > MAX*2^(b-128) (the smallest such e), over the whole fp32
    range including subnormals; an all-zero block has b = 0."""
    g = np.random.Generator(np.random.PCG64(21))
    for fmt in (0, 1):
        rows = 4000
        amax = np.exp2(g.uniform(-148.0, 127.9, rows)).astype(np.float32)
        amax[:8] = np.float32([0.0, 2.0**-149, QMAX[fmt], np.nextafter(np.float32(QMAX[fmt]), 0),
                               np.nextafter(np.float32(QMAX[fmt]), np.float32(1e9)), 1.0,
                               3.4e38, 2.0**-126])
        X = (g.uniform(-1, 1, (rows, 32)).astype(np.float32) * amax[:, None]).astype(np.float32)
        X[np.arange(rows), g.integers(0, 32, rows)] = amax * np.where(g.random(rows) < 0.5, -1, 1)
        codes, scales = oracle.quantize(X, fmt, lib=lib)
        am = np.abs(X.astype(np.float64)).max(axis=1)
        for r in range(rows):
            b = int(scales[r, 0])
            if am[r] == 0.0:
                assert b == 0
                continue
            assert am[r] <= math.ldexp(QMAX[fmt], b - 127), (fmt, am[r], b)
            assert b == 0 or am[r] > math.ldexp(QMAX[fmt], b - 128), (fmt, am[r], b)


def pin_quant_scale_invariance(lib):
    """X * 2^j (exact in fp32, no clamping) gives the same codes and every
    scale byte raised by j."""
    g = np.random.Generator(np.random.PCG64(31))
    X = (g.standard_normal((64, 256)) * np.exp2(g.integers(-6, 7, (64, 1)))).astype(np.float32)
    for fmt in (0, 1):
        c0, s0 = oracle.quantize(X, fmt, lib=lib)
        for j in (-9, 1, 13):
            c1, s1 = oracle.quantize((X * np.float32(2.0**j)).astype(np.float32), fmt, lib=lib)
            assert np.array_equal(c1, c0) and np.array_equal(s1.astype(int), s0.astype(int) + j)


def pin_quant_matches_generator(lib):
    """The input generator's quantizer (clamp + torch cast) on the skinny
    workload's recipe agrees with the oracle."""
    g = np.random.Generator(np.random.PCG64(41))
    for fmt in (0, 1):
        raw = (g.standard_normal((48, 1024)) * 0.02).astype(np.float32)
        want_c, want_s = mxinputs.mx_block_quantize(raw, fmt)
        codes, scales = oracle.quantize(raw, fmt, lib=lib)
        assert np.array_equal(scales, want_s) and np.array_equal(codes, want_c)


def pin_quant_bf16_input(lib):
    """bf16 input quantizes exactly as its fp32 widening."""
    g = np.random.Generator(np.random.PCG64(51))
    X = (g.standard_normal((16, 160)) * 3.0).astype(np.float32)
    bits = torch.from_numpy(X).to(torch.bfloat16).view(torch.uint16).numpy()
    wide = (bits.astype(np.uint32) << 16).view(np.float32)
    for fmt in (0, 1):
        a = oracle.quantize(bits, fmt, lib=lib)
        b = oracle.quantize(wide, fmt, lib=lib)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def pin_quant_ragged_and_nonfinite(lib):
    """A last block shorter than 32 is quantized on its own; a NaN or an
    infinity is rejected."""
    g = np.random.Generator(np.random.PCG64(61))
    X = g.standard_normal((5, 72)).astype(np.float32)
    X[:, 64:] *= np.float32(100.0)
    codes, scales = oracle.quantize(X, 0, lib=lib)
    tail_c, tail_s = oracle.quantize(np.ascontiguousarray(X[:, 64:]), 0, lib=lib)
    assert scales.shape == (5, 3)
    assert np.array_equal(codes[:, 64:], tail_c) and np.array_equal(scales[:, 2:], tail_s)
    for bad in (np.nan, np.inf):
        Y = X.copy()
        Y[2, 5] = bad
        try:
            oracle.quantize(Y, 0, lib=lib)
        except ValueError:
            continue
        raise AssertionError("non-finite input accepted")


# ------------------------------------------------------------- e2m1 (FP4) --

def _golden_e2m1():
    out = []
    with open(os.path.join(GOLDEN, "ocp_fp4_e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            out.append((int(code, 16), _parse_value(val)))
    return out


def pin_e2m1_golden(lib):
    """The e2m1 decoder against the OCP table (all 16 codes); codes above
    15 do not exist."""
    table = _golden_e2m1()
    assert len(table) == 16
    for code, val in table:
        got = lib.mxref_decode(4, code)
        assert same(got, val, signed_zero=True), f"e2m1 code {code:#x}: {got!r} != {val!r}"
    assert np.isnan(oracle.decode_table(4, lib)[16:]).all()


def _e2m1_as_e4m3(packed: np.ndarray) -> np.ndarray:
    """Re-encode packed e2m1 codes as e4m3 codes of the same value, using the
    test's own unpacking (low nibble = even k) and torch's e4m3 table."""
    e4 = torch_decode(0)
    vals = np.array([v for _, v in sorted(_golden_e2m1())])
    codes = mxinputs.unpack_e2m1(packed)
    want = vals[codes]
    out = np.empty(codes.shape, np.uint8)
    for c in range(16):
        hit = np.flatnonzero((e4 == vals[c]) & (np.signbit(e4) == np.signbit(vals[c])))
        assert hit.size, f"e2m1 value {vals[c]} is not an e4m3 value"
        out[codes == c] = hit[0]
    assert same(e4[out], want, signed_zero=True)
    return out


def pin_e2m1_embeds_in_e4m3(lib):
    """Every e2m1 value is an e4m3 value, so an e2m1 problem and the same
    problem re-encoded as e4m3 (unpacked by the test, decoded by torch) have
    the same exact sums, bit for bit; this ties the packed path (nibble
    order, row pitch, decode) to the pinned 8-bit path.  Mixed pairs too."""
    for (M, N, K, fa, fb, seed) in ((5, 7, 64, 4, 4, 1), (3, 4, 1056, 4, 4, 2), (6, 2, 96, 4, 0, 3),
                                    (2, 5, 128, 1, 4, 4), (1, 1, 32, 4, 4, 5)):
        p = mxinputs.random_problem(M, N, K, seed=900 + seed, fmtA=fa, fmtB=fb, scale_lo=100,
                                    scale_hi=150)
        r = oracle.gemm_full(p.A, p.As, fa, p.B, p.Bs, fb, M, N, K, nthreads=2, lib=lib)
        A8 = _e2m1_as_e4m3(p.A) if fa == 4 else p.A
        B8 = _e2m1_as_e4m3(p.B) if fb == 4 else p.B
        r8 = oracle.gemm_full(A8, p.As, 0 if fa == 4 else fa, B8, p.Bs, 0 if fb == 4 else fb,
                              M, N, K, nthreads=2, lib=lib)
        assert np.array_equal(r["sum"], r8["sum"]), f"e2m1 vs e4m3 re-encoding, case {seed}"
        assert np.array_equal(r["mag"], r8["mag"])


def pin_e2m1_integer_gemm(lib):
    """Integer-valued e2m1 codes (0, +-1, +-2, +-3, +-4, +-6), unit scales:
    C equals the int64 matrix product of the values the test packed."""
    g = np.random.Generator(np.random.PCG64(77))
    M, N, K = 19, 23, 544
    choices = np.array([0, 1, 2, 3, 4, 6, -1, -2, -3, -4, -6])
    ia = g.choice(choices, size=(M, K))
    ib = g.choice(choices, size=(N, K))
    A = mxinputs.quantize(ia.astype(np.float32), 4)
    B = mxinputs.quantize(ib.astype(np.float32), 4)
    assert A.shape == (M, K // 2)
    As = np.full((M, K // 32), 127, np.uint8)
    Bs = np.full((N, K // 32), 127, np.uint8)
    r = oracle.gemm_full(A, As, 4, B, Bs, 4, M, N, K, nthreads=3, lib=lib)
    want = ia.astype(np.int64) @ ib.astype(np.int64).T
    assert np.array_equal(r["sum"], want.astype(np.float64)), "e2m1 integer gemm"


def pin_e2m1_fraction(lib):
    """Tiny random e2m1 problems against exact rational sums (values from
    the golden table, the test's own unpacking)."""
    vals = {c: Fraction(v) for c, v in _golden_e2m1()}
    for i, (M, N, K) in enumerate(((2, 3, 64), (3, 2, 96), (1, 4, 32))):
        p = mxinputs.random_problem(M, N, K, seed=950 + i, fmtA=4, fmtB=4, scale_lo=110,
                                    scale_hi=140)
        r = oracle.gemm_full(p.A, p.As, 4, p.B, p.Bs, 4, M, N, K, nthreads=1, lib=lib)
        ca, cb = mxinputs.unpack_e2m1(p.A), mxinputs.unpack_e2m1(p.B)
        for m in range(M):
            for n in range(N):
                exact = sum(vals[int(ca[m, k])] * Fraction(2) ** (int(p.As[m, k // 32]) - 127)
                            * vals[int(cb[n, k])] * Fraction(2) ** (int(p.Bs[n, k // 32]) - 127)
                            for k in range(K))
                assert Fraction(r["sum"][m, n]) == exact, f"e2m1 case {i} ({m},{n})"


def pin_quant_e2m1(lib):
    """e2m1 quantization: the scale byte satisfies the block exponent's
    defining inequality with MAX = 6 (amax <= 6 * 2^e, not <= 6 * 2^(e-1)),
    and every code is the generator's independent nearest-even e2m1
    rounding of x * 2^-e, packed low nibble first; zero blocks get byte 0
    and keep the sign of -0."""
    g = np.random.Generator(np.random.PCG64(61))
    R, K = 9, 320
    X = (g.standard_normal((R, K)) * np.exp2(g.integers(-30, 30, size=(R, 1)))).astype(np.float32)
    X[0, :32] = 0.0
    X[0, 5] = -0.0
    X[1, :32] = np.float32(6.0) * np.float32(2.0 ** 10)       # amax exactly 6 * 2^10
    X[2, 32:64] = np.linspace(-3, 3, 32, dtype=np.float32)     # ties inside the grid
    codes, scales = oracle.quantize(X, 4, lib=lib)
    assert codes.shape == (R, K // 2)
    unpacked = mxinputs.unpack_e2m1(codes)
    for r in range(R):
        for b in range(K // 32):
            blk = X[r, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            s = int(scales[r, b])
            if amax == 0:
                assert s == 0
            else:
                e = s - 127
                assert amax <= 6.0 * 2.0 ** e and not amax <= 6.0 * 2.0 ** (e - 1), (r, b, s)
            want = mxinputs._quantize_e2m1((blk * 2.0 ** (127 - s)).astype(np.float32))
            assert np.array_equal(unpacked[r, 32 * b:32 * b + 32], want), (r, b)
    assert unpacked[0, 5] == 8 and unpacked[0, 4] == 0
    assert int(scales[1, 0]) == 127 + 10 and (unpacked[1, :32] == 7).all()


# ------------------------------------------------- e2m3 / e3m2 (FP6) --

FP6 = {"e2m3": 2, "e3m2": 3}


def _golden_fp6(name):
    out = []
    with open(os.path.join(GOLDEN, f"ocp_fp6_{name}_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            out.append((int(code, 16), _parse_value(val)))
    return out


def pin_fp6_golden(lib):
    """The 6-bit decoders against the OCP tables (all 64 codes of each);
    codes above 63 do not exist."""
    for name, fmt in FP6.items():
        table = _golden_fp6(name)
        assert len(table) == 64
        for code, val in table:
            got = lib.mxref_decode(fmt, code)
            assert same(got, val, signed_zero=True), f"{name} code {code:#x}: {got!r} != {val!r}"
        assert np.isnan(oracle.decode_table(fmt, lib)[64:]).all()


def _unpack6(packed, K):
    """The test's own reading of a packed 6-bit row: four codes in three
    bytes, code 4q + i at bits 6i .. 6i + 5 of bytes 3q .. 3q + 2 (little
    endian)."""
    p = np.asarray(packed, np.uint32)
    out = np.empty((p.shape[0], K), np.uint8)
    for q in range(K // 4):
        v = p[:, 3 * q] | (p[:, 3 * q + 1] << 8) | (p[:, 3 * q + 2] << 16)
        for i in range(4):
            out[:, 4 * q + i] = (v >> (6 * i)) & 63
    return out


def _fp6_as_e4m3(packed, name, K):
    """Re-encode packed 6-bit codes as e4m3 codes of the same value, using the
    test's own unpacking and torch's e4m3 table."""
    e4 = torch_decode(0)
    vals = np.array([v for _, v in sorted(_golden_fp6(name))])
    codes = _unpack6(packed, K)
    out = np.empty(codes.shape, np.uint8)
    for c in range(64):
        hit = np.flatnonzero((e4 == vals[c]) & (np.signbit(e4) == np.signbit(vals[c])))
        assert hit.size, f"{name} value {vals[c]} is not an e4m3 value"
        out[codes == c] = hit[0]
    assert same(e4[out], vals[codes], signed_zero=True)
    return out


def pin_fp6_embeds_in_e4m3(lib):
    """Every e2m3 and e3m2 value is an e4m3 value, so a 6-bit problem and the
    same problem re-encoded as e4m3 (unpacked by the test, decoded by torch)
    have the same exact sums, bit for bit; this ties the packed path (bit
    order, row pitch, decode) to the pinned 8-bit path.  Mixed pairs too."""
    cases = ((5, 7, 64, 2, 2, 1), (3, 4, 1056, 2, 2, 2), (4, 3, 96, 3, 3, 3), (6, 2, 128, 2, 0, 4),
             (2, 5, 160, 1, 3, 5), (1, 1, 32, 3, 2, 6), (3, 3, 64, 4, 2, 7))
    names = {2: "e2m3", 3: "e3m2"}
    for (M, N, K, fa, fb, seed) in cases:
        p = mxinputs.random_problem(M, N, K, seed=1200 + seed, fmtA=fa, fmtB=fb, scale_lo=100,
                                    scale_hi=150, sigma=2.0)
        r = oracle.gemm_full(p.A, p.As, fa, p.B, p.Bs, fb, M, N, K, nthreads=2, lib=lib)

        def as8(x, f):
            if f in names:
                return _fp6_as_e4m3(x, names[f], K), 0
            if f == 4:
                return _e2m1_as_e4m3(x), 0
            return x, f
        A8, f8a = as8(p.A, fa)
        B8, f8b = as8(p.B, fb)
        r8 = oracle.gemm_full(A8, p.As, f8a, B8, p.Bs, f8b, M, N, K, nthreads=2, lib=lib)
        assert np.array_equal(r["sum"], r8["sum"]), f"6-bit vs e4m3 re-encoding, case {seed}"
        assert np.array_equal(r["mag"], r8["mag"])


def pin_fp6_integer_gemm(lib):
    """Integer-valued e2m3 codes (0, +-1 .. +-7, all exact in e2m3), unit
    scales: C equals the int64 matrix product of the values the test packed."""
    g = np.random.Generator(np.random.PCG64(78))
    M, N, K = 17, 21, 544
    ia = g.integers(-7, 8, size=(M, K))
    ib = g.integers(-7, 8, size=(N, K))
    A = mxinputs.quantize(ia.astype(np.float32), 2)
    B = mxinputs.quantize(ib.astype(np.float32), 2)
    assert A.shape == (M, 3 * K // 4)
    assert np.array_equal(_unpack6(A, K) & 31, np.array([[{0: 0, 1: 8, 2: 16, 3: 20, 4: 24, 5: 26,
                                                           6: 28, 7: 30}[abs(v)] for v in row]
                                                         for row in ia]))
    As = np.full((M, K // 32), 127, np.uint8)
    Bs = np.full((N, K // 32), 127, np.uint8)
    r = oracle.gemm_full(A, As, 2, B, Bs, 2, M, N, K, nthreads=3, lib=lib)
    want = ia.astype(np.int64) @ ib.astype(np.int64).T
    assert np.array_equal(r["sum"], want.astype(np.float64)), "e2m3 integer gemm"


def pin_fp6_fraction(lib):
    """Tiny random 6-bit problems against exact rational sums (values from
    the golden tables, the test's own unpacking)."""
    for i, (M, N, K, name) in enumerate(((2, 3, 64, "e2m3"), (3, 2, 96, "e3m2"), (1, 4, 32, "e2m3"))):
        fmt = FP6[name]
        vals = {c: Fraction(v) for c, v in _golden_fp6(name)}
        p = mxinputs.random_problem(M, N, K, seed=1250 + i, fmtA=fmt, fmtB=fmt, scale_lo=110,
                                    scale_hi=140)
        r = oracle.gemm_full(p.A, p.As, fmt, p.B, p.Bs, fmt, M, N, K, nthreads=1, lib=lib)
        ca, cb = _unpack6(p.A, K), _unpack6(p.B, K)
        for m in range(M):
            for n in range(N):
                exact = sum(vals[int(ca[m, k])] * Fraction(2) ** (int(p.As[m, k // 32]) - 127)
                            * vals[int(cb[n, k])] * Fraction(2) ** (int(p.Bs[n, k // 32]) - 127)
                            for k in range(K))
                assert Fraction(r["sum"][m, n]) == exact, f"{name} case {i} ({m},{n})"


def pin_quant_fp6(lib):
    """6-bit quantization: the scale byte satisfies the block exponent's
    defining inequality with MAX = 7.5 (e2m3) or 28 (e3m2), and every code
    is the generator's independent nearest-even rounding of x * 2^-e,
    packed four per three bytes; zero blocks get byte 0 and keep -0."""
    g = np.random.Generator(np.random.PCG64(62))
    R, K = 7, 256
    for name, fmt in FP6.items():
        mx = 7.5 if fmt == 2 else 28.0
        X = (g.standard_normal((R, K)) * np.exp2(g.integers(-30, 30, size=(R, 1)))).astype(np.float32)
        X[0, :32] = 0.0
        X[0, 5] = -0.0
        X[1, :32] = np.float32(mx) * np.float32(2.0 ** 7)
        codes, scales = oracle.quantize(X, fmt, lib=lib)
        assert codes.shape == (R, 3 * K // 4)
        unpacked = _unpack6(codes, K)
        for r in range(R):
            for b in range(K // 32):
                blk = X[r, 32 * b:32 * b + 32].astype(np.float64)
                amax = np.abs(blk).max()
                s = int(scales[r, b])
                if amax == 0:
                    assert s == 0
                else:
                    e = s - 127
                    assert amax <= mx * 2.0 ** e and not amax <= mx * 2.0 ** (e - 1), (name, r, b, s)
                want = mxinputs._quantize_fp6((blk * 2.0 ** (127 - s)).astype(np.float32), fmt)
                assert np.array_equal(unpacked[r, 32 * b:32 * b + 32], want), (name, r, b)
        assert unpacked[0, 5] == 32 and unpacked[0, 4] == 0
        assert int(scales[1, 0]) == 127 + 7 and (unpacked[1, :32] == 31).all()


ALL_PINS = [pin_tables_match_torch, pin_spot_values, pin_special_counts, pin_bf16_rne,
            pin_bruteforce_fraction, pin_pairwise_products, pin_closed_form,
            pin_integer_gemm, pin_scale_doubling, pin_permutation, pin_numpy_matmul,
            pin_nan_propagation, pin_thread_independence, pin_scale_tile_extent,
            pin_quant_rne_vs_torch, pin_quant_block_exponent, pin_quant_scale_invariance,
            pin_quant_matches_generator, pin_quant_bf16_input, pin_quant_ragged_and_nonfinite,
            pin_e2m1_golden, pin_e2m1_embeds_in_e4m3, pin_e2m1_integer_gemm, pin_e2m1_fraction,
            pin_fp6_golden, pin_fp6_embeds_in_e4m3, pin_fp6_integer_gemm, pin_fp6_fraction,
            pin_quant_fp6,
            pin_quant_e2m1]
