"""GPU parity of the MX block quantization (mxgemm_quantize, through the C
ABI) against the CPU oracle: codes and scale bytes must agree bit for bit
(the scale is an integer decision and each code a round-to-nearest-even
decision, both taken in the same fp32 arithmetic on both sides).

Cases: random fp32 and bf16 rows spanning many binades, round-to-nearest
ties and their fp32 neighbours, subnormal and near-overflow magnitudes,
zeros of both signs, ragged stream tails, every output format (e4m3,
e5m2, e2m1, e2m3, e3m2), the full skinny workload's weight (its quantized
B must equal the workload's stored operand), and GPU-quantized operands
fed to the multiply (e2m1, and the 6-bit formats alone and beside e4m3).
"""
import numpy as np
import pytest
import torch

import level_dsl_amd as L
import mxinputs as mi
import oracle
from gpu_helpers import log

pytestmark = pytest.mark.gpu

QMAX = {0: 448.0, 1: 57344.0, 2: 7.5, 3: 28.0, 4: 6.0}


@pytest.fixture(scope="module")
def gemm():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    g = L.Gemm()
    yield g
    g.close()


def gpu_quantize(gemm, X: np.ndarray, fmt: int):
    """X: float32 array, or uint16 bf16 bit patterns."""
    if X.dtype == np.uint16:
        t = torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    else:
        t = torch.from_numpy(X).to("cuda:0")
    R, K = X.shape
    kc = L.row_bytes(fmt, K)  # e2m1: two codes per byte; e2m3 / e3m2: four per three bytes
    # guard bytes around both outputs: nothing may be written outside them
    cbuf = torch.full((R * kc + 512,), 0xA5, dtype=torch.uint8, device="cuda:0")
    sbuf = torch.full((R * K // 32 + 512,), 0x5A, dtype=torch.uint8, device="cuda:0")
    codes = cbuf[256:256 + R * kc].view(R, kc)
    scales = sbuf[256:256 + R * K // 32].view(R, K // 32)
    gemm.quantize(t, fmt, codes, scales)
    torch.cuda.synchronize()
    cb, sb = cbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert np.all(cb[:256] == 0xA5) and np.all(cb[-256:] == 0xA5), "code stored outside its range"
    assert np.all(sb[:256] == 0x5A) and np.all(sb[-256:] == 0x5A), "scale stored outside its range"
    return codes.cpu().numpy(), scales.cpu().numpy()


def check(gemm, X, fmt, where):
    want_c, want_s = oracle.quantize(X, fmt)
    got_c, got_s = gpu_quantize(gemm, X, fmt)
    bad_s = np.flatnonzero(got_s != want_s)
    assert bad_s.size == 0, f"{where}: {bad_s.size} scale bytes differ, e.g. {bad_s[:4]}"
    bad = np.flatnonzero(got_c != want_c)
    assert bad.size == 0, (f"{where}: {bad.size} codes differ, e.g. flat {bad[:4]}: got "
                           f"{got_c.ravel()[bad[:4]]} want {want_c.ravel()[bad[:4]]}")


def wide_rows(R, K, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal((R, K)) * np.exp2(g.integers(-30, 31, (R, 1)))
    return x.astype(np.float32)


@pytest.mark.parametrize("fmt", [0, 1, 4, 2, 3])
@pytest.mark.parametrize("R,K", [(37, 1120), (1, 32), (3, 96), (129, 4096)])
def test_random_fp32(gemm, fmt, R, K):
    log(f"quantize fp32 {R}x{K} fmt={fmt}")
    check(gemm, wide_rows(R, K, seed=R * 31 + K + fmt), fmt, f"fp32 {R}x{K}")


@pytest.mark.parametrize("fmt", [0, 1, 4, 2, 3])
@pytest.mark.parametrize("R,K", [(37, 1120), (5, 64)])
def test_random_bf16(gemm, fmt, R, K):
    x = wide_rows(R, K, seed=R * 17 + K + fmt)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    log(f"quantize bf16 {R}x{K} fmt={fmt}")
    check(gemm, bits, fmt, f"bf16 {R}x{K}")


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_ties_and_neighbours(gemm, fmt):
    """Blocks whose largest magnitude is exactly MAX (scale 2^0) filled with
    midpoints between neighbouring codes, their fp32 neighbours and the codes'
    own values."""
    tab = oracle.decode_table(fmt)[: 1 << (mi.CODE_BITS[fmt] - 1)]  # the non-negative codes
    fin = np.sort(tab[np.isfinite(tab)])
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)),
                           np.nextafter(mids, np.float32(0)), fin.astype(np.float32)])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    nb = (vals.size + 30) // 31
    vals = np.concatenate([vals, np.zeros(nb * 31 - vals.size, np.float32)])
    X = np.empty((nb, 32), np.float32)
    X[:, 0] = QMAX[fmt]
    X[:, 1:] = vals.reshape(nb, 31)
    # also scaled copies: the same ties at other block scales
    X = np.concatenate([X, X * np.float32(2.0 ** -40), X * np.float32(2.0 ** 60)]).astype(np.float32)
    check(gemm, X, fmt, "ties")


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_extreme_magnitudes_and_zeros(gemm, fmt):
    """Block maxima across the whole fp32 range (subnormals to 3.4e38), all-zero
    and negative-zero blocks."""
    g = np.random.Generator(np.random.PCG64(7 + fmt))
    rows = 2048
    amax = np.exp2(g.uniform(-149.0, 127.99, rows)).astype(np.float32)
    amax[:6] = np.float32([2.0 ** -149, 2.0 ** -126, 3.4e38, QMAX[fmt], 1.0, 0.0])
    X = (g.uniform(-1, 1, (rows, 64)) * amax[:, None].astype(np.float64)).astype(np.float32)
    X[np.arange(rows), g.integers(0, 64, rows)] = amax
    X[5, :] = 0.0
    X[6, :32] = -0.0
    X[7, 32:] = -0.0
    check(gemm, X, fmt, "extremes")


def test_skinny_weight_matches_workload(gemm):
    """Quantizing the skinny workload's fp32 draws on the GPU gives exactly
    that workload's stored B and B scales (sampled rows are also checked
    against the oracle)."""
    raw = mi.skinny_b_raw()
    log("skinny raw B generated")
    p = mi.workload(3)
    log("skinny workload generated")
    got_c, got_s = gpu_quantize(gemm, raw, 0)
    assert np.array_equal(got_s, p.Bs), "scale bytes differ from the workload's"
    assert np.array_equal(got_c, p.B), "codes differ from the workload's"
    rows = np.random.Generator(np.random.PCG64(3)).choice(raw.shape[0], 64, replace=False)
    want_c, want_s = oracle.quantize(np.ascontiguousarray(raw[rows]), 0)
    assert np.array_equal(got_c[rows], want_c) and np.array_equal(got_s[rows], want_s)



@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_e2m1_ties_extremes_and_zeros(gemm, xdt):
    """e2m1: every midpoint of the grid (a tie) and its fp32 neighbours, at
    three block scales; the largest magnitude sitting exactly on 6 * 2^e or
    one ulp above; blocks of zeros of both signs, tiny and huge blocks."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    mids = (grid[:-1] + grid[1:]) / 2
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(9))])
    rows = []
    for e in (-20, 0, 17):
        for sign in (1, -1):
            blk = np.zeros(32, np.float32)
            blk[:vals.size] = vals[:32] if vals.size >= 32 else vals
            blk[-1] = 6.0                              # the block maximum is exactly 6
            rows.append(sign * blk * np.float32(2.0 ** e))
    top = np.full(32, 0.3, np.float32)
    top[0] = np.nextafter(np.float32(6.0), np.float32(9))   # one ulp above 6: next scale up
    rows.append(top)
    rows.append(np.zeros(32, np.float32))
    rows.append(-np.zeros(32, np.float32))
    rows.append(np.full(32, 1e-40, np.float32))             # subnormal block
    rows.append(np.full(32, 3.0e38, np.float32))            # near the fp32 maximum
    X = np.stack(rows).reshape(len(rows), 32)
    X = np.concatenate([X, X[::-1]], axis=1)                # K = 64, two blocks per row
    if xdt == "bf16":
        X = torch.from_numpy(X).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    log(f"e2m1 quantize ties/extremes {xdt}")
    check(gemm, X, 4, f"e2m1 ties {xdt}")


def test_e2m1_quantize_feeds_the_multiply(gemm):
    """Quantize fp32 A and B to e2m1 on the GPU and multiply them: the
    product equals the oracle's product of the oracle's quantization."""
    g = np.random.Generator(np.random.PCG64(71))
    M, N, K = 96, 200, 1024
    Xa = g.standard_normal((M, K)).astype(np.float32)
    Xb = (0.02 * g.standard_normal((N, K))).astype(np.float32)
    qa, sa = gpu_quantize(gemm, Xa, 4)
    qb, sb = gpu_quantize(gemm, Xb, 4)
    ra, rsa = oracle.quantize(Xa, 4)
    rb, rsb = oracle.quantize(Xb, 4)
    assert np.array_equal(qa, ra) and np.array_equal(sa, rsa)
    assert np.array_equal(qb, rb) and np.array_equal(sb, rsb)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    C = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    gemm(t(qa), t(sa), 4, t(qb), t(sb), 4, C)
    torch.cuda.synchronize()
    ref = oracle.gemm_full(ra, rsa, 4, rb, rsb, 4, M, N, K)
    err = np.abs(C.cpu().numpy().astype(np.float64) - ref["ref32"])
    assert np.all(err <= 1e-5 * ref["mag"])


@pytest.mark.parametrize("fa,fb", [(2, 2), (3, 3), (3, 0), (0, 2)])
def test_fp6_quantize_feeds_the_multiply(gemm, fa, fb):
    """Quantize fp32 A and B on the GPU (6-bit and, where named, e4m3) and
    multiply them: e2m3 x e2m3 runs on the scaled MFMA, the other pairs
    widened; the product equals the oracle's product of the oracle's
    quantization, and the GPU codes equal the oracle's bit for bit."""
    g = np.random.Generator(np.random.PCG64(73 + fa + 8 * fb))
    M, N, K = 96, 200, 1024
    Xa = g.standard_normal((M, K)).astype(np.float32)
    Xb = (0.02 * g.standard_normal((N, K))).astype(np.float32)
    qa, sa = gpu_quantize(gemm, Xa, fa)
    qb, sb = gpu_quantize(gemm, Xb, fb)
    ra, rsa = oracle.quantize(Xa, fa)
    rb, rsb = oracle.quantize(Xb, fb)
    assert np.array_equal(qa, ra) and np.array_equal(sa, rsa)
    assert np.array_equal(qb, rb) and np.array_equal(sb, rsb)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    C = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    log(f"fp6 quantize -> multiply fmtA={fa} fmtB={fb}")
    gemm(t(qa), t(sa), fa, t(qb), t(sb), fb, C)
    torch.cuda.synchronize()
    ref = oracle.gemm_full(ra, rsa, fa, rb, rsb, fb, M, N, K)
    err = np.abs(C.cpu().numpy().astype(np.float64) - ref["ref32"])
    assert np.all(err <= 1e-5 * ref["mag"])
