"""Seeded synthetic inputs for the MX-FP8 matrix multiply.

This module is shared by the tests, the smoke check and the benchmark, and
feeds the same bytes to the CPU oracle and to the HIP library.  It holds none
of the multiply's arithmetic: it only draws numbers and turns them into 8-bit
codes and scale bytes, using torch's own fp32 -> float8 casts (round to
nearest even) after clamping, so that saturation to the format's largest
finite value replaces overflow.

Workloads (all synthetic; no dataset is involved):

  id  shape (M, N, K)     formats A/B   values                         scales          out   use_acc
  0   256, 256, 256       e4m3/e4m3     N(0,1) -> RNE, saturating      U{123..131}     f32   no
  1   4096^3              e4m3/e4m3     N(0,1) -> RNE, saturating      U{120..134}     f32   no
  2   8192^3              e4m3/e4m3     N(0,0.5^2) -> RNE, saturating  U{122..132}     bf16  no
  3   64, 28672, 8192     e4m3/e4m3     A N(0,1); B N(0,0.02^2) with   A U{125..129};  f32   no
                                        a per-32-block MX scale        B per block
  4   16384^3             e5m2/e4m3     N(0,1) -> RNE, saturating      U{118..136}     f32   yes, C_in N(0,1)

Seeds: numpy PCG64(SeedSequence([0x4D58, workload_id, tensor_id])) with
tensor_id 0 = A, 1 = B, 2 = A_scale, 3 = B_scale, 4 = C_in.

Layouts: A (M, K) row-major codes; B (N, K) codes with K contiguous
(B_mem[n*K + k] = B[k, n]); A_scale (M, K/32) and B_scale (N, K/32)
row-major bytes; C (M, N) row-major.  An e2m1 operand (format 4) holds two
codes per byte along K, the even k in the low nibble: (rows, K/2) bytes.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

SEED_ROOT = 0x4D58
FMT_E4M3 = 0
FMT_E5M2 = 1
FMT_E2M3 = 2
FMT_E3M2 = 3
FMT_E2M1 = 4
OUT_F32 = 0
OUT_BF16 = 1

# largest finite value of each format (OCP e4m3fn / e5m2)
FMT_MAX = {FMT_E4M3: 448.0, FMT_E5M2: 57344.0, FMT_E2M3: 7.5, FMT_E3M2: 28.0, FMT_E2M1: 6.0}
CODE_BITS = {FMT_E4M3: 8, FMT_E5M2: 8, FMT_E2M3: 6, FMT_E3M2: 6, FMT_E2M1: 4}


def _fp6_grid(fmt: int) -> np.ndarray:
    """The 32 non-negative magnitudes of a 6-bit format in code order (the
    code's low 5 bits), from the OCP FP6 bit fields: e2m3 is exponent bias 1
    with 3 mantissa bits, e3m2 bias 3 with 2; exponent field 0 is
    subnormal."""
    mb, bias = (3, 1) if fmt == FMT_E2M3 else (2, 3)
    out = []
    for c in range(32):
        e, m = c >> mb, c & ((1 << mb) - 1)
        if e == 0:
            out.append(m / (1 << mb) * 2.0 ** (1 - bias))
        else:
            out.append((1 + m / (1 << mb)) * 2.0 ** (e - bias))
    return np.array(out)


def _quantize_fp6(x: np.ndarray, fmt: int) -> np.ndarray:
    """fp32 values -> 6-bit codes 0..63 (unpacked): round to the nearest
    grid magnitude, ties to the even code, saturating at the largest; the
    sign (bit 5) is kept, so -0 and tiny negatives give code 32."""
    grid = _fp6_grid(fmt)
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    lo = np.clip(np.searchsorted(grid, a, side="right") - 1, 0, 31)
    hi = np.minimum(lo + 1, 31)
    d_lo, d_hi = a - grid[lo], grid[hi] - a
    up = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    idx = np.where(up, hi, lo).astype(np.uint8)
    return idx | (np.signbit(x).astype(np.uint8) << 5)


def pack_bits(codes: np.ndarray, bits: int) -> np.ndarray:
    """(rows, K) codes of `bits` bits -> (rows, ceil(bits*K/8)) bytes: code k
    at bits bits*k .. bits*k+bits-1 of the row read as one little-endian bit
    string (e2m1: the even k in the low nibble; 6-bit: four codes in three
    bytes)."""
    c = np.asarray(codes, dtype=np.uint64)
    rows, K = c.shape
    nbytes = (K * bits + 7) // 8
    out = np.zeros((rows, nbytes), np.uint8)
    for k in range(K):
        bit = k * bits
        b, sh = bit // 8, bit % 8
        v = c[:, k] << np.uint64(sh)
        out[:, b] |= (v & np.uint64(0xff)).astype(np.uint8)
        if sh + bits > 8:
            out[:, b + 1] |= (v >> np.uint64(8)).astype(np.uint8)
    return out


def unpack_bits(packed: np.ndarray, bits: int, K: int) -> np.ndarray:
    """Inverse of pack_bits: (rows, ceil(bits*K/8)) bytes -> (rows, K) codes."""
    p = np.asarray(packed, dtype=np.uint64)
    out = np.empty((p.shape[0], K), np.uint8)
    for k in range(K):
        bit = k * bits
        b, sh = bit // 8, bit % 8
        v = p[:, b] >> np.uint64(sh)
        if sh + bits > 8:
            v |= p[:, b + 1] << np.uint64(8 - sh)
        out[:, k] = (v & np.uint64((1 << bits) - 1)).astype(np.uint8)
    return out
_TORCH_FP8 = {FMT_E4M3: torch.float8_e4m3fn, FMT_E5M2: torch.float8_e5m2}

T_A, T_B, T_AS, T_BS, T_CIN = 0, 1, 2, 3, 4


def preshuffle_scales(S: np.ndarray) -> np.ndarray:
    """Row-major scale bytes (R, K/32), K/32 % 4 == 0, in the library's
    preshuffled layout, as a (ceil(R/32)*32, K/32) array: rows in groups of
    32, K blocks in groups of 4, each pair of groups one 128-byte unit of
    the 32 rows' 4-byte words in row order; padding rows are zero.  An index
    permutation only (the inputs' byte placement, no arithmetic of the
    multiply)."""
    R, KB = S.shape
    assert KB % 4 == 0, "the preshuffled layout needs K % 128 == 0"
    Rp = (R + 31) // 32 * 32
    P = np.zeros((Rp, KB), np.uint8)
    P[:R] = S
    return np.ascontiguousarray(P.reshape(Rp // 32, 32, KB // 4, 4).transpose(0, 2, 1, 3).reshape(Rp, KB))


def rng(workload: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([SEED_ROOT, int(workload), int(tensor_id)])))


def _quantize_e2m1(x: np.ndarray) -> np.ndarray:
    """fp32 values -> e2m1 codes 0..15 (unpacked): clamp to +-6, round to the
    nearest grid value, ties to the even code (mantissa bit 0); the sign is
    kept (-0 and tiny negatives give code 8).  The magnitude code is the
    number of midpoints below |x|: strictly below where the lower neighbour
    is the even code, at or below where the upper one is."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x)
    idx = ((a > 0.25).astype(np.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
           + (a > 2.5) + (a >= 3.5) + (a > 5.0)).astype(np.uint8)
    return idx | (np.signbit(x).astype(np.uint8) << 3)


def pack_e2m1(codes: np.ndarray) -> np.ndarray:
    """(rows, K) codes 0..15 -> (rows, K/2) bytes, the even k in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def quantize(x: np.ndarray, fmt: int) -> np.ndarray:
    """fp32 values -> uint8 codes: clamp to +-max, then round to nearest even.
    e2m1 and 6-bit codes come back packed along the last axis (pack_bits)."""
    if fmt == FMT_E2M1:
        return pack_e2m1(_quantize_e2m1(x))
    if fmt in (FMT_E2M3, FMT_E3M2):
        x = np.asarray(x, dtype=np.float32)
        return pack_bits(_quantize_fp6(x.reshape(-1, x.shape[-1]), fmt), 6).reshape(
            x.shape[:-1] + ((x.shape[-1] * 6 + 7) // 8,))
    lim = np.float32(FMT_MAX[fmt])
    x = np.clip(np.asarray(x, dtype=np.float32), -lim, lim)
    t = torch.from_numpy(np.ascontiguousarray(x)).to(_TORCH_FP8[fmt])
    return t.view(torch.uint8).numpy()


def normal_codes(g: np.random.Generator, shape, sigma: float, fmt: int) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return quantize(x, fmt)


def uniform_scales(g: np.random.Generator, shape, lo: int, hi: int) -> np.ndarray:
    """Scale bytes drawn uniformly from the integers lo..hi inclusive."""
    return g.integers(lo, hi + 1, size=shape, dtype=np.uint8)


def block_exponent(amax: np.ndarray, fmt: int = FMT_E4M3) -> np.ndarray:
    """Smallest integer e with amax <= max(fmt) * 2^e (the per-block recipe
    ceil(log2(amax / max))), with exact corrections; all-zero blocks get the
    smallest exponent, -127."""
    amax = np.asarray(amax, dtype=np.float64)
    lim = FMT_MAX[fmt]
    with np.errstate(divide="ignore"):
        e = np.ceil(np.log2(amax / lim))
    e = np.where(np.isfinite(e), e, -127.0).astype(np.int64)
    # exact correction of log2 rounding: amax <= lim*2^e and not <= lim*2^(e-1)
    too_small = amax > lim * np.ldexp(1.0, e)
    e = e + too_small
    too_big = (amax > 0) & (amax <= lim * np.ldexp(1.0, e - 1))
    e = e - too_big
    return np.clip(e, -127, 127)


def mx_block_quantize(x: np.ndarray, fmt: int = FMT_E4M3):
    """Per-32-element block of each row: scale byte e+127 with e from
    block_exponent, codes = RNE(x * 2^-e).  x is (rows, K) fp32, K % 32 == 0."""
    x = np.asarray(x, dtype=np.float32)
    rows, k = x.shape
    assert k % 32 == 0
    blocks = x.reshape(rows, k // 32, 32)
    e = block_exponent(np.abs(blocks).max(axis=2), fmt)          # (rows, K/32)
    scaled = blocks * np.ldexp(np.float32(1.0), -e)[:, :, None].astype(np.float32)
    codes = quantize(scaled.reshape(rows, k), fmt)
    return codes, (e + 127).astype(np.uint8)


@dataclasses.dataclass
class Problem:
    M: int
    N: int
    K: int
    fmtA: int
    fmtB: int
    A: np.ndarray        # (M, K) uint8; e2m1: (M, K/2), two codes per byte
    As: np.ndarray       # (M, ceil(K/32)) uint8
    B: np.ndarray        # (N, K) uint8, K contiguous; e2m1: (N, K/2)
    Bs: np.ndarray       # (N, ceil(K/32)) uint8
    out_dtype: int
    use_acc: bool
    Cin: Optional[np.ndarray] = None   # (M, N) float32, or uint16 bf16 bits
    name: str = ""


WORKLOADS = {
    0: dict(name="mxgemm_256cube_e4m3_f32", M=256, N=256, K=256),
    1: dict(name="mxgemm_4096cube_e4m3_f32", M=4096, N=4096, K=4096),
    2: dict(name="mxgemm_8192cube_e4m3_bf16", M=8192, N=8192, K=8192),
    3: dict(name="mxgemm_skinny_m64_n28672_k8192_e4m3_f32", M=64, N=28672, K=8192),
    4: dict(name="mxgemm_16384cube_e5m2xe4m3_acc_f32", M=16384, N=16384, K=16384),
}


def skinny_b_raw() -> np.ndarray:
    """The fp32 draws behind the skinny workload's B: (N, K) = (28672, 8192)
    samples of N(0, 0.02^2), before MX block quantization."""
    w = WORKLOADS[3]
    braw = rng(3, T_B).standard_normal(size=(w["N"], w["K"]), dtype=np.float32)
    braw *= np.float32(0.02)
    return braw


def workload(wid: int) -> Problem:
    """Build one of the five named workloads (see the module docstring)."""
    w = WORKLOADS[wid]
    M, N, K = w["M"], w["N"], w["K"]
    kb = K // 32
    if wid in (0, 1, 2):
        sigma = 0.5 if wid == 2 else 1.0
        lo, hi = {0: (123, 131), 1: (120, 134), 2: (122, 132)}[wid]
        A = normal_codes(rng(wid, T_A), (M, K), sigma, FMT_E4M3)
        B = normal_codes(rng(wid, T_B), (N, K), sigma, FMT_E4M3)
        As = uniform_scales(rng(wid, T_AS), (M, kb), lo, hi)
        Bs = uniform_scales(rng(wid, T_BS), (N, kb), lo, hi)
        out = OUT_BF16 if wid == 2 else OUT_F32
        return Problem(M, N, K, FMT_E4M3, FMT_E4M3, A, As, B, Bs, out, False, None, w["name"])
    if wid == 3:
        A = normal_codes(rng(wid, T_A), (M, K), 1.0, FMT_E4M3)
        As = uniform_scales(rng(wid, T_AS), (M, kb), 125, 129)
        braw = skinny_b_raw()
        B, Bs = mx_block_quantize(braw, FMT_E4M3)
        del braw
        return Problem(M, N, K, FMT_E4M3, FMT_E4M3, A, As, B, Bs, OUT_F32, False, None, w["name"])
    if wid == 4:
        A = normal_codes(rng(wid, T_A), (M, K), 1.0, FMT_E5M2)
        B = normal_codes(rng(wid, T_B), (N, K), 1.0, FMT_E4M3)
        As = uniform_scales(rng(wid, T_AS), (M, kb), 118, 136)
        Bs = uniform_scales(rng(wid, T_BS), (N, kb), 118, 136)
        Cin = rng(wid, T_CIN).standard_normal(size=(M, N), dtype=np.float32)
        return Problem(M, N, K, FMT_E5M2, FMT_E4M3, A, As, B, Bs, OUT_F32, True, Cin, w["name"])
    raise KeyError(wid)


def random_problem(M, N, K, *, seed, fmtA=FMT_E4M3, fmtB=FMT_E4M3, sigma=1.0,
                   scale_lo=120, scale_hi=134, out_dtype=OUT_F32, use_acc=False) -> Problem:
    """A seeded problem of any shape (K need not be a multiple of 32 for the
    oracle; the last scale column then covers a partial block)."""
    kb = (K + 31) // 32
    wid = 1000 + int(seed)
    A = normal_codes(rng(wid, T_A), (M, K), sigma, fmtA)
    B = normal_codes(rng(wid, T_B), (N, K), sigma, fmtB)
    As = uniform_scales(rng(wid, T_AS), (M, kb), scale_lo, scale_hi)
    Bs = uniform_scales(rng(wid, T_BS), (N, kb), scale_lo, scale_hi)
    Cin = None
    if use_acc:
        c = rng(wid, T_CIN).standard_normal(size=(M, N), dtype=np.float32)
        if out_dtype == OUT_BF16:
            Cin = torch.from_numpy(c).to(torch.bfloat16).view(torch.uint16).numpy()
        else:
            Cin = c
    return Problem(M, N, K, fmtA, fmtB, A, As, B, Bs, out_dtype, use_acc, Cin,
                   f"random_{M}x{N}x{K}_s{seed}")


def sample_points(M: int, N: int, count: int, seed: int, edge: int = 256):
    """Seeded random output coordinates plus the 'edge' set: the four corner
    edge x edge blocks (clipped to the matrix) and all of row M-1 and column
    N-1.  Returns (rows, cols) int64 arrays without duplicates."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, 7777, seed])))
    r = g.integers(0, M, size=count, dtype=np.int64)
    c = g.integers(0, N, size=count, dtype=np.int64)
    parts_r, parts_c = [r], [c]
    e_m, e_n = min(edge, M), min(edge, N)
    for r0 in (0, M - e_m):
        for c0 in (0, N - e_n):
            rr, cc = np.meshgrid(np.arange(r0, r0 + e_m), np.arange(c0, c0 + e_n), indexing="ij")
            parts_r.append(rr.ravel()); parts_c.append(cc.ravel())
    parts_r.append(np.full(N, M - 1)); parts_c.append(np.arange(N))
    parts_r.append(np.arange(M)); parts_c.append(np.full(M, N - 1))
    rr = np.concatenate(parts_r).astype(np.int64)
    cc = np.concatenate(parts_c).astype(np.int64)
    lin = np.unique(rr * N + cc)
    return lin // N, lin % N


def algorithmic_flops(M, N, K, use_acc=False) -> int:
    return 2 * M * N * K


def algorithmic_bytes(M, N, K, out_dtype=OUT_F32, use_acc=False) -> int:
    """A, A_scale, B, B_scale read once; C written once (and read once if use_acc)."""
    kb = math.ceil(K / 32)
    cbytes = M * N * (4 if out_dtype == OUT_F32 else 2)
    return M * K + M * kb + N * K + N * kb + cbytes * (2 if use_acc else 1)
