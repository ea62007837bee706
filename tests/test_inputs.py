"""The seeded input generators (shared by the oracle and the HIP path)."""
import numpy as np
import torch

import mxinputs as mi
import oracle


def test_quantizer_saturates_and_rounds_to_even():
    e4 = oracle.decode_table(0)
    e5 = oracle.decode_table(1)
    big = np.array([449, 464, 480, 1e9, -1e9, np.inf], np.float32)
    assert list(mi.quantize(big, 0)) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E]
    assert list(mi.quantize(np.array([60000, 1e30], np.float32), 1)) == [0x7B, 0x7B]
    # midpoints between neighbouring positive e4m3 values go to the even code
    pos = np.sort(e4[1:0x7F])
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    codes = mi.quantize(mids, 0)
    assert np.all(codes % 2 == 0)
    # every value lands on the nearest representable value
    g = np.random.Generator(np.random.PCG64(1))
    x = g.standard_normal(20000).astype(np.float32) * 40
    for fmt, tab in ((0, e4), (1, e5)):
        c = mi.quantize(x, fmt)
        v = tab[c]
        fin = tab[np.isfinite(tab)]
        nearest = np.min(np.abs(fin[None, :] - np.clip(x, -mi.FMT_MAX[fmt], mi.FMT_MAX[fmt])[:, None]
                                .astype(np.float64)), axis=1)
        assert np.all(np.abs(v - np.clip(x, -mi.FMT_MAX[fmt], mi.FMT_MAX[fmt])) == nearest)


def test_generators_are_seeded():
    a = mi.random_problem(17, 9, 96, seed=3)
    b = mi.random_problem(17, 9, 96, seed=3)
    c = mi.random_problem(17, 9, 96, seed=4)
    assert np.array_equal(a.A, b.A) and np.array_equal(a.Bs, b.Bs)
    assert not np.array_equal(a.A, c.A)
    assert a.As.min() >= 120 and a.As.max() <= 134


def test_block_exponent_is_minimal():
    g = np.random.Generator(np.random.PCG64(2))
    amax = np.abs(g.standard_normal(5000)) * 0.05
    amax = np.concatenate([amax, [448.0, 896.0, 448.0 * 2**-20, 448.0 * 2**-20 * 1.0000001, 0.0]])
    e = mi.block_exponent(amax)
    nz = amax > 0
    assert np.all(amax[nz] <= 448.0 * np.ldexp(1.0, e[nz]))
    assert np.all(amax[nz] > 448.0 * np.ldexp(1.0, e[nz] - 1))
    assert e[-1] == -127


def test_mx_block_quantize_recipe():
    g = np.random.Generator(np.random.PCG64(3))
    x = (g.standard_normal((16, 256)) * 0.02).astype(np.float32)
    codes, scales = mi.mx_block_quantize(x)
    e4 = oracle.decode_table(0)
    dec = e4[codes].reshape(16, 8, 32) * np.ldexp(1.0, scales.astype(np.int64) - 127)[:, :, None]
    blocks = x.reshape(16, 8, 32).astype(np.float64)
    # scale bytes near 127 + ceil(log2(0.02*~2.5/448)) and no saturation
    assert scales.min() >= 110 and scales.max() <= 118
    assert np.all(np.abs(codes.reshape(16, 8, 32).astype(np.int64) & 0x7F) <= 0x7E)
    # each block's largest magnitude uses the top binade of e4m3 (>= 256)
    top = np.abs(e4[codes]).reshape(16, 8, 32).max(axis=2)
    assert np.all(top >= 224.0)
    rel = np.abs(dec - blocks) / np.maximum(np.abs(blocks), 1e-30)
    big = np.abs(blocks) > 2.0**-6 * np.ldexp(1.0, scales.astype(np.int64) - 127)[:, :, None]
    assert np.all(rel[big] <= 2.0**-4 + 1e-12)


def test_sample_points_cover_edges():
    r, c = mi.sample_points(1000, 700, 500, seed=1, edge=64)
    pts = set(zip(r.tolist(), c.tolist()))
    assert (0, 0) in pts and (999, 699) in pts and (999, 0) in pts and (0, 699) in pts
    assert all((999, j) in pts for j in range(700))
    assert all((i, 699) in pts for i in range(1000))
    assert len(pts) == len(r)


def test_e2m1_quantiser_is_nearest_even():
    """The generator's e2m1 rounding against a brute-force search over the
    eight magnitudes (ties to the even code), on a dense sweep, every
    midpoint of both signs, zeros, tiny and saturating values; and packing
    round-trips."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    x = np.concatenate([np.linspace(-7, 7, 20001, dtype=np.float32), mids, -mids,
                        np.float32([0.0, -0.0, 1e-30, -1e-30, 6.0, -6.0, 100, -100])])
    got = mi._quantize_e2m1(x)
    d = np.abs(np.minimum(np.abs(x.astype(np.float64)), 6.0)[:, None] - grid[None, :])
    cand = d == d.min(axis=1, keepdims=True)
    even = cand & (np.arange(8) % 2 == 0)
    idx = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    want = (idx | (np.signbit(x) << 3)).astype(np.uint8)
    assert np.array_equal(got, want)
    codes = np.random.Generator(np.random.PCG64(5)).integers(0, 16, size=(3, 64), dtype=np.uint8)
    assert np.array_equal(mi.unpack_e2m1(mi.pack_e2m1(codes)), codes)


def test_pack_bits_round_trip_and_layout():
    g = np.random.Generator(np.random.PCG64(5))
    for bits in (4, 6, 8):
        c = g.integers(0, 1 << bits, size=(3, 64), dtype=np.uint8)
        p = mi.pack_bits(c, bits)
        assert p.shape == (3, 64 * bits // 8)
        assert np.array_equal(mi.unpack_bits(p, bits, 64), c)
    # e2m1: the even k in the low nibble; 6-bit: code 4q+i at bits 6i of bytes 3q..3q+2
    assert np.array_equal(mi.pack_bits(np.array([[1, 2]], np.uint8), 4), [[0x21]])
    assert np.array_equal(mi.pack_bits(np.array([[1, 2, 3, 4]], np.uint8), 6),
                          [[1 | (2 << 6) & 0xff, (2 >> 2) | (3 << 4) & 0xff, (3 >> 4) | (4 << 2)]])


def test_fp6_quantize_grid_and_ties():
    for fmt, mx in ((mi.FMT_E2M3, 7.5), (mi.FMT_E3M2, 28.0)):
        grid = mi._fp6_grid(fmt)
        assert grid[0] == 0 and grid[-1] == mx and np.all(np.diff(grid) > 0)
        mids = (grid[:-1] + grid[1:]) / 2
        c = mi._quantize_fp6(mids.astype(np.float32), fmt)
        assert np.all(c % 2 == 0)  # ties go to the even code
        assert mi._quantize_fp6(np.array([1e9, -1e9], np.float32), fmt).tolist() == [31, 63]


def test_preshuffle_layout_formula():
    """The preshuffled layout against its definition, byte by byte: scale
    (r, kb) at (r // 32) * 32 * KB + (kb // 4) * 128 + (r % 32) * 4 + kb % 4,
    padding rows zero; a 32-row group keeps its byte range."""
    g = np.random.Generator(np.random.PCG64(77))
    for R, KB in ((1, 4), (31, 8), (32, 4), (33, 12), (70, 16), (64, 256)):
        S = g.integers(1, 256, size=(R, KB), dtype=np.uint8)
        P = mi.preshuffle_scales(S).reshape(-1)
        Rp = (R + 31) // 32 * 32
        assert P.size == Rp * KB
        seen = np.zeros(P.size, bool)
        for r in range(R):
            for kb in range(KB):
                o = (r // 32) * 32 * KB + (kb // 4) * 128 + (r % 32) * 4 + kb % 4
                assert P[o] == S[r, kb]
                seen[o] = True
                assert r * KB // (32 * KB) == o // (32 * KB)  # same group, same range
        assert np.all(P[~seen] == 0) and np.sum(~seen) == (Rp - R) * KB
