"""Helpers for the GPU parity tests: upload a problem, run the HIP library
through its C ABI, and compare with the oracle under the agreement rule

    fp32 out:  |C_gpu - C_ref| <= 1e-5 * sum_k |a_k b_k|
    bf16 out:  |C_gpu - C_ref| <= 1e-5 * sum_k |a_k b_k| + one bf16 ulp of C_ref

(NaN must meet NaN, infinities must match exactly, -0 equals +0), where
C_ref is the oracle's exact sum rounded to fp32 (then to bf16) and the
magnitude includes |C_in| when use_acc is set.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import mxinputs as mi
import oracle

TOL_REL = 1e-5


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(p: mi.Problem):
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return t(p.A), t(p.As), t(p.B), t(p.Bs)


def alloc_c(p: mi.Problem, guard: int = 0):
    """C on the device: NaN-filled when use_acc is off (every element must be
    overwritten), else the problem's C_in.  With guard > 0 the tensor is a
    view into a larger buffer whose guard elements hold a canary."""
    dt = torch.float32 if p.out_dtype == mi.OUT_F32 else torch.bfloat16
    total = p.M * p.N + 2 * guard
    buf = torch.empty(total, dtype=dt, device="cuda:0")
    buf.fill_(float("nan"))
    if guard:
        buf[:guard] = 1.5
        buf[-guard:] = -2.25
    c = buf[guard:guard + p.M * p.N].view(p.M, p.N)
    if p.use_acc:
        if p.out_dtype == mi.OUT_F32:
            c.copy_(torch.from_numpy(p.Cin))
        else:
            c.copy_(torch.from_numpy(p.Cin.view(np.int16)).view(torch.bfloat16))
    return buf, c


def run(gemm, p: mi.Problem, variant=None, guard: int = 0, dev_inputs=None):
    A, As, B, Bs = dev_inputs if dev_inputs is not None else to_dev(p)
    buf, c = alloc_c(p, guard)
    if variant is not None:
        gemm.set_variant(variant)
    gemm(A, As, p.fmtA, B, Bs, p.fmtB, c, use_acc=p.use_acc, out_dtype=p.out_dtype)
    torch.cuda.synchronize()
    if guard:
        g0 = buf[:guard].float().cpu().numpy()
        g1 = buf[-guard:].float().cpu().numpy()
        assert np.all(g0 == 1.5) and np.all(g1 == -2.25), "store outside C"
    return c_numpy(c, p.out_dtype)


def c_numpy(c, out_dtype):
    if out_dtype == mi.OUT_F32:
        return c.cpu().numpy()
    return c.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f32(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def bf16_ulp(x):
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(x > 0, x, 1.0)))
    u = np.ldexp(1.0, (e - 7).astype(np.int64))
    return np.where((x >= 2.0**-126) & np.isfinite(x), u, 2.0**-133)


def compare(got, ref: dict, out_dtype: int, where: str = ""):
    """got: fp32 array or uint16 bf16 bits at the same points as ref."""
    if out_dtype == mi.OUT_F32:
        g = np.asarray(got, np.float64).ravel()
        r = ref["ref32"].astype(np.float64).ravel()
        tol = TOL_REL * ref["mag"].ravel()
    else:
        g = bf16_to_f32(np.asarray(got).ravel()).astype(np.float64)
        r = bf16_to_f32(ref["refbf16"].ravel()).astype(np.float64)
        tol = TOL_REL * ref["mag"].ravel() + bf16_ulp(r)
    nan_r, nan_g = np.isnan(r), np.isnan(g)
    assert np.array_equal(nan_r, nan_g), f"{where}: NaN pattern differs ({nan_g.sum()} vs {nan_r.sum()})"
    inf_r = np.isinf(r) | np.isinf(g)
    assert np.array_equal(g[inf_r], r[inf_r]), f"{where}: infinities differ"
    ok = ~(nan_r | inf_r)
    err = np.abs(g[ok] - r[ok])
    bad = err > tol[ok]
    if bad.any():
        idx = np.flatnonzero(ok)[np.flatnonzero(bad)[:5]]
        raise AssertionError(f"{where}: {bad.sum()} of {ok.sum()} outside tolerance; e.g. idx {idx} "
                             f"got {g[idx]} ref {r[idx]} tol {tol[idx]}")
    return float(np.max(err / np.maximum(tol[ok], 1e-300))) if err.size else 0.0


def oracle_full(p: mi.Problem):
    return oracle.gemm_full(p.A, p.As, p.fmtA, p.B, p.Bs, p.fmtB, p.M, p.N, p.K, cin=p.Cin)


def oracle_points(p: mi.Problem, rows, cols):
    return oracle.gemm_points(p.A, p.As, p.fmtA, p.B, p.Bs, p.fmtB, p.M, p.N, p.K, rows, cols,
                              cin=p.Cin)


def unpacked(x, fmt: int, K: int):
    """(rows, K) codes of an operand stored packed along K (sub-byte
    formats) or one code per byte."""
    bits = mi.CODE_BITS[fmt]
    return np.asarray(x) if bits == 8 else mi.unpack_bits(x, bits, K)


def native_group_extra(p: mi.Problem):
    """Extra error allowed for the native scaled-MFMA variants: each aligned
    group of 8 products is summed in a window reaching 13 bits below the
    group's largest product (measured on the device), so the bound adds
    8 * sum_g 2^(E_g - 13), E_g = floor(log2 max_{k in g} |a_k b_k|)."""
    M, N, K = p.M, p.N, p.K
    ta, tb, te = oracle.decode_table(p.fmtA), oracle.decode_table(p.fmtB), oracle.decode_table(oracle.FMT_E8M0)
    a = ta[unpacked(p.A, p.fmtA, K)] * np.repeat(te[p.As], 32, axis=1)[:, :K]
    b = tb[unpacked(p.B, p.fmtB, K)] * np.repeat(te[p.Bs], 32, axis=1)[:, :K]
    gmax = np.zeros((M, N))
    for g0 in range(0, K, 8):
        prod = np.abs(a[:, None, g0:g0 + 8] * b[None, :, g0:g0 + 8]).max(axis=2)
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(prod))
        gmax += np.where(prod > 0, np.ldexp(1.0, np.where(prod > 0, e, 0).astype(np.int64) - 13), 0)
    return 8 * gmax


def compare_native(got, ref: dict, out_dtype: int, extra, where: str = ""):
    """The native variants' bound: 1e-5 * sum|ab| + extra (+ one bf16 ulp)."""
    if out_dtype == mi.OUT_F32:
        g = np.asarray(got, np.float64)
        r = ref["ref32"].astype(np.float64)
        tol = TOL_REL * ref["mag"] + extra
    else:
        g = bf16_to_f32(got).astype(np.float64)
        r = bf16_to_f32(ref["refbf16"]).astype(np.float64)
        tol = TOL_REL * ref["mag"] + extra + bf16_ulp(r)
    bad = np.abs(g - r) > tol
    assert not bad.any(), f"{where}: {bad.sum()} outside the native bound"
