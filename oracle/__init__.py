"""CPU oracle for the MX-FP8 matrix multiply (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (``level_dsl_amd``)
never does, and this package imports nothing from it.

The arithmetic lives in ``mxref.c`` (plain C, binary64).  It is the plain
definition of the scaled dot that the TLX API Quick Reference lists as
``async_dot_scaled`` ("Matrix Multiply (MMA)" table: D = (A*scale_A) @
(B*scale_B) + D, FP8 inputs), with one uint8 scale per 32 K-elements (TLX
async-compute page, "TMEM-backed MX Scales": scale tiles of K extent
BLOCK_K // 32).  This module is argument marshalling only.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxref.c")
_LIB = os.path.join(_HERE, "libmxref.so")

FMT_E4M3 = 0
FMT_E5M2 = 1
FMT_E2M3 = 2
FMT_E3M2 = 3
FMT_E8M0 = 8

GCC_FLAGS = ["-O2", "-std=c99", "-Wall", "-Wextra", "-ffp-contract=off",
             "-fno-fast-math", "-fPIC", "-shared", "-pthread"]


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (no HIP involved)."""
    cmd = ["gcc", *GCC_FLAGS, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def _bind(lib):
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.mxref_version.restype = i32
    lib.mxref_decode.argtypes = [i32, i32]
    lib.mxref_decode.restype = ctypes.c_double
    lib.mxref_bf16_rne.argtypes = [ctypes.c_float]
    lib.mxref_bf16_rne.restype = ctypes.c_uint16
    lib.mxref_gemm_points.argtypes = [vp, vp, i32, vp, vp, i32, vp, i32,
                                      i64, i64, i64, vp, vp, i64,
                                      vp, vp, vp, vp, i32]
    lib.mxref_gemm_points.restype = i32
    lib.mxref_quantize.argtypes = [vp, i32, i64, i64, i32, vp, vp]
    lib.mxref_quantize.restype = i32
    return lib


def load(path: str = _LIB):
    """Load the built oracle, building it first only if it is absent."""
    global _lib
    if path == _LIB and _lib is not None:
        return _lib
    if not os.path.exists(path):
        build(out=path)
    lib = _bind(ctypes.CDLL(path))
    if path == _LIB:
        _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


FMT_E2M1 = 4
CODE_BITS = {FMT_E4M3: 8, FMT_E5M2: 8, FMT_E2M3: 6, FMT_E3M2: 6, FMT_E2M1: 4}


def packed_width(K: int, fmt: int) -> int:
    """Bytes per operand row: K codes of 8, 6 or 4 bits (ceil(bits*K/8))."""
    return (K * CODE_BITS[fmt] + 7) // 8


def decode_table(fmt: int, lib=None) -> np.ndarray:
    """All 256 decoded values of a format (0 e4m3, 1 e5m2, 2 e2m3, 3 e3m2,
    4 e2m1, 8 e8m0; codes past a sub-byte format's range decode to NaN)."""
    lib = lib or load()
    return np.array([lib.mxref_decode(fmt, c) for c in range(256)], dtype=np.float64)


def bf16_rne(x: np.ndarray, lib=None) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    lib = lib or load()
    x = np.asarray(x, dtype=np.float32).ravel()
    return np.array([lib.mxref_bf16_rne(float(v)) for v in x], dtype=np.uint16)


def _ptr(a):
    return None if a is None else a.ctypes.data


def gemm_points(A, As, fmtA, B, Bs, fmtB, M, N, K, rows, cols,
                cin=None, nthreads=None, lib=None):
    """Oracle outputs at points (rows[p], cols[p]).

    A: (M, K) uint8 codes; B: (N, K) uint8 codes (K contiguous); a sub-byte
    operand (e2m3 / e3m2: 6 bits, e2m1: 4 bits per code) is
    (rows, ceil(bits*K/8)) bytes, code k at bits bits*k .. bits*k+bits-1 of
    the row read as one little-endian bit string;
    As: (M, ceil(K/32)) and Bs: (N, ceil(K/32)) uint8 e8m0 bytes.
    cin: None (use_acc off), or the incoming (M, N) C as float32, or as
    uint16 bf16 bit patterns.
    Returns a dict of numpy arrays: ref32 (float32), refbf16 (uint16 bits),
    sum (float64 exact-product sum), mag (float64 sum of |products|).
    """
    lib = lib or load()
    kb = (K + 31) // 32
    A = np.ascontiguousarray(A, dtype=np.uint8).reshape(M, packed_width(K, fmtA))
    B = np.ascontiguousarray(B, dtype=np.uint8).reshape(N, packed_width(K, fmtB))
    As = np.ascontiguousarray(As, dtype=np.uint8).reshape(M, kb)
    Bs = np.ascontiguousarray(Bs, dtype=np.uint8).reshape(N, kb)
    rows = np.ascontiguousarray(rows, dtype=np.int64).ravel()
    cols = np.ascontiguousarray(cols, dtype=np.int64).ravel()
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in length")
    npts = rows.size
    cin_dtype = 0
    if cin is not None:
        cin = np.ascontiguousarray(cin)
        if cin.dtype == np.float32:
            cin_dtype = 0
        elif cin.dtype == np.uint16:
            cin_dtype = 1
        else:
            raise TypeError("cin must be float32 or uint16 (bf16 bits)")
        cin = cin.reshape(M, N)
    out = {
        "sum": np.empty(npts, np.float64),
        "mag": np.empty(npts, np.float64),
        "ref32": np.empty(npts, np.float32),
        "refbf16": np.empty(npts, np.uint16),
    }
    rc = lib.mxref_gemm_points(
        _ptr(A), _ptr(As), int(fmtA), _ptr(B), _ptr(Bs), int(fmtB),
        _ptr(cin), cin_dtype, int(M), int(N), int(K),
        _ptr(rows), _ptr(cols), int(npts),
        _ptr(out["sum"]), _ptr(out["mag"]), _ptr(out["ref32"]),
        _ptr(out["refbf16"]), int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError(f"mxref_gemm_points rejected its arguments (rc={rc})")
    return out


def gemm_full(A, As, fmtA, B, Bs, fmtB, M, N, K, cin=None, nthreads=None, lib=None):
    """Oracle over every output; arrays come back shaped (M, N)."""
    mm, nn = np.meshgrid(np.arange(M, dtype=np.int64), np.arange(N, dtype=np.int64),
                         indexing="ij")
    r = gemm_points(A, As, fmtA, B, Bs, fmtB, M, N, K, mm.ravel(), nn.ravel(),
                    cin=cin, nthreads=nthreads, lib=lib)
    return {k: v.reshape(M, N) for k, v in r.items()}


def quantize(X, fmt, lib=None):
    """MX block quantization of an (R, K) matrix: X float32, or uint16 bf16
    bit patterns.  Returns (codes (R, K) uint8 -- sub-byte formats packed as
    the operands of gemm_points are -- scales (R, ceil(K/32)) uint8).
    Raises ValueError for non-finite input (the recipe covers finite values)."""
    lib = lib or load()
    X = np.ascontiguousarray(X)
    if X.ndim != 2:
        raise ValueError("X must be 2-D")
    if X.dtype == np.float32:
        x_dtype = 0
    elif X.dtype == np.uint16:
        x_dtype = 1
    else:
        raise TypeError("X must be float32 or uint16 (bf16 bits)")
    R, K = X.shape
    codes = np.empty((R, packed_width(K, fmt)), np.uint8)
    scales = np.empty((R, (K + 31) // 32), np.uint8)
    rc = lib.mxref_quantize(_ptr(X), x_dtype, int(R), int(K), int(fmt), _ptr(codes), _ptr(scales))
    if rc == -2:
        raise ValueError("non-finite input")
    if rc != 0:
        raise ValueError(f"mxref_quantize rejected its arguments (rc={rc})")
    return codes, scales
