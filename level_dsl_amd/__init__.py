"""MI355X (gfx950) microscaled FP8 matrix multiply -- Python binding.

Thin ctypes binding of ``libmxgemm.so`` (C ABI in include/mxgemm.h), with
the same entry-point names.  It only marshals arguments: every step of the
multiply runs in the library's HIP kernels.  PyTorch supplies device memory
and streams; it is imported before the library is loaded so that both use
the one HIP runtime already in the process.

If the library has not been built this module raises on use; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the process's HIP runtime first)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmxgemm.so")

MXGEMM_FMT_E4M3 = 0
MXGEMM_FMT_E5M2 = 1
MXGEMM_FMT_E2M3 = 2
MXGEMM_FMT_E3M2 = 3
MXGEMM_FMT_E2M1 = 4
MXGEMM_OUT_F32 = 0
MXGEMM_OUT_BF16 = 1
MXGEMM_X_F32 = 0
MXGEMM_X_BF16 = 1
MXGEMM_VARIANT_AUTO = 0
MXGEMM_VARIANT_LARGE = 1
MXGEMM_VARIANT_SKINNY = 2
MXGEMM_VARIANT_LARGE_NATIVE = 3
MXGEMM_VARIANT_SKINNY_NATIVE = 4
MXGEMM_WORKSPACE_BYTES = 4096 + 256 * 64 * 112 * 4
MXGEMM_WORKSPACE_BYTES_LARGE = 4096 + 256 * 256 * 256 * 4
MXGEMM_NOALLOC_SCRATCH_BYTES = MXGEMM_WORKSPACE_BYTES
MXGEMM_SCALES_ROW_MAJOR = 0
MXGEMM_SCALES_PRESHUFFLED = 1

STATUS = {0: "MXGEMM_OK", 1: "MXGEMM_ERR_NULL", 2: "MXGEMM_ERR_FMT", 3: "MXGEMM_ERR_DTYPE",
          4: "MXGEMM_ERR_SHAPE", 5: "MXGEMM_ERR_ALIGN", 6: "MXGEMM_ERR_DEVICE",
          7: "MXGEMM_ERR_HIP", 8: "MXGEMM_ERR_HANDLE", 9: "MXGEMM_ERR_ALIAS",
          10: "MXGEMM_ERR_VARIANT", 11: "MXGEMM_ERR_WORKSPACE"}
STATUS_CODE = {v: k for k, v in STATUS.items()}

# name -> (restype, argtypes), in the order of include/mxgemm.h
_vp, _i32, _i64, _u8p = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
SIGNATURES = {
    "mxgemm_version": (_i32, []),
    "mxgemm_create": (_i32, [ctypes.POINTER(ctypes.c_void_p)]),
    "mxgemm_destroy": (_i32, [_vp]),
    "mxgemm_set_variant": (_i32, [_vp, _i32]),
    "mxgemm_set_workspace": (_i32, [_vp, _vp, ctypes.c_size_t, _vp]),
    "mxgemm_operand_buffer_bytes": (_i64, [_i32, _i32, _i64, _i64, _i64]),
    "mxgemm_set_operand_buffer": (_i32, [_vp, _vp, ctypes.c_size_t]),
    "mxgemm_widen": (_i32, [_vp, _vp, _i32, _i64, _i64, _u8p, _vp]),
    "mxgemm_set_splits": (_i32, [_vp, _i32]),
    "mxgemm_set_scale_layout": (_i32, [_vp, _i32]),
    "mxgemm_scale_bytes": (_i64, [_i32, _i64, _i64]),
    "mxgemm_preshuffle_scales": (_i32, [_vp, _u8p, _u8p, _i64, _i64, _vp]),
    "mxgemm_validate_args": (_i32, [_vp, _u8p, _i32, _vp, _u8p, _i32, _vp, _i64, _i64, _i64,
                                    _i32, _i32]),
    "mxgemm_run": (_i32, [_vp, _vp, _u8p, _i32, _vp, _u8p, _i32, _vp, _i64, _i64, _i64, _i32,
                          _i32, _vp]),
    "mxgemm_run_noalloc": (_i32, [_vp, _vp, _u8p, _i32, _vp, _u8p, _i32, _vp, _i64, _i64, _i64,
                                  _i32, _i32, _vp]),
    "mxgemm_validate_quantize": (_i32, [_vp, _i32, _i64, _i64, _i32, _u8p, _u8p]),
    "mxgemm_quantize": (_i32, [_vp, _vp, _i32, _i64, _i64, _i32, _u8p, _u8p, _vp]),
    "mxgemm_validate_copy": (_i32, [_vp, _vp, ctypes.c_uint64]),
    "mxgemm_copy": (_i32, [_vp, _vp, _vp, ctypes.c_uint64, _vp]),
    "mxgemm_status_string": (ctypes.c_char_p, [_i32]),
}

_lib = None


class MxgemmError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)} ({status_string(code)})")


def load_library(path: str = LIB_PATH):
    """Load libmxgemm.so; raises if it has not been built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_string(code: int) -> str:
    return load_library().mxgemm_status_string(int(code)).decode()


def _check(code: int, where: str):
    if code != 0:
        raise MxgemmError(code, where)


def mxgemm_version() -> int:
    return load_library().mxgemm_version()


def mxgemm_create() -> int:
    h = ctypes.c_void_p()
    _check(load_library().mxgemm_create(ctypes.byref(h)), "mxgemm_create")
    return h.value


def mxgemm_destroy(h: int) -> None:
    _check(load_library().mxgemm_destroy(h), "mxgemm_destroy")


def mxgemm_set_variant(h: int, variant: int) -> None:
    _check(load_library().mxgemm_set_variant(h, int(variant)), "mxgemm_set_variant")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def mxgemm_set_workspace(h, ws, nbytes: int, stream=None) -> None:
    """Attach a device buffer of at least MXGEMM_WORKSPACE_BYTES (256-byte
    aligned) for split-K, or detach with ws=None; zeroes its counters on
    `stream`."""
    _check(load_library().mxgemm_set_workspace(h, _ptr(ws), int(nbytes),
                                               _stream(stream) if ws is not None else None),
           "mxgemm_set_workspace")


def mxgemm_operand_buffer_bytes(fmtA: int, fmtB: int, M: int, N: int, K: int) -> int:
    """Bytes of the operand buffer a widened format pair needs (0: the pair
    runs as it is, -1: invalid arguments)."""
    return int(load_library().mxgemm_operand_buffer_bytes(int(fmtA), int(fmtB), int(M), int(N),
                                                          int(K)))


def mxgemm_set_operand_buffer(h, buf, nbytes: int) -> None:
    """Attach a device buffer (256-byte aligned) for widened operands, or
    detach with buf=None."""
    _check(load_library().mxgemm_set_operand_buffer(h, _ptr(buf), int(nbytes) if buf is not None else 0),
           "mxgemm_set_operand_buffer")


def mxgemm_widen(h, src, fmt: int, rows: int, K: int, dst, stream=None) -> None:
    """rows x K sub-byte codes (e2m1 / e2m3 / e3m2) -> rows x K e4m3 bytes
    of the same values, on `stream` (default: torch's current stream)."""
    _check(load_library().mxgemm_widen(h, _ptr(src), int(fmt), int(rows), int(K), _ptr(dst),
                                       _stream(stream)),
           "mxgemm_widen")


def row_bytes(fmt: int, K: int) -> int:
    """Bytes of an operand row of K codes: e2m1 K/2, e2m3 and e3m2 3K/4,
    e4m3 / e5m2 K."""
    if fmt == MXGEMM_FMT_E2M1:
        return K // 2
    if fmt in (MXGEMM_FMT_E2M3, MXGEMM_FMT_E3M2):
        return 3 * K // 4
    return K


def codes_per_row(fmt: int, nbytes: int) -> int:
    """K of an operand row of `nbytes` bytes (the inverse of row_bytes)."""
    if fmt == MXGEMM_FMT_E2M1:
        return 2 * nbytes
    if fmt in (MXGEMM_FMT_E2M3, MXGEMM_FMT_E3M2):
        return 4 * nbytes // 3
    return nbytes


def mxgemm_set_splits(h, splits: int) -> None:
    """K splits of later calls: 0 automatic, 1 never, S >= 2 forced."""
    _check(load_library().mxgemm_set_splits(h, int(splits)), "mxgemm_set_splits")


def mxgemm_set_scale_layout(h, layout: int) -> None:
    """Scale layout of later multiplies and quantizations through h:
    MXGEMM_SCALES_ROW_MAJOR (default) or MXGEMM_SCALES_PRESHUFFLED."""
    _check(load_library().mxgemm_set_scale_layout(h, int(layout)), "mxgemm_set_scale_layout")


def mxgemm_scale_bytes(layout: int, rows: int, K: int) -> int:
    """Bytes of a rows x K operand's scale buffer in `layout` (0: invalid)."""
    return int(load_library().mxgemm_scale_bytes(int(layout), int(rows), int(K)))


def mxgemm_preshuffle_scales(h, src, dst, rows: int, K: int, stream=None) -> None:
    """Row-major scale bytes (rows x K/32) to the preshuffled layout, on
    `stream` (default: torch's current stream)."""
    _check(load_library().mxgemm_preshuffle_scales(h, _ptr(src), _ptr(dst), int(rows), int(K),
                                                   _stream(stream)),
           "mxgemm_preshuffle_scales")


def _ptr(x) -> int:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def mxgemm_validate_args(A, A_scale, fmtA, B, B_scale, fmtB, C, M, N, K, use_acc,
                         out_dtype) -> int:
    """Returns the status code (0 = valid); pure host check."""
    return load_library().mxgemm_validate_args(
        _ptr(A), _ptr(A_scale), int(fmtA), _ptr(B), _ptr(B_scale), int(fmtB), _ptr(C),
        int(M), int(N), int(K), int(use_acc), int(out_dtype))


def mxgemm_run(h, A, A_scale, fmtA, B, B_scale, fmtB, C, M, N, K, use_acc, out_dtype,
               stream=None) -> None:
    """C (+)= (A*2^(As-127)) @ (B*2^(Bs-127)) on `stream` (default: torch's
    current stream).  Tensors are passed by device pointer; shapes and dtypes
    are the caller's responsibility, as in the C ABI."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    _check(load_library().mxgemm_run(
        h, _ptr(A), _ptr(A_scale), int(fmtA), _ptr(B), _ptr(B_scale), int(fmtB), _ptr(C),
        int(M), int(N), int(K), int(use_acc), int(out_dtype), stream), "mxgemm_run")


def mxgemm_run_noalloc(h, A, A_scale, fmtA, B, B_scale, fmtB, C, M, N, K, use_acc, out_dtype,
                       stream=None) -> None:
    """mxgemm_run with the library's fixed split-K scratch instead of an
    attached workspace: allocates nothing (calls on one GPU must not overlap)."""
    _check(load_library().mxgemm_run_noalloc(
        h, _ptr(A), _ptr(A_scale), int(fmtA), _ptr(B), _ptr(B_scale), int(fmtB), _ptr(C),
        int(M), int(N), int(K), int(use_acc), int(out_dtype), _stream(stream)), "mxgemm_run_noalloc")


def mxgemm_validate_quantize(X, x_dtype, R, K, fmt, codes, scales) -> int:
    """Returns the status code (0 = valid); pure host check."""
    return load_library().mxgemm_validate_quantize(
        _ptr(X), int(x_dtype), int(R), int(K), int(fmt), _ptr(codes), _ptr(scales))


def mxgemm_quantize(h, X, x_dtype, R, K, fmt, codes, scales, stream=None) -> None:
    """MX block quantization of the R x K matrix X into codes (R x K) and
    scales (R x K/32) on `stream` (default: torch's current stream)."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    _check(load_library().mxgemm_quantize(
        h, _ptr(X), int(x_dtype), int(R), int(K), int(fmt), _ptr(codes), _ptr(scales), stream),
        "mxgemm_quantize")


def mxgemm_validate_copy(dst, src, nbytes) -> int:
    """Returns the status code (0 = valid); pure host check."""
    return load_library().mxgemm_validate_copy(_ptr(dst), _ptr(src), int(nbytes))


def mxgemm_copy(h, dst, src, nbytes, stream=None) -> None:
    """Streaming copy of nbytes from src to dst on `stream` (default: torch's
    current stream); the achievable-bandwidth reference of the benchmark."""
    _check(load_library().mxgemm_copy(h, _ptr(dst), _ptr(src), int(nbytes), _stream(stream)),
           "mxgemm_copy")


class Gemm:
    """Owns one handle; call(...) checks tensor shapes and runs."""

    def __init__(self):
        self.h = mxgemm_create()
        self.scale_layout = MXGEMM_SCALES_ROW_MAJOR

    def close(self):
        if self.h:
            mxgemm_destroy(self.h)
            self.h = None

    def __del__(self):  # pragma: no cover
        try:
            self.close()
        except Exception:
            pass

    def set_variant(self, variant: int):
        mxgemm_set_variant(self.h, variant)

    def enable_split_k(self, device="cuda:0", stream=None, nbytes=MXGEMM_WORKSPACE_BYTES_LARGE):
        """Give the handle its own split-K workspace (a torch allocation that
        this object keeps alive); calls through this handle must then be
        ordered on one stream.  The default size never limits a split."""
        if getattr(self, "workspace", None) is None:
            self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
            mxgemm_set_workspace(self.h, self.workspace, nbytes, stream)

    def disable_split_k(self):
        if getattr(self, "workspace", None) is not None:
            mxgemm_set_workspace(self.h, None, 0)
            self.workspace = None

    def set_splits(self, splits: int):
        mxgemm_set_splits(self.h, splits)

    def ensure_operand_buffer(self, fmtA, fmtB, M, N, K, device="cuda:0"):
        """Attach an operand buffer large enough for a widened pair (a torch
        allocation this object keeps, grown as needed); calls through this
        handle must then be ordered on one stream."""
        need = mxgemm_operand_buffer_bytes(fmtA, fmtB, M, N, K)
        if need <= 0:
            return
        device = torch.device(device)
        cur = getattr(self, "opbuf", None)
        if cur is None or cur.numel() < need or cur.device != device:
            torch.cuda.synchronize(device)  # a call on any stream may still read the old buffer
            self.opbuf = torch.empty(need, dtype=torch.uint8, device=device)
            mxgemm_set_operand_buffer(self.h, self.opbuf, need)

    def set_scale_layout(self, layout: int):
        """Scales of later calls are row-major (R, K/32) tensors, or with
        MXGEMM_SCALES_PRESHUFFLED (ceil(R/32)*32, K/32) tensors holding the
        preshuffled bytes."""
        mxgemm_set_scale_layout(self.h, layout)
        self.scale_layout = layout

    def _scale_shape(self, rows: int, K: int):
        if self.scale_layout == MXGEMM_SCALES_PRESHUFFLED:
            return ((rows + 31) // 32 * 32, K // 32)
        return (rows, K // 32)

    def preshuffle_scales(self, S, stream=None):
        """A contiguous (R, K/32) uint8 device tensor of row-major scale
        bytes -> a new (ceil(R/32)*32, K/32) tensor in the preshuffled
        layout (padding rows zero)."""
        if S.dim() != 2 or S.dtype != torch.uint8 or not S.is_contiguous() or S.device.type != "cuda":
            raise ValueError("S must be a contiguous 2-D uint8 device tensor")
        R, kb = S.shape
        out = torch.empty(((R + 31) // 32 * 32, kb), dtype=torch.uint8, device=S.device)
        mxgemm_preshuffle_scales(self.h, S, out, R, 32 * kb, stream)
        return out

    def __call__(self, A, A_scale, fmtA, B, B_scale, fmtB, C, use_acc=False,
                 out_dtype=MXGEMM_OUT_F32, stream=None):
        # sub-byte operands are packed along K: e2m1 two codes per byte,
        # e2m3 / e3m2 four codes per three bytes
        M, ka = A.shape
        N = B.shape[0]
        K = codes_per_row(fmtA, ka)
        if B.shape[1] != row_bytes(fmtB, K) or A_scale.shape != self._scale_shape(M, K) or \
                B_scale.shape != self._scale_shape(N, K):
            raise ValueError("operand shapes do not match (A MxK, B NxK, scales K/32 per row, "
                             "preshuffled: rows padded to 32; e2m1: K/2 bytes per row, "
                             "e2m3 / e3m2: 3K/4)")
        want = torch.float32 if out_dtype == MXGEMM_OUT_F32 else torch.bfloat16
        if C.shape != (M, N) or C.dtype != want:
            raise ValueError(f"C must be ({M}, {N}) {want}")
        for t in (A, A_scale, B, B_scale, C):
            if not t.is_contiguous() or t.device.type != "cuda":
                raise ValueError("all operands must be contiguous device tensors")
        self.ensure_operand_buffer(fmtA, fmtB, M, N, K, A.device)
        mxgemm_run(self.h, A, A_scale, fmtA, B, B_scale, fmtB, C, M, N, K, int(bool(use_acc)),
                   out_dtype, stream)
        return C

    def quantize(self, X, fmt, codes=None, scales=None, stream=None):
        """MX block quantization of a contiguous (R, K) fp32 or bf16 device
        tensor; returns (codes (R, K) uint8, scales (R, K/32) uint8)."""
        if X.dim() != 2 or not X.is_contiguous() or X.device.type != "cuda":
            raise ValueError("X must be a contiguous 2-D device tensor")
        if X.dtype == torch.float32:
            xd = MXGEMM_X_F32
        elif X.dtype == torch.bfloat16:
            xd = MXGEMM_X_BF16
        else:
            raise ValueError("X must be float32 or bfloat16")
        R, K = X.shape
        kc = row_bytes(fmt, K)  # e2m1: two codes per byte; e2m3 / e3m2: four per three bytes
        if codes is None:
            codes = torch.empty((R, kc), dtype=torch.uint8, device=X.device)
        if scales is None:
            # preshuffled: the padding rows, which the quantizer does not
            # write, start as zeros
            scales = torch.zeros(self._scale_shape(R, K), dtype=torch.uint8, device=X.device)
        if codes.shape != (R, kc) or scales.shape != self._scale_shape(R, K) or \
                codes.dtype != torch.uint8 or scales.dtype != torch.uint8:
            raise ValueError("codes must be (R, K) (e2m1: (R, K/2), e2m3 / e3m2: (R, 3K/4)) and "
                             "scales (R, K/32) (preshuffled: rows padded to 32), uint8")
        mxgemm_quantize(self.h, X, xd, R, K, fmt, codes, scales, stream)
        return codes, scales
