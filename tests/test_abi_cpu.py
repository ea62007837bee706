"""The C-ABI library on the CPU: it loads, exports every function that
include/mxgemm.h declares, and its host-side argument checks return the
documented status codes.  No GPU call is made here."""
import os
import re
import subprocess

import pytest

import level_dsl_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxgemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mxgemm_\w+)\s*\(", text, re.M)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert names == sorted(L.SIGNATURES), names


def test_library_exports_every_declared_symbol():
    lib = L.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (mxgemm_\w+)", out))
    assert set(declared_functions()) <= exported


def test_status_strings_and_version():
    assert L.mxgemm_version() == 1
    for code in range(0, 12):
        s = L.status_string(code)
        assert s and s != "unknown status"
    assert L.status_string(99) == "unknown status"


A, AS, B, BS, C = 0x10000, 0x20001, 0x30000, 0x40003, 0x1000000


def v(**kw):
    args = dict(A=A, A_scale=AS, fmtA=0, B=B, B_scale=BS, fmtB=0, C=C, M=64, N=64, K=128,
                use_acc=0, out_dtype=0)
    args.update(kw)
    return L.mxgemm_validate_args(**args)


@pytest.mark.parametrize("kw,code", [
    ({}, "MXGEMM_OK"),
    ({"A": 0}, "MXGEMM_ERR_NULL"), ({"B_scale": 0}, "MXGEMM_ERR_NULL"), ({"C": 0}, "MXGEMM_ERR_NULL"),
    ({"fmtA": 5}, "MXGEMM_ERR_FMT"), ({"fmtB": -1}, "MXGEMM_ERR_FMT"), ({"fmtB": 7}, "MXGEMM_ERR_FMT"),
    ({"fmtA": 2}, "MXGEMM_OK"), ({"fmtA": 4}, "MXGEMM_OK"), ({"fmtB": 4}, "MXGEMM_OK"),
    ({"fmtA": 3, "fmtB": 3}, "MXGEMM_OK"), ({"fmtA": 3, "fmtB": 1}, "MXGEMM_OK"),
    ({"fmtA": 4, "fmtB": 2}, "MXGEMM_OK"),
    # B's byte range follows fmtB: C right after a 64 x 128 e2m1 B (4 KiB) is
    # disjoint from it, and overlaps the same B read as e4m3 (8 KiB)
    ({"fmtB": 4, "C": 0x31000}, "MXGEMM_OK"), ({"C": 0x31000}, "MXGEMM_ERR_ALIAS"),
    ({"fmtB": 3, "C": 0x31800}, "MXGEMM_OK"), ({"fmtB": 3, "C": 0x31000}, "MXGEMM_ERR_ALIAS"),
    ({"fmtA": 4, "fmtB": 4}, "MXGEMM_OK"), ({"fmtA": 4, "fmtB": 4, "K": 48}, "MXGEMM_ERR_SHAPE"),
    ({"out_dtype": 2}, "MXGEMM_ERR_DTYPE"), ({"use_acc": 2}, "MXGEMM_ERR_DTYPE"),
    ({"M": 0}, "MXGEMM_ERR_SHAPE"), ({"N": -3}, "MXGEMM_ERR_SHAPE"), ({"K": 0}, "MXGEMM_ERR_SHAPE"),
    ({"K": 48}, "MXGEMM_ERR_SHAPE"), ({"K": 16}, "MXGEMM_ERR_SHAPE"),
    ({"N": (1 << 20) + 1}, "MXGEMM_ERR_SHAPE"), ({"K": (1 << 21) + 32}, "MXGEMM_ERR_SHAPE"),
    ({"M": (1 << 30) + 1}, "MXGEMM_ERR_SHAPE"), ({"M": 1 << 20, "N": 1 << 17}, "MXGEMM_ERR_SHAPE"),
    ({"A": A + 8}, "MXGEMM_ERR_ALIGN"), ({"C": C + 4}, "MXGEMM_ERR_ALIGN"),
    ({"B": B + 1}, "MXGEMM_ERR_ALIGN"),
    ({"C": A + 16}, "MXGEMM_ERR_ALIAS"), ({"C": 0x40000 - 64 * 64 * 4 + 16}, "MXGEMM_ERR_ALIAS"),
    ({"M": 1, "N": 1, "K": 32}, "MXGEMM_OK"), ({"out_dtype": 1, "use_acc": 1}, "MXGEMM_OK"),
])
def test_validate_args(kw, code):
    assert v(**kw) == L.STATUS_CODE[code]


@pytest.mark.parametrize("fa,fb,M,N,K,want", [
    (0, 0, 64, 64, 128, 0), (1, 0, 64, 64, 128, 0), (4, 4, 64, 64, 128, 0), (2, 2, 64, 64, 128, 0),
    (3, 3, 64, 64, 128, 64 * 128 + 64 * 128),            # e3m2: both widened
    (4, 0, 65, 64, 128, 65 * 128 + 128 + 0),              # A widened: M*K rounded up to 256
    (0, 2, 65, 64, 128, 64 * 128),                         # B widened only
    (2, 4, 3, 5, 32, 256 + 5 * 32),                        # both, A padded to 256
    (5, 0, 64, 64, 128, -1), (0, 3, 64, 64, 48, -1), (0, 3, 0, 64, 128, -1),
])
def test_operand_buffer_bytes(fa, fb, M, N, K, want):
    assert L.mxgemm_operand_buffer_bytes(fa, fb, M, N, K) == want


def test_row_bytes_round_trip():
    for fmt, per in ((0, 1.0), (1, 1.0), (2, 0.75), (3, 0.75), (4, 0.5)):
        for K in (32, 1056, 1 << 21):
            assert L.row_bytes(fmt, K) == int(K * per)
            assert L.codes_per_row(fmt, L.row_bytes(fmt, K)) == K


def test_widen_entry_points_reject_bad_handle_without_gpu_work():
    for call in (lambda: L.mxgemm_widen(None, 0x100000, 3, 4, 128, 0x200000, 0),
                 lambda: L.mxgemm_set_operand_buffer(None, 0x100000, 4096),
                 lambda: L.mxgemm_set_operand_buffer(None, None, 0)):
        with pytest.raises(L.MxgemmError) as e:
            call()
        assert e.value.code == L.STATUS_CODE["MXGEMM_ERR_HANDLE"]


def test_run_rejects_bad_handle_without_gpu_work():
    lib = L.load_library()
    assert lib.mxgemm_run(None, A, AS, 0, B, BS, 0, C, 64, 64, 128, 0, 0, None) == \
        L.STATUS_CODE["MXGEMM_ERR_HANDLE"]
    assert lib.mxgemm_destroy(None) == 0
    assert lib.mxgemm_set_variant(None, 0) == L.STATUS_CODE["MXGEMM_ERR_HANDLE"]
    assert lib.mxgemm_create(None) == L.STATUS_CODE["MXGEMM_ERR_NULL"]


def test_product_path_has_no_oracle_or_fallback():
    """The binding and the HIP sources never reach the oracle or a CPU path."""
    pkg = os.path.join(ROOT, "level_dsl_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("no oracle", ""), f
                assert "mxref" not in text, f


def vq(**kw):
    args = dict(X=0x100000, x_dtype=0, R=64, K=128, fmt=0, codes=0x200000, scales=0x300001)
    args.update(kw)
    return L.mxgemm_validate_quantize(**args)


@pytest.mark.parametrize("kw,code", [
    ({}, "MXGEMM_OK"), ({"x_dtype": 1}, "MXGEMM_OK"), ({"fmt": 1, "R": 1, "K": 32}, "MXGEMM_OK"),
    ({"X": 0}, "MXGEMM_ERR_NULL"), ({"codes": 0}, "MXGEMM_ERR_NULL"), ({"scales": 0}, "MXGEMM_ERR_NULL"),
    ({"fmt": 2}, "MXGEMM_OK"), ({"fmt": 3}, "MXGEMM_OK"), ({"fmt": 4}, "MXGEMM_OK"),
    ({"fmt": 5}, "MXGEMM_ERR_FMT"), ({"fmt": -1}, "MXGEMM_ERR_FMT"),
    # 6-bit codes take 3/4 of a byte each: 64 x 128 codes end 6 KiB after `codes`
    ({"fmt": 3, "scales": 0x200000 + 64 * 96}, "MXGEMM_OK"),
    ({"fmt": 3, "scales": 0x200000 + 64 * 96 - 1}, "MXGEMM_ERR_ALIAS"),
    ({"x_dtype": 2}, "MXGEMM_ERR_DTYPE"),
    ({"R": 0}, "MXGEMM_ERR_SHAPE"), ({"K": 16}, "MXGEMM_ERR_SHAPE"), ({"K": 48}, "MXGEMM_ERR_SHAPE"),
    ({"K": (1 << 21) + 32}, "MXGEMM_ERR_SHAPE"), ({"R": 1 << 20, "K": 1 << 19}, "MXGEMM_ERR_SHAPE"),
    ({"X": 0x100008}, "MXGEMM_ERR_ALIGN"), ({"codes": 0x200004}, "MXGEMM_ERR_ALIGN"),
    ({"codes": 0x100000 + 64 * 128 * 4 - 16}, "MXGEMM_ERR_ALIAS"),
    ({"scales": 0x200000 + 64 * 128 - 1}, "MXGEMM_ERR_ALIAS"),
    ({"scales": 0x100000 + 64 * 128 * 2, "x_dtype": 1}, "MXGEMM_OK"),
])
def test_validate_quantize(kw, code):
    assert vq(**kw) == L.STATUS_CODE[code]


def test_quantize_rejects_bad_handle_without_gpu_work():
    with pytest.raises(L.MxgemmError) as e:
        L.mxgemm_quantize(None, 0x100000, 0, 64, 128, 0, 0x200000, 0x300000, stream=0)
    assert e.value.code == L.STATUS_CODE["MXGEMM_ERR_HANDLE"]


def test_split_k_entry_points_reject_bad_handle_without_gpu_work():
    for call in (lambda: L.mxgemm_set_workspace(None, 0x100000, L.MXGEMM_WORKSPACE_BYTES, 0),
                 lambda: L.mxgemm_set_workspace(None, None, 0),
                 lambda: L.mxgemm_set_splits(None, 2)):
        with pytest.raises(L.MxgemmError) as e:
            call()
        assert e.value.code == L.STATUS_CODE["MXGEMM_ERR_HANDLE"]


def test_workspace_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define MXGEMM_WORKSPACE_BYTES \(\(size_t\)(\d+) \+ \(size_t\)(\d+) \* (\d+) \* (\d+) \* (\d+)\)", text)
    assert m, "MXGEMM_WORKSPACE_BYTES not found"
    a, b, c, d, e = map(int, m.groups())
    assert a + b * c * d * e == L.MXGEMM_WORKSPACE_BYTES


def test_large_workspace_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define MXGEMM_WORKSPACE_BYTES_LARGE \(\(size_t\)(\d+) \+ \(size_t\)(\d+) \* (\d+) \* (\d+) \* (\d+)\)", text)
    assert m, "MXGEMM_WORKSPACE_BYTES_LARGE not found"
    a, b, c, d, e = map(int, m.groups())
    assert a + b * c * d * e == L.MXGEMM_WORKSPACE_BYTES_LARGE


@pytest.mark.parametrize("dst,src,n,code", [
    (0x100000, 0x200000, 1 << 16, "MXGEMM_OK"),
    (0, 0x200000, 1 << 16, "MXGEMM_ERR_NULL"), (0x100000, 0, 1 << 16, "MXGEMM_ERR_NULL"),
    (0x100000, 0x200000, 0, "MXGEMM_ERR_SHAPE"), (0x100000, 0x200000, 24, "MXGEMM_ERR_SHAPE"),
    (0x100000, 0x200000, (1 << 40) + 16, "MXGEMM_ERR_SHAPE"),
    (0x100008, 0x200000, 64, "MXGEMM_ERR_ALIGN"), (0x100000, 0x200004, 64, "MXGEMM_ERR_ALIGN"),
    (0x100000, 0x100000 + 64, 128, "MXGEMM_ERR_ALIAS"), (0x100000 + 64, 0x100000, 128, "MXGEMM_ERR_ALIAS"),
    (0x100000, 0x100000 + 128, 128, "MXGEMM_OK"),
])
def test_validate_copy(dst, src, n, code):
    assert L.mxgemm_validate_copy(dst, src, n) == L.STATUS_CODE[code]


@pytest.mark.parametrize("layout,rows,K,want", [
    (0, 64, 8192, 64 * 256), (0, 1, 32, 1), (0, 300, 1056, 300 * 33),
    (1, 64, 8192, 64 * 256), (1, 1, 128, 32 * 4), (1, 33, 256, 64 * 8), (1, 28672, 8192, 28672 * 256),
    (1, 300, 1056, 0),            # preshuffled needs K % 128 == 0
    (0, 0, 128, 0), (1, 10, 96, 0), (0, 10, 48, 0), (2, 64, 128, 0), (-1, 64, 128, 0),
    (0, 1 << 31, 128, 0),         # rows beyond MXGEMM_MAX_M
])
def test_scale_bytes(layout, rows, K, want):
    assert L.mxgemm_scale_bytes(layout, rows, K) == want


def test_scale_layout_entry_points_reject_bad_handle_without_gpu_work():
    for call in (lambda: L.mxgemm_set_scale_layout(None, L.MXGEMM_SCALES_PRESHUFFLED),
                 lambda: L.mxgemm_preshuffle_scales(None, 0x100000, 0x200000, 64, 256, 0)):
        with pytest.raises(L.MxgemmError) as e:
            call()
        assert e.value.code == L.STATUS_CODE["MXGEMM_ERR_HANDLE"]
