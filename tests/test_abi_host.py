"""CPU-only checks of the C-ABI library: it loads, exports every function
include/mxq.h declares, and its host-side validation answers before any
launch (so nothing here needs a GPU: invalid calls never reach the device,
and empty calls launch nothing)."""
import ctypes
import os
import re
import subprocess

import pytest

import mx9_dual_axis_amd as mxq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxq.h")
FAKE = 1 << 20          # never dereferenced: every call below fails validation or is empty


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|char|void)\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(["mx_quantize_2d_dual", "mx_quantize_grouped", "mx9_pack", "mx9_unpack",
                                  "mx9_pack_strided", "mx9_unpack_strided",
                                  "mx9_pack_axis", "mx9_unpack_axis", "mx9_pack_records", "mx9_unpack_records",
                                  "mx_gemm_nt", "mx_grouped_gemm_rows", "mx_grouped_gemm_k", "mx_status_string",
                                  "mx_quantize_2d_dual_mfma", "mx_quantize_grouped_mfma", "mx_gemm_nt_mfma",
                                  "mx_grouped_gemm_rows_mfma", "mx_grouped_gemm_k_mfma", "mx_scales_to_mfma",
                                  "mx_scales_from_mfma"])


def test_library_exports_every_declared_symbol():
    lib = mxq.library()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", mxq.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\s[TW]\s(\w+)$", out, flags=re.M))
    for name in _declared():
        assert name in exported, name


def test_status_strings():
    for code in range(10):
        s = mxq.status_string(code)
        assert s.startswith("MX_"), s
    assert "unknown" in mxq.status_string(99)


def _dual(**kw):
    a = dict(x=FAKE, M=256, N=256, ld=256, bs=32, mode=0, qr=FAKE * 2, sr=FAKE * 3, qc=FAKE * 4, sc=FAKE * 5)
    a.update(kw)
    return mxq.library().mx_quantize_2d_dual(a["x"], a["M"], a["N"], a["ld"], a["bs"], a["mode"],
                                             a["qr"], a["sr"], a["qc"], a["sc"], None)


def test_dual_validation_codes():
    assert _dual(x=None) == 1
    assert _dual(bs=16) == 3
    assert _dual(mode=1) == 4
    assert _dual(M=200) == 5 and _dual(N=100) == 5 and _dual(M=-128) == 5
    assert _dual(M=1 << 31) == 5 and _dual(N=(1 << 24) + 128, ld=(1 << 24) + 128) == 5
    assert _dual(ld=(1 << 24) + 8) == 6
    assert _dual(ld=128) == 6 and _dual(ld=260) == 6
    assert _dual(qc=FAKE * 4 + 8) == 7
    assert _dual(qc=FAKE * 2 + 4096) == 8            # q_col starts inside q_row
    assert _dual(sr=FAKE + 1024) == 8                # s_row inside the input
    assert _dual(M=0, x=None, qr=None, sr=None, qc=None, sc=None) == 0     # empty: no-op, no launch


def test_grouped_validation_codes():
    lib = mxq.library()

    def g(offs=FAKE * 6, G=4, err=FAKE * 7, **kw):
        a = dict(x=FAKE, M=256, N=256, ld=256, qr=FAKE * 2, sr=FAKE * 3, qc=FAKE * 4, sc=FAKE * 5)
        a.update(kw)
        return lib.mx_quantize_grouped(a["x"], a["M"], a["N"], a["ld"], 32, 0, offs, G,
                                       a["qr"], a["sr"], a["qc"], a["sc"], err, None)
    assert g(G=-1) == 5
    assert g(offs=None) == 1
    assert g(offs=FAKE * 6 + 2) == 7
    assert g(err=FAKE * 7 + 1) == 7
    assert g(offs=FAKE * 2 + 8) == 8                 # offsets inside q_row
    assert g(err=FAKE * 5 + 4) == 8                  # err inside s_col
    assert g(M=0, G=0, err=None, x=None, qr=None, sr=None, qc=None, sc=None) == 0


def test_mx9_validation_codes():
    lib = mxq.library()

    def pack(dtype=0, rows=4, cols=64, ld=64, bs=16, x=FAKE, q=FAKE * 2, e=FAKE * 3, p=FAKE * 4):
        return lib.mx9_pack(x, dtype, rows, cols, ld, bs, q, e, p, None)

    def unpack(rows=4, cols=64, bs=16, od=0, y=FAKE * 5, ld=64, q=FAKE * 2, e=FAKE * 3, p=FAKE * 4):
        return lib.mx9_unpack(q, e, p, rows, cols, bs, od, y, ld, None)
    assert pack(x=None) == 1 and pack(dtype=2) == 2 and pack(bs=32) == 3 and pack(rows=-1) == 5
    assert pack(ld=32) == 6 and pack(x=FAKE + 2) == 7 and pack(q=FAKE * 2 + 4) == 7
    assert pack(e=FAKE + 16) == 8
    assert pack(rows=0, x=None, q=None, e=None, p=None) == 0
    assert unpack(y=None) == 1 and unpack(od=3) == 2 and unpack(bs=8) == 3 and unpack(cols=-5) == 5
    assert unpack(ld=10) == 6 and unpack(y=FAKE * 5 + 2) == 7 and unpack(q=FAKE * 2 + 8) == 7
    assert unpack(y=FAKE * 2 + 64) == 8
    assert unpack(cols=0, y=None, q=None, e=None, p=None) == 0
    # a pitch that makes the matrix span more than any address space is rejected
    # before anything else is computed from it (no 64-bit overflow)
    assert pack(rows=1 << 31, cols=1, ld=1 << 40) == 6 and unpack(rows=1 << 31, cols=1, ld=1 << 40) == 6
    assert pack(rows=1 << 20, cols=16, ld=1 << 29) == 6 and pack(rows=1 << 10, cols=16, ld=1 << 29, x=FAKE) == 8


def test_mx9_strided_validation_codes():
    lib = mxq.library()
    # 4 rows of 64 columns: 4 blocks per row
    def pack(ld_q=96, ld_e=8, ld_p=8, rows=4, x=FAKE, q=FAKE * 2, e=FAKE * 3, p=FAKE * 4, y=None):
        return lib.mx9_pack_strided(x, 0, rows, 64, 64, 16, q, ld_q, e, ld_e, p, ld_p, None)

    def unpack(ld_q=96, ld_e=8, ld_p=8, rows=4, y=FAKE * 5, q=FAKE * 2, e=FAKE * 3, p=FAKE * 4, x=None):
        return lib.mx9_unpack_strided(q, ld_q, e, ld_e, p, ld_p, rows, 64, 16, 0, y, 64, None)
    for f in (pack, unpack):
        assert f(ld_q=48) == 6 and f(ld_q=72) == 6 and f(ld_e=3) == 6 and f(ld_p=2) == 6
        assert f(ld_q=1 << 41) == 6
        assert f(q=FAKE * 2 + 8) == 7
        assert f(e=FAKE * 2 + 300) == 8            # max_exp rows inside q's pitched span
        assert f(p=FAKE * 3 + 20) == 8             # prime inside max_exp's span
        assert f(rows=0, x=None, y=None, q=None, e=None, p=None) == 0
    # the pitched spans, not only the used bytes, take part in the overlap check
    assert pack(ld_e=1 << 20, p=FAKE * 3 + (1 << 20)) == 8


def test_mx9_axis_and_record_validation_codes():
    lib = mxq.library()

    def pack_axis(dtype=1, outer=3, length=40, inner=5, bs=16, x=FAKE, q=FAKE * 2, e=FAKE * 3, p=FAKE * 4):
        return lib.mx9_pack_axis(x, dtype, outer, length, inner, bs, q, e, p, None)

    def unpack_axis(od=1, outer=3, length=40, inner=5, bs=16, y=FAKE * 5, q=FAKE * 2, e=FAKE * 3, p=FAKE * 4):
        return lib.mx9_unpack_axis(q, e, p, outer, length, inner, bs, od, y, None)

    def pack_rec(dtype=0, outer=3, length=40, inner=5, bs=16, x=FAKE, pk=FAKE * 2, ld=54):
        return lib.mx9_pack_records(x, dtype, outer, length, inner, bs, pk, ld, None)

    def unpack_rec(od=0, outer=3, length=40, inner=5, bs=16, y=FAKE * 5, pk=FAKE * 2, ld=54):
        return lib.mx9_unpack_records(pk, ld, outer, length, inner, bs, od, y, None)
    # 3 * 5 rows of ceil(40 / 16) = 3 blocks
    assert pack_axis(x=None) == 1 and pack_axis(dtype=2) == 2 and pack_axis(bs=32) == 3
    assert pack_axis(inner=-1) == 5 and pack_axis(length=(1 << 30) + 1) == 5
    assert pack_axis(outer=1 << 20, inner=1 << 20, length=1 << 20) == 5
    # 2^24 blocks, but 2^23 tiles of one 512-thread workgroup each: the grid would need 2^32 threads
    assert pack_axis(outer=1 << 23, length=16, inner=2) == 5
    assert unpack_axis(outer=1 << 23, length=16, inner=2) == 5
    assert pack_rec(outer=1 << 23, length=16, inner=2, ld=18) == 5
    assert pack_axis(x=FAKE + 1) == 7 and pack_axis(q=FAKE * 2 + 8) == 7
    assert pack_axis(e=FAKE * 2 + 16) == 8                        # max_exp inside q
    assert pack_axis(outer=0, x=None, q=None, e=None, p=None) == 0
    assert unpack_axis(y=None) == 1 and unpack_axis(od=5) == 2 and unpack_axis(bs=8) == 3
    assert unpack_axis(y=FAKE * 5 + 1) == 7 and unpack_axis(q=FAKE * 2 + 4) == 7
    assert unpack_axis(y=FAKE * 3 - 8) == 8                       # y runs into max_exp
    assert pack_rec(pk=None) == 1 and pack_rec(dtype=7) == 2 and pack_rec(bs=15) == 3
    assert pack_rec(ld=53) == 6 and pack_rec(ld=1 << 41) == 6
    assert pack_rec(x=FAKE + 2) == 7
    assert pack_rec(pk=FAKE + 64) == 8                            # records inside the input
    assert pack_rec(length=0, x=None, pk=None) == 0
    assert pack_rec(outer=1 << 12, inner=1 << 11, length=16, ld=1 << 40) == 6
    assert unpack_rec(outer=1 << 12, inner=1 << 11, length=16, ld=1 << 40) == 6
    assert unpack_rec(pk=None) == 1 and unpack_rec(od=2) == 2 and unpack_rec(ld=10) == 6
    assert unpack_rec(y=FAKE * 5 + 2) == 7 and unpack_rec(y=FAKE * 2 + 100) == 8
    assert unpack_rec(inner=0, y=None, pk=None) == 0


def test_gemm_validation_codes():
    lib = mxq.library()

    def gemm(A=FAKE, lda=256, sA=FAKE * 2, rs=8, bs=1, B=FAKE * 3, ldb=256, sB=FAKE * 4, M=128, N=128, K=256,
             C=FAKE * 5, ldc=128, od=0):
        return lib.mx_gemm_nt(A, lda, sA, rs, bs, B, ldb, sB, 8, 1, M, N, K, C, ldc, od, None)
    assert gemm(A=None) == 1 and gemm(C=None) == 1 and gemm(od=2) == 2
    assert gemm(M=100) == 5 and gemm(K=96) == 5 and gemm(N=-128) == 5 and gemm(M=1 << 25) == 5
    assert gemm(lda=128) == 6 and gemm(lda=264) == 6 and gemm(ldc=64) == 6 and gemm(rs=-1) == 6
    assert gemm(A=FAKE + 8) == 7 and gemm(C=FAKE * 5 + 2) == 7
    assert gemm(C=FAKE + 1024) == 8                                  # C inside A
    assert gemm(sA=FAKE * 5 + 64) == 8                               # scales inside C
    assert gemm(M=0, A=None, sA=None, B=None, sB=None, C=None) == 0

    def rows(G=4, offs=FAKE * 6, bgs=1 << 16, **kw):
        a = dict(A=FAKE, sA=FAKE * 2, B=FAKE * 3, sB=FAKE * 4, C=FAKE * 5)
        a.update(kw)
        return lib.mx_grouped_gemm_rows(a["A"], 256, a["sA"], 8, 1, a["B"], 256, bgs, a["sB"], 8, 1, 1024, offs, G,
                                        128, 128, 256, a["C"], 128, 0, None)
    assert rows(G=0) == 5 and rows(offs=None) == 1 and rows(offs=FAKE * 6 + 2) == 7 and rows(bgs=-1) == 6
    assert rows(C=FAKE * 3 + 3 * (1 << 16)) == 8                     # C inside expert 3's operand

    def kgroups(G=4, cgs=128 * 128, **kw):
        a = dict(A=FAKE, sA=FAKE * 2, B=FAKE * 3, sB=FAKE * 4, C=FAKE * 5)
        a.update(kw)
        return lib.mx_grouped_gemm_k(a["A"], 256, a["sA"], 8, 1, a["B"], 256, a["sB"], 8, 1, FAKE * 6, G,
                                     128, 128, 256, a["C"], 128, cgs, 0, None)
    assert kgroups(G=0) == 5 and kgroups(cgs=128 * 127) == 6
    assert kgroups(C=FAKE * 6 - 4 * 128 * 128 * 2) == 8              # the last group's C runs into offs


def test_matrix_core_layout_validation_codes():
    """The _mfma entry points share the checks of their plain forms, with the
    scale buffers sized rows * K/32 and required 16-byte aligned."""
    lib = mxq.library()

    def dual(fn, **kw):
        a = dict(x=FAKE, M=256, N=256, ld=256, qr=FAKE * 2, sr=FAKE * 3, qc=FAKE * 4, sc=FAKE * 5)
        a.update(kw)
        return fn(a["x"], a["M"], a["N"], a["ld"], 32, 0, a["qr"], a["sr"], a["qc"], a["sc"], None)
    f = lib.mx_quantize_2d_dual_mfma
    assert dual(f, x=None) == 1 and dual(f, M=200) == 5 and dual(f, ld=128) == 6 and dual(f, sc=FAKE * 5 + 4) == 7
    assert dual(f, sr=FAKE * 2 + 4096) == 8 and dual(f, M=0, x=None, qr=None, sr=None, qc=None, sc=None) == 0
    g = lib.mx_quantize_grouped_mfma
    assert g(FAKE, 256, 256, 256, 32, 0, None, 2, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, None, None) == 1
    assert g(FAKE, 256, 256, 256, 32, 0, FAKE * 6, -1, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, None, None) == 5

    def gemm(A=FAKE, sA=FAKE * 2, B=FAKE * 3, sB=FAKE * 4, M=128, N=128, K=256, C=FAKE * 5, ldc=128):
        return lib.mx_gemm_nt_mfma(A, 256, sA, B, 256, sB, M, N, K, C, ldc, 0, None)
    assert gemm(sA=None) == 1 and gemm(K=96) == 5 and gemm(ldc=64) == 6
    assert gemm(sA=FAKE * 2 + 4) == 7 and gemm(sB=FAKE * 4 + 8) == 7
    assert gemm(sB=FAKE * 5 - 128 * 8 + 16) == 8                     # the last scale bytes run into C
    assert gemm(sB=FAKE * 5 - 128 * 8) != 8
    assert lib.mx_grouped_gemm_rows_mfma(FAKE, 256, FAKE * 2, FAKE * 3, 256, 1 << 16, FAKE * 4, 1024, None, 4,
                                         128, 128, 256, FAKE * 5, 128, 0, None) == 1
    assert lib.mx_grouped_gemm_k_mfma(FAKE, 256, FAKE * 2, FAKE * 3, 256, FAKE * 4, FAKE * 6, 4, 128, 128, 256,
                                      FAKE * 5, 128, 128 * 127, 0, None) == 6


def test_scale_conversion_validation_codes():
    lib = mxq.library()

    def to(s=FAKE, rs=16, bs=1, rows=128, blocks=16, out=FAKE * 2):
        return lib.mx_scales_to_mfma(s, rs, bs, rows, blocks, out, None)

    def frm(flat=FAKE * 2, rows=128, blocks=16, s=FAKE, rs=16, bs=1):
        return lib.mx_scales_from_mfma(flat, rows, blocks, s, rs, bs, None)
    assert to(s=None) == 1 and frm(flat=None) == 1
    assert to(rows=96) == 5 and to(blocks=6) == 5 and frm(rows=-64) == 5
    assert to(rs=-1) == 6 and frm(rs=0) == 6 and frm(rs=8) == 6          # a written view must not alias
    assert to(out=FAKE * 2 + 2) == 7
    assert to(out=FAKE + 1024) == 8 and frm(flat=FAKE + 64) == 8
    assert to(rows=0, s=None, out=None) == 0 and frm(blocks=0, s=None, flat=None) == 0


def test_binding_fails_loudly_without_the_library(monkeypatch):
    monkeypatch.setattr(mxq, "LIB_PATH", "/nonexistent/libmxq.so")
    monkeypatch.setattr(mxq, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        mxq.library()


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "mx9_dual_axis_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b|liboracle|mx_oracle|oref_", src, flags=re.M), f


def test_roof_helpers_validate_before_launch():
    """The benchmark's measurement helpers (libmxq_roof.so, not part of the
    C ABI) export their two calls and refuse bad arguments without launching."""
    lib = ctypes.CDLL(os.path.join(ROOT, "mx9_dual_axis_amd", "libmxq_roof.so"))
    lib.mxq_roof.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.mxq_roof_cast_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_void_p]
    assert lib.mxq_roof(0, FAKE, FAKE * 2, 4095, None) == -1          # not a multiple of 4 KiB
    assert lib.mxq_roof(0, FAKE + 8, FAKE * 2, 4096, None) == -1      # misaligned
    assert lib.mxq_roof(7, FAKE, FAKE * 2, 4096, None) == -1          # no such kind
    assert lib.mxq_roof_cast_stream(1, FAKE, None, 100, 128, None) == -1
    assert lib.mxq_roof_cast_stream(0, FAKE, None, 128, 128, None) == -1   # the read needs a sink
    assert lib.mxq_roof_cast_stream(3, FAKE, FAKE, 128, 128, None) == -1
