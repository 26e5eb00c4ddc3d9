"""CPU oracle for single-pass MX quantization (bindings to ``liboracle.so``).

TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library never
imports it and shares no code with it.

The arithmetic lives in ``mx_oracle.c`` (plain C, binary64, nearest-value
search for every rounding).  This module only marshals numpy arrays and, when
asked, splits the rows of a matrix across threads; blocks never straddle a
split, so the result does not depend on the thread count.

Sources (web pages):
  * pytorch/ao PR #4995 "[moe_training] Fused dual-axis MXFP8 quantization
    with correct metadata" -- the dual-axis cast, its special values and the
    uncovered-tail rule (PR description).
  * AMD-AGI/ALTO PR #33 "feat: mx9: add fused MX9 quantization kernel with
    pack/unpack" -- the MX9 storage format (Summary, Key design choices).
  * AMD-AGI/ALTO PR #31 "Add MXFP8 grouped GEMM (E4M3) for routed-expert MoE
    training" -- the contraction that consumes the MXFP8 outputs (description:
    E4M3 operands with block-32 E8M0 scales, 1-D cumulative offsets).

The matrix-core scale layout (``mfma_scale_index``) is this project's own;
no page fixes it.  It is pinned by hand-worked positions, its bijectivity,
and the matrix instruction that consumes it: contractions whose scales
differ in every row and 32-block, with one product per block, must equal
this oracle's plain-scale result bit for bit when their scales go through
``scales_to_mfma`` (the GPU tests of the contraction).  The readings the
pages leave open are listed, with their pins, in ``mx_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SOURCES = [os.path.join(_HERE, "mx_oracle.c")]

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"oracle library missing: {LIB_PATH} (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    lib.oref_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oref_e4m3_value.restype = ctypes.c_double
    lib.oref_e4m3_encode.argtypes = [ctypes.c_double]
    lib.oref_e4m3_encode.restype = ctypes.c_uint8
    lib.oref_rceil_byte.argtypes = [ctypes.c_double]
    lib.oref_rceil_byte.restype = ctypes.c_int
    for name in ("oref_mxfp8_rowwise", "oref_mxfp8_colwise"):
        f = getattr(lib, name)
        f.argtypes = [_P, _I64, _I64, _I64, _P, _P]
        f.restype = None
    lib.oref_mxfp8_dual.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P, _P]
    lib.oref_mxfp8_dual.restype = None
    lib.oref_offs_check.argtypes = [_P, _I32, _I64]
    lib.oref_offs_check.restype = ctypes.c_int
    lib.oref_mxfp8_grouped.argtypes = [_P, _I64, _I64, _I64, _P, _I32, _P, _P, _P, _P]
    lib.oref_mxfp8_grouped.restype = ctypes.c_int
    lib.oref_mx9_pack.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, _P]
    lib.oref_mx9_pack.restype = None
    lib.oref_mx9_unpack.argtypes = [_P, _P, _P, _I64, _I64, ctypes.c_int, _P, _I64]
    lib.oref_mx9_unpack.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _splits(n: int, parts: int):
    parts = max(1, min(parts, n))
    edges = [n * k // parts for k in range(parts + 1)]
    return [(edges[k], edges[k + 1]) for k in range(parts) if edges[k + 1] > edges[k]]


def _run(jobs, threads: int):
    if threads <= 1 or len(jobs) <= 1:
        for j in jobs:
            j()
        return
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for f in [ex.submit(j) for j in jobs]:
            f.result()


# --------------------------------------------------------------------------
# scalar helpers (format definitions)
# --------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    """Exact value of an OCP E4M3FN code (NaN for 0x7F / 0xFF)."""
    return _load().oref_e4m3_value(code)


def e4m3_encode(v: float) -> int:
    """E4M3FN code nearest to v, ties to even, saturating at +-448."""
    return _load().oref_e4m3_encode(float(v))


def rceil_byte(amax: float) -> int:
    """RCEIL E8M0 scale byte for a finite block maximum."""
    return _load().oref_rceil_byte(float(amax))


# --------------------------------------------------------------------------
# MXFP8 dual-axis
# --------------------------------------------------------------------------

def _as_bf16_bits(x: np.ndarray) -> np.ndarray:
    if x.dtype != np.uint16 or x.ndim != 2:
        raise TypeError("expected a 2-D uint16 array of bf16 bit patterns")
    if x.strides[1] != 2:
        raise ValueError("rows must be contiguous")
    return x


def mxfp8_rowwise(x: np.ndarray, threads: int = 1):
    """Rowwise 1x32 cast.  Returns (q_row [M,N] uint8, s_row [M,N/32] uint8)."""
    x = _as_bf16_bits(x)
    M, N = x.shape
    assert N % 32 == 0
    ld = x.strides[0] // 2
    q = np.empty((M, N), np.uint8)
    s = np.empty((M, N // 32), np.uint8)
    lib = _load()

    def job(r0, r1):
        return lambda: lib.oref_mxfp8_rowwise(_ptr(x) + r0 * ld * 2, r1 - r0, N, ld,
                                              _ptr(q) + r0 * N, _ptr(s) + r0 * (N // 32))
    _run([job(a, b) for a, b in _splits(M, threads)], threads)
    return q, s


def mxfp8_colwise(x: np.ndarray, threads: int = 1):
    """Colwise 32x1 cast.  Returns (q_col [N,M] uint8, s_col [M/32,N] uint8)."""
    x = _as_bf16_bits(x)
    M, N = x.shape
    assert M % 32 == 0
    ld = x.strides[0] // 2
    q = np.empty((N, M), np.uint8)
    s = np.empty((M // 32, N), np.uint8)
    lib = _load()
    slabs = [(32 * a, 32 * b) for a, b in _splits(M // 32, threads)]

    def job(r0, r1):
        def run():
            qt = np.empty((N, r1 - r0), np.uint8)
            lib.oref_mxfp8_colwise(_ptr(x) + r0 * ld * 2, r1 - r0, N, ld,
                                   _ptr(qt), _ptr(s) + (r0 // 32) * N)
            q[:, r0:r1] = qt
        return run
    _run([job(a, b) for a, b in slabs], threads)
    return q, s


def mxfp8_dual(x: np.ndarray, threads: int = 1):
    """Fused dual-axis cast: (q_row, s_row, q_col, s_col)."""
    q_row, s_row = mxfp8_rowwise(x, threads)
    q_col, s_col = mxfp8_colwise(x, threads)
    return q_row, s_row, q_col, s_col


def offs_check(offs: np.ndarray, M: int) -> int:
    offs = np.ascontiguousarray(offs, dtype=np.int32)
    return _load().oref_offs_check(_ptr(offs), len(offs), M)


def mxfp8_grouped(x: np.ndarray, offs, threads: int = 1):
    """Grouped cast.  Returns (code, outputs); outputs is None when the
    offsets are invalid (code 1 order, 2 alignment, 3 bounds)."""
    x = _as_bf16_bits(x)
    M, N = x.shape
    offs = np.ascontiguousarray(offs, dtype=np.int32)
    rc = offs_check(offs, M)
    if rc != 0:
        return rc, None
    ld = x.strides[0] // 2
    q_row = np.empty((M, N), np.uint8)
    s_row = np.empty((M, N // 32), np.uint8)
    q_col = np.empty((N, M), np.uint8)
    s_col = np.empty((M // 32, N), np.uint8)
    lib = _load()
    if threads <= 1:
        rc = lib.oref_mxfp8_grouped(_ptr(x), M, N, ld, _ptr(offs), len(offs),
                                    _ptr(q_row), _ptr(s_row), _ptr(q_col), _ptr(s_col))
        return rc, (q_row, s_row, q_col, s_col)
    # Threaded: every slab of rows [r0, r1) goes through the C grouped call on
    # its own, with the group ends expressed relative to r0 and clipped to the
    # slab.  Slabs start at multiples of 128, so the rebased ends stay valid
    # multiples of 128, and a slab's uncovered rows are exactly the matrix's
    # uncovered rows that fall in it; the tail rule itself is the C oracle's.
    units = M // 128
    slabs = [(128 * a, 128 * b) for a, b in _splits(units, threads)] if units else []
    if slabs:
        slabs[-1] = (slabs[-1][0], M)
    elif M:
        slabs = [(0, M)]
    codes = []

    def job(r0, r1):
        def run():
            local = np.clip(offs.astype(np.int64) - r0, 0, r1 - r0).astype(np.int32)
            qt = np.empty((N, r1 - r0), np.uint8)
            codes.append(lib.oref_mxfp8_grouped(_ptr(x) + r0 * ld * 2, r1 - r0, N, ld, _ptr(local), len(local),
                                                _ptr(q_row) + r0 * N, _ptr(s_row) + r0 * (N // 32), _ptr(qt),
                                                _ptr(s_col) + (r0 // 32) * N))
            q_col[:, r0:r1] = qt
        return run
    _run([job(a, b) for a, b in slabs], threads)
    if any(codes):
        raise AssertionError(f"oracle: a rebased slab of valid offsets was rejected ({codes})")
    return 0, (q_row, s_row, q_col, s_col)


# --------------------------------------------------------------------------
# MX9
# --------------------------------------------------------------------------

def mx9_pack(x: np.ndarray, threads: int = 1):
    """Pack fp32 (given as float32 or uint32 bits) or bf16 (uint16 bits)
    [rows, cols] along the last axis.  Returns (q [nb,16] int8,
    max_exp [nb] uint8, prime [nb,1] uint8)."""
    if x.ndim != 2 or x.strides[1] != x.itemsize:
        raise ValueError("expected a 2-D array with contiguous rows")
    if x.dtype in (np.float32, np.uint32):
        dtype = 0
    elif x.dtype == np.uint16:
        dtype = 1
    else:
        raise TypeError("fp32 (float32/uint32) or bf16 (uint16 bits) only")
    rows, cols = x.shape
    ld = x.strides[0] // x.itemsize
    nbr = (cols + 15) // 16
    nb = rows * nbr
    q = np.empty((nb, 16), np.int8)
    e = np.empty(nb, np.uint8)
    p = np.empty((nb, 1), np.uint8)
    lib = _load()

    def job(r0, r1):
        return lambda: lib.oref_mx9_pack(_ptr(x) + r0 * ld * x.itemsize, dtype, r1 - r0, cols, ld,
                                         _ptr(q) + r0 * nbr * 16, _ptr(e) + r0 * nbr,
                                         _ptr(p) + r0 * nbr)
    _run([job(a, b) for a, b in _splits(rows, threads)], threads)
    return q, e, p


def mx9_unpack(q: np.ndarray, max_exp: np.ndarray, prime: np.ndarray, rows: int, cols: int,
               out_dtype: str = "fp32", threads: int = 1) -> np.ndarray:
    """Unpack to [rows, cols]: float32 for "fp32", uint16 bf16 bits for "bf16"."""
    nbr = (cols + 15) // 16
    nb = rows * nbr
    q = np.ascontiguousarray(q, dtype=np.int8).reshape(nb, 16)
    max_exp = np.ascontiguousarray(max_exp, dtype=np.uint8).reshape(nb)
    prime = np.ascontiguousarray(prime, dtype=np.uint8).reshape(nb)
    if out_dtype == "fp32":
        y = np.empty((rows, cols), np.float32)
        od = 0
    elif out_dtype == "bf16":
        y = np.empty((rows, cols), np.uint16)
        od = 1
    else:
        raise ValueError("out_dtype must be 'fp32' or 'bf16'")
    lib = _load()

    def job(r0, r1):
        return lambda: lib.oref_mx9_unpack(_ptr(q) + r0 * nbr * 16, _ptr(max_exp) + r0 * nbr,
                                           _ptr(prime) + r0 * nbr, r1 - r0, cols, od,
                                           _ptr(y) + r0 * cols * y.itemsize, cols)
    _run([job(a, b) for a, b in _splits(rows, threads)], threads)
    return y


def _mx9_code(x: np.ndarray) -> int:
    if x.dtype in (np.float32, np.uint32):
        return 0
    if x.dtype == np.uint16:
        return 1
    raise TypeError("fp32 (float32/uint32) or bf16 (uint16 bits) only")


def _axis_view(shape, axis: int):
    shape = tuple(int(s) for s in shape)
    axis = axis % len(shape)
    outer = int(np.prod(shape[:axis], dtype=np.int64))
    inner = int(np.prod(shape[axis + 1:], dtype=np.int64))
    return outer, shape[axis], inner


def mx9_pack_axis(x: np.ndarray, axis: int = -1, threads: int = 1):
    """Pack a contiguous array in blocks of 16 along `axis` (reading: the axis
    is moved last before blocking).  Returns (q [nb,16], max_exp [nb],
    prime [nb,1]) in the order of the moved array's rows."""
    x = np.ascontiguousarray(x)
    dtype = _mx9_code(x)
    outer, length, inner = _axis_view(x.shape, axis)
    nbl = (length + 15) // 16
    nb = outer * inner * nbl
    q = np.empty((nb, 16), np.int8)
    e = np.empty(nb, np.uint8)
    p = np.empty((nb, 1), np.uint8)
    lib = _load()
    f = lib.oref_mx9_pack_axis
    f.argtypes = [_P, _I32, _I64, _I64, _I64, _I64, _I64, _P, _P, _P]
    f.restype = None

    def job(i0, i1):
        return lambda: f(_ptr(x), dtype, outer, length, inner, i0, i1, _ptr(q), _ptr(e), _ptr(p))
    _run([job(a, b) for a, b in _splits(inner, threads)], threads)
    return q, e, p


def mx9_unpack_axis(q: np.ndarray, max_exp: np.ndarray, prime: np.ndarray, shape, axis: int = -1,
                    out_dtype: str = "fp32", threads: int = 1) -> np.ndarray:
    """Inverse of mx9_pack_axis: an array of `shape`, float32 for "fp32" or
    uint16 bf16 bits for "bf16"."""
    outer, length, inner = _axis_view(shape, axis)
    nb = outer * inner * ((length + 15) // 16)
    q = np.ascontiguousarray(q, dtype=np.int8).reshape(nb, 16)
    max_exp = np.ascontiguousarray(max_exp, dtype=np.uint8).reshape(nb)
    prime = np.ascontiguousarray(prime, dtype=np.uint8).reshape(nb)
    od, ty = {"fp32": (0, np.float32), "bf16": (1, np.uint16)}[out_dtype]
    y = np.empty(tuple(shape), ty)
    lib = _load()
    f = lib.oref_mx9_unpack_axis
    f.argtypes = [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I32, _P]
    f.restype = None

    def job(i0, i1):
        return lambda: f(_ptr(q), _ptr(max_exp), _ptr(prime), outer, length, inner, i0, i1, od, _ptr(y))
    _run([job(a, b) for a, b in _splits(inner, threads)], threads)
    return y


def mx9_to_records(q: np.ndarray, max_exp: np.ndarray, prime: np.ndarray, rows: int, bpr: int) -> np.ndarray:
    """The single-byte-tensor form: uint8 [rows, 18 * bpr], one 18-byte record
    per block (exponent byte, q[16], prime)."""
    nb = rows * bpr
    q = np.ascontiguousarray(q, dtype=np.int8).reshape(nb, 16)
    max_exp = np.ascontiguousarray(max_exp, dtype=np.uint8).reshape(nb)
    prime = np.ascontiguousarray(prime, dtype=np.uint8).reshape(nb)
    out = np.empty((rows, 18 * bpr), np.uint8)
    f = _load().oref_mx9_to_records
    f.argtypes = [_P, _P, _P, _I64, _I64, _P, _I64]
    f.restype = None
    f(_ptr(q), _ptr(max_exp), _ptr(prime), rows, bpr, _ptr(out), 18 * bpr)
    return out


def mx9_from_records(packed: np.ndarray, rows: int, bpr: int):
    """Split [rows, >= 18 * bpr] records back into (q, max_exp, prime)."""
    packed = np.asarray(packed, dtype=np.uint8)
    if packed.ndim != 2 or packed.strides[1] != 1 or packed.shape[0] != rows or packed.shape[1] < 18 * bpr:
        raise ValueError("expected uint8 [rows, >= 18 * bpr] with contiguous rows")
    nb = rows * bpr
    q = np.empty((nb, 16), np.int8)
    e = np.empty(nb, np.uint8)
    p = np.empty((nb, 1), np.uint8)
    f = _load().oref_mx9_from_records
    f.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P]
    f.restype = None
    f(_ptr(packed), packed.strides[0], rows, bpr, _ptr(q), _ptr(e), _ptr(p))
    return q, e, p


# ---------------------------------------------------------------------------
# MXFP8 block-scaled contraction (ALTO PR #31, the grouped GEMM's arithmetic)
# ---------------------------------------------------------------------------

def _scale_view(s, rs: int, bs: int):
    s = np.ascontiguousarray(s, dtype=np.uint8)
    return s, int(rs), int(bs)


def mx_gemm_nt(A, sA, B, sB, *, sa_strides, sb_strides, k0: int = 0, k1: int | None = None,
               rows=None, threads: int = 1, with_abs: bool = False):
    """C[m][n] = sum_k dec(A[m,k]) 2^(sA(m,k/32)-127) dec(B[n,k]) 2^(sB(n,k/32)-127)
    over k in [k0, k1), in binary64.  A: uint8 E4M3 codes [M, >=k1] (contraction
    contiguous), B: [N, >=k1]; sA(m, b) = sA.flat[m * rs + b * bs] with
    (rs, bs) = sa_strides, likewise sB.  ``rows``: optional (m0, m1) range; the
    result has M rows either way (rows outside the range are 0).  Returns C
    (float64 [M, N]) and, with ``with_abs``, the sum of |products| per entry."""
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    M, N = A.shape[0], B.shape[0]
    k1 = A.shape[1] if k1 is None else int(k1)
    if k0 % 32 or k1 % 32:
        raise ValueError("k0 and k1 must be multiples of 32")
    sA, sa_rs, sa_bs = _scale_view(sA, *sa_strides)
    sB, sb_rs, sb_bs = _scale_view(sB, *sb_strides)
    C = np.zeros((M, N), np.float64)
    absC = np.zeros((M, N), np.float64) if with_abs else None
    m0, m1 = (0, M) if rows is None else rows
    f = _load().oref_mx_gemm_nt
    f.argtypes = [_P, _I64, _P, _I64, _I64, _P, _I64, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I64, _P, _P, _I64]
    f.restype = None

    def job(r0, r1):
        return lambda: f(_ptr(A), A.shape[1], _ptr(sA), sa_rs, sa_bs, _ptr(B), B.shape[1], _ptr(sB), sb_rs, sb_bs,
                         m0 + r0, m0 + r1, N, k0, k1, _ptr(C), _ptr(absC) if absC is not None else None, N)
    _run([job(a, b) for a, b in _splits(m1 - m0, threads)], threads)
    return (C, absC) if with_abs else C


def mx_grouped_gemm_rows(A, sA, B, sB, offs, *, sa_strides, sb_strides, threads: int = 1, with_abs: bool = False):
    """Grouped contraction over row groups (the forward of a routed-expert
    layer): rows offs[g-1] <= m < offs[g] of A multiply expert g's operand
    B[g] ([E, N, K] codes, sB[g] its scales); rows from offs[-1] on (the
    uncovered tail) give 0 (reading: the pages pad the activation buffer and
    give the padding no expert)."""
    A = np.asarray(A)
    M, N = A.shape[0], B.shape[1]
    C = np.zeros((M, N), np.float64)
    absC = np.zeros((M, N), np.float64)
    lo = 0
    for g, hi in enumerate(np.asarray(offs, dtype=np.int64)):
        if hi > lo:
            c, a = mx_gemm_nt(A, sA, B[g], sB[g], sa_strides=sa_strides, sb_strides=sb_strides,
                              rows=(int(lo), int(hi)), threads=threads, with_abs=True)
            C[lo:hi] = c[lo:hi]
            absC[lo:hi] = a[lo:hi]
        lo = hi
    return (C, absC) if with_abs else C


def mx_grouped_gemm_k(A, sA, B, sB, offs, *, sa_strides, sb_strides, threads: int = 1, with_abs: bool = False):
    """Grouped contraction over contraction-index groups (the weight
    gradient of a routed-expert layer): C[g] = sum over offs[g-1] <= k <
    offs[g] of A[:, k] B[:, k] with their block scales; an empty group gives
    0.  Returns float64 [G, M, N]."""
    offs = np.asarray(offs, dtype=np.int64)
    M, N = np.asarray(A).shape[0], np.asarray(B).shape[0]
    C = np.zeros((len(offs), M, N), np.float64)
    absC = np.zeros_like(C)
    lo = 0
    for g, hi in enumerate(offs):
        if hi > lo:
            C[g], absC[g] = mx_gemm_nt(A, sA, B, sB, sa_strides=sa_strides, sb_strides=sb_strides,
                                       k0=int(lo), k1=int(hi), threads=threads, with_abs=True)
        lo = hi
    return (C, absC) if with_abs else C


# ---------------------------------------------------------------------------
# Matrix-core scale layout (this project's layout for the MXFP8 contraction's
# consumer; the pages ask for scales in the consumer's own layout so that no
# rearrangement runs between the cast and the GEMM)
# ---------------------------------------------------------------------------

def mfma_scale_index(r, b, kb: int):
    """Byte position of scale S[r][b] (row r of the operand, 32-wide block b of
    its contraction, kb blocks per row) in the matrix-core layout: for each
    64-row group and each 4-block (128-wide) step, 64 dwords, one per lane L of
    the 16x16x128 instruction, lane L = 16 (b % 4) + r % 16 holding in byte
    (r % 64) // 16 the scale of its sub-tile (r // 16) % 4."""
    r = np.asarray(r, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    return ((((r // 64) * (kb // 4) + b // 4) * 64 + (b % 4) * 16 + r % 16) * 4 + (r % 64) // 16)


def scales_to_mfma(S):
    """Plain scales S [R, kb] (R a multiple of 64, kb of 4) -> the same bytes
    in the matrix-core layout, as a flat uint8 array of R * kb bytes."""
    S = np.asarray(S, dtype=np.uint8)
    R, kb = S.shape
    if R % 64 or kb % 4:
        raise ValueError("rows must be a multiple of 64 and blocks a multiple of 4")
    out = np.empty(R * kb, np.uint8)
    r, b = np.meshgrid(np.arange(R), np.arange(kb), indexing="ij")
    out[mfma_scale_index(r, b, kb)] = S
    return out


def scales_from_mfma(flat, R: int, kb: int):
    """Inverse of scales_to_mfma."""
    flat = np.asarray(flat, dtype=np.uint8).reshape(-1)
    r, b = np.meshgrid(np.arange(R), np.arange(kb), indexing="ij")
    return flat[mfma_scale_index(r, b, kb)]
