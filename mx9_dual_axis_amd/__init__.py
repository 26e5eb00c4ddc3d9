"""Single-pass MX quantization on AMD Instinct MI355X (gfx950).

Python binding over ``libmxq.so`` (C ABI in ``include/mxq.h``).  The binding
only marshals arguments: it allocates output tensors with torch, passes raw
device pointers, sizes and the current HIP stream, and raises on a nonzero
status.  Every step of the computation runs in the library's HIP kernels;
there is no fallback, and a missing library raises immediately.

Entry points (same names as the C ABI):
  mx_quantize_2d_dual(x)                 -> (q_row, s_row, q_col, s_col)
  mx_quantize_grouped(x, offs, err=None) -> (q_row, s_row, q_col, s_col)
  mx9_pack(x)                            -> (q, max_exp, prime)
  mx9_unpack(q, max_exp, prime, rows, cols, out_dtype) -> y
  mx9_pack_strided(x, out=(q, max_exp, prime)) / mx9_unpack_strided(q, max_exp, prime, rows, cols)
                                         (the three parts as pitched [rows, ...] views)
  mx9_pack_axis(x, axis) / mx9_unpack_axis(q, max_exp, prime, shape, axis)
  mx9_pack_records(x, axis) -> packed uint8 / mx9_unpack_records(packed, shape, axis)
  mx_gemm_nt(A, sA, B, sB)                -> C = A B^T (MXFP8 operands)
  mx_grouped_gemm_rows(A, sA, B, sB, offs) / mx_grouped_gemm_k(A, sA, B, sB, offs)
plus the signatures the pages use: ``mxfp8_quantize_2d_1x32_32x1`` (dense
when ``offs`` is None, grouped otherwise), ``convert_to_mx9`` and
``convert_from_mx9`` (with an axis), and their single-tensor forms
``convert_to_mx9_packed`` / ``convert_from_mx9_packed``.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxq.so")

MX_DTYPE_F32 = 0
MX_DTYPE_BF16 = 1
MX_SCALE_RCEIL = 0
OFFS_CODES = {0: "ok", 1: "offsets not ascending", 2: "offset not a multiple of 128",
              3: "offset outside [0, M]"}

_lib = None


class MXError(ValueError):
    """A nonzero mx_status returned by the library."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.mx_quantize_2d_dual.argtypes = [P, I64, I64, I64, I32, I32, P, P, P, P, P]
    lib.mx_quantize_grouped.argtypes = [P, I64, I64, I64, I32, I32, P, I32, P, P, P, P, P, P]
    lib.mx_quantize_2d_dual_mfma.argtypes = lib.mx_quantize_2d_dual.argtypes
    lib.mx_quantize_grouped_mfma.argtypes = lib.mx_quantize_grouped.argtypes
    lib.mx9_pack.argtypes = [P, I32, I64, I64, I64, I32, P, P, P, P]
    lib.mx9_unpack.argtypes = [P, P, P, I64, I64, I32, I32, P, I64, P]
    lib.mx9_pack_strided.argtypes = [P, I32, I64, I64, I64, I32, P, I64, P, I64, P, I64, P]
    lib.mx9_unpack_strided.argtypes = [P, I64, P, I64, P, I64, I64, I64, I32, I32, P, I64, P]
    lib.mx9_pack_axis.argtypes = [P, I32, I64, I64, I64, I32, P, P, P, P]
    lib.mx9_unpack_axis.argtypes = [P, P, P, I64, I64, I64, I32, I32, P, P]
    lib.mx9_pack_records.argtypes = [P, I32, I64, I64, I64, I32, P, I64, P]
    lib.mx9_unpack_records.argtypes = [P, I64, I64, I64, I64, I32, I32, P, P]
    lib.mx_gemm_nt.argtypes = [P, I64, P, I64, I64, P, I64, P, I64, I64, I64, I64, I64, P, I64, I32, P]
    lib.mx_grouped_gemm_rows.argtypes = [P, I64, P, I64, I64, P, I64, I64, P, I64, I64, I64, P, I32, I64, I64, I64,
                                         P, I64, I32, P]
    lib.mx_grouped_gemm_k.argtypes = [P, I64, P, I64, I64, P, I64, P, I64, I64, P, I32, I64, I64, I64, P, I64, I64,
                                      I32, P]
    lib.mx_gemm_nt_mfma.argtypes = [P, I64, P, P, I64, P, I64, I64, I64, P, I64, I32, P]
    lib.mx_scales_to_mfma.argtypes = [P, I64, I64, I64, I64, P, P]
    lib.mx_scales_from_mfma.argtypes = [P, I64, I64, P, I64, I64, P]
    lib.mx_grouped_gemm_rows_mfma.argtypes = [P, I64, P, P, I64, I64, P, I64, P, I32, I64, I64, I64, P, I64, I32, P]
    lib.mx_grouped_gemm_k_mfma.argtypes = [P, I64, P, P, I64, P, P, I32, I64, I64, I64, P, I64, I64, I32, P]
    for f in (lib.mx_quantize_2d_dual, lib.mx_quantize_grouped, lib.mx9_pack, lib.mx9_unpack,
              lib.mx9_pack_strided, lib.mx9_unpack_strided,
              lib.mx9_pack_axis, lib.mx9_unpack_axis, lib.mx9_pack_records, lib.mx9_unpack_records,
              lib.mx_gemm_nt, lib.mx_grouped_gemm_rows, lib.mx_grouped_gemm_k,
              lib.mx_quantize_2d_dual_mfma, lib.mx_quantize_grouped_mfma, lib.mx_gemm_nt_mfma,
              lib.mx_grouped_gemm_rows_mfma, lib.mx_grouped_gemm_k_mfma, lib.mx_scales_to_mfma,
              lib.mx_scales_from_mfma):
        f.restype = ctypes.c_int
    lib.mx_status_string.argtypes = [ctypes.c_int]
    lib.mx_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def library():
    """The loaded ctypes library (raises if it has not been built)."""
    return _load()


def status_string(status: int) -> str:
    return _load().mx_status_string(status).decode()


def _check(rc: int):
    if rc != 0:
        raise MXError(rc, status_string(rc))


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need_cuda(t: torch.Tensor, name: str, device: torch.device | None = None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call runs on {device}")


def _check_out(t, name: str, shape, dtypes, device: torch.device, contiguous: bool = True):
    """A caller-supplied output: a tensor on `device` (the device of the
    call's input) with one of `dtypes`, exactly `shape` and, unless told
    otherwise, contiguous.  Raises ValueError before anything is launched."""
    _need_cuda(t, name, device)
    dtypes = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")
    shapes = shape if isinstance(shape, list) else [shape]
    if tuple(t.shape) not in [tuple(int(d) for d in sh) for sh in shapes]:
        raise ValueError(f"{name} must have shape {' or '.join(str(tuple(sh)) for sh in shapes)}, not {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _out_tuple(out, k: int, what: str):
    if not isinstance(out, (tuple, list)) or len(out) != k:
        raise ValueError(f"out must be a sequence of {k} tensors ({what})")
    return tuple(out)


def _scaling(mode) -> int:
    if mode in ("rceil", MX_SCALE_RCEIL):
        return MX_SCALE_RCEIL
    return -1  # rejected by the library with MX_E_MODE


def _dual_outputs(x: torch.Tensor, out, mfma: bool):
    M, N = x.shape
    if mfma:   # flat buffers in the matrix-core scale layout
        shapes = ((M, N), (M * N // 32,), (N, M), (M * N // 32,))
    else:
        shapes = ((M, N), (M, N // 32), (N, M), (M // 32, N))
    if out is not None:
        out = _out_tuple(out, 4, "q_row, s_row, q_col, s_col")
        for t, name, sh in zip(out, ("q_row", "s_row", "q_col", "s_col"), shapes):
            _check_out(t, name, sh, (torch.uint8, torch.float8_e4m3fn) if name[0] == "q" else torch.uint8, x.device)
        return out
    return tuple(torch.empty(sh, dtype=torch.uint8, device=x.device) for sh in shapes)


def _layout(scale_layout) -> bool:
    if scale_layout not in ("plain", "mfma"):
        raise ValueError('scale_layout must be "plain" or "mfma"')
    return scale_layout == "mfma"


def _bf16_matrix(x: torch.Tensor):
    _need_cuda(x, "x")
    if x.dtype != torch.bfloat16:
        raise MXError(2, status_string(2))
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with contiguous rows")


def mx_quantize_2d_dual(x: torch.Tensor, block_size: int = 32, scaling_mode="rceil", out=None,
                        scale_layout: str = "plain"):
    """Fused dual-axis MXFP8 cast.  Returns uint8 tensors q_row [M,N] (E4M3),
    s_row [M,N/32] (E8M0), q_col [N,M] (E4M3, transposed), s_col [M/32,N].
    With scale_layout="mfma" s_row and s_col are flat [M*N/32] buffers in the
    matrix-core layout (s_row for the operand [M rows, N/32 blocks], s_col
    for [N rows, M/32 blocks]), ready for the *_mfma contractions."""
    _bf16_matrix(x)
    M, N = x.shape
    mfma = _layout(scale_layout)
    q_row, s_row, q_col, s_col = _dual_outputs(x, out, mfma)
    fn = _load().mx_quantize_2d_dual_mfma if mfma else _load().mx_quantize_2d_dual
    _check(fn(x.data_ptr(), M, N, x.stride(0), block_size, _scaling(scaling_mode), q_row.data_ptr(),
              s_row.data_ptr(), q_col.data_ptr(), s_col.data_ptr(), _stream(x.device)))
    return q_row, s_row, q_col, s_col


def mx_quantize_grouped(x: torch.Tensor, offs: torch.Tensor, block_size: int = 32, scaling_mode="rceil",
                        err: torch.Tensor | None = None, out=None, scale_layout: str = "plain"):
    """Grouped dual-axis cast: the dense outputs, with the colwise scale rows
    of the uncovered tail (rows >= offs[-1]) zeroed.  ``err`` (int32 device
    tensor of one element) receives the device-side offset check code.
    scale_layout as for mx_quantize_2d_dual."""
    _bf16_matrix(x)
    M, N = x.shape
    _need_cuda(offs, "offs", x.device)
    if offs.dtype != torch.int32 or offs.dim() != 1 or not offs.is_contiguous():
        raise ValueError("offs must be a contiguous 1-D int32 tensor")
    if err is not None:
        _need_cuda(err, "err", x.device)
        if err.dtype != torch.int32 or err.numel() != 1:
            raise ValueError("err must be a one-element int32 tensor")
    mfma = _layout(scale_layout)
    q_row, s_row, q_col, s_col = _dual_outputs(x, out, mfma)
    fn = _load().mx_quantize_grouped_mfma if mfma else _load().mx_quantize_grouped
    _check(fn(x.data_ptr(), M, N, x.stride(0), block_size, _scaling(scaling_mode),
              offs.data_ptr() if offs.numel() else None, offs.numel(), q_row.data_ptr(), s_row.data_ptr(),
              q_col.data_ptr(), s_col.data_ptr(), _ptr(err), _stream(x.device)))
    return q_row, s_row, q_col, s_col


def _mx9_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MX_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return MX_DTYPE_BF16
    return 2  # any other dtype: the library answers MX_E_DTYPE


def _mx9_outputs(out, nb: int, device: torch.device):
    """(q int8 [nb, 16], max_exp uint8 [nb], prime uint8 [nb, 1]): new, or the
    caller's checked tensors (prime may also be [nb])."""
    if out is None:
        return (torch.empty((nb, 16), dtype=torch.int8, device=device),
                torch.empty((nb,), dtype=torch.uint8, device=device),
                torch.empty((nb, 1), dtype=torch.uint8, device=device))
    q, e, p = _out_tuple(out, 3, "q, max_exp, prime")
    _check_out(q, "q", (nb, 16), torch.int8, device)
    _check_out(e, "max_exp", (nb,), torch.uint8, device)
    _check_out(p, "prime", [(nb, 1), (nb,)], torch.uint8, device)
    return q, e, p


def _mx9_inputs(q, max_exp, prime, nb: int):
    """The three parts of an MX9 tensor on one device, contiguous, of nb blocks."""
    _need_cuda(q, "q")
    for t, n in ((q, "q"), (max_exp, "max_exp"), (prime, "prime")):
        _need_cuda(t, n, q.device)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if q.dtype != torch.int8 or max_exp.dtype != torch.uint8 or prime.dtype != torch.uint8:
        raise ValueError("q must be int8, max_exp and prime uint8")
    if q.numel() != nb * 16 or max_exp.numel() != nb or prime.numel() != nb:
        raise ValueError(f"q / max_exp / prime must hold {nb} blocks ({nb * 16} / {nb} / {nb} elements)")


def mx9_pack(x: torch.Tensor, block_size: int = 16, out=None):
    """MX9 pack along the last axis.  Returns q int8 [nb,16], max_exp uint8
    [nb], prime uint8 [nb,1], nb = rows * ceil(cols/16).  x is fp32 or bf16,
    2-D with contiguous rows (a 1-D tensor is one row)."""
    _need_cuda(x, "x")
    if x.dim() == 1:
        x = x.unsqueeze(0)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with contiguous rows")
    rows, cols = x.shape
    nb = rows * ((cols + 15) // 16)
    q, e, p = _mx9_outputs(out, nb, x.device)
    _check(_load().mx9_pack(x.data_ptr(), _mx9_dtype(x), rows, cols, x.stride(0), block_size,
                            q.data_ptr(), e.data_ptr(), p.data_ptr(), _stream(x.device)))
    return q, e, p


def mx9_unpack(q: torch.Tensor, max_exp: torch.Tensor, prime: torch.Tensor, rows: int, cols: int,
               out_dtype=torch.float32, block_size: int = 16, out: torch.Tensor | None = None):
    """MX9 unpack to [rows, cols] of out_dtype (float32 or bfloat16).  `out`
    may be a wider [rows, >= cols] tensor with contiguous rows; only its
    first cols columns are written."""
    nb = rows * ((cols + 15) // 16)
    _mx9_inputs(q, max_exp, prime, nb)
    if out is not None:
        _need_cuda(out, "out", q.device)
        if out.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("out must be float32 or bfloat16")
        out_dtype = out.dtype
    od = {torch.float32: MX_DTYPE_F32, torch.bfloat16: MX_DTYPE_BF16}.get(out_dtype, 2)
    if out is None:
        y = torch.empty((rows, cols), dtype=out_dtype if od != 2 else torch.float32, device=q.device)
    else:
        y = out
        if y.dim() != 2 or y.stride(1) != 1 or y.shape[0] != rows or y.shape[1] < cols or y.stride(0) < cols:
            raise ValueError("out must be [rows, >= cols] with contiguous rows")
    _check(_load().mx9_unpack(q.data_ptr(), max_exp.data_ptr(), prime.data_ptr(), rows, cols,
                              block_size, od, y.data_ptr(), y.stride(0), _stream(q.device)))
    return y


def _pitched_part(t: torch.Tensor, name: str, rows: int, width: int, dtype, device):
    """Row pitch of a [rows, >= width] view with contiguous rows (a pitched MX9 part)."""
    _need_cuda(t, name, device)
    if t.dtype != dtype or t.dim() != 2 or t.shape[0] != rows or t.shape[1] < width or t.stride(1) != 1:
        raise ValueError(f"{name} must be {dtype} [{rows}, >= {width}] with contiguous rows")
    if rows > 1 and t.stride(0) < width:
        raise ValueError(f"{name} rows overlap (pitch {t.stride(0)} < {width})")
    return t.stride(0) if rows > 1 else width


def mx9_pack_strided(x: torch.Tensor, block_size: int = 16, out=None):
    """MX9 pack along the last axis into pitched parts: q int8 [rows, >= 16 *
    nbr], max_exp and prime uint8 [rows, >= nbr] (nbr = ceil(cols/16)), each
    with contiguous rows at its own pitch (e.g. column slices of wider
    tensors).  Only the first 16 * nbr / nbr bytes of each row are written.
    Returns (q, max_exp, prime)."""
    _need_cuda(x, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with contiguous rows")
    rows, cols = x.shape
    nbr = (cols + 15) // 16
    if out is None:
        out = (torch.empty((rows, 16 * nbr), dtype=torch.int8, device=x.device),
               torch.empty((rows, nbr), dtype=torch.uint8, device=x.device),
               torch.empty((rows, nbr), dtype=torch.uint8, device=x.device))
    q, e, p = _out_tuple(out, 3, "q, max_exp, prime")
    lq = _pitched_part(q, "q", rows, 16 * nbr, torch.int8, x.device)
    le = _pitched_part(e, "max_exp", rows, nbr, torch.uint8, x.device)
    lp = _pitched_part(p, "prime", rows, nbr, torch.uint8, x.device)
    _check(_load().mx9_pack_strided(x.data_ptr(), _mx9_dtype(x), rows, cols, x.stride(0), block_size,
                                    q.data_ptr(), lq, e.data_ptr(), le, p.data_ptr(), lp, _stream(x.device)))
    return q, e, p


def mx9_unpack_strided(q: torch.Tensor, max_exp: torch.Tensor, prime: torch.Tensor, rows: int, cols: int,
                       out_dtype=torch.float32, block_size: int = 16, out: torch.Tensor | None = None):
    """Inverse of mx9_pack_strided: reads the pitched parts, writes [rows,
    cols] of out_dtype (or the first cols columns of `out`)."""
    nbr = (cols + 15) // 16
    _need_cuda(q, "q")
    lq = _pitched_part(q, "q", rows, 16 * nbr, torch.int8, q.device)
    le = _pitched_part(max_exp, "max_exp", rows, nbr, torch.uint8, q.device)
    lp = _pitched_part(prime, "prime", rows, nbr, torch.uint8, q.device)
    if out is None:
        od = _out_code(out_dtype)
        y = torch.empty((rows, cols), dtype=out_dtype if od != 2 else torch.float32, device=q.device)
    else:
        y = out
        _need_cuda(y, "out", q.device)
        if y.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("out must be float32 or bfloat16")
        if y.dim() != 2 or y.stride(1) != 1 or y.shape[0] != rows or y.shape[1] < cols or (rows > 1 and y.stride(0) < cols):
            raise ValueError("out must be [rows, >= cols] with contiguous rows")
        od = _out_code(y.dtype)
    _check(_load().mx9_unpack_strided(q.data_ptr(), lq, max_exp.data_ptr(), le, prime.data_ptr(), lp, rows, cols,
                                      block_size, od, y.data_ptr(), y.stride(0) if rows > 1 else cols,
                                      _stream(q.device)))
    return y


def _axis_dims(shape, axis: int):
    """(outer, len, inner) of a contiguous array of `shape` blocked along `axis`."""
    shape = tuple(int(d) for d in shape)
    if not shape:
        raise ValueError("a 0-d tensor has no axis to block")
    axis = axis % len(shape)
    outer = 1
    for d in shape[:axis]:
        outer *= d
    inner = 1
    for d in shape[axis + 1:]:
        inner *= d
    return outer, shape[axis], inner


def _out_code(out_dtype) -> int:
    return {torch.float32: MX_DTYPE_F32, torch.bfloat16: MX_DTYPE_BF16}.get(out_dtype, 2)


def mx9_pack_axis(x: torch.Tensor, axis: int = -1, block_size: int = 16, out=None):
    """MX9 pack of a contiguous fp32/bf16 tensor in blocks of 16 along `axis`
    (the axis moved last before blocking).  Returns q int8 [nb,16], max_exp
    uint8 [nb], prime uint8 [nb,1] with blocks ordered (outer, inner, block)."""
    _need_cuda(x, "x")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    outer, length, inner = _axis_dims(x.shape, axis)
    nb = outer * inner * ((length + 15) // 16)
    q, e, p = _mx9_outputs(out, nb, x.device)
    _check(_load().mx9_pack_axis(x.data_ptr(), _mx9_dtype(x), outer, length, inner, block_size,
                                 q.data_ptr(), e.data_ptr(), p.data_ptr(), _stream(x.device)))
    return q, e, p


def mx9_unpack_axis(q: torch.Tensor, max_exp: torch.Tensor, prime: torch.Tensor, shape, axis: int = -1,
                    out_dtype=torch.float32, block_size: int = 16, out: torch.Tensor | None = None):
    """Inverse of mx9_pack_axis: a contiguous tensor of `shape` and out_dtype."""
    outer, length, inner = _axis_dims(shape, axis)
    nb = outer * inner * ((length + 15) // 16)
    _mx9_inputs(q, max_exp, prime, nb)
    if out is None:
        od = _out_code(out_dtype)
        y = torch.empty(tuple(shape), dtype=out_dtype if od != 2 else torch.float32, device=q.device)
    else:
        y = _check_out(out, "out", tuple(shape), (torch.float32, torch.bfloat16), q.device)
        od = _out_code(y.dtype)
    _check(_load().mx9_unpack_axis(q.data_ptr(), max_exp.data_ptr(), prime.data_ptr(), outer, length, inner,
                                   block_size, od, y.data_ptr(), _stream(q.device)))
    return y


def mx9_pack_records(x: torch.Tensor, axis: int = -1, block_size: int = 16, out: torch.Tensor | None = None):
    """MX9 in one byte tensor: uint8 [outer*inner, 18*nbl], one 18-byte record
    per block (exponent byte, q[16], prime byte).  `out` may be a wider uint8
    [outer*inner, >= 18*nbl] tensor with contiguous rows (its row pitch is
    passed to the library)."""
    _need_cuda(x, "x")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    outer, length, inner = _axis_dims(x.shape, axis)
    row = 18 * ((length + 15) // 16)
    if out is None:
        out = torch.empty((outer * inner, row), dtype=torch.uint8, device=x.device)
    else:
        _need_cuda(out, "out", x.device)
        if (out.dtype != torch.uint8 or out.dim() != 2 or out.stride(1) != 1 or out.shape[0] != outer * inner
                or out.shape[1] < row or (outer * inner > 1 and out.stride(0) < row)):
            raise ValueError("out must be uint8 [outer*inner, >= 18*nbl] with contiguous rows")
    _check(_load().mx9_pack_records(x.data_ptr(), _mx9_dtype(x), outer, length, inner, block_size,
                                    out.data_ptr(), out.stride(0), _stream(x.device)))
    return out


def mx9_unpack_records(packed: torch.Tensor, shape, axis: int = -1, out_dtype=torch.float32,
                       block_size: int = 16, out: torch.Tensor | None = None):
    """Inverse of mx9_pack_records: a contiguous tensor of `shape`."""
    _need_cuda(packed, "packed")
    outer, length, inner = _axis_dims(shape, axis)
    row = 18 * ((length + 15) // 16)
    if (packed.dtype != torch.uint8 or packed.dim() != 2 or packed.stride(1) != 1
            or packed.shape[0] != outer * inner or packed.shape[1] < row
            or (outer * inner > 1 and packed.stride(0) < row)):
        raise ValueError("packed must be uint8 [outer*inner, >= 18*nbl] with contiguous rows")
    if out is None:
        od = _out_code(out_dtype)
        y = torch.empty(tuple(shape), dtype=out_dtype if od != 2 else torch.float32, device=packed.device)
    else:
        y = _check_out(out, "out", tuple(shape), (torch.float32, torch.bfloat16), packed.device)
        od = _out_code(y.dtype)
    _check(_load().mx9_unpack_records(packed.data_ptr(), packed.stride(0), outer, length, inner, block_size, od,
                                      y.data_ptr(), _stream(packed.device)))
    return y


def _codes(t: torch.Tensor, name: str, device: torch.device | None = None):
    _need_cuda(t, name, device)
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn) or t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D E4M3 codes (uint8 or float8_e4m3fn) with contiguous rows")


def _scales(s: torch.Tensor, rows: int, k: int, name: str, device: torch.device | None = None):
    """(rs, bs) of a [rows, k/32] uint8 scale view with any strides."""
    _need_cuda(s, name, device)
    if s.dtype != torch.uint8 or s.dim() != 2 or tuple(s.shape) != (rows, k // 32):
        raise ValueError(f"{name} must be a uint8 [{rows}, {k // 32}] view (any strides)")
    return s.stride(0), s.stride(1)


def _gemm_out(out, shape, out_dtype, dev):
    if out is None:
        return torch.empty(shape, dtype=out_dtype, device=dev)
    _check_out(out, "out", tuple(shape), (torch.float32, torch.bfloat16), dev, contiguous=False)
    if out.stride(-1) != 1 or any(st < 0 for st in out.stride()):
        raise ValueError(f"out must be {tuple(shape)} with contiguous rows")
    if len(shape) == 3 and out.stride(0) < out.stride(1) * shape[1]:
        raise ValueError("the groups of out must not overlap (stride(0) >= stride(1) * M)")
    return out


def mx_gemm_nt(A: torch.Tensor, sA: torch.Tensor, B: torch.Tensor, sB: torch.Tensor, out_dtype=torch.float32,
               out: torch.Tensor | None = None):
    """C = A B^T with MXFP8 operands: A [M, K] and B [N, K] E4M3 codes
    (contraction contiguous), sA [M, K/32] and sB [N, K/32] E8M0 scale views
    (e.g. the cast's s_row, or s_col.t() for q_col operands).  C is float32
    or bfloat16 [M, N].  Both scale views in the s_row form (block stride 1)
    or both in the s_col.t() form (row stride 1), with C rows in 16-byte
    pieces, take the pipelined kernel; other views a slower general one."""
    _codes(A, "A")
    _codes(B, "B", A.device)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B must share the contraction extent")
    sa, sb = _scales(sA, M, K, "sA", A.device), _scales(sB, N, K, "sB", A.device)
    C = _gemm_out(out, (M, N), out_dtype, A.device)
    od = _out_code(C.dtype)
    _check(_load().mx_gemm_nt(A.data_ptr(), A.stride(0), sA.data_ptr(), sa[0], sa[1], B.data_ptr(), B.stride(0),
                              sB.data_ptr(), sb[0], sb[1], M, N, K, C.data_ptr(), C.stride(0), od,
                              _stream(A.device)))
    return C


def mx_grouped_gemm_rows(A: torch.Tensor, sA: torch.Tensor, B: torch.Tensor, sB: torch.Tensor, offs: torch.Tensor,
                         out_dtype=torch.float32, out: torch.Tensor | None = None):
    """Routed-expert forward: rows of group g (cumulative int32 offs) use
    expert g's B[g] ([E, N, K] codes) and sB[g] ([E, N, K/32] view); rows
    past offs[-1] give 0."""
    _codes(A, "A")
    M, K = A.shape
    if B.dim() != 3 or B.stride(2) != 1 or B.shape[2] != K:
        raise ValueError("B must be [E, N, K] codes with contiguous rows")
    E, N = B.shape[0], B.shape[1]
    if sB.dim() != 3 or tuple(sB.shape) != (E, N, K // 32) or sB.dtype != torch.uint8:
        raise ValueError("sB must be a uint8 [E, N, K/32] view")
    if offs.dtype != torch.int32 or offs.dim() != 1 or not offs.is_contiguous() or offs.numel() > E:
        raise ValueError("offs must be a contiguous int32 [G] tensor with G <= E")
    _need_cuda(offs, "offs", A.device)
    sa = _scales(sA, M, K, "sA", A.device)
    C = _gemm_out(out, (M, N), out_dtype, A.device)
    _check(_load().mx_grouped_gemm_rows(A.data_ptr(), A.stride(0), sA.data_ptr(), sa[0], sa[1], B.data_ptr(),
                                        B.stride(1), B.stride(0), sB.data_ptr(), sB.stride(1), sB.stride(2),
                                        sB.stride(0), offs.data_ptr(), offs.numel(), M, N, K, C.data_ptr(),
                                        C.stride(0), _out_code(C.dtype), _stream(A.device)))
    return C


def mx_grouped_gemm_k(A: torch.Tensor, sA: torch.Tensor, B: torch.Tensor, sB: torch.Tensor, offs: torch.Tensor,
                      out_dtype=torch.float32, out: torch.Tensor | None = None):
    """Routed-expert weight gradient: C[g] = A[:, r_g] B[:, r_g]^T over the
    contraction range r_g = [offs[g-1], offs[g]).  A [M, K], B [N, K] codes,
    sA [M, K/32], sB [N, K/32] views (the cast's s_col.t()).  Returns
    [G, M, N]."""
    _codes(A, "A")
    _codes(B, "B", A.device)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B must share the contraction extent")
    if offs.dtype != torch.int32 or offs.dim() != 1 or not offs.is_contiguous():
        raise ValueError("offs must be a contiguous int32 [G] tensor")
    _need_cuda(offs, "offs", A.device)
    G = offs.numel()
    sa, sb = _scales(sA, M, K, "sA", A.device), _scales(sB, N, K, "sB", A.device)
    C = _gemm_out(out, (G, M, N), out_dtype, A.device)
    _check(_load().mx_grouped_gemm_k(A.data_ptr(), A.stride(0), sA.data_ptr(), sa[0], sa[1], B.data_ptr(),
                                     B.stride(0), sB.data_ptr(), sb[0], sb[1], offs.data_ptr(), G, M, N, K,
                                     C.data_ptr(), C.stride(1), C.stride(0), _out_code(C.dtype), _stream(A.device)))
    return C


def _mfma_scales(s: torch.Tensor, nbytes: int, name: str, device: torch.device | None = None):
    _need_cuda(s, name, device)
    if s.dtype != torch.uint8 or not s.is_contiguous() or s.numel() != nbytes:
        raise ValueError(f"{name} must be a contiguous uint8 buffer of {nbytes} bytes (matrix-core layout)")


def mx_gemm_nt_mfma(A: torch.Tensor, sA: torch.Tensor, B: torch.Tensor, sB: torch.Tensor, out_dtype=torch.float32,
                    out: torch.Tensor | None = None):
    """mx_gemm_nt with sA, sB in the matrix-core scale layout (flat, M*K/32
    and N*K/32 bytes): the s_row / s_col of an "mfma" cast."""
    _codes(A, "A")
    _codes(B, "B", A.device)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B must share the contraction extent")
    _mfma_scales(sA, M * K // 32, "sA", A.device)
    _mfma_scales(sB, N * K // 32, "sB", A.device)
    C = _gemm_out(out, (M, N), out_dtype, A.device)
    _check(_load().mx_gemm_nt_mfma(A.data_ptr(), A.stride(0), sA.data_ptr(), B.data_ptr(), B.stride(0),
                                   sB.data_ptr(), M, N, K, C.data_ptr(), C.stride(0), _out_code(C.dtype),
                                   _stream(A.device)))
    return C


def mx_grouped_gemm_rows_mfma(A: torch.Tensor, sA: torch.Tensor, B: torch.Tensor, sB: torch.Tensor,
                              offs: torch.Tensor, out_dtype=torch.float32, out: torch.Tensor | None = None):
    """mx_grouped_gemm_rows with matrix-core scale layouts: sA flat
    [M*K/32], sB [E, N*K/32] (expert e's scales in row e)."""
    _codes(A, "A")
    M, K = A.shape
    if B.dim() != 3 or B.stride(2) != 1 or B.shape[2] != K:
        raise ValueError("B must be [E, N, K] codes with contiguous rows")
    E, N = B.shape[0], B.shape[1]
    _need_cuda(sB, "sB", A.device)
    if sB.dtype != torch.uint8 or sB.dim() != 2 or tuple(sB.shape) != (E, N * K // 32) or sB.stride(1) != 1:
        raise ValueError("sB must be a uint8 [E, N*K/32] tensor with contiguous rows")
    if offs.dtype != torch.int32 or offs.dim() != 1 or not offs.is_contiguous() or offs.numel() > E:
        raise ValueError("offs must be a contiguous int32 [G] tensor with G <= E")
    _need_cuda(offs, "offs", A.device)
    _mfma_scales(sA, M * K // 32, "sA", A.device)
    C = _gemm_out(out, (M, N), out_dtype, A.device)
    _check(_load().mx_grouped_gemm_rows_mfma(A.data_ptr(), A.stride(0), sA.data_ptr(), B.data_ptr(), B.stride(1),
                                             B.stride(0), sB.data_ptr(), sB.stride(0), offs.data_ptr(),
                                             offs.numel(), M, N, K, C.data_ptr(), C.stride(0), _out_code(C.dtype),
                                             _stream(A.device)))
    return C


def mx_grouped_gemm_k_mfma(A: torch.Tensor, sA: torch.Tensor, B: torch.Tensor, sB: torch.Tensor,
                           offs: torch.Tensor, out_dtype=torch.float32, out: torch.Tensor | None = None):
    """mx_grouped_gemm_k with sA [M*K/32], sB [N*K/32] in the matrix-core
    scale layout (the s_col of an "mfma" cast of each token-major operand)."""
    _codes(A, "A")
    _codes(B, "B", A.device)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B must share the contraction extent")
    if offs.dtype != torch.int32 or offs.dim() != 1 or not offs.is_contiguous():
        raise ValueError("offs must be a contiguous int32 [G] tensor")
    _need_cuda(offs, "offs", A.device)
    _mfma_scales(sA, M * K // 32, "sA", A.device)
    _mfma_scales(sB, N * K // 32, "sB", A.device)
    G = offs.numel()
    C = _gemm_out(out, (G, M, N), out_dtype, A.device)
    _check(_load().mx_grouped_gemm_k_mfma(A.data_ptr(), A.stride(0), sA.data_ptr(), B.data_ptr(), B.stride(0),
                                          sB.data_ptr(), offs.data_ptr(), G, M, N, K, C.data_ptr(), C.stride(1),
                                          C.stride(0), _out_code(C.dtype), _stream(A.device)))
    return C


def scales_to_mfma(s: torch.Tensor, out: torch.Tensor | None = None):
    """Plain E8M0 scales s [rows, blocks] (any strides, uint8) -> a flat
    uint8 [rows * blocks] buffer in the matrix-core scale layout."""
    _need_cuda(s, "s")
    if s.dtype != torch.uint8 or s.dim() != 2:
        raise ValueError("s must be a 2-D uint8 view")
    rows, blocks = s.shape
    if out is None:
        out = torch.empty((rows * blocks,), dtype=torch.uint8, device=s.device)
    else:
        _check_out(out, "out", (rows * blocks,), torch.uint8, s.device)
    _check(_load().mx_scales_to_mfma(s.data_ptr(), s.stride(0), s.stride(1), rows, blocks, out.data_ptr(),
                                     _stream(s.device)))
    return out


def scales_from_mfma(flat: torch.Tensor, rows: int, blocks: int, out: torch.Tensor | None = None):
    """Inverse of scales_to_mfma: a flat matrix-core buffer -> plain
    [rows, blocks] (out may be any non-aliasing strided view)."""
    _need_cuda(flat, "flat")
    if flat.dtype != torch.uint8 or not flat.is_contiguous() or flat.numel() != rows * blocks:
        raise ValueError("flat must be a contiguous uint8 buffer of rows * blocks bytes")
    if out is None:
        out = torch.empty((rows, blocks), dtype=torch.uint8, device=flat.device)
    else:
        _check_out(out, "out", (rows, blocks), torch.uint8, flat.device, contiguous=False)
    _check(_load().mx_scales_from_mfma(flat.data_ptr(), rows, blocks, out.data_ptr(), out.stride(0), out.stride(1),
                                       _stream(flat.device)))
    return out


# --- the pages' call signatures ------------------------------------------

def mxfp8_quantize_2d_1x32_32x1(x: torch.Tensor, block_size: int = 32, scaling_mode="rceil",
                                offs: torch.Tensor | None = None):
    """Dense cast when offs is None, grouped cast otherwise."""
    if offs is None:
        return mx_quantize_2d_dual(x, block_size, scaling_mode)
    return mx_quantize_grouped(x, offs, block_size, scaling_mode)


def convert_to_mx9(x: torch.Tensor, block_size: int = 16, axis: int = -1):
    """Three-part MX9 (q, max_exp, prime) in blocks along `axis`."""
    if axis % x.dim() == x.dim() - 1:
        return mx9_pack(x.reshape(-1, x.shape[-1]), block_size)
    return mx9_pack_axis(x, axis, block_size)


def convert_from_mx9(q, max_exp, prime, out_dtype, shape, block_size: int = 16, axis: int = -1):
    """Inverse of convert_to_mx9; the shape and axis are not stored."""
    shape = tuple(shape)
    if axis % len(shape) == len(shape) - 1:
        cols = shape[-1]
        rows = 1
        for s in shape[:-1]:
            rows *= s
        return mx9_unpack(q, max_exp, prime, rows, cols, out_dtype, block_size).reshape(shape)
    return mx9_unpack_axis(q, max_exp, prime, shape, axis, out_dtype, block_size)


def convert_to_mx9_packed(x: torch.Tensor, block_size: int = 16, axis: int = -1):
    """MX9 in one uint8 tensor of 18-byte records (exponent byte first)."""
    return mx9_pack_records(x, axis, block_size)


def convert_from_mx9_packed(packed, out_dtype, shape, block_size: int = 16, axis: int = -1):
    """Inverse of convert_to_mx9_packed; the shape and axis are not stored."""
    return mx9_unpack_records(packed, shape, axis, out_dtype, block_size)
