"""GPU parity over seeded random shapes, pitches, group offsets and value
mixtures: the dual-axis cast (plain and matrix-core scale layouts, dense and
grouped), MX9 (three-part form, records, any axis) and the scale layout
conversions, each compared byte for byte with the CPU oracle.  The cases are
drawn from a fixed seed, so every run checks the same set.  Operations:
pytorch/ao PR #4995 (the fused dual-axis cast) and AMD-AGI/ALTO PR #33 (MX9)."""
import numpy as np
import pytest
import torch

import mx9_dual_axis_amd as mxq
import oracle
from helpers import bf16_to_dev, host, require_gpu, say
from mx9_dual_axis_amd import synth

pytestmark = pytest.mark.gpu
THREADS = 16
DEV = "cuda:0"
NAMES = ("q_row", "s_row", "q_col", "s_col")


def _values(g, M, N):
    """bf16 bits: a mixture picked per case (normal, mixed magnitudes, every
    special kind), with random exact zeros and a few subnormal elements."""
    kind = int(g.integers(0, 3))
    seed = int(g.integers(0, 1 << 30))
    xb = (synth.normal_bf16, synth.mixed_rows, synth.special_matrix)[kind](M, N, seed)
    flat = xb.reshape(-1)
    idx = g.integers(0, flat.size, max(1, flat.size // 500))
    flat[idx] = g.integers(0, 128, idx.size).astype(np.uint16) | (g.integers(0, 2, idx.size).astype(np.uint16) << 15)
    return xb


def _same(got, want, tag):
    got = host(got) if isinstance(got, torch.Tensor) else np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (tag, got.shape, want.shape)
    if got.dtype == np.float32:
        got, want = got.view(np.uint32), want.view(np.uint32)
    bad = np.count_nonzero(got != want)
    assert bad == 0, f"{tag}: {bad} elements differ, first at {np.argwhere(got != want)[0].tolist()}"


CAST_CASES = list(range(12))


@pytest.mark.parametrize("case", CAST_CASES)
def test_cast_random_shapes(case):
    require_gpu()
    g = np.random.default_rng(1000 + case)
    M = 128 * int(g.integers(1, 9))
    N = 128 * int(g.integers(1, 9))
    pad = 8 * int(g.integers(0, 5))                          # row pitch N + pad (a multiple of 8)
    grouped = bool(g.integers(0, 2))
    mfma = bool(g.integers(0, 2))
    say(f"random cast case {case}: M={M} N={N} pitch={N + pad} grouped={grouped} mfma={mfma}")
    xb = _values(g, M, N)
    wide = np.zeros((M, N + pad), np.uint16)
    wide[:, :N] = xb
    xd = bf16_to_dev(wide)[:, :N]
    layout = "mfma" if mfma else "plain"
    if grouped:
        G = int(g.integers(1, 9))
        sizes = 128 * g.multinomial(int(g.integers(0, M // 128 + 1)), [1.0 / G] * G)
        offs = np.cumsum(sizes).astype(np.int32)
        rc, want = oracle.mxfp8_grouped(xb, offs, threads=THREADS)
        assert rc == 0
        err = torch.full((1,), -7, dtype=torch.int32, device=DEV)
        got = mxq.mx_quantize_grouped(xd, torch.from_numpy(offs).to(DEV), err=err, scale_layout=layout)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
    else:
        want = oracle.mxfp8_dual(xb, threads=THREADS)
        got = mxq.mx_quantize_2d_dual(xd, scale_layout=layout)
        torch.cuda.synchronize()
    q_row, s_row, q_col, s_col = got
    _same(q_row, want[0], f"case {case} q_row")
    _same(q_col, want[2], f"case {case} q_col")
    if mfma:
        _same(s_row, oracle.scales_to_mfma(want[1]), f"case {case} s_row (matrix-core layout)")
        _same(s_col, oracle.scales_to_mfma(np.ascontiguousarray(want[3].T)), f"case {case} s_col (matrix-core layout)")
    else:
        _same(s_row, want[1], f"case {case} s_row")
        _same(s_col, want[3], f"case {case} s_col")


MX9_CASES = list(range(12))


@pytest.mark.parametrize("case", MX9_CASES)
def test_mx9_random_shapes(case):
    require_gpu()
    g = np.random.default_rng(2000 + case)
    ndim = int(g.integers(1, 4))
    shape = tuple(int(g.integers(1, 70)) for _ in range(ndim))
    if g.integers(0, 3) == 0:                                # sometimes a long axis
        shape = shape[:-1] + (int(g.integers(16, 700)),)
    axis = int(g.integers(-ndim, ndim))
    dtype = ("fp32", "bf16")[int(g.integers(0, 2))]
    records = bool(g.integers(0, 2))
    say(f"random mx9 case {case}: shape={shape} axis={axis} dtype={dtype} records={records}")
    n = int(np.prod(shape))
    x = synth.mx9_weights(1, n, int(g.integers(0, 1 << 30)), "fp32").reshape(shape)
    flat = x.reshape(-1)
    idx = g.integers(0, n, max(1, n // 40))
    specials = np.array([0.0, -0.0, 1e-40, -3e-39, np.inf, -np.inf, np.nan, 2.0 ** -130, 3.0e38], np.float32)
    flat[idx] = specials[g.integers(0, specials.size, idx.size)]
    xh = synth.to_bf16_bits(x) if dtype == "bf16" else x
    xd = (bf16_to_dev(xh.reshape(-1)).view(shape) if dtype == "bf16" else torch.from_numpy(xh).to(DEV))
    wq, we, wp = oracle.mx9_pack_axis(xh, axis, threads=4)
    outer, length, inner = mxq._axis_dims(shape, axis)
    nbl = (length + 15) // 16
    if records:
        packed = mxq.mx9_pack_records(xd, axis)
        torch.cuda.synchronize()
        _same(packed, oracle.mx9_to_records(wq, we, wp, outer * inner, nbl), f"case {case} records")
    else:
        q, e, p = mxq.mx9_pack_axis(xd, axis)
        torch.cuda.synchronize()
        _same(q, wq, f"case {case} q")
        _same(host(e).reshape(-1), we.reshape(-1), f"case {case} max_exp")
        _same(host(p).reshape(-1), wp.reshape(-1), f"case {case} prime")
    for od, td in (("fp32", torch.float32), ("bf16", torch.bfloat16)):
        if records:
            y = mxq.mx9_unpack_records(packed, shape, axis, out_dtype=td)
        else:
            y = mxq.mx9_unpack_axis(q, e, p, shape, axis, out_dtype=td)
        torch.cuda.synchronize()
        _same(y, oracle.mx9_unpack_axis(wq, we, wp, shape, axis, od, threads=4), f"case {case} unpack {od}")


@pytest.mark.parametrize("case", list(range(6)))
def test_scale_conversions_random_views(case):
    """mx_scales_to_mfma from random plain views (row-major, transposed, with
    pitches) and back."""
    require_gpu()
    g = np.random.default_rng(3000 + case)
    R = 64 * int(g.integers(1, 9))
    kb = 4 * int(g.integers(1, 9))
    say(f"random scale conversion case {case}: R={R} kb={kb}")
    S = g.integers(0, 256, (R, kb), dtype=np.uint8)
    if g.integers(0, 2):
        buf = np.zeros((kb + int(g.integers(0, 3)), R + int(g.integers(0, 5))), np.uint8)
        buf[:kb, :R] = S.T
        view = torch.from_numpy(buf).to(DEV)[:kb, :R].t()      # row stride 1, block stride buf.shape[1]
    else:
        buf = np.zeros((R, kb + int(g.integers(0, 5))), np.uint8)
        buf[:, :kb] = S
        view = torch.from_numpy(buf).to(DEV)[:, :kb]
    flat = mxq.scales_to_mfma(view)
    torch.cuda.synchronize()
    _same(flat, oracle.scales_to_mfma(S), f"case {case} to_mfma")
    back = mxq.scales_from_mfma(flat, R, kb)
    torch.cuda.synchronize()
    _same(back, S, f"case {case} from_mfma")


def _codes(g, shape):
    c = g.integers(0, 256, shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38          # no NaN codes
    return c


@pytest.mark.parametrize("case", list(range(10)))
def test_contraction_random_shapes_and_scale_views(case):
    """mx_gemm_nt on random shapes with each operand's scales in a random
    plain form (rows, blocks, with or without a pitch) and a random output
    pitch, so that every route (the pipelined kernel's two plain forms and
    the general kernel) is taken; checked against the oracle within the
    bound the contraction tests derive (2^-10 + (K + 2) 2^-24) sum |a b|."""
    require_gpu()
    g = np.random.default_rng(4000 + case)
    M, N, K = (128 * int(g.integers(1, 5)) for _ in range(3))
    A, B = _codes(g, (M, K)), _codes(g, (N, K))
    kb = K // 32

    def scale_view(rows):
        S = g.integers(118, 137, (rows, kb), dtype=np.uint8)
        form = int(g.integers(0, 3))
        if form == 0:                                       # rows form, pitch a multiple of 4 or not
            pitch = kb + (4 * int(g.integers(0, 2)) if g.integers(0, 3) else 1)
            buf = np.zeros((rows, pitch), np.uint8)
            buf[:, :kb] = S
            return S, torch.from_numpy(buf).to(DEV)[:, :kb], (pitch, 1)
        if form == 1:                                       # blocks form (a transposed s_col)
            pitch = rows + 4 * int(g.integers(0, 2))
            buf = np.zeros((kb, pitch), np.uint8)
            buf[:, :rows] = S.T
            return S, torch.from_numpy(buf).to(DEV)[:, :rows].t(), (1, pitch)
        return S, torch.from_numpy(np.ascontiguousarray(S)).to(DEV), (kb, 1)

    SA, sa_view, sa_str = scale_view(M)
    SB, sb_view, sb_str = scale_view(N)
    out_dtype = (torch.float32, torch.bfloat16)[int(g.integers(0, 2))]
    cpad = (0, 0, 8, 1)[int(g.integers(0, 4))]
    say(f"random contraction case {case}: [{M}, {N}, {K}] sa {sa_str} sb {sb_str} C pitch N+{cpad} {out_dtype}")
    out = torch.full((M, N + cpad), 3.0, dtype=out_dtype, device=DEV)
    mxq.mx_gemm_nt(torch.from_numpy(A).to(DEV), sa_view, torch.from_numpy(B).to(DEV), sb_view, out=out[:, :N])
    torch.cuda.synchronize()
    ref, absC = oracle.mx_gemm_nt(A, SA, B, SB, sa_strides=(kb, 1), sb_strides=(kb, 1), threads=THREADS,
                                  with_abs=True)
    got = out[:, :N].float().cpu().numpy().astype(np.float64)
    tol = (2.0 ** -10 + (K + 2) * 2.0 ** -24) * absC
    if out_dtype == torch.bfloat16:
        tol = tol + 2.0 ** -8 * np.abs(ref)
    bad = np.argwhere(~(np.abs(got - ref) <= tol))
    assert len(bad) == 0, f"case {case}: {len(bad)} entries beyond the bound, first {bad[0].tolist()}"
    if cpad:
        assert torch.all(out[:, N:] == 3.0)
