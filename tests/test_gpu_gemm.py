"""GPU parity of the MXFP8 block-scaled contraction (mx_gemm_nt and its
grouped forms) against the CPU oracle.  Operation: AMD-AGI/ALTO PR #31, "Add
MXFP8 grouped GEMM (E4M3) for routed-expert MoE training" (E4M3 operands,
E8M0 scales per 32 along the contraction, 1-D cumulative offsets).

Tolerance.  The matrix cores do not add the products exactly: measured on
MI355X, a product is truncated (toward zero) to 14 significant bits of the
larger product of its adjacent pair when the two differ widely in magnitude
(448 + 2^-4.3 gives 448 + 2^-5), while products in other lanes, other
32-blocks or other instructions add in fp32.  Reading this as a tree of
truncating 14-bit adders over each 32-block (at most 6 levels, each losing
less than 2^-13 of its operands' magnitude) plus fp32 accumulation, every
element must satisfy
    |C_gpu - C_exact| <= (2^-10 + (K + 2) 2^-24) sum_k |a_k b_k|
(largest observed: 2^-11.8), with C_exact and the sum of magnitudes from the
oracle (binary64).  A bf16 output adds its own rounding, 2^-8 |C_exact|.
The bound still catches a wrong operand, scale or range: one misplaced
scale byte doubles or halves a 32-block's share of the sum, about 1/(K/32)
of sum |a_k b_k| (at least 2^-8 for K <= 8192), and a wrong group or row
moves an element by the order of the sum itself.
Operands whose products share a narrow exponent range, with scales constant
along the contraction, add exactly in that tree and in fp32; for them the
result must equal the oracle's exactly (test_exact_when_no_bits_are_lost).
"""
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


def _codes(g, shape):
    c = g.integers(0, 256, shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38          # no NaN codes
    return c


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _assert_close(got, ref, absC, K, out_dtype, tag):
    got = host(got).astype(np.float64) if got.dtype == torch.float32 else \
        host(got).astype(np.uint32).__lshift__(16).view(np.float32).astype(np.float64)
    tol = (2.0 ** -10 + (K + 2) * 2.0 ** -24) * absC
    if out_dtype == torch.bfloat16:
        tol = tol + 2.0 ** -8 * np.abs(ref)
    err = np.abs(got - ref)
    bad = np.argwhere(~(err <= tol))
    if len(bad):
        i = tuple(bad[0])
        pytest.fail(f"{tag}: {len(bad)} entries beyond the bound; first {list(i)}: got {got[i]!r} "
                    f"want {ref[i]!r} err {err[i]:.3e} tol {tol[i]:.3e}")


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (256, 384, 1024)])
def test_exact_when_no_bits_are_lost(M, N, K):
    """E4M3 values 0.25 .. 3.75 of either sign (exponent fields 6..8) and
    scales constant along the contraction: every product is a multiple of
    2^-10 below 2^4, no adjacent pair spans more than 14 bits and every
    partial sum is exact in fp32 (|C| < 2^14 * 2^(scales)), so the device
    result equals the exact one bit for bit.  This pins the operand layout,
    the per-lane scale selection and the result placement exactly."""
    require_gpu()
    say(f"mx_gemm_nt exact class [{M}, {N}, {K}]")
    g = np.random.default_rng(M * 7 + K)
    def narrow(shape):
        e = g.integers(6, 9, shape)
        return ((g.integers(0, 2, shape) << 7) | (e << 3) | g.integers(0, 8, shape)).astype(np.uint8)
    A, B = narrow((M, K)), narrow((N, K))
    sA = np.repeat(g.integers(120, 134, (M, 1), dtype=np.uint8), K // 32, axis=1)
    sB = np.repeat(g.integers(120, 134, (N, 1), dtype=np.uint8), K // 32, axis=1)
    C = mxq.mx_gemm_nt(_dev(A), _dev(sA), _dev(B), _dev(sB))
    torch.cuda.synchronize()
    ref = oracle.mx_gemm_nt(A, sA, B, sB, sa_strides=(K // 32, 1), sb_strides=(K // 32, 1), threads=THREADS)
    got = host(C).astype(np.float64)
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} entries differ"


def _narrow(g, shape):
    """E4M3 codes with exponent fields 6..8 (|value| 0.25 .. 3.75), either sign."""
    e = g.integers(6, 9, shape)
    return ((g.integers(0, 2, shape) << 7) | (e << 3) | g.integers(0, 8, shape)).astype(np.uint8)


def test_exact_grouped_forms():
    """The exact class of test_exact_when_no_bits_are_lost for both grouped
    forms: the row-grouped forward (per-row and per-expert scales constant
    along the contraction, four-step scale periods) and the contraction-
    grouped weight gradient (scales read through the colwise transpose).
    Their results must equal the oracle's bit for bit, which pins each
    group's operand, scale and range selection exactly."""
    require_gpu()
    say("grouped forms, exact class")
    g = np.random.default_rng(99)
    M, N, K, E = 768, 256, 1024, 4
    A = _narrow(g, (M, K))
    Bs = np.stack([_narrow(g, (N, K)) for _ in range(E)])
    sA = np.repeat(g.integers(120, 134, (M, 1), dtype=np.uint8), K // 32, axis=1)
    sB = np.repeat(g.integers(120, 134, (E, N, 1), dtype=np.uint8), K // 32, axis=2)
    offs = np.array([256, 256, 640, 768], np.int32)
    C = mxq.mx_grouped_gemm_rows(_dev(A), _dev(sA), _dev(Bs), _dev(sB), _dev(offs))
    torch.cuda.synchronize()
    ref = oracle.mx_grouped_gemm_rows(A, sA, Bs, sB, offs, sa_strides=(K // 32, 1), sb_strides=(K // 32, 1),
                                      threads=THREADS)
    got = host(C).astype(np.float64)
    assert np.array_equal(got, ref), f"row groups: {np.count_nonzero(got != ref)} entries differ"

    M, N, K = 256, 384, 1024
    A, B = _narrow(g, (M, K)), _narrow(g, (N, K))
    sAc = np.repeat(g.integers(120, 134, (1, M), dtype=np.uint8), K // 32, axis=0)      # [K/32, M]
    sBc = np.repeat(g.integers(120, 134, (1, N), dtype=np.uint8), K // 32, axis=0)
    offs = np.array([256, 256, 640, 896], np.int32)
    C = mxq.mx_grouped_gemm_k(_dev(A), _dev(sAc).t(), _dev(B), _dev(sBc).t(), _dev(offs))
    torch.cuda.synchronize()
    ref = oracle.mx_grouped_gemm_k(A, sAc, B, sBc, offs, sa_strides=(1, M), sb_strides=(1, N), threads=THREADS)
    got = host(C).astype(np.float64)
    assert np.array_equal(got, ref), f"contraction groups: {np.count_nonzero(got != ref)} entries differ"


def _one_hot_blocks(g, rows, K):
    """E4M3 codes that are 0 except at the first position of every 32-block,
    where they are +-1 or +-2: each 32-block then contributes one product."""
    c = np.zeros((rows, K), np.uint8)
    c[:, ::32] = g.choice(np.array([0x38, 0xB8, 0x40, 0xC0], np.uint8), (rows, K // 32))
    return c


def test_exact_one_hot_blocks_every_scale_layout():
    """Scales that differ in every row and every 32-block (exponents 125..129)
    with one nonzero product per block: every block's term is exact and the
    terms span few enough bits that fp32 sums them exactly, so each result
    must equal the oracle's bit for bit.  A scale read from the wrong row or
    block changes the result, so this pins, through the matrix instruction
    itself, the matrix-core scale layout (scales_to_mfma) and the plain
    forms, for the dense product and both grouped forms."""
    require_gpu()
    say("one-hot blocks, every scale layout, exact")
    g = np.random.default_rng(123)
    M, N, K, E = 512, 256, 1024, 3
    kb = K // 32
    A, B = _one_hot_blocks(g, M, K), _one_hot_blocks(g, N, K)
    sA = g.integers(125, 130, (M, kb), dtype=np.uint8)
    sB = g.integers(125, 130, (N, kb), dtype=np.uint8)
    ref = oracle.mx_gemm_nt(A, sA, B, sB, sa_strides=(kb, 1), sb_strides=(kb, 1), threads=THREADS)
    for form in ("mfma", "rows", "blocks"):
        if form == "mfma":
            C = mxq.mx_gemm_nt_mfma(_dev(A), _dev(oracle.scales_to_mfma(sA)), _dev(B), _dev(oracle.scales_to_mfma(sB)))
        elif form == "rows":
            C = mxq.mx_gemm_nt(_dev(A), _dev(sA), _dev(B), _dev(sB))
        else:
            C = mxq.mx_gemm_nt(_dev(A), _dev(np.ascontiguousarray(sA.T)).t(), _dev(B),
                               _dev(np.ascontiguousarray(sB.T)).t())
        torch.cuda.synchronize()
        got = host(C).astype(np.float64)
        assert np.array_equal(got, ref), f"dense ({form}): {np.count_nonzero(got != ref)} entries differ"

    Bs = np.stack([_one_hot_blocks(g, N, K) for _ in range(E)])
    sBs = g.integers(125, 130, (E, N, kb), dtype=np.uint8)
    offs = np.array([128, 384, 384], np.int32)
    ref = oracle.mx_grouped_gemm_rows(A, sA, Bs, sBs, offs, sa_strides=(kb, 1), sb_strides=(kb, 1), threads=THREADS)
    sBm = np.stack([oracle.scales_to_mfma(sBs[e]) for e in range(E)])
    for form in ("mfma", "rows"):
        if form == "mfma":
            C = mxq.mx_grouped_gemm_rows_mfma(_dev(A), _dev(oracle.scales_to_mfma(sA)), _dev(Bs), _dev(sBm),
                                              _dev(offs))
        else:
            C = mxq.mx_grouped_gemm_rows(_dev(A), _dev(sA), _dev(Bs), _dev(sBs), _dev(offs))
        torch.cuda.synchronize()
        got = host(C).astype(np.float64)
        assert np.array_equal(got, ref), f"row groups ({form}): {np.count_nonzero(got != ref)} entries differ"

    # contraction groups: A [M, K] and B [N, K] with the 32-blocks along the tokens
    offs = np.array([256, 256, 768, 896], np.int32)
    sAc, sBc = np.ascontiguousarray(sA.T), np.ascontiguousarray(sB.T)              # [K/32, M], [K/32, N]
    ref = oracle.mx_grouped_gemm_k(A, sAc, B, sBc, offs, sa_strides=(1, M), sb_strides=(1, N), threads=THREADS)
    for form in ("mfma", "blocks"):
        if form == "mfma":
            C = mxq.mx_grouped_gemm_k_mfma(_dev(A), _dev(oracle.scales_to_mfma(sA)), _dev(B),
                                           _dev(oracle.scales_to_mfma(sB)), _dev(offs))
        else:
            C = mxq.mx_grouped_gemm_k(_dev(A), _dev(sAc).t(), _dev(B), _dev(sBc).t(), _dev(offs))
        torch.cuda.synchronize()
        got = host(C).astype(np.float64)
        assert np.array_equal(got, ref), f"contraction groups ({form}): {np.count_nonzero(got != ref)} entries differ"


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (256, 384, 512), (384, 256, 1024)])
def test_dense_parity(M, N, K, out_dtype):
    require_gpu()
    say(f"mx_gemm_nt [{M}, {N}, {K}] -> {out_dtype}")
    g = np.random.default_rng(M + N + K)
    A, B = _codes(g, (M, K)), _codes(g, (N, K))
    sA = g.integers(118, 137, (M, K // 32), dtype=np.uint8)
    sB = g.integers(118, 137, (N, K // 32), dtype=np.uint8)
    C = mxq.mx_gemm_nt(_dev(A), _dev(sA), _dev(B), _dev(sB), out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref, absC = oracle.mx_gemm_nt(A, sA, B, sB, sa_strides=(K // 32, 1), sb_strides=(K // 32, 1),
                                  threads=THREADS, with_abs=True)
    _assert_close(C, ref, absC, K, out_dtype, f"dense {M}x{N}x{K}")


@pytest.mark.parametrize("K", [512, 2048])
def test_rows_form_four_step_scale_loads(K):
    """Rows-form scales whose rows are 16-byte aligned, with K a multiple of
    512, are loaded four contraction steps at a time (one 16-byte piece per
    row into a period buffer).  The same scales at a row pitch that is a
    multiple of 4 only take the per-step route: both give the same bits, and
    both match the oracle, for the dense product (ragged column tiles) and
    the row-grouped forward (groups of odd and even unit counts, a tail)."""
    require_gpu()
    say(f"rows-form scales in four-step periods, K={K}")
    g = np.random.default_rng(K + 17)
    kb = K // 32

    def pitched(S, pad):
        buf = np.zeros(S.shape[:-1] + (kb + pad,), np.uint8)
        buf[..., :kb] = S
        return torch.from_numpy(buf).to(DEV)[..., :kb]

    M, N = 384, 640
    A, B = _codes(g, (M, K)), _codes(g, (N, K))
    sA = g.integers(118, 137, (M, kb), dtype=np.uint8)
    sB = g.integers(118, 137, (N, kb), dtype=np.uint8)
    ref, absC = oracle.mx_gemm_nt(A, sA, B, sB, sa_strides=(kb, 1), sb_strides=(kb, 1), threads=THREADS,
                                  with_abs=True)
    for out_dtype in (torch.float32, torch.bfloat16):
        C4 = mxq.mx_gemm_nt(_dev(A), pitched(sA, 16), _dev(B), pitched(sB, 16), out_dtype=out_dtype)
        C1 = mxq.mx_gemm_nt(_dev(A), pitched(sA, 4), _dev(B), pitched(sB, 4), out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(C4.view(torch.int16) if out_dtype == torch.bfloat16 else C4.view(torch.int32),
                           C1.view(torch.int16) if out_dtype == torch.bfloat16 else C1.view(torch.int32))
        _assert_close(C4, ref, absC, K, out_dtype, f"dense rows-form periods K={K}")

    M, N, E = 1280, 384, 5
    A = _codes(g, (M, K))
    Bs = np.stack([_codes(g, (N, K)) for _ in range(E)])
    sA = g.integers(118, 137, (M, kb), dtype=np.uint8)
    sB = g.integers(118, 137, (E, N, kb), dtype=np.uint8)
    offs = np.array([384, 384, 640, 1024, 1152], np.int32)          # 3, 0, 2, 3, 1 units, a 128-row tail
    ref, absC = oracle.mx_grouped_gemm_rows(A, sA, Bs, sB, offs, sa_strides=(kb, 1), sb_strides=(kb, 1),
                                            threads=THREADS, with_abs=True)
    C4 = mxq.mx_grouped_gemm_rows(_dev(A), _dev(sA), _dev(Bs), _dev(sB), _dev(offs))
    C1 = mxq.mx_grouped_gemm_rows(_dev(A), pitched(sA, 4), _dev(Bs), pitched(sB, 4), _dev(offs))
    torch.cuda.synchronize()
    assert torch.equal(C4.view(torch.int32), C1.view(torch.int32))
    _assert_close(C4, ref, absC, K, torch.float32, f"row groups rows-form periods K={K}")
    assert torch.all(C4[offs[-1]:] == 0)


def test_dense_transposed_scales_and_pitches():
    """Scales read through transposed views (the colwise cast's s_col layout),
    operand row pitches above K and an output pitch above N."""
    require_gpu()
    say("mx_gemm_nt with s_col-layout scales and padded pitches")
    g = np.random.default_rng(7)
    M, N, K = 256, 128, 384
    Aw, Bw = _codes(g, (M, K + 64)), _codes(g, (N, K + 128))
    sAc = g.integers(118, 137, (K // 32, M), dtype=np.uint8)        # [K/32, M]
    sBc = g.integers(118, 137, (K // 32, N), dtype=np.uint8)
    out = torch.full((M, N + 32), 7.0, dtype=torch.float32, device=DEV)
    mxq.mx_gemm_nt(_dev(Aw)[:, :K], _dev(sAc).t(), _dev(Bw)[:, :K], _dev(sBc).t(), out=out[:, :N])
    torch.cuda.synchronize()
    ref, absC = oracle.mx_gemm_nt(Aw[:, :K], sAc, Bw[:, :K], sBc, sa_strides=(1, M), sb_strides=(1, N),
                                  threads=THREADS, with_abs=True)
    _assert_close(out[:, :N], ref, absC, K, torch.float32, "transposed scales")
    assert torch.all(out[:, N:] == 7.0)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_row_groups_parity(out_dtype):
    require_gpu()
    say(f"mx_grouped_gemm_rows -> {out_dtype}")
    g = np.random.default_rng(8)
    M, N, K, E = 1024, 256, 384, 5
    A = _codes(g, (M, K))
    sA = g.integers(118, 137, (M, K // 32), dtype=np.uint8)
    B = np.stack([_codes(g, (N, K)) for _ in range(E)])
    sBc = g.integers(118, 137, (E, K // 32, N), dtype=np.uint8)      # per expert, the colwise layout
    offs = np.array([128, 128, 512, 640, 896], np.int32)             # an empty group and a 128-row tail
    C = mxq.mx_grouped_gemm_rows(_dev(A), _dev(sA), _dev(B), _dev(sBc).transpose(1, 2), _dev(offs),
                                 out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref, absC = oracle.mx_grouped_gemm_rows(A, sA, B, sBc, offs, sa_strides=(K // 32, 1), sb_strides=(1, N),
                                            threads=THREADS, with_abs=True)
    _assert_close(C, ref, absC, K, out_dtype, "row groups")
    assert torch.all(C[offs[-1]:] == 0)


@pytest.mark.parametrize("M,covered", [(384, 256), (1664, 1664), (1664, 0), (2560, 1920), (128, 128)])
def test_row_groups_every_tile_once(M, covered):
    """Row tiles are shared out over the XCDs as contiguous covered and tail
    ranges; row-tile counts that are not multiples of 8, a buffer with no
    tail and one with no covered rows all give every output row exactly
    once, matching the oracle (tail rows 0)."""
    require_gpu()
    say(f"mx_grouped_gemm_rows schedule M={M} covered={covered}")
    g = np.random.default_rng(M + covered)
    N, K, E = 384, 256, 6
    A = _codes(g, (M, K))
    sA = g.integers(118, 137, (M, K // 32), dtype=np.uint8)
    B = np.stack([_codes(g, (N, K)) for _ in range(E)])
    sB = g.integers(118, 137, (E, N, K // 32), dtype=np.uint8)
    sizes = 128 * g.multinomial(covered // 128, np.full(E, 1.0 / E))
    offs = np.cumsum(sizes).astype(np.int32)
    assert offs[-1] == covered
    out = torch.full((M, N), 3.0, dtype=torch.float32, device=DEV)
    mxq.mx_grouped_gemm_rows(_dev(A), _dev(sA), _dev(B), _dev(sB), _dev(offs), out=out)
    torch.cuda.synchronize()
    ref, absC = oracle.mx_grouped_gemm_rows(A, sA, B, sB, offs, sa_strides=(K // 32, 1), sb_strides=(K // 32, 1),
                                            threads=THREADS, with_abs=True)
    _assert_close(out, ref, absC, K, torch.float32, f"schedule M={M}")
    assert torch.all(out[covered:] == 0)


def _clamped_ends(offs, hi):
    """The group ends the pipelined kernels read from any offsets: each
    rounded toward zero to a multiple of 128, clamped to [0, hi], then a
    running maximum.  The header leaves the expert of rows under invalid
    offsets unspecified; the kernels take this reading, under which the
    row tiles still partition the rows."""
    ends, c = [], 0
    for o in offs:
        v = int(o / 128) * 128
        c = max(c, min(max(v, 0), hi))
        ends.append(c)
    return np.array(ends, np.int32)


@pytest.mark.parametrize("offs", [[640, 128, 5000, 300], [-300, 256, 200, 768], [1100, 0, 0, 0], [200, 330, 900, 1000]])
def test_row_groups_invalid_offsets(offs):
    """Offsets that are unsorted, negative, past M or not multiples of 128:
    the forward stays inside its operands, writes every output row once, and
    gives what valid offsets at the clamped ends give (both scale forms of
    the pipelined kernel)."""
    require_gpu()
    say(f"mx_grouped_gemm_rows invalid offs {offs}")
    g = np.random.default_rng(sum(abs(o) for o in offs))
    M, N, K, E = 1024, 384, 256, 4
    A = _codes(g, (M, K))
    sA = g.integers(118, 137, (M, K // 32), dtype=np.uint8)
    B = np.stack([_codes(g, (N, K)) for _ in range(E)])
    sB = g.integers(118, 137, (E, N, K // 32), dtype=np.uint8)
    o = np.array(offs, np.int32)
    ends = _clamped_ends(offs, M)
    ref, absC = oracle.mx_grouped_gemm_rows(A, sA, B, sB, ends, sa_strides=(K // 32, 1), sb_strides=(K // 32, 1),
                                            threads=THREADS, with_abs=True)
    outs = {}
    for form in ("rows", "mfma"):
        out = torch.full((M, N), 3.0, dtype=torch.float32, device=DEV)
        if form == "rows":
            mxq.mx_grouped_gemm_rows(_dev(A), _dev(sA), _dev(B), _dev(sB), _dev(o), out=out)
        else:
            sBm = np.stack([oracle.scales_to_mfma(sB[e]) for e in range(E)])
            mxq.mx_grouped_gemm_rows_mfma(_dev(A), _dev(oracle.scales_to_mfma(sA)), _dev(B), _dev(sBm), _dev(o),
                                          out=out)
        torch.cuda.synchronize()
        _assert_close(out, ref, absC, K, torch.float32, f"invalid offs {offs} ({form})")
        assert torch.all(out[int(ends[-1]):] == 0)
        outs[form] = out
    assert torch.equal(outs["rows"], outs["mfma"])


def _clamp_range(lo_raw, hi_raw, K):
    """The contraction range [k_lo, k_hi) the pipelined kernel reads for one
    group from its two raw offsets: k_lo is the previous offset clamped to
    [0, K], k_hi the group's clamped to [k_lo, K], both rounded down to a
    multiple of 128 from 0 and from k_lo."""
    lo = min(max(lo_raw, 0), K)
    lo -= lo % 128
    hi = min(max(hi_raw, lo), K)
    hi -= (hi - lo) % 128
    return lo, hi


@pytest.mark.parametrize("offs", [[300, 100, 900, 5000], [-128, 640, 512, 1024]])
def test_contraction_groups_invalid_offsets(offs):
    """The weight gradient under invalid offsets: each group's range is its
    two offsets clamped to multiples of 128 inside [0, K] (ranges may then
    overlap or be empty); every access stays inside the operands and each
    group's result is the contraction over its clamped range."""
    require_gpu()
    say(f"mx_grouped_gemm_k invalid offs {offs}")
    g = np.random.default_rng(7 + sum(abs(o) for o in offs))
    M, N, K = 256, 384, 1024
    A, B = _codes(g, (M, K)), _codes(g, (N, K))
    sAc = g.integers(118, 137, (K // 32, M), dtype=np.uint8)
    sBc = g.integers(118, 137, (K // 32, N), dtype=np.uint8)
    C = mxq.mx_grouped_gemm_k(_dev(A), _dev(sAc).t(), _dev(B), _dev(sBc).t(), _dev(np.array(offs, np.int32)))
    torch.cuda.synchronize()
    prev = 0
    for e, raw in enumerate(offs):
        lo, hi = _clamp_range(prev, raw, K)
        prev = raw
        if hi == lo:
            assert torch.all(C[e] == 0), f"group {e} over an empty range"
            continue
        ref, absC = oracle.mx_grouped_gemm_k(np.ascontiguousarray(A[:, lo:hi]), sAc[lo // 32:hi // 32],
                                             np.ascontiguousarray(B[:, lo:hi]), sBc[lo // 32:hi // 32],
                                             np.array([hi - lo], np.int32), sa_strides=(1, M), sb_strides=(1, N),
                                             threads=THREADS, with_abs=True)
        _assert_close(C[e], ref[0], absC[0], hi - lo, torch.float32, f"group {e} [{lo}, {hi})")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_contraction_groups_parity(out_dtype):
    require_gpu()
    say(f"mx_grouped_gemm_k -> {out_dtype}")
    g = np.random.default_rng(9)
    M, N, K = 256, 384, 1024
    A, B = _codes(g, (M, K)), _codes(g, (N, K))
    sAc = g.integers(118, 137, (K // 32, M), dtype=np.uint8)
    sBc = g.integers(118, 137, (K // 32, N), dtype=np.uint8)
    offs = np.array([256, 256, 640, 896], np.int32)                  # an empty group, a 128-long tail
    C = mxq.mx_grouped_gemm_k(_dev(A), _dev(sAc).t(), _dev(B), _dev(sBc).t(), _dev(offs), out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref, absC = oracle.mx_grouped_gemm_k(A, sAc, B, sBc, offs, sa_strides=(1, M), sb_strides=(1, N),
                                         threads=THREADS, with_abs=True)
    assert C.shape == (4, M, N)
    for e in range(4):
        kk = int(offs[e] - (offs[e - 1] if e else 0))
        _assert_close(C[e], ref[e], absC[e], max(kk, 1), out_dtype, f"group {e}")
    assert torch.all(C[1] == 0)


@pytest.mark.parametrize("case", ["scale_pitch_not_4", "c_pitch_not_16B", "row_groups_rows_form", "mixed_forms"])
def test_plain_scale_routes(case):
    """Plain scales reach the pipelined kernel when both operands' scales are
    in the rows form (block stride 1, row stride a multiple of 4) or both in
    the blocks form (row stride 1, block stride a multiple of 4) and C rows
    are 16-byte pieces; other views take the general kernel.  Each route
    matches the oracle."""
    require_gpu()
    say(f"mx_gemm plain-scale route: {case}")
    g = np.random.default_rng(31 + len(case))
    M, N, K = 384, 256, 640
    A, B = _codes(g, (M, K)), _codes(g, (N, K))
    if case == "row_groups_rows_form":
        E = 3
        Bs = np.stack([_codes(g, (N, K)) for _ in range(E)])
        sA = g.integers(118, 137, (M, K // 32), dtype=np.uint8)
        sB = g.integers(118, 137, (E, N, K // 32), dtype=np.uint8)
        offs = np.array([128, 128, 256], np.int32)
        C = mxq.mx_grouped_gemm_rows(_dev(A), _dev(sA), _dev(Bs), _dev(sB), _dev(offs))
        torch.cuda.synchronize()
        ref, absC = oracle.mx_grouped_gemm_rows(A, sA, Bs, sB, offs, sa_strides=(K // 32, 1),
                                                sb_strides=(K // 32, 1), threads=THREADS, with_abs=True)
        _assert_close(C, ref, absC, K, torch.float32, case)
        assert torch.all(C[offs[-1]:] == 0)
        return
    if case == "scale_pitch_not_4":
        sAw = g.integers(118, 137, (M, K // 32 + 1), dtype=np.uint8)     # row stride 21
        sBw = g.integers(118, 137, (N, K // 32 + 1), dtype=np.uint8)
        C = mxq.mx_gemm_nt(_dev(A), _dev(sAw)[:, :K // 32], _dev(B), _dev(sBw)[:, :K // 32])
        sA, sB = sAw, sBw                                               # read through row stride 21
        sa, sb = (K // 32 + 1, 1), (K // 32 + 1, 1)
    elif case == "c_pitch_not_16B":
        sA = g.integers(118, 137, (M, K // 32), dtype=np.uint8)
        sB = g.integers(118, 137, (N, K // 32), dtype=np.uint8)
        out = torch.full((M, N + 1), 5.0, dtype=torch.float32, device=DEV)
        mxq.mx_gemm_nt(_dev(A), _dev(sA), _dev(B), _dev(sB), out=out[:, :N])
        C = out[:, :N]
        sa, sb = (K // 32, 1), (K // 32, 1)
    else:                                                                 # A rows form, B blocks form
        sA = g.integers(118, 137, (M, K // 32), dtype=np.uint8)
        sBc = g.integers(118, 137, (K // 32, N), dtype=np.uint8)
        C = mxq.mx_gemm_nt(_dev(A), _dev(sA), _dev(B), _dev(sBc).t())
        sB = sBc
        sa, sb = (K // 32, 1), (1, N)
    torch.cuda.synchronize()
    ref, absC = oracle.mx_gemm_nt(A, sA, B, sB, sa_strides=sa, sb_strides=sb, threads=THREADS, with_abs=True)
    _assert_close(C, ref, absC, K, torch.float32, case)
    if case == "c_pitch_not_16B":
        assert torch.all(out[:, N] == 5.0)


def test_consumes_the_cast_outputs_forward_and_weight_gradient():
    """End to end on the device: the dual-axis cast quantizes bf16 operands
    and the contraction consumes its outputs as they are laid out (q_row with
    s_row; q_col with s_col read transposed).  The GEMM matches the oracle on
    the same bytes, and the product of the quantized operands stays close to
    the product of the bf16 operands (SNR recorded, loose floor)."""
    require_gpu()
    say("cast -> contraction, forward and weight gradient")
    M, K, N = 512, 768, 384
    X = synth.normal_bf16(M, K, 21)                 # activations [tokens, K]
    W = synth.normal_bf16(K, N, 22)                 # weight [K, N]
    dY = synth.normal_bf16(M, N, 23)                # output gradient [tokens, N]
    qx = mxq.mx_quantize_2d_dual(bf16_to_dev(X))    # q_row [M, K], s_row [M, K/32], q_col [K, M], s_col [M/32, K]
    qw = mxq.mx_quantize_2d_dual(bf16_to_dev(W))    # q_col [N, K], s_col [K/32, N]
    qd = mxq.mx_quantize_2d_dual(bf16_to_dev(dY))   # q_col [N, M], s_col [M/32, N]
    # forward: out = X W
    out = mxq.mx_gemm_nt(qx[0], qx[1], qw[2], qw[3].t())
    # weight gradient: dW = X^T dY, contraction over tokens
    dW = mxq.mx_gemm_nt(qx[2], qx[3].t(), qd[2], qd[3].t())
    torch.cuda.synchronize()
    hx, hw, hd = [tuple(host(t) for t in q) for q in (qx, qw, qd)]
    ref, absC = oracle.mx_gemm_nt(hx[0], hx[1], hw[2], hw[3], sa_strides=(K // 32, 1), sb_strides=(1, N),
                                  threads=THREADS, with_abs=True)
    _assert_close(out, ref, absC, K, torch.float32, "forward")
    ref2, abs2 = oracle.mx_gemm_nt(hx[2], hx[3], hd[2], hd[3], sa_strides=(1, K), sb_strides=(1, N),
                                   threads=THREADS, with_abs=True)
    _assert_close(dW, ref2, abs2, M, torch.float32, "weight gradient")
    xf, wf, df = (synth.bf16_bits_to_f32(a).astype(np.float64) for a in (X, W, dY))
    for name, got, exact in (("forward", host(out), xf @ wf), ("weight gradient", host(dW), xf.T @ df)):
        snr = 10 * np.log10((exact ** 2).sum() / ((exact - got) ** 2).sum())
        say(f"  {name}: SNR of the MXFP8 product vs the bf16 product {snr:.1f} dB")
        assert snr > 20.0


def test_rejections():
    require_gpu()
    say("mx_gemm_nt rejections")
    a = torch.zeros((128, 128), dtype=torch.uint8, device=DEV)
    s = torch.zeros((128, 4), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        mxq.mx_gemm_nt(a, s[:, :3], a, s)
    with pytest.raises(mxq.MXError) as ei:
        mxq.mx_gemm_nt(a[:, :96], s[:, :3], a[:, :96], s[:, :3])
    assert ei.value.status == 5


# ---------------------------------------------------------------- full sizes

def test_full_size_grouped_forward_and_weight_gradient_sampled():
    """The grouped activation buffer bf16 [16384, 5120] with 64 groups, cast on
    the device, consumed by both grouped contractions (expert operands of 256
    rows of random codes); sampled rows of every group and of the tail are
    compared with the oracle."""
    require_gpu()
    say("full size: grouped cast [16384, 5120] -> grouped contractions, sampled")
    xb, offs = synth.grouped()
    M, K = xb.shape
    N, E = 256, len(offs)
    xd = bf16_to_dev(xb)
    od = _dev(offs)
    q_row, s_row, q_col, s_col = mxq.mx_quantize_grouped(xd, od)
    g = np.random.default_rng(10)
    Bf = np.stack([_codes(g, (N, K)) for _ in range(E)])
    sBf = g.integers(118, 137, (E, N, K // 32), dtype=np.uint8)
    C = mxq.mx_grouped_gemm_rows(q_row, s_row, _dev(Bf), _dev(sBf), od)
    torch.cuda.synchronize()
    hq, hs = host(q_row), host(s_row)
    lo = 0
    rows = []
    for e, hi in enumerate(offs):
        if hi > lo:
            rows += [(e, int(lo)), (e, int(hi) - 1)]
        lo = hi
    hC = host(C)
    for e, r in rows[::3]:
        ref, absC = oracle.mx_gemm_nt(hq[r:r + 1], hs[r:r + 1], Bf[e], sBf[e], sa_strides=(K // 32, 1),
                                      sb_strides=(K // 32, 1), threads=THREADS, with_abs=True)
        _assert_close(torch.from_numpy(hC[r:r + 1]), ref, absC, K, torch.float32, f"forward row {r} expert {e}")
    assert np.all(hC[offs[-1]:] == 0)
    del C, hC
    # weight gradient: A = q_col [K, M] with s_col read as [K, M/32]; B = random codes over the tokens
    Bt = _codes(g, (N, M))
    sBt = g.integers(118, 137, (M // 32, N), dtype=np.uint8)
    dW = mxq.mx_grouped_gemm_k(q_col, s_col.t(), _dev(Bt), _dev(sBt).t(), od, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    hqc, hsc = host(q_col), host(s_col)
    krows = [0, 1111, K - 1]
    lo = 0
    for e, hi in enumerate(offs):
        if e % 9 == 0 or e == E - 1:
            got = dW[e, krows]
            ref = np.zeros((len(krows), N))
            absC = np.zeros((len(krows), N))
            if hi > lo:
                for i, kr in enumerate(krows):
                    r1, a1 = oracle.mx_gemm_nt(hqc[kr:kr + 1], hsc[:, kr:kr + 1], Bt, sBt, sa_strides=(1, 1),
                                               sb_strides=(1, N), k0=int(lo), k1=int(hi), with_abs=True)
                    ref[i], absC[i] = r1[0], a1[0]
            _assert_close(got, ref, absC, max(int(hi - lo), 1), torch.bfloat16, f"weight gradient group {e}")
        lo = hi
