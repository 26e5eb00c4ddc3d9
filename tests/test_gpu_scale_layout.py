"""GPU parity of the matrix-core scale layout: the dual-axis cast with
scale_layout="mfma" (pytorch/ao PR #4995, "[moe_training] Fused dual-axis
MXFP8 quantization with correct metadata": the kernel writes the consumer's
swizzled scale layout itself) and the contractions that read it (AMD-AGI/ALTO
PR #31, "Add MXFP8 grouped GEMM (E4M3) for routed-expert MoE training").

The cast must give the oracle's codes byte for byte and the oracle's scales
permuted by oracle.scales_to_mfma (s_row as the operand [M rows, N/32
blocks], s_col transposed to the operand [N rows, M/32 blocks]).  The
contractions must meet the oracle within the matrix cores' measured bound
(see test_gpu_gemm.py) and equal the strided-view contraction on the same
bytes exactly (same instructions, same order).
"""
import numpy as np
import pytest
import torch

import mx9_dual_axis_amd as mxq
import oracle
from helpers import bf16_to_dev, host, require_gpu, say
from mx9_dual_axis_amd import synth
from test_gpu_gemm import DEV, _assert_close, _codes, _dev

pytestmark = pytest.mark.gpu
THREADS = 16


def _want_mfma(want):
    """The oracle's dual-axis outputs with both scale tensors in the matrix-core layout."""
    q_row, s_row, q_col, s_col = want
    return q_row, oracle.scales_to_mfma(s_row), q_col, oracle.scales_to_mfma(np.ascontiguousarray(s_col.T))


def _dirty(M, N, dev, fill=0xA5):
    kw = dict(dtype=torch.uint8, device=dev)
    return tuple(torch.full(s, fill, **kw) for s in ((M, N), (M * N // 32,), (N, M), (M * N // 32,)))


def _assert_equal(got, want, tag):
    for name, g, w in zip(("q_row", "s_row", "q_col", "s_col"), got, want):
        g = host(g)
        assert g.shape == w.shape, (tag, name, g.shape, w.shape)
        bad = np.count_nonzero(g != w)
        if bad:
            idx = np.argwhere(g != w)[:5]
            pytest.fail(f"{tag}: {name} differs in {bad} bytes, first at {idx.tolist()}")


@pytest.mark.parametrize("M,N,kind,seed", [
    (128, 128, "special", 1),
    (256, 384, "normal", 2),
    (384, 1152, "special", 3),      # N % 512 != 0
    (640, 2560, "mixed", 4),
])
def test_dense_cast_in_the_matrix_core_layout(M, N, kind, seed):
    dev = require_gpu()
    say(f"mfma-layout cast M={M} N={N} kind={kind}")
    xb = {"normal": synth.normal_bf16, "special": synth.special_matrix, "mixed": synth.mixed_rows}[kind](M, N, seed)
    out = _dirty(M, N, dev)
    mxq.mx_quantize_2d_dual(bf16_to_dev(xb), out=out, scale_layout="mfma")
    torch.cuda.synchronize()
    _assert_equal(out, _want_mfma(oracle.mxfp8_dual(xb, threads=THREADS)), f"{M}x{N}")


@pytest.mark.parametrize("offs", [[128, 128, 384, 512], [0, 640], [256, 768, 896]])
def test_grouped_cast_in_the_matrix_core_layout(offs):
    dev = require_gpu()
    M, N = 896, 640
    say(f"mfma-layout grouped cast M={M} N={N} offs={offs}")
    xb = synth.special_matrix(M, N, 7)
    o = np.array(offs, np.int32)
    err = torch.full((1,), -1, dtype=torch.int32, device=dev)
    out = _dirty(M, N, dev)
    mxq.mx_quantize_grouped(bf16_to_dev(xb), _dev(o), err=err, out=out, scale_layout="mfma")
    torch.cuda.synchronize()
    rc, want = oracle.mxfp8_grouped(xb, o, threads=THREADS)
    assert rc == 0 and int(err.item()) == 0
    _assert_equal(out, _want_mfma(want), f"grouped {offs}")


def test_layout_is_a_permutation_of_the_plain_call():
    """Both layouts of one input on the device: the same multiset of bytes,
    placed by the oracle's index function."""
    dev = require_gpu()
    M, N = 512, 1024
    say("mfma layout vs plain layout on the device")
    xd = bf16_to_dev(synth.mixed_rows(M, N, 9))
    plain = [host(t) for t in mxq.mx_quantize_2d_dual(xd)]
    mf = [host(t) for t in mxq.mx_quantize_2d_dual(xd, scale_layout="mfma")]
    torch.cuda.synchronize()
    assert np.array_equal(mf[0], plain[0]) and np.array_equal(mf[2], plain[2])
    assert np.array_equal(oracle.scales_from_mfma(mf[1], M, N // 32), plain[1])
    assert np.array_equal(oracle.scales_from_mfma(mf[3], N, M // 32), plain[3].T)


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (256, 384, 1024)])
def test_gemm_reads_the_layout(M, N, K):
    require_gpu()
    say(f"mx_gemm_nt_mfma [{M}, {N}, {K}]")
    g = np.random.default_rng(M + 3 * K)
    A, B = _codes(g, (M, K)), _codes(g, (N, K))
    sA = g.integers(118, 137, (M, K // 32), dtype=np.uint8)
    sB = g.integers(118, 137, (N, K // 32), dtype=np.uint8)
    C = mxq.mx_gemm_nt_mfma(_dev(A), _dev(oracle.scales_to_mfma(sA)), _dev(B), _dev(oracle.scales_to_mfma(sB)))
    Cs = mxq.mx_gemm_nt(_dev(A), _dev(sA), _dev(B), _dev(sB))
    torch.cuda.synchronize()
    ref, absC = oracle.mx_gemm_nt(A, sA, B, sB, sa_strides=(K // 32, 1), sb_strides=(K // 32, 1),
                                  threads=THREADS, with_abs=True)
    _assert_close(C, ref, absC, K, torch.float32, "mfma layout")
    assert torch.equal(C, Cs)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_grouped_gemms_read_the_layout(out_dtype):
    require_gpu()
    say(f"grouped contractions, mfma layout -> {out_dtype}")
    g = np.random.default_rng(11)
    M, N, K, E = 1024, 256, 384, 5
    A = _codes(g, (M, K))
    sA = g.integers(118, 137, (M, K // 32), dtype=np.uint8)
    B = np.stack([_codes(g, (N, K)) for _ in range(E)])
    sB = g.integers(118, 137, (E, N, K // 32), dtype=np.uint8)
    sBm = np.stack([oracle.scales_to_mfma(sB[e]) for e in range(E)])
    offs = np.array([128, 128, 512, 640, 896], np.int32)
    C = mxq.mx_grouped_gemm_rows_mfma(_dev(A), _dev(oracle.scales_to_mfma(sA)), _dev(B), _dev(sBm), _dev(offs),
                                      out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref, absC = oracle.mx_grouped_gemm_rows(A, sA, B, sB, offs, sa_strides=(K // 32, 1), sb_strides=(K // 32, 1),
                                            threads=THREADS, with_abs=True)
    _assert_close(C, ref, absC, K, out_dtype, "row groups, mfma layout")
    assert torch.all(C[offs[-1]:] == 0)

    M2, N2, K2 = 256, 384, 1024
    A2, B2 = _codes(g, (M2, K2)), _codes(g, (N2, K2))
    sA2 = g.integers(118, 137, (M2, K2 // 32), dtype=np.uint8)
    sB2 = g.integers(118, 137, (N2, K2 // 32), dtype=np.uint8)
    offs2 = np.array([256, 256, 640, 896], np.int32)
    C2 = mxq.mx_grouped_gemm_k_mfma(_dev(A2), _dev(oracle.scales_to_mfma(sA2)), _dev(B2),
                                    _dev(oracle.scales_to_mfma(sB2)), _dev(offs2), out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref2, abs2 = oracle.mx_grouped_gemm_k(A2, sA2, B2, sB2, offs2, sa_strides=(K2 // 32, 1),
                                          sb_strides=(K2 // 32, 1), threads=THREADS, with_abs=True)
    for e in range(4):
        kk = int(offs2[e] - (offs2[e - 1] if e else 0))
        _assert_close(C2[e], ref2[e], abs2[e], max(kk, 1), out_dtype, f"contraction group {e}, mfma layout")
    assert torch.all(C2[1] == 0)


def test_grouped_cast_feeds_both_grouped_gemms():
    """End to end on the device with no rearrangement in between: the grouped
    cast in the matrix-core layout feeds the row-grouped forward (q_row,
    s_row) and the contraction-grouped weight gradient (q_col, s_col), and
    both equal the strided-view path on the plain cast bit for bit and the
    oracle within the bound."""
    require_gpu()
    M, K, N, E = 2048, 512, 256, 6
    say(f"grouped cast (mfma layout) -> grouped contractions, M={M} K={K} N={N}")
    xb = synth.normal_bf16(M, K, 31)
    dyb = synth.normal_bf16(M, N, 32)
    offs = np.array([256, 256, 768, 1280, 1536, 1920], np.int32)      # an empty group, a 128-row tail
    od = _dev(offs)
    xd, dyd = bf16_to_dev(xb), bf16_to_dev(dyb)
    qx = mxq.mx_quantize_grouped(xd, od, scale_layout="mfma")
    qd = mxq.mx_quantize_grouped(dyd, od, scale_layout="mfma")
    px = mxq.mx_quantize_grouped(xd, od)
    pd = mxq.mx_quantize_grouped(dyd, od)
    g = np.random.default_rng(12)
    W = np.stack([_codes(g, (N, K)) for _ in range(E)])
    sW = g.integers(118, 137, (E, N, K // 32), dtype=np.uint8)
    sWm = np.stack([oracle.scales_to_mfma(sW[e]) for e in range(E)])
    Y = mxq.mx_grouped_gemm_rows_mfma(qx[0], qx[1], _dev(W), _dev(sWm), od)
    Yp = mxq.mx_grouped_gemm_rows(px[0], px[1], _dev(W), _dev(sW), od)
    dW = mxq.mx_grouped_gemm_k_mfma(qx[2], qx[3], qd[2], qd[3], od)         # [E, K, N]
    dWp = mxq.mx_grouped_gemm_k(px[2], px[3].t(), pd[2], pd[3].t(), od)
    torch.cuda.synchronize()
    assert torch.equal(Y, Yp) and torch.equal(dW, dWp)
    hx = [host(t) for t in px]
    hd = [host(t) for t in pd]
    ref, absC = oracle.mx_grouped_gemm_rows(hx[0], hx[1], W, sW, offs, sa_strides=(K // 32, 1),
                                            sb_strides=(K // 32, 1), threads=THREADS, with_abs=True)
    _assert_close(Y, ref, absC, K, torch.float32, "forward")
    ref2, abs2 = oracle.mx_grouped_gemm_k(hx[2], hx[3], hd[2], hd[3], offs, sa_strides=(1, K),
                                          sb_strides=(1, N), threads=THREADS, with_abs=True)
    for e in range(E):
        kk = int(offs[e] - (offs[e - 1] if e else 0))
        _assert_close(dW[e], ref2[e], abs2[e], max(kk, 1), torch.float32, f"weight gradient group {e}")


def test_unaligned_output_rows_take_the_strided_kernel():
    """An output pitch that leaves C rows off 16-byte boundaries cannot take
    the 16-byte stores of the pipelined form; the first kernel reads the
    matrix-core layout then.  Same results as the aligned call."""
    require_gpu()
    say("mx_gemm_nt_mfma with an odd output pitch")
    g = np.random.default_rng(13)
    M, N, K = 256, 384, 512
    A, B = _codes(g, (M, K)), _codes(g, (N, K))
    sA = g.integers(118, 137, (M, K // 32), dtype=np.uint8)
    sB = g.integers(118, 137, (N, K // 32), dtype=np.uint8)
    dA, dB = _dev(A), _dev(B)
    msA, msB = _dev(oracle.scales_to_mfma(sA)), _dev(oracle.scales_to_mfma(sB))
    wide = torch.full((M, N + 3), -1.0, dtype=torch.float32, device=DEV)
    mxq.mx_gemm_nt_mfma(dA, msA, dB, msB, out=wide[:, :N])
    C = mxq.mx_gemm_nt_mfma(dA, msA, dB, msB)
    torch.cuda.synchronize()
    ref, absC = oracle.mx_gemm_nt(A, sA, B, sB, sa_strides=(K // 32, 1), sb_strides=(K // 32, 1),
                                  threads=THREADS, with_abs=True)
    _assert_close(wide[:, :N], ref, absC, K, torch.float32, "odd pitch")
    _assert_close(C, ref, absC, K, torch.float32, "aligned")
    assert torch.all(wide[:, N:] == -1.0)


def test_ragged_tiles_of_the_large_tile_form():
    """M and N that are odd multiples of 128 leave the 256 x 256 tiles ragged
    at the bottom and the right (rows wrap onto valid rows for the loads,
    their results are not stored); the contraction grouped over K uses the
    same tiles."""
    require_gpu()
    say("mx_gemm_nt_mfma with ragged 256 x 256 tiles")
    g = np.random.default_rng(14)
    M, N, K = 384, 640, 384
    A, B = _codes(g, (M, K)), _codes(g, (N, K))
    sA = g.integers(118, 137, (M, K // 32), dtype=np.uint8)
    sB = g.integers(118, 137, (N, K // 32), dtype=np.uint8)
    out = torch.full((M, N + 8), 5.0, dtype=torch.bfloat16, device=DEV)
    mxq.mx_gemm_nt_mfma(_dev(A), _dev(oracle.scales_to_mfma(sA)), _dev(B), _dev(oracle.scales_to_mfma(sB)),
                        out=out[:, :N])
    offs = np.array([128, 384], np.int32)
    Cg = mxq.mx_grouped_gemm_k_mfma(_dev(A), _dev(oracle.scales_to_mfma(sA)), _dev(B),
                                    _dev(oracle.scales_to_mfma(sB)), _dev(offs))
    torch.cuda.synchronize()
    ref, absC = oracle.mx_gemm_nt(A, sA, B, sB, sa_strides=(K // 32, 1), sb_strides=(K // 32, 1),
                                  threads=THREADS, with_abs=True)
    _assert_close(out[:, :N], ref, absC, K, torch.bfloat16, "ragged tiles")
    assert torch.all(out[:, N:] == 5.0)
    refg, absg = oracle.mx_grouped_gemm_k(A, sA, B, sB, offs, sa_strides=(K // 32, 1), sb_strides=(K // 32, 1),
                                          threads=THREADS, with_abs=True)
    for e in range(2):
        _assert_close(Cg[e], refg[e], absg[e], 256 if e else 128, torch.float32, f"ragged group {e}")


def test_rejections():
    dev = require_gpu()
    say("mfma-layout rejections")
    a = torch.zeros((128, 128), dtype=torch.uint8, device=dev)
    s = torch.zeros((512,), dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError):
        mxq.mx_gemm_nt_mfma(a, s[:256], a, s)
    with pytest.raises(mxq.MXError) as ei:
        big = torch.zeros((520,), dtype=torch.uint8, device=dev)
        mxq.mx_gemm_nt_mfma(a, big[4:516], a, s)       # scales not 16-byte aligned
    assert ei.value.status == 7
    with pytest.raises(ValueError):
        mxq.mx_quantize_2d_dual(torch.zeros((128, 128), dtype=torch.bfloat16, device=dev), scale_layout="swizzled")


# ---------------------------------------------------------------- full sizes

def test_full_size_grouped_cast_and_contractions_in_the_matrix_core_layout():
    """The workloads the bench times in the matrix-core layout: the grouped
    cast of bf16 [16384, 5120] (64 groups), its outputs consumed by the
    row-grouped forward (64 experts of [2048, 5120]) and the contraction-
    grouped weight gradient (dY [2048, 16384] over the token groups).  The
    cast's scale bytes of sampled rows and slabs equal the oracle's, placed
    by the layout's index function; sampled output rows of every few groups
    meet the oracle's contraction within the bound."""
    dev = require_gpu()
    say("full size: grouped cast [16384, 5120] (mfma layout) -> grouped contractions, sampled")
    xb, offs = synth.grouped()
    M, K = xb.shape
    N, E = 2048, len(offs)
    od = _dev(offs)
    q_row, s_row, q_col, s_col = mxq.mx_quantize_grouped(bf16_to_dev(xb), od, scale_layout="mfma")
    torch.cuda.synchronize()
    hs_row, hs_col = host(s_row), host(s_col)
    # scales of sampled rows (rowwise) and slabs (colwise) against the oracle
    rows = np.array([0, 1, 4095, 8191, 12287, 12288, M - 1])
    _, sr = oracle.mxfp8_rowwise(np.ascontiguousarray(xb[rows]), threads=THREADS)
    r, b = np.meshgrid(rows, np.arange(K // 32), indexing="ij")
    assert np.array_equal(hs_row[oracle.mfma_scale_index(r, b, K // 32)], sr)
    tail = int(offs[-1]) // 32
    for i in (0, 200, tail - 1, tail, M // 32 - 1):
        _, sc = oracle.mxfp8_colwise(np.ascontiguousarray(xb[32 * i:32 * i + 32]), threads=THREADS)
        want = sc[0] if i < tail else np.zeros_like(sc[0])
        n = np.arange(K)
        assert np.array_equal(hs_col[oracle.mfma_scale_index(n, np.full_like(n, i), M // 32)], want), f"slab {i}"
    hq_row, hq_col = host(q_row), host(q_col)
    sr_plain = oracle.scales_from_mfma(hs_row, M, K // 32)          # [M, K/32]
    sc_plain = oracle.scales_from_mfma(hs_col, K, M // 32)          # [K, M/32]

    g = np.random.default_rng(15)
    W = np.stack([_codes(g, (N, K)) for _ in range(E)])
    sW = g.integers(118, 137, (E, N, K // 32), dtype=np.uint8)
    sWm = np.stack([oracle.scales_to_mfma(sW[e]) for e in range(E)])
    Y = host(mxq.mx_grouped_gemm_rows_mfma(q_row, s_row, _dev(W), _dev(sWm), od))
    lo = 0
    for e, hi in enumerate(offs):
        if hi > lo and e % 7 == 0:
            for rr in (int(lo), int(hi) - 1):
                ref, absC = oracle.mx_gemm_nt(hq_row[rr:rr + 1], sr_plain[rr:rr + 1], W[e], sW[e],
                                              sa_strides=(K // 32, 1), sb_strides=(K // 32, 1), threads=THREADS,
                                              with_abs=True)
                _assert_close(torch.from_numpy(Y[rr:rr + 1]), ref, absC, K, torch.float32, f"forward row {rr}")
        lo = hi
    assert np.all(Y[int(offs[-1]):] == 0)
    del Y, W

    dY = _codes(g, (N, M))
    sdY = g.integers(118, 137, (N, M // 32), dtype=np.uint8)
    dW = mxq.mx_grouped_gemm_k_mfma(q_col, s_col, _dev(dY), _dev(oracle.scales_to_mfma(sdY)), od,
                                    out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    krows = [0, 2047, K - 1]
    lo = 0
    for e, hi in enumerate(offs):
        if e % 9 == 0 or e == E - 1:
            got = dW[e, krows]
            ref = np.zeros((len(krows), N))
            absC = np.zeros((len(krows), N))
            if hi > lo:
                for j, kr in enumerate(krows):
                    r1, a1 = oracle.mx_gemm_nt(hq_col[kr:kr + 1], sc_plain[kr:kr + 1], dY, sdY,
                                               sa_strides=(M // 32, 1), sb_strides=(M // 32, 1),
                                               k0=int(lo), k1=int(hi), with_abs=True)
                    ref[j], absC[j] = r1[0], a1[0]
            _assert_close(got, ref, absC, max(int(hi - lo), 1), torch.bfloat16, f"weight gradient group {e}")
        lo = hi


def test_full_size_dense_contraction_sampled():
    """The dense [8192]^3 product the bench times, in the matrix-core layout:
    sampled rows (first, last, and rows of different 256-row tiles and wave
    quarters) against the oracle."""
    require_gpu()
    say("full size: dense [8192]^3 contraction (mfma layout), sampled rows")
    D = 8192
    g = np.random.default_rng(16)
    A, B = _codes(g, (D, D)), _codes(g, (D, D))
    sA = g.integers(118, 137, (D, D // 32), dtype=np.uint8)
    sB = g.integers(118, 137, (D, D // 32), dtype=np.uint8)
    C = mxq.mx_gemm_nt_mfma(_dev(A), _dev(oracle.scales_to_mfma(sA)), _dev(B), _dev(oracle.scales_to_mfma(sB)),
                            out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for rr in (0, 77, 4096 + 200, D - 1):
        ref, absC = oracle.mx_gemm_nt(A[rr:rr + 1], sA[rr:rr + 1], B, sB, sa_strides=(D // 32, 1),
                                      sb_strides=(D // 32, 1), threads=THREADS, with_abs=True)
        _assert_close(C[rr:rr + 1], ref, absC, D, torch.bfloat16, f"dense row {rr}")


def test_pipeline_edge_cases():
    """The pipelined contraction at its boundaries: one 128-wide step
    (nothing prefetched), one-step groups, groups that are all empty (every
    output zero), a forward whose rows are all past the last offset, and
    three-stage row groups with exactly two steps."""
    require_gpu()
    say("pipelined contraction edge cases")
    g = np.random.default_rng(17)

    def mats(M, N, K):
        A, B = _codes(g, (M, K)), _codes(g, (N, K))
        sA = g.integers(118, 137, (M, K // 32), dtype=np.uint8)
        sB = g.integers(118, 137, (N, K // 32), dtype=np.uint8)
        return A, B, sA, sB

    # one step, fp32 and bf16
    A, B, sA, sB = mats(256, 384, 128)
    for od in (torch.float32, torch.bfloat16):
        C = mxq.mx_gemm_nt_mfma(_dev(A), _dev(oracle.scales_to_mfma(sA)), _dev(B), _dev(oracle.scales_to_mfma(sB)),
                                out_dtype=od)
        torch.cuda.synchronize()
        ref, absC = oracle.mx_gemm_nt(A, sA, B, sB, sa_strides=(4, 1), sb_strides=(4, 1), threads=THREADS,
                                      with_abs=True)
        _assert_close(C, ref, absC, 128, od, f"K = 128 {od}")

    # contraction groups of one step each, and all-empty groups
    A, B, sA, sB = mats(256, 256, 512)
    mA, mB = _dev(oracle.scales_to_mfma(sA)), _dev(oracle.scales_to_mfma(sB))
    offs = np.array([128, 256, 384, 512], np.int32)
    C = mxq.mx_grouped_gemm_k_mfma(_dev(A), mA, _dev(B), mB, _dev(offs))
    torch.cuda.synchronize()
    ref, absC = oracle.mx_grouped_gemm_k(A, sA, B, sB, offs, sa_strides=(16, 1), sb_strides=(16, 1),
                                         threads=THREADS, with_abs=True)
    for e in range(4):
        _assert_close(C[e], ref[e], absC[e], 128, torch.float32, f"one-step group {e}")
    Z = mxq.mx_grouped_gemm_k_mfma(_dev(A), mA, _dev(B), mB, _dev(np.zeros(3, np.int32)))
    torch.cuda.synchronize()
    assert torch.all(Z == 0)

    # row groups: every row past the last offset, then two-step rows
    E = 3
    Bw = np.stack([_codes(g, (256, 256)) for _ in range(E)])
    sBw = g.integers(118, 137, (E, 256, 8), dtype=np.uint8)
    sBm = _dev(np.stack([oracle.scales_to_mfma(sBw[e]) for e in range(E)]))
    A2 = _codes(g, (384, 256))
    sA2 = g.integers(118, 137, (384, 8), dtype=np.uint8)
    out = torch.full((384, 256), 3.0, dtype=torch.float32, device=DEV)
    mxq.mx_grouped_gemm_rows_mfma(_dev(A2), _dev(oracle.scales_to_mfma(sA2)), _dev(Bw), sBm,
                                  _dev(np.zeros(E, np.int32)), out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    offs2 = np.array([128, 128, 384], np.int32)
    Y = mxq.mx_grouped_gemm_rows_mfma(_dev(A2), _dev(oracle.scales_to_mfma(sA2)), _dev(Bw), sBm, _dev(offs2))
    torch.cuda.synchronize()
    ref, absC = oracle.mx_grouped_gemm_rows(A2, sA2, Bw, sBw, offs2, sa_strides=(8, 1), sb_strides=(8, 1),
                                            threads=THREADS, with_abs=True)
    _assert_close(Y, ref, absC, 256, torch.float32, "two-step row groups")


@pytest.mark.parametrize("R,kb,view", [(64, 4, "rows"), (256, 160, "rows"), (384, 12, "transposed"),
                                       (128, 8, "pitched")])
def test_scale_conversions(R, kb, view):
    """mx_scales_to_mfma / mx_scales_from_mfma: the oracle's index function,
    from and to row-major, transposed (the colwise cast's s_col read as its
    operand's scales) and pitched views."""
    dev = require_gpu()
    say(f"scale layout conversion R={R} kb={kb} view={view}")
    g = np.random.default_rng(R + kb)
    S = g.integers(0, 256, (R, kb), dtype=np.uint8)
    want = oracle.scales_to_mfma(S)
    if view == "rows":
        src = _dev(S)
    elif view == "transposed":
        src = _dev(np.ascontiguousarray(S.T)).t()
    else:
        wide = torch.zeros((R, kb + 12), dtype=torch.uint8, device=dev)
        wide[:, :kb] = _dev(S)
        src = wide[:, :kb]
    flat = mxq.scales_to_mfma(src)
    torch.cuda.synchronize()
    assert np.array_equal(host(flat), want)
    back = torch.full((kb, R), 0xEE, dtype=torch.uint8, device=dev).t() if view == "transposed" else None
    back = mxq.scales_from_mfma(flat, R, kb, out=back)
    torch.cuda.synchronize()
    assert np.array_equal(host(back.contiguous()), S)


def test_converted_plain_scales_feed_the_fast_contraction():
    """The plain-layout cast, its scales converted, the pipelined contraction:
    the same result as the strided-view contraction on the plain scales."""
    dev = require_gpu()
    say("plain cast -> converted scales -> pipelined contraction")
    M, K, N = 512, 768, 256
    xd = bf16_to_dev(synth.normal_bf16(M, K, 51))
    q_row, s_row, q_col, s_col = mxq.mx_quantize_2d_dual(xd)
    g = np.random.default_rng(52)
    W = _codes(g, (N, K))
    sW = g.integers(118, 137, (N, K // 32), dtype=np.uint8)
    C1 = mxq.mx_gemm_nt(q_row, s_row, _dev(W), _dev(sW))
    C2 = mxq.mx_gemm_nt_mfma(q_row, mxq.scales_to_mfma(s_row), _dev(W), mxq.scales_to_mfma(_dev(sW)))
    # weight gradient operand: q_col [K, M] with s_col [M/32, K] read transposed
    G1 = mxq.mx_gemm_nt(q_col, s_col.t(), q_col, s_col.t())
    G2 = mxq.mx_gemm_nt_mfma(q_col, mxq.scales_to_mfma(s_col.t()), q_col, mxq.scales_to_mfma(s_col.t()))
    torch.cuda.synchronize()
    assert torch.equal(C1, C2) and torch.equal(G1, G2)
