"""Pins for the oracle's MXFP8 block-scaled contraction (AMD-AGI/ALTO PR #31,
"Add MXFP8 grouped GEMM (E4M3) for routed-expert MoE training": E4M3
operands with E8M0 scales per 32 elements of the contraction, grouped by
1-D cumulative offsets).

Sources of truth other than the oracle's own arithmetic:
  * torch's float8_e4m3fn decoder and numpy's float64 matmul (a library
    decode + a library contraction of the dequantized operands);
  * closed forms: all-ones operands, one-hot rows, per-block powers of two;
  * exact rationals (fractions.Fraction) on a small case;
  * linearity: the contraction-grouped form summed over its groups equals the
    contraction over the covered range; the row-grouped form equals per-group
    dense products, with the tail zero.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

DEC = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _codes(g, shape):
    c = g.integers(0, 256, shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38          # no NaN codes
    return c


def _deq(codes, scales, rs, bs):
    """Dequantized operand [R, K] from codes and a strided scale view, with the library decoder."""
    R, K = codes.shape
    r = np.arange(R)[:, None]
    b = (np.arange(K) // 32)[None, :]
    s = scales.reshape(-1)[r * rs + b * bs].astype(np.float64)
    return DEC[codes] * np.exp2(s - 127)


@pytest.mark.parametrize("layout", ["row-major scales", "transposed scales"])
def test_matches_library_decode_and_matmul(layout):
    g = np.random.default_rng(1)
    M, N, K = 48, 40, 256
    A, B = _codes(g, (M, K)), _codes(g, (N, K))
    if layout == "row-major scales":
        sA, sB = g.integers(110, 140, (M, K // 32), dtype=np.uint8), g.integers(110, 140, (N, K // 32), dtype=np.uint8)
        sa, sb = (K // 32, 1), (K // 32, 1)
    else:   # the colwise cast's layout: [K/32, rows]
        sA, sB = g.integers(110, 140, (K // 32, M), dtype=np.uint8), g.integers(110, 140, (K // 32, N), dtype=np.uint8)
        sa, sb = (1, M), (1, N)
    C = oracle.mx_gemm_nt(A, sA, B, sB, sa_strides=sa, sb_strides=sb, threads=3)
    want = _deq(A, sA, *sa) @ _deq(B, sB, *sb).T
    np.testing.assert_allclose(C, want, rtol=1e-12, atol=1e-300)


def test_closed_forms():
    K = 128
    ones = np.full((4, K), 0x38, np.uint8)                     # E4M3 1.0
    s = np.full((4, K // 32), 127, np.uint8)
    C = oracle.mx_gemm_nt(ones, s, ones, s, sa_strides=(K // 32, 1), sb_strides=(K // 32, 1))
    assert np.all(C == K)
    # per-block powers of two: block b of A row m scaled by 2^(m + b), of B row n by 2^(-n)
    sA = np.array([[127 + m + b for b in range(K // 32)] for m in range(4)], np.uint8)
    sB = np.array([[127 - n] * (K // 32) for n in range(4)], np.uint8)
    C = oracle.mx_gemm_nt(ones, sA, ones, sB, sa_strides=(K // 32, 1), sb_strides=(K // 32, 1))
    for m in range(4):
        for n in range(4):
            assert C[m, n] == sum(32 * 2.0 ** (m + b - n) for b in range(K // 32))
    # a one-hot row picks one contraction index: C[m][n] = dec(B[n][k_m])
    g = np.random.default_rng(2)
    B = _codes(g, (6, K))
    A = np.zeros((4, K), np.uint8)
    ks = [0, 31, 32, 127]
    for m, k in enumerate(ks):
        A[m, k] = 0x38
    C = oracle.mx_gemm_nt(A, np.full((4, 4), 127, np.uint8), B, np.full((6, 4), 127, np.uint8),
                          sa_strides=(4, 1), sb_strides=(4, 1))
    for m, k in enumerate(ks):
        np.testing.assert_array_equal(C[m], DEC[B[:, k]])


def test_exact_rationals_small():
    g = np.random.default_rng(3)
    M, N, K = 3, 2, 64
    A, B = _codes(g, (M, K)), _codes(g, (N, K))
    sA = g.integers(120, 134, (M, 2), dtype=np.uint8)
    sB = g.integers(120, 134, (N, 2), dtype=np.uint8)
    C = oracle.mx_gemm_nt(A, sA, B, sB, sa_strides=(2, 1), sb_strides=(2, 1))
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for k in range(K):
                a = Fraction(DEC[A[m, k]]) * Fraction(2) ** (int(sA[m, k // 32]) - 127)
                b = Fraction(DEC[B[n, k]]) * Fraction(2) ** (int(sB[n, k // 32]) - 127)
                tot += a * b
            # binary64 accumulation in k order: within K * 2^-53 of the exact sum of magnitudes
            mag = sum(abs(Fraction(DEC[A[m, k]]) * Fraction(DEC[B[n, k]])) * Fraction(2) ** (int(sA[m, k // 32]) + int(sB[n, k // 32]) - 254) for k in range(K))
            assert abs(Fraction(C[m, n]) - tot) <= mag * K * Fraction(1, 2 ** 53)


def test_nan_codes_and_nan_scales_propagate():
    K = 64
    A = np.full((2, K), 0x38, np.uint8)
    B = np.full((2, K), 0x38, np.uint8)
    A[0, 5] = 0x7F
    sA = np.full((2, 2), 127, np.uint8)
    sB = np.full((2, 2), 127, np.uint8)
    sB[1, 1] = 255
    C = oracle.mx_gemm_nt(A, sA, B, sB, sa_strides=(2, 1), sb_strides=(2, 1))
    assert np.isnan(C[0]).all() and np.isnan(C[1, 1]) and C[1, 0] == K


def test_abs_sum_is_the_contraction_of_magnitudes():
    g = np.random.default_rng(4)
    A, B = _codes(g, (8, 96)), _codes(g, (5, 96))
    s1, s2 = np.full((8, 3), 127, np.uint8), np.full((5, 3), 125, np.uint8)
    _, absC = oracle.mx_gemm_nt(A, s1, B, s2, sa_strides=(3, 1), sb_strides=(3, 1), with_abs=True)
    np.testing.assert_allclose(absC, np.abs(_deq(A, s1, 3, 1)) @ np.abs(_deq(B, s2, 3, 1)).T, rtol=1e-12)


def test_row_groups_equal_per_group_products_and_zero_tail():
    g = np.random.default_rng(5)
    M, N, K, E = 512, 24, 128, 4
    A = _codes(g, (M, K))
    sA = g.integers(118, 136, (M, K // 32), dtype=np.uint8)
    B = np.stack([_codes(g, (N, K)) for _ in range(E)])
    sB = g.integers(118, 136, (E, K // 32, N), dtype=np.uint8)     # colwise-cast layout per expert
    offs = np.array([128, 128, 384, 384], np.int32)                  # group 1 and group 3 empty; tail 128 rows
    C = oracle.mx_grouped_gemm_rows(A, sA, B, sB, offs, sa_strides=(K // 32, 1), sb_strides=(1, N))
    lo = 0
    for e, hi in enumerate(offs):
        want = _deq(A[lo:hi], sA[lo:hi], K // 32, 1) @ _deq(B[e], sB[e], 1, N).T
        np.testing.assert_allclose(C[lo:hi], want, rtol=1e-12, atol=1e-300)
        lo = hi
    assert np.all(C[offs[-1]:] == 0)


def test_contraction_groups_sum_to_the_covered_contraction():
    g = np.random.default_rng(6)
    M, N, K = 16, 12, 640
    A, B = _codes(g, (M, K)), _codes(g, (N, K))
    sA = g.integers(120, 134, (K // 32, M), dtype=np.uint8)          # colwise-cast layouts
    sB = g.integers(120, 134, (K // 32, N), dtype=np.uint8)
    offs = np.array([128, 128, 384, 512], np.int32)                   # one empty group, tail 128
    Cg = oracle.mx_grouped_gemm_k(A, sA, B, sB, offs, sa_strides=(1, M), sb_strides=(1, N))
    assert Cg.shape == (4, M, N) and np.all(Cg[1] == 0)
    full = oracle.mx_gemm_nt(A, sA, B, sB, sa_strides=(1, M), sb_strides=(1, N), k0=0, k1=512)
    np.testing.assert_allclose(Cg.sum(axis=0), full, rtol=1e-12, atol=1e-300)
    lo = 0
    for e, hi in enumerate(offs):
        want = _deq(A[:, lo:hi], sA[lo // 32:hi // 32], 1, M) @ _deq(B[:, lo:hi], sB[lo // 32:hi // 32], 1, N).T
        np.testing.assert_allclose(Cg[e], want, rtol=1e-12, atol=1e-300)
        lo = hi
