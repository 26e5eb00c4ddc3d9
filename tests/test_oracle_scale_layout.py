"""Pins for the matrix-core scale layout (the consumer layout in which the
cast can emit its E8M0 scales and the MXFP8 contraction reads them; pages:
pytorch/ao PR #4995, whose kernel emits the consumer's scale layout directly
so that no rearrangement runs in between).  The layout itself is this
project's own; these tests pin that the oracle's index function is a bijection
with the stated lane and byte assignment, worked by hand."""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("R,kb", [(64, 4), (128, 8), (192, 12), (256, 160)])
def test_is_a_bijection_and_inverts(R, kb):
    r, b = np.meshgrid(np.arange(R), np.arange(kb), indexing="ij")
    idx = oracle.mfma_scale_index(r, b, kb)
    assert np.array_equal(np.sort(idx.reshape(-1)), np.arange(R * kb))
    S = np.random.default_rng(R + kb).integers(0, 256, (R, kb), dtype=np.uint8)
    assert np.array_equal(oracle.scales_from_mfma(oracle.scales_to_mfma(S), R, kb), S)


def test_hand_worked_positions():
    kb = 8                                    # two 128-wide steps per row
    # row 0, block 0: group 0, step 0, lane 0, byte 0
    assert oracle.mfma_scale_index(0, 0, kb) == 0
    # row 16, block 0: lane 0 again, byte 1 (second 16-row sub-tile)
    assert oracle.mfma_scale_index(16, 0, kb) == 1
    # row 5, block 2: lane 2 * 16 + 5 = 37, byte 0 -> 148
    assert oracle.mfma_scale_index(5, 2, kb) == 148
    # row 63, block 7: step 1 (256 bytes in), lane 3 * 16 + 15 = 63, byte 3
    assert oracle.mfma_scale_index(63, 7, kb) == 256 + 63 * 4 + 3
    # row 64, block 0: the second 64-row group starts after kb / 4 steps of 256 bytes
    assert oracle.mfma_scale_index(64, 0, kb) == 2 * 256


def test_a_wave_reads_one_dword_per_lane():
    """For each 64-row group g and step s the 256 bytes at (g * kb/4 + s) * 256
    are exactly the scales of rows 64 g .. 64 g + 63 and blocks 4 s .. 4 s + 3,
    lane L's dword holding rows 64 g + 16 q + L % 16 (q = 0..3) of block
    4 s + L // 16."""
    R, kb = 128, 8
    S = np.arange(R * kb, dtype=np.int64).reshape(R, kb) % 251
    flat = oracle.scales_to_mfma(S.astype(np.uint8)).reshape(R // 64, kb // 4, 64, 4)
    for g in range(R // 64):
        for s in range(kb // 4):
            for L in range(64):
                want = [S[64 * g + 16 * q + L % 16, 4 * s + L // 16] for q in range(4)]
                assert list(flat[g, s, L]) == want
