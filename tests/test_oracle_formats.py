"""Pins for the oracle's number formats and its RCEIL scale rule.

Each test checks the oracle against something other than itself: torch's
own float8_e4m3fn codec (a third-party library), the constants the
pytorch/ao PR #4995 page prints, or a closed form derived on paper from the
E4M3 and bf16 definitions.
"""
import json
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "pages_constants.json")) as f:
        return json.load(f)


def _bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


# --- E4M3 codec -------------------------------------------------------------

def test_e4m3_decode_matches_torch_for_every_code():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        v = oracle.e4m3_value(c)
        if np.isnan(ref[c]):
            assert np.isnan(v), hex(c)
        else:
            assert v == ref[c] and np.signbit(v) == np.signbit(ref[c]), hex(c)
    # OCP E4M3FN: only 0x7F / 0xFF are NaN, max finite is 448
    assert [c for c in range(256) if np.isnan(oracle.e4m3_value(c))] == [0x7F, 0xFF]


def test_e4m3_max_is_page_constant(golden_dir):
    g = _golden(golden_dir)
    assert oracle.e4m3_value(0x7E) == g["e4m3_max_finite"]["value"]


def test_e4m3_encode_identity_on_all_finite_codes():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(oracle.e4m3_value(c)) == c, hex(c)


def test_e4m3_midpoints_tie_to_even_code():
    # midpoints between neighbouring finite codes (positive and negative)
    for c in range(0, 0x7E):
        lo, hi = oracle.e4m3_value(c), oracle.e4m3_value(c + 1)
        mid = (lo + hi) / 2  # exact in binary64
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == even, hex(c)
        assert oracle.e4m3_encode(-mid) == 0x80 | even, hex(c)


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(11)
    # bf16-representable values scaled into and around the E4M3 range
    bits = rng.integers(0, 1 << 16, 20000, dtype=np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    vals = vals[np.isfinite(vals)]
    scale = np.exp2(rng.integers(-140, 140, vals.size)).astype(np.float64)
    v = vals * scale
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0) & (np.abs(v) < 3e38)]
    # torch converts via fp32; restrict to values exact in fp32's normal range or tiny
    f32 = v.astype(np.float32).astype(np.float64)
    v = v[(f32 == v)]
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(x) for x in v], dtype=np.uint8)
    assert v.size > 5000
    np.testing.assert_array_equal(got, ref)


def test_e4m3_encode_saturates_and_keeps_sign():
    assert oracle.e4m3_encode(float("inf")) == 0x7E
    assert oracle.e4m3_encode(float("-inf")) == 0xFE
    assert oracle.e4m3_encode(1e30) == 0x7E
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(-1e-30) == 0x80
    assert oracle.e4m3_encode(0.0) == 0x00
    # 464 is the midpoint of 448 and the next (non-finite) step: satfinite gives 448
    assert oracle.e4m3_encode(464.0) == 0x7E


# --- RCEIL ------------------------------------------------------------------

def test_rceil_cutoff_is_the_pages_constant(golden_dir):
    g = _golden(golden_dir)
    cut = struct.unpack("<f", struct.pack("<I", int(g["mxfp8_rceil_cutoff_fp32_bits"]["value"], 16)))[0]
    assert Fraction(cut) == Fraction(448) / 2 ** 127
    assert oracle.rceil_byte(cut) == 0
    # bf16 0x0460 is the same value; the next bf16 up needs scale byte 1
    assert _bf16_value(0x0460) == cut
    assert oracle.rceil_byte(_bf16_value(0x0461)) == 1
    # the buggy cutoff 0x04E00000 = 448*2^-126 is one binade too high: it needs byte 1
    bug = struct.unpack("<f", struct.pack("<I", int(g["mxfp8_buggy_cutoff_fp32_bits"]["value"], 16)))[0]
    assert Fraction(bug) == Fraction(448) / 2 ** 126
    assert oracle.rceil_byte(bug) == 1


def _closed_form(bits: int) -> int:
    """Scale byte from a bf16 magnitude's fields: 448 = 1.75 * 2^8, so
    ceil(log2(A/448)) = (ea - 135) + [1 + ma/128 > 1.75] for normal A;
    biased by 127 and clamped to the E8M0 range."""
    ea, ma = (bits >> 7) & 0xFF, bits & 0x7F
    return min(max(ea - 8 + (1 if ma > 0x60 else 0), 0), 254)


def test_rceil_closed_form_all_finite_bf16_magnitudes():
    for bits in range(0, 0x7F80):          # every finite non-negative bf16
        assert oracle.rceil_byte(_bf16_value(bits)) == _closed_form(bits), hex(bits)
    assert _closed_form(0x7F7F) == 247


def test_rceil_minimality_and_bound():
    rng = np.random.default_rng(5)
    for bits in rng.integers(1, 0x7F80, 3000):
        a = Fraction(_bf16_value(int(bits)))
        b = oracle.rceil_byte(float(a))
        # scaled maximum fits E4M3's range ...
        assert a * Fraction(2) ** (127 - b) <= 448
        # ... and one step smaller would not (unless at the E8M0 floor)
        if b > 0:
            assert a * Fraction(2) ** (127 - (b - 1)) > 448
