"""Seeded synthetic inputs for the dual-axis MXFP8 cast and MX9.

This module only draws inputs.  It holds none of the quantization
arithmetic, and both the GPU path's tests/benchmark and the CPU oracle
consume the same host arrays it returns.

Every generator is numpy ``Generator(PCG64(seed))``.  Values are drawn in
fp32 (fp64 where a scale would leave fp32's range) and rounded to bf16 by
torch's CPU cast (round to nearest even).  bf16 arrays are returned as
``uint16`` bit patterns, fp32 arrays as ``float32``.

Workloads (the shapes the two pages' MoE activations and weights use):
  dual_small   bf16 [256, 256] N(0,1)                                  seed 1
  dual_mixed   bf16 [8192, 7168] rows scaled 2^U(-20,20), 1% x1000,
               2% of aligned 32x32 tiles zero                          seed 2
  grouped      bf16 [16384, 5120] N(0,1); 64 groups, sizes 128*multinomial(96),
               offs[-1] = 12288 < 16384                                seed 3
  mx9_weights  fp32 [4096, 14336]: 90% N(0,0.02), 10% t(3)*0.02; bf16 = RNE(fp32)
                                                                       seed 4
  stress       bf16 [32768, 8192] N(0,1); 0.5% of tiles x2^-130, 0.5% of tiles
               near bf16 max, Inf/NaN at rate 1e-6                     seed 5
"""
from __future__ import annotations

import numpy as np
import torch

BF16_POS_INF = 0x7F80
BF16_NEG_INF = 0xFF80
BF16_QNAN = 0x7FC0
BF16_NEG_NAN = 0xFFC1
BF16_MAX = 3.3895313892515355e38


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 (or fp64, via fp32) values to bf16, nearest even; uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _tile_mask(g: np.random.Generator, M: int, N: int, rate: float, t: int = 32) -> np.ndarray:
    return g.random((M // t, N // t)) < rate


def _expand(mask: np.ndarray, t: int = 32) -> np.ndarray:
    return np.repeat(np.repeat(mask, t, axis=0), t, axis=1)


def normal_bf16(M: int, N: int, seed: int) -> np.ndarray:
    g = rng(seed)
    return to_bf16_bits(g.standard_normal((M, N), dtype=np.float32))


def dual_small(seed: int = 1) -> np.ndarray:
    return normal_bf16(256, 256, seed)


def mixed_rows(M: int, N: int, seed: int) -> np.ndarray:
    """Rows scaled by 2^U(-20,20) times N(0,1); each element x1000 with
    probability 0.01; then 2% of the aligned 32x32 tiles set to zero, so
    both the rowwise and the colwise blocks see all-zero blocks."""
    g = rng(seed)
    x = g.standard_normal((M, N), dtype=np.float32)
    x *= np.exp2(g.uniform(-20.0, 20.0, (M, 1))).astype(np.float32)
    x[g.random((M, N), dtype=np.float32) < 0.01] *= 1000.0
    x[_expand(_tile_mask(g, M, N, 0.02))] = 0.0
    return to_bf16_bits(x)


def dual_mixed(seed: int = 2) -> np.ndarray:
    return mixed_rows(8192, 7168, seed)


def group_offsets(seed: int, groups: int = 64, covered: int = 12288, unit: int = 128) -> np.ndarray:
    """Cumulative int32 group ends: sizes are unit * multinomial(covered/unit,
    uniform over groups), so empty groups occur; offs[-1] == covered."""
    g = rng(seed + 1000)
    sizes = unit * g.multinomial(covered // unit, np.full(groups, 1.0 / groups))
    return np.cumsum(sizes).astype(np.int32)


def grouped(seed: int = 3):
    """(x bf16 [16384, 5120], offs int32 [64])."""
    return normal_bf16(16384, 5120, seed), group_offsets(seed)


def mx9_weights(rows: int, cols: int, seed: int, dtype: str = "fp32") -> np.ndarray:
    """90% N(0, 0.02), 10% Student-t(3) * 0.02.  dtype "bf16" returns the
    RNE-to-bf16 of the same fp32 draw (uint16 bits)."""
    g = rng(seed)
    x = g.standard_normal((rows, cols), dtype=np.float32) * np.float32(0.02)
    heavy = g.random((rows, cols), dtype=np.float32) < 0.1
    x[heavy] = (g.standard_t(3, int(heavy.sum())) * 0.02).astype(np.float32)
    if dtype == "fp32":
        return x
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(dtype)


def stress(M: int = 32768, N: int = 8192, seed: int = 5) -> np.ndarray:
    """N(0,1) with, in this order: 0.5% of aligned 32x32 tiles scaled by
    2^-130 (bf16 subnormal range); 0.5% of the other tiles replaced by
    sign * U(0.5, 1) * bf16-max; each element, with probability 1e-6,
    replaced by one of +Inf, -Inf, NaN 0x7FC0, NaN 0xFFC1."""
    g = rng(seed)
    x = g.standard_normal((M, N), dtype=np.float32)
    sub = _tile_mask(g, M, N, 0.005)
    big = _tile_mask(g, M, N, 0.005) & ~sub
    subm = _expand(sub)
    x[subm] = (x[subm].astype(np.float64) * 2.0 ** -130).astype(np.float32)
    del subm
    bigm = _expand(big)
    nb = int(bigm.sum())
    x[bigm] = (np.where(g.random(nb) < 0.5, -1.0, 1.0) * g.uniform(0.5, 1.0, nb) * BF16_MAX).astype(np.float32)
    del bigm
    xb = to_bf16_bits(x)
    del x
    flat = xb.reshape(-1)
    k = int(g.binomial(flat.size, 1e-6))
    pos = g.integers(0, flat.size, k)
    specials = np.array([BF16_POS_INF, BF16_NEG_INF, BF16_QNAN, BF16_NEG_NAN], np.uint16)
    flat[pos] = specials[g.integers(0, 4, k)]
    return xb


def special_matrix(M: int, N: int, seed: int) -> np.ndarray:
    """Small bf16 matrix (M, N multiples of 32) that plants every special
    case in both rowwise and colwise blocks: zero blocks, -0, Inf, -Inf,
    NaN of both signs, bf16 subnormals, values near bf16 max, the E8M0
    byte-0/1 cutoff and its neighbours, exact powers of two, and E4M3
    rounding midpoints, over an N(0,1) background with row scales."""
    g = rng(seed)
    x = g.standard_normal((M, N), dtype=np.float32)
    x *= np.exp2(g.uniform(-30.0, 30.0, (M, 1))).astype(np.float32)
    xb = to_bf16_bits(x)
    nbr, nbc = M // 32, N // 32
    kinds = g.integers(0, 12, (nbr, nbc))
    for i in range(nbr):
        for j in range(nbc):
            blk = xb[32 * i:32 * i + 32, 32 * j:32 * j + 32]
            k = kinds[i, j]
            r, c = g.integers(0, 32, 2)
            if k == 0:
                blk[:] = 0
                blk[r, :] = 0x8000                      # -0 row
            elif k == 1:
                blk[r, c] = BF16_POS_INF
            elif k == 2:
                blk[r, c] = BF16_NEG_INF
                blk[(r + 5) % 32, c] = BF16_POS_INF
            elif k == 3:
                blk[r, c] = BF16_QNAN if g.random() < 0.5 else BF16_NEG_NAN
            elif k == 4:                                 # subnormal-only block
                blk[:] = g.integers(0, 0x80, (32, 32)) | (g.integers(0, 2, (32, 32)) << 15)
            elif k == 5:                                 # cutoff neighbours
                vals = np.array([0x0460, 0x0461, 0x045F, 0x0040, 0x8460, 0x0001, 0x0000], np.uint16)
                blk[:] = vals[g.integers(0, vals.size, (32, 32))]
            elif k == 6:                                 # near bf16 max
                blk[:] = 0x7F00 + g.integers(0, 0x80, (32, 32)) | (g.integers(0, 2, (32, 32)) << 15)
            elif k == 7:                                 # exact powers of two and 448-ish maxima
                e = g.integers(1, 255, (32, 32))
                blk[:] = (e << 7) | (g.integers(0, 2, (32, 32)) << 15)
                blk[r, c] = 0x43E0                       # 448
            elif k == 8:                                 # mix of tiny and normal (underflow to 0)
                blk[:] = g.integers(0x0080, 0x0400, (32, 32))
                blk[r, c] = 0x7000
            # other kinds keep the random background
    return xb


def config(i: int):
    """Inputs of workload i (1..5) as named in the module docstring."""
    if i == 1:
        return {"name": "dual_small", "x": dual_small()}
    if i == 2:
        return {"name": "dual_mixed", "x": dual_mixed()}
    if i == 3:
        x, offs = grouped()
        return {"name": "grouped", "x": x, "offs": offs}
    if i == 4:
        return {"name": "mx9_weights", "x_fp32": mx9_weights(4096, 14336, 4, "fp32"),
                "x_bf16": mx9_weights(4096, 14336, 4, "bf16")}
    if i == 5:
        return {"name": "stress", "x": stress()}
    raise ValueError(i)
