"""GPU parity at the extremes of the accepted shapes: the dual-axis cast at
its largest extent along either axis (2^24 columns, 2^24 rows), MX9 over more
than 2^31 elements, and MX9 along axis 0 with element rows longer than 2^26
bytes (the axis pack's general load route).  Inputs are drawn on the device
with a seeded generator; sampled tiles, rows or columns are copied back and
compared with the CPU oracle byte for byte (every block the cast and MX9 form
is local to its tile, row or column, so the oracle sees exactly the bytes
the kernel saw).  Operations: pytorch/ao PR #4995 (the fused dual-axis cast)
and AMD-AGI/ALTO PR #33 (MX9 pack/unpack, the axis argument)."""
import numpy as np
import pytest
import torch

import mx9_dual_axis_amd as mxq
import oracle
from helpers import host, require_gpu, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _normal(shape, seed, dtype):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV, dtype=torch.float32).to(dtype)


def _specials(x, points):
    """Plant Inf, -Inf, NaN and a subnormal at the given (row, col) points."""
    vals = [float("inf"), float("-inf"), float("nan"), 2.0 ** -130]
    for k, (r, c) in enumerate(points):
        x[r, c] = vals[k % len(vals)]


def _check_dual_tile(x, outs, r0, c0, tag):
    """Compare the 128 x 128 tile at (r0, c0) of every cast output with the oracle."""
    q_row, s_row, q_col, s_col = outs
    xt = host(x[r0:r0 + 128, c0:c0 + 128].contiguous())
    wq_row, ws_row, wq_col, ws_col = oracle.mxfp8_dual(xt)
    got = (host(q_row[r0:r0 + 128, c0:c0 + 128]), host(s_row[r0:r0 + 128, c0 // 32:c0 // 32 + 4]),
           host(q_col[c0:c0 + 128, r0:r0 + 128]), host(s_col[r0 // 32:r0 // 32 + 4, c0:c0 + 128]))
    for name, g, w in zip(("q_row", "s_row", "q_col", "s_col"), got, (wq_row, ws_row, wq_col, ws_col)):
        bad = np.count_nonzero(g != w)
        assert bad == 0, f"{tag} tile ({r0}, {c0}) {name}: {bad} bytes differ"


@pytest.mark.parametrize("M,N", [(128, 1 << 24), (1 << 24, 128)])
def test_dual_axis_longest_extents(M, N):
    require_gpu()
    say(f"extremes: dual-axis cast [{M}, {N}]")
    x = _normal((M, N), 7 + (M > N), torch.bfloat16)
    _specials(x, [(5, N - 3), (M - 1, N - 1), (M - 100, 77), (64, N // 2 + 1)])
    outs = mxq.mx_quantize_2d_dual(x)
    torch.cuda.synchronize()
    tiles_m, tiles_n = M // 128, N // 128
    g = np.random.default_rng(M + N)
    picks = {(0, 0), (tiles_m - 1, tiles_n - 1), ((M - 100) // 128, 0), (0, (N // 2 + 1) // 128)}
    picks |= {(int(a), int(b)) for a, b in zip(g.integers(0, tiles_m, 6), g.integers(0, tiles_n, 6))}
    for tm, tn in sorted(picks):
        _check_dual_tile(x, outs, 128 * tm, 128 * tn, f"[{M}, {N}]")


def test_mx9_over_two_to_the_31_elements():
    require_gpu()
    rows, cols = 32776, 65552                 # 2,148,532,352 elements (> 2^31)
    say(f"extremes: MX9 pack/unpack bf16 [{rows}, {cols}]")
    x = _normal((rows, cols), 11, torch.bfloat16)
    _specials(x, [(rows - 1, cols - 1), (rows - 2, cols - 17), (0, 5), (rows // 2, cols - 16)])
    q, e, p = mxq.mx9_pack(x)
    y = mxq.mx9_unpack(q, e, p, rows, cols, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    bpr = cols // 16
    g = np.random.default_rng(12)
    sample = sorted({0, rows // 2, rows - 2, rows - 1} | {int(r) for r in g.integers(0, rows, 4)})
    for r in sample:
        xr = host(x[r:r + 1])
        wq, we, wp = oracle.mx9_pack(xr)
        blk = slice(r * bpr, (r + 1) * bpr)
        assert np.array_equal(host(q[blk]), wq), f"row {r}: q"
        assert np.array_equal(host(e[blk]), we.reshape(-1)), f"row {r}: max_exp"
        assert np.array_equal(host(p[blk]).reshape(-1), wp.reshape(-1)), f"row {r}: prime"
        wy = oracle.mx9_unpack(wq, we, wp, 1, cols, "bf16")
        assert np.array_equal(host(y[r:r + 1]), wy), f"row {r}: unpack"


def test_mx9_axis0_rows_longer_than_2_to_the_26_bytes():
    require_gpu()
    length, inner = 40, (1 << 24) + 2         # fp32 rows of 64 MiB + 8 bytes; 3 blocks along axis 0, the last ragged
    say(f"extremes: MX9 along axis 0, fp32 [{length}, {inner}]")
    x = _normal((length, inner), 13, torch.float32)
    _specials(x, [(39, inner - 1), (3, inner - 2), (17, 0), (32, 12345)])
    q, e, p = mxq.mx9_pack_axis(x, 0)
    y = mxq.mx9_unpack_axis(q, e, p, (length, inner), 0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    nbl = (length + 15) // 16
    g = np.random.default_rng(14)
    cols = np.array(sorted({0, 1, 12345, inner - 2, inner - 1} | {int(c) for c in g.integers(0, inner, 6)}))
    xs = host(x[:, torch.from_numpy(cols).to(DEV)].contiguous())
    wq, we, wp = oracle.mx9_pack_axis(xs, 0)
    idx = (cols[:, None] * nbl + np.arange(nbl)[None, :]).reshape(-1)
    it = torch.from_numpy(idx).to(DEV)
    assert np.array_equal(host(q[it]), wq), "q"
    assert np.array_equal(host(e[it]).reshape(-1), we.reshape(-1)), "max_exp"
    assert np.array_equal(host(p[it]).reshape(-1), wp.reshape(-1)), "prime"
    wy = oracle.mx9_unpack_axis(wq, we, wp, xs.shape, 0, "fp32")
    got = host(y[:, torch.from_numpy(cols).to(DEV)].contiguous())
    assert np.array_equal(got.view(np.uint32), wy.view(np.uint32)), "unpack"
