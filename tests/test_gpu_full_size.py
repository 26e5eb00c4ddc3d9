"""Byte parity at the workloads' full sizes: every output byte of the GPU
path against the CPU oracle, in the launch configuration the benchmark
times.

Workloads (seeded, mx9_dual_axis_amd.synth):
  * dual_small  bf16 [256, 256] N(0,1)
  * dual_mixed  bf16 [8192, 7168], mixed-magnitude rows, zero tiles
                (plain and matrix-core scale layouts)
  * grouped     bf16 [16384, 5120], 64 groups covering 12288 rows
                (plain and matrix-core scale layouts)
  * weights     MX9 pack / unpack of fp32 [4096, 14336] and its bf16 rounding,
                unpacked to both output types
  * stress      bf16 [32768, 8192] with Inf / NaN, subnormal and near-max
                tiles, through the dual-axis cast and MX9 pack / unpack

Operations: pytorch/ao PR #4995 "[moe_training] Fused dual-axis MXFP8
quantization with correct metadata" (the cast, its grouped tail) and
AMD-AGI/ALTO PR #33 "feat: mx9: add fused MX9 quantization kernel with
pack/unpack" (MX9).  The oracle runs on 16 threads; its grouped call is the C
grouped function on row slabs.
"""
import numpy as np
import pytest
import torch

import mx9_dual_axis_amd as mxq
import oracle
from helpers import bf16_to_dev, host, require_gpu, say
from mx9_dual_axis_amd import synth

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]
THREADS = 16
NAMES = ("q_row", "s_row", "q_col", "s_col")


def _same(got, want, tag):
    g = host(got) if isinstance(got, torch.Tensor) else got
    assert g.shape == want.shape, (tag, g.shape, want.shape)
    if not np.array_equal(g, want):
        bad = np.argwhere(g != want)
        idx = bad[:5]
        pytest.fail(f"{tag}: {len(bad)} entries differ, first at {idx.tolist()}: "
                    f"got {[int(g[tuple(i)]) for i in idx]} want {[int(want[tuple(i)]) for i in idx]}")


def _dirty(shapes, dev, fill=0xA5):
    return tuple(torch.full(s, fill, dtype=torch.uint8, device=dev) for s in shapes)


def _plain_shapes(M, N):
    return ((M, N), (M, N // 32), (N, M), (M // 32, N))


def _mfma_shapes(M, N):
    return ((M, N), (M * N // 32,), (N, M), (M * N // 32,))


def _to_mfma(want):
    q_row, s_row, q_col, s_col = want
    return q_row, oracle.scales_to_mfma(s_row), q_col, oracle.scales_to_mfma(np.ascontiguousarray(s_col.T))


def _release():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ inputs

@pytest.fixture(scope="module")
def mixed():
    say("generating dual_mixed bf16 [8192, 7168] (seed 2)")
    x = synth.dual_mixed()
    say("  oracle: dual-axis cast of dual_mixed")
    return x, oracle.mxfp8_dual(x, threads=THREADS)


@pytest.fixture(scope="module")
def grouped():
    say("generating grouped bf16 [16384, 5120], 64 groups (seed 3)")
    x, offs = synth.grouped()
    assert offs[-1] == 12288
    say("  oracle: grouped cast")
    rc, want = oracle.mxfp8_grouped(x, offs, threads=THREADS)
    assert rc == 0
    return x, offs, want


@pytest.fixture(scope="module")
def stress():
    say("generating stress bf16 [32768, 8192] (seed 5)")
    return synth.stress()


# ------------------------------------------------------------ dual-axis cast

def test_dual_small_every_byte():
    dev = require_gpu()
    say("full size: dual_small [256, 256]")
    x = synth.dual_small()
    out = _dirty(_plain_shapes(256, 256), dev)
    mxq.mx_quantize_2d_dual(bf16_to_dev(x), out=out)
    for name, g, w in zip(NAMES, out, oracle.mxfp8_dual(x)):
        _same(g, w, f"dual_small {name}")


@pytest.mark.parametrize("layout", ["plain", "mfma"])
def test_dual_mixed_every_byte(mixed, layout):
    dev = require_gpu()
    x, want = mixed
    M, N = x.shape
    say(f"full size: dual_mixed [{M}, {N}], {layout} scales")
    out = _dirty(_plain_shapes(M, N) if layout == "plain" else _mfma_shapes(M, N), dev)
    mxq.mx_quantize_2d_dual(bf16_to_dev(x), out=out, scale_layout=layout)
    w = want if layout == "plain" else _to_mfma(want)
    for name, g, ww in zip(NAMES, out, w):
        _same(g, ww, f"dual_mixed {layout} {name}")
    del out
    _release()


@pytest.mark.parametrize("layout", ["plain", "mfma"])
def test_grouped_every_byte(grouped, layout):
    dev = require_gpu()
    x, offs, want = grouped
    M, N = x.shape
    say(f"full size: grouped [{M}, {N}], G = {len(offs)}, covered {int(offs[-1])}, {layout} scales")
    err = torch.full((1,), -7, dtype=torch.int32, device=dev)
    out = _dirty(_plain_shapes(M, N) if layout == "plain" else _mfma_shapes(M, N), dev)
    mxq.mx_quantize_grouped(bf16_to_dev(x), torch.from_numpy(offs).to(dev), err=err, out=out, scale_layout=layout)
    assert int(err.item()) == 0
    w = want if layout == "plain" else _to_mfma(want)
    for name, g, ww in zip(NAMES, out, w):
        _same(g, ww, f"grouped {layout} {name}")
    # the tail really is there: 128 block rows of zero colwise scales
    assert not want[3][int(offs[-1]) // 32:].any() and want[3][:int(offs[-1]) // 32].any()
    del out
    _release()


def test_stress_cast_every_byte(stress):
    """The benchmark's cast: the large-call path (diagonal tile order and the
    streamed share of q_row) on every tile."""
    dev = require_gpu()
    x = stress
    M, N = x.shape
    say(f"full size: stress dual-axis cast [{M}, {N}]")
    out = _dirty(_plain_shapes(M, N), dev)
    mxq.mx_quantize_2d_dual(bf16_to_dev(x), out=out)
    got = [host(t) for t in out]
    del out
    _release()
    say("  oracle: dual-axis cast of the stress matrix")
    want = oracle.mxfp8_dual(x, threads=THREADS)
    for name, g, w in zip(NAMES, got, want):
        say(f"  compare {name}")
        _same(g, w, f"stress {name}")
    # the specials reached the outputs: poisoned blocks on both axes, Inf blocks colwise
    assert (want[1] == 255).any() and (want[3] == 255).any() and (want[3] == 254).any()


# -------------------------------------------------------------------- MX9

def _pack_unpack_every_byte(x, tag, out_dtypes=("fp32", "bf16")):
    dev = require_gpu()
    rows, cols = x.shape
    xd = bf16_to_dev(x) if x.dtype == np.uint16 else torch.from_numpy(x).to(dev)
    nb = rows * ((cols + 15) // 16)
    out = (torch.full((nb, 16), 0x5A, dtype=torch.int8, device=dev),
           torch.full((nb,), 0xA5, dtype=torch.uint8, device=dev),
           torch.full((nb, 1), 0xA5, dtype=torch.uint8, device=dev))
    q, e, p = mxq.mx9_pack(xd, out=out)
    del xd
    ys = {od: mxq.mx9_unpack(q, e, p, rows, cols, out_dtype=torch.float32 if od == "fp32" else torch.bfloat16)
          for od in out_dtypes}
    hq, he, hp = host(q), host(e), host(p)
    hy = {od: host(y) for od, y in ys.items()}
    del q, e, p, ys, out
    _release()
    say(f"  oracle: MX9 pack of {tag}")
    wq, we, wp = oracle.mx9_pack(x, threads=THREADS)
    _same(hq, wq, f"{tag} q")
    _same(he, we, f"{tag} max_exp")
    _same(hp, wp, f"{tag} prime")
    for od in out_dtypes:
        say(f"  oracle: MX9 unpack of {tag} to {od}")
        wy = oracle.mx9_unpack(wq, we, wp, rows, cols, od, threads=THREADS)
        bits = np.uint32 if od == "fp32" else np.uint16
        _same(hy[od].view(bits), wy.view(bits), f"{tag} unpack {od}")
    return wq, we, wp


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_mx9_weights_every_byte(dtype):
    require_gpu()
    say(f"full size: MX9 weights [4096, 14336] {dtype}, pack and unpack to fp32 and bf16")
    x = synth.mx9_weights(4096, 14336, 4, dtype)
    wq, we, wp = _pack_unpack_every_byte(x, f"weights {dtype}")
    assert int(we.min()) >= 1 and int(we.max()) <= 254 and int(np.abs(wq.astype(np.int16)).max()) <= 127


def test_mx9_stress_every_byte(stress):
    require_gpu()
    say("full size: MX9 pack / unpack of the stress matrix [32768, 8192]")
    _, we, _ = _pack_unpack_every_byte(stress, "stress")
    assert int((we == 255).sum()) >= 1


def test_mx9_fp32_wide_pack_partial_last_workgroup():
    """An fp32 contiguous pack large enough for the eight-group flat kernel
    (at least 8192 workgroups of 512 blocks), with a block count that is not
    a multiple of 512, so its last workgroup is partial."""
    require_gpu()
    rows, cols = 4099, 16400                   # 1025 blocks per row, 4,201,475 blocks
    nb = rows * cols // 16
    assert nb > 8191 * 512 and nb % 512 != 0
    say(f"full size: MX9 fp32 [{rows}, {cols}], {nb} blocks")
    x = synth.mx9_weights(rows, cols, 41, "fp32")
    bits = x.view(np.uint32)
    bits[rows - 1, cols - 7] = 0x7F800000      # Inf in the last (partial) workgroup
    bits[rows - 1, cols - 40] = 0x00000123     # a subnormal there too
    _pack_unpack_every_byte(x, "fp32 wide", out_dtypes=("fp32",))
