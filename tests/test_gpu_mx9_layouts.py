"""GPU parity of MX9 along any axis (mx9_pack_axis / mx9_unpack_axis) and in
the single-byte-tensor form (mx9_pack_records / mx9_unpack_records) against
the CPU oracle: every q, max_exp, prime and record byte, and every unpacked
value, must be equal.  Format and calls: AMD-AGI/ALTO PR #33 "feat: mx9: add
fused MX9 quantization kernel with pack/unpack" (the axis argument; the
commit that packs MX9 into a single uint8 tensor)."""
import numpy as np
import pytest
import torch

import mx9_dual_axis_amd as mxq
import oracle
from helpers import bf16_to_dev, host, require_gpu, say
from mx9_dual_axis_amd import synth

pytestmark = pytest.mark.gpu
THREADS = 16


def _to_dev(x):
    if x.dtype == np.uint16:
        return bf16_to_dev(x.reshape(-1)).view(x.shape)
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def _tensor(shape, kind, seed):
    """fp32 or bf16-bit array of `shape` with the weights' value mixture and
    every special kind (zeros, -0, subnormals, Inf, NaN) sprinkled in."""
    n = int(np.prod(shape))
    x = synth.mx9_weights(1, n, seed, "fp32").reshape(shape)
    g = synth.rng(seed + 1000)
    flat = x.reshape(-1)
    idx = g.choice(n, size=max(1, n // 50), replace=False)
    specials = np.array([0.0, -0.0, 1e-40, -3e-39, np.inf, -np.inf, np.nan, 2.0 ** -130], np.float32)
    flat[idx] = specials[g.integers(0, len(specials), len(idx))]
    if kind == "bf16":
        return synth.to_bf16_bits(x)
    return x


def _same(got, want, tag):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (tag, got.shape, want.shape)
    if got.dtype == np.float32:
        got, want = got.view(np.uint32), want.view(np.uint32)
    bad = np.count_nonzero(got != want)
    if bad:
        i = np.argwhere(got != want)[0]
        pytest.fail(f"{tag}: {bad} differ; first at {i.tolist()}: got {got[tuple(i)]} want {want[tuple(i)]}")


SHAPES = [
    ((64, 48), 0),          # columns of a matrix
    ((53, 7), 0),           # ragged length along the axis, narrow inner
    ((3, 40, 5), 1),        # middle axis
    ((2, 3, 33), 2),        # last axis through the axis call
    ((17, 4, 600), 0),      # several workgroups of inner positions
    ((5, 300, 70), 1),      # more than 16 blocks per (o, i): several block groups per row
    ((5, 300, 71), 1),      # the same with an odd inner extent (one inner position per lane)
    ((1, 16, 1), 1),        # one block
]


@pytest.mark.parametrize("kind", ["fp32", "bf16"])
@pytest.mark.parametrize("shape,axis", SHAPES)
def test_axis_pack_unpack_parity(shape, axis, kind):
    require_gpu()
    say(f"mx9 axis parity {kind} {shape} axis={axis}")
    x = _tensor(shape, kind, sum(shape) * 7 + axis)
    xd = _to_dev(x)
    q, e, p = mxq.mx9_pack_axis(xd, axis)
    torch.cuda.synchronize()
    wq, we, wp = oracle.mx9_pack_axis(x, axis, threads=4)
    _same(host(q), wq, "q")
    _same(host(e), we, "max_exp")
    _same(host(p), wp, "prime")
    for od, td in (("fp32", torch.float32), ("bf16", torch.bfloat16)):
        y = mxq.mx9_unpack_axis(q, e, p, shape, axis, out_dtype=td)
        torch.cuda.synchronize()
        _same(host(y), oracle.mx9_unpack_axis(wq, we, wp, shape, axis, od, threads=4), f"unpack {od}")


@pytest.mark.parametrize("kind", ["fp32", "bf16"])
@pytest.mark.parametrize("shape,axis", SHAPES + [((96, 256), 1), ((1000, 64), 1), ((7, 4096), 1), ((3, 4112), 1)])
def test_records_pack_unpack_parity(shape, axis, kind):
    """Records of the same blocks: the flat path (last axis, length a multiple
    of 16, contiguous records) and the strided path (everything else)."""
    require_gpu()
    say(f"mx9 records parity {kind} {shape} axis={axis}")
    x = _tensor(shape, kind, sum(shape) * 11 + axis)
    xd = _to_dev(x)
    outer, length, inner = mxq._axis_dims(shape, axis)
    nbl = (length + 15) // 16
    packed = mxq.mx9_pack_records(xd, axis)
    torch.cuda.synchronize()
    wq, we, wp = oracle.mx9_pack_axis(x, axis, threads=4)
    want = oracle.mx9_to_records(wq, we, wp, outer * inner, nbl)
    _same(host(packed), want, "records")
    for od, td in (("fp32", torch.float32), ("bf16", torch.bfloat16)):
        y = mxq.mx9_unpack_records(packed, shape, axis, out_dtype=td)
        torch.cuda.synchronize()
        _same(host(y), oracle.mx9_unpack_axis(wq, we, wp, shape, axis, od, threads=4), f"unpack {od}")


@pytest.mark.parametrize("kind", ["fp32", "bf16"])
def test_records_with_pitch_leave_the_gap_alone(kind):
    """Rows of records at a pitch wider than the records: the gap bytes keep
    their contents, and the unpack reads the rows at that pitch."""
    require_gpu()
    say(f"mx9 records with a row pitch, {kind}")
    shape = (40, 96)                                  # 6 records = 108 bytes per row
    x = _tensor(shape, kind, 77)
    xd = _to_dev(x)
    wide = torch.full((40, 128), 0xA5, dtype=torch.uint8, device="cuda:0")
    mxq.mx9_pack_records(xd, -1, out=wide)
    torch.cuda.synchronize()
    hw = host(wide)
    wq, we, wp = oracle.mx9_pack(x)
    _same(hw[:, :108], oracle.mx9_to_records(wq, we, wp, 40, 6), "records")
    assert np.all(hw[:, 108:] == 0xA5)
    for od, td in (("fp32", torch.float32), ("bf16", torch.bfloat16)):
        y = mxq.mx9_unpack_records(wide, shape, -1, out_dtype=td)
        torch.cuda.synchronize()
        _same(host(y), oracle.mx9_unpack(wq, we, wp, 40, 96, od), f"unpack {od}")


def test_records_match_the_three_part_form_and_unpack_the_same():
    """pack_records == to_records(pack) on the device path too, and both
    forms unpack to the same values."""
    require_gpu()
    say("mx9 records vs three-part form, bf16 [256, 1024]")
    x = synth.mx9_weights(256, 1024, 31, "bf16")
    xd = _to_dev(x)
    q, e, p = mxq.mx9_pack(xd)
    packed = mxq.mx9_pack_records(xd)
    torch.cuda.synchronize()
    assert np.array_equal(host(packed), oracle.mx9_to_records(host(q), host(e), host(p), 256, 64))
    y3 = mxq.mx9_unpack(q, e, p, 256, 1024, out_dtype=torch.bfloat16)
    yr = mxq.mx9_unpack_records(packed, (256, 1024), -1, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y3.view(torch.int16), yr.view(torch.int16))


def test_empty_and_rejections():
    require_gpu()
    say("mx9 axis / records: empty tensors and rejections")
    z = torch.empty((0, 32), dtype=torch.float32, device="cuda:0")
    q, e, p = mxq.mx9_pack_axis(z, 0)
    assert q.shape == (0, 16)
    assert mxq.mx9_pack_records(z, 1).shape == (0, 36)
    with pytest.raises(mxq.MXError) as ei:
        mxq.mx9_pack_axis(torch.zeros((4, 32), dtype=torch.float16, device="cuda:0"), 0)
    assert ei.value.status == 2
    with pytest.raises(mxq.MXError) as ei:
        mxq.mx9_pack_records(torch.zeros((4, 32), device="cuda:0"), -1, block_size=32)
    assert ei.value.status == 3


def test_graph_capture_records():
    require_gpu()
    say("mx9 records in a captured graph")
    x = synth.mx9_weights(64, 512, 9, "bf16")
    xd = _to_dev(x)
    packed = mxq.mx9_pack_records(xd)
    y = mxq.mx9_unpack_records(packed, (64, 512), -1, out_dtype=torch.bfloat16)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mxq.mx9_pack_records(xd, out=packed)
        mxq.mx9_unpack_records(packed, (64, 512), -1, out=y)
    wq, we, wp = oracle.mx9_pack(x)
    want_p = oracle.mx9_to_records(wq, we, wp, 64, 32)
    want_y = oracle.mx9_unpack(wq, we, wp, 64, 512, "bf16")
    for rep in range(3):
        packed.fill_(3)
        y.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(packed), want_p), rep
        assert np.array_equal(host(y), want_y), rep


# ---------------------------------------------------------------- full sizes

@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_full_size_weights_records_and_axis0(dtype):
    """The [4096, 14336] weights: records along the last axis (flat path) and
    the three-part form along axis 0 (tiled path), every byte against the
    oracle, and both unpacks."""
    require_gpu()
    say(f"mx9 full size weights [4096, 14336] {dtype}: records and axis 0, every byte")
    x = synth.mx9_weights(4096, 14336, 4, dtype)
    xd = _to_dev(x)
    td = torch.float32 if dtype == "fp32" else torch.bfloat16
    packed = mxq.mx9_pack_records(xd)
    y = mxq.mx9_unpack_records(packed, x.shape, -1, out_dtype=td)
    hp, hy = host(packed), host(y)
    del packed, y
    wq, we, wp = oracle.mx9_pack(x, threads=THREADS)
    _same(hp, oracle.mx9_to_records(wq, we, wp, 4096, 14336 // 16), "records")
    _same(hy, oracle.mx9_unpack(wq, we, wp, 4096, 14336, dtype, threads=THREADS), "records unpack")
    del hp, hy, wq, we, wp
    q, e, p = mxq.mx9_pack_axis(xd, 0)
    ya = mxq.mx9_unpack_axis(q, e, p, x.shape, 0, out_dtype=td)
    hq, he, hpr, hya = host(q), host(e), host(p), host(ya)
    del q, e, p, ya, xd
    torch.cuda.empty_cache()
    cq, ce, cp = oracle.mx9_pack_axis(x, 0, threads=THREADS)
    _same(hq, cq, "axis-0 q")
    _same(he, ce, "axis-0 max_exp")
    _same(hpr, cp, "axis-0 prime")
    _same(hya, oracle.mx9_unpack_axis(cq, ce, cp, x.shape, 0, dtype, threads=THREADS), "axis-0 unpack")
