"""GPU parity of MX9 pack / unpack (mx9_pack, mx9_unpack) against the CPU
oracle: q, max_exp, prime and the unpacked values must be equal bit for bit.
Format: AMD-AGI/ALTO PR #33 "feat: mx9: add fused MX9 quantization kernel
with pack/unpack"."""
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
        return bf16_to_dev(x)
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def _check_pack(x, tag, dev_x=None):
    rows, cols = x.shape
    xd = _to_dev(x) if dev_x is None else dev_x
    nb = rows * ((cols + 15) // 16)
    out = (torch.full((nb, 16), 0x5A, dtype=torch.int8, device=xd.device),
           torch.full((nb,), 0xA5, dtype=torch.uint8, device=xd.device),
           torch.full((nb, 1), 0xA5, dtype=torch.uint8, device=xd.device))
    q, e, p = mxq.mx9_pack(xd, out=out)
    torch.cuda.synchronize()
    wq, we, wp = oracle.mx9_pack(x, threads=THREADS)
    for name, g, w in (("q", q, wq), ("max_exp", e, we), ("prime", p, wp)):
        g = host(g)
        bad = np.count_nonzero(g != w)
        if bad:
            i = np.argwhere(g != w)[0]
            pytest.fail(f"{tag}: {name} differs in {bad} entries; first {i.tolist()} got {g[tuple(i)]} want {w[tuple(i)]}")
    return q, e, p, (wq, we, wp)


def _check_unpack(q, e, p, rows, cols, tag, out_dtype="fp32"):
    td = torch.float32 if out_dtype == "fp32" else torch.bfloat16
    y = mxq.mx9_unpack(q, e, p, rows, cols, out_dtype=td)
    torch.cuda.synchronize()
    want = oracle.mx9_unpack(host(q), host(e), host(p), rows, cols, out_dtype, threads=THREADS)
    g = host(y)
    gb = g.view(np.uint32) if out_dtype == "fp32" else g
    wb = want.view(np.uint32) if out_dtype == "fp32" else want
    bad = np.count_nonzero(gb != wb)
    if bad:
        i = np.argwhere(gb != wb)[0]
        pytest.fail(f"{tag}: unpack {out_dtype} differs in {bad}; first {i.tolist()} got {hex(gb[tuple(i)])} want {hex(wb[tuple(i)])}")
    return y


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("rows,cols", [(16, 64), (64, 1024), (33, 200), (7, 5), (128, 4096), (1, 16),
                                       (5, 128), (3, 4112), (9, 2048)])
def test_pack_unpack_parity(dtype, rows, cols):
    require_gpu()
    say(f"mx9 parity {dtype} [{rows}, {cols}]")
    x = synth.mx9_weights(rows, cols, rows * 31 + cols, dtype)
    q, e, p, _ = _check_pack(x, f"{dtype} {rows}x{cols}")
    for od in ("fp32", "bf16"):
        _check_unpack(q, e, p, rows, cols, f"{dtype} {rows}x{cols}", od)


def test_special_values_and_subnormals():
    require_gpu()
    say("mx9 special values")
    g = np.random.default_rng(3)
    x = synth.mx9_weights(64, 256, 3)
    bits = x.view(np.uint32)
    bits[0, :16] = 0                                          # zeros
    bits[1, :16] = g.integers(0, 1 << 23, 16)                 # subnormal block
    bits[1, 16:32] = g.integers(0, 1 << 23, 16) | (1 << 31)
    bits[2, 3] = 0x7F800000; bits[2, 20] = 0xFF800000         # +-Inf
    bits[3, 7] = 0x7FC00000; bits[3, 40] = 0xFFC12345         # NaNs
    bits[4, :16] = 0x7F7FFFFF                                 # fp32 max
    bits[5, :16] = [0x3FFF0000, 0x3F810000, 0x3F830000, 0x3F7F8000] * 4   # clamp and ties
    bits[6, :] = (g.integers(1, 255, 256) << 23) | g.integers(0, 1 << 23, 256)  # all binades
    # blocks whose exponent byte runs 3..18 (either side of where the float
    # scale replaces ldexp), partnered with subnormals and the smallest
    # normals, some of which round to +-1 or sit on ties
    for t in range(16):
        blk = bits[7, 16 * t:16 * t + 16]
        blk[:] = (g.integers(0, 2, 16) << 23) | g.integers(0, 1 << 23, 16)
        blk[0] = ((3 + t) << 23) | int(g.integers(0, 1 << 23))
        blk[1 + t % 15] = (1 << 22) if t % 2 else (3 << 21)
        blk[:] |= (g.integers(0, 2, 16) << 31).astype(np.uint32)
    q, e, p, _ = _check_pack(x, "specials fp32")
    _check_unpack(q, e, p, 64, 256, "specials", "fp32")
    _check_unpack(q, e, p, 64, 256, "specials", "bf16")
    xb = synth.special_matrix(64, 256, 4)
    q, e, p, _ = _check_pack(xb, "specials bf16")
    _check_unpack(q, e, p, 64, 256, "specials bf16", "bf16")


def test_every_bf16_pattern_lone():
    require_gpu()
    say("mx9 lone bf16 patterns")
    pats = np.arange(65536, dtype=np.uint32)
    x = np.zeros((65536, 16), np.uint16)
    x[pats, pats % 16] = pats.astype(np.uint16)
    q, e, p, _ = _check_pack(x, "lone patterns")
    _check_unpack(q, e, p, 65536, 16, "lone patterns", "bf16")
    _check_unpack(q, e, p, 65536, 16, "lone patterns", "fp32")


def test_exhaustive_unpack():
    require_gpu()
    say("mx9 exhaustive unpack")
    S = np.repeat(np.arange(256), 2 * 256)
    P = np.tile(np.repeat(np.arange(2), 256), 256)
    Q = np.tile(np.arange(-128, 128), 512)
    nb = S.size // 16
    q = torch.from_numpy(Q.astype(np.int8).reshape(nb, 16)).cuda()
    e = torch.from_numpy(S.reshape(nb, 16)[:, 0].astype(np.uint8)).cuda()
    p = torch.from_numpy((P.reshape(nb, 16)[:, 0] * 0xFF).astype(np.uint8).reshape(nb, 1)).cuda()
    for od in ("fp32", "bf16"):
        _check_unpack(q, e, p, 1, S.size, "exhaustive", od)
        _check_unpack(q, e, p, nb, 16, "exhaustive rows", od)


def test_strided_and_unaligned_inputs():
    require_gpu()
    say("mx9 strided input and output")
    wide = synth.mx9_weights(48, 300, 5)
    xd = _to_dev(wide)[:, 7:263]                              # ld 300, start unaligned
    q, e, p, _ = _check_pack(np.ascontiguousarray(wide[:, 7:263]), "strided fp32", dev_x=xd)
    wideb = synth.mx9_weights(48, 300, 6, "bf16")
    xdb = _to_dev(wideb)[:, 16:272]                           # ld 300 (600 B rows): not 16-byte rows
    _check_pack(np.ascontiguousarray(wideb[:, 16:272]), "strided bf16", dev_x=xdb)
    # unpack into a wider output: only cols columns are written
    yw = torch.full((48, 300), 7.0, dtype=torch.float32, device="cuda:0")
    mxq.mx9_unpack(q, e, p, 48, 256, out=yw)
    torch.cuda.synchronize()
    want = oracle.mx9_unpack(host(q), host(e), host(p), 48, 256, "fp32")
    got = host(yw)
    assert np.array_equal(got[:, :256].view(np.uint32), want.view(np.uint32))
    assert (got[:, 256:] == 7.0).all()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_every_kernel_path(dtype):
    """Flat (contiguous), vector (strided, 16-byte aligned rows) and general
    (unaligned or ragged) kernels of pack and unpack, for both dtypes."""
    dev = require_gpu()
    say(f"mx9 kernel paths {dtype}")
    wide = synth.mx9_weights(40, 512, 21, dtype)
    esz = 4 if dtype == "fp32" else 2
    cases = {
        "flat": (wide[:, :256], _to_dev(np.ascontiguousarray(wide[:, :256]))),
        "vector": (wide[:, 128:384], _to_dev(wide)[:, 128:384]),          # ld 512, aligned rows
        "general": (wide[:, 3:203], _to_dev(wide)[:, 3:203]),             # unaligned, ragged
    }
    for name, (host_x, dev_x) in cases.items():
        rows, cols = host_x.shape
        if name == "vector":
            assert dev_x.stride(0) * esz % 16 == 0 and dev_x.data_ptr() % 16 == 0
        q, e, p, _ = _check_pack(np.ascontiguousarray(host_x), f"{dtype} {name}", dev_x=dev_x)
        for od, td in (("fp32", torch.float32), ("bf16", torch.bfloat16)):
            want = oracle.mx9_unpack(host(q), host(e), host(p), rows, cols, od)
            # contiguous output (flat), wider aligned output (vector), odd pitch (general)
            for pitch in (cols, cols + 64, cols + 3):
                y = torch.full((rows, pitch), 5, dtype=td, device=dev)
                mxq.mx9_unpack(q, e, p, rows, cols, out=y)
                torch.cuda.synchronize()
                got = host(y)[:, :cols]
                gb = got.view(np.uint32) if od == "fp32" else got
                wb = want.view(np.uint32) if od == "fp32" else want
                assert np.array_equal(gb, wb), (dtype, name, od, pitch)
                if pitch > cols:
                    assert bool((y[:, cols:].float() == 5).all()), (dtype, name, od, pitch)


def test_rejections_and_empty():
    dev = require_gpu()
    say("mx9 rejections")
    with pytest.raises(mxq.MXError) as ei:
        mxq.mx9_pack(torch.zeros((4, 16), dtype=torch.float16, device=dev))
    assert ei.value.status == 2
    with pytest.raises(mxq.MXError) as ei:
        mxq.mx9_pack(torch.zeros((4, 16), dtype=torch.float32, device=dev), block_size=32)
    assert ei.value.status == 3
    q, e, p = mxq.mx9_pack(torch.zeros((4, 16), dtype=torch.float32, device=dev))
    with pytest.raises(mxq.MXError) as ei:
        mxq.mx9_unpack(q, e, p, 4, 16, out_dtype=torch.float16)
    assert ei.value.status == 2
    # caller outputs and inputs: wrong device, dtype, size or layout raise in the binding
    x = torch.zeros((4, 32), dtype=torch.float32, device=dev)
    good = (torch.zeros((8, 16), dtype=torch.int8, device=dev), torch.zeros((8,), dtype=torch.uint8, device=dev),
            torch.zeros((8, 1), dtype=torch.uint8, device=dev))
    for k, bad in ((0, torch.zeros((8, 16), dtype=torch.int8)),                   # host
                   (0, torch.zeros((7, 16), dtype=torch.int8, device=dev)),       # too small
                   (1, torch.zeros((8,), dtype=torch.int8, device=dev)),          # dtype
                   (2, torch.zeros((8, 2), dtype=torch.uint8, device=dev)[:, :1])):  # not contiguous
        out = list(good)
        out[k] = bad
        with pytest.raises(ValueError) as ei:
            mxq.mx9_pack(x, out=tuple(out))
        assert not isinstance(ei.value, mxq.MXError)
    with pytest.raises(ValueError):
        mxq.mx9_unpack(good[0], good[1], good[2], 4, 32, out=torch.zeros((4, 32), dtype=torch.float32))
    with pytest.raises(ValueError):
        mxq.mx9_unpack(good[0], good[1], good[2], 4, 32, out=torch.zeros((4, 32), dtype=torch.float16, device=dev))
    with pytest.raises(ValueError):
        mxq.mx9_unpack(good[0].cpu(), good[1], good[2], 4, 32)
    with pytest.raises(ValueError):
        mxq.mx9_pack_records(x, out=torch.zeros((4, 36), dtype=torch.uint8))
    with pytest.raises(ValueError):
        mxq.mx9_unpack_axis(good[0], good[1], good[2], (4, 32), 1, out=torch.zeros((4, 32), device=dev).t())
    q, e, p = mxq.mx9_pack(torch.zeros((0, 16), dtype=torch.float32, device=dev))
    assert q.shape == (0, 16)
    y = mxq.mx9_unpack(q, e, p, 0, 16)
    assert y.shape == (0, 16)


def test_graph_capture():
    require_gpu()
    say("mx9 in a captured graph")
    x = synth.mx9_weights(64, 512, 8, "bf16")
    xd = _to_dev(x)
    q, e, p = mxq.mx9_pack(xd)
    y = mxq.mx9_unpack(q, e, p, 64, 512, out_dtype=torch.bfloat16)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mxq.mx9_pack(xd, out=(q, e, p))
        mxq.mx9_unpack(q, e, p, 64, 512, out=y)
    wq, we, wp = oracle.mx9_pack(x)
    wy = oracle.mx9_unpack(wq, we, wp, 64, 512, "bf16")
    for rep in range(3):
        q.fill_(3); e.fill_(3); p.fill_(3); y.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(q), wq) and np.array_equal(host(e), we) and np.array_equal(host(p), wp)
        assert np.array_equal(host(y), wy), rep


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("rows,cols", [(33, 200), (64, 1024), (1, 48), (130, 16)])
def test_pitched_parts(dtype, rows, cols):
    """mx9_pack_strided / mx9_unpack_strided: q, max_exp and prime as column
    slices of wider tensors (each at its own row pitch) hold the oracle's
    bytes in their used columns and leave the rest untouched; the unpack reads
    them back at those pitches."""
    dev = require_gpu()
    say(f"mx9 pitched parts {dtype} [{rows}, {cols}]")
    x = synth.mx9_weights(rows, cols, 7 * rows + cols, dtype)
    nbr = (cols + 15) // 16
    qw = torch.full((rows, 16 * nbr + 48), 0x5A, dtype=torch.int8, device=dev)
    ew = torch.full((rows, nbr + 5), 0xA5, dtype=torch.uint8, device=dev)
    pw = torch.full((rows, nbr + 9), 0xA5, dtype=torch.uint8, device=dev)
    q, e, p = qw[:, 16:16 + 16 * nbr], ew[:, 3:3 + nbr], pw[:, :nbr]
    mxq.mx9_pack_strided(_to_dev(x), out=(q, e, p))
    torch.cuda.synchronize()
    wq, we, wp = oracle.mx9_pack(x, threads=THREADS)
    assert np.array_equal(host(q), wq.reshape(rows, 16 * nbr))
    assert np.array_equal(host(e), we.reshape(rows, nbr))
    assert np.array_equal(host(p), wp.reshape(rows, nbr))
    hq, he, hp = host(qw), host(ew), host(pw)
    assert (hq[:, :16] == 0x5A).all() and (hq[:, 16 + 16 * nbr:] == 0x5A).all()
    assert (he[:, :3] == 0xA5).all() and (he[:, 3 + nbr:] == 0xA5).all() and (hp[:, nbr:] == 0xA5).all()
    for od, td in (("fp32", torch.float32), ("bf16", torch.bfloat16)):
        want = oracle.mx9_unpack(wq, we, wp, rows, cols, od)
        yw = torch.full((rows, cols + 8), 3, dtype=td, device=dev)
        mxq.mx9_unpack_strided(q, e, p, rows, cols, out=yw[:, :cols])
        torch.cuda.synchronize()
        got = host(yw)
        bits = np.uint32 if od == "fp32" else np.uint16
        assert np.array_equal(got[:, :cols].view(bits), want.view(bits)), od
        assert bool((yw[:, cols:].float() == 3).all())
    # the contiguous call is the special case with packed pitches
    q2, e2, p2 = mxq.mx9_pack_strided(_to_dev(x))
    assert np.array_equal(host(q2), wq.reshape(rows, 16 * nbr)) and np.array_equal(host(p2), wp.reshape(rows, nbr))


# ---------------------------------------------------------------- full sizes
# Every byte of the full-size workloads is compared with the oracle in
# test_gpu_full_size.py; here, the round trip's quality at full size.

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_full_size_weights_snr(dtype):
    """SNR of the [4096, 14336] weights' round trip (the page reports about
    46 dB for clean data and about 42 dB with outliers; this mixture has a
    heavy tail, so the bound is the clean-data figure less the outlier loss)."""
    require_gpu()
    say(f"mx9 full size weights [4096, 14336] {dtype}: SNR")
    x = synth.mx9_weights(4096, 14336, 4, dtype)
    xd = _to_dev(x)
    q, e, p = mxq.mx9_pack(xd)
    y = mxq.mx9_unpack(q, e, p, 4096, 14336, out_dtype=torch.float32 if dtype == "fp32" else torch.bfloat16)
    assert int(e.min()) >= 1 and int(e.max()) <= 254 and int(q.abs().max()) <= 127
    xf = xd.float()
    snr = 10 * torch.log10((xf * xf).sum() / ((xf - y.float()) ** 2).sum()).item()
    say(f"  SNR {dtype}: {snr:.2f} dB")
    assert snr > 40.0
