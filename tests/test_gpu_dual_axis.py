"""GPU parity of the fused dual-axis MXFP8 cast (mx_quantize_2d_dual) and
its grouped variant (mx_quantize_grouped) against the CPU oracle: every
output byte must be equal.  Operation: pytorch/ao PR #4995 "[moe_training]
Fused dual-axis MXFP8 quantization with correct metadata"."""
import numpy as np
import pytest
import torch

import mx9_dual_axis_amd as mxq
import oracle
from helpers import bf16_to_dev, host, require_gpu, say
from mx9_dual_axis_amd import synth

pytestmark = pytest.mark.gpu
THREADS = 16
NAMES = ("q_row", "s_row", "q_col", "s_col")


def _assert_equal(got, want, tag):
    for name, g, w in zip(NAMES, got, want):
        g = host(g) if isinstance(g, torch.Tensor) else g
        assert g.shape == w.shape, (tag, name, g.shape, w.shape)
        bad = np.count_nonzero(g != w)
        if bad:
            idx = np.argwhere(g != w)[:5]
            pytest.fail(f"{tag}: {name} differs in {bad} bytes, first at {idx.tolist()}: "
                        f"got {[int(g[tuple(i)]) for i in idx]} want {[int(w[tuple(i)]) for i in idx]}")


def _dirty_outputs(M, N, dev, fill=0xA5):
    kw = dict(dtype=torch.uint8, device=dev)
    return tuple(torch.full(s, fill, **kw) for s in ((M, N), (M, N // 32), (N, M), (M // 32, N)))


@pytest.mark.parametrize("M,N,kind,seed", [
    (256, 256, "normal", 1),          # the 256x256 workload
    (128, 128, "special", 2),         # one tile
    (384, 640, "special", 3),         # 3 x 5 tiles, every special block kind
    (1024, 384, "mixed", 4),          # mixed-magnitude rows, zero tiles
    (640, 1152, "special", 5),
])
def test_dense_parity(M, N, kind, seed):
    dev = require_gpu()
    say(f"dense parity M={M} N={N} kind={kind} seed={seed}")
    xb = {"normal": synth.normal_bf16, "special": synth.special_matrix, "mixed": synth.mixed_rows}[kind](M, N, seed)
    out = _dirty_outputs(M, N, dev)
    mxq.mx_quantize_2d_dual(bf16_to_dev(xb), out=out)
    torch.cuda.synchronize()
    _assert_equal(out, oracle.mxfp8_dual(xb, threads=THREADS), f"{M}x{N} {kind}")


@pytest.mark.parametrize("M,N", [
    (128, 15872),    # one tile row, 124 tiles across (tile-row count not a multiple of 8)
    (256, 16384),    # wide rows
    (384, 2560),     # three tile rows
    (1152, 1152),    # 9 x 9 tiles: consecutive tiles of a tile row on different XCDs
])
def test_rowwise_scale_shapes(M, N):
    """s_row is written with one 4-byte store per tile row; shapes whose tile
    rows do and do not stay on one XCD give the same bytes."""
    dev = require_gpu()
    say(f"s_row shapes M={M} N={N}")
    xb = synth.mixed_rows(M, N, M + N)
    out = _dirty_outputs(M, N, dev)
    mxq.mx_quantize_2d_dual(bf16_to_dev(xb), out=out)
    torch.cuda.synchronize()
    _assert_equal(out, oracle.mxfp8_dual(xb, threads=THREADS), f"{M}x{N}")


def test_dense_strided_input():
    """Row pitch larger than N (a column slice of a wider matrix)."""
    dev = require_gpu()
    say("dense parity with ld_x > N")
    wide = synth.special_matrix(256, 512, 6)
    xd = bf16_to_dev(wide)[:, 128:384]
    assert xd.stride(0) == 512
    got = mxq.mx_quantize_2d_dual(xd)
    torch.cuda.synchronize()
    _assert_equal(got, oracle.mxfp8_dual(np.ascontiguousarray(wide[:, 128:384])), "strided")


def test_every_bf16_pattern_both_axes():
    """All 65536 bf16 patterns, each as the lone non-zero of its block, at
    every position, rowwise and colwise, plus a dense random layout of all
    patterns."""
    require_gpu()
    say("exhaustive bf16 patterns")
    pats = np.arange(65536, dtype=np.uint32)
    x = np.zeros((2048, 1024), np.uint16)
    # each row block (m, j) gets one pattern at position (m + j) % 32
    m = np.repeat(np.arange(2048), 32)
    j = np.tile(np.arange(32), 2048)
    x[m, 32 * j + (m + j) % 32] = pats.astype(np.uint16)
    got = mxq.mx_quantize_2d_dual(bf16_to_dev(x))
    _assert_equal(got, oracle.mxfp8_dual(x, threads=THREADS), "lone patterns")
    perm = np.random.default_rng(0).permutation(65536).astype(np.uint16)
    xd = np.tile(perm, 4).reshape(512, 512)
    got = mxq.mx_quantize_2d_dual(bf16_to_dev(xd))
    _assert_equal(got, oracle.mxfp8_dual(xd, threads=THREADS), "dense patterns")


def test_repeatable_and_dirty_buffers():
    dev = require_gpu()
    say("determinism and dirty destinations")
    xb = synth.special_matrix(512, 512, 7)
    xd = bf16_to_dev(xb)
    a = _dirty_outputs(512, 512, dev, 0x00)
    b = _dirty_outputs(512, 512, dev, 0xFF)
    mxq.mx_quantize_2d_dual(xd, out=a)
    mxq.mx_quantize_2d_dual(xd, out=b)
    mxq.mx_quantize_2d_dual(xd, out=b)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("N", [384, 1024])
def test_runs_on_the_callers_stream_and_in_a_graph(N):
    dev = require_gpu()
    say(f"stream and graph capture N={N}")
    M = 256
    xb = synth.special_matrix(M, N, 8)
    want = oracle.mxfp8_dual(xb, threads=THREADS)
    xd = bf16_to_dev(xb)
    s = torch.cuda.Stream()
    out = _dirty_outputs(M, N, dev)
    with torch.cuda.stream(s):
        mxq.mx_quantize_2d_dual(xd, out=out)
    s.synchronize()
    _assert_equal(out, want, "side stream")
    out = _dirty_outputs(M, N, dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mxq.mx_quantize_2d_dual(xd, out=out)
    for rep in range(3):
        for o in out:
            o.fill_(0xA5 + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _assert_equal(out, want, f"graph replay {rep}")


@pytest.mark.parametrize("N", [256, 1024])
def test_grouped_parity_and_tail(N):
    dev = require_gpu()
    M = 1024
    xb = synth.special_matrix(M, N, 9)
    xd = bf16_to_dev(xb)
    cases = [[128, 128, 512], [0, 0, 0], [1024], [256, 256, 768, 768], [0], [384]]
    for offs in cases:
        say(f"grouped parity offs={offs}")
        rc, want = oracle.mxfp8_grouped(xb, np.array(offs, np.int32), threads=THREADS)
        assert rc == 0
        err = torch.full((1,), -7, dtype=torch.int32, device=dev)
        out = _dirty_outputs(M, N, dev)
        mxq.mx_quantize_grouped(xd, torch.tensor(offs, dtype=torch.int32, device=dev), err=err, out=out)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        _assert_equal(out, want, f"grouped {offs}")
    # G = 0 is dense, and err is written
    err = torch.full((1,), -7, dtype=torch.int32, device=dev)
    got = mxq.mx_quantize_grouped(xd, torch.zeros(0, dtype=torch.int32, device=dev), err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    _assert_equal(got, oracle.mxfp8_dual(xb, threads=THREADS), "grouped G=0")


@pytest.mark.parametrize("offs,code", [
    ([256, 128], 1), ([100], 2), ([128, 2048], 3), ([-128], 3), ([128, 130, 64], 2), ([0, 1152], 3),
])
def test_grouped_invalid_offsets_reported(offs, code):
    dev = require_gpu()
    say(f"invalid offs={offs}")
    M, N = 1024, 128
    assert oracle.offs_check(np.array(offs, np.int32), M) == code
    xd = bf16_to_dev(synth.normal_bf16(M, N, 10))
    err = torch.full((1,), -7, dtype=torch.int32, device=dev)
    mxq.mx_quantize_grouped(xd, torch.tensor(offs, dtype=torch.int32, device=dev), err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == code


def test_many_groups_validation():
    """More groups than threads in a workgroup; the first bad entry decides."""
    dev = require_gpu()
    say("validation with 3000 groups")
    M, N = 512, 128
    offs = np.sort(np.random.default_rng(1).integers(0, 5, 3000)) * 128
    xd = bf16_to_dev(synth.normal_bf16(M, N, 11))
    for bad_at, bad_val in ((None, None), (2999, 7), (1500, 0), (300, 10 ** 6)):
        o = offs.copy()
        if bad_at is not None:
            o[bad_at] = bad_val
        err = torch.full((1,), -7, dtype=torch.int32, device=dev)
        mxq.mx_quantize_grouped(xd, torch.tensor(o, dtype=torch.int32, device=dev), err=err)
        torch.cuda.synchronize()
        assert int(err.item()) == oracle.offs_check(o.astype(np.int32), M)


def test_empty_matrix():
    dev = require_gpu()
    say("empty matrices")
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=dev)
    outs = mxq.mx_quantize_2d_dual(x)
    assert [tuple(o.shape) for o in outs] == [(0, 256), (0, 8), (256, 0), (0, 256)]
    err = torch.full((1,), -7, dtype=torch.int32, device=dev)
    mxq.mx_quantize_grouped(x, torch.tensor([0, 0], dtype=torch.int32, device=dev), err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    mxq.mx_quantize_grouped(x, torch.tensor([128], dtype=torch.int32, device=dev), err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 3


def test_host_rejections():
    dev = require_gpu()
    say("host-side rejections")
    x = torch.zeros((256, 256), dtype=torch.bfloat16, device=dev)
    with pytest.raises(mxq.MXError) as e:
        mxq.mx_quantize_2d_dual(x[:, :200])
    assert e.value.status == 5
    with pytest.raises(mxq.MXError) as e:
        mxq.mx_quantize_2d_dual(torch.zeros((200, 256), dtype=torch.bfloat16, device=dev))
    assert e.value.status == 5
    with pytest.raises(mxq.MXError) as e:
        mxq.mx_quantize_2d_dual(x, block_size=16)
    assert e.value.status == 3
    with pytest.raises(mxq.MXError) as e:
        mxq.mx_quantize_2d_dual(x, scaling_mode="floor")
    assert e.value.status == 4
    with pytest.raises(mxq.MXError) as e:
        mxq.mx_quantize_2d_dual(torch.zeros((256, 256), dtype=torch.float16, device=dev))
    assert e.value.status == 2
    q_row, s_row, q_col, s_col = _dirty_outputs(256, 256, dev)
    with pytest.raises(mxq.MXError) as e:   # q_col aliasing q_row
        mxq.mx_quantize_2d_dual(x, out=(q_row, s_row, q_row, s_col))
    assert e.value.status == 8
    with pytest.raises(mxq.MXError) as e:   # output aliasing the input
        mxq.mx_quantize_2d_dual(x, out=(x.view(torch.uint8).reshape(-1)[:65536].view(256, 256), s_row, q_col, s_col))
    assert e.value.status == 8


def test_caller_outputs_checked_before_launch():
    """Caller-supplied outputs of the wrong device, dtype, shape or layout
    raise in the binding; nothing is launched."""
    dev = require_gpu()
    say("binding checks of caller outputs")
    x = torch.zeros((256, 128), dtype=torch.bfloat16, device=dev)
    good = list(_dirty_outputs(256, 128, dev))
    bad_cases = {
        "host q_row": torch.zeros((256, 128), dtype=torch.uint8),
        "short q_col": torch.zeros((128, 128), dtype=torch.uint8, device=dev),
        "int8 s_row": torch.zeros((256, 4), dtype=torch.int8, device=dev),
        "strided s_col": torch.zeros((8, 256), dtype=torch.uint8, device=dev)[:, ::2],
    }
    slots = {"host q_row": 0, "short q_col": 2, "int8 s_row": 1, "strided s_col": 3}
    for name, t in bad_cases.items():
        out = list(good)
        out[slots[name]] = t
        with pytest.raises(ValueError) as e:
            mxq.mx_quantize_2d_dual(x, out=tuple(out))
        assert not isinstance(e.value, mxq.MXError), name
    with pytest.raises(ValueError):
        mxq.mx_quantize_2d_dual(x, out=tuple(good[:3]))
    with pytest.raises(ValueError):      # plain-layout buffers passed for the matrix-core layout
        mxq.mx_quantize_2d_dual(x, out=tuple(good), scale_layout="mfma")
    with pytest.raises(ValueError):
        mxq.mx_quantize_grouped(x, torch.zeros(1, dtype=torch.int32), out=tuple(good))
    for o in good:                       # untouched
        assert int((o != 0xA5).sum()) == 0


# ---------------------------------------------------------------- full sizes
# Every output byte of the workloads at full size is compared with the
# oracle in test_gpu_full_size.py; here, properties of the full-size call.

def test_full_size_mixed_properties():
    """bf16 [8192, 7168]: for finite input the colwise outputs equal the
    rowwise outputs of the transpose, and repeated calls give the same bytes."""
    dev = require_gpu()
    say("full size [8192, 7168]: transposition and determinism")
    xd = bf16_to_dev(synth.dual_mixed())
    out = _dirty_outputs(*xd.shape, dev)
    mxq.mx_quantize_2d_dual(xd, out=out)
    qr_t, sr_t, _, _ = mxq.mx_quantize_2d_dual(xd.t().contiguous())
    torch.cuda.synchronize()
    assert torch.equal(out[2], qr_t) and torch.equal(out[3], sr_t.t())
    again = _dirty_outputs(*xd.shape, dev, 0x11)
    mxq.mx_quantize_2d_dual(xd, out=again)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(out, again))
