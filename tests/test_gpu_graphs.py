"""Every entry point runs on the caller's stream and can be captured in a HIP
graph (the C ABI's convention: no allocation, no synchronization, work only
on the given stream).  Each captured call is replayed several times, with
the outputs overwritten and the device synchronized in between, and every
replay must reproduce the oracle's bytes (casts, MX9) or the eager result
bit for bit (contractions, whose eager result is checked against the oracle
elsewhere).  Calls issued on two streams, whose kernels may overlap, give
the bytes of the same calls made one after another."""
import numpy as np
import pytest
import torch

import mx9_dual_axis_amd as mxq
import oracle
from helpers import bf16_to_dev, host, require_gpu, say
from mx9_dual_axis_amd import synth

pytestmark = pytest.mark.gpu
THREADS = 16
DEV = "cuda:0"


def _codes(g, shape):
    c = g.integers(0, 256, shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38
    return torch.from_numpy(c).to(DEV)


def _replay(graph, outs, check, reps=3):
    for rep in range(reps):
        for o in outs:
            o.view(torch.uint8).fill_(0x5A + rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        check(rep)


def test_mx9_pack_and_unpack_in_a_graph():
    require_gpu()
    say("graph capture: mx9 pack (flat and axis 0) and unpack")
    rows, cols = 512, 1024
    w = synth.mx9_weights(rows, cols, 3, "fp32")
    x = torch.from_numpy(w).to(DEV)
    nb = rows * cols // 16
    q = torch.empty((nb, 16), dtype=torch.int8, device=DEV)
    e = torch.empty((nb,), dtype=torch.uint8, device=DEV)
    p = torch.empty((nb, 1), dtype=torch.uint8, device=DEV)
    qa = torch.empty_like(q)
    ea = torch.empty_like(e)
    pa = torch.empty_like(p)
    y = torch.empty((rows, cols), dtype=torch.bfloat16, device=DEV)
    wq, we, wp = oracle.mx9_pack(w, threads=THREADS)
    wqa, wea, wpa = oracle.mx9_pack_axis(w, 0, threads=THREADS)
    wy = oracle.mx9_unpack(wq, we, wp, rows, cols, out_dtype="bf16", threads=THREADS)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        mxq.mx9_pack(x, out=(q, e, p))          # warm the library outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            mxq.mx9_pack(x, out=(q, e, p))
            mxq.mx9_pack_axis(x, 0, out=(qa, ea, pa))
            mxq.mx9_unpack(q, e, p, rows, cols, torch.bfloat16, out=y)

    def check(rep):
        assert np.array_equal(host(q).reshape(-1).view(np.uint8), np.asarray(wq).reshape(-1).view(np.uint8)), rep
        assert np.array_equal(host(e).reshape(-1), np.asarray(we).reshape(-1)), rep
        assert np.array_equal(host(p).reshape(-1), np.asarray(wp).reshape(-1)), rep
        assert np.array_equal(host(qa).reshape(-1).view(np.uint8), np.asarray(wqa).reshape(-1).view(np.uint8)), rep
        assert np.array_equal(host(ea).reshape(-1), np.asarray(wea).reshape(-1)), rep
        assert np.array_equal(host(y).reshape(-1), np.asarray(wy).reshape(-1)), rep
    _replay(g, (q, e, p, qa, ea, pa, y), check)


def test_matrix_core_cast_and_contractions_in_a_graph():
    require_gpu()
    say("graph capture: grouped cast (mfma layout) -> grouped forward and weight gradient, dense")
    M, K, N, E = 1024, 512, 256, 4
    xb = synth.normal_bf16(M, K, 41)
    offs = torch.tensor([256, 256, 640, 896], dtype=torch.int32, device=DEV)
    xd = bf16_to_dev(xb)
    g = np.random.default_rng(42)
    W = _codes(g, (E, N, K))
    sW = torch.from_numpy(g.integers(118, 137, (E, N * K // 32), dtype=np.uint8)).to(DEV)
    dY = _codes(g, (N, M))
    sdY = torch.from_numpy(g.integers(118, 137, (N * M // 32,), dtype=np.uint8)).to(DEV)
    kw = dict(dtype=torch.uint8, device=DEV)
    cast = (torch.empty((M, K), **kw), torch.empty((M * K // 32,), **kw), torch.empty((K, M), **kw),
            torch.empty((M * K // 32,), **kw))
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    dW = torch.empty((E, K, N), dtype=torch.float32, device=DEV)
    D = torch.empty((M, N), dtype=torch.float32, device=DEV)

    def run():
        mxq.mx_quantize_grouped(xd, offs, out=cast, scale_layout="mfma")
        mxq.mx_grouped_gemm_rows_mfma(cast[0], cast[1], W, sW, offs, out=Y)
        mxq.mx_grouped_gemm_k_mfma(cast[2], cast[3], dY, sdY, offs, out=dW)
        mxq.mx_gemm_nt_mfma(cast[0], cast[1], W[0], sW[0], out=D)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        run()
    s.synchronize()
    want = [t.clone() for t in (*cast, Y, dW, D)]
    rc, wcast = oracle.mxfp8_grouped(xb, offs.cpu().numpy(), threads=THREADS)
    assert rc == 0
    assert np.array_equal(host(cast[0]), wcast[0]) and np.array_equal(host(cast[2]), wcast[2])
    assert np.array_equal(host(cast[1]), oracle.scales_to_mfma(wcast[1]))
    assert np.array_equal(host(cast[3]), oracle.scales_to_mfma(np.ascontiguousarray(wcast[3].T)))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            run()

    def check(rep):
        for a, b in zip((*cast, Y, dW, D), want):
            assert torch.equal(a, b), rep
    _replay(graph, (*cast, Y, dW, D), check)


def test_concurrent_calls_on_two_streams():
    """The library holds no state between calls: the cast, the MX9 pack and
    unpack and a contraction issued alternately on two streams (so that their
    kernels may run at the same time) give the same bytes as the same calls
    made one after another on the default stream."""
    require_gpu()
    say("concurrent calls on two streams")
    g = np.random.default_rng(77)
    M, N = 1024, 2048
    xs = [bf16_to_dev(synth.special_matrix(M, N, 40 + i)) for i in range(2)]
    ws = [torch.from_numpy(synth.mx9_weights(512, 1000, 50 + i, "fp32")).to(DEV) for i in range(2)]
    As = [_codes(g, (512, 1024)) for _ in range(2)]
    sAs = [torch.from_numpy(g.integers(118, 137, (512, 32), dtype=np.uint8)).to(DEV) for _ in range(2)]

    def work(i):
        cast = mxq.mx_quantize_2d_dual(xs[i])
        q, e, p = mxq.mx9_pack(ws[i])
        y = mxq.mx9_unpack(q, e, p, ws[i].shape[0], ws[i].shape[1], out_dtype=torch.bfloat16)
        c = mxq.mx_gemm_nt(As[i], sAs[i], As[1 - i], sAs[1 - i])
        return list(cast) + [q, e, p, y, c]

    want = [work(i) for i in range(2)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        got = [None, None]
        for i in (0, 1):
            with torch.cuda.stream(streams[i]):
                got[i] = work(i)
        torch.cuda.synchronize()
        for i in (0, 1):
            for k, (a, b) in enumerate(zip(got[i], want[i])):
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"rep {rep} stream {i} output {k}"
