#!/usr/bin/env python3
"""Benchmark of the single-pass MX quantization hot path on one MI355X.

One step = the whole path over one batch: the fused dual-axis MXFP8 cast of a
bf16 [32768, 8192] matrix (the stress workload: N(0,1) with subnormal and
near-max tiles and Inf/NaN at rate 1e-6), then MX9 pack of the same matrix,
then MX9 unpack back to bf16.  Inputs are resident in HBM before timing.

Prints ONE JSON line.  ``value`` is the step's algorithmic bytes (what the
method must read and write, per kernel) divided by the step time, in GB/s.
``roofline`` describes the dominant operation, the dual-axis cast: its
algorithmic bytes per call over its average call time from HIP events on the
launch stream (the call is one kernel), against MI355X's 8 TB/s HBM peak.
``traffic`` is the HBM byte count per call from the committed rocprofv3
FETCH_SIZE / WRITE_SIZE summary, reported only while the kernel source
matches the source those counters were taken on.  ``gpu_roofs`` gives, for
context, what the same GPU reaches for a plain copy, read and write of the
cast's byte volume with hand-written streaming kernels, and
``roofline.frac_of_gpu_copy`` the cast's rate against that copy.
``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload (a multithreaded leg of about ten seconds and a single-thread leg).

``configs`` holds the other workloads, each timed per call with HIP events
while rotating three input/output buffer sets so that MI355X's 256 MB
last-level cache cannot serve a call from the previous one: the dense cast of
the mixed-magnitude bf16 [8192, 7168] matrix, the grouped cast of bf16
[16384, 5120] with 64 groups, and MX9 pack/unpack of the fp32 and bf16
[4096, 14336] weights in three forms: three tensors along the last axis,
one tensor of 18-byte records, and three tensors along axis 0; the casts and
contractions in the matrix-core scale layout; and the dual-axis cast of the
stress matrix timed alone (back-to-back calls), to compare with its time
inside the step.  Each workload is also timed back to back between one pair
of events over the same rotation (``back_to_back_us``), which leaves out the
idle time of the per-call event records.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--skip-cpu] [--skip-configs]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
EVENT_EVERY = 5            # timed steps per event-bracketed dual-axis call
M, N = 32768, 8192
DUAL_BYTES_PER_ELEM = 2 + 1 + 1 + 1 / 32 + 1 / 32          # bf16 in; E4M3 x2 + E8M0 x2 out
PACK_BF16_BYTES_PER_ELEM = 2 + 1 + 1 / 16 + 1 / 16         # bf16 in; q + max_exp + prime out
UNPACK_BF16_BYTES_PER_ELEM = 1 + 1 / 16 + 1 / 16 + 2       # q + max_exp + prime in; bf16 out
KERNEL_SOURCES = ["mx9_dual_axis_amd/csrc/dual_axis.hip"]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "dual_axis_stress_counters.txt")


def source_digest() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic():
    """HBM bytes per dual-axis launch from the committed counter summary, or
    None when absent or taken on a different kernel source."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    txt = open(COUNTERS_FILE).read()
    m_src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_src or not m_b or m_src.group(1) != source_digest():
        return None
    return float(m_b.group(1))


def gpu_roofs(dev, volume: int, launches: int = 10):
    """What this GPU achieves for plain streams of `volume` bytes: a copy
    (half the volume read, half written), a read and a write, each by the
    hand-written kernels of libmxq_roof.so (one 16-byte non-temporal access
    per lane, 4 KiB per workgroup), alternating two buffers of `volume` bytes
    so the 256 MB last-level cache cannot serve one launch from the last."""
    import torch
    lib_path = os.path.join(ROOT, "mx9_dual_axis_amd", "libmxq_roof.so")
    if not os.path.exists(lib_path):
        raise RuntimeError(f"{lib_path} is missing (run __graft_entry__.build())")
    lib = ctypes.CDLL(lib_path)
    lib.mxq_roof.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.mxq_roof.restype = ctypes.c_int
    vol = volume // 8192 * 8192
    half = vol // 2
    bufs = [torch.zeros(vol, dtype=torch.uint8, device=dev) for _ in range(2)]
    sink = torch.zeros(4096, dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def launch(kind, i):
        b = bufs[i % 2].data_ptr()
        if kind == 0:
            rc = lib.mxq_roof(0, b, b + half, half, stream)
        elif kind == 1:
            rc = lib.mxq_roof(1, b, sink.data_ptr(), vol, stream)
        else:
            rc = lib.mxq_roof(2, None, b, vol, stream)
        if rc != 0:
            raise RuntimeError(f"mxq_roof({kind}) failed ({rc})")

    out = {}
    for kind, name in ((0, "copy"), (1, "read"), (2, "write")):
        for i in range(2):
            launch(kind, i)
        e0, e1 = HipEvent(), HipEvent()
        e0.record()
        for i in range(launches):
            launch(kind, i)
        e1.record()
        torch.cuda.synchronize()
        out[f"{name}_GB_s"] = round(vol * launches / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    out["bytes_per_launch"] = vol
    out["kernels"] = "libmxq_roof.so: one 16-byte non-temporal load and/or store per lane, 4 KiB per workgroup"
    del bufs

    # the cast's own three streams, each alone (mxq_roof_cast_stream): the
    # tiled bf16 read, the q_row write and the q_col write, in the cast's tile
    # order with its per-lane accesses
    lib.mxq_roof_cast_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_void_p]
    lib.mxq_roof_cast_stream.restype = ctypes.c_int
    streams = {}
    for sid, name, nbytes in ((0, "x_read", 2 * M * N), (1, "q_row_write", M * N), (2, "q_col_write", M * N)):
        sbufs = [torch.zeros(nbytes, dtype=torch.uint8, device=dev) for _ in range(2)]

        def launch(i):
            rc = lib.mxq_roof_cast_stream(sid, sbufs[i % 2].data_ptr(), sink.data_ptr(), M, N, stream)
            if rc != 0:
                raise RuntimeError(f"mxq_roof_cast_stream({sid}) failed ({rc})")

        for i in range(2):
            launch(i)
        e0, e1 = HipEvent(), HipEvent()
        e0.record()
        for i in range(launches):
            launch(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / launches
        streams[name] = {"us": round(us, 2), "bytes": nbytes, "GB_s": round(nbytes / us / 1e3, 1)}
        del sbufs
    streams["sum_us"] = round(sum(v["us"] for v in streams.values()), 2)
    out["cast_streams_alone"] = streams
    del sink
    return out


def cpu_baseline(xb, threads: int, budget_s: float, single_rows: int):
    """The oracle, as it stands, on leading rows of the workload: dual-axis
    cast + MX9 pack + MX9 unpack (bf16).  The multithreaded leg processes
    chunks of 256 rows until ``budget_s`` seconds have passed; the
    single-thread leg processes ``single_rows`` rows."""
    import oracle
    per_row = N * (DUAL_BYTES_PER_ELEM + PACK_BF16_BYTES_PER_ELEM + UNPACK_BF16_BYTES_PER_ELEM)

    def run(rows_slice, nthreads):
        oracle.mxfp8_dual(rows_slice, threads=nthreads)
        q, e, p = oracle.mx9_pack(rows_slice, threads=nthreads)
        oracle.mx9_unpack(q, e, p, rows_slice.shape[0], N, "bf16", threads=nthreads)

    chunk, rows, busy = 256, 0, 0.0
    while busy < budget_s and rows + chunk <= xb.shape[0]:
        t0 = time.perf_counter()
        run(xb[rows:rows + chunk], threads)
        busy += time.perf_counter() - t0
        rows += chunk
    t0 = time.perf_counter()
    run(xb[:single_rows], 1)
    one = time.perf_counter() - t0
    return {"value": round(rows * per_row / busy / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"first {rows} of {M} rows ({rows * N} elements) of the stress workload, "
                      f"dual-axis cast + MX9 pack + unpack, {busy:.1f} s on {threads} threads",
            "single_thread": {"value": round(single_rows * per_row / one / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"first {single_rows} rows, same operations, {one:.1f} s"}}


class HipEvent:
    """A HIP timing event on the current torch stream, created with
    hipEventDisableSystemFence.  A default event performs a system-scope
    release (L2 writeback and invalidation) when it is recorded, which leaves
    the GPU idle for about 6 us per record on MI355X and disturbs the work
    that follows; the HIP runtime documents this flag for events that only
    measure time.  The HIP runtime is the one torch has already loaded."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            hip = ctypes.CDLL("libamdhip64.so.7")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        self.h = ctypes.c_void_p()
        rc = self._lib().hipEventCreateWithFlags(ctypes.byref(self.h), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        import torch
        rc = self._lib().hipEventRecord(self.h, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (both recorded and complete)."""
        ms = ctypes.c_float()
        rc = self._lib().hipEventElapsedTime(ctypes.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.h:
            self._hip.hipEventDestroy(self.h)


class Timings(list):
    """Per-call durations in seconds; `back_to_back` is the average duration
    of the same calls launched back to back between one pair of events."""
    back_to_back = None


def time_rotating(calls, launches: int):
    """Per-call durations (seconds, from HIP events on the launch stream) of
    `launches` calls cycling through `calls` (one per buffer set).  Each
    bracketed call also holds the idle time of its two event records (about
    5 us on MI355X), so the same calls are then timed back to back as well."""
    import torch
    for c in calls:
        c()
    evs = [(HipEvent(), HipEvent()) for _ in range(launches)]
    for a, b in evs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    calls[-1]()         # a queued call, so the first bracketed one does not wait for the host
    for i, (a, b) in enumerate(evs):
        a.record()
        calls[i % len(calls)]()
        b.record()
    torch.cuda.synchronize()
    ts = Timings(a.elapsed_time(b) * 1e-3 for a, b in evs)
    e0, e1 = HipEvent(), HipEvent()
    e0.record()
    for i in range(launches):
        calls[i % len(calls)]()
    e1.record()
    torch.cuda.synchronize()
    ts.back_to_back = e0.elapsed_time(e1) * 1e-3 / launches
    return ts


def summarize(ts, nbytes):
    b2b = getattr(ts, "back_to_back", None)
    ts = sorted(ts)
    med = ts[len(ts) // 2]
    mean = sum(ts) / len(ts)
    out = {"us": round(mean * 1e6, 2), "median_us": round(med * 1e6, 2), "bytes": int(nbytes),
           "GB_s": round(nbytes / mean / 1e9, 1), "frac": round(nbytes / mean / 1e9 / PEAK_HBM_GBS, 4)}
    if b2b:
        out.update({"back_to_back_us": round(b2b * 1e6, 2), "back_to_back_GB_s": round(nbytes / b2b / 1e9, 1),
                    "back_to_back_frac": round(nbytes / b2b / 1e9 / PEAK_HBM_GBS, 4)})
    return out


def measure_configs(dev, launches: int, sets: int = 3):
    """The other workloads, each over `sets` rotating buffer sets."""
    import numpy as np
    import torch

    import mx9_dual_axis_amd as mxq
    from mx9_dual_axis_amd import synth

    def dev_bf16(xb):
        return torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)

    u8 = dict(dtype=torch.uint8, device=dev)
    res = {}

    def dual_sets(xb, offs=None, layout="plain"):
        Mc, Nc = xb.shape
        x0 = dev_bf16(xb)
        xs = [x0] + [x0.clone() for _ in range(sets - 1)]
        outs = [(torch.empty((Mc, Nc), **u8), torch.empty((Mc, Nc // 32), **u8),
                 torch.empty((Nc, Mc), **u8), torch.empty((Mc // 32, Nc), **u8)) for _ in range(sets)]
        if layout == "mfma":
            outs = [(q, sr.view(-1), qc, sc.view(-1)) for q, sr, qc, sc in outs]
        if offs is None:
            return [lambda x=x, o=o: mxq.mx_quantize_2d_dual(x, out=o, scale_layout=layout) for x, o in zip(xs, outs)]
        od = torch.from_numpy(offs).to(dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        return [lambda x=x, o=o: mxq.mx_quantize_grouped(x, od, err=err, out=o, scale_layout=layout)
                for x, o in zip(xs, outs)]

    print("bench: dense cast, mixed bf16 [8192, 7168]", file=sys.stderr, flush=True)
    xb = synth.dual_mixed()
    calls = dual_sets(xb)
    res["dual_mixed"] = dict(workload="dense dual-axis cast, mixed-magnitude bf16 [8192, 7168]",
                             **summarize(time_rotating(calls, launches), xb.size * DUAL_BYTES_PER_ELEM))
    del calls
    calls = dual_sets(xb, layout="mfma")
    res["dual_mixed_mfma"] = dict(workload="dense dual-axis cast, mixed-magnitude bf16 [8192, 7168], scales in "
                                           "the matrix-core layout",
                                  **summarize(time_rotating(calls, launches), xb.size * DUAL_BYTES_PER_ELEM))
    del calls

    print("bench: grouped cast, bf16 [16384, 5120], 64 groups", file=sys.stderr, flush=True)
    xb, offs = synth.grouped()
    calls = dual_sets(xb, offs)
    res["grouped"] = dict(workload="grouped dual-axis cast, bf16 [16384, 5120], 64 groups, offs[-1] = "
                                   f"{int(offs[-1])}",
                          **summarize(time_rotating(calls, launches), xb.size * DUAL_BYTES_PER_ELEM + 4 * offs.size))
    del calls
    calls = dual_sets(xb, offs, layout="mfma")
    res["grouped_mfma"] = dict(workload="grouped dual-axis cast, bf16 [16384, 5120], 64 groups, scales in the "
                                        "matrix-core layout",
                               **summarize(time_rotating(calls, launches), xb.size * DUAL_BYTES_PER_ELEM + 4 * offs.size))
    del calls

    print("bench: MX9 pack/unpack, weights [4096, 14336] fp32 and bf16", file=sys.stderr, flush=True)
    w32 = synth.mx9_weights(4096, 14336, 4, "fp32")
    rows, cols = w32.shape
    nb = rows * cols // 16
    for name, host_x, tdt, in_b in (("fp32", w32, torch.float32, 4), ("bf16", synth.to_bf16_bits(w32),
                                                                      torch.bfloat16, 2)):
        x0 = (torch.from_numpy(host_x).to(dev) if name == "fp32" else dev_bf16(host_x))
        xs = [x0] + [x0.clone() for _ in range(sets - 1)]
        packs = [(torch.empty((nb, 16), dtype=torch.int8, device=dev), torch.empty((nb,), **u8),
                  torch.empty((nb, 1), **u8)) for _ in range(sets)]
        ys = [torch.empty((rows, cols), dtype=tdt, device=dev) for _ in range(sets)]
        elem_b = in_b + 1 + 1 / 16 + 1 / 16
        pk = [lambda x=x, o=o: mxq.mx9_pack(x, out=o) for x, o in zip(xs, packs)]
        res[f"mx9_pack_{name}"] = dict(workload=f"MX9 pack, {name} weights [4096, 14336]",
                                       **summarize(time_rotating(pk, launches), rows * cols * elem_b))
        up = [lambda o=o, y=y: mxq.mx9_unpack(*o, rows, cols, out=y) for o, y in zip(packs, ys)]
        res[f"mx9_unpack_{name}"] = dict(workload=f"MX9 unpack to {name}, [4096, 14336]",
                                         **summarize(time_rotating(up, launches), rows * cols * elem_b))
        del packs, pk, up
        # the same weights as one byte tensor of 18-byte records (last axis)
        recs = [torch.empty((rows, cols // 16 * 18), **u8) for _ in range(sets)]
        pk = [lambda x=x, o=o: mxq.mx9_pack_records(x, -1, out=o) for x, o in zip(xs, recs)]
        res[f"mx9_pack_records_{name}"] = dict(workload=f"MX9 pack to 18-byte records, {name} weights [4096, 14336]",
                                               **summarize(time_rotating(pk, launches), rows * cols * elem_b))
        up = [lambda o=o, y=y: mxq.mx9_unpack_records(o, (rows, cols), -1, out=y) for o, y in zip(recs, ys)]
        res[f"mx9_unpack_records_{name}"] = dict(workload=f"MX9 unpack from records to {name}, [4096, 14336]",
                                                 **summarize(time_rotating(up, launches), rows * cols * elem_b))
        del recs, pk, up
        # blocks along axis 0 (down the columns) of the same weights
        packs = [(torch.empty((nb, 16), dtype=torch.int8, device=dev), torch.empty((nb,), **u8),
                  torch.empty((nb, 1), **u8)) for _ in range(sets)]
        pk = [lambda x=x, o=o: mxq.mx9_pack_axis(x, 0, out=o) for x, o in zip(xs, packs)]
        res[f"mx9_pack_axis0_{name}"] = dict(workload=f"MX9 pack along axis 0, {name} weights [4096, 14336]",
                                             **summarize(time_rotating(pk, launches), rows * cols * elem_b))
        up = [lambda o=o, y=y: mxq.mx9_unpack_axis(*o, (rows, cols), 0, out=y) for o, y in zip(packs, ys)]
        res[f"mx9_unpack_axis0_{name}"] = dict(workload=f"MX9 unpack along axis 0 to {name}, [4096, 14336]",
                                               **summarize(time_rotating(up, launches), rows * cols * elem_b))
        del xs, packs, ys, pk, up
    torch.cuda.synchronize()
    res.update(measure_gemm(dev, launches))
    return res


PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0


def measure_gemm(dev, launches: int):
    """The consumer contraction on the matrix cores: the routed-expert forward
    and weight gradient over the grouped activation buffer (its cast outputs,
    64 experts of 2048 output features), and a dense 8192^3 product.  Rates
    are useful FLOP/s (2 per multiply-add over the covered rows) and minimal
    HBM bytes, each workload judged against the roof that binds it: the
    routed-expert shapes are HBM-bound (each expert's weights serve about 192
    rows; the weight gradient writes a [5120, 2048] result per group), the
    dense product is bound by the matrix cores."""
    import numpy as np
    import torch

    import mx9_dual_axis_amd as mxq
    from mx9_dual_axis_amd import synth

    def tsum(ts, flops, workload, nbytes):
        """Rates against both roofs; `bound` is the one that limits the
        workload at peak (time at the roof = the larger of FLOP / 5.0 PFLOP/s
        and minimal HBM bytes / 8 TB/s), `frac` = that time / measured time."""
        b2b = getattr(ts, "back_to_back", None)
        ts = sorted(ts)
        mean = sum(ts) / len(ts)
        tf = flops / mean / 1e12
        t_mfma = flops / (PEAK_FP8_TFLOPS * 1e12)
        t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
        out = {"workload": workload, "us": round(mean * 1e6, 2), "median_us": round(ts[len(ts) // 2] * 1e6, 2),
               "flop": int(flops), "hbm_bytes": int(nbytes), "TFLOP_s": round(tf, 1),
               "GB_s": round(nbytes / mean / 1e9, 1), "bound": "mfma" if t_mfma >= t_hbm else "hbm",
               "frac": round(max(t_mfma, t_hbm) / mean, 4)}
        if b2b:
            out.update({"back_to_back_us": round(b2b * 1e6, 2), "back_to_back_frac": round(max(t_mfma, t_hbm) / b2b, 4)})
        return out

    print("bench: MXFP8 contractions (grouped forward, weight gradient, dense)", file=sys.stderr, flush=True)
    g = np.random.default_rng(11)
    xb, offs = synth.grouped()
    Mt, K = xb.shape
    N, E = 2048, len(offs)
    covered = int(offs[-1])
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
    od = torch.from_numpy(offs).to(dev)
    q_row, s_row, q_col, s_col = mxq.mx_quantize_grouped(x, od)
    m_row, ms_row, m_col, ms_col = mxq.mx_quantize_grouped(x, od, scale_layout="mfma")
    del x

    def codes(shape):
        c = torch.from_numpy(g.integers(0, 256, shape, dtype=np.uint8)).to(dev)
        return torch.where((c & 0x7F) == 0x7F, torch.full_like(c, 0x38), c)

    def scales(shape):
        return torch.from_numpy(g.integers(118, 137, shape, dtype=np.uint8)).to(dev)

    res = {}
    W = codes((E, N, K))
    sW = scales((E, N, K // 32))
    out = torch.empty((Mt, N), dtype=torch.bfloat16, device=dev)
    fwd = [lambda: mxq.mx_grouped_gemm_rows(q_row, s_row, W, sW, od, out=out)]
    # minimal HBM bytes: covered activation rows and their scales, the weights
    # and scales of every non-empty expert, the whole bf16 output
    busy = int(np.count_nonzero(np.diff(np.concatenate([[0], offs])) > 0))
    fwd_bytes = covered * K * (1 + 1 / 32) + busy * N * K * (1 + 1 / 32) + Mt * N * 2
    res["gemm_grouped_forward"] = tsum(time_rotating(fwd, launches), 2.0 * covered * N * K,
                                       f"grouped forward, cast activations [{Mt}, {K}] (64 groups, {covered} rows) "
                                       f"x 64 experts [{N}, {K}] -> bf16", fwd_bytes)
    sWm = sW.reshape(E, N * K // 32)       # random bytes: read as the matrix-core layout
    fwd = [lambda: mxq.mx_grouped_gemm_rows_mfma(m_row, ms_row, W, sWm, od, out=out)]
    res["gemm_grouped_forward_mfma"] = tsum(time_rotating(fwd, launches), 2.0 * covered * N * K,
                                            "grouped forward as above, scales in the matrix-core layout", fwd_bytes)
    del W, sW, sWm, out, fwd
    dY = codes((N, Mt))
    sdY = scales((Mt // 32, N))
    dW = torch.empty((E, K, N), dtype=torch.bfloat16, device=dev)
    wg = [lambda: mxq.mx_grouped_gemm_k(q_col, s_col.t(), dY, sdY.t(), od, out=dW)]
    # minimal HBM bytes: the covered token columns of both operands with
    # their scales, and the whole bf16 output of every group
    wg_bytes = covered * (K + N) * (1 + 1 / 32) + E * K * N * 2
    res["gemm_grouped_wgrad"] = tsum(time_rotating(wg, launches), 2.0 * covered * N * K,
                                     f"grouped weight gradient, cast q_col [{K}, {Mt}] x dY [{N}, {Mt}] over 64 groups "
                                     f"-> bf16 [64, {K}, {N}]", wg_bytes)
    sdYm = sdY.reshape(-1)
    wg = [lambda: mxq.mx_grouped_gemm_k_mfma(m_col, ms_col, dY, sdYm, od, out=dW)]
    res["gemm_grouped_wgrad_mfma"] = tsum(time_rotating(wg, launches), 2.0 * covered * N * K,
                                          "grouped weight gradient as above, scales in the matrix-core layout",
                                          wg_bytes)
    del dY, sdY, sdYm, dW, wg, q_row, s_row, q_col, s_col, m_row, ms_row, m_col, ms_col
    D = 8192
    A, B = codes((D, D)), codes((D, D))
    sA, sB = scales((D, D // 32)), scales((D, D // 32))
    C = torch.empty((D, D), dtype=torch.bfloat16, device=dev)
    dn = [lambda: mxq.mx_gemm_nt(A, sA, B, sB, out=C)]
    dn_bytes = 2 * D * D * (1 + 1 / 32) + D * D * 2
    res["gemm_dense_8192"] = tsum(time_rotating(dn, launches), 2.0 * D ** 3, "dense [8192, 8192, 8192] -> bf16",
                                  dn_bytes)
    sAm, sBm = sA.reshape(-1), sB.reshape(-1)
    dn = [lambda: mxq.mx_gemm_nt_mfma(A, sAm, B, sBm, out=C)]
    res["gemm_dense_8192_mfma"] = tsum(time_rotating(dn, launches), 2.0 * D ** 3,
                                       "dense [8192, 8192, 8192] -> bf16, scales in the matrix-core layout", dn_bytes)
    del A, B, sA, sB, sAm, sBm, C, dn
    torch.cuda.synchronize()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--skip-cpu", action="store_true", help="omit the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="multithreaded oracle leg budget")
    ap.add_argument("--cpu-single-rows", type=int, default=256)
    ap.add_argument("--skip-configs", action="store_true", help="omit the other workloads")
    ap.add_argument("--config-launches", type=int, default=30)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(the method needs no exchange between GPUs; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mx9_dual_axis_amd as mxq
    from mx9_dual_axis_amd import synth

    dev = torch.device("cuda:0")
    print("bench: generating the stress workload bf16 [32768, 8192] (seed 5)", file=sys.stderr, flush=True)
    xb = synth.stress(M, N, 5)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
    u8 = dict(dtype=torch.uint8, device=dev)
    dual_out = (torch.empty((M, N), **u8), torch.empty((M, N // 32), **u8),
                torch.empty((N, M), **u8), torch.empty((M // 32, N), **u8))
    nb = M * N // 16
    mx9_out = (torch.empty((nb, 16), dtype=torch.int8, device=dev), torch.empty((nb,), **u8),
               torch.empty((nb, 1), **u8))
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def step(ev=None, all_kernels=False):
        if ev: ev[0].record()
        mxq.mx_quantize_2d_dual(x, out=dual_out)
        if ev: ev[1].record()
        mxq.mx9_pack(x, out=mx9_out)
        if ev and all_kernels: ev[2].record()
        mxq.mx9_unpack(*mx9_out, M, N, out=y)
        if ev and all_kernels: ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, bracketed by synchronizations.  Each
    # event record still costs the GPU a little time, so inside the timed
    # region only the dual-axis call (the roofline's operation) is bracketed
    # by events.  Every event is recorded once before the timed region.
    def make_events(n, count=None):
        evs = [[HipEvent() for _ in range(n)] for _ in range(args.steps if count is None else count)]
        for ev in evs:
            for e in ev:
                e.record()
        torch.cuda.synchronize()
        return evs

    # The dual-axis call of every EVENT_EVERY-th timed step is bracketed by
    # events: each record leaves the GPU idle for a few microseconds, which
    # bracketing every step would add to the step time.  The bracketed steps
    # are the last of each run of EVENT_EVERY, never the first step after the
    # synchronization: with an empty queue the GPU would reach the opening
    # event before the host had enqueued the cast, and the host's enqueue
    # time would count as kernel time.
    bracketed = [k for k in range(args.steps) if k % EVENT_EVERY == EVENT_EVERY - 1] or [args.steps - 1]
    evs = make_events(2, len(bracketed))
    slot = {k: i for i, k in enumerate(bracketed)}
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[slot[k]] if k in slot else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dual_times = [ev[0].elapsed_time(ev[1]) * 1e-3 for ev in evs]

    # per-kernel breakdown: a second, separate pass of K steps with events
    # between all three calls (not the timed region), after two unbracketed
    # steps that give the GPU a queue to work through
    evs4 = make_events(4)
    step()
    step()
    for k in range(args.steps):
        step(evs4[k], all_kernels=True)
    torch.cuda.synchronize()
    per_kernel = {"dual_axis": [], "mx9_pack": [], "mx9_unpack": []}
    for ev in evs4:
        per_kernel["dual_axis"].append(ev[0].elapsed_time(ev[1]) * 1e-3)
        per_kernel["mx9_pack"].append(ev[1].elapsed_time(ev[2]) * 1e-3)
        per_kernel["mx9_unpack"].append(ev[2].elapsed_time(ev[3]) * 1e-3)
    elems = M * N
    kbytes = {"dual_axis": elems * DUAL_BYTES_PER_ELEM, "mx9_pack": elems * PACK_BF16_BYTES_PER_ELEM,
              "mx9_unpack": elems * UNPACK_BF16_BYTES_PER_ELEM}
    kernels = {k: summarize(ts, kbytes[k]) for k, ts in per_kernel.items()}
    kernels["note"] = "separate pass with events between all three calls; the timed region brackets only the dual-axis call"
    step_bytes = sum(kbytes.values())
    ms_per_step = wall / args.steps * 1e3
    value = step_bytes / (wall / args.steps) / 1e9

    # context: a device-to-device copy of one dual-axis launch's byte volume
    half = int(kbytes["dual_axis"] // 2)
    src = torch.empty(half, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = HipEvent(), HipEvent()
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * half * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    # and the same volume through torch's vectorized elementwise kernel (a
    # streaming read and write of 16-byte pieces; hipMemcpyAsync's copy kernel
    # is slower on MI355X)
    src32, dst32 = src.view(torch.int32), dst.view(torch.int32)
    torch.bitwise_not(src32, out=dst32)
    e0, e1 = HipEvent(), HipEvent()
    e0.record()
    for _ in range(10):
        torch.bitwise_not(src32, out=dst32)
    e1.record()
    torch.cuda.synchronize()
    stream_gbs = 2 * half * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst, src32, dst32
    # and by the hand-written streams: this GPU's own roof for the cast's volume
    roofs = gpu_roofs(dev, int(kbytes["dual_axis"]))

    # context: the dual-axis cast alone on the same matrix, back-to-back calls
    # alternating two output sets (the 1.09 GB per call exceeds the 256 MB
    # last-level cache, so no call is served from the previous one)
    alone = None
    if not args.skip_configs:
        print("bench: dual-axis cast alone on the stress matrix", file=sys.stderr, flush=True)
        outs2 = [dual_out, tuple(torch.empty_like(t) for t in dual_out)]
        calls = [lambda o=o: mxq.mx_quantize_2d_dual(x, out=o) for o in outs2]
        alone = dict(workload="dense dual-axis cast alone (back-to-back calls), stress bf16 [32768, 8192]",
                     **summarize(time_rotating(calls, args.config_launches), kbytes["dual_axis"]))
        del outs2, calls

    dual = summarize(dual_times, kbytes["dual_axis"])
    line = {
        "metric": "achieved HBM GB/s (fraction of MI355X peak) for dual-axis MXFP8 + MX9",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded stress workload: N(0,1), 0.5% subnormal tiles, 0.5% near-max tiles, Inf/NaN 1e-6)",
        "config": {"workload": "stress bf16 [32768, 8192]: dual-axis MXFP8 cast + MX9 pack + MX9 unpack to bf16",
                   "M": M, "N": N, "block_mxfp8": 32, "block_mx9": 16, "scaling_mode": "rceil",
                   "step_algorithmic_bytes": int(step_bytes)},
        "roofline": {"bound": "hbm", "achieved": dual["GB_s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(dual["GB_s"] / PEAK_HBM_GBS, 4), "traffic": committed_traffic(),
                     "kernel": "dual_axis_kernel<false, 0> (one dual-axis call)",
                     "algorithmic_bytes_per_launch": dual["bytes"],
                     "avg_launch_us": dual["us"],
                     "launches_timed": len(dual_times),
                     "timed_every_nth_step": EVENT_EVERY,
                     "bracketed_steps": bracketed,
                     "frac_of_gpu_copy": round(dual["GB_s"] / roofs["copy_GB_s"], 4)},
        "kernels": kernels,
        "copy_GB_s": round(copy_gbs, 1),
        "stream_copy_GB_s": round(stream_gbs, 1),
        "gpu_roofs": roofs,
        "kernel_source_sha256_16": source_digest(),
    }
    del x, dual_out, mx9_out, y
    line["configs"] = None if args.skip_configs else {"dual_stress_alone": alone,
                                                      **measure_configs(dev, args.config_launches)}
    if not args.skip_cpu:
        threads = max(1, min(16, os.cpu_count() or 1))
        print(f"bench: timing the CPU oracle for {args.cpu_seconds:.0f} s on {threads} threads", file=sys.stderr,
              flush=True)
        line["cpu_baseline"] = cpu_baseline(xb, threads, args.cpu_seconds, args.cpu_single_rows)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
