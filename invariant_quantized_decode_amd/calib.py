"""Calibration rates that frame the decode projection's roofline figures (libw8calib.so, declared
in include/w8calib.h): the practical HBM read ceiling of one launch, and the dense bf16
matrix-core rate.  Not part of the decode path; bench.py reports both beside its line.

Marshalling only, like the main binding: both measurements run the library's kernels and fail
loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import math
import os

_LIB = None
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw8calib.so")

READ_THREADS = 512   # threads per workgroup of w8c_stream_read
MFMA_THREADS = 256   # threads per workgroup of w8c_mfma_bf16
MFMA_CHAINS = 4      # independent accumulator chains per wave
MFMA_FLOPS = 2 * 32 * 32 * 16  # one v_mfma_f32_32x32x16_bf16


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.w8c_stream_read.argtypes, L.w8c_stream_read.restype = [P, I64, I32, P, SZ, P], ctypes.c_int
        L.w8c_mfma_bf16.argtypes, L.w8c_mfma_bf16.restype = [I32, I32, P, SZ, P], ctypes.c_int
        L.w8c_strip_read.argtypes, L.w8c_strip_read.restype = [P, P, I32, I32, I32, P, SZ, P], ctypes.c_int
        _LIB = L
    return _LIB


def _check(status: int, what: str) -> None:
    if status != 0:
        raise RuntimeError(f"{what} failed with status {status}")


def stream_read_gbs(nbytes: int, workgroups=(192, 256, 512, 1024, 2048), replays: int = 8) -> dict:
    """GB/s of one launch that reads `nbytes` once, per workgroup count.  The buffers rotate over
    copies totalling >= 1 GiB (the 256 MB Infinity Cache cannot serve them); launches are replayed
    from a HIP graph and timed with events on the graph's stream."""
    import torch
    L = _lib()
    dev = torch.device("cuda", torch.cuda.current_device())
    nbytes = nbytes // 16 * 16
    copies = max(2, math.ceil((1 << 30) / nbytes))
    bufs = [torch.zeros(nbytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
    sink = torch.empty(max(workgroups) * READ_THREADS, dtype=torch.int32, device=dev)
    stream = torch.cuda.Stream()
    out = {}
    for wg in workgroups:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(graph, stream=stream):
                for b in bufs:
                    _check(L.w8c_stream_read(b.data_ptr(), nbytes, wg, sink.data_ptr(), sink.numel() * 4,
                                             stream.cuda_stream), "w8c_stream_read")
            graph.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(replays):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) / 1e3 / (replays * copies)
        out[wg] = nbytes / sec / 1e9
        del graph
    del bufs, sink
    return out


def strip_read_gbs(N: int, K: int, workgroups: int = 256, replays: int = 8) -> float:
    """GB/s (codes + scales) of one launch that reads the packed layout of an [N, K] projection the
    way the persistent projection streams it (w8c_strip_read), over copies totalling >= 1 GiB,
    replayed from a HIP graph and timed with events on the graph's stream."""
    import torch
    L = _lib()
    dev = torch.device("cuda", torch.cuda.current_device())
    strips, pairs = (N + 31) // 32, (K // 32 + 1) // 2
    cb, sb = strips * pairs * 2048, strips * pairs * 128
    copies = max(2, math.ceil((1 << 30) / (cb + sb)))
    bufs = [(torch.zeros(cb, dtype=torch.uint8, device=dev), torch.zeros(sb, dtype=torch.uint8, device=dev))
            for _ in range(copies)]
    sink = torch.empty(workgroups * READ_THREADS, dtype=torch.int32, device=dev)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            for c, s in bufs:
                _check(L.w8c_strip_read(c.data_ptr(), s.data_ptr(), strips, pairs, workgroups, sink.data_ptr(),
                                        sink.numel() * 4, stream.cuda_stream), "w8c_strip_read")
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(replays):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / (replays * copies)
    del graph, bufs, sink
    return (cb + sb) / sec / 1e9


def mfma_bf16_tflops(workgroups: int = 4096, iters: int = 2048, launches: int = 3) -> float:
    """Dense bf16 matrix-core TFLOP/s: every wave runs independent chains of
    v_mfma_f32_32x32x16_bf16 with no memory traffic."""
    import torch
    L = _lib()
    dev = torch.device("cuda", torch.cuda.current_device())
    sink = torch.empty(workgroups * MFMA_THREADS, dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        _check(L.w8c_mfma_bf16(workgroups, iters, sink.data_ptr(), sink.numel() * 4, stream.cuda_stream),
               "w8c_mfma_bf16")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            _check(L.w8c_mfma_bf16(workgroups, iters, sink.data_ptr(), sink.numel() * 4, stream.cuda_stream),
                   "w8c_mfma_bf16")
        e1.record(stream)
        torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / launches
    flops = workgroups * (MFMA_THREADS // 64) * MFMA_CHAINS * iters * MFMA_FLOPS
    return flops / sec / 1e12
