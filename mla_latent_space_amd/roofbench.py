"""Measured roofline denominators: a thin ctypes binding over ``include/mla_roofbench.h``
(``libmla_roofbench.so`` in this package directory), and the measurement that bench.py
reports beside the published peaks.

The published MI355X figures (8 TB/s of HBM, 2.5 PFLOP/s of dense bf16 MFMA at the 2.4 GHz
peak clock) stay the headline denominators; these give what this device reaches with a plain
read stream and with MFMA chains that do nothing else, and the shader clock under MFMA load.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_roofbench.so")
STREAM_THREADS = 512          # threads per work-group of the stream read
MFMA_FLOPS = 2 * 32 * 32 * 16  # one v_mfma_f32_32x32x16_bf16
MFMA_PER_ROUND = 4             # independent accumulators per wave

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmla_roofbench.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m mla_latent_space_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    c_i32, c_i64, c_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    L.mla_rb_stream_read.restype = c_i32
    L.mla_rb_stream_read.argtypes = [c_p, c_i64, c_p, c_i32, c_p]
    L.mla_rb_mfma_bf16_loop.restype = c_i32
    L.mla_rb_mfma_bf16_loop.argtypes = [c_i32, c_i32, c_i32, c_p, c_p, c_p]
    _lib = L
    return L


def _check(status: int, what: str) -> None:
    if status != 0:
        raise RuntimeError(f"{what} returned {status}")


def stream_read(src: torch.Tensor, sink: torch.Tensor, blocks: int) -> None:
    """One read of all of ``src`` (a contiguous CUDA tensor of a multiple of 16 bytes) into
    ``sink`` (uint8, 16 * 512 * blocks bytes), on the current stream."""
    nbytes = src.numel() * src.element_size()
    if not (src.is_cuda and sink.is_cuda and src.is_contiguous() and sink.is_contiguous()):
        raise ValueError("src and sink must be contiguous CUDA tensors")
    if sink.numel() * sink.element_size() < 16 * STREAM_THREADS * blocks:
        raise ValueError("sink is smaller than 16 * 512 * blocks bytes")
    stream = torch.cuda.current_stream(src.device).cuda_stream
    _check(lib().mla_rb_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), blocks, stream), "mla_rb_stream_read")


def mfma_loop(blocks: int, waves_per_simd: int, iters: int, sink: torch.Tensor, clocks: torch.Tensor) -> None:
    """One MFMA loop on the current stream; ``sink`` float32 [4 * 256 * waves_per_simd * blocks],
    ``clocks`` int64 [4 * blocks] (the counters, read as unsigned)."""
    if sink.dtype != torch.float32 or sink.numel() < 4 * 256 * waves_per_simd * blocks or not sink.is_cuda:
        raise ValueError("sink must be a CUDA float32 tensor of 4 * 256 * waves_per_simd * blocks elements")
    if clocks.dtype != torch.int64 or clocks.numel() < 4 * blocks or not clocks.is_cuda:
        raise ValueError("clocks must be a CUDA int64 tensor of 4 * blocks elements")
    stream = torch.cuda.current_stream(sink.device).cuda_stream
    _check(lib().mla_rb_mfma_bf16_loop(blocks, waves_per_simd, iters, sink.data_ptr(), clocks.data_ptr(), stream),
           "mla_rb_mfma_bf16_loop")


def _events_us(fn, reps: int) -> float:
    """Mean µs of ``fn`` over ``reps`` back-to-back calls, one pair of events on the current stream."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def measure(device: int = 0, stream_bytes: int = 1 << 30, reps: int = 20) -> dict:
    """The measured denominators on ``device``:
    - ``stream_read_gbps``: a read of ``stream_bytes`` (larger than the 256-MB Infinity Cache,
      so every pass comes from HBM) by 4 work-groups of 512 threads per CU, each on its own
      contiguous share;
    - ``mfma_bf16_tflops``: 256 work-groups (one per CU) of MFMA chains, one and two waves per
      SIMD, each call ≈2 ms, after enough calls to bring the clock to its loaded state;
    - ``clock_ghz``: the shader clock during the two-wave MFMA loop (s_memtime against the
      100-MHz counter, mean over work-groups), and the bf16 peak scaled to that clock."""
    dev = torch.device("cuda", device)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    src = torch.empty(stream_bytes, dtype=torch.uint8, device=dev)
    blocks = 4 * cus
    sink = torch.empty(16 * STREAM_THREADS * blocks, dtype=torch.uint8, device=dev)
    for _ in range(3):
        stream_read(src, sink, blocks)
    gbps = stream_bytes / (_events_us(lambda: stream_read(src, sink, blocks), reps) * 1e-6) / 1e9
    del src, sink

    iters = 16384
    res = {}
    clock = None
    for wps in (1, 2):
        msink = torch.empty(4 * 256 * wps * cus, dtype=torch.float32, device=dev)
        clocks = torch.zeros(4 * cus, dtype=torch.int64, device=dev)
        for _ in range(10):
            mfma_loop(cus, wps, iters, msink, clocks)
        us = _events_us(lambda: mfma_loop(cus, wps, iters, msink, clocks), 5)
        flops = cus * 4 * wps * iters * MFMA_PER_ROUND * MFMA_FLOPS
        res[f"{wps}_wave_per_simd"] = round(flops / (us * 1e-6) / 1e12, 1)
        if wps == 2:
            c = clocks.view(cus, 4).cpu().numpy().astype("uint64").astype("float64")
            clock = float(((c[:, 1] - c[:, 0]) / (c[:, 3] - c[:, 2]) * 0.1).mean())
        expect = 256.0 * iters
        if not bool((msink == expect).all()):
            raise RuntimeError("MFMA loop: accumulator sums differ from 256 * iters")
    return {"stream_read_gbps": round(gbps, 1), "mfma_bf16_tflops": res,
            "clock_ghz_under_mfma": round(clock, 3),
            "bf16_peak_at_that_clock_tflops": round(2 * 32 * 32 * 16 / 32 * 4 * cus * clock * 1e9 / 1e12, 1)}
