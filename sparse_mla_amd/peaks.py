"""ctypes binding of libmla_peaks.so (include/mla_peaks.h): the attainable-
peak microbenchmarks that price the decode against what the chip attains.
Argument marshalling only; each call enqueues one launch on the current
stream (or `stream`)."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_peaks.so")
ROW_BYTES = 1152

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_mla_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)
_p, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
_lib.mlap_stream_read.argtypes = [_p, _sz, _i32, _p, _p]
_lib.mlap_row_gather.argtypes = [_p, _sz, _p, _i32, _i32, _p, _p]
_lib.mlap_mfma_bf16.argtypes = [_i32, _i32, _p, _p]
for _f in (_lib.mlap_stream_read, _lib.mlap_row_gather, _lib.mlap_mfma_bf16):
    _f.restype = ctypes.c_int


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise RuntimeError(f"{fn}: {'argument rejected' if rc == 1 else 'launch failed'} ({rc})")


def _cuda(t: torch.Tensor, name: str, dtype) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous CUDA {dtype} tensor")


def stream_read(src: torch.Tensor, sink: torch.Tensor, num_wg: int = 4096, stream=None) -> int:
    """One streaming read of all of `src` (any dtype, contiguous); returns the bytes read."""
    if not isinstance(src, torch.Tensor) or not src.is_cuda or not src.is_contiguous():
        raise TypeError("src must be a contiguous CUDA tensor")
    _cuda(sink, "sink", torch.int32)
    nbytes = src.numel() * src.element_size()
    _check("mlap_stream_read", _lib.mlap_stream_read(src.data_ptr(), nbytes, num_wg, sink.data_ptr(),
                                                     _stream(stream)))
    return nbytes


def row_gather(cache: torch.Tensor, rows: torch.Tensor, num_wg: int, rows_per_wg: int, sink: torch.Tensor,
               stream=None) -> int:
    """One gather of num_wg * rows_per_wg rows of 1152 bytes; returns the bytes moved."""
    if not isinstance(cache, torch.Tensor) or not cache.is_cuda or not cache.is_contiguous():
        raise TypeError("cache must be a contiguous CUDA tensor")
    _cuda(rows, "rows", torch.int32)
    _cuda(sink, "sink", torch.int32)
    if rows.numel() < num_wg * rows_per_wg:
        raise ValueError("rows holds fewer than num_wg * rows_per_wg entries")
    nbytes = cache.numel() * cache.element_size()
    _check("mlap_row_gather", _lib.mlap_row_gather(cache.data_ptr(), nbytes, rows.data_ptr(), num_wg, rows_per_wg,
                                                   sink.data_ptr(), _stream(stream)))
    return num_wg * rows_per_wg * ROW_BYTES


def mfma_bf16(num_wg: int, iters: int, sink: torch.Tensor, stream=None) -> float:
    """One launch of dense bf16 MFMAs; returns the FLOPs issued."""
    _cuda(sink, "sink", torch.float32)
    if sink.numel() < num_wg * 256:
        raise ValueError("sink needs num_wg * 256 floats")
    _check("mlap_mfma_bf16", _lib.mlap_mfma_bf16(num_wg, iters, sink.data_ptr(), _stream(stream)))
    return float(num_wg) * 4 * iters * 16 * 2 * 32 * 32 * 16


def measure(reps: int = 8, stream: Optional[torch.cuda.Stream] = None) -> dict:
    """Attainable peaks on the current device, each microbenchmark launched
    `reps` times back to back after two warm-up launches, bracketed by HIP
    events on one stream.  The streaming read covers a 2 GiB buffer per
    launch.  The gathers move 256 workgroups x 512 rows of 1152 bytes per
    launch (the decode's share at 64 sequences x 2048 keys, 151 MB) from a
    2 GB region, from one of 8 row sets in turn, so that about 1.2 GB of
    distinct rows pass per cycle and the 256 MB memory-side cache cannot serve
    them: random rows, and for the streaming figure by LDS-DMA, 8 contiguous
    ranges (workgroup w reads rows 512 w .. of its range)."""
    s = torch.cuda.current_stream() if stream is None else stream
    dev = s.device
    sink = torch.zeros(4096 * 256, dtype=torch.int32, device=dev)
    fsink = torch.zeros(256 * 256, dtype=torch.float32, device=dev)

    def timed(launch):
        for i in range(2):
            launch(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        amount = 0.0
        for i in range(reps):
            amount += launch(i)
        e1.record(s)
        e1.synchronize()
        return amount / (e0.elapsed_time(e1) * 1e-3)

    out = {}
    buf = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    out["stream_read_GBps"] = timed(lambda i: stream_read(buf, sink, 4096, s)) / 1e9
    nrows = (2 << 30) // ROW_BYTES
    per = 256 * 512
    g = torch.Generator(device="cpu").manual_seed(20251)
    rand_rows = torch.randint(0, nrows, (8, per), generator=g, dtype=torch.int32).to(dev)
    seq_rows = torch.arange(8 * per, dtype=torch.int32, device=dev).view(8, per)
    cache = buf[: nrows * ROW_BYTES]
    out["stream_lds_dma_GBps"] = timed(lambda i: row_gather(cache, seq_rows[i % 8], 256, 512, sink, s)) / 1e9
    out["row_gather_GBps"] = timed(lambda i: row_gather(cache, rand_rows[i % 8], 256, 512, sink, s)) / 1e9
    del buf, cache
    out["mfma_bf16_TFLOPs"] = timed(lambda i: mfma_bf16(256, 8000, fsink, s)) / 1e12
    return out
