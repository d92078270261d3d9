"""Binding of libgqe_calib.so: the calibration kernels the benchmark uses for its measured ceilings
(a sustained dense bf16 MFMA loop with the clock it ran at, and a streaming HBM read).  Argument
marshalling only; raises if the library is not built."""
from __future__ import annotations

import ctypes
import os

import torch

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqe_calib.so")
_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_PATH):
            raise RuntimeError(f"{_PATH} is missing: build it with `python -m sparse_routed_query_amd.build`")
        lib = ctypes.CDLL(_PATH)
        P = ctypes.c_void_p
        lib.gqe_calib_mfma.argtypes = [P, P, ctypes.c_int, ctypes.c_int, P]
        lib.gqe_calib_mfma.restype = ctypes.c_int
        lib.gqe_calib_read.argtypes = [P, ctypes.c_longlong, P, ctypes.c_int, P]
        lib.gqe_calib_read.restype = ctypes.c_int
        _lib = lib
    return _lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def mfma(sink: torch.Tensor, clk: torch.Tensor, blocks: int, iters: int) -> None:
    """blocks * 4 waves, each 4 * iters v_mfma_f32_32x32x16_bf16 (32768 FLOP each).  sink: float32 [blocks * 256];
    clk: int64 [2] (shader-clock ticks, 100 MHz ticks of one wave)."""
    assert sink.is_cuda and sink.dtype == torch.float32 and sink.numel() >= blocks * 256
    assert clk.is_cuda and clk.dtype == torch.int64 and clk.numel() >= 2
    rc = load().gqe_calib_mfma(ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(clk.data_ptr()), blocks, iters,
                               _stream())
    if rc != 0:
        raise RuntimeError("gqe_calib_mfma failed")


def read(src: torch.Tensor, sink: torch.Tensor, blocks: int) -> None:
    """Streaming read of every byte of src (contiguous, size a multiple of 16).  sink: int32 [blocks]."""
    nbytes = src.numel() * src.element_size()
    assert src.is_cuda and src.is_contiguous() and nbytes % 16 == 0
    assert sink.is_cuda and sink.dtype == torch.int32 and sink.numel() >= blocks
    rc = load().gqe_calib_read(ctypes.c_void_p(src.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), blocks,
                               _stream())
    if rc != 0:
        raise RuntimeError("gqe_calib_read failed")
