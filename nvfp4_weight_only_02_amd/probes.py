"""Binding of libnvfp4_probes (include/nvfp4_probes.h): measurement aids the
benchmark times beside the decode projection.  Argument marshalling only; the
library must be built (``python -m nvfp4_weight_only_02_amd.build``)."""
from __future__ import annotations

import ctypes
import os

import torch

from . import Nvfp4Error, _dev, _stream

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4_probes.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "nvfp4_probes.h")
RATE_MFMA, RATE_VALU = 0, 1
XSTAGE_LOADS, XSTAGE_FULL = 0, 1

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded probe library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libnvfp4_probes.so is not built (run `python -m nvfp4_weight_only_02_amd.build`)")
        L = ctypes.CDLL(LIB_PATH)
        L.nvfp4_probe_block_rate.restype = ctypes.c_int
        L.nvfp4_probe_block_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                             ctypes.c_size_t, ctypes.c_void_p]
        L.nvfp4_probe_read_stream.restype = ctypes.c_int
        L.nvfp4_probe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
        L.nvfp4_probe_empty.restype = ctypes.c_int
        L.nvfp4_probe_empty.argtypes = [ctypes.c_int, ctypes.c_void_p]
        L.nvfp4_probe_x_stage.restype = ctypes.c_int
        L.nvfp4_probe_x_stage.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        raise Nvfp4Error(status, what)


def block_rate(path: int, n: int, blocks: int, sink: torch.Tensor, stream=None) -> None:
    """Per-block arithmetic-rate probe (RATE_MFMA or RATE_VALU) for n tokens;
    ``sink`` is a float32 device tensor of >= 256*512 elements."""
    _dev(sink, torch.float32, "sink")
    _check(lib().nvfp4_probe_block_rate(int(path), int(n), int(blocks), sink.data_ptr(), sink.numel() * 4,
                                        _stream(stream, sink)), "nvfp4_probe_block_rate")


def read_stream(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read every byte of ``buf`` once (the read ceiling of its size)."""
    _dev(buf, torch.uint8, "buf")
    _dev(sink, torch.int32, "sink")
    _check(lib().nvfp4_probe_read_stream(buf.data_ptr(), buf.numel(), sink.data_ptr(),
                                             _stream(stream, buf, sink)),
           "nvfp4_probe_read_stream")


def empty(workgroups: int, stream=None) -> None:
    """A launch of ``workgroups`` 512-thread workgroups that do nothing."""
    _check(lib().nvfp4_probe_empty(int(workgroups), _stream(stream)), "nvfp4_probe_empty")


def x_stage(X: torch.Tensor, workgroups: int, reps: int, mode: int, sink: torch.Tensor, stream=None) -> None:
    """The GEMV's activation staging alone (XSTAGE_LOADS or XSTAGE_FULL) for
    X bf16 [n, K], ``reps`` times per launch on ``workgroups`` workgroups."""
    _dev(X, torch.bfloat16, "X")
    _dev(sink, torch.int32, "sink")
    if X.dim() != 2:
        raise ValueError("X must be [n, K]")
    _check(lib().nvfp4_probe_x_stage(X.data_ptr(), X.shape[0], X.shape[1], int(workgroups), int(reps), int(mode),
                                     sink.data_ptr(), _stream(stream, X, sink)), "nvfp4_probe_x_stage")
