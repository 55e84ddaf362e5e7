"""ctypes binding of libmxstream.so, the streaming bandwidth probe
(include/mxstream.h).  Measurement only: the benchmark times it at the casts'
read:write byte mixes to report what plain streaming reaches on the device."""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch

from . import _build

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_build.STREAM_LIB_PATH):
            raise RuntimeError(f"{_build.STREAM_LIB_PATH} is not built; run __graft_entry__.build() first")
        h = ctypes.CDLL(_build.STREAM_LIB_PATH)
        h.mxstream_mix.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        h.mxstream_mix.restype = ctypes.c_int
        _lib = h
    return _lib


def mix(ins: Sequence[torch.Tensor], outs: Sequence[torch.Tensor], nbytes: int, *, unroll: int = 8, grid: int = 4096,
        stream=None) -> None:
    """Stream `nbytes` from each tensor of `ins` and to each of `outs` (GPU
    tensors of at least nbytes bytes, 16-byte aligned)."""
    for t in list(ins) + list(outs):
        if not t.is_cuda or t.numel() * t.element_size() < nbytes:
            raise ValueError("probe buffers must be GPU tensors of at least nbytes bytes")
    pin = (ctypes.c_void_p * len(ins))(*[t.data_ptr() for t in ins])
    pout = (ctypes.c_void_p * len(outs))(*[t.data_ptr() for t in outs])
    if stream is None:
        stream = torch.cuda.current_stream(ins[0].device)
    st = lib().mxstream_mix(pin, len(ins), pout, len(outs), nbytes, unroll, grid, int(stream.cuda_stream))
    if st != 0:
        raise RuntimeError(f"mxstream_mix failed with status {st}")
