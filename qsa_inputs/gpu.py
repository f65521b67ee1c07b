"""GPU fill of seeded inputs (same definition as the numpy generator).

Used to build large device-resident workloads without a host round trip;
element i of stream (seed, stream) equals ``normal_bf16(seed, stream, i)``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from .gen import normal_table

_LIB = None
_TABLES = {}
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqsa_fill.so")


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with indexer_selected_sparse_pooled_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.qsa_fill_normal_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.qsa_fill_normal_bf16.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _table(device):
    key = str(device)
    if key not in _TABLES:
        t = torch.from_numpy(normal_table().astype(np.int16).copy()).to(device)
        _TABLES[key] = t
    return _TABLES[key]


def fill_normal_bf16(out: torch.Tensor, seed: int, stream: int, start: int = 0, cuda_stream=None) -> None:
    """Fill a contiguous bf16 CUDA tensor with elements [start, start + numel)."""
    if not out.is_cuda or out.dtype not in (torch.bfloat16, torch.int16) or not out.is_contiguous():
        raise TypeError("out must be a contiguous bf16 CUDA tensor")
    s = torch.cuda.current_stream(out.device) if cuda_stream is None else cuda_stream
    rc = _lib().qsa_fill_normal_bf16(seed & (2**64 - 1), stream & (2**64 - 1), start, out.numel(),
                                     ctypes.c_void_p(_table(out.device).data_ptr()),
                                     ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"qsa_fill_normal_bf16 failed ({rc})")
