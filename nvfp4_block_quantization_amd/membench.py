"""ctypes binding of libnvfp4_membench.so (include/nvfp4_membench.h): HBM
read, write and copy streams, the bandwidth ceilings of this GPU that the
quantization kernels are measured against."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4_membench.so")
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run nvfp4_block_quantization_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        P, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.membench_copy.argtypes = [P, P, sz, i32, P]
        L.membench_read.argtypes = [P, sz, P, i32, P]
        L.membench_write.argtypes = [P, sz, ctypes.c_uint32, i32, P]
        for f in (L.membench_copy, L.membench_read, L.membench_write):
            f.restype = i32
        _lib = L
    return _lib


def _buf(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous GPU tensor")
    n = t.numel() * t.element_size()
    if n % 16:
        raise ValueError(f"{name} must hold a multiple of 16 bytes")
    return n


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ok(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed ({rc})")


def copy(dst: torch.Tensor, src: torch.Tensor, grid: int = 0) -> None:
    n = _buf(src, "src")
    if _buf(dst, "dst") < n or dst.device != src.device:
        raise ValueError("dst must be at least as large as src, on the same GPU")
    _ok(lib().membench_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()), n, grid, _stream(src)),
        "membench_copy")


def read(src: torch.Tensor, sink: torch.Tensor, grid: int = 0) -> None:
    n = _buf(src, "src")
    if sink.dtype != torch.int32 or sink.numel() < 4 or sink.device != src.device:
        raise ValueError("sink must be 4 int32 on the same GPU")
    _ok(lib().membench_read(ctypes.c_void_p(src.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()), grid, _stream(src)),
        "membench_read")


def write(dst: torch.Tensor, value: int = 0, grid: int = 0) -> None:
    n = _buf(dst, "dst")
    _ok(lib().membench_write(ctypes.c_void_p(dst.data_ptr()), n, value & 0xFFFFFFFF, grid, _stream(dst)),
        "membench_write")
