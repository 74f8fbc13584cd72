"""Python binding of libnvfp4.so, the gfx950 NVFP4 block-quantization library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/nvfp4.h).  PyTorch provides device memory
and the current stream.  There is no CPU fallback: without the built library
or without a GPU tensor these functions raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "nvfp4.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(8)
IN_BF16, IN_F32 = 0, 1
BLOCKS = {"1d": 0, "2d": 1}
RULES = {"none": 0, "mse": 1, "mae": 2, "maxerr": 3}


class Config(ctypes.Structure):
    _fields_ = [
        ("block", ctypes.c_int32),
        ("emit_rowwise", ctypes.c_int32),
        ("emit_colwise", ctypes.c_int32),
        ("rht", ctypes.c_int32),
        ("rht_sign_mask", ctypes.c_uint32),
        ("sr", ctypes.c_int32),
        ("sr_seed", ctypes.c_uint64),
        ("row_offset", ctypes.c_int64),
        ("rule", ctypes.c_int32),
        ("scale_cap", ctypes.c_float),
    ]


class Outputs(ctypes.Structure):
    _fields_ = [
        ("codes_row", ctypes.c_void_p),
        ("scales_row", ctypes.c_void_p),
        ("codes_col", ctypes.c_void_p),
        ("scales_col", ctypes.c_void_p),
        ("tensor_scale", ctypes.c_void_p),
    ]


class MXConfig(ctypes.Structure):
    _fields_ = [
        ("emit_rowwise", ctypes.c_int32),
        ("emit_colwise", ctypes.c_int32),
        ("sr", ctypes.c_int32),
        ("sr_seed", ctypes.c_uint64),
        ("row_offset", ctypes.c_int64),
    ]


class MXOutputs(ctypes.Structure):
    _fields_ = [
        ("codes_row", ctypes.c_void_p),
        ("scales_row", ctypes.c_void_p),
        ("codes_col", ctypes.c_void_p),
        ("scales_col", ctypes.c_void_p),
    ]


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {lib().nvfp4_status_string(status).decode()} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libnvfp4.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run nvfp4_block_quantization_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        P, i64, u64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int
        L.nvfp4_abi_version.restype = i32
        L.nvfp4_abi_version.argtypes = []
        L.nvfp4_status_string.restype = ctypes.c_char_p
        L.nvfp4_status_string.argtypes = [i32]
        L.nvfp4_rht_signs_from_seed.restype = ctypes.c_uint32
        L.nvfp4_rht_signs_from_seed.argtypes = [u64]
        L.nvfp4_amax_workspace_bytes.restype = ctypes.c_size_t
        L.nvfp4_amax_workspace_bytes.argtypes = [i64, i64]
        L.nvfp4_amax.restype = i32
        L.nvfp4_amax.argtypes = [P, i32, i64, i64, ctypes.POINTER(Config), P, P, ctypes.c_size_t, P]
        L.nvfp4_quantize.restype = i32
        L.nvfp4_quantize.argtypes = [P, i32, i64, i64, ctypes.POINTER(Config), P, ctypes.POINTER(Outputs), P]
        L.nvfp4_dequantize.restype = i32
        L.nvfp4_dequantize.argtypes = [P, P, P, i64, i64, i32, P, P]
        L.nvfp4_error_stats.restype = i32
        L.nvfp4_error_stats.argtypes = [P, i32, i64, i64, ctypes.POINTER(Config), P, ctypes.c_float, ctypes.c_int32,
                                        P, P]
        L.nvfp4_gemm.restype = i32
        L.nvfp4_gemm.argtypes = [P, P, P, i32, P, P, P, i32, i64, i64, i64, P, P]
        L.nvfp4_mxfp4_gemm.restype = i32
        L.nvfp4_mxfp4_gemm.argtypes = [P, P, P, P, i64, i64, i64, P, P]
        L.nvfp4_mxfp4_quantize.restype = i32
        L.nvfp4_mxfp4_quantize.argtypes = [P, i32, i64, i64, ctypes.POINTER(MXConfig), ctypes.POINTER(MXOutputs), P]
        L.nvfp4_mxfp4_dequantize.restype = i32
        L.nvfp4_mxfp4_dequantize.argtypes = [P, P, i64, i64, P, P]
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != OK:
        raise NVFP4Error(status, what)


def _dtype_code(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return IN_BF16
    if x.dtype == torch.float32:
        return IN_F32
    raise TypeError(f"input must be bfloat16 or float32, got {x.dtype}")


def _gpu2d(x: torch.Tensor, name: str) -> None:
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise TypeError(f"{name} must be a GPU tensor (no CPU path)")
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 2-D tensor")


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device, stream: torch.cuda.Stream | None):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def abi_version() -> int:
    return lib().nvfp4_abi_version()


def rht_signs_from_seed(seed: int) -> int:
    return int(lib().nvfp4_rht_signs_from_seed(seed))


def make_config(block: str = "1d", rowwise: bool = True, colwise: bool = False, rht: bool = False,
                rht_mask: int = 0, sr: bool = False, sr_seed: int = 0, row_offset: int = 0,
                rule: str = "none", scale_cap: float = 448.0) -> Config:
    return Config(BLOCKS[block], int(rowwise), int(colwise), int(rht), rht_mask & 0xFFFFFFFF, int(sr),
                  sr_seed, row_offset, RULES[rule], scale_cap)


def amax_workspace_bytes(rows: int, cols: int) -> int:
    return int(lib().nvfp4_amax_workspace_bytes(rows, cols))


def amax(x: torch.Tensor, rht: bool = False, rht_mask: int = 0, out: torch.Tensor | None = None,
         workspace: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """Per-tensor amax (of the Hadamard-transformed blocks when rht) -> float32 tensor of shape (1,)."""
    _gpu2d(x, "x")
    rows, cols = x.shape
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    nbytes = amax_workspace_bytes(rows, cols)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=x.device)
    cfg = make_config(rht=rht, rht_mask=rht_mask)
    st = lib().nvfp4_amax(_ptr(x), _dtype_code(x), rows, cols, ctypes.byref(cfg), _ptr(out), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream(x.device, stream))
    _check(st, "nvfp4_amax")
    return out


def allocate_outputs(rows: int, cols: int, block: str = "1d", rowwise: bool = True, colwise: bool = False,
                     device: torch.device | str = "cuda") -> dict:
    o = {"tensor_scale": torch.empty(1, dtype=torch.float32, device=device)}
    u8 = dict(dtype=torch.uint8, device=device)
    if rowwise:
        o["codes_row"] = torch.empty((rows, cols // 2), **u8)
        o["scales_row"] = torch.empty(((rows // 16, cols // 16) if block == "2d" else (rows, cols // 16)), **u8)
    if colwise:
        o["codes_col"] = torch.empty((cols, rows // 2), **u8)
        o["scales_col"] = torch.empty(((cols // 16, rows // 16) if block == "2d" else (cols, rows // 16)), **u8)
    return o


def quantize(x: torch.Tensor, amax_t: torch.Tensor, block: str = "1d", rowwise: bool = True,
             colwise: bool = False, rht: bool = False, rht_mask: int = 0, sr: bool = False, sr_seed: int = 0,
             rule: str = "none", scale_cap: float = 448.0, row_offset: int = 0, out: dict | None = None,
             stream: torch.cuda.Stream | None = None) -> dict:
    """NVFP4-quantize x with the given (device) amax; returns a dict of output tensors."""
    _gpu2d(x, "x")
    rows, cols = x.shape
    if out is None:
        out = allocate_outputs(rows, cols, block, rowwise, colwise, x.device)
    cfg = make_config(block, rowwise, colwise, rht, rht_mask, sr, sr_seed, row_offset, rule, scale_cap)
    o = Outputs(out["codes_row"].data_ptr() if rowwise else None, out["scales_row"].data_ptr() if rowwise else None,
                out["codes_col"].data_ptr() if colwise else None, out["scales_col"].data_ptr() if colwise else None,
                out["tensor_scale"].data_ptr() if out.get("tensor_scale") is not None else None)
    st = lib().nvfp4_quantize(_ptr(x), _dtype_code(x), rows, cols, ctypes.byref(cfg), _ptr(amax_t), ctypes.byref(o),
                              _stream(x.device, stream))
    _check(st, "nvfp4_quantize")
    return out


def dequantize(codes: torch.Tensor, scales: torch.Tensor, tensor_scale: torch.Tensor, rows: int, cols: int,
               block: str = "1d", out: torch.Tensor | None = None,
               stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """fp32 [rows][cols] from packed codes, E4M3 scales and the tensor scale."""
    _gpu2d(codes, "codes")
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=codes.device)
    st = lib().nvfp4_dequantize(_ptr(codes), _ptr(scales), _ptr(tensor_scale), rows, cols, BLOCKS[block], _ptr(out),
                                _stream(codes.device, stream))
    _check(st, "nvfp4_dequantize")
    return out


def error_stats(x: torch.Tensor, amax_t: torch.Tensor, block: str = "1d", rht: bool = False, rht_mask: int = 0,
                rule: str = "none", scale_cap: float = 448.0, bin_width: float = 0.25, nbins: int = 26,
                out: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """(3, nbins) float64 on the GPU: per scaled-value bin, the element count, the
    sum of squared quantization errors and the same for an exact-scale reference."""
    _gpu2d(x, "x")
    rows, cols = x.shape
    if out is None:
        out = torch.empty((3, nbins), dtype=torch.float64, device=x.device)
    cfg = make_config(block, True, False, rht, rht_mask, False, 0, 0, rule, scale_cap)
    st = lib().nvfp4_error_stats(_ptr(x), _dtype_code(x), rows, cols, ctypes.byref(cfg), _ptr(amax_t), bin_width,
                                 nbins, _ptr(out), _stream(x.device, stream))
    _check(st, "nvfp4_error_stats")
    return out


# ---- MXFP4 (32-element blocks, E8M0 power-of-two scales, no tensor scale) ----

def mxfp4_allocate_outputs(rows: int, cols: int, rowwise: bool = True, colwise: bool = False,
                           device: torch.device | str = "cuda") -> dict:
    u8 = dict(dtype=torch.uint8, device=device)
    o = {}
    if rowwise:
        o["codes_row"] = torch.empty((rows, cols // 2), **u8)
        o["scales_row"] = torch.empty((rows, cols // 32), **u8)
    if colwise:
        o["codes_col"] = torch.empty((cols, rows // 2), **u8)
        o["scales_col"] = torch.empty((cols, rows // 32), **u8)
    return o


def mxfp4_quantize(x: torch.Tensor, rowwise: bool = True, colwise: bool = False, sr: bool = False,
                   sr_seed: int = 0, row_offset: int = 0, out: dict | None = None,
                   stream: torch.cuda.Stream | None = None) -> dict:
    """MXFP4-quantize x (one pass, no amax); returns a dict of output tensors."""
    _gpu2d(x, "x")
    rows, cols = x.shape
    if out is None:
        out = mxfp4_allocate_outputs(rows, cols, rowwise, colwise, x.device)
    cfg = MXConfig(int(rowwise), int(colwise), int(sr), sr_seed, row_offset)
    o = MXOutputs(out["codes_row"].data_ptr() if rowwise else None, out["scales_row"].data_ptr() if rowwise else None,
                  out["codes_col"].data_ptr() if colwise else None, out["scales_col"].data_ptr() if colwise else None)
    st = lib().nvfp4_mxfp4_quantize(_ptr(x), _dtype_code(x), rows, cols, ctypes.byref(cfg), ctypes.byref(o),
                                    _stream(x.device, stream))
    _check(st, "nvfp4_mxfp4_quantize")
    return out


def mxfp4_dequantize(codes: torch.Tensor, scales: torch.Tensor, rows: int, cols: int,
                     out: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """fp32 [rows][cols] from packed codes and E8M0 scales."""
    _gpu2d(codes, "codes")
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=codes.device)
    st = lib().nvfp4_mxfp4_dequantize(_ptr(codes), _ptr(scales), rows, cols, _ptr(out),
                                      _stream(codes.device, stream))
    _check(st, "nvfp4_mxfp4_dequantize")
    return out


# ---- the consumer: FP4 GEMM (C = A B^T, operands with K contiguous) ------------

def gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, a_tensor_scale: torch.Tensor, b_codes: torch.Tensor,
         b_scales: torch.Tensor, b_tensor_scale: torch.Tensor, a_block: str = "1d", b_block: str = "1d",
         out: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """float32 [M][N] = A B^T from NVFP4 row copies (codes [M][K/2], [N][K/2])."""
    _gpu2d(a_codes, "a_codes")
    _gpu2d(b_codes, "b_codes")
    M, K = a_codes.shape[0], 2 * a_codes.shape[1]
    N = b_codes.shape[0]
    if 2 * b_codes.shape[1] != K:
        raise ValueError("A and B must have the same K")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a_codes.device)
    st = lib().nvfp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(a_tensor_scale), BLOCKS[a_block], _ptr(b_codes),
                          _ptr(b_scales), _ptr(b_tensor_scale), BLOCKS[b_block], M, N, K, _ptr(out),
                          _stream(a_codes.device, stream))
    _check(st, "nvfp4_gemm")
    return out


def mxfp4_gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, b_codes: torch.Tensor, b_scales: torch.Tensor,
               out: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """float32 [M][N] = A B^T from MXFP4 row copies (codes [M][K/2], [N][K/2])."""
    _gpu2d(a_codes, "a_codes")
    _gpu2d(b_codes, "b_codes")
    M, K = a_codes.shape[0], 2 * a_codes.shape[1]
    N = b_codes.shape[0]
    if 2 * b_codes.shape[1] != K:
        raise ValueError("A and B must have the same K")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a_codes.device)
    st = lib().nvfp4_mxfp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), M, N, K, _ptr(out),
                                _stream(a_codes.device, stream))
    _check(st, "nvfp4_mxfp4_gemm")
    return out
