"""Python binding of libnvfp4.so, the gfx950 NVFP4 block-quantization library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/nvfp4.h).  PyTorch provides device memory
and the current stream.  There is no CPU fallback: without the built library
or without a GPU tensor these functions raise.

The C ABI cannot see buffer sizes, so this module checks every tensor it
passes on (dtype, contiguity, exact shape, one device for all of them) and
raises before calling the library; a wrong buffer would otherwise become an
out-of-bounds device access.
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
        ("rht_sign_mask", ctypes.c_uint16),
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
        L.nvfp4_rht_signs_from_seed.restype = ctypes.c_uint16
        L.nvfp4_rht_signs_from_seed.argtypes = [u64]
        L.nvfp4_amax_workspace_bytes.restype = ctypes.c_size_t
        L.nvfp4_amax_workspace_bytes.argtypes = [i64, i64]
        L.nvfp4_amax.restype = i32
        L.nvfp4_amax.argtypes = [P, i32, i64, i64, ctypes.POINTER(Config), P, P, ctypes.c_size_t, P]
        L.nvfp4_amax_noalloc.restype = i32
        L.nvfp4_amax_noalloc.argtypes = [P, i32, i64, i64, ctypes.POINTER(Config), P, P]
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


# ---- argument checks (all before any library call; device checks last) ---------

def _tensor(t, name: str, dtype: torch.dtype, shape: tuple | None = None, min_numel: int | None = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} must hold at least {min_numel} elements, got {t.numel()}")


def _input2d(x, name: str = "x") -> tuple:
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 2-D tensor")
    _dtype_code(x)
    return tuple(x.shape)


def _same_gpu(first: torch.Tensor, **others) -> torch.device:
    """Every tensor on one GPU (there is no CPU path)."""
    if first.device.type != "cuda":
        raise TypeError("tensors must be GPU tensors (no CPU path)")
    for name, t in others.items():
        if t is not None and t.device != first.device:
            raise TypeError(f"{name} is on {t.device}, expected {first.device} like the other arguments")
    return first.device


def _dims(rows: int, cols: int) -> None:
    if not (isinstance(rows, int) and isinstance(cols, int)) or rows < 0 or cols < 0:
        raise ValueError(f"rows and cols must be non-negative ints, got {rows!r}, {cols!r}")


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
    if block not in BLOCKS:
        raise ValueError(f"block must be one of {sorted(BLOCKS)}, got {block!r}")
    if rule not in RULES:
        raise ValueError(f"rule must be one of {sorted(RULES)}, got {rule!r}")
    if not 0 <= rht_mask <= 0xFFFF:
        raise ValueError(f"rht_mask is a 16-bit sign mask, got {rht_mask:#x}")
    if not 0 <= sr_seed < 1 << 64:
        raise ValueError("sr_seed must fit in 64 bits")
    return Config(BLOCKS[block], int(rowwise), int(colwise), int(rht), rht_mask, int(sr),
                  sr_seed, row_offset, RULES[rule], scale_cap)


def amax_workspace_bytes(rows: int, cols: int) -> int:
    return int(lib().nvfp4_amax_workspace_bytes(rows, cols))


def amax(x: torch.Tensor, rht: bool = False, rht_mask: int = 0, out: torch.Tensor | None = None,
         workspace: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """Per-tensor amax (of the Hadamard-transformed blocks when rht) -> float32 tensor of shape (1,)."""
    rows, cols = _input2d(x)
    cfg = make_config(rht=rht, rht_mask=rht_mask)
    nbytes = amax_workspace_bytes(rows, cols)
    if out is not None:
        _tensor(out, "out", torch.float32, min_numel=1)
    if workspace is not None:
        _tensor(workspace, "workspace", torch.uint8, min_numel=nbytes)
    dev = _same_gpu(x, out=out, workspace=workspace)
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=dev)
    st = lib().nvfp4_amax(_ptr(x), _dtype_code(x), rows, cols, ctypes.byref(cfg), _ptr(out), _ptr(workspace),
                          workspace.numel(), _stream(dev, stream))
    _check(st, "nvfp4_amax")
    return out


def amax_noalloc(x: torch.Tensor, rht: bool = False, rht_mask: int = 0, out: torch.Tensor | None = None,
                 stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """nvfp4_amax_noalloc: the amax pass with the library's per-GPU scratch array
    instead of a workspace (calls that overlap on one GPU race)."""
    rows, cols = _input2d(x)
    cfg = make_config(rht=rht, rht_mask=rht_mask)
    if out is not None:
        _tensor(out, "out", torch.float32, min_numel=1)
    dev = _same_gpu(x, out=out)
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=dev)
    st = lib().nvfp4_amax_noalloc(_ptr(x), _dtype_code(x), rows, cols, ctypes.byref(cfg), _ptr(out),
                                  _stream(dev, stream))
    _check(st, "nvfp4_amax_noalloc")
    return out


def output_shapes(rows: int, cols: int, block: str = "1d", rowwise: bool = True, colwise: bool = False) -> dict:
    """Shapes of nvfp4_quantize's outputs (uint8 except the float32 tensor scale)."""
    sh = {"tensor_scale": (1,)}
    if rowwise:
        sh["codes_row"] = (rows, cols // 2)
        sh["scales_row"] = (rows // 16, cols // 16) if block == "2d" else (rows, cols // 16)
    if colwise:
        sh["codes_col"] = (cols, rows // 2)
        sh["scales_col"] = (cols // 16, rows // 16) if block == "2d" else (cols, rows // 16)
    return sh


def allocate_outputs(rows: int, cols: int, block: str = "1d", rowwise: bool = True, colwise: bool = False,
                     device: torch.device | str = "cuda") -> dict:
    return {k: torch.empty(v, dtype=torch.float32 if k == "tensor_scale" else torch.uint8, device=device)
            for k, v in output_shapes(rows, cols, block, rowwise, colwise).items()}


def _check_outputs(out: dict, shapes: dict, optional: tuple = ()) -> None:
    if not isinstance(out, dict):
        raise TypeError("out must be a dict of tensors")
    for k, shape in shapes.items():
        t = out.get(k)
        if t is None:
            if k in optional:
                continue
            raise ValueError(f"out is missing {k!r}")
        _tensor(t, f"out[{k!r}]", torch.float32 if k == "tensor_scale" else torch.uint8,
                min_numel=1 if k == "tensor_scale" else None, shape=None if k == "tensor_scale" else shape)


def quantize(x: torch.Tensor, amax_t: torch.Tensor, block: str = "1d", rowwise: bool = True,
             colwise: bool = False, rht: bool = False, rht_mask: int = 0, sr: bool = False, sr_seed: int = 0,
             rule: str = "none", scale_cap: float = 448.0, row_offset: int = 0, out: dict | None = None,
             stream: torch.cuda.Stream | None = None) -> dict:
    """NVFP4-quantize x with the given (device) amax; returns a dict of output tensors."""
    rows, cols = _input2d(x)
    cfg = make_config(block, rowwise, colwise, rht, rht_mask, sr, sr_seed, row_offset, rule, scale_cap)
    _tensor(amax_t, "amax_t", torch.float32, min_numel=1)
    shapes = output_shapes(rows, cols, block, rowwise, colwise)
    if out is not None:
        _check_outputs(out, shapes, optional=("tensor_scale",))
    dev = _same_gpu(x, amax_t=amax_t, **({f"out[{k!r}]": v for k, v in out.items() if k in shapes}
                                          if out is not None else {}))
    if out is None:
        out = allocate_outputs(rows, cols, block, rowwise, colwise, dev)
    o = Outputs(out["codes_row"].data_ptr() if rowwise else None, out["scales_row"].data_ptr() if rowwise else None,
                out["codes_col"].data_ptr() if colwise else None, out["scales_col"].data_ptr() if colwise else None,
                out["tensor_scale"].data_ptr() if out.get("tensor_scale") is not None else None)
    st = lib().nvfp4_quantize(_ptr(x), _dtype_code(x), rows, cols, ctypes.byref(cfg), _ptr(amax_t), ctypes.byref(o),
                              _stream(dev, stream))
    _check(st, "nvfp4_quantize")
    return out


def dequantize(codes: torch.Tensor, scales: torch.Tensor, tensor_scale: torch.Tensor, rows: int, cols: int,
               block: str = "1d", out: torch.Tensor | None = None,
               stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """fp32 [rows][cols] from packed codes, E4M3 scales and the tensor scale."""
    _dims(rows, cols)
    if block not in BLOCKS:
        raise ValueError(f"block must be one of {sorted(BLOCKS)}, got {block!r}")
    _tensor(codes, "codes", torch.uint8, shape=(rows, cols // 2))
    _tensor(scales, "scales", torch.uint8, shape=(rows // 16, cols // 16) if block == "2d" else (rows, cols // 16))
    _tensor(tensor_scale, "tensor_scale", torch.float32, min_numel=1)
    if out is not None:
        _tensor(out, "out", torch.float32, shape=(rows, cols))
    dev = _same_gpu(codes, scales=scales, tensor_scale=tensor_scale, out=out)
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    st = lib().nvfp4_dequantize(_ptr(codes), _ptr(scales), _ptr(tensor_scale), rows, cols, BLOCKS[block], _ptr(out),
                                _stream(dev, stream))
    _check(st, "nvfp4_dequantize")
    return out


def error_stats(x: torch.Tensor, amax_t: torch.Tensor, block: str = "1d", rht: bool = False, rht_mask: int = 0,
                rule: str = "none", scale_cap: float = 448.0, bin_width: float = 0.25, nbins: int = 26,
                out: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """(3, nbins) float64 on the GPU: per scaled-value bin, the element count, the
    sum of squared quantization errors and the same for an exact-scale reference."""
    rows, cols = _input2d(x)
    cfg = make_config(block, True, False, rht, rht_mask, False, 0, 0, rule, scale_cap)
    _tensor(amax_t, "amax_t", torch.float32, min_numel=1)
    if not isinstance(nbins, int) or not 1 <= nbins <= 64:
        raise ValueError(f"nbins must be an int in [1, 64], got {nbins!r}")
    if out is not None:
        _tensor(out, "out", torch.float64, shape=(3, nbins))
    dev = _same_gpu(x, amax_t=amax_t, out=out)
    if out is None:
        out = torch.empty((3, nbins), dtype=torch.float64, device=dev)
    st = lib().nvfp4_error_stats(_ptr(x), _dtype_code(x), rows, cols, ctypes.byref(cfg), _ptr(amax_t), bin_width,
                                 nbins, _ptr(out), _stream(dev, stream))
    _check(st, "nvfp4_error_stats")
    return out


# ---- MXFP4 (32-element blocks, E8M0 power-of-two scales, no tensor scale) ----

def mxfp4_output_shapes(rows: int, cols: int, rowwise: bool = True, colwise: bool = False) -> dict:
    sh = {}
    if rowwise:
        sh["codes_row"] = (rows, cols // 2)
        sh["scales_row"] = (rows, cols // 32)
    if colwise:
        sh["codes_col"] = (cols, rows // 2)
        sh["scales_col"] = (cols, rows // 32)
    return sh


def mxfp4_allocate_outputs(rows: int, cols: int, rowwise: bool = True, colwise: bool = False,
                           device: torch.device | str = "cuda") -> dict:
    return {k: torch.empty(v, dtype=torch.uint8, device=device)
            for k, v in mxfp4_output_shapes(rows, cols, rowwise, colwise).items()}


def mxfp4_quantize(x: torch.Tensor, rowwise: bool = True, colwise: bool = False, sr: bool = False,
                   sr_seed: int = 0, row_offset: int = 0, out: dict | None = None,
                   stream: torch.cuda.Stream | None = None) -> dict:
    """MXFP4-quantize x (one pass, no amax); returns a dict of output tensors."""
    rows, cols = _input2d(x)
    if not 0 <= sr_seed < 1 << 64:
        raise ValueError("sr_seed must fit in 64 bits")
    shapes = mxfp4_output_shapes(rows, cols, rowwise, colwise)
    if out is not None:
        _check_outputs(out, shapes)
    dev = _same_gpu(x, **({f"out[{k!r}]": v for k, v in out.items() if k in shapes} if out is not None else {}))
    if out is None:
        out = mxfp4_allocate_outputs(rows, cols, rowwise, colwise, dev)
    cfg = MXConfig(int(rowwise), int(colwise), int(sr), sr_seed, row_offset)
    o = MXOutputs(out["codes_row"].data_ptr() if rowwise else None, out["scales_row"].data_ptr() if rowwise else None,
                  out["codes_col"].data_ptr() if colwise else None, out["scales_col"].data_ptr() if colwise else None)
    st = lib().nvfp4_mxfp4_quantize(_ptr(x), _dtype_code(x), rows, cols, ctypes.byref(cfg), ctypes.byref(o),
                                    _stream(dev, stream))
    _check(st, "nvfp4_mxfp4_quantize")
    return out


def mxfp4_dequantize(codes: torch.Tensor, scales: torch.Tensor, rows: int, cols: int,
                     out: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """fp32 [rows][cols] from packed codes and E8M0 scales."""
    _dims(rows, cols)
    _tensor(codes, "codes", torch.uint8, shape=(rows, cols // 2))
    _tensor(scales, "scales", torch.uint8, shape=(rows, cols // 32))
    if out is not None:
        _tensor(out, "out", torch.float32, shape=(rows, cols))
    dev = _same_gpu(codes, scales=scales, out=out)
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    st = lib().nvfp4_mxfp4_dequantize(_ptr(codes), _ptr(scales), rows, cols, _ptr(out), _stream(dev, stream))
    _check(st, "nvfp4_mxfp4_dequantize")
    return out


# ---- the consumer: FP4 GEMM (C = A B^T, operands with K contiguous) ------------

def _gemm_operand(codes, name: str) -> tuple:
    if not isinstance(codes, torch.Tensor) or codes.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor")
    _tensor(codes, name, torch.uint8)
    return codes.shape[0], 2 * codes.shape[1]


def gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, a_tensor_scale: torch.Tensor, b_codes: torch.Tensor,
         b_scales: torch.Tensor, b_tensor_scale: torch.Tensor, a_block: str = "1d", b_block: str = "1d",
         out: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """float32 [M][N] = A B^T from NVFP4 row copies (codes [M][K/2], [N][K/2])."""
    M, K = _gemm_operand(a_codes, "a_codes")
    N, Kb = _gemm_operand(b_codes, "b_codes")
    if Kb != K:
        raise ValueError("A and B must have the same K")
    for blk in (a_block, b_block):
        if blk not in BLOCKS:
            raise ValueError(f"block must be one of {sorted(BLOCKS)}, got {blk!r}")
    _tensor(a_scales, "a_scales", torch.uint8, shape=(M // 16, K // 16) if a_block == "2d" else (M, K // 16))
    _tensor(b_scales, "b_scales", torch.uint8, shape=(N // 16, K // 16) if b_block == "2d" else (N, K // 16))
    _tensor(a_tensor_scale, "a_tensor_scale", torch.float32, min_numel=1)
    _tensor(b_tensor_scale, "b_tensor_scale", torch.float32, min_numel=1)
    if out is not None:
        _tensor(out, "out", torch.float32, shape=(M, N))
    dev = _same_gpu(a_codes, a_scales=a_scales, a_tensor_scale=a_tensor_scale, b_codes=b_codes, b_scales=b_scales,
                    b_tensor_scale=b_tensor_scale, out=out)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=dev)
    st = lib().nvfp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(a_tensor_scale), BLOCKS[a_block], _ptr(b_codes),
                          _ptr(b_scales), _ptr(b_tensor_scale), BLOCKS[b_block], M, N, K, _ptr(out),
                          _stream(dev, stream))
    _check(st, "nvfp4_gemm")
    return out


def mxfp4_gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, b_codes: torch.Tensor, b_scales: torch.Tensor,
               out: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """float32 [M][N] = A B^T from MXFP4 row copies (codes [M][K/2], [N][K/2])."""
    M, K = _gemm_operand(a_codes, "a_codes")
    N, Kb = _gemm_operand(b_codes, "b_codes")
    if Kb != K:
        raise ValueError("A and B must have the same K")
    _tensor(a_scales, "a_scales", torch.uint8, shape=(M, K // 32))
    _tensor(b_scales, "b_scales", torch.uint8, shape=(N, K // 32))
    if out is not None:
        _tensor(out, "out", torch.float32, shape=(M, N))
    dev = _same_gpu(a_codes, a_scales=a_scales, b_codes=b_codes, b_scales=b_scales, out=out)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=dev)
    st = lib().nvfp4_mxfp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), M, N, K, _ptr(out),
                                _stream(dev, stream))
    _check(st, "nvfp4_mxfp4_gemm")
    return out
