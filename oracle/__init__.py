"""ctypes binding of the plain C oracle (nvfp4_oracle.c).

TEST INFRASTRUCTURE ONLY: this is the reference the GPU path is checked
against.  Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import it; the product package never does.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_nvfp4.so")

IN_BF16, IN_F32 = 0, 1
RULE_NONE, RULE_MSE, RULE_MAE, RULE_MAXERR = 0, 1, 2, 3
RULES = {"none": RULE_NONE, "mse": RULE_MSE, "mae": RULE_MAE, "maxerr": RULE_MAXERR}


def build() -> str:
    """Compile the oracle with a fixed binary32 operation order (no FMA contraction)."""
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-pthread", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class Config(ctypes.Structure):
    _fields_ = [
        ("block_2d", ctypes.c_int32),
        ("emit_row", ctypes.c_int32),
        ("emit_col", ctypes.c_int32),
        ("rht", ctypes.c_int32),
        ("rht_mask", ctypes.c_uint32),
        ("sr", ctypes.c_int32),
        ("sr_seed", ctypes.c_uint64),
        ("row_offset", ctypes.c_int64),
        ("rule", ctypes.c_int32),
        ("cap", ctypes.c_float),
    ]


_lib = None


def _signatures():
    P = ctypes.c_void_p
    i64, u64, u32, f32, i32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_float, ctypes.c_int
    return {
        "orc_bf16_to_f32": (f32, [ctypes.c_uint16]),
        "orc_e2m1_rne": (ctypes.c_uint8, [f32]),
        "orc_e2m1_sr": (ctypes.c_uint8, [f32, u32]),
        "orc_e2m1_value": (f32, [ctypes.c_uint8]),
        "orc_e4m3_rne_sat": (ctypes.c_uint8, [f32]),
        "orc_e4m3_value": (f32, [ctypes.c_uint8]),
        "orc_philox4x32_10": (None, [P, P, P]),
        "orc_sr_word": (u32, [u64, u64]),
        "orc_rht_mask_from_seed": (u32, [u64]),
        "orc_rht16": (None, [P, u32, P]),
        "orc_quantize_block": (None, [P, i32, f32, i32, i32, P, P, P, P, P]),
        "orc_amax": (f32, [P, i32, i64, i64, i32, u32]),
        "orc_tensor_scale": (f32, [f32, f32]),
        "orc_quantize": (i32, [P, i32, i64, i64, ctypes.POINTER(Config), f32, P, P, P, P, P, P, P, i32]),
        "orc_dequantize": (None, [P, P, f32, i64, i64, i32, P]),
        "orc_e2m1_rne_n": (None, [P, i64, P]),
        "orc_e2m1_sr_n": (None, [P, P, i64, P]),
        "orc_e4m3_rne_sat_n": (None, [P, i64, P]),
        "orc_sr_words_n": (None, [u64, P, i64, P]),
        "orc_philox_n": (None, [P, P, i64, P]),
        "orc_e8m0_value": (f32, [ctypes.c_uint8]),
        "orc_mx_scale_code": (ctypes.c_uint8, [f32]),
        "orc_mxfp4_quantize": (i32, [P, i32, i64, i64, i32, i32, i32, u64, i64, P, P, P, P]),
        "orc_mxfp4_dequantize": (None, [P, P, i64, i64, P]),
        "orc_gemm_fp4": (i32, [i32, P, P, f32, i32, P, P, f32, i32, i64, i64, i64, P, P]),
        "orc_error_stats": (i32, [P, i32, i64, i64, ctypes.POINTER(Config), f32, f32, i32, P]),
    }


def _bind(path: str) -> ctypes.CDLL:
    L = ctypes.CDLL(path)
    for name, (res, args) in _signatures().items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def lib():
    global _lib
    if _lib is None:
        src_mtime = max(os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "nvfp4_oracle.h")))
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < src_mtime:
            build()
        _lib = _bind(_LIB)
    return _lib


def build_variant(source: str, out_dir: str, name: str = "variant") -> str:
    """Compile another text of nvfp4_oracle.c (same header, same flags) into
    out_dir; the tests use this to plant a mistake in a copy of the oracle and
    check that the pins catch it."""
    src = os.path.join(out_dir, f"{name}.c")
    with open(src, "w") as f:
        f.write(source)
    so = os.path.join(out_dir, f"lib{name}.so")
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread",
           "-I", _HERE, "-o", so, src, "-lm"]
    subprocess.run(cmd, check=True)
    return so


def source() -> str:
    with open(_SRC) as f:
        return f.read()


@contextlib.contextmanager
def library(path: str):
    """Route every call of this module through another build of the oracle
    (e.g. one from build_variant) for the duration of the block."""
    global _lib
    saved = lib()
    _lib = _bind(path)
    try:
        yield
    finally:
        _lib = saved


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ---- scalar / vector forms of the format functions ------------------------

def e2m1_rne(z) -> np.ndarray:
    z = np.ascontiguousarray(z, dtype=np.float32).ravel()
    out = np.empty(z.shape, np.uint8)
    lib().orc_e2m1_rne_n(_ptr(z), z.size, _ptr(out))
    return out


def e2m1_sr(z, words) -> np.ndarray:
    z = np.ascontiguousarray(z, dtype=np.float32).ravel()
    w = np.ascontiguousarray(words, dtype=np.uint32).ravel()
    assert z.size == w.size
    out = np.empty(z.shape, np.uint8)
    lib().orc_e2m1_sr_n(_ptr(z), _ptr(w), z.size, _ptr(out))
    return out


def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(code)


def e4m3_rne_sat(r) -> np.ndarray:
    r = np.ascontiguousarray(r, dtype=np.float32).ravel()
    out = np.empty(r.shape, np.uint8)
    lib().orc_e4m3_rne_sat_n(_ptr(r), r.size, _ptr(out))
    return out


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(code)


def philox(ctr, key) -> np.ndarray:
    """ctr: (n,4) uint32, key: (n,2) uint32 -> (n,4) uint32."""
    c = np.ascontiguousarray(ctr, dtype=np.uint32).reshape(-1, 4)
    k = np.ascontiguousarray(key, dtype=np.uint32).reshape(-1, 2)
    assert c.shape[0] == k.shape[0]
    out = np.empty_like(c)
    lib().orc_philox_n(_ptr(c), _ptr(k), c.shape[0], _ptr(out))
    return out


def sr_words(seed: int, idx) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.uint64).ravel()
    out = np.empty(idx.shape, np.uint32)
    lib().orc_sr_words_n(seed, _ptr(idx), idx.size, _ptr(out))
    return out


def rht_mask_from_seed(seed: int) -> int:
    return int(lib().orc_rht_mask_from_seed(seed))


def rht16(x, mask: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.size == 16
    y = np.empty(16, np.float32)
    lib().orc_rht16(_ptr(x), mask, _ptr(y))
    return y


def quantize_block(y, s_t: float, rule: str = "none", sr: bool = False, words=None):
    """Returns (codes[n] uint8, scale code, chose4, (err6, err4))."""
    y = np.ascontiguousarray(y, dtype=np.float32).ravel()
    n = y.size
    assert n in (16, 256)
    w = None
    if sr:
        w = np.ascontiguousarray(words, dtype=np.uint32).ravel()
        assert w.size == n
    codes = np.empty(n, np.uint8)
    sb = np.zeros(1, np.uint8)
    ch = np.zeros(1, np.uint8)
    err = np.zeros(2, np.float32)
    lib().orc_quantize_block(_ptr(y), n, s_t, RULES[rule], int(sr), _ptr(w), _ptr(codes), _ptr(sb), _ptr(ch), _ptr(err))
    return codes, int(sb[0]), bool(ch[0]), (float(err[0]), float(err[1]))


# ---- tensor level ---------------------------------------------------------

def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return IN_F32
    if x.dtype == np.uint16:  # bf16 bit patterns
        return IN_BF16
    raise TypeError("oracle input must be float32 or uint16 (bf16 bit patterns)")


def amax(x: np.ndarray, rht: bool = False, mask: int = 0) -> float:
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    return float(lib().orc_amax(_ptr(x), _dtype_code(x), rows, cols, int(rht), mask))


def tensor_scale(a: float, cap: float) -> float:
    return float(lib().orc_tensor_scale(a, cap))


def make_config(block: str = "1d", emit_row: bool = True, emit_col: bool = False, rht: bool = False,
                rht_mask: int = 0, sr: bool = False, sr_seed: int = 0, row_offset: int = 0,
                rule: str = "none", cap: float = 448.0) -> Config:
    return Config(1 if block == "2d" else 0, int(emit_row), int(emit_col), int(rht), rht_mask, int(sr),
                  sr_seed, row_offset, RULES[rule], cap)


def quantize(x: np.ndarray, cfg: Config, a: float, nthreads: int = 1, picks: bool = False) -> dict:
    """Full-tensor quantization; returns a dict of numpy outputs."""
    x = np.ascontiguousarray(x)
    M, N = x.shape
    out = {}
    sb_cols = N // 16
    if cfg.emit_row:
        out["codes_row"] = np.zeros((M, N // 2), np.uint8)
        out["scales_row"] = np.zeros(((M // 16, sb_cols) if cfg.block_2d else (M, sb_cols)), np.uint8)
    if cfg.emit_col:
        out["codes_col"] = np.zeros((N, M // 2), np.uint8)
        out["scales_col"] = np.zeros(((N // 16, M // 16) if cfg.block_2d else (N, M // 16)), np.uint8)
    ts = np.zeros(1, np.float32)
    pr = np.zeros(out["scales_row"].shape, np.uint8) if (picks and cfg.emit_row) else None
    pc = np.zeros(out["scales_col"].shape, np.uint8) if (picks and cfg.emit_col) else None
    rc = lib().orc_quantize(_ptr(x), _dtype_code(x), M, N, ctypes.byref(cfg), a,
                            _ptr(out.get("codes_row")), _ptr(out.get("scales_row")),
                            _ptr(out.get("codes_col")), _ptr(out.get("scales_col")),
                            _ptr(ts), _ptr(pr), _ptr(pc), nthreads)
    if rc != 0:
        raise ValueError(f"oracle rejected the shape/config (code {rc})")
    out["tensor_scale"] = float(ts[0])
    if pr is not None:
        out["pick_row"] = pr
    if pc is not None:
        out["pick_col"] = pc
    return out


def dequantize(codes: np.ndarray, scales: np.ndarray, s_t: float, rows: int, cols: int, block: str = "1d") -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.empty((rows, cols), np.float32)
    lib().orc_dequantize(_ptr(codes), _ptr(scales), s_t, rows, cols, 1 if block == "2d" else 0, _ptr(out))
    return out


# ---- MXFP4 -------------------------------------------------------------------

def e8m0_value(code: int) -> float:
    return float(lib().orc_e8m0_value(code))


def mx_scale_code(block_max: float) -> int:
    return int(lib().orc_mx_scale_code(block_max))


def mxfp4_quantize(x: np.ndarray, emit_row: bool = True, emit_col: bool = False, sr: bool = False,
                   sr_seed: int = 0, row_offset: int = 0) -> dict:
    """MXFP4 row copy (codes_row [M, N/2], scales_row [M, N/32]) and/or column
    copy (codes_col [N, M/2], scales_col [N, M/32]) as E8M0 scale codes."""
    x = np.ascontiguousarray(x)
    M, N = x.shape
    out = {}
    cr = sr_ = cc = sc = None
    if emit_row:
        cr = out["codes_row"] = np.zeros((M, N // 2), np.uint8)
        sr_ = out["scales_row"] = np.zeros((M, N // 32), np.uint8)
    if emit_col:
        cc = out["codes_col"] = np.zeros((N, M // 2), np.uint8)
        sc = out["scales_col"] = np.zeros((N, M // 32), np.uint8)
    rc = lib().orc_mxfp4_quantize(_ptr(x), _dtype_code(x), M, N, int(emit_row), int(emit_col), int(sr), sr_seed,
                                  row_offset, _ptr(cr), _ptr(sr_), _ptr(cc), _ptr(sc))
    if rc != 0:
        raise ValueError(f"oracle rejected the MXFP4 shape (code {rc})")
    return out


def mxfp4_dequantize(codes: np.ndarray, scales: np.ndarray, rows: int, cols: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.empty((rows, cols), np.float32)
    lib().orc_mxfp4_dequantize(_ptr(codes), _ptr(scales), rows, cols, _ptr(out))
    return out


# ---- error analysis ------------------------------------------------------------

def error_stats(x: np.ndarray, cfg: Config, a: float, bin_width: float = 0.25, nbins: int = 26) -> np.ndarray:
    """(3, nbins) float64: per scaled-value bin, the element count, the sum of
    squared errors of the quantized path and of the exact-scale reference."""
    x = np.ascontiguousarray(x)
    M, N = x.shape
    out = np.zeros((3, nbins), np.float64)
    rc = lib().orc_error_stats(_ptr(x), _dtype_code(x), M, N, ctypes.byref(cfg), a, bin_width, nbins, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle rejected the error-analysis arguments (code {rc})")
    return out


# ---- the consumer GEMM -------------------------------------------------------------

def gemm_fp4(mx: bool, a_codes, a_scales, b_codes, b_scales, M: int, N: int, K: int, a_ts: float = 1.0,
             b_ts: float = 1.0, a_2d: bool = False, b_2d: bool = False):
    """C = A B^T on FP4 operands (float32 [M][N]) and sum |A B| (float64 [M][N])."""
    ac = np.ascontiguousarray(a_codes, dtype=np.uint8)
    asc = np.ascontiguousarray(a_scales, dtype=np.uint8)
    bc = np.ascontiguousarray(b_codes, dtype=np.uint8)
    bsc = np.ascontiguousarray(b_scales, dtype=np.uint8)
    c = np.empty((M, N), np.float32)
    cabs = np.empty((M, N), np.float64)
    rc = lib().orc_gemm_fp4(int(mx), _ptr(ac), _ptr(asc), a_ts, int(a_2d), _ptr(bc), _ptr(bsc), b_ts, int(b_2d),
                            M, N, K, _ptr(c), _ptr(cabs))
    if rc != 0:
        raise ValueError(f"oracle rejected the GEMM shape (code {rc})")
    return c, cabs
