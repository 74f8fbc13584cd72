"""Seeded synthetic inputs and the five NVFP4 quantization workloads.

This module draws numbers only; it holds none of the quantization arithmetic.
The GPU tests, the oracle-side checks and the benchmark all take their input
bytes from here, so every side sees identical tensors.
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")


def build() -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-fPIC", "-shared", "-pthread", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        L.synth_generate.restype = ctypes.c_int
        L.synth_generate.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_uint64,
                                     ctypes.c_void_p, ctypes.c_int]
        _lib = L
    return _lib


def generate(kind: int, rows: int, cols: int, seed: int = 0, nthreads: int | None = None) -> np.ndarray:
    """kind 1 -> float32 array; kinds 2..5 -> uint16 array of bf16 bit patterns."""
    if nthreads is None:
        nthreads = min(16, os.cpu_count() or 1)
    out = np.empty((rows, cols), np.float32 if kind == 1 else np.uint16)
    rc = _L().synth_generate(kind, rows, cols, seed, out.ctypes.data_as(ctypes.c_void_p), nthreads)
    if rc != 0:
        raise ValueError(f"synth_generate failed ({rc})")
    return out


def digest(x: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(x).view(np.uint8)).hexdigest()


# The five workloads: shape, input recipe and quantization options.
#   rule: 4/6 selection rule ("none" = always scale the block max to 6)
#   cap:  E4M3 limit used for the tensor scale
CONFIGS = {
    1: dict(name="256x256 fp32, 1x16 rows, RNE, cap 448, + dequantize",
            rows=256, cols=256, kind=1, dtype="f32", block="1d", emit_row=True, emit_col=False,
            rht=False, rht_seed=0, sr=False, sr_seed=0, rule="none", cap=448.0, dequant=True),
    2: dict(name="8192x4096 bf16 activation, 1x16 rows, 4/6 MSE, RNE, cap 256",
            rows=8192, cols=4096, kind=2, dtype="bf16", block="1d", emit_row=True, emit_col=False,
            rht=False, rht_seed=0, sr=False, sr_seed=0, rule="mse", cap=256.0, dequant=False),
    3: dict(name="5120x20480 bf16 weight, 16x16 tiles, row + col copies, RNE, cap 448",
            rows=5120, cols=20480, kind=3, dtype="bf16", block="2d", emit_row=True, emit_col=True,
            rht=False, rht_seed=0, sr=False, sr_seed=0, rule="none", cap=448.0, dequant=False),
    4: dict(name="8192x5120 bf16 gradient, RHT16, 1x16 rows, SR seed 1234, 4/6 MAE, cap 256",
            rows=8192, cols=5120, kind=4, dtype="bf16", block="1d", emit_row=True, emit_col=False,
            rht=True, rht_seed=1234, sr=True, sr_seed=1234, rule="mae", cap=256.0, dequant=False),
    5: dict(name="65536x8192 bf16 activation, 1x16 row + col copies, SR seed 7, 4/6 MAE, cap 256",
            rows=65536, cols=8192, kind=5, dtype="bf16", block="1d", emit_row=True, emit_col=True,
            rht=False, rht_seed=0, sr=True, sr_seed=7, rule="mae", cap=256.0, dequant=False),
}

# Config 5 is also run with 4/6 off (standard NVFP4, cap 448) to measure the 4/6 cost.
CONFIG5_PLAIN = dict(CONFIGS[5], name="65536x8192 bf16, 1x16 row + col copies, SR seed 7, no 4/6, cap 448",
                     rule="none", cap=448.0)

# Config 2 with 4/6 off (cap 448): the secondary 4/6-cost point (row copy only).
CONFIG2_PLAIN = dict(CONFIGS[2], name="8192x4096 bf16 activation, 1x16 rows, no 4/6, RNE, cap 448",
                     rule="none", cap=448.0)

# The weight with Four Over Six and stochastic rounding on its 16x16 tiles, both
# copies (activations, weights and gradients all in 4/6 format).
CONFIG3_SR = dict(CONFIGS[3], name="5120x20480 bf16 weight, 16x16 tiles, row + col copies, 4/6 MAE, SR seed 5, "
                                   "cap 256", rule="mae", sr=True, sr_seed=5, cap=256.0)


def config(k: int, rows: int | None = None, cols: int | None = None, **overrides) -> dict:
    """A copy of workload k, optionally at another shape (same recipe and options)."""
    c = dict(CONFIGS[k])
    if rows is not None:
        c["rows"] = rows
    if cols is not None:
        c["cols"] = cols
    c.update(overrides)
    return c


def inputs(c: dict, seed: int = 0) -> np.ndarray:
    return generate(c["kind"], c["rows"], c["cols"], seed)
