"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import nvfp4_block_quantization_amd as nv

pytestmark = pytest.mark.skipif(not os.path.exists(nv.LIB_PATH), reason="libnvfp4.so not built")

FAKE = 0x10000  # 16-byte aligned dummy device address (never dereferenced: validation fails first)


def _declared_functions():
    src = open(nv.HEADER_PATH).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 7
    L = nv.lib()
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    assert nv.abi_version() == 2
    for s in range(8):
        assert nv.lib().nvfp4_status_string(s)


def test_rht_mask_from_seed_matches_oracle(orc):
    for seed in (0, 1, 7, 1234, 2 ** 40 + 3):
        assert nv.rht_signs_from_seed(seed) == orc.rht_mask_from_seed(seed)


def _q(rows=64, cols=64, x=FAKE, dtype=0, cfg=None, amax=FAKE, outs=None):
    cfg = cfg or nv.make_config()
    outs = outs or nv.Outputs(FAKE, FAKE, FAKE, FAKE, FAKE)
    return nv.lib().nvfp4_quantize(ctypes.c_void_p(x) if x else None, dtype, rows, cols, ctypes.byref(cfg),
                                   ctypes.c_void_p(amax) if amax else None, ctypes.byref(outs), None)


def test_quantize_validation():
    assert _q(cols=24) == nv.ERR_SHAPE
    assert _q(rows=-1) == nv.ERR_SHAPE
    assert _q(rows=8, cfg=nv.make_config(colwise=True)) == nv.ERR_SHAPE
    assert _q(rows=8, cfg=nv.make_config(block="2d")) == nv.ERR_SHAPE
    assert _q(rows=16, cols=(1 << 24) + 16, cfg=nv.make_config(colwise=True)) == nv.ERR_SHAPE
    assert _q(rows=16, cols=(1 << 24) + 16, cfg=nv.make_config(block="2d")) == nv.ERR_SHAPE
    assert _q(cfg=nv.make_config(block="2d", rht=True)) == nv.ERR_UNSUPPORTED
    assert _q(cfg=nv.make_config(colwise=True, rht=True)) == nv.ERR_UNSUPPORTED
    assert _q(cfg=nv.make_config(scale_cap=300.0)) == nv.ERR_UNSUPPORTED
    assert _q(cfg=nv.make_config(rowwise=False, colwise=False)) == nv.ERR_UNSUPPORTED
    bad_rule = nv.make_config()
    bad_rule.rule = 7
    assert _q(cfg=bad_rule) == nv.ERR_UNSUPPORTED
    assert _q(dtype=5) == nv.ERR_DTYPE
    assert _q(x=0) == nv.ERR_NULL
    assert _q(amax=0) == nv.ERR_NULL
    assert _q(outs=nv.Outputs(None, FAKE, None, None, FAKE)) == nv.ERR_NULL
    assert _q(x=FAKE + 4) == nv.ERR_ALIGN
    assert _q(outs=nv.Outputs(FAKE + 8, FAKE, None, None, FAKE)) == nv.ERR_ALIGN


def test_amax_and_dequantize_validation():
    L = nv.lib()
    cfg = nv.make_config(rht=True)
    ws = nv.amax_workspace_bytes(64, 64)
    assert 4 <= ws <= 4096
    P = ctypes.c_void_p
    assert L.nvfp4_amax(P(FAKE), 0, 64, 24, ctypes.byref(cfg), P(FAKE), P(FAKE), ws, None) == nv.ERR_SHAPE
    assert L.nvfp4_amax(P(FAKE), 0, 64, 64, None, P(FAKE), P(FAKE), ws - 4, None) == nv.ERR_WORKSPACE
    assert L.nvfp4_amax(P(FAKE), 0, 64, 64, None, None, P(FAKE), ws, None) == nv.ERR_NULL
    assert L.nvfp4_amax(P(FAKE + 2), 0, 64, 64, None, P(FAKE), P(FAKE), ws, None) == nv.ERR_ALIGN
    assert L.nvfp4_amax(P(FAKE), 3, 64, 64, None, P(FAKE), P(FAKE), ws, None) == nv.ERR_DTYPE
    assert L.nvfp4_dequantize(P(FAKE), P(FAKE), P(FAKE), 16, 24, 0, P(FAKE), None) == nv.ERR_SHAPE
    assert L.nvfp4_dequantize(P(FAKE), P(FAKE), P(FAKE), 8, 32, 1, P(FAKE), None) == nv.ERR_SHAPE
    assert L.nvfp4_dequantize(P(FAKE), P(FAKE), P(FAKE), 16, 32, 2, P(FAKE), None) == nv.ERR_UNSUPPORTED
    assert L.nvfp4_dequantize(None, P(FAKE), P(FAKE), 16, 32, 0, P(FAKE), None) == nv.ERR_NULL
    assert L.nvfp4_dequantize(P(FAKE + 8), P(FAKE), P(FAKE), 16, 32, 0, P(FAKE), None) == nv.ERR_ALIGN


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(TypeError):
        nv.amax(torch.zeros(16, 16, dtype=torch.bfloat16))


def _mx(rows=64, cols=64, x=FAKE, dtype=0, cfg=None, outs=None):
    cfg = cfg or nv.MXConfig(1, 0, 0, 0, 0)
    outs = outs or nv.MXOutputs(FAKE, FAKE, FAKE, FAKE)
    return nv.lib().nvfp4_mxfp4_quantize(ctypes.c_void_p(x) if x else None, dtype, rows, cols, ctypes.byref(cfg),
                                         ctypes.byref(outs), None)


def test_mxfp4_validation():
    assert _mx(cols=48) == nv.ERR_SHAPE
    assert _mx(rows=-32) == nv.ERR_SHAPE
    assert _mx(rows=48, cfg=nv.MXConfig(0, 1, 0, 0, 0)) == nv.ERR_SHAPE
    assert _mx(rows=32, cols=(1 << 24) + 32, cfg=nv.MXConfig(0, 1, 0, 0, 0)) == nv.ERR_SHAPE
    assert _mx(cfg=nv.MXConfig(0, 0, 0, 0, 0)) == nv.ERR_UNSUPPORTED
    assert _mx(dtype=2) == nv.ERR_DTYPE
    assert _mx(x=0) == nv.ERR_NULL
    assert _mx(outs=nv.MXOutputs(FAKE, None, None, None)) == nv.ERR_NULL
    assert _mx(cfg=nv.MXConfig(1, 1, 0, 0, 0), outs=nv.MXOutputs(FAKE, FAKE, FAKE, None)) == nv.ERR_NULL
    assert _mx(x=FAKE + 8) == nv.ERR_ALIGN
    assert _mx(outs=nv.MXOutputs(FAKE + 4, FAKE, None, None)) == nv.ERR_ALIGN
    assert _mx(rows=0) == nv.OK  # empty: nothing to do
    P = ctypes.c_void_p
    L = nv.lib()
    assert L.nvfp4_mxfp4_dequantize(P(FAKE), P(FAKE), 32, 48, P(FAKE), None) == nv.ERR_SHAPE
    assert L.nvfp4_mxfp4_dequantize(None, P(FAKE), 32, 32, P(FAKE), None) == nv.ERR_NULL
    assert L.nvfp4_mxfp4_dequantize(P(FAKE), P(FAKE), 32, 32, P(FAKE + 4), None) == nv.ERR_ALIGN


def test_error_stats_validation():
    L = nv.lib()
    P = ctypes.c_void_p

    def es(rows=64, cols=64, cfg=None, w=0.25, nb=26, x=FAKE, amax=FAKE, out=FAKE):
        cfg = cfg or nv.make_config()
        return L.nvfp4_error_stats(P(x) if x else None, 0, rows, cols, ctypes.byref(cfg), P(amax) if amax else None,
                                   w, nb, P(out) if out else None, None)
    assert es(rows=8) == nv.ERR_SHAPE
    assert es(cols=24) == nv.ERR_SHAPE
    assert es(cfg=nv.make_config(sr=True)) == nv.ERR_UNSUPPORTED
    assert es(cfg=nv.make_config(block="2d", rht=True)) == nv.ERR_UNSUPPORTED
    assert es(w=0.3) == nv.ERR_UNSUPPORTED
    assert es(w=0.0) == nv.ERR_UNSUPPORTED
    assert es(nb=0) == nv.ERR_UNSUPPORTED
    assert es(nb=65) == nv.ERR_UNSUPPORTED
    assert es(out=0) == nv.ERR_NULL
    assert es(amax=0) == nv.ERR_NULL
    assert es(x=FAKE + 4) == nv.ERR_ALIGN


def test_gemm_validation():
    L = nv.lib()
    P = ctypes.c_void_p
    f = P(FAKE)

    def g(M=64, N=64, K=128, ab=0, bb=0, ac=FAKE, c=FAKE):
        return L.nvfp4_gemm(P(ac) if ac else None, f, f, ab, f, f, f, bb, M, N, K, P(c) if c else None, None)
    assert g(K=192) == nv.ERR_SHAPE
    assert g(M=8, ab=1) == nv.ERR_SHAPE
    assert g(N=24, bb=1) == nv.ERR_SHAPE
    assert g(ab=3) == nv.ERR_UNSUPPORTED
    assert g(c=0) == nv.ERR_NULL
    assert g(ac=0) == nv.ERR_NULL
    assert g(ac=FAKE + 8) == nv.ERR_ALIGN
    assert g(c=FAKE + 2) == nv.ERR_ALIGN
    assert g(M=0) == nv.OK
    assert L.nvfp4_mxfp4_gemm(f, f, f, f, 64, 64, 192, f, None) == nv.ERR_SHAPE
    assert L.nvfp4_mxfp4_gemm(None, f, f, f, 64, 64, 256, f, None) == nv.ERR_NULL
    assert L.nvfp4_mxfp4_gemm(f, f, P(FAKE + 4), f, 64, 64, 256, f, None) == nv.ERR_ALIGN


# ------------------------------------------------ binding argument checks ----
# The C ABI cannot see buffer sizes, so the binding checks every tensor before
# calling it.  Device checks come last, which lets these CPU tests reach each
# shape/dtype rejection; a call whose tensors are all well formed but on the
# CPU ends in the "no CPU path" error.

def _t(*shape, dtype=None):
    torch = pytest.importorskip("torch")
    return torch.zeros(shape, dtype=dtype or torch.uint8)


def test_binding_quantize_checks_every_buffer():
    torch = pytest.importorskip("torch")
    x = torch.zeros(32, 64, dtype=torch.bfloat16)
    a = torch.zeros(1, dtype=torch.float32)
    good = nv.allocate_outputs(32, 64, "1d", True, True, "cpu")
    with pytest.raises(TypeError, match="GPU"):
        nv.quantize(x, a, colwise=True, out=good)
    with pytest.raises(TypeError, match="amax_t"):
        nv.quantize(x, a.double(), out=good)
    with pytest.raises(ValueError, match="amax_t"):
        nv.quantize(x, torch.zeros(0, dtype=torch.float32), out=good)
    for key, bad in (("codes_row", _t(32, 16)), ("scales_row", _t(32, 2)), ("codes_col", _t(64, 8)),
                     ("scales_col", _t(4, 2)), ("codes_row", _t(32, 32, dtype=torch.int8))):
        o = dict(good)
        o[key] = bad
        with pytest.raises((ValueError, TypeError), match=key):
            nv.quantize(x, a, colwise=True, out=o)
    o = dict(good)
    del o["codes_col"]
    with pytest.raises(ValueError, match="codes_col"):
        nv.quantize(x, a, colwise=True, out=o)
    # a 2D row copy has one scale per tile: the 1D-shaped scales are refused
    with pytest.raises(ValueError, match="scales_row"):
        nv.quantize(x, a, block="2d", out=good)
    with pytest.raises(ValueError, match="contiguous"):
        nv.quantize(x.t(), a)
    with pytest.raises(TypeError):
        nv.quantize(x.to(torch.float16), a)
    with pytest.raises(ValueError, match="16-bit"):
        nv.quantize(x, a, rht=True, rht_mask=0x1FFFF)
    with pytest.raises(ValueError, match="rule"):
        nv.quantize(x, a, rule="l2")


def test_binding_amax_dequantize_error_stats_checks():
    torch = pytest.importorskip("torch")
    x = torch.zeros(32, 64, dtype=torch.float32)
    with pytest.raises(ValueError, match="workspace"):
        nv.amax(x, workspace=torch.zeros(0, dtype=torch.uint8))
    with pytest.raises(TypeError, match="out"):
        nv.amax(x, out=torch.zeros(1, dtype=torch.float64))
    with pytest.raises(TypeError, match="GPU"):
        nv.amax(x, out=torch.zeros(1), workspace=torch.zeros(4096, dtype=torch.uint8))
    ts = torch.zeros(1)
    with pytest.raises(ValueError, match="codes"):
        nv.dequantize(_t(32, 16), _t(32, 4), ts, 32, 64)      # rows/cols disagree with codes.shape
    with pytest.raises(ValueError, match="scales"):
        nv.dequantize(_t(32, 32), _t(32, 4), ts, 32, 64, block="2d")
    with pytest.raises(ValueError, match="out"):
        nv.dequantize(_t(32, 32), _t(32, 4), ts, 32, 64, out=torch.zeros(32, 32))
    with pytest.raises(TypeError, match="tensor_scale"):
        nv.dequantize(_t(32, 32), _t(32, 4), ts.half(), 32, 64)
    with pytest.raises(TypeError, match="GPU"):
        nv.dequantize(_t(32, 32), _t(32, 4), ts, 32, 64)
    a = torch.zeros(1)
    with pytest.raises(ValueError, match="out"):
        nv.error_stats(x, a, nbins=8, out=torch.zeros(3, 9, dtype=torch.float64))
    with pytest.raises(ValueError, match="nbins"):
        nv.error_stats(x, a, nbins=65)


def test_binding_mxfp4_and_gemm_checks():
    torch = pytest.importorskip("torch")
    x = torch.zeros(64, 64, dtype=torch.bfloat16)
    good = nv.mxfp4_allocate_outputs(64, 64, True, True, "cpu")
    o = dict(good)
    o["scales_col"] = _t(64, 4)
    with pytest.raises(ValueError, match="scales_col"):
        nv.mxfp4_quantize(x, colwise=True, out=o)
    with pytest.raises(TypeError, match="GPU"):
        nv.mxfp4_quantize(x, colwise=True, out=good)
    with pytest.raises(ValueError, match="scales"):
        nv.mxfp4_dequantize(_t(64, 32), _t(64, 4), 64, 64)
    ts = torch.zeros(1)
    with pytest.raises(ValueError, match="same K"):
        nv.gemm(_t(64, 64), _t(64, 8), ts, _t(64, 32), _t(64, 4), ts)
    with pytest.raises(ValueError, match="b_scales"):
        nv.gemm(_t(64, 64), _t(64, 8), ts, _t(64, 64), _t(64, 8), ts, b_block="2d")
    with pytest.raises(ValueError, match="out"):
        nv.gemm(_t(64, 64), _t(64, 8), ts, _t(32, 64), _t(32, 8), ts, out=torch.zeros(64, 64))
    with pytest.raises(TypeError, match="GPU"):
        nv.gemm(_t(64, 64), _t(64, 8), ts, _t(32, 64), _t(32, 8), ts)
    with pytest.raises(ValueError, match="a_scales"):
        nv.mxfp4_gemm(_t(64, 64), _t(64, 8), _t(32, 64), _t(32, 4))
    with pytest.raises(TypeError, match="GPU"):
        nv.mxfp4_gemm(_t(64, 64), _t(64, 4), _t(32, 64), _t(32, 4))


def test_amax_noalloc_validation():
    """The allocation-free amax rejects bad arguments on the host, before it
    looks up its per-GPU scratch array or launches anything."""
    L = nv.lib()
    P = ctypes.c_void_p
    cfg = nv.make_config(rht=True)
    assert L.nvfp4_amax_noalloc(P(FAKE), 0, 64, 24, ctypes.byref(cfg), P(FAKE), None) == nv.ERR_SHAPE
    assert L.nvfp4_amax_noalloc(P(FAKE), 0, -1, 64, None, P(FAKE), None) == nv.ERR_SHAPE
    assert L.nvfp4_amax_noalloc(P(FAKE), 0, 64, 64, None, None, None) == nv.ERR_NULL
    assert L.nvfp4_amax_noalloc(None, 0, 64, 64, None, P(FAKE), None) == nv.ERR_NULL
    assert L.nvfp4_amax_noalloc(P(FAKE + 4), 0, 64, 64, None, P(FAKE), None) == nv.ERR_ALIGN
    assert L.nvfp4_amax_noalloc(P(FAKE), 7, 64, 64, None, P(FAKE), None) == nv.ERR_DTYPE
