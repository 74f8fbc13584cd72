"""Pins of the oracle's MXFP4 functions (32-element blocks, power-of-two E8M0
scales; the contrast format of "Pretraining Large Language Models with NVFP4",
section 1).  The scale rule is the OCP Microscaling one (a reading: the pages
do not spell it out); everything else is pinned by brute force, the defining
range of the scaled block max and the behaviour section 1 describes."""
import math
from fractions import Fraction

import numpy as np
import pytest

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _bf16_to_f32(u16):
    return (u16.astype(np.uint32) << 16).view(np.float32)


def _nibbles(codes):
    """[.., n/2] packed bytes -> [.., n] codes, element 2k in the low nibble."""
    c = np.asarray(codes)
    out = np.empty(c.shape[:-1] + (2 * c.shape[-1],), np.uint8)
    out[..., 0::2] = c & 15
    out[..., 1::2] = c >> 4
    return out


def _brute_exponent(m: float) -> int:
    """The unique integer e in [-127, 127] with 4 <= m / 2^e < 8, found by
    search with exact arithmetic; clamped to the E8M0 range."""
    if m == 0.0:
        return -127
    fm = Fraction(m)
    for e in range(-127, 128):
        q = fm / (Fraction(2) ** e)
        if 4 <= q < 8:
            return e
    return -127 if fm < Fraction(4) * Fraction(2) ** -127 else 127


def _brute_code(y: float, e: int) -> int:
    """Nearest of the 16 E2M1 values times 2^e to y, by exact distance; ties to
    the even grid index; beyond the largest value, the largest (saturation)."""
    fy = Fraction(y)
    mag = abs(fy) / (Fraction(2) ** e)
    best = None
    for k, g in enumerate(GRID):
        d = abs(mag - Fraction(g))
        if best is None or d < best[0] or (d == best[0] and k % 2 == 0):
            best = (d, k)
    k = best[1]
    return k | (8 if y < 0 or (y == 0 and math.copysign(1.0, y) < 0) else 0)


def test_e8m0_values(orc):
    assert orc.e8m0_value(127) == 1.0
    assert orc.e8m0_value(0) == 2.0 ** -127
    assert orc.e8m0_value(254) == 2.0 ** 127
    assert math.isnan(orc.e8m0_value(255))  # the MX specification's NaN encoding
    for c in range(253):
        assert orc.e8m0_value(c + 1) == 2 * orc.e8m0_value(c)


def test_scale_code_brute_force(orc):
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 0x7F7FFFFF, 3000, dtype=np.uint32)  # every finite positive float32 magnitude
    special = np.array([0x00000001, 0x00800000, 0x01000000, 0x01800000, 0x3F800000, 0x40800000,
                        0x40FFFFFF, 0x41000000, 0x7F7FFFFF], np.uint32)
    for m in np.concatenate([bits, special]).view(np.float32):
        assert orc.mx_scale_code(float(m)) == _brute_exponent(float(m)) + 127, m
    assert orc.mx_scale_code(0.0) == 0


def test_block_brute_force(orc):
    """Codes and scales of random blocks against exhaustive nearest-value search."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 96)).astype(np.float32)
    x *= np.exp2(rng.integers(-20, 20, (6, 1))).astype(np.float32)
    x[0, :32] = 0.0
    x[1, 5] = -0.0
    x[2, 40] = 7.0 * abs(x[2, 32:64]).max()   # a scaled block max in (6, 8): saturates
    out = orc.mxfp4_quantize(x)
    codes = _nibbles(out["codes_row"])
    for r in range(6):
        for j in range(3):
            blk = x[r, 32 * j:32 * j + 32].astype(np.float64)
            e = _brute_exponent(float(np.abs(blk).max()))
            assert out["scales_row"][r, j] == e + 127
            for k in range(32):
                assert codes[r, 32 * j + k] == _brute_code(float(blk[k]), e), (r, j, k)


def test_scaled_block_max_range(orc):
    """The block max lands in [4, 8) after scaling, so its magnitude code is 6
    (value 4) or 7 (value 6, which also takes everything from 5 to 8)."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-30, 30, (64, 1)))).astype(np.float32)
    out = orc.mxfp4_quantize(x)
    codes = _nibbles(out["codes_row"]).reshape(64, 8, 32)
    amax_pos = np.abs(x).reshape(64, 8, 32).argmax(axis=2)
    top = np.take_along_axis(codes, amax_pos[..., None], axis=2)[..., 0] & 7
    assert set(np.unique(top)) <= {6, 7}
    blk_max = np.abs(x).reshape(64, 8, 32).max(axis=2).astype(np.float64)
    scale = np.exp2(out["scales_row"].astype(np.float64) - 127)
    q = blk_max / scale
    assert np.all((q >= 4) & (q < 8))


def test_outliers_crush_small_values(orc):
    """Section 1's contrast: one outlier sets a power-of-two scale for all 32
    elements and the ordinary values fall to zero, while NVFP4's 16-element
    blocks keep the half without the outlier."""
    x = np.full((1, 32), 0.75, np.float32)
    x[0, 0] = 100.0
    mx = _nibbles(orc.mxfp4_quantize(x)["codes_row"])[0]
    assert mx[0] == 7 and np.all(mx[1:] == 0)           # 100 -> 6 * 16 = 96; 0.75 / 16 -> 0
    cfg = orc.make_config(block="1d", rule="none", cap=448.0)
    nv = orc.quantize(x, cfg, orc.amax(x))
    nv_codes = _nibbles(nv["codes_row"])[0]
    assert np.all(nv_codes[16:] != 0)                      # the outlier-free block keeps them
    deq = orc.dequantize(nv["codes_row"], nv["scales_row"], nv["tensor_scale"], 1, 32, "1d")
    assert np.all(np.abs(deq[0, 16:] - 0.75) < 0.05)  # off only by the E4M3 rounding of the block scale


def test_nvfp4_error_below_mxfp4(orc, wl):
    """Smaller blocks with finer E4M3 scales give a lower error than MXFP4 on
    the same data (the claim of section 1), on the outlier-laden fp32 workload."""
    c = wl.config(1)
    x = wl.inputs(c)
    mx = orc.mxfp4_quantize(x)
    xm = orc.mxfp4_dequantize(mx["codes_row"], mx["scales_row"], *x.shape)
    cfg = orc.make_config(block="1d", rule="none", cap=448.0)
    nv = orc.quantize(x, cfg, orc.amax(x))
    xn = orc.dequantize(nv["codes_row"], nv["scales_row"], nv["tensor_scale"], *x.shape, "1d")
    e_mx = np.mean((xm.astype(np.float64) - x) ** 2)
    e_nv = np.mean((xn.astype(np.float64) - x) ** 2)
    assert e_nv < 0.8 * e_mx


def test_column_copy_is_row_copy_of_transpose(orc):
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((96, 64)) * 3).astype(np.float32)
    both = orc.mxfp4_quantize(x, emit_row=True, emit_col=True)
    t = orc.mxfp4_quantize(np.ascontiguousarray(x.T))
    assert np.array_equal(both["codes_col"], t["codes_row"])
    assert np.array_equal(both["scales_col"], t["scales_row"])


def test_bf16_input_matches_f32(orc):
    rng = np.random.default_rng(2)
    u = rng.integers(0, 1 << 16, (64, 64), dtype=np.uint32).astype(np.uint16)
    u[(u & 0x7F80) == 0x7F80] = 0x3F80  # no inf / nan
    a = orc.mxfp4_quantize(u, emit_col=True, sr=True, sr_seed=4)
    b = orc.mxfp4_quantize(_bf16_to_f32(u), emit_col=True, sr=True, sr_seed=4)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_dequantize_round_trip(orc):
    """Values on the scaled grid, with the block max in [4, 8) * 2^e, come back exactly."""
    rng = np.random.default_rng(8)
    e = rng.integers(-30, 30, (8, 4))
    g = np.array(GRID)[rng.integers(0, 8, (8, 4, 32))] * rng.choice([-1, 1], (8, 4, 32))
    g[..., 0] = 6.0
    x = (g * np.exp2(e)[..., None]).reshape(8, 128).astype(np.float32)
    out = orc.mxfp4_quantize(x)
    assert np.array_equal(out["scales_row"], (e + 127).astype(np.uint8))
    back = orc.mxfp4_dequantize(out["codes_row"], out["scales_row"], 8, 128)
    assert np.array_equal(back, x)


def test_stochastic_rounding_unbiased(orc):
    """E[dequantized] equals the input: every block is [6, v, v, ...] with scale
    1, so each v rounds stochastically between its two grid neighbours."""
    vals = np.array([0.3, 1.2, 2.6, 5.0], np.float32)
    n = 1 << 14
    x = np.empty((n, 32), np.float32)
    x[:, 0] = 6.0
    x[:, 1:] = np.tile(np.repeat(vals, 8)[1:], (n, 1))
    out = orc.mxfp4_quantize(x, sr=True, sr_seed=99)
    assert np.all(out["scales_row"] == 127)
    d = orc.mxfp4_dequantize(out["codes_row"], out["scales_row"], n, 32).astype(np.float64)
    col_of = np.repeat(vals, 8)
    for k, v in enumerate(vals):
        cols = [c for c in range(1, 32) if col_of[c] == v]
        sample = d[:, cols].ravel()
        lo = max(g for g in GRID if g <= v)
        hi = min(g for g in GRID if g >= v)
        assert set(np.unique(sample)) == {lo, hi}
        sd = (hi - lo) / 2 / math.sqrt(sample.size)
        assert abs(sample.mean() - v) < 5 * sd, v


def test_rejects_ragged_shapes(orc):
    with pytest.raises(ValueError):
        orc.mxfp4_quantize(np.zeros((4, 48), np.float32))
    with pytest.raises(ValueError):
        orc.mxfp4_quantize(np.zeros((48, 32), np.float32), emit_col=True)
