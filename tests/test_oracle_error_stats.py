"""Pins of the oracle's error analysis by scaled value ("Technical summary:
Four Over Six (4/6)", "Problem statement": the rounding error of values near
the block max, around the scaled value 5, dominates, while the quantization of
the scale factor itself matters little)."""
from fractions import Fraction

import numpy as np
import pytest

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _bf16_to_f32(u16):
    return (u16.astype(np.uint32) << 16).view(np.float32)


def _as_f32(x):
    return _bf16_to_f32(x) if x.dtype == np.uint16 else x.astype(np.float32)


def _transformed(orc, x, mask):
    """The values actually quantized: x, or its 16-point transform per row block."""
    y = _as_f32(x).copy()
    if mask is None:
        return y
    M, N = y.shape
    for r in range(M):
        for j in range(N // 16):
            y[r, 16 * j:16 * j + 16] = orc.rht16(y[r, 16 * j:16 * j + 16], mask)
    return y


def _setup(orc, wl, k, rows, cols, rule):
    c = wl.config(k, rows, cols)
    x = wl.inputs(c)
    mask = orc.rht_mask_from_seed(c["rht_seed"]) if c["rht"] else 0
    a = orc.amax(x, rht=c["rht"], mask=mask)
    cap = 448.0 if rule == "none" else 256.0
    cfg = orc.make_config(block=c["block"], rht=c["rht"], rht_mask=mask, rule=rule, cap=cap)
    return c, x, mask, a, cfg


CASES = [(2, 64, 256, "none"), (2, 64, 256, "mse"), (4, 32, 512, "mae"), (3, 64, 128, "none"), (3, 64, 128, "maxerr")]


@pytest.mark.parametrize("k,rows,cols,rule", CASES)
def test_bins_and_sums_recomputed_from_quantize(orc, wl, k, rows, cols, rule):
    """Counts and squared errors per bin, rebuilt from the (separately pinned)
    quantize and dequantize outputs with numpy."""
    c, x, mask, a, cfg = _setup(orc, wl, k, rows, cols, rule)
    st = orc.error_stats(x, cfg, a, 0.25, 26)
    q = orc.quantize(x, cfg, a)
    xh = orc.dequantize(q["codes_row"], q["scales_row"], q["tensor_scale"], rows, cols, c["block"])
    y = _transformed(orc, x, mask if c["rht"] else None)
    eps = (y - xh).astype(np.float32).astype(np.float64)
    # the scaled value z = fl(y * e), e = fl(1 / fl(dec(sb) * S_t)) of the block's chosen scale
    s_t = np.float32(q["tensor_scale"])
    dec = np.array([orc.e4m3_value(v) for v in range(256)], np.float32)
    if c["block"] == "2d":
        sb = np.repeat(np.repeat(q["scales_row"], 16, axis=0), 16, axis=1)
    else:
        sb = np.repeat(q["scales_row"], 16, axis=1)
    d = (dec[sb] * s_t).astype(np.float32)
    with np.errstate(divide="ignore"):
        e = np.where(d != 0, (np.float32(1) / d).astype(np.float32), np.float32(0))
    z = (y * e).astype(np.float32)
    b = np.minimum(np.floor(np.abs(z) * 4).astype(np.int64), 25)
    counts = np.bincount(b.ravel(), minlength=26)
    sse = np.bincount(b.ravel(), weights=(eps ** 2).ravel(), minlength=26)
    assert np.array_equal(st[0], counts.astype(np.float64))
    assert st[0].sum() == rows * cols
    # the same exact squares summed in another order: relative difference within n * 2^-53
    tol = counts * 2.0 ** -52 * sse + 1e-300
    assert np.all(np.abs(st[1] - sse) <= tol)


def _nearest_even(q: Fraction) -> Fraction:
    best = None
    for k, g in enumerate(GRID):
        dist = abs(q - Fraction(g))
        if best is None or dist < best[0] or (dist == best[0] and k % 2 == 0):
            best = (dist, k)
    return Fraction(GRID[best[1]])


def test_exact_scale_reference_brute_force(orc, wl):
    """The exact-scale error sums, rebuilt with rationals in the oracle's
    element order (so the binary64 sums agree exactly)."""
    c, x, mask, a, cfg = _setup(orc, wl, 2, 16, 64, "mse")
    st = orc.error_stats(x, cfg, a, 0.5, 13)
    q = orc.quantize(x, cfg, a, picks=True)
    y = _as_f32(x)
    s_t = np.float32(q["tensor_scale"])
    dec = np.array([orc.e4m3_value(v) for v in range(256)], np.float32)
    ref = np.zeros(13)
    for r in range(16):
        for j in range(4):
            blk = y[r, 16 * j:16 * j + 16]
            T = 4 if q["pick_row"][r, j] else 6
            m = Fraction(float(np.abs(blk).max()))
            dd = np.float32(dec[q["scales_row"][r, j]] * s_t)
            ee = np.float32(np.float32(1) / dd) if dd != 0 else np.float32(0)
            for v in blk:
                z = np.float32(v * ee)
                b = min(int(np.floor(abs(float(z)) * 2)), 12)
                xs = 0.0 if m == 0 else float(_nearest_even(T * abs(Fraction(float(v))) / m) * m / T)
                es = float(v) - np.copysign(xs, float(v))
                ref[b] += es * es
    assert np.array_equal(st[2], ref)


def test_error_near_five_dominates_after_the_transform(orc, wl):
    """On the transformed gradient (near-Gaussian blocks), standard NVFP4's
    per-element error peaks in the bins around the scaled value 5 and the
    [4, 6) range carries several times its share of elements; Four Over Six
    lowers the total error and that range's share."""
    c, x, mask, a, cfg = _setup(orc, wl, 4, 64, 1024, "none")
    st = orc.error_stats(x, cfg, a, 0.25, 26)
    mean = st[1] / np.maximum(st[0], 1)
    peak = np.argmax(np.where(st[0] > 100, mean, 0)) * 0.25
    assert 4.5 <= peak < 5.5
    share_err = st[1][16:24].sum() / st[1].sum()
    share_el = st[0][16:24].sum() / st[0].sum()
    assert share_err > 2.5 * share_el and share_err > 0.5
    cfg46 = orc.make_config(rht=True, rht_mask=mask, rule="mse", cap=256.0)
    st46 = orc.error_stats(x, cfg46, a, 0.25, 26)
    assert st46[1].sum() < 0.85 * st[1].sum()
    assert st46[1][16:24].sum() / st46[1].sum() < share_err


@pytest.mark.parametrize("k", [2, 3, 4, 5])
def test_scale_factor_quantization_matters_little(orc, wl, k):
    """Exact (unquantized) block scales change the total squared error by
    under 10% on every workload's data."""
    c, x, mask, a, cfg = _setup(orc, wl, k, 64, 512, "none")
    st = orc.error_stats(x, cfg, a)
    assert abs(1.0 - st[2].sum() / st[1].sum()) < 0.10


def test_rejects_unsupported(orc):
    x = np.zeros((16, 32), np.float32)
    with pytest.raises(ValueError):
        orc.error_stats(x, orc.make_config(sr=True), 1.0)
    with pytest.raises(ValueError):
        orc.error_stats(x, orc.make_config(), 1.0, bin_width=0.3)
    with pytest.raises(ValueError):
        orc.error_stats(np.zeros((8, 32), np.float32), orc.make_config(), 1.0)
