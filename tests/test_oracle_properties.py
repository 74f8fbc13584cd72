"""Property-based pins of the oracle (hypothesis): invariants that follow from
the definitions and must hold for every input, so a dropped term, a wrong sign
or a swapped operand anywhere in the block arithmetic fails one of them."""
import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402
from hypothesis.extra import numpy as hnp  # noqa: E402

SETTINGS = settings(max_examples=150, deadline=None, derandomize=True)
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

finite = st.floats(min_value=-1e4, max_value=1e4, allow_nan=False, allow_infinity=False, width=32)
blocks = hnp.arrays(np.float32, 16, elements=finite)
rules = st.sampled_from(["none", "mse", "mae", "maxerr"])


def _vals(orc, codes):
    return np.array([orc.e2m1_value(int(c)) for c in codes], np.float64)


def _step(a):
    """E2M1 grid step at magnitude a (< 6)."""
    return 0.5 if a < 2 else (1.0 if a < 4 else 2.0)


@SETTINGS
@given(y=blocks, s_t=st.sampled_from([1.0, 0.37, 2.0 ** -9, 1 / 1536.0]), rule=rules)
def test_nearest_rounding_within_half_a_step(orc, y, s_t, rule):
    """Round-to-nearest: every scaled value lands within half a grid step of its
    code (or saturates at 6), and the chosen candidate's error is never larger
    than the scale-to-6 error."""
    codes, sb, chose4, (e6, e4) = orc.quantize_block(y, np.float32(s_t), rule)
    d = np.float32(orc.e4m3_value(sb) * np.float32(s_t))
    if d == 0:
        assert np.all((codes & 7) == 0)
        return
    e = np.float32(np.float32(1) / d)
    if not np.isfinite(e):
        return
    z = (y * e).astype(np.float32).astype(np.float64)
    v = _vals(orc, codes)
    for zi, vi in zip(z, v):
        a = abs(zi)
        if a >= 6:
            assert abs(vi) == 6
        else:
            assert abs(a - abs(vi)) <= _step(a) / 2
            assert vi == 0 or np.sign(vi) == np.sign(zi)
    if rule != "none":
        assert (e4 < e6) == chose4


@SETTINGS
@given(y=blocks, rule=rules, sr=st.booleans(), seed=st.integers(0, 2 ** 32))
def test_sign_symmetry(orc, y, rule, sr, seed):
    """Negating the block negates every code and keeps the scale (the decision
    depends only on magnitudes and the element's random word)."""
    words = orc.sr_words(seed, np.arange(16, dtype=np.uint64)) if sr else None
    s_t = np.float32(0.01)
    c1, sb1, ch1, _ = orc.quantize_block(y, s_t, rule, sr, words)
    c2, sb2, ch2, _ = orc.quantize_block(-y, s_t, rule, sr, words)
    assert sb1 == sb2 and ch1 == ch2
    assert np.array_equal(c1 & 7, c2 & 7)
    nz = (c1 & 7) != 0
    assert np.array_equal((c1 ^ c2)[nz] & 8, np.full(nz.sum(), 8, np.uint8))


@SETTINGS
@given(y=hnp.arrays(np.float32, 16, elements=st.floats(-100, 100, allow_nan=False, width=32)),
       k=st.integers(-20, 20), rule=rules, sr=st.booleans())
def test_power_of_two_scale_invariance(orc, y, k, rule, sr):
    """Scaling the data and the tensor scale by the same power of two changes
    nothing in the codes or the block scale: every step of the block arithmetic
    commutes with an exact power-of-two factor."""
    words = orc.sr_words(5, np.arange(16, dtype=np.uint64)) if sr else None
    s_t = np.float32(0.05)
    f = np.float32(2.0 ** k)
    c1, sb1, ch1, _ = orc.quantize_block(y, s_t, rule, sr, words)
    c2, sb2, ch2, _ = orc.quantize_block((y * f).astype(np.float32), np.float32(s_t * f), rule, sr, words)
    assert sb1 == sb2 and ch1 == ch2
    assert np.array_equal(c1, c2)


@SETTINGS
@given(r=hnp.arrays(np.float32, 64, elements=st.floats(0, 1000, allow_nan=False, width=32)))
def test_encoders_are_monotone(orc, r):
    rs = np.sort(r)
    e4 = orc.e4m3_rne_sat(rs)
    assert np.all(np.diff(e4.astype(int)) >= 0)
    z = np.sort(r / 100).astype(np.float32)
    e2 = orc.e2m1_rne(z) & 7
    assert np.all(np.diff(e2.astype(int)) >= 0)


@SETTINGS
@given(x=hnp.arrays(np.float32, (8, 64), elements=st.floats(-50, 50, allow_nan=False, width=32)),
       k=st.integers(-30, 30))
def test_mxfp4_power_of_two_scale_shift(orc, x, k):
    """MXFP4: scaling a tensor by 2^k keeps every code and shifts every scale code
    by k (as long as the scales stay inside the E8M0 range)."""
    a = orc.mxfp4_quantize(x)
    b = orc.mxfp4_quantize((x * np.float32(2.0 ** k)).astype(np.float32))
    keep = (a["scales_row"].astype(int) + k >= 1) & (a["scales_row"].astype(int) + k <= 252) & (a["scales_row"] > 0)
    rows, blk = np.nonzero(keep)
    for r, j in zip(rows, blk):
        assert int(b["scales_row"][r, j]) == int(a["scales_row"][r, j]) + k
        assert np.array_equal(b["codes_row"][r, 16 * j:16 * j + 16], a["codes_row"][r, 16 * j:16 * j + 16])


@SETTINGS
@given(perm_seed=st.integers(0, 1000))
def test_rows_are_independent(orc, wl, perm_seed):
    """Without stochastic rounding (whose words depend on the position) the row
    copy of a row-permuted tensor is the row-permuted row copy."""
    x = wl.generate(2, 32, 64, seed=3)
    perm = np.random.default_rng(perm_seed).permutation(32)
    cfg = orc.make_config(rule="mae", cap=256.0)
    a = orc.amax(x)
    q1 = orc.quantize(x, cfg, a)
    q2 = orc.quantize(np.ascontiguousarray(x[perm]), cfg, a)
    assert np.array_equal(q1["codes_row"][perm], q2["codes_row"])
    assert np.array_equal(q1["scales_row"][perm], q2["scales_row"])
