"""Pins of the oracle's number formats against facts the pages and the
mathematics fix (not against the oracle itself)."""
import numpy as np
import pytest

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _f32_from_bits(b):
    return np.asarray(b, dtype=np.uint32).view(np.float32)


def brute_e2m1(z):
    """Nearest E2M1 magnitude by exhaustive distance; an exact tie goes to the even grid index."""
    z = np.asarray(z, np.float32)
    a = np.abs(z.astype(np.float64))
    d = np.abs(a[:, None] - GRID[None, :])
    dmin = d.min(axis=1, keepdims=True)
    pref = np.where(d == dmin, (np.arange(8) % 2)[None, :], 2)
    k = np.argmin(pref, axis=1)  # first minimum: the even index when two points tie
    sign = (z.view(np.uint32) >> 31).astype(np.uint8)
    return (sign << 3) | k.astype(np.uint8)


def test_e2m1_grid_and_steps_from_page(orc):
    # Four Over Six summary, "Problem statement": steps 0.5 on [0,2], 1 on [2,4], 2 on [4,6]; max 6.
    vals = [orc.e2m1_value(k) for k in range(8)]
    assert vals == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    steps = np.diff(vals)
    assert list(steps[:4]) == [0.5] * 4 and list(steps[4:6]) == [1.0, 1.0] and steps[6] == 2.0
    assert [orc.e2m1_value(8 + k) for k in range(8)] == [-v for v in vals]


def test_four_is_two_thirds_of_six(orc):
    # same section: with the block max at 6, the representable 4 is 66.6% (= 2/3) of it
    assert orc.e2m1_value(6) / orc.e2m1_value(7) == pytest.approx(2.0 / 3.0, abs=0)
    assert int(100 * orc.e2m1_value(6) / orc.e2m1_value(7) * 10) == 666


def test_e2m1_rne_exact_grid_points_and_ties(orc):
    for k, g in enumerate(GRID):
        assert orc.e2m1_rne(np.float32(g))[0] == k
        assert orc.e2m1_rne(np.float32(-g))[0] == 8 | k
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for t, k in ties.items():
        assert orc.e2m1_rne(np.float32(t))[0] == k, t
    # saturation and signed zero
    assert list(orc.e2m1_rne(np.array([6.5, 7.0, 1e30, np.inf], np.float32))) == [7] * 4
    assert orc.e2m1_rne(np.float32(-0.0))[0] == 8
    assert orc.e2m1_rne(np.float32(-1e-30))[0] == 8


def test_e2m1_rne_brute_force_sweep(orc):
    # every 97th fp32 pattern in [0, 8) plus all midpoints and their neighbours, both signs
    pats = np.arange(0, 0x41000000, 97, dtype=np.uint64).astype(np.uint32)
    mids = (GRID[:-1] + GRID[1:]) / 2
    mb = np.array(mids, np.float32).view(np.uint32)
    near = np.concatenate([mb - 1, mb, mb + 1, np.array(GRID, np.float32).view(np.uint32)])
    pats = np.concatenate([pats, near.astype(np.uint32)])
    z = _f32_from_bits(pats)
    z = np.concatenate([z, -z])
    for i in range(0, z.size, 1 << 21):
        zz = z[i:i + (1 << 21)]
        np.testing.assert_array_equal(orc.e2m1_rne(zz), brute_e2m1(zz))


def _e4m3_table():
    vals = []
    for c in range(0x7F):  # 0x7F is NaN in E4M3FN
        e, m = c >> 3, c & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10))
    return np.array(vals)


def brute_e4m3(r):
    """Nearest of the 127 finite non-negative E4M3 values, ties to even code, saturating at 448."""
    t = _e4m3_table()
    r = np.minimum(np.asarray(r, np.float64), 448.0)
    out = np.empty(r.size, np.uint8)
    for i in range(0, r.size, 50000):
        rr = r[i:i + 50000]
        d = np.abs(rr[:, None] - t[None, :])
        dmin = d.min(axis=1, keepdims=True)
        pref = np.where(d == dmin, (np.arange(t.size) % 2)[None, :], 2)
        out[i:i + 50000] = np.argmin(pref, axis=1)
    return out


def test_e4m3_decode_format_facts(orc):
    assert orc.e4m3_value(0x7E) == 448.0          # largest finite E4M3
    assert orc.e4m3_value(0x08) == 2.0 ** -6      # smallest normal
    assert orc.e4m3_value(0x01) == 2.0 ** -9      # smallest subnormal
    assert orc.e4m3_value(0x38) == 1.0            # bias 7
    assert orc.e4m3_value(0x50) == 8.0 and orc.e4m3_value(0x54) == 12.0


def test_e4m3_encode_brute_force(orc):
    t = _e4m3_table().astype(np.float32)
    mids = ((t[:-1].astype(np.float64) + t[1:]) / 2).astype(np.float32)
    tb, mb = t.view(np.uint32), mids.view(np.uint32)
    pts = np.concatenate([tb, tb + 1, tb[1:] - 1, mb, mb + 1, mb - 1]).view(np.float32)
    rng = np.random.default_rng(1)
    rnd = rng.uniform(0, 470, 400000).astype(np.float32)
    tiny = rng.uniform(0, 2.0 ** -5, 100000).astype(np.float32)
    r = np.concatenate([pts, rnd, tiny, np.float32([0.0, 448.0, 449.0, 464.0, 465.0, 1e20])])
    r = r[r >= 0]
    np.testing.assert_array_equal(orc.e4m3_rne_sat(r), brute_e4m3(r))
    assert orc.e4m3_rne_sat(np.float32([np.inf]))[0] == 0x7E


def test_e4m3_encode_matches_torch_cast(orc):
    torch = pytest.importorskip("torch")
    # torch's float8_e4m3fn cast rounds to nearest even; it does not saturate above 464, so stay below.
    pats = np.arange(0, int(np.float32(448.0).view(np.uint32)) + 1, 13, dtype=np.uint64).astype(np.uint32)
    r = pats.view(np.float32)
    ref = torch.from_numpy(r.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(orc.e4m3_rne_sat(r), ref)
