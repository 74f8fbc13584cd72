"""The bound behind the strip kernel's 4/6 error estimates, checked on the CPU.

Where the kernel decides a 4/6 block without the exact errors, it estimates
each candidate's error E_T from residuals in the scaled domain,
r = fl(fl(y * e) - v), as d * sum|r| (MAE), d * (d * sum r^2) (MSE) or
d * max|r| (MAXERR), and trusts the estimates only when they differ by more
than the sum of per-candidate bounds
    MAE:    2^-18 a + 2^-21 n m      MSE: 2^-16 a + 2^-24 n m^2
    MAXERR: 2^-19 a + 2^-21 m
(a the estimate, n the values in the block, m the block max), and only where
the tensor scale S_t has fl(6 S_t) within [2^-48, 2^48] and the scale-to-6
factor d is non-zero (other blocks take the exact errors).  Here the
estimates are formed in binary32 with the kernel's summation orders, the exact
errors come from the oracle, and every block must satisfy
|estimate - E_T| <= bound / 2, i.e. the bounds hold with a factor two to
spare, over ordinary, outlier, sparse, constant and extreme-magnitude blocks.
"""
import numpy as np
import pytest

import oracle

F = np.float32
RULES = ("mse", "mae", "maxerr")


def candidate(y, s_t, T, rule, sr, words):
    """Scale d, reciprocal e, scaled values z and E2M1 values v of one candidate."""
    m = F(np.max(np.abs(y)))
    r = F(m / F(F(T) * s_t))
    sb = int(oracle.e4m3_rne_sat(np.array([r], F))[0])
    d = F(F(oracle.e4m3_value(sb)) * s_t)
    e = F(0.0) if d == 0 else F(F(1.0) / d)
    if not np.isfinite(e):
        e = F(0.0)
    z = (y * e).astype(F)
    if sr:
        w = words if T == 6 else ((words.astype(np.uint64) << 1) & 0xFFFFFFFF).astype(np.uint32)
        codes = oracle.e2m1_sr(z, w)
    else:
        codes = oracle.e2m1_rne(z)
    v = np.array([oracle.e2m1_value(int(c)) for c in codes], F)
    return d, z, v


def acc(rule, a, r):
    if rule == "mse":
        return F(np.float64(r) * np.float64(r) + np.float64(a))
    if rule == "maxerr":
        return F(max(a, abs(r)))
    return F(a + abs(r))


def first(rule, r):
    return F(r * r) if rule == "mse" else F(abs(r))


def join(rule, a, b):
    return F(max(a, b)) if rule == "maxerr" else F(a + b)


def lane_sum(rule, res, sr):
    """One lane's 16 residuals in the kernel's order: four chains, then (0+1)+(2+3)."""
    if sr:  # chain c: elements 8 (c >> 1) + (c & 1) + 2 j
        chains = [[8 * (c >> 1) + (c & 1) + 2 * j for j in range(4)] for c in range(4)]
    else:  # chain c: bytes c & 1 (+2) of the low (c even) or high register
        chains = [[8 * (c & 1) + 4 * j + 2 * (c >> 1) + h for j in range(2) for h in range(2)] for c in range(4)]
    a = []
    for ch in chains:
        s = first(rule, res[ch[0]])
        for k in ch[1:]:
            s = acc(rule, s, res[k])
        a.append(s)
    return join(rule, join(rule, a[0], a[1]), join(rule, a[2], a[3]))


def row_sum(rule, parts):
    """Across the 16 lanes of a tile: the pairwise tree of the DPP reduction."""
    p = list(parts)
    while len(p) > 1:
        p = [join(rule, p[2 * i], p[2 * i + 1]) for i in range(len(p) // 2)]
    return p[0]


def estimate(rule, y, s_t, T, sr, words):
    d, z, v = candidate(y, s_t, T, rule, sr, words)
    res = (z - v).astype(F)
    if y.size == 16:
        s = lane_sum(rule, res, sr)
    else:
        s = row_sum(rule, [lane_sum(rule, res[16 * i:16 * i + 16], sr) for i in range(16)])
    return F(d * F(d * s)) if rule == "mse" else F(d * s)


def bound(rule, a, n, m):
    a, m = float(a), float(m)
    if rule == "mae":
        return 2.0 ** -18 * a + 2.0 ** -21 * n * m
    if rule == "maxerr":
        return 2.0 ** -19 * a + 2.0 ** -21 * m
    return 2.0 ** -16 * a + 2.0 ** -24 * n * m * m


def blocks(n, count, rng):
    """Blocks of n values from several families, with their tensor amax."""
    out = []
    for i in range(count):
        fam = i % 6
        scale = F(10.0 ** rng.uniform(-12, 12))
        if fam == 0:
            y = rng.standard_normal(n)
        elif fam == 1:  # one large outlier
            y = rng.standard_normal(n)
            y[rng.integers(n)] *= 40.0
        elif fam == 2:  # sparse
            y = rng.standard_normal(n) * (rng.random(n) < 0.2)
            y[rng.integers(n)] = 1.0 + rng.random()
        elif fam == 3:  # constant
            y = np.full(n, 1.0 + rng.random())
        elif fam == 4:  # heavy-tailed
            y = rng.standard_t(3, n)
        else:  # uniform, both signs
            y = rng.uniform(-1, 1, n)
        y = (y * scale).astype(F)
        amax = F(np.max(np.abs(y)) * F(1.0 + 30.0 * rng.random() ** 3))
        out.append((y, amax))
    return out


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("n", [16, 256])
def test_estimates_within_half_the_bound(rule, sr, n):
    rng = np.random.default_rng({16: 1, 256: 2}[n] * 10 + RULES.index(rule) + 5 * sr)
    worst = 0.0
    checked = 0
    for y, amax in blocks(n, 600 if n == 16 else 90, rng):
        cap = 256.0 if rng.random() < 0.5 else 448.0
        s_t = F(oracle.tensor_scale(float(amax), cap))
        words = oracle.sr_words(int(rng.integers(1 << 30)), np.arange(n, dtype=np.uint64) + 4096)
        _, _, _, (e6, e4) = oracle.quantize_block(y, float(s_t), rule, sr=sr, words=words)
        m = F(np.max(np.abs(y)))
        den6 = F(F(6.0) * s_t)
        if not (2.0 ** -48 <= den6 <= 2.0 ** 48) or candidate(y, s_t, 6, rule, sr, words)[0] == 0:
            continue  # the kernel forms the exact errors for these blocks
        for T, E in ((6, e6), (4, e4)):
            a = estimate(rule, y, s_t, T, sr, words)
            if not (np.isfinite(a) and np.isfinite(E)):
                continue
            b = bound(rule, a, n, m)
            ratio = abs(float(a) - float(E)) / b if b > 0 else 0.0
            worst = max(worst, ratio)
            checked += 1
            assert ratio <= 0.5, (rule, sr, n, T, float(a), float(E), b)
    assert checked > 100
    print(f"worst |estimate - E| / bound = {worst:.3g} over {checked} candidates")
