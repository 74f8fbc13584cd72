"""Independent pins of the oracle where stochastic rounding meets Four Over Six
and the element index.

"Pretraining Large Language Models with NVFP4", section 2d: a value between
two grid points rounds up with probability equal to its fractional distance.
"Technical summary: Four Over Six (4/6)", "Adaptive block scaling algorithm":
quantize each block with both scales, measure each candidate's error against
the original values, keep the smaller.  The reading pinned here: each element
draws one Philox word keyed by its index (row_offset + r) * cols + c in the
input tensor, shared by the row copy, the column copy and both candidates;
the scale-to-6 candidate decides with bits 31..10 of the word, the scale-to-4
candidate with bits 30..9, and each candidate's error is taken on its own
stochastically rounded codes.

Everything on the reference side of these tests is written here from those
statements in float64 (exact quotients, exhaustive nearest-point searches); it
shares no arithmetic with the oracle.  The only oracle routines used as inputs
are separately pinned ones: the Philox word of an index (against torch's
Philox engine) and the 16-point transform (against scipy's Hadamard matrix).

The last test plants mistakes in a copy of the oracle's C source (on the CPU)
and checks that each of these pins fails on it.
"""
import numpy as np
import pytest

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E4M3 = np.array([(c & 7) * 2.0 ** -9 if c < 8 else (8 + (c & 7)) * 2.0 ** ((c >> 3) - 10) for c in range(127)])
E4M3_MID = (E4M3[:-1] + E4M3[1:]) / 2
TWO22 = float(1 << 22)


def _bf16_to_f32(u16):
    return (u16.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------- naive reference ----

def _nearest_e4m3(r):
    """Nearest finite E4M3 value to r >= 0 (ties to the even code), saturating at 448."""
    r = np.minimum(r, 448.0)
    d = np.abs(E4M3[None, :] - r[:, None])
    cand = d == d.min(axis=1, keepdims=True)
    codes = np.arange(127)
    even = np.where(cand & (codes % 2 == 0), codes, 1000).min(axis=1)
    first = np.argmax(cand, axis=1)
    return np.where(even < 1000, even, first)


def _sr_round(a, u):
    """Stochastic E2M1 rounding of magnitudes a >= 0 with 22-bit thresholds u:
    between lo <= a < hi, up iff u + floor(f * 2^22) >= 2^22, f = (a - lo) / (hi - lo);
    a >= 6 gives 6.  Returns (grid index, distance of f * 2^22 to the decision edge)."""
    lo = np.clip(np.searchsorted(GRID, a, side="right") - 1, 0, 7)
    top = lo >= 7
    lo_c = np.minimum(lo, 6)
    f = (a - GRID[lo_c]) / (GRID[lo_c + 1] - GRID[lo_c])
    F = np.floor(f * TWO22)
    up = (u + F) >= TWO22
    k = np.where(top, 7, lo_c + up)
    edge = np.where(top, np.inf, np.abs(f * TWO22 - (TWO22 - u)))
    # distance to a grid point (where lo itself changes), relative to the step
    step = GRID[lo_c + 1] - GRID[lo_c]
    near_grid = np.minimum(np.abs(a - GRID[lo_c]), np.abs(GRID[lo_c + 1] - a)) / step
    near_grid = np.where(top, np.abs(a - 6.0) / 2.0, near_grid)
    return k, edge, near_grid


def naive_blocks(Y, s_t, rule, words):
    """Both 4/6 candidates of every block (rows of Y, float64 values of the
    quantized tensor) with stochastic rounding, and the choice; plus flags for
    blocks whose result a binary32 implementation may legitimately decide
    differently (a value within a few units of 2^-24 of a decision edge)."""
    Y = np.asarray(Y, np.float64)
    nb, n = Y.shape
    m = np.abs(Y).max(axis=1)
    sign = np.signbit(Y).astype(np.uint8) << 3
    out = {}
    for T in (6.0, 4.0):
        den = T * float(s_t)
        r = np.where((m > 0) & (den > 0), m / den if den > 0 else 0.0, 0.0)
        sb = _nearest_e4m3(r)
        amb_r = np.any(np.abs(r[:, None] - E4M3_MID[None, :]) <= 2.0 ** -20 * np.maximum(r[:, None], 2.0 ** -9),
                       axis=1) | (np.abs(r - 448.0) <= 2.0 ** -20 * 448.0)
        d = E4M3[sb] * float(s_t)
        with np.errstate(divide="ignore", invalid="ignore"):
            z = np.where(d[:, None] > 0, Y / d[:, None], 0.0)
        a = np.abs(z)
        if T == 6.0:
            u = (words >> np.uint32(10)).astype(np.float64)
        else:
            u = ((words << np.uint32(1)) >> np.uint32(10)).astype(np.float64)
        k, edge, near_grid = _sr_round(a, u)
        amb_el = (edge <= 4.0) | (near_grid <= 2.0 ** -20 * np.maximum(a, 1.0) / 0.5)
        xh = np.where(sign, -1.0, 1.0) * GRID[k] * d[:, None]
        eps = Y - xh
        if rule == "mse":
            E = np.sum(eps * eps, axis=1)
        elif rule == "mae":
            E = np.sum(np.abs(eps), axis=1)
        else:
            E = np.max(np.abs(eps), axis=1)
        out[T] = dict(sb=sb, codes=(sign | k.astype(np.uint8)), E=E, amb_r=amb_r, amb_el=amb_el)
    pick4 = out[4.0]["E"] < out[6.0]["E"]
    # binary32 error sums of up to 256 terms sit within a few 2^-20 of the exact ones
    slack = 2.0 ** -20 * n * (m * m if rule == "mse" else m)
    close = np.abs(out[4.0]["E"] - out[6.0]["E"]) <= 1e-5 * (out[4.0]["E"] + out[6.0]["E"]) + slack
    return out, pick4, close


def sr_four_over_six_disagreements(picks, scales, codes, Y, s_t, rule, words):
    """Blocks where the oracle's (pick, scale, codes) differ from the naive
    reference without a flagged reason.  codes: (nb, n) uint8, one per element."""
    ref, pick4, close = naive_blocks(Y, s_t, rule, words)
    bad = []
    for b in range(Y.shape[0]):
        T = 4.0 if pick4[b] else 6.0
        same = (bool(picks[b]) == bool(pick4[b]) and scales[b] == ref[T]["sb"][b]
                and np.array_equal(codes[b], ref[T]["codes"][b]))
        if same:
            continue
        explained = close[b] or any(ref[t]["amb_r"][b] for t in (6.0, 4.0))
        if not explained and bool(picks[b]) == bool(pick4[b]) and scales[b] == ref[T]["sb"][b]:
            diff = codes[b] != ref[T]["codes"][b]
            explained = bool(np.all(ref[T]["amb_el"][b][diff]))
        if not explained and bool(picks[b]) != bool(pick4[b]):
            explained = any(np.any(ref[t]["amb_el"][b]) for t in (6.0, 4.0))
        if not explained:
            bad.append(b)
    return bad, int(np.count_nonzero(pick4))


def _unpack_rows(packed, rows, cols):
    return np.stack([packed & 15, packed >> 4], axis=-1).reshape(rows, cols)


# -------------------------------------------- tensor cases for the pins ----

SEED = {4: 1234, 5: 7, 3: 5}


def case_blocks(orc, wl, kind, copy, rule, rows, cols, row_offset=0, data_seed=4):
    """Quantize a band of workload `kind` with the oracle (stochastic rounding,
    4/6 `rule`, cap 256) and return the per-block inputs for the naive check:
    (picks, scales, codes, Y, s_t, words)."""
    raw = wl.generate(kind, rows, cols, seed=data_seed)
    x = _bf16_to_f32(raw)
    seed = SEED[kind]
    rht = kind == 4
    mask = orc.rht_mask_from_seed(1234) if rht else 0
    block = "2d" if copy == "2d" else "1d"
    A = orc.amax(x, rht=rht, mask=mask)
    cfg = orc.make_config(block=block, emit_row=copy in ("row", "2d"), emit_col=copy == "col", rht=rht,
                          rht_mask=mask, sr=True, sr_seed=seed, row_offset=row_offset, rule=rule, cap=256.0)
    out = orc.quantize(x, cfg, A, picks=True)
    s_t = out["tensor_scale"]
    r_idx = (row_offset + np.arange(rows, dtype=np.uint64))[:, None] * np.uint64(cols)
    idx = r_idx + np.arange(cols, dtype=np.uint64)[None, :]          # element index of (r, c)
    W = orc.sr_words(seed, idx).reshape(rows, cols)
    if copy == "row":
        Y = x.reshape(rows, cols // 16, 16).astype(np.float64)
        if rht:
            Y = np.stack([orc.rht16(b, mask) for b in x.reshape(-1, 16)]).reshape(rows, cols // 16, 16)
        Y = Y.reshape(-1, 16)
        words = W.reshape(-1, 16)
        codes = _unpack_rows(out["codes_row"], rows, cols).reshape(-1, 16)
        return out["pick_row"].reshape(-1), out["scales_row"].reshape(-1), codes, Y, s_t, words
    if copy == "col":
        # column c, rows 16i .. 16i+15; the copy is stored as the transpose
        Y = x.T.reshape(cols, rows // 16, 16).reshape(-1, 16).astype(np.float64)
        words = W.T.reshape(-1, 16)
        codes = _unpack_rows(out["codes_col"], cols, rows).reshape(-1, 16)
        return out["pick_col"].reshape(-1), out["scales_col"].reshape(-1), codes, Y, s_t, words
    # 16x16 tiles, elements in row-major order inside the tile
    def tiles(a):
        return a.reshape(rows // 16, 16, cols // 16, 16).transpose(0, 2, 1, 3).reshape(-1, 256)
    Y = tiles(x.astype(np.float64))
    words = tiles(W)
    codes = tiles(_unpack_rows(out["codes_row"], rows, cols))
    return out["pick_row"].reshape(-1), out["scales_row"].reshape(-1), codes, Y, s_t, words


CASES = [  # (workload, copy, rows, cols, row offset)
    (4, "row", 32, 5120, 0),                 # gradient: transform + SR + 4/6 (its stated rule is MAE)
    (5, "row", 32, 8192, 0),                 # activation mixture, row copy
    (5, "col", 64, 2048, 0),                 # activation mixture, column copy
    (5, "row", 16, 8192, (1 << 21) + 48),    # element indices above 2^34: counter high word non-zero
    (3, "2d", 64, 1024, 0),                  # weight, 16x16 tiles with SR + 4/6
]


@pytest.mark.parametrize("rule", ["mse", "mae", "maxerr"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"w{c[0]}-{c[1]}-{c[2]}x{c[3]}-off{c[4]}")
def test_sr_four_over_six_matches_naive(orc, wl, case, rule):
    kind, copy, rows, cols, off = case
    picks, scales, codes, Y, s_t, words = case_blocks(orc, wl, kind, copy, rule, rows, cols, off)
    bad, n4 = sr_four_over_six_disagreements(picks, scales, codes, Y, s_t, rule, words)
    assert not bad, f"{len(bad)} of {len(picks)} blocks differ from the naive reference (first {bad[:5]})"
    # both candidates win somewhere, so both candidates' rounding is exercised
    assert 0 < n4 < len(picks)


# ---------------------------------------------------------- element index ----

def _band_equal(whole, part, r0, r1, M, N, cfg_block, emit_row, emit_col, mx=False):
    """The rows [r0, r1) of `whole` against the band result `part`."""
    ok = True
    if emit_row:
        ok &= np.array_equal(whole["codes_row"][r0:r1], part["codes_row"])
        if cfg_block == "2d":
            ok &= np.array_equal(whole["scales_row"][r0 // 16:r1 // 16], part["scales_row"])
        else:
            ok &= np.array_equal(whole["scales_row"][r0:r1], part["scales_row"])
    if emit_col:
        ok &= np.array_equal(whole["codes_col"][:, r0 // 2:r1 // 2], part["codes_col"])
        blk = 32 if mx else 16
        ok &= np.array_equal(whole["scales_col"][:, r0 // blk:r1 // blk], part["scales_col"])
    return bool(ok)


SHARD_CASES = [  # (name, kind, rows, cols, band edges)
    ("nvfp4-1d-row-col", 5, 96, 320, (0, 32, 48, 96)),
    ("nvfp4-2d", 3, 96, 320, (0, 16, 64, 96)),
    ("nvfp4-rht-row", 4, 40, 320, (0, 7, 23, 40)),
    ("mxfp4-row-col", 5, 128, 320, (0, 32, 96, 128)),
]


def shard_mismatches(orc, wl, name, kind, rows, cols, edges, base=0):
    """Quantize the whole tensor with row_offset = base, and each band [r0, r1)
    with row_offset = base + r0: the bands must reproduce the whole result."""
    x = _bf16_to_f32(wl.generate(kind, rows, cols, seed=8))
    bad = []
    if name.startswith("mxfp4"):
        whole = orc.mxfp4_quantize(x, True, True, True, 99, base)
        for r0, r1 in zip(edges[:-1], edges[1:]):
            part = orc.mxfp4_quantize(x[r0:r1], True, True, True, 99, base + r0)
            if not _band_equal(whole, part, r0, r1, rows, cols, "1d", True, True, mx=True):
                bad.append((r0, r1))
        return bad
    rht = "rht" in name
    block = "2d" if "2d" in name else "1d"
    ecol = not rht
    mask = orc.rht_mask_from_seed(3) if rht else 0
    A = orc.amax(x, rht=rht, mask=mask)
    cfg = lambda off: orc.make_config(block=block, emit_row=True, emit_col=ecol, rht=rht, rht_mask=mask, sr=True,
                                      sr_seed=99, row_offset=off, rule="mae", cap=256.0)
    whole = orc.quantize(x, cfg(base), A)
    for r0, r1 in zip(edges[:-1], edges[1:]):
        part = orc.quantize(x[r0:r1], cfg(base + r0), A)   # the shared tensor amax of the whole tensor
        if not _band_equal(whole, part, r0, r1, rows, cols, block, True, ecol):
            bad.append((r0, r1))
    return bad


@pytest.mark.parametrize("base", [0, (1 << 22) + 16])
@pytest.mark.parametrize("case", SHARD_CASES, ids=lambda c: c[0])
def test_row_bands_with_row_offset_reproduce_the_whole_tensor(orc, wl, case, base):
    """Sharding rows over devices: a band quantized with row_offset = its first
    global row gives the same bytes as the whole tensor (every block is
    independent, the tensor amax is shared, and each element keeps its word)."""
    name, kind, rows, cols, edges = case
    assert shard_mismatches(orc, wl, name, kind, rows, cols, edges, base) == []


def index_mismatches(orc, wl, row_offset, rows=48, cols=96, seed=31):
    """Every block of the row and column copies (NVFP4 1D, SR, 4/6 MAE) against
    orc.quantize_block fed the words of the elements' own indices
    (row_offset + r) * cols + c, and the MXFP4 copies against a naive
    per-element rounding with those words.  Returns a list of what differs."""
    x = _bf16_to_f32(wl.generate(5, rows, cols, seed=seed))
    A = orc.amax(x)
    cfg = orc.make_config(emit_row=True, emit_col=True, sr=True, sr_seed=seed, row_offset=row_offset, rule="mae",
                          cap=256.0)
    out = orc.quantize(x, cfg, A)
    s_t = out["tensor_scale"]
    idx = ((row_offset + np.arange(rows, dtype=np.uint64))[:, None] * np.uint64(cols)
           + np.arange(cols, dtype=np.uint64)[None, :])
    W = orc.sr_words(seed, idx).reshape(rows, cols)
    bad = []
    row_codes = _unpack_rows(out["codes_row"], rows, cols)
    for r in range(rows):
        for j in range(cols // 16):
            c, sb, _, _ = orc.quantize_block(x[r, 16 * j:16 * j + 16], s_t, "mae", True, W[r, 16 * j:16 * j + 16])
            if not (np.array_equal(c, row_codes[r, 16 * j:16 * j + 16]) and sb == out["scales_row"][r, j]):
                bad.append(("row", r, j))
    col_codes = _unpack_rows(out["codes_col"], cols, rows)
    for c_ in range(cols):
        for i in range(rows // 16):
            c, sb, _, _ = orc.quantize_block(x[16 * i:16 * i + 16, c_], s_t, "mae", True, W[16 * i:16 * i + 16, c_])
            if not (np.array_equal(c, col_codes[c_, 16 * i:16 * i + 16]) and sb == out["scales_col"][c_, i]):
                bad.append(("col", c_, i))
    # MXFP4: power-of-two scale from the (separately pinned) scale rule; z = y * 2^-e exactly;
    # each element rounds with its own word (bits 31..10)
    rows_mx = rows - rows % 32
    xm = x[:rows_mx]
    mo = orc.mxfp4_quantize(xm, True, True, True, seed, row_offset)
    Wm = W[:rows_mx]

    def mx_naive(vals, words):
        m = float(np.max(np.abs(vals)))
        sc = orc.mx_scale_code(m)
        z = vals.astype(np.float64) * 2.0 ** (127 - sc)
        k, _, _ = _sr_round(np.abs(z), (words >> np.uint32(10)).astype(np.float64))
        return (np.signbit(vals).astype(np.uint8) << 3) | k.astype(np.uint8), sc
    mrow = _unpack_rows(mo["codes_row"], rows_mx, cols)
    for r in range(rows_mx):
        for j in range(cols // 32):
            c, sc = mx_naive(xm[r, 32 * j:32 * j + 32], Wm[r, 32 * j:32 * j + 32])
            if not (np.array_equal(c, mrow[r, 32 * j:32 * j + 32]) and sc == mo["scales_row"][r, j]):
                bad.append(("mx-row", r, j))
    mcol = _unpack_rows(mo["codes_col"], cols, rows_mx)
    for c_ in range(cols):
        for i in range(rows_mx // 32):
            c, sc = mx_naive(xm[32 * i:32 * i + 32, c_], Wm[32 * i:32 * i + 32, c_])
            if not (np.array_equal(c, mcol[c_, 32 * i:32 * i + 32]) and sc == mo["scales_col"][c_, i]):
                bad.append(("mx-col", c_, i))
    return bad


@pytest.mark.parametrize("row_offset", [0, 5, (1 << 27) + 3])
def test_copies_use_the_element_index_words(orc, wl, row_offset):
    """Both copies (and the MXFP4 copies) of each element round with the word
    of the element's index in the input tensor, (row_offset + r) * cols + c:
    the column copy shares the row copy's word rather than numbering its own
    transposed layout.  row_offset * cols reaches past 2^32 in the last case."""
    assert index_mismatches(orc, wl, row_offset) == []


# ------------------------------------------- planted mistakes are caught ----

MUTANTS = {
    # each: (text in the oracle, replacement, the pin that must catch it)
    "errors-from-nearest-codes": (
        "float xh = orc_e2m1_value(codes[i]) * d;",
        "float xh = orc_e2m1_value(orc_e2m1_rne(y[i] * e)) * d;",
        "sr46"),
    "candidate-words-swapped": (
        "T == 4.0f ? rwords[i] << 1 : rwords[i]",
        "T == 4.0f ? rwords[i] : rwords[i] << 1",
        "sr46"),
    "same-bits-for-both-candidates": (
        "T == 4.0f ? rwords[i] << 1 : rwords[i]",
        "rwords[i]",
        "sr46"),
    "column-index-transposed": (
        "idx[k] = (cfg->row_offset + r) * N + c;",
        "idx[k] = c * M + (cfg->row_offset + r);",
        "index"),
    "row-offset-ignored": (
        "idx[k] = (cfg->row_offset + r) * N + j * 16 + k;",
        "idx[k] = r * N + j * 16 + k;",
        "shard"),
    "row-offset-added-once": (
        "idx[k] = (cfg->row_offset + r) * N + c;",
        "idx[k] = r * N + c + cfg->row_offset;",
        "shard"),
    "mx-column-index-transposed": (
        "idx[k] = (uint64_t)((row_offset + j * 32 + k) * cols + c);",
        "idx[k] = (uint64_t)(c * rows + row_offset + j * 32 + k);",
        "index"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(orc, wl, tmp_path, name):
    old, new, pin = MUTANTS[name]
    src = orc.source()
    assert src.count(old) >= 1, f"mutation site for {name} not found in the oracle source"
    variant = orc.build_variant(src.replace(old, new), str(tmp_path), name.replace("-", "_"))
    with orc.library(variant):
        if pin == "sr46":
            caught = False
            for case in (CASES[0], CASES[1], CASES[4]):
                for rule in ("mae", "mse"):
                    kind, copy, rows, cols, off = case
                    args = case_blocks(orc, wl, kind, copy, rule, rows, cols, off)
                    bad, _ = sr_four_over_six_disagreements(*args[:5], rule, args[5])
                    caught |= len(bad) > 0
            assert caught, f"the 4/6 stochastic-rounding pin misses mutant {name}"
        elif pin == "index":
            assert index_mismatches(orc, wl, 5), f"the element-index pin misses mutant {name}"
        else:
            found = any(shard_mismatches(orc, wl, *case, base=(1 << 22) + 16) for case in SHARD_CASES)
            assert found, f"the sharding pin misses mutant {name}"
