"""Pins of the oracle's Hadamard transform, Philox generator and stochastic
rounding against closed forms, library routines and statistics."""
import ctypes
import json
import os
import subprocess

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "four_over_six_examples.json")


# ---------------------------------------------------------------- RHT ----

def _h_from_oracle(orc):
    cols = []
    for k in range(16):
        e = np.zeros(16, np.float32)
        e[k] = 1.0
        cols.append(4.0 * orc.rht16(e, 0).astype(np.float64))
    return np.stack(cols, axis=1)  # column k = H e_k


def test_rht_is_sylvester_hadamard(orc):
    # Pretraining-with-NVFP4 explainer, section 2b: the transform mixes each block with a Hadamard matrix.
    scipy_linalg = pytest.importorskip("scipy.linalg")
    H = _h_from_oracle(orc)
    assert np.array_equal(H, scipy_linalg.hadamard(16).astype(np.float64))
    assert np.array_equal(H @ H.T, 16.0 * np.eye(16))
    assert set(np.unique(H)) == {-1.0, 1.0}


def test_rht_closed_forms(orc):
    y = orc.rht16(np.ones(16, np.float32), 0)
    assert y[0] == 4.0 and np.all(y[1:] == 0.0)
    e0 = np.zeros(16, np.float32)
    e0[0] = 1.0
    assert np.all(orc.rht16(e0, 0) == 0.25)


def test_rht_sign_mask_and_inverse(orc):
    scipy_linalg = pytest.importorskip("scipy.linalg")
    H = scipy_linalg.hadamard(16).astype(np.float64)
    rng = np.random.default_rng(3)
    for mask in (0x0000, 0xFFFF, 0xA5C3, 0x1234):
        D = np.diag([-1.0 if (mask >> i) & 1 else 1.0 for i in range(16)])
        # dyadic inputs: every intermediate is exact, so the result equals the exact product
        x = rng.integers(-64, 64, 16).astype(np.float32)
        y = orc.rht16(x, mask)
        assert np.array_equal(y.astype(np.float64), H @ D @ x.astype(np.float64) / 4.0)
        # inverse: x = D H y / 4 (H symmetric, H H = 16 I)
        assert np.array_equal(D @ H @ y.astype(np.float64) / 4.0, x.astype(np.float64))
        # random reals: within a few ulp of the exact product; Parseval within fp32 error
        x = rng.standard_normal(16).astype(np.float32)
        y = orc.rht16(x, mask).astype(np.float64)
        ref = H @ D @ x.astype(np.float64) / 4.0
        assert np.max(np.abs(y - ref)) <= 8 * np.finfo(np.float32).eps * np.max(np.abs(x)) * 4
        assert abs(np.sum(y * y) - np.sum(x.astype(np.float64) ** 2)) <= 64 * 2.0 ** -23 * np.sum(x.astype(np.float64) ** 2)


# ------------------------------------------------------------- Philox ----

@pytest.fixture(scope="module")
def torch_philox(tmp_path_factory):
    """torch's header-only Philox4_32 engine, an independent implementation of the published generator."""
    torch = pytest.importorskip("torch")
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    hdr = os.path.join(inc, "ATen", "core", "PhiloxRNGEngine.h")
    if not os.path.exists(hdr):
        pytest.skip("torch Philox header not available")
    d = tmp_path_factory.mktemp("philox")
    src = d / "ref.cpp"
    src.write_text(
        "#include <ATen/core/PhiloxRNGEngine.h>\n"
        "extern \"C\" void ref_stream(uint64_t seed, uint64_t subseq, uint64_t offset, int n, uint32_t* out) {\n"
        "  at::Philox4_32 e(seed, subseq, offset);\n"
        "  for (int i = 0; i < n; ++i) out[i] = e();\n"
        "}\n")
    so = d / "ref.so"
    subprocess.run(["g++", "-std=c++17", "-O1", "-fPIC", "-shared", "-I", inc, "-o", str(so), str(src)], check=True)
    L = ctypes.CDLL(str(so))
    L.ref_stream.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p]
    L.ref_stream.restype = None

    def stream(seed, subseq, offset, n):
        out = np.empty(n, np.uint32)
        L.ref_stream(seed, subseq, offset, n, out.ctypes.data_as(ctypes.c_void_p))
        return out
    return stream


def test_philox_matches_library(orc, torch_philox):
    rng = np.random.default_rng(5)
    for seed in (0, 1, 7, 1234, 0xFFFFFFFF, 0x123456789ABCDEF0):
        for q in list(rng.integers(0, 2 ** 40, 20)) + [0, 1, 2 ** 32 - 1, 2 ** 32]:
            q = int(q)
            ref = torch_philox(seed, 0, q, 4)  # counter (q lo, q hi, 0, 0), key (seed lo, seed hi)
            ctr = np.array([[q & 0xFFFFFFFF, q >> 32, 0, 0]], np.uint32)
            key = np.array([[seed & 0xFFFFFFFF, seed >> 32]], np.uint32)
            assert np.array_equal(orc.philox(ctr, key)[0], ref)
            idx = np.arange(4 * q, 4 * q + 4, dtype=np.uint64)
            assert np.array_equal(orc.sr_words(seed, idx), ref)
    # the Hadamard sign stream uses counter word 3 = 1 (subsequence 2^32 in torch's terms)
    for seed in (0, 1234, 99):
        assert orc.rht_mask_from_seed(seed) == int(torch_philox(seed, 1 << 32, 0, 1)[0]) & 0xFFFF


def test_philox_uniformity(orc):
    w = orc.sr_words(1234, np.arange(1 << 20, dtype=np.uint64))
    b = w.view(np.uint8)
    counts = np.bincount(b, minlength=256)
    exp = b.size / 256
    chi2 = np.sum((counts - exp) ** 2 / exp)
    assert chi2 < 255 + 6 * np.sqrt(2 * 255)  # ~6 sigma of a chi-square with 255 dof
    u = (w >> 10).astype(np.float64) / 2 ** 22
    assert abs(u.mean() - 0.5) < 6 * np.sqrt(1 / 12 / u.size)


# ----------------------------------------------------- stochastic rounding

def test_sr_page_example_60_40(orc):
    g = json.load(open(GOLDEN))["sr_example"]
    n = g["draws"]
    z = np.full(n, g["z"], np.float32)
    w = orc.sr_words(1234, np.arange(n, dtype=np.uint64))
    codes = orc.e2m1_sr(z, w)
    vals = np.array([orc.e2m1_value(int(c)) for c in range(16)])[codes]
    assert set(np.unique(vals)) == {g["lo"], g["hi"]}
    frac_up = np.mean(vals == g["hi"])
    sigma = np.sqrt(g["p_up"] * (1 - g["p_up"]) / n)
    assert abs(frac_up - g["p_up"]) < 5 * sigma
    assert abs(vals.mean() - float(np.float32(g["z"]))) < 5 * sigma * (g["hi"] - g["lo"])


def test_sr_unbiased_over_range(orc):
    rng = np.random.default_rng(11)
    n = 1_000_000
    a = rng.uniform(-6, 6, n).astype(np.float32)
    w = orc.sr_words(99, np.arange(n, dtype=np.uint64))
    v = np.array([orc.e2m1_value(int(c)) for c in range(16)])[orc.e2m1_sr(a, w)]
    err = v - a.astype(np.float64)
    # per-element variance <= (gap/2)^2 with gap <= 2
    assert abs(err.mean()) < 5 * 1.0 / np.sqrt(n)


def test_sr_special_cases(orc):
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)
    w = orc.sr_words(5, np.arange(4096, dtype=np.uint64))
    for k, gv in enumerate(grid):  # grid points never move
        assert np.all(orc.e2m1_sr(np.full(4096, gv, np.float32), w) == k)
        assert np.all(orc.e2m1_sr(np.full(4096, -gv, np.float32), w) == 8 | k)
    big = np.array([6.0, 6.5, 7.9, 1e9, np.inf], np.float32)
    assert np.all(orc.e2m1_sr(big, w[:5]) == 7)
    # decision threshold: z = 2 + 2^-21 -> f = 2^-21, F = 2: up iff (w >> 10) >= 2^22 - 2
    z = np.float32(2.0 + 2.0 ** -21)
    for wd, up in ((((1 << 22) - 2) << 10, 1), ((((1 << 22) - 2) << 10) - 1, 0), (0xFFFFFFFF, 1), (0, 0)):
        assert orc.e2m1_sr(np.array([z]), np.array([wd], np.uint32))[0] == (4 + up)
