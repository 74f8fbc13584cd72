"""Pins of the oracle's FP4 GEMM (the consumer of the quantized copies): numpy
float64 products of operands decoded through the pinned format functions, and
closed forms."""
import numpy as np
import pytest


def _decode_codes(orc, codes):
    vals = np.array([orc.e2m1_value(c) for c in range(16)], np.float64)
    c = np.asarray(codes)
    lo, hi = vals[c & 15], vals[c >> 4]
    out = np.empty(c.shape[:-1] + (2 * c.shape[-1],))
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def _nv_operand(orc, q, rows, K, two_d):
    dec = np.array([orc.e4m3_value(v) for v in range(256)], np.float64)
    s = dec[q["scales_row"]]
    s = np.repeat(np.repeat(s, 16, axis=0), 16, axis=1) if two_d else np.repeat(s, 16, axis=1)
    return _decode_codes(orc, q["codes_row"]) * s * float(q["tensor_scale"])


def _mx_operand(orc, q):
    e = np.array([orc.e8m0_value(v) for v in range(255)] + [np.nan], np.float64)
    return _decode_codes(orc, q["codes_row"]) * np.repeat(e[q["scales_row"]], 32, axis=1)


@pytest.mark.parametrize("b2d", [False, True])
def test_nvfp4_gemm_matches_float64_product(orc, wl, b2d):
    M, N, K = 48, 32, 160
    xa = wl.generate(5, M, K, seed=1)
    xb = wl.generate(3, N, K, seed=2)
    qa = orc.quantize(xa, orc.make_config(rule="mae", cap=256.0), orc.amax(xa))
    qb = orc.quantize(xb, orc.make_config(block="2d" if b2d else "1d"), orc.amax(xb))
    c, cabs = orc.gemm_fp4(False, qa["codes_row"], qa["scales_row"], qb["codes_row"], qb["scales_row"], M, N, K,
                           qa["tensor_scale"], qb["tensor_scale"], False, b2d)
    A = _nv_operand(orc, qa, M, K, False)
    B = _nv_operand(orc, qb, N, K, b2d)
    ref = A @ B.T
    bound = (K * 2.0 ** -52) * (np.abs(A) @ np.abs(B).T) + np.abs(ref) * 2.0 ** -24
    assert np.all(np.abs(c.astype(np.float64) - ref) <= bound)
    assert np.allclose(cabs, np.abs(A) @ np.abs(B).T, rtol=1e-12, atol=0)
    # the dequantized product approximates the float product of the inputs
    xf = (xa.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xw = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rel = np.linalg.norm(c - xf @ xw.T) / np.linalg.norm(xf @ xw.T)
    assert rel < 0.3  # 4-bit operands; the weight carries x30 outliers


def test_mxfp4_gemm_matches_float64_product(orc, wl):
    M, N, K = 40, 24, 256
    xa = wl.generate(1, M, K, seed=3)
    xb = wl.generate(2, N, K, seed=4)
    qa = orc.mxfp4_quantize(xa)
    qb = orc.mxfp4_quantize(xb)
    c, cabs = orc.gemm_fp4(True, qa["codes_row"], qa["scales_row"], qb["codes_row"], qb["scales_row"], M, N, K)
    A, B = _mx_operand(orc, qa), _mx_operand(orc, qb)
    ref = A @ B.T
    bound = (K * 2.0 ** -52) * (np.abs(A) @ np.abs(B).T) + np.abs(ref) * 2.0 ** -24
    assert np.all(np.abs(c.astype(np.float64) - ref) <= bound)


def test_gemm_closed_forms(orc):
    K = 64
    ones = np.full((3, K // 2), 0x22, np.uint8)     # every element 1.0
    mx_unit = np.full((3, K // 32), 127, np.uint8)  # 2^0
    c, _ = orc.gemm_fp4(True, ones, mx_unit, ones, mx_unit, 3, 3, K)
    assert np.all(c == K)
    # a one-hot A row picks one column of B: C[0][n] = B[n][5] * scale
    a = np.zeros((1, K // 2), np.uint8)
    a[0, 2] = 0x70                                   # element 5 = 6.0
    sa = np.full((1, K // 32), 128, np.uint8)        # 2^1
    rng = np.random.default_rng(0)
    b = rng.integers(0, 256, (4, K // 2), dtype=np.uint8)
    sb = np.full((4, K // 32), 126, np.uint8)        # 2^-1
    c, _ = orc.gemm_fp4(True, a, sa, b, sb, 1, 4, K)
    vals = [orc.e2m1_value(int(v)) for v in range(16)]
    assert np.array_equal(c[0], np.array([6.0 * 2 * vals[int(b[n, 2]) >> 4] * 0.5 for n in range(4)], np.float32))
    # NVFP4: tensor scales multiply the product; E4M3 code 0x38 = 1.0
    s1 = np.full((3, K // 16), 0x38, np.uint8)
    c, _ = orc.gemm_fp4(False, ones, s1, ones, s1, 3, 3, K, 0.5, 0.25)
    assert np.all(c == K * 0.125)


def test_gemm_rejects_bad_shapes(orc):
    z = np.zeros((16, 24), np.uint8)
    with pytest.raises(ValueError):
        orc.gemm_fp4(True, z, z, z, z, 16, 16, 48)
    with pytest.raises(ValueError):
        orc.gemm_fp4(False, z, z, z, z, 8, 16, 48, 1.0, 1.0, True, False)
