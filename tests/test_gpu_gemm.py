"""GPU parity of the FP4 GEMM consumer (nvfp4_gemm, nvfp4_mxfp4_gemm) against
the oracle's exact-product GEMM.

The matrix cores accumulate in fp32: each instruction adds its exact products
to the running sum with at most one unit of 2^-24 of (|running sum| +
sum |products|) of error (measured on the device for single instructions), so
after K / k_i instructions (k_i = 64 values per MXFP4 instruction, 16 per fp16
instruction) |C - exact| <= 2 (K / k_i) 2^-24 sum |A B|.  The oracle itself is
within K 2^-53 sum |A B| + 2^-24 |C| of the exact value, and NVFP4 adds one
rounding for the tensor-scale multiply; the tests allow the sum of these."""
import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
nv = pytest.importorskip("nvfp4_block_quantization_amd")

pytestmark = pytest.mark.gpu


def say(msg: str) -> None:
    print(f"[gpu-gemm] {msg}", flush=True)


def g(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def tolerance(cabs, ref, K, k_i):
    return (2 * (K // k_i) + 2) * 2.0 ** -24 * cabs + 2.0 ** -23 * np.abs(ref.astype(np.float64)) + 1e-38


def check(got, ref, cabs, K, k_i, tag):
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    tol = tolerance(cabs, ref, K, k_i)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{tag}: {bad.sum()} outputs off, first {i.tolist()}: got {got[tuple(i)]} "
                             f"ref {ref[tuple(i)]} tol {tol[tuple(i)]}")
    say(f"{tag}: max err / tol = {float((err / tol).max()):.3g}")


def rand_nv(rng, rows, K, two_d=False):
    codes = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    srows = rows // 16 if two_d else rows
    scales = rng.integers(0x20, 0x60, (srows, K // 16), dtype=np.uint8)
    return codes, scales


def rand_mx(rng, rows, K):
    return rng.integers(0, 256, (rows, K // 2), dtype=np.uint8), rng.integers(112, 140, (rows, K // 32), dtype=np.uint8)


@pytest.mark.parametrize("M,N,K,a2d,b2d", [(256, 256, 256, False, False), (200, 136, 384, False, False),
                                           (128, 160, 256, False, True), (96, 64, 128, True, True),
                                           (1, 1, 128, False, False), (384, 272, 1152, False, True),
                                           (520, 300, 640, False, False)])
def test_nvfp4_gemm_random_operands(M, N, K, a2d, b2d):
    rng = np.random.default_rng(M * 7 + N + K)
    ac, asc = rand_nv(rng, M, K, a2d)
    bc, bsc = rand_nv(rng, N, K, b2d)
    ats, bts = np.float32(0.0123), np.float32(3.5e-3)
    say(f"nvfp4 gemm {M}x{N}x{K} a2d={a2d} b2d={b2d}")
    c = nv.gemm(g(ac), g(asc), g(np.array([ats])), g(bc), g(bsc), g(np.array([bts])),
                "2d" if a2d else "1d", "2d" if b2d else "1d")
    torch.cuda.synchronize()
    ref, cabs = oracle.gemm_fp4(False, ac, asc, bc, bsc, M, N, K, float(ats), float(bts), a2d, b2d)
    check(c.cpu().numpy(), ref, cabs, K, 16, f"nv-{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (200, 136, 384), (128, 128, 128), (1, 3, 128),
                                   (320, 130, 1280)])
def test_mxfp4_gemm_random_operands(M, N, K):
    rng = np.random.default_rng(M * 5 + N * 3 + K)
    ac, asc = rand_mx(rng, M, K)
    bc, bsc = rand_mx(rng, N, K)
    say(f"mxfp4 gemm {M}x{N}x{K}")
    c = nv.mxfp4_gemm(g(ac), g(asc), g(bc), g(bsc))
    torch.cuda.synchronize()
    ref, cabs = oracle.gemm_fp4(True, ac, asc, bc, bsc, M, N, K)
    check(c.cpu().numpy(), ref, cabs, K, 64, f"mx-{M}x{N}x{K}")


def test_gemm_of_quantized_workloads():
    """Operands quantized by the oracle from workload data: activations (the
    gradient-shaped 8192x5120 tensor's first rows) times the 16x16-tiled weight's
    column copy, in both formats."""
    xa = workloads.generate(4, 192, 1024, seed=5)
    xw = workloads.generate(3, 1024, 320, seed=6)  # weight [K][N]: its column copy is B [N][K]
    qa = oracle.quantize(xa, oracle.make_config(), oracle.amax(xa))
    qw = oracle.quantize(xw, oracle.make_config(block="2d", emit_row=False, emit_col=True), oracle.amax(xw))
    say("nvfp4 gemm of quantized workload tensors 192x320x1024")
    c = nv.gemm(g(qa["codes_row"]), g(qa["scales_row"]), g(np.array([qa["tensor_scale"]], np.float32)),
                g(qw["codes_col"]), g(qw["scales_col"]), g(np.array([qw["tensor_scale"]], np.float32)), "1d", "2d")
    torch.cuda.synchronize()
    ref, cabs = oracle.gemm_fp4(False, qa["codes_row"], qa["scales_row"], qw["codes_col"], qw["scales_col"], 192, 320,
                                1024, float(qa["tensor_scale"]), float(qw["tensor_scale"]), False, True)
    check(c.cpu().numpy(), ref, cabs, 1024, 16, "nv-quantized")
    ma = oracle.mxfp4_quantize(xa)
    mw = oracle.mxfp4_quantize(xw, emit_row=False, emit_col=True)
    say("mxfp4 gemm of quantized workload tensors 192x320x1024")
    c = nv.mxfp4_gemm(g(ma["codes_row"]), g(ma["scales_row"]), g(mw["codes_col"]), g(mw["scales_col"]))
    torch.cuda.synchronize()
    ref, cabs = oracle.gemm_fp4(True, ma["codes_row"], ma["scales_row"], mw["codes_col"], mw["scales_col"], 192, 320,
                                1024)
    check(c.cpu().numpy(), ref, cabs, 1024, 64, "mx-quantized")


def test_gemm_full_size_sampled():
    """8192 x 20480 x 5120 (the activation x weight product the bench times),
    random operands; the oracle recomputes sampled rows and columns."""
    M, N, K = 8192, 20480, 5120
    rng = np.random.default_rng(11)
    rows = np.array([0, 1, 127, 128, 4095, 5000, 8190, 8191])
    cols = np.concatenate([np.arange(0, 32), np.arange(20480 - 32, 20480), rng.integers(0, N, 32)])
    for fmt in ("nv", "mx"):
        if fmt == "nv":
            ac, asc = rand_nv(rng, M, K)
            bc, bsc = rand_nv(rng, N, K, two_d=True)
            ats, bts = np.float32(0.01), np.float32(0.002)
            say("full-size nvfp4 gemm 8192x20480x5120")
            c = nv.gemm(g(ac), g(asc), g(np.array([ats])), g(bc), g(bsc), g(np.array([bts])), "1d", "2d")
        else:
            ac, asc = rand_mx(rng, M, K)
            bc, bsc = rand_mx(rng, N, K)
            say("full-size mxfp4 gemm 8192x20480x5120")
            c = nv.mxfp4_gemm(g(ac), g(asc), g(bc), g(bsc))
        torch.cuda.synchronize()
        got = c[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()].cpu().numpy()
        if fmt == "nv":
            # the 2D scales of the sampled B rows, re-indexed to one scale row per sampled row
            bs_rows = bsc[cols // 16]
            ref, cabs = oracle.gemm_fp4(False, ac[rows], asc[rows], bc[cols], bs_rows, len(rows), len(cols), K,
                                        float(ats), float(bts), False, False)
            check(got, ref, cabs, K, 16, "nv-full-sampled")
        else:
            ref, cabs = oracle.gemm_fp4(True, ac[rows], asc[rows], bc[cols], bsc[cols], len(rows), len(cols), K)
            check(got, ref, cabs, K, 64, "mx-full-sampled")
        # determinism: a second run writes identical bits
        c2 = nv.gemm(g(ac), g(asc), g(np.array([ats])), g(bc), g(bsc), g(np.array([bts])), "1d", "2d") \
            if fmt == "nv" else nv.mxfp4_gemm(g(ac), g(asc), g(bc), g(bsc))
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int32), c2.view(torch.int32))
        del c, c2
        torch.cuda.empty_cache()


def test_gemm_empty_k_writes_zeros():
    """K = 0: C is the empty sum, zero everywhere (written by a fill kernel)."""
    for fmt in ("nv", "mx"):
        M, N = 300, 72
        out = torch.full((M, N), 7.0, device="cuda")
        ac = torch.empty((M, 0), dtype=torch.uint8, device="cuda")
        bc = torch.empty((N, 0), dtype=torch.uint8, device="cuda")
        ts = torch.ones(1, device="cuda")
        say(f"{fmt} gemm with K = 0, {M}x{N}")
        if fmt == "nv":
            nv.gemm(ac, ac, ts, bc, bc, ts, "1d", "1d", out=out)
        else:
            nv.mxfp4_gemm(ac, ac, bc, bc, out=out)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out).item() == 0
