"""GPU parity of the MXFP4 variant (32-element blocks, E8M0 scales): the HIP
path through the C ABI against the CPU oracle, bit for bit."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
nv = pytest.importorskip("nvfp4_block_quantization_amd")

pytestmark = pytest.mark.gpu

KEYS = ("codes_row", "scales_row", "codes_col", "scales_col")


def say(msg: str) -> None:
    print(f"[gpu-mxfp4] {msg}", flush=True)


def to_gpu(x: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def f32_bits(a) -> np.ndarray:
    return np.asarray(a, np.float32).view(np.uint32)


def compare(x, tag, row=True, col=False, sr=False, seed=0, row_offset=0):
    say(f"{tag}: {x.shape[0]}x{x.shape[1]} {x.dtype} row={row} col={col} sr={sr} row_offset={row_offset}")
    out = nv.mxfp4_quantize(to_gpu(x), rowwise=row, colwise=col, sr=sr, sr_seed=seed, row_offset=row_offset)
    torch.cuda.synchronize()
    ref = oracle.mxfp4_quantize(x, emit_row=row, emit_col=col, sr=sr, sr_seed=seed, row_offset=row_offset)
    for k in KEYS:
        if k in ref:
            got = out[k].cpu().numpy()
            if not np.array_equal(got, ref[k]):
                bad = np.argwhere(got != ref[k])
                raise AssertionError(f"{tag}: {k} differs at {len(bad)} places, first {bad[:5].tolist()}")
    return out, ref


# several 256x64 strips with ragged tails: 64-column strips half full, a 32-row last sub-tile
SHAPES = [(256, 256), (64, 96), (288, 160), (96, 2080), (352, 32)]


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("path", ["row", "row+col", "col"])
def test_mxfp4_matrix(rows, cols, sr, dtype, path):
    x = workloads.generate(1 if dtype == "f32" else 5, rows, cols, seed=31)
    compare(x, f"mx-{path}-{dtype}-sr{int(sr)}", row=path != "col", col=path != "row", sr=sr, seed=77)


def test_mxfp4_row_copy_any_row_count():
    x = workloads.generate(2, 50, 4128, seed=3)
    compare(x, "mx-rows50", sr=True, seed=5)


@pytest.mark.parametrize("row_offset", [8192 * 3, (1 << 36) // 160, (1 << 34) // 160 - 20])
@pytest.mark.parametrize("col", [True, False])
def test_mxfp4_row_offset(row_offset, col):
    # element indices below 2^34, above it, and crossing it inside the tensor
    x = workloads.generate(4, 64, 160, seed=2)
    compare(x, f"mx-row-offset-{row_offset}", row=True, col=col, sr=True, seed=9, row_offset=row_offset)


def test_mxfp4_edge_cases():
    z = np.zeros((64, 64), np.float32)
    compare(z, "mx-zeros", col=True)
    compare(-z, "mx-negzeros", col=True, sr=True, seed=1)
    rng = np.random.default_rng(4)
    # tiny elements beside a block max of ~1: their scaled values are subnormal
    tiny = (rng.standard_normal((64, 64)) * 1e-40).astype(np.float32)
    tiny[::7, ::5] = 1.0
    compare(tiny, "mx-tiny-subnormal-z", col=True)
    compare(-tiny, "mx-tiny-subnormal-z-neg", col=True, sr=True, seed=2)
    # subnormal block maxima (scale code 0) and the largest magnitudes (code 252)
    sub = (rng.standard_normal((64, 64)) * 1e-41).astype(np.float32)
    compare(sub, "mx-subnormal-blocks", col=True, sr=True, seed=3)
    huge = (rng.standard_normal((64, 64)) * 1e37).astype(np.float32)
    huge[3, 3] = np.float32(3.4e38)
    out, _ = compare(huge, "mx-huge", col=True)
    assert int(out["scales_row"].max().item()) == 252
    # one outlier crushes its block (section 1's contrast with NVFP4)
    x = np.full((32, 64), 0.75, np.float32)
    x[0, 0] = 100.0
    out, _ = compare(x, "mx-outlier", col=True)
    assert int(out["codes_row"][0, 1:16].max().item()) == 0


@pytest.mark.parametrize("rows,cols", [(256, 256), (96, 2080)])
def test_mxfp4_dequantize(rows, cols):
    x = workloads.generate(5, rows, cols, seed=6)
    out, ref = compare(x, "mx-deq", col=True, sr=True, seed=8)
    say(f"mx dequantize row copy {rows}x{cols}, column copy {cols}x{rows}")
    d = nv.mxfp4_dequantize(out["codes_row"], out["scales_row"], rows, cols)
    r = oracle.mxfp4_dequantize(ref["codes_row"], ref["scales_row"], rows, cols)
    assert np.array_equal(f32_bits(d.cpu().numpy()), f32_bits(r))
    d = nv.mxfp4_dequantize(out["codes_col"], out["scales_col"], cols, rows)
    r = oracle.mxfp4_dequantize(ref["codes_col"], ref["scales_col"], cols, rows)
    assert np.array_equal(f32_bits(d.cpu().numpy()), f32_bits(r))


def test_mxfp4_dequantize_every_code_and_scale():
    """All 256 scale codes (0: 2^-127, 255: NaN) against all 16 element codes."""
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 256, (256, 16), dtype=np.uint8)
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    say("mx dequantize: every E8M0 code")
    d = nv.mxfp4_dequantize(to_gpu(codes), to_gpu(scales), 256, 32)
    r = oracle.mxfp4_dequantize(codes, scales, 256, 32)
    got = d.cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(r)) and np.isnan(r[255]).all()
    ok = ~np.isnan(r)
    assert np.array_equal(f32_bits(got[ok]), f32_bits(r[ok]))


def _oracle_mx_bands(x, rows, cols, band=4096, **kw):
    """The MXFP4 oracle over row bands on up to 16 host threads (the C oracle
    releases the interpreter lock), assembled into whole-tensor outputs; bands
    are whole 32-row blocks and carry their global row offset, so the result
    is the single-call result."""
    codes_row = np.empty((rows, cols // 2), np.uint8)
    scales_row = np.empty((rows, cols // 32), np.uint8)
    codes_col = np.empty((cols, rows // 2), np.uint8)
    scales_col = np.empty((cols, rows // 32), np.uint8)

    def run(r0):
        r1 = min(rows, r0 + band)
        ref = oracle.mxfp4_quantize(x[r0:r1], emit_row=True, emit_col=True, row_offset=r0, **kw)
        codes_row[r0:r1] = ref["codes_row"]
        scales_row[r0:r1] = ref["scales_row"]
        codes_col[:, r0 // 2:r1 // 2] = ref["codes_col"]
        scales_col[:, r0 // 32:r1 // 32] = ref["scales_col"]

    with ThreadPoolExecutor(max_workers=max(1, min(os.cpu_count() or 1, 16))) as pool:
        list(pool.map(run, range(0, rows, band)))
    return {"codes_row": codes_row, "scales_row": scales_row, "codes_col": codes_col, "scales_col": scales_col}


def test_mxfp4_full_size_whole():
    """65536x8192 bf16 (the mixture-of-Gaussians activation), row and column
    copies with stochastic rounding: every output byte against the oracle,
    then a rerun that must write the same bytes."""
    c = workloads.CONFIGS[5]
    rows, cols = c["rows"], c["cols"]
    say(f"mx full size: generating {rows}x{cols}")
    x = workloads.inputs(c, seed=0)
    xg = to_gpu(x)
    say("mx full size: GPU quantize")
    out = nv.mxfp4_quantize(xg, rowwise=True, colwise=True, sr=True, sr_seed=7)
    torch.cuda.synchronize()
    say("mx full size: oracle in row bands")
    ref = _oracle_mx_bands(x, rows, cols, sr=True, sr_seed=7)
    for k in KEYS:
        got = out[k].cpu().numpy()
        if not np.array_equal(got, ref[k]):
            bad = np.argwhere(got != ref[k])
            raise AssertionError(f"mx full size: {k} differs at {len(bad)} places, first {bad[:5].tolist()}")
    say("mx full size: determinism rerun")
    out2 = nv.mxfp4_quantize(xg, rowwise=True, colwise=True, sr=True, sr_seed=7)
    torch.cuda.synchronize()
    for k in KEYS:
        assert torch.equal(out[k], out2[k]), k
    assert int(out["scales_row"].max().item()) <= 252 and int(out["scales_col"].max().item()) <= 252
    del xg, out, out2
    torch.cuda.empty_cache()


def test_mxfp4_full_size_row_copy_rne():
    """8192x4096 bf16 (the activation with outlier columns), the MXFP4 row copy
    alone with round-to-nearest, which the row kernel computes: every output
    byte against the oracle, then a rerun that must write the same bytes."""
    c = workloads.CONFIGS[2]
    rows, cols = c["rows"], c["cols"]
    say(f"mx row copy full size: generating {rows}x{cols}")
    x = workloads.inputs(c, seed=0)
    xg = to_gpu(x)
    say("mx row copy full size: GPU quantize")
    out = nv.mxfp4_quantize(xg, rowwise=True, colwise=False, sr=False)
    torch.cuda.synchronize()
    say("mx row copy full size: oracle in row bands")
    ref = _oracle_mx_bands(x, rows, cols, sr=False)
    for k in ("codes_row", "scales_row"):
        got = out[k].cpu().numpy()
        if not np.array_equal(got, ref[k]):
            bad = np.argwhere(got != ref[k])
            raise AssertionError(f"mx row copy full size: {k} differs at {len(bad)} places, first {bad[:5].tolist()}")
    say("mx row copy full size: determinism rerun")
    out2 = nv.mxfp4_quantize(xg, rowwise=True, colwise=False, sr=False)
    torch.cuda.synchronize()
    for k in ("codes_row", "scales_row"):
        assert torch.equal(out[k], out2[k]), k
    del xg, out, out2
    torch.cuda.empty_cache()
