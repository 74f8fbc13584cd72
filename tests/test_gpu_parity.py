"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, bit for
bit, on the same seeded inputs: small shapes and the five full-size workloads,
every output byte."""
import os

import numpy as np
import pytest

import oracle
import workloads

torch = pytest.importorskip("torch")
nv = pytest.importorskip("nvfp4_block_quantization_amd")

pytestmark = pytest.mark.gpu


def say(msg: str) -> None:
    print(f"[gpu-parity] {msg}", flush=True)


def to_gpu(x: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def f32_bits(a) -> np.ndarray:
    return np.asarray(a, np.float32).view(np.uint32)


def gpu_quantize(xg, c, amax_t=None):
    if amax_t is None:
        amax_t = nv.amax(xg, rht=c["rht"], rht_mask=c.get("rht_mask", 0))
    out = nv.quantize(xg, amax_t, block=c["block"], rowwise=c["emit_row"], colwise=c["emit_col"], rht=c["rht"],
                      rht_mask=c.get("rht_mask", 0), sr=c["sr"], sr_seed=c["sr_seed"], rule=c["rule"],
                      scale_cap=c["cap"], row_offset=c.get("row_offset", 0))
    return amax_t, out


def oracle_cfg(c, row_offset=None):
    return oracle.make_config(block=c["block"], emit_row=c["emit_row"], emit_col=c["emit_col"], rht=c["rht"],
                              rht_mask=c.get("rht_mask", 0), sr=c["sr"], sr_seed=c["sr_seed"],
                              row_offset=c.get("row_offset", 0) if row_offset is None else row_offset,
                              rule=c["rule"], cap=c["cap"])


def with_mask(c):
    c = dict(c)
    c["rht_mask"] = nv.rht_signs_from_seed(c["rht_seed"]) if c["rht"] else 0
    return c


def compare_all(x, c, tag):
    """Whole-tensor parity for a small case."""
    say(f"{tag}: shape {c['rows']}x{c['cols']} block={c['block']} row={c['emit_row']} col={c['emit_col']} "
        f"rht={c['rht']} sr={c['sr']} rule={c['rule']} cap={c['cap']}")
    xg = to_gpu(x)
    a_t, out = gpu_quantize(xg, c)
    torch.cuda.synchronize()
    A = oracle.amax(x, rht=c["rht"], mask=c.get("rht_mask", 0))
    assert f32_bits(a_t.cpu().numpy())[0] == f32_bits(A), f"{tag}: amax"
    ref = oracle.quantize(x, oracle_cfg(c), A)
    assert f32_bits(out["tensor_scale"].cpu().numpy())[0] == f32_bits(ref["tensor_scale"]), f"{tag}: tensor scale"
    for k in ("codes_row", "scales_row", "codes_col", "scales_col"):
        if k in ref:
            got = out[k].cpu().numpy()
            if not np.array_equal(got, ref[k]):
                bad = np.argwhere(got != ref[k])
                raise AssertionError(f"{tag}: {k} differs at {len(bad)} places, first {bad[:5].tolist()}")
    return xg, a_t, out, ref


# ------------------------------------------------------- small, whole ----

SMALL = [
    # (workload, rows, cols): several tiles plus a ragged tail in both directions
    (1, 256, 256),
    (1, 33, 80),
    (2, 272, 4112),
    (3, 80, 336),
    (3, 144, 208),
    (4, 48, 1040),
    (5, 144, 400),
    (5, 208, 176),
]


@pytest.mark.parametrize("k,rows,cols", SMALL)
def test_small_workloads_bit_exact(k, rows, cols):
    c = with_mask(workloads.config(k, rows, cols))
    x = workloads.inputs(c, seed=0)
    compare_all(x, c, f"workload{k}")
    if k == 5:
        compare_all(x, dict(c, rule="none", cap=448.0), "workload5-plain")


@pytest.mark.parametrize("rule", ["none", "mse", "mae", "maxerr"])
@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("path", ["row", "row+col", "col", "2d", "2d-row", "row-rht"])
def test_option_matrix(rule, sr, dtype, path):
    rows, cols = 80, 208
    kind = 1 if dtype == "f32" else 5
    x = workloads.generate(kind, rows, cols, seed=21)
    c = dict(rows=rows, cols=cols, block="2d" if path.startswith("2d") else "1d",
             emit_row=path != "col", emit_col=path in ("row+col", "col", "2d"), rht=path == "row-rht",
             rht_mask=0xB3E1 if path == "row-rht" else 0, sr=sr, sr_seed=99, rule=rule,
             cap=256.0 if rule != "none" else 448.0)
    compare_all(x, c, f"matrix-{path}-{dtype}-{rule}-sr{int(sr)}")


# Row offsets: a small one; one whose Philox counters (idx / 4) have a nonzero
# high word; one whose counters cross 2^32 inside the tensor (the low counter
# word wraps between lanes of one workgroup).
@pytest.mark.parametrize("row_offset", [4096, (1 << 36) // 96, (1 << 34) // 96 - 20])
@pytest.mark.parametrize("path", ["1d", "2d", "row"])
def test_row_offset_keys_the_random_stream(row_offset, path):
    x = workloads.generate(5, 64, 96, seed=4)
    c = dict(rows=64, cols=96, block="2d" if path == "2d" else "1d", emit_row=True, emit_col=path != "row",
             rht=False, sr=True, sr_seed=7, rule="mae", cap=256.0, row_offset=row_offset)
    compare_all(x, c, f"row-offset-{row_offset}-{path}")


def test_dequantize_matches_oracle():
    for k, rows, cols in ((1, 256, 256), (3, 80, 336), (5, 144, 400)):
        c = workloads.config(k, rows, cols)
        x = workloads.inputs(c)
        xg, a_t, out, ref = compare_all(x, c, f"dequant-{k}")
        st = ref["tensor_scale"]
        blk = c["block"]
        if c["emit_row"]:
            say(f"dequantize row copy {rows}x{cols} block={blk}")
            d = nv.dequantize(out["codes_row"], out["scales_row"], out["tensor_scale"], rows, cols, blk)
            r = oracle.dequantize(ref["codes_row"], ref["scales_row"], st, rows, cols, blk)
            assert np.array_equal(f32_bits(d.cpu().numpy()), f32_bits(r))
        if c["emit_col"]:
            say(f"dequantize col copy {cols}x{rows} block={blk}")
            d = nv.dequantize(out["codes_col"], out["scales_col"], out["tensor_scale"], cols, rows, blk)
            r = oracle.dequantize(ref["codes_col"], ref["scales_col"], st, cols, rows, blk)
            assert np.array_equal(f32_bits(d.cpu().numpy()), f32_bits(r))
            if blk == "2d":  # both orientations dequantize to the same tensor
                d_row = nv.dequantize(out["codes_row"], out["scales_row"], out["tensor_scale"], rows, cols, blk)
                assert torch.equal(d_row.view(torch.int32), d.t().contiguous().view(torch.int32))


def test_edge_cases():
    # empty tensor: amax 0, tensor scale 0
    say("edge: empty")
    xg = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda")
    a = nv.amax(xg)
    out = nv.quantize(xg, a)
    torch.cuda.synchronize()
    assert a.item() == 0.0 and out["tensor_scale"].item() == 0.0
    base = dict(block="1d", emit_row=True, emit_col=True, rht=False, sr=False, sr_seed=0, rule="mae", cap=256.0)
    # zeros, signed zeros, a single nonzero, tiny (subnormal-range) and huge values
    z = np.zeros((32, 48), np.float32)
    compare_all(z, dict(base, rows=32, cols=48), "edge-zeros")
    compare_all(-z, dict(base, rows=32, cols=48), "edge-negzeros")
    one = z.copy()
    one[5, 7] = -3.5
    compare_all(one, dict(base, rows=32, cols=48, sr=True, sr_seed=3), "edge-single")
    rng = np.random.default_rng(2)
    tiny = (rng.standard_normal((32, 48)) * 1e-39).astype(np.float32)
    compare_all(tiny, dict(base, rows=32, cols=48), "edge-tiny")
    compare_all(tiny, dict(base, rows=32, cols=48, block="2d", rule="mse"), "edge-tiny-2d")
    huge = (rng.standard_normal((32, 48)) * 1e37).astype(np.float32)
    compare_all(huge, dict(base, rows=32, cols=48, sr=True, sr_seed=5), "edge-huge")
    # a caller-provided amax smaller than the data (saturating blocks) and larger (tiny scales)
    x = workloads.generate(5, 32, 48, seed=8)
    xg = to_gpu(x)
    for A in (0.5, 1e6, 3.0e-30):
        c = dict(base, rows=32, cols=48, sr=True, sr_seed=11)
        say(f"edge: given amax {A}")
        a_t = torch.tensor([A], dtype=torch.float32, device="cuda")
        _, out = gpu_quantize(xg, c, a_t)
        ref = oracle.quantize(x, oracle_cfg(c), float(np.float32(A)))
        for k in ("codes_row", "scales_row", "codes_col", "scales_col"):
            assert np.array_equal(out[k].cpu().numpy(), ref[k]), (A, k)


def test_rht_mask_derivation():
    for seed in (0, 1234, 2 ** 33 + 5):
        assert nv.rht_signs_from_seed(seed) == oracle.rht_mask_from_seed(seed)


def test_invalid_arguments_raise_on_gpu():
    xg = torch.zeros((8, 24), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nv.NVFP4Error):
        nv.quantize(xg, nv.amax(torch.zeros((8, 32), dtype=torch.bfloat16, device="cuda")))


# ---------------------------------------------------- full size, whole ----

def _oracle_threads() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


def _assert_same(tag, key, got: np.ndarray, ref: np.ndarray) -> None:
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        raise AssertionError(f"{tag}: {key} differs at {len(bad)} places, first {bad[:5].tolist()}")


# Several full 256-row strips plus a partial last strip (the strip kernel's
# partial write-out of codes and scales), with 4/6 and stochastic rounding.
MULTI_STRIP = [(272, 208), (320, 80), (528, 208)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("path", ["1d-row-col", "2d-row-col"])
@pytest.mark.parametrize("rows,cols", MULTI_STRIP)
def test_multi_strip_sr_four_over_six(rows, cols, path, dtype):
    k = 5 if dtype == "bf16" else 1
    c = workloads.config(k, rows, cols, block="2d" if path.startswith("2d") else "1d", emit_row=True,
                         emit_col=True, rht=False, sr=True, sr_seed=41, rule="mae", cap=256.0)
    x = workloads.generate(k, rows, cols, seed=12)
    compare_all(x, c, f"strips-{rows}x{cols}-{path}-{dtype}")


FULL = {1: workloads.CONFIGS[1], 2: workloads.CONFIGS[2], 3: workloads.CONFIGS[3], 4: workloads.CONFIGS[4],
        5: workloads.CONFIGS[5], "5plain": workloads.CONFIG5_PLAIN, "2plain": workloads.CONFIG2_PLAIN,
        "3sr": workloads.CONFIG3_SR}


@pytest.mark.parametrize("k", list(FULL))
def test_full_size_workloads_whole(k):
    """Every output byte of the full-size workloads against the oracle (row
    bands of the oracle run on up to 16 host threads; blocks are independent,
    so threading does not change its bits), then a rerun that must write the
    same bytes."""
    c = with_mask(FULL[k])
    rows, cols = c["rows"], c["cols"]
    tag = f"full workload {k}"
    say(f"{tag}: generating {rows}x{cols}")
    x = workloads.inputs(c, seed=0)
    xg = to_gpu(x)
    say(f"{tag}: GPU amax + quantize")
    a_t, out = gpu_quantize(xg, c)
    torch.cuda.synchronize()
    say(f"{tag}: oracle amax")
    A = oracle.amax(x, rht=c["rht"], mask=c.get("rht_mask", 0))
    assert f32_bits(a_t.cpu().numpy())[0] == f32_bits(A)
    say(f"{tag}: oracle quantize on {_oracle_threads()} threads")
    ref = oracle.quantize(x, oracle_cfg(c), A, nthreads=_oracle_threads())
    assert f32_bits(out["tensor_scale"].cpu().numpy())[0] == f32_bits(ref["tensor_scale"])
    for key in ("codes_row", "scales_row", "codes_col", "scales_col"):
        if key in ref:
            _assert_same(tag, key, out[key].cpu().numpy(), ref[key])
    # determinism: a second run writes identical bytes
    say(f"{tag}: determinism rerun")
    _, out2 = gpu_quantize(xg, c, a_t)
    torch.cuda.synchronize()
    for key in ("codes_row", "scales_row", "codes_col", "scales_col"):
        if key in out:
            assert torch.equal(out[key], out2[key]), key
    if k == 1:
        say(f"{tag}: dequantize")
        d = nv.dequantize(out["codes_row"], out["scales_row"], out["tensor_scale"], rows, cols)
        r = oracle.dequantize(ref["codes_row"], ref["scales_row"], ref["tensor_scale"], rows, cols)
        assert np.array_equal(f32_bits(d.cpu().numpy()), f32_bits(r))
    del xg, out, out2, ref
    torch.cuda.empty_cache()


def test_full_size_dequantize_workload5_row_copy():
    """The row copy of the 65536x8192 activation, dequantized on the GPU (the
    launch the benchmark times), against the oracle's dequantization of the
    same codes, scales and tensor scale: every value bit for bit."""
    c = with_mask(FULL[5])
    rows, cols = c["rows"], c["cols"]
    tag = "full dequantize workload 5"
    say(f"{tag}: generating {rows}x{cols}")
    x = workloads.inputs(c, seed=0)
    xg = to_gpu(x)
    del x
    say(f"{tag}: GPU amax + quantize + dequantize")
    _, out = gpu_quantize(xg, c)
    del xg
    d = nv.dequantize(out["codes_row"], out["scales_row"], out["tensor_scale"], rows, cols)
    torch.cuda.synchronize()
    got = d.cpu().numpy()
    codes, scales = out["codes_row"].cpu().numpy(), out["scales_row"].cpu().numpy()
    s_t = float(out["tensor_scale"].cpu().numpy()[0])
    del d, out
    torch.cuda.empty_cache()
    say(f"{tag}: oracle dequantize")
    ref = oracle.dequantize(codes, scales, s_t, rows, cols)
    _assert_same(tag, "dequantized", f32_bits(got), f32_bits(ref))
