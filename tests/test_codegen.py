"""Code-generation checks on the gfx950 assembly of the quantization kernels
(compiled here from source; no GPU needed).

The E2M1 converts write one byte of their destination register and can write
it before the second of their two source values has been read.  A destination
that shares a register with a source therefore lets the second slot round a
value whose low byte has already been replaced, which showed up on the device
as rare run-to-run differences in the second slot's codes.  Every fp4 convert
in the generated code must keep its destination apart from its sources."""
import os
import re
import shutil
import subprocess

import pytest

from nvfp4_block_quantization_amd import build as nvbuild

HIPCC = nvbuild.HIPCC
FP4_ENCODE = ("v_cvt_scalef32_pk_fp4_f32", "v_cvt_scalef32_sr_pk_fp4_f32")


def _vregs(operand: str) -> set:
    regs = set()
    for lo, hi, one in re.findall(r"v\[(\d+):(\d+)\]|v(\d+)", operand):
        if one:
            regs.add(int(one))
        else:
            regs.update(range(int(lo), int(hi) + 1))
    return regs


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which(HIPCC)):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "nvfp4.s"
    flags = [f for f in nvbuild.FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [HIPCC, *flags, "--cuda-device-only", "-S", "-o", str(out), nvbuild.SOURCES[0]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


def test_fp4_converts_keep_destination_apart_from_sources(device_asm):
    """Every scaled convert (the E2M1 encoders and the E2M1 decoder of the 4/6
    error and the dequantizer) keeps its destination apart from its sources."""
    seen, encoders, bad = 0, 0, []
    for line in device_asm.splitlines():
        line = line.strip()
        op = line.split(None, 1)[0] if line else ""
        if not op.startswith("v_cvt_scalef32"):
            continue
        seen += 1
        encoders += op in FP4_ENCODE
        dst, src_a, src_b = [o.strip() for o in line.split(None, 1)[1].split(",")[:3]]
        if _vregs(dst) & (_vregs(src_a) | _vregs(src_b)):
            bad.append(line)
    assert encoders > 1000, "the quantization kernels should contain the fp4 encoders"
    assert not bad, f"{len(bad)} converts share a register between destination and source, e.g. {bad[:3]}"
