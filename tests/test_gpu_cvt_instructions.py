"""Exhaustive GPU pin of the gfx950 conversion instructions the quantizers
rely on (tests/pins/gfx950_cvt_check.hip): the FP4 encode with unit scale on
every non-NaN binary32 input against nearest-even-with-saturation, the FP4
decode against the signed grid, the nibble/byte layout, the fp32->bf16
conversion against round-to-nearest-even, and the FP8 (E4M3) encode on every
input up to 448 in magnitude against the nearest format value (ties to the
even code) with its decode and byte layout."""
import os
import subprocess

import pytest

from gpu_util import announce, gpu_device

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "pins", "_build", "gfx950_cvt_check")


def test_conversion_instructions_exhaustive():
    gpu_device()
    if not os.path.exists(EXE):
        pytest.fail("tests/pins/_build/gfx950_cvt_check is not built (run the package build)")
    announce("gfx950_cvt_check: all 2^32 inputs")
    out = subprocess.run([EXE], capture_output=True, text=True, timeout=120, check=True).stdout.split()
    fp4_bad, bf16_bad, decode_ok, layout = int(out[0]), int(out[1]), int(out[2]), out[3]
    fp8_bad, fp8_decode_ok, fp8_layout = int(out[4]), int(out[5]), out[6]
    assert fp4_bad == 0
    assert bf16_bad == 0
    assert decode_ok == 1
    # byte k = codes of the k-th pair, first value in the low nibble:
    # (0.5,1)->0x21, (1.5,2)->0x43, (3,4)->0x65, (6,-0.5)->0x97
    assert layout == "0x97654321"
    # FP8: nearest even on every |x| <= 448 (the quantizer clamps to 448),
    # every non-NaN code decodes to its value; bytes in element order:
    # 1.0 -> 0x38, -2.0 -> 0xC0, 448 -> 0x7E, 2^-9 -> 0x01
    assert fp8_bad == 0
    assert fp8_decode_ok == 1
    assert fp8_layout == "0x017ec038"
