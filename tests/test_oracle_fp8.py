"""Pins of the oracle's FP8 (E4M3) per-tensor QDQ.

Pages: 'Model-Optimizer 实战 ... W4A4 NVFP4 精度' (nlpx.cn), section '3. QAD'
(attention projections FP8 W8A8, KV cache FP8) and 'NVIDIA AI bringt
Nemotron-3-Nano-30B auf NVFP4 ...' (chatgpz.de) (FP8 KV cache).  Reading:
one FP32 scale per tensor, s = amax/448; code = sign | E4M3(|x|/s), nearest
even, saturating; y = bf16(dec(code) * s).

Pins: a hand-derived tensor (tests/golden/fp8_worked_example.json); the codec
against torch's float8_e4m3fn cast on every bf16 value it represents without
overflow; the dequantized value against torch's float8 decode; re-quantizing
the output with the same scale reproduces the codes; the error bound (half
an E4M3 step); the zero tensor; a frozen scale is used as given.
"""
import json
import os

import numpy as np
import pytest
import torch

from nvfp4_quantization_aware_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def f32(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def test_worked_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "fp8_worked_example.json")))
    x = np.array(g["x"], np.float32)
    codes, ts, y = orc.fp8_quantize(x)
    assert ts == np.float32(g["tscale"])
    assert codes.tolist() == g["codes"]
    assert y.tolist() == g["y_bf16"]


def test_codes_against_torch_float8_all_bf16(orc):
    # every finite bf16 value with |v| <= 464 (beyond it torch's E4M3FN cast
    # overflows to NaN where the reading saturates at 448), scale 1
    bits = np.arange(1 << 16, dtype=np.uint32)
    v = f32(bits)
    keep = np.isfinite(v) & (np.abs(v) <= 464)
    vb = bits[keep].astype(np.uint16)
    codes, _, y = orc.fp8_quantize(vb, tscale=1.0)
    ref = torch.from_numpy(f32(vb).copy()).to(torch.float8_e4m3fn)
    assert np.array_equal(codes, ref.view(torch.uint8).numpy())
    ref_y = ref.float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, ref_y)


def test_saturation(orc):
    x = np.array([480, 1e6, -1e30, 447.9], np.float32)
    codes, _, _ = orc.fp8_quantize(x, tscale=1.0)
    assert codes.tolist() == [0x7E, 0x7E, 0xFE, 0x7E]


@pytest.mark.parametrize("seed", [1, 2])
def test_requantize_and_error_bound(orc, seed):
    x = synth.outlier_tensor_f32(256, 1024, seed=seed).numpy() if seed == 1 else \
        synth.bf16_bits(synth.gaussian_weight_bf16(64, 256, seed=seed))
    codes, s, y = orc.fp8_quantize(x)
    # re-quantizing the output with the same scale gives the same codes
    codes2, s2, y2 = orc.fp8_quantize(y, tscale=s)
    assert s2 == s and np.array_equal(codes2, codes) and np.array_equal(y2, y)
    # |x - dec*s| <= half an E4M3 step at that magnitude (plus bf16 input rounding: none for bf16 x)
    xf = x if x.dtype == np.float32 else f32(x)
    dec = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    a = np.abs(xf.astype(np.float64)) / s
    step = np.where(a < 2.0**-6, 2.0**-9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0**-6))) - 3))
    assert np.all(np.abs(a - np.abs(dec)) <= step / 2 * (1 + 1e-6))


def test_zero_tensor_and_frozen_scale(orc):
    x = np.array([0.0, -0.0, 0.0, 0.0], np.float32)
    codes, s, y = orc.fp8_quantize(x)
    assert s == 1.0 and codes.tolist() == [0, 0x80, 0, 0] and y.tolist() == [0, 0x8000, 0, 0]
    x = np.array([1.0, 2.0, 3.0, 100.0], np.float32)
    codes, s, _ = orc.fp8_quantize(x, tscale=0.25)
    # 4, 8, 12 exact; 400 is the midpoint of 384 and 416 -> the even mantissa, 384
    assert s == 0.25 and codes.tolist() == [72, 80, 84, 124]
