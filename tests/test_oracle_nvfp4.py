"""Pins of the oracle's NVFP4 quantizer (dynamic and frozen scales).

Format facts from the page 'NVIDIA AI bringt Nemotron-3-Nano-30B auf NVFP4
...' (chatgpz.de), section 'NVFP4-Format und warum es wichtig ist?': blocks of
16, an E4M3 scale per block, an FP32 scale per tensor, 4-bit float values, and
about 1.8x less memory than FP8.  Dynamic scales are recomputed every step and
frozen ones are kept fixed (page '使用量化感知蒸馏技术构建Nemotron 3.5 Lightning
NVFP4模型', section '量化尺度处理策略').

Pins used: hand-derived worked examples (tests/golden), constructed exact
ties from the rounding definition, closed forms (storage size, power-of-two
scaling), invariants (error bound, block maximum at the top of the grid,
frozen idempotence, amax) and special cases (zero tensor, tiny blocks).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from nvfp4_quantization_aware_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bits_of(values):
    """bf16 bit patterns of floats that are exactly representable in bf16."""
    f = np.array(values, np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def _unpack(codes):
    lo = codes & 0xF
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


def test_worked_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "nvfp4_worked_example.json")))
    x = np.array(g["x_f32"], np.float32).reshape(g["rows"], g["cols"])
    codes, scales, ts, y = orc.nvfp4_quantize(x)
    assert ts == g["tscale"]
    assert scales.reshape(-1).tolist() == g["scales"]
    assert codes.reshape(-1).tolist() == g["codes_packed"]
    assert _unpack(codes).reshape(-1).tolist() == g["codes_unpacked"]
    assert np.array_equal(y.reshape(-1), _bits_of(g["y"]))


def test_small_scales(orc):
    g = json.load(open(os.path.join(GOLDEN, "nvfp4_small_scales.json")))
    x = np.concatenate([np.array(b["x"], np.float32) for b in g["blocks"]])[None, :]
    codes, scales, ts, y = orc.nvfp4_quantize(x)
    assert ts == g["tscale"]
    assert scales.reshape(-1).tolist() == [b["scale"] for b in g["blocks"]]
    un = _unpack(codes).reshape(len(g["blocks"]), 16)
    for i, b in enumerate(g["blocks"]):
        assert un[i].tolist() == b["codes"], i
    yb = orc.f32_from_bf16(y.reshape(-1))
    assert yb[4 * 16] == g["blocks"][4]["y0"]
    # zero effective scale: signed zeros out
    assert y.reshape(-1)[2 * 16 + 1] == 0x8000 and y.reshape(-1)[2 * 16] == 0


# ties at every rounding midpoint and the neighbours on either side, at many
# power-of-two tensor scales 2^j and block scales 2^m
MID = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
AT = [0, 2, 2, 4, 4, 6, 6]          # ties go to the even index
ABOVE = [1, 2, 3, 4, 5, 6, 7]
BELOW = [0, 1, 2, 3, 4, 5, 6]


@pytest.mark.parametrize("j", [-20, -7, 0, 3, 11])
@pytest.mark.parametrize("m", [-9, -8, -6, -3, 0, 4, 8])
def test_exact_ties(orc, j, m):
    s = 2.0 ** (j + m)
    blocks = [[2688.0 * 2.0**j] + [0.0] * 15]
    expect = [[7] + [0] * 15]
    for which, table in ((0, AT), (1, ABOVE), (-1, BELOW)):
        vals, exp = [6.0 * s], [7]
        for t, e in zip(MID, table):
            v = np.float32(t * s)
            if which == 1:
                v = np.nextafter(v, np.float32(np.inf))
            elif which == -1:
                v = np.nextafter(v, np.float32(0))
            vals.append(float(v))
            exp.append(e)
            vals.append(-float(v))
            exp.append(8 + e)
        blocks.append(vals + [0.0])
        expect.append(exp + [0])
    x = np.array(blocks, np.float32).reshape(1, -1)
    codes, scales, ts, _ = orc.nvfp4_quantize(x)
    assert ts == 2.0**j
    sb = scales.reshape(-1)
    assert orc.e4m3_decode(int(sb[1])) == 2.0**m
    assert _unpack(codes).reshape(-1, 16).tolist() == expect


def test_zero_tensor(orc):
    x = np.zeros((3, 64), np.float32)
    x[1, 5] = -0.0
    codes, scales, ts, y = orc.nvfp4_quantize(x)
    assert ts == 1.0
    assert not scales.any()
    assert _unpack(codes)[1, 5] == 8 and (_unpack(codes).reshape(-1) & 7).max() == 0
    assert y[1, 5] == 0x8000 and np.count_nonzero(y) == 1


def test_storage_is_4p5_bits_per_element(orc):
    x = synth.outlier_tensor_f32(seed=1).numpy()
    codes, scales, _, _ = orc.nvfp4_quantize(x)
    bits = 8.0 * (codes.nbytes + scales.nbytes) / x.size
    assert bits == 4.5
    # the page's "about 1.8x less memory than FP8"
    assert round(8.0 / bits, 1) == 1.8


def test_amax_exact(orc):
    x = synth.outlier_tensor_f32(seed=7).numpy()
    assert orc.amax(x) == np.abs(x).max()
    w, _ = synth.moe_weights_bf16(experts=1, rows=64, cols=256, seed=7, with_grad=False)
    bits = synth.bf16_bits(w[0])
    assert orc.amax(bits) == np.abs(w[0].float().numpy()).max()
    assert orc.tensor_scale(orc.amax(x)) == np.float32(np.abs(x).max()) / np.float32(2688.0)


@pytest.mark.parametrize("k", [-12, -3, 5, 40])
def test_power_of_two_scaling(orc, k):
    x = synth.outlier_tensor_f32(rows=64, cols=256, seed=11).numpy()
    c0, s0, t0, y0 = orc.nvfp4_quantize(x)
    c1, s1, t1, y1 = orc.nvfp4_quantize((x * np.float32(2.0**k)).astype(np.float32))
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
    assert t1 == t0 * 2.0**k
    assert np.array_equal(orc.f32_from_bf16(y0) * np.float32(2.0**k), orc.f32_from_bf16(y1))


def _seff(orc, scales, ts):
    tab = orc.e4m3_decode_table()
    return (tab[scales].astype(np.float32) * np.float32(ts)).astype(np.float32)


def test_error_bound_and_block_max(orc):
    x = synth.outlier_tensor_f32(seed=1).numpy()
    codes, scales, ts, y = orc.nvfp4_quantize(x)
    seff = np.repeat(_seff(orc, scales, ts), 16, axis=1).astype(np.float64)
    xd = x.astype(np.float64)
    yd = orc.f32_from_bf16(y).astype(np.float64)
    r = np.abs(xd) / seff
    # grid spacing / 2 around |r|: 0.25 up to 2, 0.5 up to 4, 1 up to 6
    half = np.where(r <= 2, 0.25, np.where(r <= 4, 0.5, 1.0))
    bound = seff * half + np.abs(xd) * 2.0**-23 + np.abs(yd) * 2.0**-8
    assert np.all(np.abs(xd - yd) <= bound * (1 + 1e-12))
    # every block's largest element lands on the top of the grid (idx 7)
    idx = (_unpack(codes) & 7).reshape(-1, 16)
    amax_pos = np.argmax(np.abs(x).reshape(-1, 16), axis=1)
    sb = scales.reshape(-1)
    normal = sb >= 0x08
    assert np.all(idx[np.arange(idx.shape[0]), amax_pos][normal] == 7)


def test_frozen_matches_dynamic_and_is_idempotent(orc):
    w, _ = synth.moe_weights_bf16(experts=1, rows=128, cols=512, seed=2, with_grad=False)
    xb = synth.bf16_bits(w[0])
    c0, s0, t0, y0 = orc.nvfp4_quantize(xb)
    # frozen with the dynamic scales reproduces the dynamic result
    c1, s1, t1, y1 = orc.nvfp4_quantize(xb, s0, t0)
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1) and t1 == t0 and np.array_equal(y0, y1)
    # QDQ(QDQ(x)) == QDQ(x) with frozen scales
    c2, _, _, y2 = orc.nvfp4_quantize(y0, s0, t0)
    assert np.array_equal(c2, c0) and np.array_equal(y2, y0)


def test_frozen_scale_saturates(orc):
    # a frozen scale smaller than the dynamic one clips the block maximum to +-6
    x = np.array([[6.0, -6.0, 3.0] + [0.0] * 13], np.float32)
    x[0, 3] = 2688.0  # tensor amax -> tensor scale 1 (dynamic reference)
    scales = np.array([[0x30]], np.uint8)  # 0.5
    codes, _, _, y = orc.nvfp4_quantize(x, scales, 1.0)
    un = _unpack(codes)[0]
    assert un[0] == 7 and un[1] == 15 and un[2] == 7 and un[3] == 7
    assert orc.f32_from_bf16(y)[0, :4].tolist() == [3.0, -3.0, 3.0, 3.0]


def test_bf16_input_config_like(orc):
    # activations with heavy tails: every code's magnitude is consistent with
    # |x| / s_eff within the grid's rounding intervals
    xb, _ = synth.student_t_activations_bf16(tokens=64, hidden=512, seed=3, with_grad=False)
    bits = synth.bf16_bits(xb)
    codes, scales, ts, y = orc.nvfp4_quantize(bits)
    x = orc.f32_from_bf16(bits).astype(np.float64)
    seff = np.repeat(_seff(orc, scales, ts), 16, axis=1).astype(np.float64)
    r = np.abs(x) / seff
    idx = _unpack(codes) & 7
    lo = np.array([0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])[idx]
    hi = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, np.inf])[idx]
    eps = 2.0**-23
    assert np.all(r >= lo * (1 - eps)) and np.all(r <= hi * (1 + eps))
    sign = (_unpack(codes) >> 3).astype(bool)
    assert np.array_equal(sign, np.signbit(orc.f32_from_bf16(bits)))
