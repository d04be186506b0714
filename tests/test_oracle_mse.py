"""Pins of the oracle's MSE scale calibration (frozen-scale variant).

Page '使用量化感知蒸馏技术构建Nemotron 3.5 Lightning NVFP4模型' (163.com),
section '量化尺度处理策略': frozen-scale QAD starts from MSE-calibrated scales,
because the MSE scale search is too costly to repeat every step.  Candidates
are amax*k/6 for 64 values of k spread over [0.5, 1].

Pins: the k grid against exact rationals; a hand-derived block
(tests/golden/mse_worked_block.json); the selection rule against the full
candidate table; an MSE computed independently in binary64 from the chosen
codes; and the exhaustive premise that lets a search visit only the distinct
E4M3 codes (they form a contiguous, non-decreasing run in k).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from nvfp4_quantization_aware_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _nearest_f32(q: Fraction) -> np.float32:
    f = np.float32(float(q))
    best = f
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d, db = abs(Fraction(float(c)) - q), abs(Fraction(float(best)) - q)
        if d < db or (d == db and (int(np.float32(c).view(np.uint32)) & 1) == 0):
            best = c
    return best


def test_kgrid_exact(orc):
    k = orc.mse_kgrid(64, 0.5, 1.0)
    for i in range(64):
        assert k[i] == _nearest_f32(Fraction(63 + i, 126)), i
    assert k[0] == 0.5 and k[-1] == 1.0


def test_worked_block(orc):
    g = json.load(open(os.path.join(GOLDEN, "mse_worked_block.json")))
    blk = np.array(g["block"], np.float32)
    sc, err, cc, ce = orc.mse_calibrate_blocks(blk, g["tscale"], detail=True)
    assert sc[0] == g["best_scale"] and err[0] == g["best_err"]
    for code, e in g["err_by_code"].items():
        sel = cc[0] == int(code)
        assert sel.any() and np.all(ce[0][sel] == e)
    assert cc[0].min() == 0x30 and cc[0].max() == 0x38


def test_selection_is_first_minimum(orc):
    w = synth.gaussian_weight_bf16(rows=32, cols=256, seed=4)
    x = orc.f32_from_bf16(synth.bf16_bits(w)).reshape(-1, 16)
    s_g = orc.tensor_scale(orc.amax(x))
    sc, err, cc, ce = orc.mse_calibrate_blocks(x, s_g, detail=True)
    first = np.argmin(ce, axis=1)
    assert np.array_equal(sc, cc[np.arange(len(sc)), first])
    assert np.array_equal(err, ce.min(axis=1))
    # k = 1 (the last candidate) is the dynamic scale; calibration never loses to it
    assert np.all(err <= ce[:, -1])


def test_tensor_calibration_matches_blockwise(orc):
    w = synth.gaussian_weight_bf16(rows=64, cols=128, seed=4)
    bits = synth.bf16_bits(w)
    scales, ts = orc.mse_calibrate(bits)
    assert ts == orc.tensor_scale(orc.amax(bits))
    sc, _ = orc.mse_calibrate_blocks(orc.f32_from_bf16(bits).reshape(-1, 16), ts)
    assert np.array_equal(scales.reshape(-1), sc)


def _mse64(orc, x, scales, ts):
    """Block MSE in binary64 from the frozen quantizer's codes."""
    codes, _, _, _ = orc.nvfp4_quantize(x.reshape(1, -1), scales.reshape(1, -1), ts)
    c = np.stack([codes & 0xF, codes >> 4], -1).reshape(-1)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    val = np.where(c & 8, -1.0, 1.0) * grid[c & 7]
    seff = np.repeat(orc.e4m3_decode_table()[scales.reshape(-1)].astype(np.float64) * ts, 16)
    d = x.reshape(-1).astype(np.float64) - val * seff
    return (d * d).reshape(-1, 16).sum(1)


def test_calibrated_beats_dynamic_in_binary64(orc):
    w = synth.gaussian_weight_bf16(rows=64, cols=512, seed=4)
    bits = synth.bf16_bits(w)
    x = orc.f32_from_bf16(bits)
    cal, ts = orc.mse_calibrate(bits)
    _, dyn, ts2, _ = orc.nvfp4_quantize(bits)
    assert ts == ts2
    e_cal = _mse64(orc, x, cal, ts)
    e_dyn = _mse64(orc, x, dyn, ts)
    assert np.all(e_cal <= e_dyn * (1 + 1e-5) + 1e-30)
    assert e_cal.sum() < e_dyn.sum()
    # and the scales differ somewhere: the search is not a no-op
    assert np.count_nonzero(cal != dyn) > 0


def test_exact_block_has_zero_error(orc):
    # [a, 0, ...] with a = 6 * 2^m * s_g is represented exactly at k = 1
    for m in (-5, 0, 3):
        s_g = 0.125
        a = 6.0 * 2.0**m * s_g
        blk = np.array([a] + [0.0] * 15, np.float32)
        sc, err = orc.mse_calibrate_blocks(blk, s_g)
        assert err[0] == 0.0 and orc.e4m3_decode(int(sc[0])) * s_g * 6 == a


@pytest.mark.parametrize("s_g", [1.0, 3.7e-5, 2.0**-20, 0.0625 / 3.0])
def test_candidate_codes_contiguous_for_every_bf16_amax(orc, s_g):
    # every positive finite bf16 magnitude as a block amax
    h = np.arange(1, 0x7F80, dtype=np.uint16)
    a = orc.f32_from_bf16(h)
    blocks = np.zeros((a.size, 16), np.float32)
    blocks[:, 0] = a
    _, _, cc, _ = orc.mse_calibrate_blocks(blocks, np.float32(s_g), detail=True)
    step = np.diff(cc.astype(np.int32), axis=1)
    assert step.min() >= 0 and step.max() <= 1
    span = cc[:, -1].astype(np.int32) - cc[:, 0].astype(np.int32) + 1
    assert span.max() <= 9
