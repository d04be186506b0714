"""Pins of the oracle's frozen-scale SGD weight step.

Page '使用量化感知蒸馏技术构建Nemotron 3.5 Lightning NVFP4模型' (163.com):
section '量化尺度处理策略' (with frozen scales only the weights are updated)
and section '训练配置' (constant learning rate, gradient clipping at norm
1.0).  No optimizer is named; the reading is plain SGD with the step
a = fl32(lr * clip_coef) through the clipped straight-through gradient:
w' = w where |w| > 6 s_eff, else round_w(fma32(-a, g, w)).

Pins: a hand-derived fixture (tests/golden/frozen_sgd_step_worked_example.json)
with nearest-even ties, signed zeros, subnormals and two cases where rounding
to binary32 first and then to bf16 differs from rounding the exact value
once; exact rational arithmetic on random steps (numpy's binary32 product for
a, Fraction for the update, its nearest-even binary32 by integer arithmetic
and torch's binary32-to-bf16 rounding), with weights straddling the clip limit; and the
special cases a zero step, a zero block scale (every nonzero weight clipped)
and agreement of the clip decisions with the oracle's clipped backward.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bits(h, dtype):
    v = np.array([int(x, 16) for x in h], np.uint32)
    return v.astype(np.uint16) if dtype == "bf16" else v.view(np.float32)


def _f64(a: np.ndarray) -> np.ndarray:
    return ((a.astype(np.uint32) << 16).view(np.float32) if a.dtype == np.uint16 else a).astype(np.float64)


@pytest.mark.parametrize("name", ["A", "B", "C"])
def test_worked_example(orc, name):
    d = json.load(open(os.path.join(GOLDEN, "frozen_sgd_step_worked_example.json")))
    c = [c for c in d["cases"] if c["name"] == name][0]
    w = _bits(c["w_bits"], c["w_dtype"])
    g = _bits(c["g_bits"], c["g_dtype"])
    out, nc = orc.nvfp4_frozen_sgd_step(w, g, np.array(c["scales"], np.uint8), c["tscale"], c["lr"],
                                        c["clip_coef"])
    want = _bits(c["expected_bits"], c["w_dtype"])
    assert nc == c["n_clipped"]
    got = out.view(np.uint32) if out.dtype == np.float32 else out
    assert got.tolist() == (want.view(np.uint32) if want.dtype == np.float32 else want).tolist()


def _e4m3(code: np.ndarray) -> np.ndarray:
    return torch.from_numpy(code.astype(np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def _round_f32(x: Fraction) -> float:
    """Nearest-even binary32 of an exact nonzero rational (normal or
    subnormal; no overflow in these tests), by integer arithmetic."""
    sign = -1 if x < 0 else 1
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1                                                  # 2^e <= x < 2^(e+1)
    q = Fraction(2) ** (max(e, -126) - 23)                      # spacing of binary32 at x
    n = x / q
    m = n.numerator // n.denominator
    r = n - m
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return sign * float(m * q)


def _exact_step(w, g, scales, s_g, lr, clip, w_bf16):
    """Reference by exact arithmetic, element by element: the expected output
    bits and the mask of clipped weights."""
    a = np.float32(lr) * np.float32(clip)                       # numpy binary32 product
    s_eff = (_e4m3(scales) * np.float32(s_g)).astype(np.float32)  # binary32 product per block
    lim = 6.0 * np.repeat(s_eff.astype(np.float64), 16)         # exact in binary64
    wf, gf = _f64(w), _f64(g)
    clipped = np.abs(wf) > lim
    out = np.empty(w.size, np.float32)
    af = Fraction(float(a))
    for i in range(w.size):
        if clipped[i]:
            out[i] = wf[i]
            continue
        d = Fraction(wf[i]) - af * Fraction(gf[i])
        if d != 0:
            out[i] = _round_f32(d)
        else:   # an exact zero: -0 only when both terms are -0
            neg_w = np.signbit(wf[i])
            neg_p = (gf[i] > 0) or (gf[i] == 0 and not np.signbit(gf[i]))   # sign of -a*g, a > 0
            out[i] = -0.0 if (neg_w and neg_p) else 0.0
    if w_bf16:
        ob = torch.from_numpy(out).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return np.where(clipped, w, ob), clipped
    return np.where(clipped, w.view(np.uint32), out.view(np.uint32)), clipped


@pytest.mark.parametrize("w_bf16,g_bf16", [(True, True), (False, True), (True, False), (False, False)])
def test_random_steps_against_exact_arithmetic(orc, w_bf16, g_bf16):
    rng = np.random.default_rng(11 + 2 * w_bf16 + g_bf16)
    nb = 400
    scales = rng.integers(0x20, 0x48, nb).astype(np.uint8)
    s_g = float(np.float32(rng.uniform(0.01, 2.0)))
    s_eff = np.repeat((_e4m3(scales) * np.float32(s_g)).astype(np.float64), 16)
    # weights spread from far inside to just outside the block's range
    wf = (s_eff * 6.0 * rng.uniform(-1.1, 1.1, nb * 16)).astype(np.float32)
    gf = (rng.standard_normal(nb * 16) * 10.0 ** rng.uniform(-3, 1, nb * 16)).astype(np.float32)
    if w_bf16:
        w = torch.from_numpy(wf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    else:
        w = wf
    g = torch.from_numpy(gf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16) if g_bf16 else gf
    for lr, clip in [(0.013, 0.77), (float(np.float32(1.0 / 3.0)), 1.0), (5e-6, 1.0), (0.25, 0.5)]:
        out, nc = orc.nvfp4_frozen_sgd_step(w, g, scales, s_g, lr, clip)
        want, clipped = _exact_step(w, g, scales, s_g, lr, clip, w_bf16)
        got = out if w_bf16 else out.view(np.uint32)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (lr, clip, bad[:5], got[bad[:5]], want[bad[:5]])
        assert nc == int(clipped.sum()) and 0 < nc < w.size


def test_zero_step_and_zero_scale(orc):
    rng = np.random.default_rng(3)
    w = (rng.standard_normal(256) * 0.5).astype(np.float32)
    w[:4] = [0.0, -0.0, 3.0, -3.0]
    g = rng.standard_normal(256).astype(np.float32)
    sc = np.full(16, 0x38, np.uint8)
    out, nc = orc.nvfp4_frozen_sgd_step(w, g, sc, 1.0, 0.0, 1.0)
    nz = w != 0
    assert np.array_equal(out.view(np.uint32)[nz], w.view(np.uint32)[nz])
    assert nc == int((np.abs(w) > 6.0).sum())
    out, nc = orc.nvfp4_frozen_sgd_step(w, g, sc, 1.0, 1.0, 0.0)
    assert np.array_equal(out.view(np.uint32)[nz], w.view(np.uint32)[nz])
    # block scale 0: the range is {0}; every nonzero weight is clipped and kept
    out, nc = orc.nvfp4_frozen_sgd_step(w, g, np.zeros(16, np.uint8), 1.0, 0.5, 1.0)
    assert nc == int(nz.sum())
    assert np.array_equal(out.view(np.uint32)[nz], w.view(np.uint32)[nz])
    assert np.array_equal(out[~nz], (-np.float32(0.5) * g[~nz]) + 0.0 * w[~nz])


def test_clip_decisions_match_clipped_backward(orc):
    # the step moves exactly the weights whose clipped gradient is passed
    rng = np.random.default_rng(4)
    nb = 512
    sc = rng.integers(0x28, 0x40, nb).astype(np.uint8)
    s_g = 0.37
    s_eff = np.repeat(_e4m3(sc).astype(np.float64) * np.float32(s_g), 16)
    w = torch.from_numpy((s_eff * 6.0 * rng.uniform(-1.05, 1.05, nb * 16)).astype(np.float32))
    w = w.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    g = np.full(nb * 16, 0x3F80, np.uint16)                   # gradient 1 everywhere
    gx, nc_bwd = orc.nvfp4_qdq_bwd_clipped(g, w, sc, s_g)
    out, nc = orc.nvfp4_frozen_sgd_step(w, g, sc, s_g, 2.0 ** -20, 1.0)
    assert nc == nc_bwd
    # a step of 2^-20 moves no bf16 weight of this size, so compare with a
    # step that does: lr large enough to change every passed weight
    out, nc = orc.nvfp4_frozen_sgd_step(w, g, sc, s_g, 1e6, 1.0)
    moved = out != w
    assert np.array_equal(moved, gx != 0)
