"""Pins of the oracle's clipped straight-through backward.

Page '使用量化感知蒸馏技术构建Nemotron 3.5 Lightning NVFP4模型' (163.com),
section '量化尺度处理策略': with frozen scales only the weights train.  The
pages print no clipping rule; the reading is that the gradient passes where
|x| <= 6 * s_eff exactly (the range the block can represent), with s_eff the
forward's binary32 effective scale, and is +0 where the quantizer saturates.

Pins: a hand-derived fixture (tests/golden/clipped_ste_worked_example.json)
whose fp32 tensor puts elements between 6 * s_eff and its binary32 rounding,
so a comparison against the rounded product fails it; the decision against
exact rational arithmetic on elements straddling the limit; agreement with
the oracle's own quantizer (every clipped element is coded at the top of the
E2M1 grid, and where 6 * s_eff is exact in bf16 the forward output of a
clipped element is exactly +-6 * s_eff); passthrough bit for bit in every
dtype combination, -0 included.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from nvfp4_quantization_aware_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def u32(h):
    return np.array([int(v, 16) for v in h], np.uint32)


def bf16_of(vals):
    f = np.asarray(vals, np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), f), "value not exact in bf16"
    return bits


def test_worked_example_bf16(orc):
    g = json.load(open(os.path.join(GOLDEN, "clipped_ste_worked_example.json")))["A"]
    x = u32(g["x_bits"]).astype(np.uint16)
    gy = bf16_of(g["grad"])
    gx, nc = orc.nvfp4_qdq_bwd_clipped(gy, x, np.array(g["scales"], np.uint8), g["tscale"])
    assert nc == g["n_clipped"]
    assert gx.tolist() == bf16_of(g["grad_x"]).tolist()
    assert ((gx == gy) | (gx == 0)).all()


def test_worked_example_fp32_exact_limit(orc):
    g = json.load(open(os.path.join(GOLDEN, "clipped_ste_worked_example.json")))["B"]
    x = u32(g["x_bits"]).view(np.float32)
    gy = u32(g["grad_bits"]).view(np.float32)
    ts = float(u32([g["tscale_bits"]]).view(np.float32)[0])
    gx, nc = orc.nvfp4_qdq_bwd_clipped(gy, x, np.array(g["scales"], np.uint8), ts)
    assert nc == g["n_clipped"]
    assert gx.view(np.uint32).tolist() == u32(g["grad_x_bits"]).tolist()


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_exact_rational_limit(orc, seed):
    # elements placed on and around the binary32 neighbours of 6 * s_eff for
    # random codes and tensor scales; decide each with exact rationals
    rng = np.random.default_rng(seed)
    nb = 64
    codes = rng.integers(0, 127, nb).astype(np.uint8)
    s_g = np.float32(rng.uniform(0.5, 2.0)) * np.float32(2.0) ** np.float32(rng.integers(-20, 20))
    s_g = np.float32(s_g)
    dec = np.array([orc.e4m3_decode(c) for c in codes], np.float32)
    s_eff = (dec * s_g).astype(np.float32)         # one binary32 product each
    x = np.empty((nb, 16), np.float32)
    for b in range(nb):
        c = np.float32(np.float32(6.0) * s_eff[b])
        pts = [c]
        for _ in range(3):
            pts.append(np.nextafter(pts[-1], np.float32(np.inf)))
        lo = [c]
        for _ in range(3):
            lo.append(np.nextafter(lo[-1], np.float32(0)))
        vals = pts + lo[1:] + [np.float32(0), np.float32(-0.0), np.float32(1e-30), np.float32(1e30)]
        vals = vals + [-v for v in vals[:16 - len(vals)]]
        x[b] = np.array(vals[:16], np.float32)
    gy = rng.standard_normal((nb, 16)).astype(np.float32)
    gx, nc = orc.nvfp4_qdq_bwd_clipped(gy.ravel(), x.ravel(), codes, float(s_g))
    gx = gx.reshape(nb, 16)
    clipped = 0
    for b in range(nb):
        lim = 6 * Fraction(float(s_eff[b]))
        for j in range(16):
            ok = abs(Fraction(float(x[b, j]))) <= lim
            clipped += not ok
            want = gy[b, j] if ok else np.float32(0)
            assert gx[b, j].view(np.uint32) == np.float32(want).view(np.uint32), (b, j)
    assert nc == clipped and clipped > 0


def test_agrees_with_quantizer_saturation(orc):
    # dynamic scales from the oracle's own forward on Student-t activations:
    # a clipped element is coded at the top of the E2M1 grid; where 6*s_eff is
    # exact in bf16 its forward output is exactly +-6*s_eff
    x = synth.student_t_activations_bf16(64, 256, seed=7)[0]
    xb = synth.bf16_bits(x).ravel()
    codes, scales, ts, y = orc.nvfp4_quantize(xb.reshape(64, 256))
    gy = np.ones(xb.size, np.float32)
    gx, nc = orc.nvfp4_qdq_bwd_clipped(gy, xb, scales.ravel(), ts)
    nib = np.empty(xb.size, np.uint8)
    nib[0::2] = codes.ravel() & 15
    nib[1::2] = codes.ravel() >> 4
    clipped = gx == 0
    assert nc == int(clipped.sum()) and nc > 0
    assert ((nib[clipped] & 7) == 7).all()
    dec = np.array([orc.e4m3_decode(c) for c in range(128)], np.float32)
    s_eff = (dec[scales.ravel() & 127] * np.float32(ts)).astype(np.float32)
    lim = np.repeat((np.float32(6) * s_eff).astype(np.float32), 16)
    yf = (y.ravel().astype(np.uint32) << 16).view(np.float32)
    exact = (torch.from_numpy(lim).to(torch.bfloat16).float().numpy() == lim)
    sel = clipped & exact
    assert sel.any()
    assert np.array_equal(np.abs(yf[sel]), lim[sel])
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    assert (np.abs(xf[sel]) > lim[sel]).all()


@pytest.mark.parametrize("gt", ["bf16", "fp32"])
@pytest.mark.parametrize("xt", ["bf16", "fp32"])
def test_passthrough_bits_all_dtypes(orc, gt, xt):
    rng = np.random.default_rng(11)
    n = 16 * 40
    xf = (rng.standard_normal(n) * 3).astype(np.float32)
    xf[::7] = -0.0
    gf = rng.standard_normal(n).astype(np.float32)
    gf[::5] = -0.0
    x = bf16_of((xf.view(np.uint32) & 0xFFFF0000).view(np.float32)) if xt == "bf16" else xf
    gy = bf16_of((gf.view(np.uint32) & 0xFFFF0000).view(np.float32)) if gt == "bf16" else gf
    scales = np.full(n // 16, 0x38, np.uint8)        # s_eff = 1, limit 6
    gx, nc = orc.nvfp4_qdq_bwd_clipped(gy, x, scales, 1.0)
    xv = (x.astype(np.uint32) << 16).view(np.float32) if xt == "bf16" else x
    keep = np.abs(xv) <= 6
    assert nc == int((~keep).sum()) and nc > 0
    assert np.array_equal(gx[keep], gy[keep])
    assert (gx[~keep] == 0).all() and not np.signbit(gx[~keep].astype(np.float32)).any()
    assert gx.dtype == gy.dtype


def test_size_mismatch_rejected(orc):
    with pytest.raises(ValueError):
        orc.nvfp4_qdq_bwd_clipped(np.zeros(32, np.float32), np.zeros(16, np.float32), np.zeros(1, np.uint8), 1.0)
