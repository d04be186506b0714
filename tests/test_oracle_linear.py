"""Pins of the oracle's W4A4 fake-quant linear layer.

Page 'Model-Optimizer 实战 ... W4A4 NVFP4 精度' (nlpx.cn), section '3. QAD': the
student is the W4A4 NVFP4 model (weights and activations NVFP4).  The oracle
is the NVFP4 QDQ oracle (pinned in test_oracle_nvfp4.py) applied to both
operands, followed by a binary64 matrix product.

Pins: a hand-derived product; exact power-of-two equivariance of the whole
layer (scaling w by 2 doubles every tensor and block scale exactly, so y
doubles exactly); the backward as the transposed products, checked against
central finite differences of sum(y * grad_y) through the straight-through
estimator (the QDQ outputs held fixed).
"""
import numpy as np

from nvfp4_quantization_aware_amd import synth


def test_hand_derived_product(orc):
    # 16 ones: amax 1, s_g = 1/2688, block scale E4M3(448) = 448, s_eff = 1/6,
    # 1/(1/6) = 6 -> code 6 -> y = 6 * (1/6) = 1: QDQ is exact, y = 16
    x = np.ones((1, 16), np.float32)
    w = np.ones((1, 16), np.float32)
    y, xq, wq = orc.w4a4_linear_fwd(x, w)
    assert y.shape == (1, 1) and y[0, 0] == 16.0
    assert np.all(xq == 0x3F80) and np.all(wq == 0x3F80)


def test_power_of_two_equivariance(orc):
    x = synth.bf16_bits(synth.gaussian_weight_bf16(24, 64, seed=7))
    w = synth.bf16_bits(synth.gaussian_weight_bf16(12, 64, seed=8))
    y1, _, _ = orc.w4a4_linear_fwd(x, w)
    w2 = ((w.astype(np.uint32) + (1 << 7)) & 0xFFFF).astype(np.uint16)   # exponent + 1: w * 2 (no zeros here)
    assert np.array_equal((w2.astype(np.uint32) << 16).view(np.float32), 2 * (w.astype(np.uint32) << 16).view(np.float32))
    y2, _, _ = orc.w4a4_linear_fwd(x, w2)
    assert np.array_equal(y2, 2 * y1)


def test_backward_is_the_transposed_products(orc):
    rng = np.random.default_rng(3)
    x = synth.bf16_bits(synth.gaussian_weight_bf16(8, 32, seed=1))
    w = synth.bf16_bits(synth.gaussian_weight_bf16(5, 32, seed=2))
    _, xq, wq = orc.w4a4_linear_fwd(x, w)
    gy = synth.bf16_bits(synth.gaussian_weight_bf16(8, 5, seed=3))
    gx, gw = orc.w4a4_linear_bwd(gy, xq, wq)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xf, wf, gf = f(xq), f(wq), f(gy)
    loss = lambda a, b: np.sum((a @ b.T) * gf)
    h = 2.0 ** -12
    for (i, k) in [(0, 0), (3, 17), (7, 31)]:
        e = np.zeros_like(xf); e[i, k] = h
        assert abs((loss(xf + e, wf) - loss(xf - e, wf)) / (2 * h) - gx[i, k]) < 1e-9
    for (j, k) in [(0, 0), (4, 9)]:
        e = np.zeros_like(wf); e[j, k] = h
        assert abs((loss(xf, wf + e) - loss(xf, wf - e)) / (2 * h) - gw[j, k]) < 1e-9


def test_frozen_weight_scales_compose(orc):
    # with frozen weight scales the weight operand is exactly the frozen QDQ
    # of w (which the NVFP4 pins cover) and the product changes accordingly
    x = synth.bf16_bits(synth.gaussian_weight_bf16(6, 64, seed=4))
    w = synth.bf16_bits(synth.gaussian_weight_bf16(5, 64, seed=5))
    sc, ts = orc.mse_calibrate(w)
    y, xq, wq = orc.w4a4_linear_fwd(x, w, sc, ts)
    assert np.array_equal(wq, orc.nvfp4_quantize(w, sc, ts)[3])
    assert np.array_equal(xq, orc.nvfp4_quantize(x)[3])
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(y, f(xq) @ f(wq).T)
    yd, _, wqd = orc.w4a4_linear_fwd(x, w)
    assert not np.array_equal(wqd, wq)   # the calibrated scales differ from the dynamic ones here
