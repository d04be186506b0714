"""GPU parity of fp8_quantize (FP8 E4M3 per-tensor QDQ) against the oracle.

Codes, tensor scales and bf16 outputs must equal the oracle's bit for bit:
dynamic scales (one pass for tensors that fit on chip, amax pass first for
larger ones) and frozen scales, bf16 and fp32 inputs, ragged tails, signed
zeros, saturation, an all-zero tensor, and the full MoE-weight and
activation shapes on sampled tensors / rows.
"""
import numpy as np
import pytest
import torch

import nvfp4_quantization_aware_amd as q
from nvfp4_quantization_aware_amd import synth
from gpu_util import announce, gpu_device, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


def check_fp8(orc, x, label, tscale=None):
    x3 = x if x.dim() == 3 else x.unsqueeze(0)
    B = x3.shape[0]
    announce("fp8_quantize %s shape=%s dtype=%s frozen=%s" % (label, tuple(x3.shape), x3.dtype, tscale is not None))
    t_in = None if tscale is None else torch.as_tensor(np.asarray(tscale, np.float32), device=x3.device)
    codes, ts, y = q.fp8_quantize(x3, t_in)
    torch.cuda.synchronize()
    xc, cg, tg, yg = host(x3), host(codes), host(ts), host(y)
    for b in range(B):
        rc, rt, ry = orc.fp8_quantize(xc[b], None if tscale is None else float(tscale[b]))
        assert tg[b].view(np.uint32) == np.float32(rt).view(np.uint32), (label, b, tg[b], rt)
        bad = np.argwhere(cg[b] != rc)
        assert bad.size == 0, (label, b, "codes", bad[:5], cg[b][tuple(bad[0])], rc[tuple(bad[0])])
        bad = np.argwhere(yg[b] != ry)
        assert bad.size == 0, (label, b, "y", bad[:5])
    return codes, ts, y


def test_fp8_outlier_fp32(dev, orc):
    x = synth.outlier_tensor_f32(256, 1024, seed=1).to(dev)
    check_fp8(orc, x, "outliers fp32")


@pytest.mark.parametrize("shape,dtype", [((4, 64, 256), torch.bfloat16), ((3, 7, 24), torch.float32),
                                         ((2, 33, 40), torch.bfloat16), ((1, 1, 8), torch.bfloat16)])
def test_fp8_small(dev, orc, shape, dtype):
    g = torch.Generator().manual_seed(sum(shape))
    x = (torch.randn(shape, generator=g) * 3).to(dtype).to(dev)
    check_fp8(orc, x, "small")


def test_fp8_frozen_quotient_overflow(dev, orc):
    # a frozen scale far below the elements: x / s exceeds the binary32 range
    # (the oracle's quotient is inf and saturates to +-448), with the
    # reciprocal division (s = 2^-80) and IEEE division (s = 2^-81)
    x = torch.randn((2, 8, 64), generator=torch.Generator().manual_seed(13)) * 1e30
    x[:, :, ::5] = 3.0e38
    x[:, :, 1::5] = -3.0e38
    x[:, :, 2::5] = -0.0
    x[:, 0, :] = 2.0 ** -75                      # ordinary quotients in the same tensor
    check_fp8(orc, x.to(dev), "frozen overflow", tscale=[2.0 ** -80, 2.0 ** -81])


def test_fp8_frozen_and_saturation(dev, orc):
    g = torch.Generator().manual_seed(8)
    x = (torch.randn((2, 16, 64), generator=g) * 100).to(torch.bfloat16).to(dev)
    check_fp8(orc, x, "frozen", tscale=[0.05, 3.0])     # many values beyond 448 * s: saturate


def test_fp8_zero_and_signed_zero(dev, orc):
    x = torch.zeros((2, 4, 16), dtype=torch.float32)
    x[1, 1, 3] = -0.0
    x[1, 2, 5] = 2.0 ** -140                            # tiny against its own amax
    x[1, 3, 7] = -1.0
    check_fp8(orc, x.to(dev), "zeros")


def test_fp8_tiny_scale(dev, orc):
    # tensor scale below 2^-80: every quotient by IEEE division
    x = (torch.randn((1, 8, 32), generator=torch.Generator().manual_seed(3)) * 2.0**-100).to(torch.float32)
    check_fp8(orc, x.to(dev), "tiny")


def test_fp8_moe_experts_sampled(dev, orc):
    announce("fp8 moe 128x2048x4096 generate")
    w, _ = synth.moe_weights_bf16(seed=2, device=dev, with_grad=False)
    announce("fp8_quantize moe 128x2048x4096")
    codes, ts, y = q.fp8_quantize(w)
    torch.cuda.synchronize()
    for b in (0, 77, 127):
        rc, rt, ry = orc.fp8_quantize(host(w[b]))
        assert host(ts)[b] == np.float32(rt)
        assert np.array_equal(host(codes[b]), rc) and np.array_equal(host(y[b]), ry)


def test_fp8_activation_rows_sampled(dev, orc):
    announce("fp8 activations 32768x4096 generate")
    x, _ = synth.student_t_activations_bf16(32768, 4096, seed=3, device=dev)
    announce("fp8_quantize activations 32768x4096 (amax pass first)")
    codes, ts, y = q.fp8_quantize(x)
    torch.cuda.synchronize()
    xh = host(x)
    rc, rt, _ = orc.fp8_quantize(xh[:1])                 # scale of the whole tensor below
    amax = np.abs((xh.astype(np.uint32) << 16).view(np.float32)).max()
    s = np.float32(amax) / np.float32(448)
    assert host(ts)[0] == s
    rows = [0, 1, 12345, 32767]
    rc, _, ry = orc.fp8_quantize(xh[rows], tscale=float(s))
    assert np.array_equal(host(codes[rows]), rc) and np.array_equal(host(y[rows]), ry)
