"""Empty inputs through every entry point: no error, outputs of the right
(empty) shapes, and the values that are still defined -- the tensor scale of
an empty tensor is the zero tensor's (1.0) or the frozen one given, as in the
oracle; the amax of an empty tensor is 0; the KL losses of zero rows are 0;
the W4A4 backward with M or N == 0 gives an all-zero other gradient.
"""
import numpy as np
import pytest
import torch

import nvfp4_quantization_aware_amd as q
from gpu_util import announce, gpu_device, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


def test_empty_quantizers(dev, orc):
    announce("empty tensors: quantize, QDQ, FP8, MSE, amax, STE")
    bf = torch.bfloat16
    x = torch.empty((3, 0, 64), dtype=bf, device=dev)
    codes, scales, ts, y = q.nvfp4_quantize(x)
    torch.cuda.synchronize()
    assert codes.shape == (3, 0, 32) and scales.shape == (3, 0, 4) and y.shape == (3, 0, 64)
    ref_ts = orc.nvfp4_quantize(np.zeros((0, 64), np.float32))[2]
    assert ref_ts == 1.0 and host(ts).tolist() == [ref_ts] * 3
    frozen = torch.tensor([0.5, 0.25, 2.0], device=dev)
    _, _, ts_f, _ = q.nvfp4_quantize(x, torch.empty((3, 0, 4), dtype=torch.uint8, device=dev), frozen)
    c8, t8, y8 = q.fp8_quantize(torch.empty((2, 0, 16), device=dev))
    _, t8f, _ = q.fp8_quantize(torch.empty((2, 0, 16), device=dev), torch.tensor([3.0, 0.125], device=dev))
    sc, tsm = q.nvfp4_mse_calibrate(torch.empty((2, 0, 32), dtype=bf, device=dev))
    am = q.nvfp4_amax(torch.empty((4, 0, 16), dtype=bf, device=dev))
    gx = q.nvfp4_qdq_bwd(torch.empty(0, dtype=bf, device=dev))
    gc = q.nvfp4_qdq_bwd_clipped(x, x, torch.empty((3, 0, 4), dtype=torch.uint8, device=dev), frozen)
    yq = q.nvfp4_qdq_fwd(torch.empty((0, 128), device=dev))
    torch.cuda.synchronize()
    assert host(ts_f).tolist() == [0.5, 0.25, 2.0]
    assert orc.nvfp4_quantize(np.zeros((0, 64), np.float32), np.zeros((0, 4), np.uint8), 0.25)[2] == 0.25
    assert c8.shape == (2, 0, 16) and y8.shape == (2, 0, 16)
    assert host(t8).tolist() == [orc.fp8_quantize(np.zeros((0, 16), np.float32))[1]] * 2 == [1.0, 1.0]
    assert host(t8f).tolist() == [3.0, 0.125]
    assert sc.shape == (2, 0, 2) and host(tsm).tolist() == [orc.mse_calibrate(np.zeros((0, 32), np.float32))[1]] * 2
    assert host(am).tolist() == [0.0] * 4
    assert gx.numel() == 0 and gc.shape == x.shape and yq.shape == (0, 128)


@pytest.mark.parametrize("fn", ["kl", "topk", "topp"])
def test_empty_kl(dev, fn):
    announce("empty KL (%s): zero token rows" % fn)
    t = torch.empty((0, 1024), dtype=torch.bfloat16, device=dev)
    if fn == "kl":
        out = q.qad_kl_fwd_bwd(t, t, row_loss=True)
    elif fn == "topk":
        out = q.qad_kl_topk_fwd_bwd(t, t, 10, row_loss=True)
    else:
        out = q.qad_kl_topp_fwd_bwd(t, t, 0.9, row_loss=True, tau=True)
    torch.cuda.synchronize()
    assert float(out[0].item()) == 0.0
    assert out[1].numel() == 0 and out[2].shape == (0, 1024)


def assert_packed_is_quantization(packed, x):
    # the packed operand holds the codes, block scales and tensor scale that
    # nvfp4_quantize gives for the same tensor
    R, C = x.shape
    codes, scales, ts = q.nvfp4_unpack(packed, R, C)
    rc, rs, rt, _ = q.nvfp4_quantize(x, y=False)
    assert torch.equal(codes.reshape(-1), rc.reshape(-1)) and torch.equal(scales.reshape(-1), rs.reshape(-1))
    assert torch.equal(ts.reshape(-1), rt.reshape(-1))


def test_empty_linear(dev):
    announce("empty W4A4 linear: M = 0 and N = 0")
    bf = torch.bfloat16
    w = torch.randn(32, 64, device=dev).to(bf)
    y, xq, wq = q.qad_w4a4_linear_fwd(torch.empty((0, 64), dtype=bf, device=dev), w)
    gx, gw = q.qad_w4a4_linear_bwd(torch.empty((0, 32), dtype=bf, device=dev), xq, wq, 64)
    x = torch.randn(16, 64, device=dev).to(bf)
    y2, xq2, wq2 = q.qad_w4a4_linear_fwd(x, torch.empty((0, 64), dtype=bf, device=dev))
    gx2, gw2 = q.qad_w4a4_linear_bwd(torch.empty((16, 0), dtype=bf, device=dev), xq2, wq2, 64)
    torch.cuda.synchronize()
    assert y.shape == (0, 32) and gx.shape == (0, 64) and gw.shape == (32, 64)
    assert torch.count_nonzero(gw).item() == 0
    assert_packed_is_quantization(wq, w)
    assert y2.shape == (16, 0) and gw2.shape == (0, 64) and gx2.shape == (16, 64)
    assert torch.count_nonzero(gx2).item() == 0
    assert_packed_is_quantization(xq2, x)
