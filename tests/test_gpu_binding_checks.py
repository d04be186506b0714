"""The binding checks every tensor argument before its pointer reaches the
library: a caller's output of the wrong size, dtype or layout, a teacher and
student of different dtypes or a workspace that is not bytes raise in Python
and launch nothing (the library could not tell a short buffer from a good
one).  A valid call after the rejected ones still gives the right result.
"""
import pytest
import torch

import nvfp4_quantization_aware_amd as q
from gpu_util import announce, gpu_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


def test_binding_rejects_bad_arguments(dev):
    announce("binding argument checks")
    bf = torch.bfloat16
    x = torch.randn(4, 64, 256, device=dev).to(bf)
    t = torch.randn(8, 1024, device=dev).to(bf)
    s = torch.randn(8, 1024, device=dev).to(bf)
    bad = [
        (lambda: q.nvfp4_qdq_fwd(x, y=torch.empty(4, 64, 128, dtype=bf, device=dev)), "y must hold"),
        (lambda: q.nvfp4_qdq_fwd(x, y=torch.empty(4, 64, 256, device=dev)), "y must be"),
        (lambda: q.nvfp4_quantize(x, codes=torch.empty(4, 64, 128, dtype=bf, device=dev)), "codes must be"),
        (lambda: q.nvfp4_quantize(x, scales_out=torch.empty(4, 64, 8, dtype=torch.uint8, device=dev)),
         "scales_out must hold"),
        (lambda: q.nvfp4_quantize(x, ws=torch.empty(1 << 20, device=dev)), "ws must be"),
        (lambda: q.nvfp4_qdq_fwd(x.transpose(1, 2)), "x must be contiguous"),
        (lambda: q.nvfp4_qdq_fwd(x, torch.zeros(4 * 64 * 16, dtype=torch.uint8, device=dev),
                                 torch.ones(3, device=dev)), "tscale_in must hold"),
        (lambda: q.nvfp4_qdq_bwd(x, torch.empty(4, 64, 256, device=dev)), "grad_x must be"),
        (lambda: q.nvfp4_qdq_bwd_clipped(x, x, torch.zeros(10, dtype=torch.uint8, device=dev),
                                         torch.ones(4, device=dev)), "scales"),
        (lambda: q.nvfp4_mse_calibrate(x, tscale_out=torch.empty(3, device=dev)), "tscale_out must hold"),
        (lambda: q.fp8_quantize(x, y=torch.empty(10, dtype=bf, device=dev)), "y must hold"),
        (lambda: q.qad_kl_fwd_bwd(t, s.float()), "student must be"),
        (lambda: q.qad_kl_fwd_bwd(t, s, grad=torch.empty(1024, 8, dtype=bf, device=dev).t()), "grad must be"),
        (lambda: q.qad_kl_fwd_bwd(t, s, row_loss=torch.empty(7, device=dev)), "row_loss must hold"),
        (lambda: q.qad_kl_topk_fwd_bwd(t, s, 10, loss_out=torch.empty(1, dtype=bf, device=dev)), "loss_out must be"),
        (lambda: q.qad_kl_topp_fwd_bwd(t, s, 0.9, tau=torch.empty(9, device=dev)), "tau must hold"),
        (lambda: q.qad_w4a4_linear_fwd(t, s, y=torch.empty(4, 8, dtype=bf, device=dev)), "y must hold"),
        (lambda: q.qad_w4a4_linear_bwd(torch.empty(16, dtype=bf, device=dev), torch.empty(16, dtype=torch.uint8,
                                                                                            device=dev),
                                       torch.empty(16, dtype=torch.uint8, device=dev), 16), "grad_y \\[M, N\\]"),
        (lambda: q.qad_w4a4_linear_bwd(torch.empty(8, 16, dtype=bf, device=dev), torch.empty(5, dtype=torch.uint8,
                                                                                               device=dev),
                                       torch.empty(5, dtype=torch.uint8, device=dev), 32), "xq must hold"),
        (lambda: q.qad_check_finite(torch.zeros(3, dtype=bf, device=dev)), "values must be"),
    ]
    for i, (f, msg) in enumerate(bad):
        with pytest.raises(ValueError, match=msg):
            f()
    # a valid call still works: QDQ of a constant tensor is the constant
    c = torch.full((2, 32), 3.0, device=dev)
    y = q.nvfp4_qdq_fwd(c)
    torch.cuda.synchronize()
    assert torch.equal(y.float(), c)
