"""GPU parity of the W4A4 fake-quant linear layer (qad_w4a4_linear_fwd/_bwd).

The quantized operands xq, wq must equal the oracle's NVFP4 QDQ outputs bit
for bit (dynamic scales, or for w frozen MSE-calibrated scales).  The products are bf16 values of fp32-accumulated sums, compared with
the binary64 oracle product within the bound that arithmetic allows: half a
bf16 ulp of the result plus 2 K 2^-24 sum_k |a_k b_k| (fp32 rounding of up to
K products and partial sums in any order).
"""
import numpy as np
import pytest
import torch

import nvfp4_quantization_aware_amd as q
from nvfp4_quantization_aware_amd import synth
from gpu_util import announce, bf16_ulp, gpu_device, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


def f64(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_product_close(got_bits, ref, absprod, K, label):
    got = f64(got_bits)
    bound = 0.5 * bf16_ulp(np.abs(ref)) + 2 * K * 2.0**-24 * absprod
    bad = np.abs(got - ref) > bound
    assert not bad.any(), (label, np.argwhere(bad)[:3], (np.abs(got - ref) - bound).max())


def run_case(dev, orc, M, N, K, dtype, seed, frozen=False):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn((M, K), generator=g) * 2).to(dtype)
    w = (torch.randn((N, K), generator=g) * 0.05).to(dtype)
    gy = (torch.randn((M, N), generator=g) * 1e-3).to(torch.bfloat16)
    ws_in = wt_in = None
    if frozen:   # the oracle's MSE-calibrated weight scales, frozen
        sc, ts = orc.mse_calibrate(host(w))
        ws_in, wt_in = sc, ts
    announce("qad_w4a4_linear_fwd/bwd M=%d N=%d K=%d %s frozen=%s" % (M, N, K, dtype, frozen))
    if frozen:
        y, xq, wq = q.qad_w4a4_linear_fwd(x.to(dev), w.to(dev), w_scales_in=torch.from_numpy(sc).to(dev),
                                          w_tscale_in=torch.tensor([ts], dtype=torch.float32, device=dev))
    else:
        y, xq, wq = q.qad_w4a4_linear_fwd(x.to(dev), w.to(dev))
    gx, gw = q.qad_w4a4_linear_bwd(gy.to(dev), xq, wq)
    torch.cuda.synchronize()
    yr, xqr, wqr = orc.w4a4_linear_fwd(host(x), host(w), ws_in, wt_in)
    assert np.array_equal(host(xq), xqr) and np.array_equal(host(wq), wqr)
    xf, wf, gf = f64(xqr), f64(wqr), f64(host(gy))
    assert_product_close(host(y), yr, np.abs(xf) @ np.abs(wf).T, K, "y")
    gxr, gwr = orc.w4a4_linear_bwd(host(gy), xqr, wqr)
    assert_product_close(host(gx), gxr, np.abs(gf) @ np.abs(wf), N, "grad_x")
    assert_product_close(host(gw), gwr, np.abs(gf).T @ np.abs(xf), M, "grad_w")


@pytest.mark.parametrize("M,N,K,dtype", [(64, 32, 128, torch.bfloat16), (37, 19, 48, torch.float32),
                                         (256, 512, 1024, torch.bfloat16), (1, 1, 16, torch.bfloat16)])
def test_linear_small(dev, orc, M, N, K, dtype):
    run_case(dev, orc, M, N, K, dtype, seed=M + N + K)


@pytest.mark.parametrize("M,N,K,dtype", [(64, 32, 128, torch.bfloat16), (40, 24, 256, torch.float32)])
def test_linear_frozen_weight_scales(dev, orc, M, N, K, dtype):
    run_case(dev, orc, M, N, K, dtype, seed=7 * M + N, frozen=True)


def test_linear_expert_shape_sampled(dev, orc):
    # one MoE expert's projection: 8192 tokens x 4096 -> 2048 (the weight shape of the MoE workload)
    M, N, K = 8192, 2048, 4096
    announce("linear 8192x2048x4096 generate")
    x, _ = synth.student_t_activations_bf16(M, K, seed=3, device=dev)
    w = synth.moe_weights_bf16(experts=1, rows=N, cols=K, seed=2, device=dev, with_grad=False)[0][0]
    announce("qad_w4a4_linear_fwd 8192x2048x4096")
    y, xq, wq = q.qad_w4a4_linear_fwd(x, w)
    gy = (torch.randn((M, N), device=dev) * 1e-3).to(torch.bfloat16)
    gx, gw = q.qad_w4a4_linear_bwd(gy, xq, wq)
    torch.cuda.synchronize()
    xqr = orc.nvfp4_quantize(host(x))[3]
    wqr = orc.nvfp4_quantize(host(w))[3]
    assert np.array_equal(host(xq), xqr.reshape(M, K)) and np.array_equal(host(wq), wqr.reshape(N, K))
    rows = [0, 1, 4097, 8191]
    xf, wf = f64(xqr.reshape(M, K)[rows]), f64(wqr.reshape(N, K))
    assert_product_close(host(y)[rows], xf @ wf.T, np.abs(xf) @ np.abs(wf).T, K, "y rows")
    gf = f64(host(gy))
    cols = [0, 100, 4095]
    assert_product_close(host(gx)[rows], gf[rows] @ wf, np.abs(gf[rows]) @ np.abs(wf), N, "grad_x rows")
    xall = f64(xqr.reshape(M, K))
    assert_product_close(host(gw)[:, cols], gf.T @ xall[:, cols], np.abs(gf).T @ np.abs(xall[:, cols]), M, "grad_w cols")
