"""GPU parity of the W4A4 fake-quant linear layer (qad_w4a4_linear_fwd/_bwd).

The packed operands xq, wq (E2M1 codes, E4M3 block scales, tensor scale) must
equal the oracle's NVFP4 quantization of x and w bit for bit (dynamic
scales, or for w frozen MSE-calibrated scales).  The products -- computed by
the library's MFMA kernel from those packed operands -- are bf16 values of
fp32-accumulated sums of the bf16 QDQ values' products, compared with the
binary64 oracle product of the oracle's QDQ values within the bound that
arithmetic allows: half a bf16 ulp of the result plus 2 K 2^-24 sum_k
|a_k b_k| (fp32 rounding of up to K products and partial sums in any order).
Shapes span several 256 x 256 (forward) and 256 x 128 (backward) tiles of
64-deep steps with ragged edges in every dimension, each of the kernel's
three load forms, rows whose lengths break 16-byte alignment (bf16 grad_y
with N % 8 != 0), single elements, and one MoE expert's projection
8192 x 2048 x 4096 compared in full.
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


def check_packed(orc, packed, xh, R, C, scales_in=None, tscale_in=None):
    """The packed operand equals the oracle's quantization of xh, part by part."""
    codes, scales, ts = q.nvfp4_unpack(packed, R, C)
    if scales_in is None:
        rc, rs, rt, _ = orc.nvfp4_quantize(xh)
    else:
        rc, rs, rt, _ = orc.nvfp4_quantize(xh, scales_in, tscale_in)
    assert np.array_equal(host(codes), rc.reshape(R, C // 2))
    assert np.array_equal(host(scales), rs.reshape(R, C // 16))
    assert host(ts)[0].view(np.uint32) == np.float32(rt).view(np.uint32)


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
    gx, gw = q.qad_w4a4_linear_bwd(gy.to(dev), xq, wq, K)
    torch.cuda.synchronize()
    check_packed(orc, xq, host(x), M, K)
    check_packed(orc, wq, host(w), N, K, ws_in, wt_in)
    yr, xqr, wqr = orc.w4a4_linear_fwd(host(x), host(w), ws_in, wt_in)
    xf, wf, gf = f64(xqr), f64(wqr), f64(host(gy))
    assert_product_close(host(y), yr, np.abs(xf) @ np.abs(wf).T, K, "y")
    gxr, gwr = orc.w4a4_linear_bwd(host(gy), xqr, wqr)
    assert_product_close(host(gx), gxr, np.abs(gf) @ np.abs(wf), N, "grad_x")
    assert_product_close(host(gw), gwr, np.abs(gf).T @ np.abs(xf), M, "grad_w")


# Each product takes one of three load forms, chosen per launch: whole tiles
# (M % 256, N % tile, K % 64 all 0, e.g. 256 x 512 x 1024), aligned rows
# (K % 32 == 0 for the NVFP4 operands, N % 8 or N % 4 for the bf16
# gradient, e.g. 64 x 32 x 128), or element by element (e.g. 37 x 19 x 48,
# 300 x 260 x 208 with K % 32 = 16).
@pytest.mark.parametrize("M,N,K,dtype", [(64, 32, 128, torch.bfloat16), (37, 19, 48, torch.float32),
                                         (256, 512, 1024, torch.bfloat16), (1, 1, 16, torch.bfloat16),
                                         (300, 260, 208, torch.bfloat16), (129, 131, 80, torch.float32),
                                         (200, 136, 4112, torch.bfloat16), (512, 768, 320, torch.bfloat16)])
def test_linear_small(dev, orc, M, N, K, dtype):
    run_case(dev, orc, M, N, K, dtype, seed=M + N + K)


# 256-wide forward tiles (at least 256 of them) in the two load forms other
# than whole tiles: a ragged last tile row (M = 8200, aligned rows) and rows
# of K % 32 = 16 (element by element)
@pytest.mark.parametrize("M,N,K", [(8200, 2048, 4096), (8192, 2048, 4112)])
def test_linear_wide_tiles_ragged(dev, orc, M, N, K):
    run_case(dev, orc, M, N, K, torch.bfloat16, seed=M + K)


@pytest.mark.parametrize("M,N,K,dtype", [(64, 32, 128, torch.bfloat16), (40, 24, 256, torch.float32)])
def test_linear_frozen_weight_scales(dev, orc, M, N, K, dtype):
    run_case(dev, orc, M, N, K, dtype, seed=7 * M + N, frozen=True)


def test_linear_expert_shape_full(dev, orc):
    # one MoE expert's projection: 8192 tokens x 4096 -> 2048 (the weight
    # shape of the MoE workload), every element of y, grad_x and grad_w
    # against the binary64 products of the oracle's QDQ values
    M, N, K = 8192, 2048, 4096
    announce("linear 8192x2048x4096 generate")
    x, _ = synth.student_t_activations_bf16(M, K, seed=3, device=dev)
    w = synth.moe_weights_bf16(experts=1, rows=N, cols=K, seed=2, device=dev, with_grad=False)[0][0]
    announce("qad_w4a4_linear_fwd 8192x2048x4096")
    y, xq, wq = q.qad_w4a4_linear_fwd(x, w)
    gy = (torch.randn((M, N), device=dev) * 1e-3).to(torch.bfloat16)
    gx, gw = q.qad_w4a4_linear_bwd(gy, xq, wq, K)
    torch.cuda.synchronize()
    check_packed(orc, xq, host(x), M, K)
    check_packed(orc, wq, host(w), N, K)
    xf = f64(orc.nvfp4_quantize(host(x))[3].reshape(M, K))
    wf = f64(orc.nvfp4_quantize(host(w))[3].reshape(N, K))
    gf = f64(host(gy))
    assert_product_close(host(y), xf @ wf.T, np.abs(xf) @ np.abs(wf).T, K, "y")
    assert_product_close(host(gx), gf @ wf, np.abs(gf) @ np.abs(wf), N, "grad_x")
    assert_product_close(host(gw), gf.T @ xf, np.abs(gf).T @ np.abs(xf), M, "grad_w")
