"""GPU parity of the NVFP4 entry points against the CPU oracle.

Packed E2M1 codes, E4M3 block scales, FP32 tensor scales, bf16 QDQ outputs
and STE gradients must equal the oracle's bit for bit.  Small cases run the
oracle on the whole tensor (several tiles and a ragged tail); the full-size
workloads run in the benchmark's launch configuration and are checked on
sampled rows/blocks, which the oracle computes one by one once it has the
tensor scale from the whole tensor's amax.
"""
import json
import os

import numpy as np
import pytest
import torch

import nvfp4_quantization_aware_amd as q
from nvfp4_quantization_aware_amd import synth
from gpu_util import announce, gpu_device, host

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


def _as_np_input(x: torch.Tensor) -> np.ndarray:
    return host(x)


def check_quantize(orc, x: torch.Tensor, label: str, frozen=None):
    """Run nvfp4_quantize on x ([B,R,C] or [R,C]) and compare every output
    with the oracle tensor by tensor.  frozen = (scales u8[B,R,C/16], tscale f32[B])."""
    x3 = x if x.dim() == 3 else x.unsqueeze(0)
    B = x3.shape[0]
    announce("nvfp4_quantize %s shape=%s dtype=%s frozen=%s" % (label, tuple(x3.shape), x3.dtype, frozen is not None))
    if frozen is None:
        codes, scales, ts, y = q.nvfp4_quantize(x3)
    else:
        s_in = torch.from_numpy(frozen[0]).to(x3.device)
        t_in = torch.from_numpy(np.asarray(frozen[1], np.float32)).to(x3.device)
        codes, scales, ts, y = q.nvfp4_quantize(x3, s_in, t_in)
    torch.cuda.synchronize()
    xc, cg, sg, tg, yg = host(x3), host(codes), host(scales), host(ts), host(y)
    for b in range(B):
        if frozen is None:
            rc, rs, rt, ry = orc.nvfp4_quantize(xc[b])
        else:
            rc, rs, rt, ry = orc.nvfp4_quantize(xc[b], frozen[0][b], float(frozen[1][b]))
        assert tg[b].view(np.uint32) == np.float32(rt).view(np.uint32), (label, b, tg[b], rt)
        assert np.array_equal(sg[b].reshape(rs.shape), rs), (label, b, "scales")
        bad = np.argwhere(cg[b].reshape(rc.shape) != rc)
        assert bad.size == 0, (label, b, "codes", bad[:5])
        bad = np.argwhere(yg[b].reshape(ry.shape) != ry)
        assert bad.size == 0, (label, b, "y", bad[:5])
    return codes, scales, ts, y


def test_worked_example(dev, orc):
    g = json.load(open(os.path.join(GOLDEN, "nvfp4_worked_example.json")))
    x = torch.tensor(g["x_f32"], dtype=torch.float32, device=dev).reshape(1, g["rows"], g["cols"])
    codes, scales, ts, y = check_quantize(orc, x, "worked-example")
    assert host(codes).reshape(-1).tolist() == g["codes_packed"]
    assert host(scales).reshape(-1).tolist() == g["scales"]


def test_outlier_tensor_fp32_full(dev, orc):
    # fp32 256 x 1024, N(0,1) with 0.1 % outliers x50 -- the whole workload
    x = synth.outlier_tensor_f32(seed=1).to(dev)
    check_quantize(orc, x, "fp32-256x1024")


@pytest.mark.parametrize("dtype,B,R,C,seed", [
    ("bf16", 3, 7, 48, 11),      # ragged: 42 units per tensor
    ("fp32", 2, 5, 16, 12),
    ("bf16", 1, 1, 16, 13),      # a single block
    ("fp32", 1, 333, 80, 14),
    ("bf16", 2, 1000, 2064, 15),  # many tiles, ragged tail
    ("fp32", 5, 64, 1040, 16),
])
def test_dynamic_shapes(dev, orc, dtype, B, R, C, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = torch.randn((B, R, C), generator=g) * 3.0
    x = x.to(torch.bfloat16 if dtype == "bf16" else torch.float32).to(dev)
    check_quantize(orc, x, "random-%s" % dtype)


def test_moe_experts_small(dev, orc):
    w, _ = synth.moe_weights_bf16(experts=4, rows=256, cols=512, seed=2, with_grad=False)
    check_quantize(orc, w.to(dev), "moe-4x256x512")


def test_activations_small(dev, orc):
    x, _ = synth.student_t_activations_bf16(tokens=512, hidden=4096, seed=3, with_grad=False)
    check_quantize(orc, x.to(dev), "act-512x4096")


def _tie_tensor(j, m):
    s = 2.0 ** (j + m)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    blocks = [[2688.0 * 2.0**j] + [0.0] * 15]
    for which in (0, 1, -1):
        vals = [6.0 * s]
        for t in mids:
            v = np.float32(t * s)
            if which == 1:
                v = np.nextafter(v, np.float32(np.inf))
            elif which == -1:
                v = np.nextafter(v, np.float32(0))
            vals += [float(v), -float(v)]
        blocks.append(vals + [0.0])
    return np.array(blocks, np.float32).reshape(1, -1)


def test_edge_cases(dev, orc):
    C = 64
    cases = {}
    cases["zero"] = np.zeros((4, C), np.float32)
    z = np.zeros((4, C), np.float32)
    z[1, 3] = -0.0
    z[2, :] = -0.0
    cases["neg-zero"] = z
    eq = np.full((4, C), 0.37, np.float32)
    eq[:, ::2] *= -1
    cases["all-equal"] = eq
    tiny = np.random.default_rng(5).normal(0, 1, (4, C)).astype(np.float32)
    tiny[1, 16:32] = -1e-30        # a block far below the others: scale rounds to 0
    tiny[2, 0:16] = 2.0**-12       # E4M3 subnormal block scales
    tiny[3, 0:16] = -3e-3
    cases["underflow-subnormal"] = tiny
    cases["tiny-tensor"] = (np.random.default_rng(6).normal(0, 1, (4, C)) * 1e-30).astype(np.float32)
    cases["huge-tensor"] = (np.random.default_rng(7).normal(0, 1, (4, C)) * 1e36).astype(np.float32)
    for name, arr in cases.items():
        check_quantize(orc, torch.from_numpy(arr).to(dev), name)
    for j, m in [(-20, -9), (0, 0), (3, -6), (11, 8), (-7, 4)]:
        check_quantize(orc, torch.from_numpy(_tie_tensor(j, m)).to(dev), "ties-j%d-m%d" % (j, m))
    # batch with one all-zero expert in the middle
    w, _ = synth.moe_weights_bf16(experts=3, rows=32, cols=128, seed=8, with_grad=False)
    w[1].zero_()
    check_quantize(orc, w.to(dev), "batch-with-zero-expert")
    # bf16 negative tiny values and -0
    b = torch.tensor([[-0.0, -1e-20, 1e-20, -3.0] * 8], dtype=torch.bfloat16)
    check_quantize(orc, b.to(dev), "bf16-neg-tiny")


def test_frozen_scales(dev, orc):
    w = synth.gaussian_weight_bf16(rows=64, cols=256, seed=4)
    xb = host(w)
    # scales below the dynamic ones: block maxima saturate at 6
    scales, ts = orc.mse_calibrate(xb, 64, 0.5, 1.0)
    check_quantize(orc, w.unsqueeze(0).to(dev), "frozen-mse", frozen=(scales[None], np.array([ts])))
    # arbitrary valid codes and a tensor scale unrelated to the data
    rng = np.random.default_rng(9)
    rs = rng.integers(0, 0x7F, size=(2, 64, 16)).astype(np.uint8)
    x2 = torch.randn((2, 64, 256), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    check_quantize(orc, x2.to(dev), "frozen-random", frozen=(rs, np.array([1e-3, 7.5], np.float32)))
    # a frozen tensor scale below the reciprocal-division range
    x3 = (torch.randn((1, 8, 64), generator=torch.Generator().manual_seed(4)) * 1e-25).to(torch.float32)
    rs3 = rng.integers(0, 0x7F, size=(1, 8, 4)).astype(np.uint8)
    check_quantize(orc, x3.to(dev), "frozen-tiny-scale", frozen=(rs3, np.array([1e-28], np.float32)))


def test_frozen_quotient_overflow(dev, orc):
    # frozen scales far below the elements: x / s_eff exceeds the binary32
    # range (the oracle's quotient is inf and saturates to +-6); tensor scale
    # 2^-80 (reciprocal division) and 2^-81 (IEEE division), signed zeros and
    # ordinary values in the same blocks
    x = torch.empty((2, 4, 64), dtype=torch.float32)
    g = torch.Generator().manual_seed(12)
    x.copy_(torch.randn((2, 4, 64), generator=g) * 1e30)
    x[:, :, ::7] = 3.0e38
    x[:, :, 1::7] = -3.0e38
    x[:, :, 2::7] = -0.0
    x[:, :, 3::7] = 0.0
    x[:, :, 4::7] = 1e-30
    x[:, 0, :16] = 2.0 ** -88                      # an ordinary block under the tiny scale
    rs = np.full((2, 4, 4), 1, np.uint8)          # E4M3 code 1: 2^-9
    rs[:, :, 3] = 0                               # s_eff = 0: signed zeros
    rs[:, 1, 2] = 0x7E                            # 448
    for ts in (2.0 ** -80, 2.0 ** -81):
        check_quantize(orc, x.to(dev), "frozen-overflow ts=%g" % ts, frozen=(rs, np.array([ts, ts], np.float32)))


def test_qdq_fwd_equals_quantize_y(dev, orc):
    w, _ = synth.moe_weights_bf16(experts=2, rows=128, cols=256, seed=21, with_grad=False)
    w = w.to(dev)
    announce("nvfp4_qdq_fwd vs nvfp4_quantize")
    y1 = q.nvfp4_qdq_fwd(w)
    _, _, _, y2 = q.nvfp4_quantize(w)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("n,dtype", [(1, torch.bfloat16), (7, torch.bfloat16), (8, torch.bfloat16),
                                     (1000003, torch.bfloat16), (5, torch.float32), (262147, torch.float32)])
def test_ste_backward_is_identity(dev, n, dtype):
    g = torch.randn(n, generator=torch.Generator().manual_seed(n)).to(dtype).to(dev)
    announce("nvfp4_qdq_bwd n=%d %s" % (n, dtype))
    gx = q.nvfp4_qdq_bwd(g)
    torch.cuda.synchronize()
    assert torch.equal(gx.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                       g.view(torch.int16 if dtype == torch.bfloat16 else torch.int32))


def test_amax(dev, orc):
    cases = [torch.randn((3, 17, 64)) * 5, (torch.randn((2, 9, 40)) * 2).to(torch.bfloat16),
             -torch.arange(1, 65, dtype=torch.float32).reshape(1, 1, 64), torch.zeros((2, 1, 8))]
    for x in cases:
        announce("nvfp4_amax %s %s" % (tuple(x.shape), x.dtype))
        a = q.nvfp4_amax(x.to(dev))
        torch.cuda.synchronize()
        xc = host(x)
        for b in range(x.shape[0]):
            assert np.float32(host(a)[b]).view(np.uint32) == np.float32(orc.amax(xc[b])).view(np.uint32)
    bad = torch.tensor([[1.0, float("nan"), 2.0, 3.0]], device=dev)
    a = q.nvfp4_amax(bad)
    assert not q.qad_check_finite(a)
    assert q.qad_check_finite(q.nvfp4_amax(torch.ones((1, 4), device=dev)))


@pytest.mark.parametrize("dtype,shape,n,kmin,kmax", [
    ("bf16", (256, 512), 64, 0.5, 1.0),
    ("fp32", (64, 1024), 64, 0.5, 1.0),
    ("bf16", (3, 40, 96), 16, 0.6, 1.0),
    ("bf16", (128, 64), 1, 0.9, 0.9),
    ("fp32", (2, 17, 32), 200, 0.25, 1.0),
])
def test_mse_calibrate(dev, orc, dtype, shape, n, kmin, kmax):
    g = torch.Generator().manual_seed(sum(shape) + n)
    w = torch.randn(shape, generator=g) * 0.02
    w[..., ::37] *= 15.0
    w = w.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    w3 = w if w.dim() == 3 else w.unsqueeze(0)
    announce("nvfp4_mse_calibrate %s %s n=%d k=[%g,%g]" % (dtype, shape, n, kmin, kmax))
    sc, ts = q.nvfp4_mse_calibrate(w3.to(dev), n, kmin, kmax)
    torch.cuda.synchronize()
    wc = host(w3)
    for b in range(w3.shape[0]):
        rs, rt = orc.mse_calibrate(wc[b], n, kmin, kmax)
        assert host(ts)[b] == np.float32(rt)
        bad = np.argwhere(host(sc)[b].reshape(rs.shape) != rs)
        assert bad.size == 0, bad[:5]
    # then the frozen QDQ with the calibrated scales
    check_quantize(orc, w3.to(dev), "frozen-after-mse", frozen=(host(sc), host(ts)))


@pytest.mark.parametrize("dtype,shape", [("bf16", (32, 256, 2048)), ("fp32", (64, 256, 1024))])
def test_mse_calibrate_large_batch(dev, orc, dtype, shape):
    # a batch of many tensors in one grid (workgroups of several tensors
    # resident together, each reading its own tensor scale); every scale of
    # every tensor is compared
    g = torch.Generator().manual_seed(shape[0])
    w = torch.randn(shape, generator=g) * 0.02
    w[..., ::29] *= 12.0
    w = w.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    announce("nvfp4_mse_calibrate batch %s %s" % (dtype, shape))
    sc, ts = q.nvfp4_mse_calibrate(w.to(dev))
    torch.cuda.synchronize()
    wc, sch, tsh = host(w), host(sc), host(ts)
    for b in range(shape[0]):
        rs, rt = orc.mse_calibrate(wc[b])
        assert tsh[b] == np.float32(rt), b
        assert np.array_equal(sch[b].reshape(rs.shape), rs), b


def test_deterministic(dev):
    w, _ = synth.moe_weights_bf16(experts=4, rows=256, cols=512, seed=2, with_grad=False)
    w = w.to(dev)
    announce("determinism")
    a = q.nvfp4_quantize(w)
    b = q.nvfp4_quantize(w)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.uint8), v.view(torch.uint8))


# ---- full-size workloads, sampled ------------------------------------------
def _rows(t: torch.Tensor, rows) -> np.ndarray:
    return host(t.index_select(0, torch.as_tensor(rows, device=t.device)))


def _sampled_rows_check(orc, xh, b, rows, s_g, codes, scales, y, label, scales_in=None):
    blk = xh[b][rows]  # [nr, C]
    rc, rs, ry = orc.nvfp4_quantize_blocks(blk, s_g, None if scales_in is None else scales_in)
    assert np.array_equal(_rows(scales[b], rows).reshape(-1), rs), (label, b, "scales")
    assert np.array_equal(_rows(codes[b], rows).reshape(-1, 8), rc), (label, b, "codes")
    assert np.array_equal(_rows(y[b], rows).reshape(-1, 16), ry), (label, b, "y")


def test_moe_full_size(dev, orc):
    # 128 experts x 2048 x 4096 bf16: QDQ forward + STE backward as timed;
    # every expert's tensor scale, block scales, codes and QDQ output against
    # the oracle in full
    announce("full-size MoE 128x2048x4096 generate")
    w, grad = synth.moe_weights_bf16(seed=2, device=dev)
    announce("full-size MoE quantize + qdq_fwd + qdq_bwd")
    codes, scales, ts, y = q.nvfp4_quantize(w)
    y2 = q.nvfp4_qdq_fwd(w)
    gx = q.nvfp4_qdq_bwd(grad)
    torch.cuda.synchronize()
    assert torch.equal(gx.view(torch.int16), grad.view(torch.int16))
    assert torch.equal(y2.view(torch.int16), y.view(torch.int16))
    del gx, y2, grad
    tsh = host(ts)
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=8) as pool:   # the oracle's C calls release the GIL
        for b0 in range(0, 128, 16):
            refs = list(pool.map(lambda b: orc.nvfp4_quantize(host(w[b])), range(b0, b0 + 16)))
            for b, (rc, rs, rt, ry) in zip(range(b0, b0 + 16), refs):
                assert tsh[b] == np.float32(rt), b
                assert np.array_equal(host(scales[b]).reshape(rs.shape), rs), (b, "scales")
                assert np.array_equal(host(codes[b]).reshape(rc.shape), rc), (b, "codes")
                assert np.array_equal(host(y[b]).reshape(ry.shape), ry), (b, "y")


def test_activations_full_size(dev, orc):
    # 32768 x 4096 bf16 (256 MiB): the whole tensor against the oracle
    announce("full-size activations 32768x4096 generate")
    x, grad = synth.student_t_activations_bf16(seed=3, device=dev)
    announce("full-size activations quantize + qdq_fwd + qdq_bwd")
    x3 = x.unsqueeze(0)
    codes, scales, ts, y = q.nvfp4_quantize(x3)
    y2 = q.nvfp4_qdq_fwd(x3)
    gx = q.nvfp4_qdq_bwd(grad)
    torch.cuda.synchronize()
    assert torch.equal(gx.view(torch.int16), grad.view(torch.int16))
    assert torch.equal(y2.view(torch.int16), y.view(torch.int16))
    del gx, y2, grad
    rc, rs, rt, ry = orc.nvfp4_quantize(host(x3)[0])
    assert host(ts)[0] == np.float32(rt)
    assert np.array_equal(host(scales[0]).reshape(rs.shape), rs)
    assert np.array_equal(host(codes[0]).reshape(rc.shape), rc)
    assert np.array_equal(host(y[0]).reshape(ry.shape), ry)


def test_mse_full_size_sampled(dev, orc):
    announce("full-size 8192x8192 generate")
    w = synth.gaussian_weight_bf16(seed=4, device=dev).unsqueeze(0)
    announce("full-size nvfp4_mse_calibrate + frozen quantize")
    sc, ts = q.nvfp4_mse_calibrate(w)
    codes, scales, ts2, y = q.nvfp4_quantize(w, sc, ts)
    torch.cuda.synchronize()
    wh = host(w)
    s_g = orc.tensor_scale(orc.amax(wh[0]))
    assert host(ts)[0] == np.float32(s_g) and host(ts2)[0] == np.float32(s_g)
    rows = np.sort(np.random.default_rng(2).choice(8192, 256, replace=False))
    blocks = orc.f32_from_bf16(wh[0][rows]).reshape(-1, 16)
    rs, _ = orc.mse_calibrate_blocks(blocks, s_g)
    assert np.array_equal(_rows(sc[0], rows).reshape(-1), rs)
    assert np.array_equal(_rows(scales[0], rows).reshape(-1), rs)
    _sampled_rows_check(orc, wh, 0, rows, s_g, codes, scales, y, "frozen", scales_in=rs)
