"""nvfp4_quantize_noalloc (no workspace: the library's fixed scratch) against
nvfp4_quantize with a workspace of its own.

Both run the same kernels, so every output (packed E2M1 codes, E4M3 block
scales, fp32 tensor scale, bf16 QDQ values) must agree bit for bit.  The
scratch keeps the previous call's records, so each test makes calls in a
row, a large one first and then smaller ones, and checks every call.
"""
import numpy as np
import pytest
import torch

import nvfp4_quantization_aware_amd as q
from nvfp4_quantization_aware_amd import synth
from gpu_util import announce, gpu_device, host

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 16 << 20   # the fixed scratch the header states


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


def outputs_like(x: torch.Tensor):
    n = x.numel()
    B = x.shape[0] if x.dim() == 3 else 1
    return (torch.empty(n // 2, dtype=torch.uint8, device=x.device),
            torch.empty(n // 16, dtype=torch.uint8, device=x.device),
            torch.empty(B, dtype=torch.float32, device=x.device),
            torch.empty(n, dtype=torch.bfloat16, device=x.device))


def assert_same(label, got, want):
    for name, a, b in zip(("codes", "scales", "tscale", "y"), got, want):
        ha, hb = host(a).reshape(-1), host(b).reshape(-1)
        if ha.dtype == np.float32:
            ha, hb = ha.view(np.uint32), hb.view(np.uint32)
        bad = np.flatnonzero(ha != hb)
        assert bad.size == 0, (label, name, bad[:5], ha[bad[:5]], hb[bad[:5]])


def run_both(x: torch.Tensor, label: str, scales_in=None, tscale_in=None):
    announce("nvfp4_quantize_noalloc %s shape=%s dtype=%s frozen=%s"
             % (label, tuple(x.shape), x.dtype, tscale_in is not None))
    got = outputs_like(x)
    q.nvfp4_quantize_noalloc(x, *got, scales_in=scales_in, tscale_in=tscale_in)
    want = q.nvfp4_quantize(x, scales_in, tscale_in)
    torch.cuda.synchronize()
    assert_same(label, got, want)
    return got


def test_two_calls_large_then_small(dev):
    # a 64 Mi-element tensor (amax pass, then quantize), then a 128-expert
    # MoE batch (one pass per expert), then a small ragged fp32 batch: each
    # later call reuses the scratch the earlier one left full of records
    x0 = synth.gaussian_weight_bf16(rows=8192, cols=8192, seed=21, device=dev).unsqueeze(0)
    run_both(x0, "64Mi gaussian")
    del x0
    x1 = synth.moe_weights_bf16(experts=128, rows=256, cols=512, seed=22, device=dev, with_grad=False)[0]
    run_both(x1, "moe 128x256x512")
    del x1
    x2 = synth.outlier_tensor_f32(rows=3 * 100, cols=48, seed=23, device=dev).reshape(3, 100, 48)
    run_both(x2, "ragged f32 3x100x48")


def test_second_call_smaller_same_tensor_count(dev):
    a = synth.student_t_activations_bf16(tokens=4096, hidden=4096, seed=24, device=dev, with_grad=False)[0]
    a = a.reshape(8, 512, 4096)
    run_both(a, "activations 8x512x4096")
    b = a[:, :100, :1024].contiguous()
    run_both(b, "activations 8x100x1024")


def test_frozen_scales_after_dynamic(dev):
    x = synth.moe_weights_bf16(experts=4, rows=512, cols=1024, seed=25, device=dev, with_grad=False)[0]
    _, s, t, _ = run_both(x, "dynamic 4x512x1024")
    x2 = synth.moe_weights_bf16(experts=4, rows=512, cols=1024, seed=26, device=dev, with_grad=False)[0]
    run_both(x2, "frozen 4x512x1024", scales_in=s, tscale_in=t)


def test_largest_batch_that_fits_and_one_beyond(dev):
    # many 16-element tensors: the records, not the data, fill the scratch
    def need(B):
        return q.qad_workspace_bytes(q.QAD_OP_QUANTIZE, B, 1, 16)
    lo, hi = 1, 1 << 20
    while lo < hi:
        mid = (lo + hi + 1) // 2
        lo, hi = (mid, hi) if need(mid) <= SCRATCH_BYTES else (lo, mid - 1)
    B = lo
    assert need(B) <= SCRATCH_BYTES < need(B + 1)
    x = synth.outlier_tensor_f32(rows=B + 1, cols=16, seed=27, device=dev).to(torch.bfloat16)
    run_both(x[:B].reshape(B, 1, 16).contiguous(), "largest batch %d x 1 x 16" % B)
    xb = x.reshape(B + 1, 1, 16)
    announce("nvfp4_quantize_noalloc %d x 1 x 16 (beyond the scratch)" % (B + 1))
    with pytest.raises(q.QadError) as e:
        q.nvfp4_quantize_noalloc(xb, *outputs_like(xb))
    assert "WORKSPACE" in str(e.value)
    torch.cuda.synchronize()
    run_both(synth.outlier_tensor_f32(rows=64, cols=32, seed=28, device=dev), "after the rejected call 64x32")


def test_empty_and_oracle(dev, orc):
    # an empty batch writes nothing and needs no scratch; a tiny tensor after
    # it also matches the oracle
    e = torch.empty(2, 0, 32, dtype=torch.bfloat16, device=dev)
    announce("nvfp4_quantize_noalloc empty 2x0x32")
    _, _, te, _ = q.nvfp4_quantize_noalloc(e, *outputs_like(e))
    torch.cuda.synchronize()
    assert np.array_equal(host(te), np.ones(2, np.float32))
    x = synth.outlier_tensor_f32(rows=5, cols=80, seed=29, device=dev)
    codes, scales, ts, y = run_both(x, "tiny 5x80")
    rc, rs, rt, ry = orc.nvfp4_quantize(host(x))
    assert host(ts)[0].view(np.uint32) == np.float32(rt).view(np.uint32)
    assert np.array_equal(host(scales), rs.reshape(-1))
    assert np.array_equal(host(codes), rc.reshape(-1))
    assert np.array_equal(host(y), ry.reshape(-1))
