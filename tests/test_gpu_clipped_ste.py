"""GPU parity of nvfp4_qdq_bwd_clipped (the clipped straight-through backward)
against the oracle, bit for bit.

Scales fed to both sides come from the oracle's own forward (dynamic scales)
or from a seeded generator (arbitrary frozen codes and tensor scales), never
from the HIP path.  Cases: the hand-derived fixture (elements on, just above
and just below 6 * s_eff, in bf16 and fp32), every grad/x dtype combination
on shapes that span several workgroup chunks with a ragged last chunk, zero
scale codes, in-place use, and the full MoE-weight shape (128 x 2048 x 4096
bf16) with the library's own dynamic scales checked equal to the oracle's on
sampled experts before their gradients are compared.
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


def dev_tensor(a: np.ndarray, dev):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(dev)


def run_and_check(orc, dev, gy, x, scales, tscale, label, in_place=False):
    """gy, x: numpy [B, R, C] (float32 or bf16 bits); scales u8 [B, R, C/16];
    tscale float32 [B]."""
    B, R, Cc = x.shape
    announce("nvfp4_qdq_bwd_clipped %s B=%d R=%d C=%d g=%s x=%s in_place=%s"
             % (label, B, R, Cc, gy.dtype, x.dtype, in_place))
    gy_d, x_d = dev_tensor(gy, dev), dev_tensor(x, dev)
    sc_d = dev_tensor(scales, dev)
    ts_d = dev_tensor(np.asarray(tscale, np.float32), dev)
    out = q.nvfp4_qdq_bwd_clipped(gy_d, x_d, sc_d, ts_d, grad_x=gy_d if in_place else None)
    torch.cuda.synchronize()
    got = host(out)
    for b in range(B):
        ref, _ = orc.nvfp4_qdq_bwd_clipped(gy[b].ravel(), x[b].ravel(), scales[b].ravel(), float(tscale[b]))
        g = got[b].ravel()
        bad = np.nonzero(g.view(np.uint16 if g.dtype == np.uint16 else np.uint32)
                         != ref.view(np.uint16 if ref.dtype == np.uint16 else np.uint32))[0]
        assert bad.size == 0, (label, b, bad[:8])
    return got


def to_dtype(f: np.ndarray, bf16: bool) -> np.ndarray:
    if not bf16:
        return f.astype(np.float32)
    return host(torch.from_numpy(f.astype(np.float32)).to(torch.bfloat16))


def test_worked_example(dev, orc):
    g = json.load(open(os.path.join(GOLDEN, "clipped_ste_worked_example.json")))
    u32 = lambda h: np.array([int(v, 16) for v in h], np.uint32)
    A = g["A"]
    xa = u32(A["x_bits"]).astype(np.uint16).reshape(1, 1, 32)
    ga = to_dtype(np.array(A["grad"], np.float32), True).reshape(1, 1, 32)
    got = run_and_check(orc, dev, ga, xa, np.array(A["scales"], np.uint8).reshape(1, 1, 2),
                        np.array([A["tscale"]], np.float32), "golden bf16")
    assert got.ravel().tolist() == to_dtype(np.array(A["grad_x"], np.float32), True).tolist()
    Bx = g["B"]
    xb = u32(Bx["x_bits"]).view(np.float32).reshape(1, 1, 32)
    gb = u32(Bx["grad_bits"]).view(np.float32).reshape(1, 1, 32)
    ts = u32([Bx["tscale_bits"]]).view(np.float32)
    got = run_and_check(orc, dev, gb, xb, np.array(Bx["scales"], np.uint8).reshape(1, 1, 2), ts, "golden fp32")
    assert got.ravel().view(np.uint32).tolist() == u32(Bx["grad_x_bits"]).tolist()


@pytest.mark.parametrize("gbf", [True, False])
@pytest.mark.parametrize("xbf", [True, False])
@pytest.mark.parametrize("shape", [(2, 5, 8208), (3, 33, 48), (1, 1, 16)])
def test_dynamic_scales_from_oracle(dev, orc, gbf, xbf, shape):
    # scales of the oracle's own dynamic forward: the block holding a block
    # maximum is clipped whenever its E4M3 scale rounded down
    rng = np.random.default_rng(sum(shape) + 2 * gbf + xbf)
    B, R, Cc = shape
    xf = (rng.standard_t(3, size=shape) * 0.5).astype(np.float32)
    x = to_dtype(xf, xbf)
    gy = to_dtype(rng.standard_normal(shape).astype(np.float32), gbf)
    scales = np.empty((B, R, Cc // 16), np.uint8)
    ts = np.empty(B, np.float32)
    for b in range(B):
        _, sc, t, _ = orc.nvfp4_quantize(x[b])
        scales[b], ts[b] = sc, t
    got = run_and_check(orc, dev, gy, x, scales, ts, "dynamic")
    if B * R * Cc >= 4096:
        assert (got == 0).any() and (got != 0).any()


@pytest.mark.parametrize("gbf,xbf", [(True, True), (False, True), (True, False)])
def test_random_frozen_codes(dev, orc, gbf, xbf):
    # arbitrary frozen codes (zero, subnormal, large) and tensor scales
    rng = np.random.default_rng(5 + gbf + 2 * xbf)
    B, R, Cc = 3, 17, 1024 + 64
    x = to_dtype((rng.standard_normal((B, R, Cc)) * 4).astype(np.float32), xbf)
    gy = to_dtype(rng.standard_normal((B, R, Cc)).astype(np.float32), gbf)
    scales = rng.integers(0, 127, (B, R, Cc // 16)).astype(np.uint8)
    scales[:, 0, :] = 0                      # s_eff = 0: only signed zeros pass
    ts = np.array([2.0 ** -6, 0.37, 1e-3], np.float32)
    run_and_check(orc, dev, gy, x, scales, ts, "frozen random")


def test_in_place(dev, orc):
    rng = np.random.default_rng(9)
    x = to_dtype((rng.standard_normal((2, 64, 256)) * 3).astype(np.float32), True)
    gy = to_dtype(rng.standard_normal((2, 64, 256)).astype(np.float32), True)
    scales = np.full((2, 64, 16), 0x38, np.uint8)
    run_and_check(orc, dev, gy, x, scales, np.array([0.5, 0.25], np.float32), "in place", in_place=True)


def test_moe_full_size_sampled(dev, orc):
    # 128 experts x 2048 x 4096 bf16 with the forward's dynamic scales; the
    # library's scales are first checked equal to the oracle's on the sampled
    # experts, then the clipped gradients are compared there in full
    announce("clipped STE full-size MoE 128x2048x4096 generate")
    w, grad = synth.moe_weights_bf16(seed=2, device=dev)
    announce("clipped STE full-size MoE quantize + clipped backward")
    _, scales, ts, _ = q.nvfp4_quantize(w)
    gx = q.nvfp4_qdq_bwd_clipped(grad, w, scales, ts)
    torch.cuda.synchronize()
    assert int((gx == 0).sum()) > 0
    for b in (0, 63, 127):
        xh, gh = host(w[b]), host(grad[b])
        _, sc_ref, ts_ref, _ = orc.nvfp4_quantize(xh)
        assert np.array_equal(host(scales[b]).reshape(sc_ref.shape), sc_ref), b
        assert host(ts)[b] == np.float32(ts_ref), b
        ref, n_clip = orc.nvfp4_qdq_bwd_clipped(gh.ravel(), xh.ravel(), sc_ref.ravel(), ts_ref)
        assert n_clip > 0
        assert np.array_equal(host(gx[b]).ravel(), ref), b
