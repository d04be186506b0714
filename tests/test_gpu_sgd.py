"""GPU parity of nvfp4_frozen_sgd_step (the frozen-scale SGD weight step with
the clipped straight-through gradient fused in) against the oracle, bit for
bit.

Frozen scales fed to both sides come from the oracle's own forward or from a
seeded generator (arbitrary codes and tensor scales), never from the HIP
path.  Cases: the hand-derived fixture (ties, signed zeros, subnormals,
double rounding, binary32 weights), every weight/gradient dtype combination
on shapes spanning several workgroup chunks with a ragged last chunk, zero
scale codes, a zero step, in-place use, and the full 128-expert batch
(128 x 2048 x 4096 bf16) compared in full in the launch configuration the
benchmark times.
"""
import json
import os
from concurrent.futures import ThreadPoolExecutor

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


def to_dtype(f: np.ndarray, bf16: bool) -> np.ndarray:
    if not bf16:
        return f.astype(np.float32)
    return host(torch.from_numpy(f.astype(np.float32)).to(torch.bfloat16))


def bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)


def run_and_check(orc, dev, w, g, scales, tscale, lr, clip, label, in_place=False):
    """w, g: numpy [B, R, C] (float32 or bf16 bits); scales u8 [B, R, C/16];
    tscale float32 [B]."""
    B, R, Cc = w.shape
    announce("nvfp4_frozen_sgd_step %s B=%d R=%d C=%d w=%s g=%s lr=%g clip=%g in_place=%s"
             % (label, B, R, Cc, w.dtype, g.dtype, lr, clip, in_place))
    w_d, g_d = dev_tensor(w, dev), dev_tensor(g, dev)
    out = q.nvfp4_frozen_sgd_step(w_d, g_d, dev_tensor(scales, dev), dev_tensor(np.asarray(tscale, np.float32), dev),
                                  lr, clip, w_out=w_d if in_place else None)
    torch.cuda.synchronize()
    got = host(out)
    for b in range(B):
        ref, _ = orc.nvfp4_frozen_sgd_step(w[b].ravel(), g[b].ravel(), scales[b].ravel(), float(tscale[b]), lr, clip)
        bad = np.nonzero(bits(got[b].ravel()) != bits(ref))[0]
        assert bad.size == 0, (label, b, bad[:8], got[b].ravel()[bad[:8]], ref[bad[:8]])
    return got


@pytest.mark.parametrize("name", ["A", "B", "C"])
def test_worked_example(dev, orc, name):
    d = json.load(open(os.path.join(GOLDEN, "frozen_sgd_step_worked_example.json")))
    c = [c for c in d["cases"] if c["name"] == name][0]
    u = lambda h, dt: (np.array([int(v, 16) for v in h], np.uint32).astype(np.uint16) if dt == "bf16"
                       else np.array([int(v, 16) for v in h], np.uint32).view(np.float32))
    w = u(c["w_bits"], c["w_dtype"]).reshape(1, 1, -1)
    g = u(c["g_bits"], c["g_dtype"]).reshape(1, 1, -1)
    sc = np.array(c["scales"], np.uint8).reshape(1, 1, -1)
    got = run_and_check(orc, dev, w, g, sc, np.array([c["tscale"]], np.float32), c["lr"], c["clip_coef"],
                        "golden " + name)
    assert bits(got.ravel()).tolist() == bits(u(c["expected_bits"], c["w_dtype"])).tolist()


@pytest.mark.parametrize("gbf", [True, False])
@pytest.mark.parametrize("wbf", [True, False])
@pytest.mark.parametrize("shape", [(2, 5, 8208), (3, 33, 48), (1, 1, 16)])
def test_scales_from_oracle_forward(dev, orc, gbf, wbf, shape):
    # frozen scales of the oracle's forward on the weights before a drift:
    # the drifted weights cross their blocks' limits in both directions
    rng = np.random.default_rng(sum(shape) + 2 * gbf + wbf)
    B, R, Cc = shape
    w0 = to_dtype((rng.standard_t(3, size=shape) * 0.02).astype(np.float32), wbf)
    scales = np.empty((B, R, Cc // 16), np.uint8)
    ts = np.empty(B, np.float32)
    for b in range(B):
        _, sc, t, _ = orc.nvfp4_quantize(w0[b])
        scales[b], ts[b] = sc, t
    w0f = (w0.astype(np.uint32) << 16).view(np.float32) if wbf else w0
    wf = w0f * (1.0 + 0.05 * rng.standard_normal(shape)).astype(np.float32)
    w = to_dtype(wf, wbf)
    g = to_dtype(rng.standard_normal(shape).astype(np.float32), gbf)
    for lr, clip in [(1e-3, 1.0), (0.013, 0.37)]:
        got = run_and_check(orc, dev, w, g, scales, ts, lr, clip, "forward scales")
        if B * R * Cc >= 4096:
            moved = bits(got) != bits(w)
            assert moved.any() and (~moved).any()


@pytest.mark.parametrize("gbf,wbf", [(True, True), (False, True), (True, False)])
def test_random_frozen_codes(dev, orc, gbf, wbf):
    # arbitrary frozen codes (zero, subnormal, large) and tensor scales
    rng = np.random.default_rng(5 + gbf + 2 * wbf)
    B, R, Cc = 3, 17, 1024 + 64
    w = to_dtype((rng.standard_normal((B, R, Cc)) * 4).astype(np.float32), wbf)
    g = to_dtype(rng.standard_normal((B, R, Cc)).astype(np.float32), gbf)
    scales = rng.integers(0, 127, (B, R, Cc // 16)).astype(np.uint8)
    scales[:, 0, :] = 0                      # s_eff = 0: only signed zeros step
    ts = np.array([2.0 ** -6, 0.37, 1e-3], np.float32)
    run_and_check(orc, dev, w, g, scales, ts, 0.25, 0.5, "frozen random")
    run_and_check(orc, dev, w, g, scales, ts, 0.0, 1.0, "zero step")


def test_in_place(dev, orc):
    rng = np.random.default_rng(9)
    w = to_dtype((rng.standard_normal((2, 64, 256)) * 3).astype(np.float32), True)
    g = to_dtype(rng.standard_normal((2, 64, 256)).astype(np.float32), True)
    scales = np.full((2, 64, 16), 0x38, np.uint8)
    run_and_check(orc, dev, w, g, scales, np.array([0.5, 0.25], np.float32), 0.125, 1.0, "in place", in_place=True)


def test_empty(dev):
    w = torch.empty(2, 0, 32, dtype=torch.bfloat16, device=dev)
    announce("nvfp4_frozen_sgd_step empty 2x0x32")
    out = q.nvfp4_frozen_sgd_step(w, w.clone(), torch.empty(0, dtype=torch.uint8, device=dev),
                                  torch.ones(2, device=dev), 0.1)
    torch.cuda.synchronize()
    assert out.numel() == 0


def test_moe_full_size(dev, orc):
    # the 128-expert batch with seeded frozen codes (E4M3 0.125 .. 16 times a
    # tensor scale near amax / 2688): most blocks clip some weights; every
    # expert is compared in full, on 8 host threads
    announce("frozen SGD step full-size MoE 128x2048x4096 generate")
    w, grad = synth.moe_weights_bf16(seed=2, device=dev)
    rng = np.random.default_rng(31)
    scales = rng.integers(0x20, 0x5A, (128, 2048, 256)).astype(np.uint8)
    ts = np.full(128, 0.4 / 2688, np.float32) * rng.uniform(0.5, 2.0, 128).astype(np.float32)
    sc_d, ts_d = dev_tensor(scales, dev), dev_tensor(ts, dev)
    lr, clip = 0.05, 0.61
    announce("frozen SGD step full-size MoE step")
    out = q.nvfp4_frozen_sgd_step(w, grad, sc_d, ts_d, lr, clip)
    torch.cuda.synchronize()

    def check(b):
        wh, gh = host(w[b]).ravel(), host(grad[b]).ravel()
        ref, n_clip = orc.nvfp4_frozen_sgd_step(wh, gh, scales[b].ravel(), float(ts[b]), lr, clip)
        got = host(out[b]).ravel()
        bad = np.flatnonzero(got != ref)
        return b, n_clip, int((ref != wh).sum()), bad[:5]

    total_clip = total_moved = 0
    with ThreadPoolExecutor(8) as ex:
        for b0 in range(0, 128, 16):
            for b, n_clip, moved, bad in ex.map(check, range(b0, b0 + 16)):
                assert bad.size == 0, (b, bad)
                total_clip += n_clip
                total_moved += moved
    assert total_clip > 0 and total_moved > 0
