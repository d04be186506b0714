"""Seeded random sweeps of the main entry points against the oracle: shapes,
dtypes, scale modes, value ranges and temperatures drawn from a fixed
generator, each case checked by the same rules as the focused tests (codes,
scales, tensor scales and QDQ outputs bit for bit; KL within the 1e-5 rules).
They look for edge cases the hand-picked shapes miss: ragged tails at every
offset, vocabularies on both sides of segment boundaries, tensor scales from
2^-100 to 2^100 (both division paths), sparse tensors, exact ties.  The
top-k / top-p cases go through those tests' own checkers (random k, top_p,
temperature, dtypes, tie-heavy teachers; case 16 is a single row whose KL is
near 0).
"""
import numpy as np
import pytest
import torch

import nvfp4_quantization_aware_amd as q
from nvfp4_quantization_aware_amd import synth
from gpu_util import announce, assert_kl_grad_close, assert_kl_loss_close, gpu_device, host, kl_probs
import test_gpu_kl_topk
import test_gpu_kl_topp
import test_gpu_linear

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


def random_tensor(rng, shape, dtype):
    """float32 values of a randomly chosen character, then cast to dtype"""
    kind = rng.integers(0, 5)
    scale = float(2.0 ** rng.uniform(-100, 100))
    if kind == 0:
        x = rng.standard_normal(shape) * scale
    elif kind == 1:
        x = rng.standard_t(3, size=shape) * scale
    elif kind == 2:   # sparse: mostly exact zeros (and some -0)
        x = rng.standard_normal(shape) * scale * (rng.random(shape) < 0.05)
        x[rng.random(shape) < 0.01] = -0.0
    elif kind == 3:   # E2M1 grid points and midpoints times one scale
        grid = np.array([0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6])
        x = rng.choice(grid, size=shape) * np.where(rng.random(shape) < 0.5, -1, 1) * scale
    else:             # heavy outliers
        x = rng.standard_normal(shape) * scale
        x[rng.random(shape) < 0.002] *= 1e3
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


@pytest.mark.parametrize("case", range(24))
def test_nvfp4_quantize_sweep(dev, orc, case):
    rng = np.random.default_rng(1000 + case)
    dtype = ["bf16", "fp32"][case % 2]
    B, R, C = int(rng.integers(1, 5)), int(rng.integers(1, 300)), 16 * int(rng.integers(1, 300))
    x = random_tensor(rng, (B, R, C), dtype)
    frozen = case % 3 == 2
    announce("nvfp4 sweep case %d %s B=%d R=%d C=%d frozen=%s" % (case, dtype, B, R, C, frozen))
    xh = host(x)
    if frozen:
        sc = rng.integers(0, 127, (B, R, C // 16)).astype(np.uint8)
        ts = (2.0 ** rng.uniform(-90, 60, B)).astype(np.float32)
        codes, scales, tsd, y = q.nvfp4_quantize(x.to(dev), torch.from_numpy(sc).to(dev), torch.from_numpy(ts).to(dev))
    else:
        codes, scales, tsd, y = q.nvfp4_quantize(x.to(dev))
    torch.cuda.synchronize()
    cg, sg, tg, yg = host(codes), host(scales), host(tsd), host(y)
    for b in range(B):
        if frozen:
            rc, rs, rt, ry = orc.nvfp4_quantize(xh[b], sc[b], float(ts[b]))
        else:
            rc, rs, rt, ry = orc.nvfp4_quantize(xh[b])
        assert tg[b].view(np.uint32) == np.float32(rt).view(np.uint32), (case, b)
        assert np.array_equal(sg[b].reshape(rs.shape), rs), (case, b, "scales")
        assert np.array_equal(cg[b].reshape(rc.shape), rc), (case, b, "codes")
        assert np.array_equal(yg[b].reshape(ry.shape), ry), (case, b, "y")


@pytest.mark.parametrize("case", range(8))
def test_fp8_quantize_sweep(dev, orc, case):
    rng = np.random.default_rng(2000 + case)
    dtype = ["bf16", "fp32"][case % 2]
    B, R, C = int(rng.integers(1, 4)), int(rng.integers(1, 200)), 8 * int(rng.integers(1, 400))
    x = random_tensor(rng, (B, R, C), dtype)
    frozen = case % 4 == 3
    ts = (2.0 ** rng.uniform(-90, 60, B)).astype(np.float32) if frozen else None
    announce("fp8 sweep case %d %s B=%d R=%d C=%d frozen=%s" % (case, dtype, B, R, C, frozen))
    codes, tsd, y = q.fp8_quantize(x.to(dev), None if ts is None else torch.from_numpy(ts).to(dev))
    torch.cuda.synchronize()
    xh, cg, tg, yg = host(x), host(codes), host(tsd), host(y)
    for b in range(B):
        rc, rt, ry = orc.fp8_quantize(xh[b], None if ts is None else float(ts[b]))
        assert tg[b].view(np.uint32) == np.float32(rt).view(np.uint32), (case, b)
        assert np.array_equal(cg[b], rc), (case, b, "codes")
        assert np.array_equal(yg[b], ry), (case, b, "y")


@pytest.mark.parametrize("case", range(12))
def test_kl_sweep(dev, orc, case):
    rng = np.random.default_rng(3000 + case)
    tokens = int(rng.integers(1, 24))
    if case % 3 == 0:     # on and around a segment boundary (16384 logits)
        vocab = 16384 * int(rng.integers(1, 9)) + 8 * int(rng.integers(-1, 2))
    else:
        vocab = 8 * int(rng.integers(1, 20000))
    vocab = max(vocab, 8)
    T = float(rng.choice([0.5, 1.0, 2.0]))
    in_dt = [torch.bfloat16, torch.float32][case % 2]
    g_dt = [torch.bfloat16, torch.float32][(case // 2) % 2]
    std = float(rng.uniform(0.5, 8.0))
    t, s = synth.logits_bf16(tokens=tokens, vocab=vocab, teacher_std=std, seed=3000 + case)
    t, s = t.to(in_dt), s.to(in_dt)
    announce("kl sweep case %d tokens=%d vocab=%d T=%g in=%s grad=%s" % (case, tokens, vocab, T, in_dt, g_dt))
    loss, rows, g = q.qad_kl_fwd_bwd(t.to(dev), s.to(dev), temperature=T, grad_dtype=g_dt, row_loss=True)
    torch.cuda.synchronize()
    ref_loss, ref_rows, ref_g = orc.kl_fwd_bwd(host(t), host(s), T=T)
    assert_kl_loss_close(float(host(loss)[0]), ref_loss)
    assert_kl_loss_close(host(rows), ref_rows)
    assert_kl_grad_close(host(g), ref_g, kl_probs(host(t), host(s), T), 1.0 / tokens, T)


@pytest.mark.parametrize("case", range(6))
def test_clipped_ste_sweep(dev, orc, case):
    rng = np.random.default_rng(4000 + case)
    xt, gt = ["bf16", "fp32"][case % 2], ["bf16", "fp32"][(case // 2) % 2]
    B, R, C = int(rng.integers(1, 4)), int(rng.integers(1, 200)), 16 * int(rng.integers(1, 300))
    x = random_tensor(rng, (B, R, C), xt)
    gy = random_tensor(rng, (B, R, C), gt)
    xh = host(x)
    sc = np.empty((B, R, C // 16), np.uint8)
    ts = np.empty(B, np.float32)
    for b in range(B):   # the oracle's own dynamic forward scales
        _, s_b, t_b, _ = orc.nvfp4_quantize(xh[b])
        sc[b], ts[b] = s_b.reshape(R, C // 16), t_b
    announce("clipped STE sweep case %d x=%s g=%s B=%d R=%d C=%d" % (case, xt, gt, B, R, C))
    gx = q.nvfp4_qdq_bwd_clipped(gy.to(dev), x.to(dev), torch.from_numpy(sc).to(dev), torch.from_numpy(ts).to(dev))
    torch.cuda.synchronize()
    gh, gyh = host(gx), host(gy)
    for b in range(B):
        ref, _ = orc.nvfp4_qdq_bwd_clipped(gyh[b].ravel(), xh[b].ravel(), sc[b].ravel(), float(ts[b]))
        assert np.array_equal(gh[b].ravel(), ref), (case, b)


@pytest.mark.parametrize("case", range(24))
def test_topk_topp_sweep(dev, orc, case):
    rng = np.random.default_rng(9000 + case)
    tokens = int(rng.integers(1, 40))
    if case % 3 == 0:
        vocab = 16384 * int(rng.integers(1, 4)) + 8 * int(rng.integers(-2, 3))
    else:
        vocab = 8 * int(rng.integers(1, 6000))
    vocab = max(vocab, 8)
    T = float(rng.choice([0.5, 1.0, 2.0]))
    in_dt = [torch.bfloat16, torch.float32][case % 2]
    g_dt = [torch.bfloat16, torch.float32][(case // 2) % 2]
    t, s = synth.logits_bf16(tokens=tokens, vocab=vocab, teacher_std=float(rng.uniform(0.5, 6)), seed=9000 + case)
    if case % 5 == 4:   # tie-heavy teacher on a coarse grid
        t = (torch.round(t.float() * 2) / 2).to(torch.bfloat16)
    t, s = t.to(in_dt), s.to(in_dt)
    if case % 2 == 0:
        k = int(rng.integers(1, vocab + 3))
        test_gpu_kl_topk.run_and_check(dev, orc, t, s, k, T, g_dt, "sweep %d" % case)
    else:
        p = float(rng.choice([1e-4, 0.1, 0.5, 0.9, 0.99, 1.0])) if case % 7 else float(rng.uniform(0.01, 1.0))
        test_gpu_kl_topp.run_and_check(dev, orc, t, s, p, T, g_dt, "sweep %d" % case)


@pytest.mark.parametrize("case", range(12))
def test_mse_calibrate_sweep(dev, orc, case):
    # random shapes, dtypes, candidate counts and k ranges (the grid kept no
    # coarser than k_min/16 per step, as the library requires), magnitudes
    # from 2^-40 to 2^40 with outlier columns; every scale compared
    rng = np.random.default_rng(7000 + case)
    B, R, C = int(rng.integers(1, 4)), int(rng.integers(1, 120)), 16 * int(rng.integers(1, 200))
    dt = [torch.bfloat16, torch.float32][case % 2]
    n = int(rng.choice([1, 2, 16, 64, 128]))
    kmin = float(rng.choice([0.25, 0.5, 0.75, 0.9]))
    kmax = 1.0 if n > 1 else kmin
    if n > 1 and (kmax - kmin) / (n - 1) > kmin / 16:
        n = int(np.ceil((kmax - kmin) * 16 / kmin)) + 1
    x = torch.from_numpy(rng.standard_normal((B, R, C)).astype(np.float32) * float(2.0 ** rng.uniform(-40, 40)))
    x[..., ::int(rng.integers(3, 50))] *= float(rng.uniform(1, 40))
    x = x.to(dt)
    announce("mse sweep case %d B=%d R=%d C=%d %s n=%d k=[%g,%g]" % (case, B, R, C, dt, n, kmin, kmax))
    sc, ts = q.nvfp4_mse_calibrate(x.to(dev), n, kmin, kmax)
    torch.cuda.synchronize()
    xh = host(x)
    for b in range(B):
        rs, rt = orc.mse_calibrate(xh[b], n, kmin, kmax)
        assert host(ts)[b] == np.float32(rt), (case, b)
        assert np.array_equal(host(sc)[b].reshape(rs.shape), rs), (case, b)


@pytest.mark.parametrize("case", range(8))
def test_linear_sweep(dev, orc, case):
    # random M, N, K through the W4A4 linear's own checker; every fourth with
    # the oracle's MSE-calibrated weight scales frozen
    rng = np.random.default_rng(8000 + case)
    M, N, K = int(rng.integers(1, 700)), int(rng.integers(1, 700)), 16 * int(rng.integers(1, 80))
    dt = [torch.bfloat16, torch.float32][case % 2]
    test_gpu_linear.run_case(dev, orc, M, N, K, dt, seed=8000 + case, frozen=case % 4 == 3)
