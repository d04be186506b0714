"""GPU parity of the fused KL(teacher || student) loss and gradient.

Tolerances (the oracle is binary64; the kernels compute in fp32):
  * mean loss and every per-row loss: |L - L_ref| <= 1e-5 |L_ref| (a row
    whose exact KL is 0: |L| <= 1e-12, the second-order rounding);
  * gradient, element by element: |g - g_ref| <= 1e-5 |g_ref| + 1e-6 (p + q)
    grad_scale / T, plus one fp32 ulp (fp32 output) or half a bf16 ulp
    (bf16 output); per row (fp32), the L2 error within 1e-5 of the
    reference's L2 norm plus 1e-6 of that of (p + q) grad_scale / T.
Full-size logits (8192 x 131072) are checked on 64 sampled rows; the mean over
all rows is checked against the per-row losses the kernel wrote.
"""
import numpy as np
import pytest
import torch

import nvfp4_quantization_aware_amd as q
from nvfp4_quantization_aware_amd import synth
from gpu_util import announce, assert_kl_grad_close, assert_kl_loss_close, gpu_device, host, kl_probs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


def run_kl(dev, t, s, T, grad_dtype, label):
    announce("qad_kl_fwd_bwd %s %s T=%g grad=%s" % (label, tuple(t.shape), T, grad_dtype))
    loss, rows, g = q.qad_kl_fwd_bwd(t.to(dev), s.to(dev), temperature=T, grad_dtype=grad_dtype, row_loss=True)
    torch.cuda.synchronize()
    return float(host(loss)[0]), host(rows), None if g is None else host(g)


@pytest.mark.parametrize("tokens,vocab,T,in_dt,g_dt", [
    (64, 4096, 1.0, torch.bfloat16, torch.bfloat16),
    (64, 4096, 1.0, torch.bfloat16, torch.float32),
    (6, 131072, 1.0, torch.bfloat16, torch.float32),
    (5, 1000, 2.0, torch.float32, torch.float32),
    (3, 8, 1.0, torch.bfloat16, torch.bfloat16),
    (33, 12344, 0.5, torch.bfloat16, torch.bfloat16),
    (2, 24584, 1.0, torch.float32, torch.bfloat16),
    (3, 1 << 20, 1.0, torch.bfloat16, torch.float32),        # 64 segments of 16384 logits
    (2, (1 << 20) + 8, 1.0, torch.bfloat16, torch.bfloat16),  # one unit past 64 segments: two-pass kernel
])
def test_kl_small(dev, orc, tokens, vocab, T, in_dt, g_dt):
    t, s = synth.logits_bf16(tokens=tokens, vocab=vocab, seed=tokens * 7 + vocab)
    t, s = t.to(in_dt), s.to(in_dt)
    loss, rows, g = run_kl(dev, t, s, T, g_dt, "small")
    ref_loss, ref_rows, ref_g = orc.kl_fwd_bwd(host(t), host(s), T=T)
    assert_kl_loss_close(loss, ref_loss)
    assert_kl_loss_close(rows, ref_rows)
    assert_kl_grad_close(g, ref_g, kl_probs(host(t), host(s), T), 1.0 / tokens, T)


@pytest.mark.parametrize("g_dt", [torch.bfloat16, None])
def test_kl_many_rounds(dev, orc, g_dt):
    # 1024 rows x 5 segments (the last one ragged): many more workgroups than
    # fit on the device at once, so exchanges span many dispatch waves
    t, s = synth.logits_bf16(tokens=1024, vocab=65544, seed=17)
    loss, rows, g = run_kl(dev, t, s, 1.0, g_dt, "many rounds")
    ref_loss, ref_rows, ref_g = orc.kl_fwd_bwd(host(t), host(s), grad_scale=1.0 / 1024)
    assert_kl_loss_close(loss, ref_loss)
    assert_kl_loss_close(rows, ref_rows)
    if g_dt is not None:
        assert_kl_grad_close(g, ref_g, kl_probs(host(t), host(s), 1.0), 1.0 / 1024, 1.0)


@pytest.mark.parametrize("T,std,vocab", [(0.5, 8.0, 131072), (0.25, 8.0, 16384), (0.5, 5.0, 23744)])
@pytest.mark.parametrize("g_dt", [torch.float32, torch.bfloat16])
def test_kl_near_one_hot_rows(dev, orc, T, std, vocab, g_dt):
    # low temperature and wide logits: both distributions nearly one-hot at
    # the same entry, so the gradient q - p is many orders of magnitude below
    # the probabilities it is the difference of, and the KL of some rows is
    # far below the two terms of its difference form
    t, s = synth.logits_bf16(tokens=16, vocab=vocab, teacher_std=std, seed=int(100 * T + std))
    loss, rows, g = run_kl(dev, t, s, T, g_dt, "near one-hot")
    ref_loss, ref_rows, ref_g = orc.kl_fwd_bwd(host(t), host(s), T=T)
    assert_kl_loss_close(loss, ref_loss)
    assert_kl_loss_close(rows, ref_rows)
    assert_kl_grad_close(g, ref_g, kl_probs(host(t), host(s), T), 1.0 / 16, T)


@pytest.mark.parametrize("shift,noise,T", [(0.0, 0.02, 1.0), (-5.0, 0.2, 1.0), (12.0, 0.05, 0.5), (0.0, 0.0005, 2.0)])
def test_kl_small_kl_rows(dev, orc, shift, noise, T):
    # students very close to the teacher, or shifted from it by a constant:
    # the per-row KL (down to ~1e-7 nats) is far below the terms of the
    # difference form, so these rows take the term-wise form and must still
    # be within 1e-5 of the oracle
    t, s = synth.logits_bf16(tokens=12, vocab=40000, teacher_std=3.0, noise_std=noise, seed=int(1000 * noise) + 7)
    s = (s.float() + shift).to(torch.bfloat16)
    loss, rows, g = run_kl(dev, t, s, T, torch.float32, "small KL shift %g noise %g" % (shift, noise))
    ref_loss, ref_rows, ref_g = orc.kl_fwd_bwd(host(t), host(s), T=T)
    assert_kl_loss_close(loss, ref_loss)
    assert_kl_loss_close(rows, ref_rows)
    assert_kl_grad_close(g, ref_g, kl_probs(host(t), host(s), T), 1.0 / 12, T)


def test_kl_forward_only_matches(dev):
    t, s = synth.logits_bf16(tokens=16, vocab=2048, seed=3)
    announce("qad_kl forward only")
    l0, r0, _ = q.qad_kl_fwd_bwd(t.to(dev), s.to(dev), grad_dtype=None, row_loss=True)
    l1, r1, _ = q.qad_kl_fwd_bwd(t.to(dev), s.to(dev), row_loss=True)
    torch.cuda.synchronize()
    assert torch.equal(l0, l1) and torch.equal(r0, r1)


def test_kl_identical_distributions(dev):
    t, _ = synth.logits_bf16(tokens=8, vocab=8192, seed=4)
    loss, rows, g = run_kl(dev, t, t.clone(), 1.0, torch.float32, "identical")
    assert loss == 0.0 and np.all(rows == 0.0)
    # equal logits give x = log2(q / p) = 0 exactly, hence a zero gradient
    assert np.all(g == 0.0)


def test_kl_deterministic(dev):
    t, s = synth.logits_bf16(tokens=32, vocab=16384, seed=5)
    a = run_kl(dev, t, s, 1.0, torch.bfloat16, "run1")
    b = run_kl(dev, t, s, 1.0, torch.bfloat16, "run2")
    assert a[0] == b[0] and np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])


def test_kl_full_size_sampled(dev, orc):
    announce("full-size logits 8192x131072 generate")
    t, s = synth.logits_bf16(seed=5, device=dev)
    announce("full-size qad_kl_fwd_bwd bf16 gradient")
    loss, rows, g = q.qad_kl_fwd_bwd(t, s, row_loss=True)
    torch.cuda.synchronize()
    loss = float(host(loss)[0])
    rows_h = host(rows).astype(np.float64)
    assert abs(loss - rows_h.mean()) <= 1e-6 * abs(loss)
    assert 0.08 < loss < 0.16
    # 64 rows: both ends, and 62 spread over the rest with a seeded offset
    rng = np.random.default_rng(64)
    pick = sorted({0, 8191} | set(int(x) for x in np.arange(62) * 132 + rng.integers(1, 132, 62)))
    idx = torch.as_tensor(pick, device=dev)
    th, sh = host(t.index_select(0, idx)), host(s.index_select(0, idx))
    gh = host(g.index_select(0, idx))
    _, ref_rows, ref_g = orc.kl_fwd_bwd(th, sh, grad_scale=1.0 / 8192)
    assert_kl_loss_close(rows_h[pick], ref_rows)
    assert_kl_grad_close(gh, ref_g, kl_probs(th, sh, 1.0), 1.0 / 8192, 1.0)
