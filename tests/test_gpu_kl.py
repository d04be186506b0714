"""GPU parity of the fused KL(teacher || student) loss and gradient.

Tolerances (the oracle is binary64; the kernels accumulate in fp32):
  * mean loss: |L - L_ref| <= 1e-5 |L_ref|;
  * per-row loss: |r - r_ref| <= 1e-5 |r_ref| + 1e-6 -- a row's KL is the
    difference of O(1) terms (E_p[t-s]/T and the log-sum-exp gap), so fp32
    leaves an absolute floor of a few 1e-7 nats on rows whose KL is near 0;
  * fp32 gradient: per row, max and L2 error <= 1e-5 of the row's max / L2
    norm of the reference;
  * bf16 gradient: the bf16 rounding of a value inside that fp32 band;
  * on near one-hot rows (low T, wide logits) the gradient q - p is far
    below the probabilities it is the difference of; there the band is
    1e-6 of max(p + q) (and of its L2), the fp32 floor of that difference.
Full-size logits (8192 x 131072) are checked on sampled rows; the mean over
all rows is checked against the per-row losses the kernel wrote.
"""
import numpy as np
import pytest
import torch

import nvfp4_quantization_aware_amd as q
from nvfp4_quantization_aware_amd import synth
from gpu_util import announce, assert_kl_grad_close, gpu_device, host, prob_scale

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


def _check_rows(rows_dev, rows_ref):
    rows_dev = np.asarray(rows_dev, np.float64)
    err = np.abs(rows_dev - rows_ref)
    assert np.all(err <= 1e-5 * np.abs(rows_ref) + 1e-6), (err.max(), np.argmax(err))


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
    assert abs(loss - ref_loss) <= 1e-5 * abs(ref_loss)
    _check_rows(rows, ref_rows)
    assert_kl_grad_close(g, ref_g)


@pytest.mark.parametrize("g_dt", [torch.bfloat16, None])
def test_kl_many_rounds(dev, orc, g_dt):
    # 1024 rows x 5 segments (the last one ragged): many more workgroups than
    # fit on the device at once, so exchanges span many dispatch waves
    t, s = synth.logits_bf16(tokens=1024, vocab=65544, seed=17)
    loss, rows, g = run_kl(dev, t, s, 1.0, g_dt, "many rounds")
    ref_loss, ref_rows, ref_g = orc.kl_fwd_bwd(host(t), host(s), grad_scale=1.0 / 1024)
    assert abs(loss - ref_loss) <= 1e-5 * abs(ref_loss)
    _check_rows(rows, ref_rows)
    if g_dt is not None:
        assert_kl_grad_close(g, ref_g)


@pytest.mark.parametrize("T,std,vocab", [(0.5, 8.0, 131072), (0.25, 8.0, 16384), (0.5, 5.0, 23744)])
@pytest.mark.parametrize("g_dt", [torch.float32, torch.bfloat16])
def test_kl_near_one_hot_rows(dev, orc, T, std, vocab, g_dt):
    # low temperature and wide logits: both distributions nearly one-hot at
    # the same entry, so the gradient q - p is many orders of magnitude below
    # the probabilities; fp32 then reaches the fp32 floor of the difference
    # (1e-6 of the probabilities), not 1e-5 of the tiny gradient itself
    t, s = synth.logits_bf16(tokens=16, vocab=vocab, teacher_std=std, seed=int(100 * T + std))
    loss, rows, g = run_kl(dev, t, s, T, g_dt, "near one-hot")
    ref_loss, ref_rows, ref_g = orc.kl_fwd_bwd(host(t), host(s), T=T)
    assert abs(loss - ref_loss) <= 1e-5 * abs(ref_loss)
    _check_rows(rows, ref_rows)
    assert_kl_grad_close(g, ref_g, floor=prob_scale(host(t), host(s), T, 1.0 / 16))


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
    # (q - p) is computed as one fused multiply-add: exact up to one rounding
    assert np.abs(g).max() <= 1e-7 / 8


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
    pick = [0, 1, 2047, 4096, 6000, 8191]
    idx = torch.as_tensor(pick, device=dev)
    th, sh = host(t.index_select(0, idx)), host(s.index_select(0, idx))
    gh = host(g.index_select(0, idx))
    _, ref_rows, ref_g = orc.kl_fwd_bwd(th, sh, grad_scale=1.0 / 8192)
    _check_rows(rows_h[pick], ref_rows)
    assert_kl_grad_close(gh, ref_g)
