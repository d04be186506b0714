"""GPU parity of the teacher-top-k KL (qad_kl_topk_fwd_bwd) against the oracle.

The kept set of a row is every entry whose teacher logit is at least the k-th
largest (ties kept); both softmaxes are renormalised over it and the gradient
is exactly 0 elsewhere.  Tolerances as for the full-vocabulary KL: mean and
per-row loss within 1e-5 relative (1e-12 absolute where the exact KL is 0,
as with a single kept entry), gradient element by element within 1e-5 of
the element plus 1e-6 of the renormalised (p + q) grad_scale / T (plus one
fp32 ulp, or half a bf16 ulp).  The kept set itself is compared exactly: the
gradient must be 0 at every entry outside it.
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


def _as_f64(a):
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _kept(th, k):
    tv = _as_f64(th)
    kk = min(k, tv.shape[1])
    tau = -np.sort(-tv, axis=1)[:, kk - 1:kk]
    return tv >= tau


def run_and_check(dev, orc, t, s, k, T, g_dt, label, grad_scale=None):
    announce("qad_kl_topk_fwd_bwd %s %s k=%d T=%g grad=%s" % (label, tuple(t.shape), k, T, g_dt))
    loss, rows, g = q.qad_kl_topk_fwd_bwd(t.to(dev), s.to(dev), k, temperature=T, grad_scale=grad_scale,
                                          grad_dtype=g_dt, row_loss=True)
    torch.cuda.synchronize()
    th, sh = host(t), host(s)
    ref_loss, ref_rows, ref_g, cnt = orc.kl_topk_fwd_bwd(th, sh, k, T=T, grad_scale=grad_scale)
    loss = float(host(loss)[0])
    assert_kl_loss_close(loss, ref_loss)
    assert_kl_loss_close(host(rows), ref_rows)
    if g is not None:
        gh = host(g)
        kept = _kept(th, k)
        assert np.array_equal(kept.sum(axis=1), cnt)
        assert np.all(gh[~kept] == 0), "gradient outside the kept set"
        gs = grad_scale if grad_scale is not None else 1.0 / t.shape[0]
        assert_kl_grad_close(gh, ref_g, kl_probs(th, sh, T, kept), gs, T)
    return loss


@pytest.mark.parametrize("tokens,vocab,k,T,in_dt,g_dt", [
    (16, 4096, 64, 1.0, torch.bfloat16, torch.float32),
    (8, 2048, 1, 1.0, torch.bfloat16, torch.bfloat16),
    (5, 1000, 1000, 2.0, torch.float32, torch.float32),      # k = V: the full vocabulary
    (5, 1000, 5000, 1.0, torch.bfloat16, torch.float32),     # k > V
    (7, 12344, 4096, 0.5, torch.bfloat16, torch.bfloat16),   # ragged last units
    (3, 8, 3, 1.0, torch.bfloat16, torch.bfloat16),
    (4, 131072, 4096, 1.0, torch.bfloat16, torch.bfloat16),
    (3, 24584, 300, 1.0, torch.float32, torch.bfloat16),
    (2, (1 << 20) + 8, 4096, 1.0, torch.bfloat16, torch.bfloat16),  # past 64 record segments: one workgroup per row
    # k / V ~ 5.5%: about 36% of 8-entry units hold a kept entry, ~184 of a
    # wave's 512, so some waves pack theirs for pass 2 and some (over 192)
    # take the plain loop, in the same workgroups; bf16 and fp32 gradients,
    # and a ragged last segment
    (6, 65536, 3600, 1.0, torch.bfloat16, torch.bfloat16),
    (4, 65536, 3600, 1.0, torch.bfloat16, torch.float32),
    (5, 40008, 2300, 0.7, torch.bfloat16, torch.bfloat16),
])
def test_topk_small(dev, orc, tokens, vocab, k, T, in_dt, g_dt):
    t, s = synth.logits_bf16(tokens=tokens, vocab=vocab, seed=tokens * 11 + vocab + k)
    run_and_check(dev, orc, t.to(in_dt), s.to(in_dt), k, T, g_dt, "small")


@pytest.mark.parametrize("in_dt", [torch.bfloat16, torch.float32])
def test_topk_many_ties(dev, orc, in_dt):
    # teacher on a coarse grid: hundreds of entries tie with the k-th largest
    rng = np.random.default_rng(7)
    t = torch.from_numpy(np.round(rng.normal(0, 3, (6, 8192)) * 4) / 4).to(in_dt)
    s = (t.double() + torch.from_numpy(rng.normal(0, 0.5, (6, 8192)))).to(in_dt)
    run_and_check(dev, orc, t, s, 512, 1.0, torch.float32, "ties")


@pytest.mark.parametrize("k", [50, 4096, 90000])
def test_topk_count_overflow_rows(dev, orc, k):
    # more than 65535 equal bf16 teacher logits in a row: the one-read key
    # counts overflow and those rows are redone by the radix rounds; k lands
    # above, inside and below the tied group
    rng = np.random.default_rng(k)
    t = torch.from_numpy(rng.normal(0, 3, (3, 131072))).to(torch.bfloat16)
    t[0, rng.choice(131072, 70000, replace=False)] = 0.5
    t[2, rng.choice(131072, 100000, replace=False)] = -1.25
    s = (t.double() + torch.from_numpy(rng.normal(0, 0.5, (3, 131072)))).to(torch.bfloat16)
    run_and_check(dev, orc, t, s, k, 1.0, torch.float32, "count overflow")


@pytest.mark.parametrize("k", [1, 100, 700])
def test_topk_rows_of_changing_scale(dev, orc, k):
    # one workgroup takes every (CU count)-th row and counts only the keys at
    # or above a bound taken from its previous row; blocks of rows with other
    # offsets and spreads put the k-th key below that bound (the row is
    # redone by the radix rounds), far above it, or between k and 4k keys
    # past it
    rng = np.random.default_rng(40 + k)
    rows, vocab = 1100, 2048
    shift = rng.choice([-60.0, -2.0, 0.0, 3.0, 60.0], size=(rows + 63) // 64).repeat(64)[:rows]
    std = rng.choice([0.25, 1.0, 3.0, 8.0], size=(rows + 31) // 32).repeat(32)[:rows]
    tf = rng.normal(0, 1, (rows, vocab)) * std[:, None] + shift[:, None]
    t = torch.from_numpy(tf).to(torch.bfloat16)
    s = (t.double() + torch.from_numpy(rng.normal(0, 0.5, (rows, vocab)))).to(torch.bfloat16)
    run_and_check(dev, orc, t, s, k, 1.0, torch.bfloat16, "changing row scale")


@pytest.mark.parametrize("in_dt", [torch.float32, torch.bfloat16])
def test_topk_signed_zero_ties(dev, orc, in_dt):
    # -0 and +0 are equal teacher logits: both are kept when zero is the k-th
    # value (bf16 teachers take the key-count kernel, fp32 ones the radix rounds)
    t = torch.zeros(2, 64, dtype=torch.float32)
    t[:, :10] = torch.arange(1, 11, dtype=torch.float32)
    t[:, 20:30] = -0.0
    t[:, 40:] = -5.0
    s = torch.linspace(-1, 1, 128, dtype=torch.float32).reshape(2, 64)
    run_and_check(dev, orc, t.to(in_dt), s.to(in_dt), 12, 1.0, torch.float32, "signed zeros")


@pytest.mark.parametrize("k", [1, 65, 200, 448, 449, 512, 640, 1000])
def test_topk_bf16_keys_around_zero(dev, orc, k):
    # bf16 teachers made only of values around zero: +-denormals, +-0, +-tiny
    # normals, each repeated 64 times, so k lands on every step of their
    # order, across the sign and the denormal range (the key-count kernel's
    # ordering and its -0 = +0 folding)
    vals = np.array([3e-38, 1e-38, 2e-39, 5e-40, 1e-40, 0.0, -0.0, -1e-40, -5e-40, -2e-39, -1e-38, -3e-38,
                     1e-3, -1e-3, 7.0, -7.0], np.float32)
    rng = np.random.default_rng(k)
    t = torch.from_numpy(np.stack([rng.permutation(np.repeat(vals, 64)) for _ in range(3)])).to(torch.bfloat16)
    s = (t.float() + torch.from_numpy(rng.normal(0, 0.5, t.shape).astype(np.float32))).to(torch.bfloat16)
    run_and_check(dev, orc, t, s, k, 1.0, torch.float32, "bf16 keys around zero")


def test_topk_identical(dev):
    t, _ = synth.logits_bf16(tokens=4, vocab=8192, seed=4)
    announce("qad_kl_topk_fwd_bwd identical")
    loss, rows, g = q.qad_kl_topk_fwd_bwd(t.to(dev), t.clone().to(dev), 100, grad_dtype=torch.float32, row_loss=True)
    torch.cuda.synchronize()
    assert float(loss.item()) == 0.0 and torch.all(rows == 0)
    assert float(g.abs().max()) == 0.0


def test_topk_deterministic_and_forward_only(dev):
    t, s = synth.logits_bf16(tokens=16, vocab=16384, seed=9)
    t, s = t.to(dev), s.to(dev)
    announce("qad_kl_topk_fwd_bwd determinism")
    a = q.qad_kl_topk_fwd_bwd(t, s, 1024, row_loss=True)
    b = q.qad_kl_topk_fwd_bwd(t, s, 1024, row_loss=True)
    c = q.qad_kl_topk_fwd_bwd(t, s, 1024, grad_dtype=None, row_loss=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1]) and c[2] is None


def test_topk_full_size_sampled(dev, orc):
    announce("full-size logits 8192x131072 generate")
    t, s = synth.logits_bf16(seed=5, device=dev)
    announce("full-size qad_kl_topk_fwd_bwd k=4096 bf16 gradient")
    loss, rows, g = q.qad_kl_topk_fwd_bwd(t, s, 4096, row_loss=True)
    torch.cuda.synchronize()
    loss = float(host(loss)[0])
    rows_h = host(rows).astype(np.float64)
    assert abs(loss - rows_h.mean()) <= 1e-6 * abs(loss)
    rng = np.random.default_rng(4096)
    pick = sorted({0, 8191} | set(int(x) for x in np.arange(30) * 270 + rng.integers(1, 270, 30)))
    idx = torch.as_tensor(pick, device=dev)
    th, sh = host(t.index_select(0, idx)), host(s.index_select(0, idx))
    gh = host(g.index_select(0, idx))
    _, ref_rows, ref_g, cnt = orc.kl_topk_fwd_bwd(th, sh, 4096, grad_scale=1.0 / 8192)
    assert_kl_loss_close(rows_h[pick], ref_rows)
    kept = _kept(th, 4096)
    assert np.all(gh[~kept] == 0)
    assert_kl_grad_close(gh, ref_g, kl_probs(th, sh, 1.0, kept), 1.0 / 8192, 1.0)
