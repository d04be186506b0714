"""GPU parity of the teacher-top-p (nucleus) KL (qad_kl_topp_fwd_bwd) against
the oracle.

The threshold of a row is the largest teacher value at which the teacher mass
of the entries at or above it reaches top_p.  The library sums the masses
exactly in fixed point from the same exponentials its KL kernels use, so its
choice can differ from the oracle's exact-arithmetic one only where the
accumulated mass lies within the exponentials' error of top_p.  The tests
require the identical threshold wherever the oracle's decision margin
exceeds 1e-5; elsewhere the library's threshold must be a valid nucleus
boundary within 1e-5 (checked with the oracle's binary64 masses).  On the
set the library chose, loss and gradient follow the rules of the top-k KL:
mean and per-row loss within 1e-5 relative (1e-12 absolute where the exact
KL is 0), gradient element by element within 1e-5 of the element plus 1e-6
of the renormalised (p + q) grad_scale / T (plus one fp32 ulp, or half a
bf16 ulp), and exactly 0 outside the set.
"""
import numpy as np
import pytest
import torch

import nvfp4_quantization_aware_amd as q
from nvfp4_quantization_aware_amd import synth
from gpu_util import announce, assert_kl_grad_close, assert_kl_loss_close, gpu_device, host, kl_probs

pytestmark = pytest.mark.gpu

DECISION_TOL = 1e-5


@pytest.fixture(scope="module")
def dev():
    return gpu_device()


def _as_f64(a):
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _masses(tv_row: np.ndarray, tau: float, T: float):
    """binary64 teacher mass strictly above and at or above tau"""
    x = tv_row / T
    p = np.exp(x - x.max())
    p /= p.sum()
    return p[tv_row > tau].sum(), p[tv_row >= tau].sum()


def run_and_check(dev, orc, t, s, top_p, T, g_dt, label, grad_scale=None):
    announce("qad_kl_topp_fwd_bwd %s %s top_p=%g T=%g grad=%s" % (label, tuple(t.shape), top_p, T, g_dt))
    loss, rows, g, tau = q.qad_kl_topp_fwd_bwd(t.to(dev), s.to(dev), top_p, temperature=T, grad_scale=grad_scale,
                                               grad_dtype=g_dt, row_loss=True, tau=True)
    torch.cuda.synchronize()
    th, sh = host(t), host(s)
    tv = _as_f64(th)
    p32 = float(np.float32(top_p))
    ref = orc.kl_topp_fwd_bwd(th, sh, p32, T=T, grad_scale=grad_scale)
    ref_loss, ref_rows, ref_g, cnt, ref_tau, mass = ref
    tg = host(tau).astype(np.float64)
    redo = []
    for r in range(t.shape[0]):
        margin = min(p32 - mass[r, 0], mass[r, 1] - p32) if p32 < 1 else np.inf
        if tg[r] == ref_tau[r]:
            continue
        assert margin <= DECISION_TOL, (label, r, tg[r], ref_tau[r], margin)
        assert np.any(tv[r] == tg[r]), "threshold is not a teacher value of the row"
        above, incl = _masses(tv[r], tg[r], T)
        assert above < p32 + DECISION_TOL and incl >= p32 - DECISION_TOL, (label, r, above, incl)
        redo.append(r)
    gs = grad_scale if grad_scale is not None else 1.0 / t.shape[0]
    for r in redo:  # compare with the oracle on the set the library chose
        k = int((tv[r] > tg[r]).sum()) + 1
        _, rr, gr, _ = orc.kl_topk_fwd_bwd(th[r:r + 1], sh[r:r + 1], k, T=T, grad_scale=gs)
        ref_rows[r], ref_g[r] = rr[0], gr[0]
    ref_loss = float(ref_rows.mean())
    loss = float(host(loss)[0])
    assert_kl_loss_close(loss, ref_loss)
    assert_kl_loss_close(host(rows), ref_rows)
    kept = tv >= tg[:, None]
    if g is not None:
        gh = host(g)
        assert np.all(gh[~kept] == 0), "gradient outside the kept set"
        assert_kl_grad_close(gh, ref_g, kl_probs(th, sh, T, kept), gs, T)
    return tg, kept.sum(axis=1)


@pytest.mark.parametrize("tokens,vocab,top_p,T,in_dt,g_dt", [
    (16, 4096, 0.9, 1.0, torch.bfloat16, torch.float32),
    (8, 2048, 0.5, 1.0, torch.bfloat16, torch.bfloat16),
    (5, 1000, 1.0, 2.0, torch.float32, torch.float32),        # top_p = 1: every entry
    (5, 1000, 1e-6, 1.0, torch.bfloat16, torch.float32),      # only the argmax group
    (7, 12344, 0.95, 0.5, torch.bfloat16, torch.bfloat16),    # ragged last units
    (3, 8, 0.7, 1.0, torch.bfloat16, torch.bfloat16),
    (4, 131072, 0.9, 1.0, torch.bfloat16, torch.bfloat16),
    (3, 24584, 0.8, 1.0, torch.float32, torch.bfloat16),      # 32-bit keys: three radix rounds
    (2, (1 << 20) + 8, 0.9, 1.0, torch.bfloat16, torch.bfloat16),  # past 64 record segments: one workgroup per row
])
def test_topp_small(dev, orc, tokens, vocab, top_p, T, in_dt, g_dt):
    t, s = synth.logits_bf16(tokens=tokens, vocab=vocab, seed=tokens * 13 + vocab)
    run_and_check(dev, orc, t.to(in_dt), s.to(in_dt), top_p, T, g_dt, "small")


def test_topp_full_vocab_equals_kl(dev, orc):
    t, s = synth.logits_bf16(tokens=6, vocab=16384, seed=3)
    t, s = t.to(dev), s.to(dev)
    announce("qad_kl_topp_fwd_bwd top_p=1 vs qad_kl_fwd_bwd")
    a = q.qad_kl_topp_fwd_bwd(t, s, 1.0, grad_dtype=torch.float32, row_loss=True, tau=True)
    b = q.qad_kl_fwd_bwd(t, s, grad_dtype=torch.float32, row_loss=True)
    torch.cuda.synchronize()
    assert torch.equal(a[3], t.float().min(dim=1).values)
    assert torch.allclose(a[1], b[1], rtol=1e-5, atol=0.0)


@pytest.mark.parametrize("in_dt", [torch.bfloat16, torch.float32])
def test_topp_many_ties(dev, orc, in_dt):
    # teacher on a coarse grid: large groups of tied values at the boundary
    rng = np.random.default_rng(17)
    t = torch.from_numpy(np.round(rng.normal(0, 3, (6, 8192)) * 4) / 4).to(in_dt)
    s = (t.double() + torch.from_numpy(rng.normal(0, 0.5, (6, 8192)))).to(in_dt)
    for p in (0.3, 0.9):
        run_and_check(dev, orc, t, s, p, 1.0, torch.float32, "ties")


@pytest.mark.parametrize("top_p", [0.2, 0.9, 1.0])
def test_topp_count_overflow_rows(dev, orc, top_p):
    # more than 65535 equal bf16 teacher logits in a row: the one-read key
    # counts overflow and those rows are redone by the radix rounds
    rng = np.random.default_rng(int(top_p * 10))
    t = torch.from_numpy(rng.normal(0, 3, (3, 131072))).to(torch.bfloat16)
    t[0, rng.choice(131072, 70000, replace=False)] = 0.5
    t[2, rng.choice(131072, 100000, replace=False)] = 9.0
    s = (t.double() + torch.from_numpy(rng.normal(0, 0.5, (3, 131072)))).to(torch.bfloat16)
    run_and_check(dev, orc, t, s, top_p, 1.0, torch.float32, "count overflow")


@pytest.mark.parametrize("in_dt", [torch.float32, torch.bfloat16])
def test_topp_signed_zero_group(dev, orc, in_dt):
    # -0 and +0 are one teacher value: kept together when zero is the boundary
    # (bf16 teachers take the key-count kernel, fp32 ones the radix rounds)
    t = torch.full((2, 64), -30.0, dtype=torch.float32)
    t[:, 20:30] = -0.0
    t[:, 30:40] = 0.0
    s = torch.linspace(-1, 1, 128, dtype=torch.float32).reshape(2, 64)
    tg, n = run_and_check(dev, orc, t.to(in_dt), s.to(in_dt), 0.5, 1.0, torch.float32, "signed zeros")
    assert (tg == 0).all() and (n == 20).all()


def test_topp_identical(dev):
    t, _ = synth.logits_bf16(tokens=4, vocab=8192, seed=4)
    announce("qad_kl_topp_fwd_bwd identical")
    loss, rows, g, _ = q.qad_kl_topp_fwd_bwd(t.to(dev), t.clone().to(dev), 0.9, grad_dtype=torch.float32,
                                             row_loss=True)
    torch.cuda.synchronize()
    assert float(loss.item()) == 0.0 and torch.all(rows == 0)
    assert float(g.abs().max()) <= 1e-7 / 4


def test_topp_deterministic_and_forward_only(dev):
    t, s = synth.logits_bf16(tokens=16, vocab=16384, seed=9)
    t, s = t.to(dev), s.to(dev)
    announce("qad_kl_topp_fwd_bwd determinism")
    a = q.qad_kl_topp_fwd_bwd(t, s, 0.9, row_loss=True, tau=True)
    b = q.qad_kl_topp_fwd_bwd(t, s, 0.9, row_loss=True, tau=True)
    c = q.qad_kl_topp_fwd_bwd(t, s, 0.9, grad_dtype=None, row_loss=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1]) and c[2] is None and c[3] is None


def test_topp_full_size_sampled(dev, orc):
    announce("full-size logits 8192x131072 generate")
    t, s = synth.logits_bf16(seed=5, device=dev)
    announce("full-size qad_kl_topp_fwd_bwd top_p=0.9 bf16 gradient")
    loss, rows, g, tau = q.qad_kl_topp_fwd_bwd(t, s, 0.9, row_loss=True, tau=True)
    torch.cuda.synchronize()
    loss = float(host(loss)[0])
    rows_h = host(rows).astype(np.float64)
    assert abs(loss - rows_h.mean()) <= 1e-6 * abs(loss)
    tau_h = host(tau).astype(np.float64)
    # thresholds and losses of 48 sampled rows
    pick = sorted(set([0, 1, 4097, 8191] + list(np.random.default_rng(2).choice(8192, 44, replace=False))))
    idx = torch.as_tensor(pick, device=dev)
    th, sh = host(t.index_select(0, idx)), host(s.index_select(0, idx))
    p32 = float(np.float32(0.9))
    _, ref_rows, _, _, ref_tau, mass = orc.kl_topp_fwd_bwd(th, sh, p32, grad_scale=1.0 / 8192, want_grad=False)
    margin = np.minimum(p32 - mass[:, 0], mass[:, 1] - p32)
    same = tau_h[pick] == ref_tau
    assert np.all(same | (margin <= DECISION_TOL))
    assert_kl_loss_close(rows_h[pick][same], ref_rows[same])
    # loss and gradient of 16 of them in full
    sixteen = [pick.index(r) for r in (0, 1, 4097, 8191)] + [i for i in range(len(pick)) if pick[i] not in
                                                              (0, 1, 4097, 8191)][:12]
    rows16 = [pick[i] for i in sixteen]
    gh = host(g.index_select(0, torch.as_tensor(rows16, device=dev)))
    _, _, ref_g, _, ref_t16, _ = orc.kl_topp_fwd_bwd(th[sixteen], sh[sixteen], p32, grad_scale=1.0 / 8192)
    assert np.array_equal(ref_t16, tau_h[rows16])
    kept = _as_f64(th[sixteen]) >= ref_t16[:, None]
    assert np.all(gh[~kept] == 0)
    assert_kl_grad_close(gh, ref_g, kl_probs(th[sixteen], sh[sixteen], 1.0, kept), 1.0 / 8192, 1.0)
